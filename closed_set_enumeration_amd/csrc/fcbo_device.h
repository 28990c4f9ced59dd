// Device kernels of libfcbo: Close-by-One concept enumeration on gfx950.
//
// Sets are LSB-first 64-bit bitmaps (element e = bit e&63 of word e>>6); one
// 64-bit word per wavefront lane.  The context lives on the device twice:
// rows (object -> attributes, N x WM words) and cols (attribute -> objects,
// M x WN words); page "hnwysp.cn/news/97538" section 3.1 and page
// "hotelren.com/news/5603750" section 2.3 keep both layouts for the two
// derivation directions.
//
// Enumeration is level-synchronous (page 4, section 2.1): the concepts of one
// level are the parents of the next.  Unlike page 4 the full canonical test of
// CbO (page 1, sections 2.1-2.2 and 4.3) is kept, so every concept is produced
// once and no sort-unique pass is needed.  Frontier extents are stored as
// sorted object lists (CSR), not bitmaps: deep in the tree an extent holds a
// handful of objects, so a list is hundreds of times smaller than a bitmap of
// N bits.
//
// Per level (parents in three classes by extent size a):
//   k_local_test     every parent: closure tests counted, item pairs, the mid
//                    and huge lists; a <= 64: parents packed into wavefronts,
//                    one lane per candidate, rows staged in LDS; child records
//   k_mid_test       64 < a <= 4096 (intents up to 8 words): closure tests by
//                    incidence, one D per carried attribute in LDS; records;
//                    a wavefront per parent up to 512 objects, a workgroup
//                    per parent above (k_mid_test_wide)
//   k_huge_*         larger parents: one item per (test, 64-word chunk of the
//                    extent bitmap), or per test over the object list
//   scans            child and object offsets per parent (exact sizes)
//   k_*_write        children (C, D, j) stored in parent order, then j order
// After the last level the output order comes from the CbO tree (subtree sizes
// bottom-up, positions top-down), k_output_intents and k_output_block write the
// caller's rows.
//
// The task pool (an alternative schedule, section at the end): the level loop
// expands only the parents with more than kPoolTaskMax objects, and k_pool
// enumerates the subtree of every smaller concept depth-first, one wavefront
// per task; k_pool_commit moves its concepts into the store, k_tail_position
// places them after their tasks, k_pool_stats counts over the whole store.
// Lattice cover edges (k_cover_*) are computed from a finished store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fcbo {

constexpr int kWave = 64;
constexpr int kSmallMax = 64;       // parents with at most this many objects use the local path
constexpr int kBlock = 256;         // threads per block for wave-per-item kernels
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kScanBlocks = 1024;   // blocks of the multi-block exclusive scan
constexpr uint64_t kScanSmallMax = 8192; // host-known lengths up to this are scanned by one workgroup
constexpr int kOutTileWords = 1024; // extent words staged in LDS per output tile
constexpr int kBmpMaxWords = 16384; // big parents use extent bitmaps when N <= 64 * this
constexpr int kMidMax = 4096;       // parents with more objects are huge (tested a chunk at a time)
constexpr int kMidWaves = 4;        // wavefronts per block of the incidence kernel
constexpr int kMidCand = 128;       // candidates whose D a wavefront keeps in LDS at a time
constexpr int kMidWide = 512;       // mid parents with more objects get a whole workgroup each
constexpr int kWideThreads = 512;   // threads of that workgroup (at least 64 x 8 candidates)
constexpr int kWideWaves = kWideThreads / kWave;

// Device counters shared by the kernels of one level, each in a 128-byte line
// of its own: atomics on one 64-byte segment are serialised by the memory
// system (about 12 ns each on MI355X), so counters that share a segment slow
// each other down.  The values below are word offsets.
constexpr int kCntPad = 16;
// Child records (of the mid parents, and of the local parents) are reserved
// through this many counters, each owning an equal region of its record buffer
// (a wavefront or workgroup picks one by its index).
constexpr int kRecStripes = 32;
enum {
    CNT_HUGE = 0 * kCntPad,      // number of huge parents
    CNT_TESTS = 1 * kCntPad,     // closure tests of this level
    CNT_PAIRS = 2 * kCntPad,     // (parent, j > cursor) pairs of this level
    CNT_OVERFLOW = 3 * kCntPad,  // a per-test or record buffer was too small: the level is redone
    CNT_CHILDREN = 4 * kCntPad,  // children of this level
    CNT_OBJS = 5 * kCntPad,      // objects in the children's extents
    CNT_THUGE = 6 * kCntPad,     // closure tests of the huge parents
    CNT_SMALL_OBJS = 7 * kCntPad, // objects in the extents of local parents
    CNT_BIG_SCAN = 8 * kCntPad,  // sum over huge parents of tests x objects
    CNT_MID = 9 * kCntPad,       // number of mid parents
    CNT_HUGEPASS = 10 * kCntPad, // passing huge tests
    CNT_MID_OBJS = 11 * kCntPad, // objects in the extents of mid parents
    CNT_MIDW = 12 * kCntPad,     // number of wide mid parents (kept at the back of mid_idx)
    CNT_NEXT_MID = 13 * kCntPad, // children that will be mid parents (64 < |C| <= mid_max)
    CNT_NEXT_HUGE = 14 * kCntPad, // children that will be huge parents (|C| > mid_max)
    CNT_WIDEREC = 15 * kCntPad,  // child records of the wide mid parents
    CNT_HUGE_NZW = 16 * kCntPad, // sum over huge parents of tests x non-zero words of the extent
    CNT_HUGE_COBJS = 17 * kCntPad, // objects of the huge parents' children
    CNT_MIDREC = 18 * kCntPad,   // kRecStripes counters, one line each: mid record slots per stripe
    CNT_LOCREC = (18 + kRecStripes) * kCntPad,  // kRecStripes counters: local record slots per stripe
    CNT_N = (18 + 2 * kRecStripes) * kCntPad  // words of one level's counters
};

// Huge parents, tested one closure test at a time: one work item per (test,
// 64-word chunk of the extent bitmap), or one wavefront per test scanning the
// object list when N is too large for bitmaps.
struct BigSet {
    uint32_t *idx;     // parent index of each member (order not fixed)
    uint32_t *n;       // closure tests (candidates) of each member
    uint64_t *off;     // exclusive scan of n; off[members] = tests of the set
    uint64_t *tasks;   // per test: member << 16 | j
    uint32_t *size;    // per test: |C| if it passed, else 0
    uint64_t *sscan;   // exclusive scan of size
    uint64_t *plist;   // passing tests
    uint64_t cap;      // capacity of tasks / size / sscan / plist (and the huge accumulators)
    uint64_t *bmp;     // extent bitmap of each member (members x wn), or null: use the lists
    uint64_t bmp_cap;  // words
    int cnt_slot, tot_slot, pass_slot;  // counters: members, tests, passing tests
};

// The per-level arguments, passed by value.
struct LevelArgs {
    const uint64_t *rows;  // N x wm
    const uint64_t *cols;  // M x wn
    int n, m, wn, wm;
    uint64_t tail_m;       // valid bits of the last intent word
    // concept store
    uint64_t *intents;     // K x wm
    int32_t *cursor;       // K, the attribute that generated the concept (-1 for the root)
    uint64_t *loff;        // K + 1 offsets into objs
    uint32_t *objs;        // extent lists, ascending object ids
    uint64_t lo, P;        // parents are concepts [lo, lo + P)
    uint64_t child_lo;     // index of the first child (= lo + P)
    uint64_t child_obj_lo; // offset in objs of the first child's list
    // per-level scratch, indexed by parent p in [0, P)
    uint64_t *pass;        // per huge parent (member index), wm words: its passing attributes
    uint64_t pass_cap;     // huge parents pass can hold
    uint32_t *nchild;      // children per parent
    uint64_t *nobj;        // objects in the children's extents per parent (a huge parent's
                           // children can hold more than 2^32 objects together)
    uint64_t *cbase;       // exclusive scan of nchild (P + 1)
    uint64_t *obase;       // exclusive scan of nobj (P + 1)
    uint32_t *mid_idx;     // mid parents (order not fixed)
    int mid_max;           // parents with more objects are huge
    uint64_t *mrec;        // child records of the mid parents (see k_mid_test)
    uint64_t mrec_region;  // records per stripe: stripe s owns [s * mrec_region, (s + 1) * mrec_region)
    uint64_t *wrec;        // child records of the wide mid parents, same layout
    uint64_t wrec_cap;     // records
    uint64_t *lrec;        // child records of the local parents, in chunks of 64 slots
    uint32_t *lfill;       // records used in each chunk of lrec
    uint64_t lrec_region;  // slots per stripe (a multiple of 64), laid out like mrec
    BigSet huge;           // huge parents
    uint64_t *dt;          // per huge test: AND of the rows of C, wm words
    uint32_t *tcnt;        // per huge test: |C|
    uint32_t *icnt;        // per (huge test, 64-word chunk): objects of C in the chunk, then offsets
    int nchunk;            // ceil(wn / 64)
    uint64_t tail_n;       // valid bits of the last extent word
    uint64_t *counters;    // CNT_* of this level
    uint64_t *counters_next; // CNT_* of the next level, cleared by the local test kernel
    int chunk;             // parents per chunk of the local test (at most LocalCfg::kChunk)
    uint64_t child_cap;    // concepts the store can hold (intents, cursors, list offsets)
    uint64_t obj_cap;      // list entries the store can hold
    int pool_max;          // parents with at most this many objects are left to the task
                           // pool (no tests, no children here); -1 without the pool
};

// ---------------------------------------------------------------------------
// small helpers

// Whether the store has room for the children this level counted.  The child
// writes are issued before the host has read the counts, so every write kernel
// checks this first and does nothing when the store must grow (the host then
// grows it and issues the writes again).
__device__ __forceinline__ bool store_has_room(const LevelArgs &A)
{
    return A.child_lo + A.counters[CNT_CHILDREN] <= A.child_cap &&
           A.child_obj_lo + A.counters[CNT_OBJS] <= A.obj_cap;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Bits of word u whose attribute index is greater than y.
__device__ __forceinline__ uint64_t above_mask(int y, int u)
{
    int lo = y - 64 * u;
    if (lo < 0) return ~0ull;
    if (lo >= 63) return 0ull;
    return ~0ull << (lo + 1);
}

// Bits 0 .. b-1 of a word (b in [0, 63]).
__device__ __forceinline__ uint64_t below_mask(int b) { return b ? ((1ull << b) - 1ull) : 0ull; }

// Position of the k-th (0-based) set bit of x; k < popcount(x).
__device__ __forceinline__ int select64(uint64_t x, int k)
{
    int pos = 0;
    int c = __popc((uint32_t)x);
    if (k >= c) { k -= c; x >>= 32; pos += 32; }
    uint32_t v = (uint32_t)x;
    c = __popc(v & 0xFFFFu);
    if (k >= c) { k -= c; v >>= 16; pos += 16; }
    c = __popc(v & 0xFFu);
    if (k >= c) { k -= c; v >>= 8; pos += 8; }
    c = __popc(v & 0xFu);
    if (k >= c) { k -= c; v >>= 4; pos += 4; }
    c = __popc(v & 0x3u);
    if (k >= c) { k -= c; v >>= 2; pos += 2; }
    if (k >= (int)(v & 1u)) pos += 1;
    return pos;
}

// --- wavefront collectives on the DPP network ------------------------------------
//
// Data-parallel-primitive moves shift values between lanes inside the VALU:
// row_shr:n within each row of 16 lanes, row_bcast:15 / :31 from the last lane
// of a row (or of rows 0-1) to the following rows, and whole-wave shifts by
// one lane.  A 64-lane inclusive scan is six such steps (Hillis-Steele inside
// the rows, then the two row broadcasts) with no trip through the LDS permute
// unit; a reduction is the scan read back from lane 63.
namespace dpp {
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
constexpr int kWaveShl1 = 0x130, kWaveShr1 = 0x138;
}  // namespace dpp

// v from the lane the DPP control selects; lanes without a source (or outside
// the row mask) get `fill`.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v, uint32_t fill)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)v, CTRL, ROWS, 0xF, false);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_move64(uint64_t v, uint64_t fill)
{
    const uint32_t lo = dpp_move<CTRL, ROWS>((uint32_t)v, (uint32_t)fill);
    const uint32_t hi = dpp_move<CTRL, ROWS>((uint32_t)(v >> 32), (uint32_t)(fill >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Inclusive scan with an associative op whose identity is `id`.
template <typename T, typename Op>
__device__ __forceinline__ T wave_incl_scan_op(T x, T id, Op op)
{
    if constexpr (sizeof(T) == 8) {
        x = op(x, dpp_move64<dpp::kRowShr1, 0xF>(x, id));
        x = op(x, dpp_move64<dpp::kRowShr2, 0xF>(x, id));
        x = op(x, dpp_move64<dpp::kRowShr4, 0xF>(x, id));
        x = op(x, dpp_move64<dpp::kRowShr8, 0xF>(x, id));
        x = op(x, dpp_move64<dpp::kRowBcast15, 0xA>(x, id));
        x = op(x, dpp_move64<dpp::kRowBcast31, 0xC>(x, id));
    } else {
        x = op(x, (T)dpp_move<dpp::kRowShr1, 0xF>(x, id));
        x = op(x, (T)dpp_move<dpp::kRowShr2, 0xF>(x, id));
        x = op(x, (T)dpp_move<dpp::kRowShr4, 0xF>(x, id));
        x = op(x, (T)dpp_move<dpp::kRowShr8, 0xF>(x, id));
        x = op(x, (T)dpp_move<dpp::kRowBcast15, 0xA>(x, id));
        x = op(x, (T)dpp_move<dpp::kRowBcast31, 0xC>(x, id));
    }
    return x;
}

// Value of a wave-uniform lane, for every lane.
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int l)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

__device__ __forceinline__ uint64_t lane_value64(uint64_t v, int l)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_and(uint64_t v)
{
    return lane_value64(wave_incl_scan_op<uint64_t>(v, ~0ull, [](uint64_t x, uint64_t y) { return x & y; }),
                        kWave - 1);
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
    return lane_value(wave_incl_scan_op<uint32_t>(v, 0u, [](uint32_t x, uint32_t y) { return x + y; }), kWave - 1);
}

__device__ __forceinline__ uint64_t wave_sum64(uint64_t v)
{
    return lane_value64(wave_incl_scan_op<uint64_t>(v, 0ull, [](uint64_t x, uint64_t y) { return x + y; }),
                        kWave - 1);
}

__device__ __forceinline__ uint64_t wave_incl_scan64(uint64_t v)
{
    return wave_incl_scan_op<uint64_t>(v, 0ull, [](uint64_t x, uint64_t y) { return x + y; });
}

// Exclusive prefix sum over the lanes of a wavefront.
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v)
{
    return wave_incl_scan_op<uint32_t>(v, 0u, [](uint32_t x, uint32_t y) { return x + y; }) - v;
}

// Exclusive prefix sum over a 256-thread block (u64); returns the block total.
__device__ __forceinline__ uint64_t block_excl_scan(uint64_t v, uint64_t *s_wave, uint64_t &total)
{
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    const uint64_t x = wave_incl_scan64(v);
    if (lane == kWave - 1) s_wave[wv] = x;
    __syncthreads();
    uint64_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
        uint64_t sw = s_wave[w];
        before += (w < wv) ? sw : 0ull;
        all += sw;
    }
    __syncthreads();
    total = all;
    return before + x - v;
}

// Loop bound helper: compile-time word count when WMC <= 8, runtime otherwise.
template <int WMC>
__device__ __forceinline__ int words_of(int wm) { return WMC <= 8 ? WMC : wm; }

// The k-th set bit, in attribute numbering, of a WMC-word set.
template <int WMC>
__device__ __forceinline__ int select_words(const uint64_t (&x)[WMC], int wm, int k)
{
    int j = 0;
    bool found = false;
#pragma unroll
    for (int u = 0; u < WMC; ++u) {
        if (u < words_of<WMC>(wm) && !found) {
            int c = __popcll(x[u]);
            if (k < c) {
                j = 64 * u + select64(x[u], k);
                found = true;
            } else {
                k -= c;
            }
        }
    }
    return j;
}

// ---------------------------------------------------------------------------
// context construction

// p[0, n) = v.  Used wherever a buffer must start cleared (a kernel rather
// than a memset node, so the clears behave the same in any launch context).
__global__ void __launch_bounds__(kBlock) k_fill_u64(uint64_t *p, uint64_t n, uint64_t v)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// dst[i] = src[i] - sub + add for i < n: extent-list offsets of a run of
// concepts whose lists move to another place of the object store.
__global__ void __launch_bounds__(kBlock) k_shift_offsets(const uint64_t *__restrict__ src, uint64_t n, uint64_t sub,
                                                          uint64_t add, uint64_t *__restrict__ dst)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
        dst[i] = src[i] - sub + add;
}

// *p = v (one thread).
__global__ void k_set_u32(uint32_t *p, uint32_t v)
{
    *p = v;
}

// Clear the bits past the last attribute in every row.
__global__ void k_mask_rows(uint64_t *rows, int n, int wm, uint64_t tail_m)
{
    uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g < (uint64_t)n) rows[g * wm + wm - 1] &= tail_m;
}

// cols[j][w] = objects 64w..64w+63 that have attribute j.  One wavefront per
// (object word w, attribute word v): lane l reads row 64w+l, 64 ballots turn
// the 64x64 bit block around, lane t keeps the ballot of bit t.  No atomics.
__global__ void __launch_bounds__(kBlock) k_transpose(const uint64_t *__restrict__ rows, uint64_t *__restrict__ cols,
                                                       int n, int m, int wn, int wm)
{
    const int lane = lane_id();
    const uint64_t wave = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    if (wave >= (uint64_t)wn * wm) return;
    const int w = (int)(wave % wn), v = (int)(wave / wn);
    const int64_t g = (int64_t)w * 64 + lane;
    const uint64_t x = g < n ? rows[g * wm + v] : 0ull;
    uint64_t mine = 0;
#pragma unroll 8
    for (int t = 0; t < 64; ++t) {
        uint64_t b = __ballot((x >> t) & 1ull);
        if (lane == t) mine = b;
    }
    const int j = 64 * v + lane;
    if (j < m) cols[(uint64_t)j * wn + w] = mine;
}

// Root concept: extent = every object, intent = AND of all rows (page 4,
// section 1.2), cursor -1.  The intent is filled with all attributes here and
// narrowed by k_root_and.
__global__ void k_root_init(uint64_t *intents, int32_t *cursor, uint64_t *loff, uint32_t *objs,
                            int n, int wm, uint64_t tail_m)
{
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < (uint64_t)n) objs[i] = (uint32_t)i;
    if (i < (uint64_t)wm) intents[i] = (i == (uint64_t)wm - 1) ? tail_m : ~0ull;
    if (i == 0) {
        cursor[0] = -1;
        loff[0] = 0;
        loff[1] = (uint64_t)n;
    }
}

__global__ void __launch_bounds__(kBlock) k_root_and(const uint64_t *__restrict__ rows, uint64_t *intent0, int n, int wm)
{
    __shared__ uint64_t s_red[kWavesPerBlock];
    const int u = blockIdx.y;
    uint64_t acc = ~0ull;
    for (uint64_t g = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; g < (uint64_t)n;
         g += (uint64_t)gridDim.x * blockDim.x)
        acc &= rows[g * wm + u];
    acc = wave_and(acc);
    if (lane_id() == 0) s_red[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t r = ~0ull;
        for (int w = 0; w < kWavesPerBlock; ++w) r &= s_red[w];
        if (r != ~0ull) atomicAnd((unsigned long long *)&intent0[u], (unsigned long long)r);
    }
}

// ---------------------------------------------------------------------------
// per-level kernels
//
// Parents fall in three classes by extent size a:
//   local   a <= 64          k_local_test, one 64-bit object mask per candidate
//   mid     64 < a <= mid_max k_mid_test, closure tests by incidence
//   huge    a > mid_max      one work item per (test, 64-word chunk) of the
//                            extent bitmap, or per test over the object list

// Append the values of the flagged lanes to list[*counter], one atomic per wavefront.
__device__ __forceinline__ void wave_append(bool flag, uint32_t value, uint32_t *list, uint64_t *counter)
{
    const uint64_t bal = __ballot(flag);
    if (!bal) return;
    const int lane = lane_id();
    const int leader = __ffsll((unsigned long long)bal) - 1;
    uint64_t base = 0;
    if (lane == leader) base = atomicAdd((unsigned long long *)counter, (unsigned long long)__popcll(bal));
    base = lane_value64(base, leader);
    if (flag) list[base + __popcll(bal & below_mask(lane))] = value;
}

__device__ __forceinline__ uint64_t wave_or(uint64_t v)
{
    return lane_value64(wave_incl_scan_op<uint64_t>(v, 0ull, [](uint64_t x, uint64_t y) { return x | y; }),
                        kWave - 1);
}

// --- local parents (|A| <= 64): closure tests packed across parents -----------
//
// For a candidate j (j > y, j not in B) let c_j be the objects of A having j.
// C = A AND col[j] restricted to A is c_j; D = C' is the AND of their rows, and
// the canonical test asks that D adds no attribute below j to B (page 1,
// section 4.3: bits 0..j-1 compared, bit j excluded).
//
// Candidates split in two kinds:
//   * j carried by some object of A (the set U): c_j is non-empty and is tested
//     in full;
//   * j carried by no object of A: C is empty, D = M, so the test passes only
//     when every attribute below j is in B, i.e. j is the first attribute not in
//     B (called j0 below).  That single candidate, when above y, yields the
//     bottom concept; it is tested like the others with c_j empty.
// Attribute-saturation pruning (page 1, section 2.3) is the j-in-B skip: with B
// closed, A inside col[j] holds exactly when j is in B.
//
// Local parents have a handful of objects and about as many candidates, so one
// wavefront serves many of them at once.  A wavefront takes a chunk of
// consecutive parents (one per lane for the metadata, intents staged in LDS) and
// cuts it into groups whose objects fit 64 LDS row slots and whose (parent,
// intent word) pairs fit 64 lanes.  Per group: one lane per object slot stages
// its row; one lane per (parent, word) ORs the parent's staged rows into U and
// turns U into candidate bits; the candidates, in parent-major and ascending j order, are
// then tested 64 at a time, one per lane, and passing children leave records
// (layout in k_mid_test) with the object mask c_j in word 3, so the child write
// needs no recomputation.  Child ranks and object offsets within a parent are
// segmented scans over the lanes plus a per-parent carry between rounds.

// A level with few parents gets smaller chunks, halved down to kLocalMinChunk
// until there are kLocalChunksPerCu chunks per compute unit: with 64 parents
// per chunk the shallow levels (tens of thousands of parents, each with
// hundreds of candidates) would occupy a fraction of the wavefront slots.
constexpr int kLocalChunksPerCu = 16;
constexpr int kLocalMinChunk = 8;

// Occupancy: the per-wavefront LDS is the staged rows (64 x WMC words) plus the
// chunk's intents (kChunk x WMC words).  Intents of 5 to 8 words take chunks of
// 16 parents, two per wavefront, so that a workgroup's LDS leaves room for
// seven wavefronts per SIMD; the register budget that allows (72 VGPRs, a few
// dozen bytes spilled) is faster on them than five wavefronts without spills
// (ctx50000x400: local test 2.30 -> 1.95 ms).  Up to four words the 64-parent
// chunk leaves room for eight; seven (72 VGPRs) measured best there.  Eight
// words cannot be held to the budget of seven and keep the compiler's choice.
template <int WMC>
struct LocalCfg {
    static constexpr int kWaves = WMC <= 8 ? kWavesPerBlock : 1;  // wavefronts per block
    static constexpr int kThreads = kWave * kWaves;
    static constexpr int kChunk = WMC <= 4 ? kWave : WMC <= 8 ? 16 : 512 / WMC;  // parents per chunk
    static constexpr int kChunksPerWave = WMC <= 4 ? 1 : WMC <= 8 ? 2 : 1;      // at launch
    static constexpr int kWavesPerEu = WMC <= 7 ? 7 : 1;                       // occupancy asked for
};

__device__ __forceinline__ uint64_t uniform64(uint64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Set bits of a uniform mask below the calling lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Reserve `n = popcount(bal)` consecutive slots of a device counter for the
// flagged lanes of a wavefront; returns this lane's slot.
__device__ __forceinline__ uint64_t wave_slot(uint64_t bal, uint64_t *counter)
{
    const int leader = __ffsll((unsigned long long)bal) - 1;
    uint64_t base = 0;
    if (lane_id() == leader) base = atomicAdd((unsigned long long *)counter, (unsigned long long)__popcll(bal));
    base = lane_value64(base, leader);
    return base + lanes_below(bal);
}

__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bits 0 .. b of a word (b in [0, 63]).
__device__ __forceinline__ uint64_t upto_mask(int b) { return (2ull << b) - 1ull; }

template <int WMC>
__global__ void __launch_bounds__(LocalCfg<WMC>::kThreads)
    __attribute__((amdgpu_waves_per_eu(LocalCfg<WMC>::kWavesPerEu))) k_local_test(LevelArgs A)
{
    constexpr int kW = LocalCfg<WMC>::kWaves;
    constexpr int CH = LocalCfg<WMC>::kChunk;
    // the group's object rows, slot-major; spare slots let the c_j reads below
    // run past a group's last slot without a guard (seven for reads eight at a
    // time up to four words, three for reads four at a time up to eight: the
    // most that keeps seven workgroups per CU)
    constexpr int kRowPad = WMC <= 4 ? 7 : WMC <= 8 ? 3 : 0;
    __shared__ uint64_t s_rows[kW][(kSmallMax + kRowPad) * WMC];
    __shared__ uint64_t s_b[kW][CH * WMC];            // the chunk's intents, padding bits past M set
    __shared__ uint32_t s_seg[kW][kWave];             // per group parent: first slot | objects << 8
    // per group parent: children, their objects; before the tests, per (parent,
    // word) lane the first attributes of the objects (below)
    __shared__ __align__(8) uint32_t s_run[kW][2 * kWave];
    __shared__ uint8_t s_owner[kW][kWave];            // group parent whose slots start here
    __shared__ uint8_t s_mark[kW][kWave];             // per round: (parent, word) lane whose candidates start here
    __shared__ uint64_t s_sum[5][kW];                 // level counters, per wavefront
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = words_of<WMC>(A.wm);
    const int gmax = kWave / wm;  // parents per group: one lane per (parent, word)
    // the wavefront's level counters (uniform, summed once per chunk): tests,
    // item pairs, objects of local and of mid parents, list entries the huge
    // tests would scan
    uint64_t n_tests = 0, n_pairs = 0, n_local_objs = 0, n_mid_objs = 0, n_big_scan = 0;
    uint64_t *R = s_rows[wv];
    const uint32_t *R32 = (const uint32_t *)R;
    uint64_t *SB = s_b[wv];
    uint32_t *SEG = s_seg[wv];
    uint32_t *RUN = s_run[wv];
    uint8_t *OWN = s_owner[wv];
    uint8_t *MARK = s_mark[wv];
    const uint64_t rstride = 4 + (uint64_t)A.wm;
    // Record slots are reserved 64 at a time per wavefront (a chunk) and filled
    // in order: a round's passing children take the rest of the current chunk
    // and go on at the start of a new one, so only a wavefront's last chunk is
    // left part-filled.  The wavefront's stripe owns slots [rlo, rhi).
    const int stripe = (int)(((uint64_t)blockIdx.x * kW + wv) % kRecStripes);
    const uint64_t rlo = (uint64_t)stripe * A.lrec_region, rhi = rlo + A.lrec_region;
    uint64_t rchunk = ~0ull;  // first slot of the current record chunk
    uint32_t fill = kWave;    // slots used in it
    auto next_chunk = [&]() {
        if (rchunk != ~0ull && lane == 0 && rchunk < rhi) A.lfill[rchunk / kWave] = fill;
        uint64_t c = 0;
        if (lane == 0)
            c = atomicAdd((unsigned long long *)&A.counters[CNT_LOCREC + stripe * kCntPad], (unsigned long long)kWave);
        rchunk = rlo + uniform64(c);
        fill = 0;
        if (rchunk + kWave > rhi && lane == 0) A.counters[CNT_OVERFLOW] = 1;
    };
    // slot of record k of a round's n (uniform n in [1, 64], k < n)
    auto reserve = [&](uint32_t n, uint32_t k) -> uint64_t {
        if (fill == (uint32_t)kWave) next_chunk();
        const uint32_t room = (uint32_t)kWave - fill;
        const uint64_t at = rchunk + fill + k;
        if (n <= room) {
            fill += n;
            return at;
        }
        fill = kWave;
        next_chunk();
        fill = n - room;
        return k < room ? at : rchunk + (k - room);
    };
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < CNT_N; i += blockDim.x) A.counters_next[i] = 0;
    const int chunk = (A.chunk >= 1 && A.chunk < CH) ? A.chunk : CH;
    const uint64_t nchunks = (A.P + chunk - 1) / chunk;
    for (uint64_t ch = (uint64_t)blockIdx.x * kW + wv; ch < nchunks; ch += (uint64_t)gridDim.x * kW) {
        const uint64_t p0 = ch * chunk;
        const int nq = (int)((A.P - p0) < (uint64_t)chunk ? (A.P - p0) : (uint64_t)chunk);
        // parent lanes: list start, size (0 unless local), cursor
        uint64_t o0 = 0, sz = 0;
        int a = 0, y = 0;
        bool act = false;
        if (lane < nq) {
            const uint64_t c = A.lo + p0 + lane;
            o0 = A.loff[c];
            sz = A.loff[c + 1] - o0;
            y = A.cursor[c];
            act = sz <= (uint64_t)kSmallMax && (int64_t)sz > (int64_t)A.pool_max;
            a = act ? (int)sz : 0;
        }
        {
            const uint64_t *src = A.intents + (A.lo + p0) * (uint64_t)A.wm;
            for (int t = lane; t < nq * wm; t += kWave) {
                uint64_t b = src[t];
                if (t % wm == wm - 1) b |= ~A.tail_m;
                SB[t] = b;
            }
        }
        wave_sync();
        {
            // every parent of the chunk: closure tests (attributes above the
            // cursor outside B), item pairs, class; mid and huge parents go to
            // their lists, with counts cleared for their test kernels
            uint32_t nt = 0;
            if (lane < nq)
                for (int u = 0; u < wm; ++u) nt += (uint32_t)__popcll(~SB[lane * wm + u] & above_mask(y, u));
            const bool is_huge = lane < nq && sz > (uint64_t)A.mid_max;
            const bool is_mid = lane < nq && !is_huge && sz > (uint64_t)kSmallMax;
            // per chunk the sums but the last fit 32 bits (at most 64 parents of
            // at most M tests and mid_max objects each)
            n_tests += wave_sum(nt);
            n_pairs += wave_sum(lane < nq ? (uint32_t)(A.m - 1 - y) : 0u);
            n_local_objs += wave_sum(act ? (uint32_t)sz : 0u);
            n_mid_objs += wave_sum(is_mid ? (uint32_t)sz : 0u);
            n_big_scan += wave_sum64(is_huge ? sz * nt : 0ull);
            const BigSet &S = A.huge;
            const uint64_t hb = __ballot(is_huge);
            if (hb) {
                const uint64_t hpos = wave_slot(hb, &A.counters[S.cnt_slot]);
                if (is_huge) {
                    S.idx[hpos] = (uint32_t)(p0 + lane);
                    S.n[hpos] = nt;
                }
            }
            // mid parents: the narrow ones from the front of mid_idx, the wide
            // ones (more than kMidWide objects) from the back
            const bool is_wide = is_mid && sz > (uint64_t)kMidWide;
            wave_append(is_mid && !is_wide, (uint32_t)(p0 + lane), A.mid_idx, &A.counters[CNT_MID]);
            const uint64_t wb = __ballot(is_wide);
            if (wb) {
                const uint64_t wpos = wave_slot(wb, &A.counters[CNT_MIDW]);
                if (is_wide) A.mid_idx[A.P - 1 - wpos] = (uint32_t)(p0 + lane);
            }
            if (lane < nq && !act) {  // mid and huge parents, and those left to the pool
                A.nchild[p0 + lane] = 0;
                A.nobj[p0 + lane] = 0;
            }
        }
        int j0 = -1;  // first attribute outside B, when above y
        if (act) {
            for (int u = 0; u < wm; ++u) {
                const uint64_t nb = ~SB[lane * wm + u];
                if (nb) {
                    j0 = 64 * u + __ffsll((unsigned long long)nb) - 1;
                    break;
                }
            }
            if (j0 <= y) j0 = -1;
        }
        const uint32_t pre = wave_excl_scan((uint32_t)a);
        for (int s = 0; s < nq;) {
            // the group: parents [s, e), their objects in slots [0, S)
            const uint32_t base = lane_value(pre, s);
            const bool in = lane >= s && lane < s + gmax && lane < nq && pre + (uint32_t)a - base <= (uint32_t)kSmallMax;
            const int e = s + __popcll(__ballot(in));
            const int S = (int)(lane_value(pre, e - 1) + lane_value((uint32_t)a, e - 1) - base);
            // FIRST[(q, u)]: the first attributes outside B of the objects of
            // group parent q that fall in word u (one bit per object); it lives
            // in the RUN table until the candidates are known
            uint64_t *FIRST = (uint64_t *)RUN;
            FIRST[lane] = 0;
            if (in) {
                SEG[lane - s] = (pre - base) | ((uint32_t)a << 8);
                if (a > 0) OWN[pre - base] = (uint8_t)(lane - s);
            }
            const uint64_t starts = wave_or(in && a > 0 ? (1ull << (pre - base)) : 0ull);
            wave_sync();
            {
                // object slots: stage the row, mark its first attribute outside B
                const uint64_t below = starts & upto_mask(lane);
                const int st = below ? 63 - __clzll((long long)below) : 0;
                const int q = OWN[st];
                const uint64_t oq = __shfl(o0, s + q);
                if (lane < S) {
                    const uint64_t g = A.objs[oq + (uint64_t)(lane - st)];
                    uint64_t row[WMC];
#pragma unroll
                    for (int u = 0; u < WMC; ++u) row[u] = (u < wm) ? A.rows[g * A.wm + u] : 0ull;
                    int fu = -1;
                    uint64_t fx = 0;
#pragma unroll
                    for (int u = WMC - 1; u >= 0; --u) {
                        if (u < wm) {
                            R[lane * WMC + u] = row[u];
                            const uint64_t nb = row[u] & ~SB[(s + q) * wm + u];
                            if (nb) {
                                fu = u;
                                fx = nb;
                            }
                        }
                    }
                    if (fu >= 0) atomicOr((unsigned long long *)&FIRST[q * wm + fu], (unsigned long long)(fx & (0ull - fx)));
                }
            }
            wave_sync();
            // (parent, word) lanes: U = OR of the parent's staged rows, candidate
            // bits, their place in the group's list.
            //
            // A candidate j carried by a single object i of A has c_j = {i} and
            // D = row i, and it passes exactly when j is the first attribute of
            // that row outside B.  So of the candidates carried once only the
            // objects' first attributes can pass; the others are decided
            // without a test and leave the list.  The candidates kept: those
            // carried at least twice (TWO), the objects' first attributes, and
            // j0 (carried by none).
            const int G = e - s;
            const int pq = lane / wm < G ? lane / wm : G - 1;
            const int pu = lane - pq * wm;
            const int yq = __shfl(y, s + pq);
            const int j0q = __shfl(j0, s + pq);
            const bool actq = __shfl((int)act, s + pq) != 0;
            uint64_t x = 0;
            if (lane < G * wm) {
                const uint32_t sgq = SEG[pq];
                const int fq = (int)(sgq & 0xFFu), nq = (int)(sgq >> 8);
                uint64_t two = 0;
                for (int i = 0; i < nq; ++i) {
                    const uint64_t r = R[(fq + i) * WMC + pu];
                    two |= x & r;
                    x |= r;
                }
                if (actq) {
                    x &= ~SB[(s + pq) * wm + pu] & above_mask(yq, pu) & (two | FIRST[lane]);
                    if (j0q >= 0 && (j0q >> 6) == pu) x |= 1ull << (j0q & 63);
                } else {
                    x = 0;
                }
            }
            wave_sync();
            if (in) {
                RUN[2 * (lane - s)] = 0;
                RUN[2 * (lane - s) + 1] = 0;
            }
            const uint32_t cnt = (uint32_t)__popcll(x);
            const uint32_t pos = wave_excl_scan(cnt);
            const uint32_t total = lane_value(pos + cnt, kWave - 1);
            for (uint32_t r0 = 0; r0 < total; r0 += kWave) {
                // this lane's candidate: number r0 + lane of the list, held by the
                // (parent, word) lane whose prefix is the last one not above it
                const uint32_t gidx = r0 + (uint32_t)lane;
                const bool live = gidx < total;
                // The (parent, word) lane t owning candidate gidx: a lane whose
                // range starts inside the round marks its first position (the
                // wavefront's LDS writes land in program order, so the marks
                // overwrite the clearing), an inclusive max-scan carries every
                // mark to the end of its range, and positions before the first
                // mark belong to the last lane whose range starts at or before
                // r0 (every marking lane lies above it).
                MARK[lane] = 0;
                if (cnt > 0 && pos > r0 && pos < r0 + (uint32_t)kWave) MARK[pos - r0] = (uint8_t)lane;
                wave_sync();
                const int own0 = 63 - __clzll((long long)__ballot(pos <= r0));
                int t = (int)wave_incl_scan_op<uint32_t>((uint32_t)MARK[lane], 0u,
                                                         [](uint32_t a, uint32_t b) { return a > b ? a : b; });
                t = t > own0 ? t : own0;
                const uint64_t xt = __shfl(x, t);
                const uint32_t rank = gidx - __shfl(pos, t);
                const int tq = t / wm;
                const int qc = live ? tq : 0;
                const int j = live ? 64 * (t - tq * wm) + select64(xt, (int)rank) : 0;
                const int wj = j >> 6, bj = j & 63;
                const uint32_t sg = SEG[qc];
                const int first = (int)(sg & 0xFFu), na = live ? (int)(sg >> 8) : 0;
                // c_j: objects of the parent having j (32-bit LDS reads, one bit each)
                // (reads issued kCb at a time, so their LDS latencies overlap)
                uint64_t c = 0;
                {
                    constexpr int kCb = (WMC <= 4 || WMC > 8) ? 8 : 4;
                    const uint32_t *col32 = R32 + 2 * (first * WMC + wj) + (bj >> 5);
                    const uint32_t sh = (uint32_t)(bj & 31);
                    for (int i0 = 0; i0 < na; i0 += kCb) {
                        uint32_t v[kCb];
#pragma unroll
                        for (int k = 0; k < kCb; ++k)
                            v[k] = (kRowPad >= kCb - 1 || i0 + k < na) ? col32[2 * WMC * (i0 + k)] : 0u;
#pragma unroll
                        for (int k = 0; k < kCb; ++k) c |= (uint64_t)((v[k] >> sh) & 1u) << (i0 + k);
                    }
                    // bits past the parent's objects came from spare or other slots
                    if (kRowPad >= kCb - 1) c &= (na >= 64) ? ~0ull : below_mask(na);
                }
                // D = AND of the rows of c_j
                uint64_t D[WMC];
#pragma unroll
                for (int u = 0; u < WMC; ++u) D[u] = ~0ull;
                uint64_t cc = c;
                while (cc) {
                    const int i = __ffsll((unsigned long long)cc) - 1;
                    cc &= cc - 1ull;
#pragma unroll
                    for (int u = 0; u < WMC; ++u)
                        if (u < wm) D[u] &= R[(first + i) * WMC + u];
                }
                // canonical test: the first attribute of D outside B must be j itself
                int fu = WMC;
                uint64_t fx = 0;
                const uint64_t *Bq = SB + (s + qc) * wm;
#pragma unroll
                for (int u = WMC - 1; u >= 0; --u) {
                    const uint64_t xb = (u < wm) ? (D[u] & ~Bq[u]) : 0ull;
                    if (xb) {
                        fu = u;
                        fx = xb;
                    }
                }
                const bool pass = live && fu == wj && (__ffsll((unsigned long long)fx) - 1) == bj;
                const uint64_t bal = __ballot(pass);
                // segments of equal parent among the live lanes
                // neighbours' parents (whole-wave shifts by one lane; the ends only
                // matter through `lane == 0` and `lane == kWave - 1` below)
                const int prevq = (int)dpp_move<dpp::kWaveShr1, 0xF>((uint32_t)qc, 0u);
                const int nextq = (int)dpp_move<dpp::kWaveShl1, 0xF>((uint32_t)qc, 0u);
                const bool head = live && (lane == 0 || prevq != qc);
                const bool tail = live && (lane == kWave - 1 || r0 + (uint32_t)lane + 1 >= total || nextq != qc);
                const uint64_t heads = __ballot(head);
                const uint64_t hb = heads & upto_mask(lane);
                const int hl = hb ? 63 - __clzll((long long)hb) : 0;
                const uint64_t inseg = upto_mask(lane) & ~below_mask(hl);
                const uint32_t sz = pass ? (uint32_t)__popcll(c) : 0u;
                const uint32_t ex = wave_excl_scan(sz);
                const uint32_t exh = __shfl(ex, hl);
                if (bal) {
                    const uint64_t slot = reserve((uint32_t)__popcll(bal), lanes_below(bal));
                    if (pass) {
                        if (slot < rhi) {
                            const uint32_t rank = RUN[2 * qc] + (uint32_t)__popcll(bal & inseg & ~(1ull << lane));
                            const uint32_t objoff = RUN[2 * qc + 1] + (ex - exh);
                            uint64_t *rec = A.lrec + slot * rstride;
                            rec[0] = (p0 + (uint64_t)(s + qc)) | ((uint64_t)j << 32);
                            rec[1] = (uint64_t)rank | ((uint64_t)sz << 32);
                            rec[2] = objoff;
                            rec[3] = c;
#pragma unroll
                            for (int u = 0; u < WMC; ++u)
                                if (u < wm) rec[4 + u] = (u == wm - 1) ? (D[u] & A.tail_m) : D[u];
                        }
                    }
                    if (tail) {
                        RUN[2 * qc] += (uint32_t)__popcll(bal & inseg);
                        RUN[2 * qc + 1] += ex - exh + sz;
                    }
                }
                wave_sync();
            }
            // per-parent totals
            if (in && act) {
                A.nchild[p0 + lane] = RUN[2 * (lane - s)];
                A.nobj[p0 + lane] = RUN[2 * (lane - s) + 1];
            }
            wave_sync();
            s = e;
        }
    }
    if (rchunk != ~0ull && lane == 0 && rchunk < rhi) A.lfill[rchunk / kWave] = fill;
    // level counters: one atomic per workgroup and counter
    const uint64_t v[5] = {n_tests, n_pairs, n_local_objs, n_mid_objs, n_big_scan};
#pragma unroll
    for (int i = 0; i < 5; ++i)
        if (lane == 0) s_sum[i][wv] = v[i];
    __syncthreads();
    if (threadIdx.x < 5) {
        uint64_t sum = 0;
        for (int w = 0; w < kW; ++w) sum += s_sum[threadIdx.x][w];
        const int slot[5] = {CNT_TESTS, CNT_PAIRS, CNT_SMALL_OBJS, CNT_MID_OBJS, CNT_BIG_SCAN};
        if (sum) atomicAdd((unsigned long long *)&A.counters[slot[threadIdx.x]], (unsigned long long)sum);
    }
}

// Children of the local parents, one thread per record slot: intent, cursor and
// list bounds from the record, the extent list picked from the parent's list by
// the object mask.  Every load of a slot is issued before its stores (the
// record in full, then the parent's offsets, then the object ids eight at a
// time), so a thread waits for three memory latencies per child rather than
// one per word.
template <int WMC>
__global__ void __launch_bounds__(kBlock) k_local_write(LevelArgs A)
{
    if (A.counters[CNT_OVERFLOW] || !store_has_room(A)) return;
    const int wm = words_of<WMC>(A.wm);
    const uint64_t rstride = 4 + (uint64_t)A.wm;
    // Slots of stripe st: [st * region, st * region + count_st), in chunks of
    // 64.  The chunks are walked interleaved, chunk c of every stripe before
    // chunk c + 1 of any (their reservation order, roughly): flat slot f lies in
    // chunk f / 64 / kRecStripes of stripe (f / 64) % kRecStripes.
    const uint64_t nt = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int lane = lane_id();
    // the stripe counts, one per lane, loaded together
    const uint64_t counts = lane < kRecStripes ? A.counters[CNT_LOCREC + lane * kCntPad] : 0ull;
    uint64_t smax = 0;
    for (int st = 0; st < kRecStripes; ++st) smax = max(smax, lane_value64(counts, st));
    for (uint64_t f = t; f < smax * kRecStripes; f += nt) {
        // a wavefront's 64 threads share the chunk (t starts at a multiple
        // of 64 and the thread count is one), so st is uniform
        const uint64_t ch = f / kWave;
        const int st = __builtin_amdgcn_readfirstlane((int)(ch % kRecStripes));
        const uint64_t k = (ch / kRecStripes) * kWave + f % kWave;  // slot within the stripe
        if (k >= lane_value64(counts, st)) continue;
        const uint64_t i = (uint64_t)st * A.lrec_region + k;
        if ((uint32_t)(i % kWave) >= A.lfill[i / kWave]) continue;  // unused slot of a closed chunk
        const uint64_t *rec = A.lrec + i * rstride;
        const uint64_t w0 = rec[0], w1 = rec[1], w2 = rec[2];
        uint64_t c = rec[3];
        uint64_t d[WMC <= 8 ? WMC : 1];
#pragma unroll
        for (int u = 0; u < (WMC <= 8 ? WMC : 1); ++u) d[u] = (WMC <= 8 && u < wm) ? rec[4 + u] : 0ull;
        const uint64_t p = w0 & 0xFFFFFFFFull;
        const uint64_t cb = A.cbase[p], ob = A.obase[p], so = A.loff[A.lo + p];
        const uint32_t cnt = (uint32_t)(w1 >> 32);
        const uint64_t child = A.child_lo + cb + (w1 & 0xFFFFFFFFull);
        const uint64_t obeg = A.child_obj_lo + ob + w2;
        const uint32_t *src = A.objs + so;
        uint64_t q = obeg;
        while (c) {
            uint32_t v[8];
            int nv = 0;
#pragma unroll
            for (int k8 = 0; k8 < 8; ++k8) {
                const int idx = c ? __ffsll((unsigned long long)c) - 1 : 0;  // src[0] exists: c was not empty
                v[k8] = src[idx];
                nv += c ? 1 : 0;
                c &= c - 1ull;
            }
#pragma unroll
            for (int k8 = 0; k8 < 8; ++k8)
                if (k8 < nv) A.objs[q + k8] = v[k8];
            q += (uint64_t)nv;
        }
        if constexpr (WMC <= 8) {
#pragma unroll
            for (int u = 0; u < WMC; ++u)
                if (u < wm) A.intents[child * A.wm + u] = d[u];
        } else {
            for (int u = 0; u < A.wm; ++u) A.intents[child * A.wm + u] = rec[4 + u];
        }
        A.cursor[child] = (int32_t)(w0 >> 32);
        A.loff[child] = obeg;
        A.loff[child + 1] = obeg + cnt;
    }
}

// Huge parents: one task per (parent, candidate j), task = member << 16 | j,
// laid out at the scanned offsets so the tests of a parent are adjacent.
//
// With bitmaps enabled the wavefront also writes the member's extent as a
// bitmap, straight from its intent: A = B' is the AND of the columns of the
// attributes of B (all objects when B is empty), so no list is walked.  For the
// chunked set it clears the per-test accumulators as well.
template <int WMC>
__global__ void __launch_bounds__(kBlock) k_huge_tasks(LevelArgs A)
{
    const BigSet &S = A.huge;
    const int lane = lane_id();
    const int wm = words_of<WMC>(A.wm);
    const uint64_t nset = A.counters[S.cnt_slot];
    const uint64_t tset = S.off[nset];
    if (tset > S.cap || (S.bmp && nset * (uint64_t)A.wn > S.bmp_cap) || nset > A.pass_cap) {
        if (blockIdx.x == 0 && threadIdx.x == 0) A.counters[CNT_OVERFLOW] = 1;
        return;
    }
    for (uint64_t bi = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; bi < nset;
         bi += (uint64_t)gridDim.x * kWavesPerBlock) {
        const uint64_t c0 = A.lo + S.idx[bi];
        const int y = A.cursor[c0];
        if (lane < wm) A.pass[bi * A.wm + lane] = 0;  // passing attributes, set by the tests
        uint64_t cand[WMC], bset[WMC];
#pragma unroll
        for (int u = 0; u < WMC; ++u) {
            cand[u] = 0;
            bset[u] = 0;
            if (u < wm) {
                bset[u] = A.intents[c0 * A.wm + u];
                uint64_t bx = bset[u];
                if (u == wm - 1) bx |= ~A.tail_m;
                cand[u] = ~bx & above_mask(y, u);
            }
        }
        // non-zero words of the extent (the column words a test needs), for
        // the statistics' byte count
        uint32_t nzw = 0;
        if (S.bmp) {
            uint64_t *row = S.bmp + bi * (uint64_t)A.wn;
            for (int w = lane; w < A.wn; w += kWave) {
                uint64_t v = (w == A.wn - 1) ? A.tail_n : ~0ull;
#pragma unroll
                for (int u = 0; u < WMC; ++u) {
                    if (u < wm) {
                        uint64_t b = bset[u];
                        while (b) {
                            const int m = 64 * u + __ffsll((unsigned long long)b) - 1;
                            b &= b - 1ull;
                            v &= A.cols[(uint64_t)m * A.wn + w];
                        }
                    }
                }
                row[w] = v;
                nzw += v != 0 ? 1u : 0u;
            }
        } else {
            // the sorted list: one word per run of objects with equal g >> 6
            const uint64_t o0 = A.loff[c0], o1 = A.loff[c0 + 1];
            for (uint64_t o = o0 + lane; o < o1; o += kWave)
                nzw += (o == o0 || (A.objs[o - 1] >> 6) != (A.objs[o] >> 6)) ? 1u : 0u;
        }
        const uint32_t n = S.n[bi];
        const uint64_t znz = (uint64_t)wave_sum(nzw) * n;
        if (lane == 0 && znz) atomicAdd((unsigned long long *)&A.counters[CNT_HUGE_NZW], (unsigned long long)znz);
        const uint64_t base = S.off[bi];
        for (uint32_t k = lane; k < n; k += kWave) {
            S.tasks[base + k] = (bi << 16) | (uint64_t)select_words<WMC>(cand, wm, (int)k);
            if (S.bmp) {
                A.tcnt[base + k] = 0;
                for (int u = 0; u < wm; ++u) A.dt[(base + k) * A.wm + u] = ~0ull;
            }
        }
    }
}

// Mark a passing test of set S: pass bit, sibling count, object count, and
// append it to the set's pass list.
__device__ __forceinline__ void big_record_pass(const LevelArgs &A, const BigSet &S, uint64_t t, uint64_t bi,
                                                uint64_t p, int j, uint32_t cnt)
{
    atomicOr((unsigned long long *)&A.pass[bi * A.wm + (j >> 6)], (unsigned long long)(1ull << (j & 63)));
    atomicAdd(&A.nchild[p], 1u);
    atomicAdd((unsigned long long *)&A.nobj[p], (unsigned long long)cnt);
    atomicAdd((unsigned long long *)&A.counters[CNT_HUGE_COBJS], (unsigned long long)cnt);
    const uint64_t pos = atomicAdd((unsigned long long *)&A.counters[S.pass_slot], 1ull);
    S.plist[pos] = t;
    if (cnt > (uint32_t)A.mid_max)
        atomicAdd((unsigned long long *)&A.counters[CNT_NEXT_HUGE], 1ull);
    else if (cnt > (uint32_t)kSmallMax)
        atomicAdd((unsigned long long *)&A.counters[CNT_NEXT_MID], 1ull);
}

// Rank of attribute j among the passing attributes of huge parent bi.
template <int WMC>
__device__ __forceinline__ int pass_rank(const LevelArgs &A, uint64_t bi, int j)
{
    const int wj = j >> 6, bj = j & 63;
    int rank = 0;
#pragma unroll
    for (int u = 0; u < WMC; ++u) {
        if (u < words_of<WMC>(A.wm) && u <= wj) {
            const uint64_t pm = A.pass[bi * A.wm + u];
            rank += __popcll(u < wj ? pm : (pm & below_mask(bj)));
        }
    }
    return rank;
}

// --- list scan (any N): the parent's object list is read 256 entries a step -----

// Scan the extent list of a big parent for the objects having attribute j
// (their bit in col[j]), four 64-entry chunks per step so the loads overlap.
// Calls f(in, g, chunk_ballot) per chunk in list order.
template <typename F>
__device__ __forceinline__ void scan_list_for_attr(const LevelArgs &A, uint64_t o0, uint64_t o1, int j, F f)
{
    const int lane = lane_id();
    const uint64_t *col = A.cols + (uint64_t)j * A.wn;
    for (uint64_t o = o0; o < o1; o += 4 * kWave) {
        uint32_t g[4];
        bool in[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint64_t idx = o + (uint64_t)(s * kWave + lane);
            g[s] = idx < o1 ? A.objs[idx] : 0xFFFFFFFFu;
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) in[s] = g[s] != 0xFFFFFFFFu && ((col[g[s] >> 6] >> (g[s] & 63)) & 1ull);
#pragma unroll
        for (int s = 0; s < 4; ++s) f(in[s], g[s], __ballot(in[s]));
    }
}

// --- mid parents (64 < |A| <= mid_max): closure tests by incidence ------------
//
// For a parent (A, B, y) let J be the attributes outside B above y, and U the
// members of J carried by some object of A.  Every incidence (object g of A,
// attribute j in U that g has) ANDs row g into D_j and counts g into |C_j|,
// with one D_j per member of U kept in LDS.  C_j is then exactly the objects of
// A having j, D_j = C_j' (page 1, sections 2.1 and 4.2), and the canonical test
// of j reads D_j (page 1, section 4.3).  Work per parent is the number of
// incidences, not candidates x |A|.  A candidate of J outside U has C = {} and
// D = M, so only the first attribute not in B can pass that way (the bottom).
//
// Passing children are emitted as records of 4 + wm words:
//   [0] parent | j << 32, [1] sibling rank | |C| << 32, [2] object offset of
//   the child's list inside the parent's children, [3] the objects of C as a
//   mask over the parent's list (local parents only, else 0), [4..] D.
//
// A wavefront keeps the D of kMidCand members of U at a time (small tables,
// so that many wavefronts fit a compute unit); a parent with more members is
// tested a slice of U per pass over its list.  Records are reserved per round
// of 64 tests and carry their rank and object offset.

template <int WMC>
__global__ void __launch_bounds__(kWave * kMidWaves) k_mid_test(LevelArgs A)
{
    __shared__ uint64_t s_d[kMidWaves][kMidCand * WMC];
    __shared__ uint32_t s_c[kMidWaves][kMidCand];
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = words_of<WMC>(A.wm);
    uint64_t *Dt = s_d[wv];
    uint32_t *Ct = s_c[wv];
    uint32_t next_mid = 0;
    bool overflow = false;
    const int stripe = (int)(((uint64_t)blockIdx.x * kMidWaves + wv) % kRecStripes);
    const uint64_t count = A.counters[CNT_MID];
    const uint64_t rstride = 4 + (uint64_t)A.wm;
    auto reserve = [&](uint32_t n) -> uint64_t {  // record slots, uniform
        uint64_t base = 0;
        if (lane == 0) base = atomicAdd((unsigned long long *)&A.counters[CNT_MIDREC + stripe * kCntPad], (unsigned long long)n);
        base = uniform64(base);
        if (base + n > A.mrec_region) overflow = true;
        return (uint64_t)stripe * A.mrec_region + base;
    };
    const uint64_t rhi = (uint64_t)(stripe + 1) * A.mrec_region;
    for (uint64_t it = (uint64_t)blockIdx.x * kMidWaves + wv; it < count; it += (uint64_t)gridDim.x * kMidWaves) {
        const uint64_t p = A.mid_idx[it];
        const uint64_t c0 = A.lo + p;
        const uint64_t o0 = A.loff[c0], o1 = A.loff[c0 + 1];
        const int y = A.cursor[c0];
        uint64_t Bx[WMC];
#pragma unroll
        for (int u = 0; u < WMC; ++u) {
            Bx[u] = ~0ull;
            if (u < wm) {
                Bx[u] = A.intents[c0 * A.wm + u];
                if (u == wm - 1) Bx[u] |= ~A.tail_m;
            }
        }
        // the parent's object ids, 64 a step, loaded together once (lanes past
        // the list take the zero row after the last object); then all their
        // rows for U at once, so a parent waits for two loads, not two per step
        constexpr int kSteps = kMidWide / kWave;
        const int nsteps = (int)((o1 - o0 + kWave - 1) / kWave);
        uint32_t ids[kSteps];
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
            const uint64_t o = o0 + (uint64_t)(st * kWave + lane);
            ids[st] = (st < nsteps && o < o1) ? A.objs[o] : (uint32_t)A.n;
        }
        uint64_t U[WMC];
#pragma unroll
        for (int u = 0; u < WMC; ++u) U[u] = 0;
#pragma unroll
        for (int st = 0; st < kSteps; ++st)
            if (st < nsteps)
#pragma unroll
                for (int u = 0; u < WMC; ++u)
                    if (u < wm) U[u] |= A.rows[(uint64_t)ids[st] * A.wm + u];
        int nU = 0, j0 = -1;
        int pre[WMC];
#pragma unroll
        for (int u = 0; u < WMC; ++u) {
            pre[u] = nU;
            if (u < wm) {
                const uint64_t nb = ~Bx[u];
                if (j0 < 0 && nb) j0 = 64 * u + __ffsll((unsigned long long)nb) - 1;
                U[u] = wave_or(U[u]) & nb & above_mask(y, u);
                nU += __popcll(U[u]);
            }
        }
        bool bottom = false;
        if (j0 > y) {
            bottom = true;
#pragma unroll
            for (int u = 0; u < WMC; ++u)
                if (u == (j0 >> 6) && ((U[u] >> (j0 & 63)) & 1ull)) bottom = false;
        }
        uint32_t rank = 0, objoff = 0;
        if (bottom) {
            const uint64_t at = reserve(1);
            if (lane == 0 && at < rhi) {
                uint64_t *rec = A.mrec + at * rstride;
                rec[0] = p | ((uint64_t)j0 << 32);
                rec[1] = 0;
                rec[2] = 0;
                rec[3] = 0;
                for (int u = 0; u < wm; ++u) rec[4 + u] = (u == wm - 1) ? A.tail_m : ~0ull;
            }
            rank = 1;
        }
        for (int lo = 0; lo < nU; lo += kMidCand) {
            const int nc = nU - lo < kMidCand ? nU - lo : kMidCand;
            uint64_t Us[WMC];
#pragma unroll
            for (int u = 0; u < WMC; ++u) {
                Us[u] = 0;
                if (u < wm) {
                    const int cu = __popcll(U[u]);
                    const int klo = lo - pre[u], khi = lo + nc - pre[u];
                    if (klo < cu && khi > 0) {
                        uint64_t m = U[u];
                        if (klo > 0) m &= ~below_mask(select64(U[u], klo));
                        if (khi < cu) m &= below_mask(select64(U[u], khi));
                        Us[u] = m;
                    }
                }
            }
            for (int x = lane; x < nc * WMC; x += kWave) Dt[x] = ~0ull;
            for (int x = lane; x < nc; x += kWave) Ct[x] = 0;
            wave_sync();
            // incidences, a step of 64 objects at a time; the next step's rows
            // are loaded while this step's incidences run
            uint64_t row[WMC];
#pragma unroll
            for (int u = 0; u < WMC; ++u) row[u] = (u < wm) ? A.rows[(uint64_t)ids[0] * A.wm + u] : 0ull;
#pragma unroll
            for (int st = 0; st < kSteps; ++st) {
                if (st >= nsteps) break;
                uint64_t nxt[WMC];
#pragma unroll
                for (int u = 0; u < WMC; ++u)
                    nxt[u] = (st + 1 < kSteps && st + 1 < nsteps && u < wm)
                                 ? A.rows[(uint64_t)ids[st + 1 < kSteps ? st + 1 : st] * A.wm + u]
                                 : 0ull;
#pragma unroll
                for (int u = 0; u < WMC; ++u) {
                    uint64_t x = row[u] & Us[u];
                    while (x) {
                        const int b = __ffsll((unsigned long long)x) - 1;
                        x &= x - 1ull;
                        const int r = pre[u] + __popcll(U[u] & below_mask(b)) - lo;
#pragma unroll
                        for (int v = 0; v < WMC; ++v)
                            if (v < wm) atomicAnd((unsigned long long *)&Dt[r * WMC + v], (unsigned long long)row[v]);
                        atomicAdd(&Ct[r], 1u);
                    }
                }
#pragma unroll
                for (int u = 0; u < WMC; ++u) row[u] = nxt[u];
            }
            wave_sync();
            for (int r0 = 0; r0 < nc; r0 += kWave) {
                const int rl = r0 + lane;
                const bool active = rl < nc;
                const int j = active ? select_words<WMC>(U, wm, lo + rl) : 0;
                const int wj = j >> 6, bj = j & 63;
                uint64_t bad = 0;
                if (active) {
#pragma unroll
                    for (int u = 0; u < WMC; ++u) {
                        if (u < wm && u <= wj) {
                            const uint64_t extra = Dt[rl * WMC + u] & ~Bx[u];
                            bad |= (u < wj) ? extra : (extra & below_mask(bj));
                        }
                    }
                }
                const bool pass = active && bad == 0;
                const uint32_t cnt = pass ? Ct[rl] : 0u;
                next_mid += (uint32_t)__popcll(__ballot(pass && cnt > (uint32_t)kSmallMax));
                const uint64_t bal = __ballot(pass);
                if (!bal) continue;
                const uint32_t np = (uint32_t)__popcll(bal);
                const uint64_t base = reserve(np);
                const uint32_t before = (uint32_t)__popcll(bal & below_mask(lane));
                const uint32_t off = objoff + wave_excl_scan(cnt);
                if (pass && base + before < rhi) {
                    uint64_t *rec = A.mrec + (base + before) * rstride;
                    rec[0] = p | ((uint64_t)j << 32);
                    rec[1] = (uint64_t)(rank + before) | ((uint64_t)cnt << 32);
                    rec[2] = off;
                    rec[3] = 0;
#pragma unroll
                    for (int u = 0; u < WMC; ++u)
                        if (u < wm) rec[4 + u] = (u == wm - 1) ? (Dt[rl * WMC + u] & A.tail_m) : Dt[rl * WMC + u];
                }
                rank += np;
                objoff += wave_sum(cnt);
            }
            wave_sync();
        }
        if (lane == 0) {
            A.nchild[p] = rank;
            A.nobj[p] = objoff;
        }
    }
    if (overflow && lane == 0) A.counters[CNT_OVERFLOW] = 1;
    if (next_mid && lane == 0) atomicAdd((unsigned long long *)&A.counters[CNT_NEXT_MID], (unsigned long long)next_mid);
}

// Wide mid parents (more than kMidWide objects): the same incidence method with
// one workgroup per parent.  Its wavefronts split the object list and share one
// D table (LDS atomics are atomic across the workgroup), so the longest parent
// no longer sets the length of the launch; every candidate of U then gets a
// thread of its own for the canonical test, and ranks and object offsets come
// from a workgroup scan.  Records as in k_mid_test, one block per parent.
template <int WMC>
__global__ void __launch_bounds__(kWideThreads) k_mid_test_wide(LevelArgs A)
{
    constexpr int kMaxCand = kWave * WMC;
    static_assert(kMaxCand <= kWideThreads, "one thread per candidate");
    __shared__ uint64_t s_d[kMaxCand * WMC];
    __shared__ uint32_t s_c[kMaxCand];
    __shared__ uint64_t s_u[WMC];
    __shared__ uint32_t s_wsum[2][kWideWaves];  // per wavefront: passing tests, their objects
    __shared__ uint64_t s_base;
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int tid = (int)threadIdx.x;
    const int wm = words_of<WMC>(A.wm);
    uint32_t next_mid = 0;
    const uint64_t count = A.counters[CNT_MIDW];
    const uint64_t rstride = 4 + (uint64_t)A.wm;
    for (uint64_t it = blockIdx.x; it < count; it += gridDim.x) {
        const uint64_t p = A.mid_idx[A.P - 1 - it];
        const uint64_t c0 = A.lo + p;
        const uint64_t o0 = A.loff[c0], o1 = A.loff[c0 + 1];
        const int y = A.cursor[c0];
        uint64_t Bx[WMC];
#pragma unroll
        for (int u = 0; u < WMC; ++u) {
            Bx[u] = ~0ull;
            if (u < wm) {
                Bx[u] = A.intents[c0 * A.wm + u];
                if (u == wm - 1) Bx[u] |= ~A.tail_m;
            }
        }
        if (tid < WMC) s_u[tid] = 0;
        __syncthreads();
        // U: candidates carried by some object of A
        // the parent's object ids, kWideThreads a step, loaded together once
        // (threads past the list take the zero row after the last object)
        constexpr int kSteps = kMidMax / kWideThreads;
        const int nsteps = (int)((o1 - o0 + kWideThreads - 1) / kWideThreads);
        uint32_t ids[kSteps];
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
            const uint64_t o = o0 + (uint64_t)(st * kWideThreads + tid);
            ids[st] = (st < nsteps && o < o1) ? A.objs[o] : (uint32_t)A.n;
        }
        uint64_t U[WMC];
#pragma unroll
        for (int u = 0; u < WMC; ++u) U[u] = 0;
#pragma unroll
        for (int st = 0; st < kSteps; ++st)
            if (st < nsteps)
#pragma unroll
                for (int u = 0; u < WMC; ++u)
                    if (u < wm) U[u] |= A.rows[(uint64_t)ids[st] * A.wm + u];
#pragma unroll
        for (int u = 0; u < WMC; ++u) {
            if (u < wm) {
                const uint64_t v = wave_or(U[u]);
                if (lane == 0 && v) atomicOr((unsigned long long *)&s_u[u], (unsigned long long)v);
            }
        }
        __syncthreads();
        int nU = 0, j0 = -1;
        int pre[WMC];  // members of U in the words before u
#pragma unroll
        for (int u = 0; u < WMC; ++u) {
            pre[u] = nU;
            U[u] = 0;
            if (u < wm) {
                const uint64_t nb = ~Bx[u];
                if (j0 < 0 && nb) j0 = 64 * u + __ffsll((unsigned long long)nb) - 1;
                U[u] = s_u[u] & nb & above_mask(y, u);
                nU += __popcll(U[u]);
            }
        }
        for (int x = tid; x < nU * WMC; x += kWideThreads) s_d[x] = ~0ull;
        for (int x = tid; x < nU; x += kWideThreads) s_c[x] = 0;
        __syncthreads();
        // incidences, a step at a time, the next step's rows loaded meanwhile
        uint64_t row[WMC];
#pragma unroll
        for (int u = 0; u < WMC; ++u) row[u] = (u < wm) ? A.rows[(uint64_t)ids[0] * A.wm + u] : 0ull;
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
            if (st >= nsteps) break;
            uint64_t nxt[WMC];
#pragma unroll
            for (int u = 0; u < WMC; ++u)
                nxt[u] = (st + 1 < kSteps && st + 1 < nsteps && u < wm)
                             ? A.rows[(uint64_t)ids[st + 1 < kSteps ? st + 1 : st] * A.wm + u]
                             : 0ull;
#pragma unroll
            for (int u = 0; u < WMC; ++u) {
                uint64_t x = row[u] & U[u];
                while (x) {
                    const int b = __ffsll((unsigned long long)x) - 1;
                    x &= x - 1ull;
                    const int r = pre[u] + __popcll(U[u] & below_mask(b));
#pragma unroll
                    for (int v = 0; v < WMC; ++v)
                        if (v < wm) atomicAnd((unsigned long long *)&s_d[r * WMC + v], (unsigned long long)row[v]);
                    atomicAdd(&s_c[r], 1u);
                }
            }
#pragma unroll
            for (int u = 0; u < WMC; ++u) row[u] = nxt[u];
        }
        __syncthreads();
        // the first attribute outside B, carried by no object: C = {}, D = M, rank 0
        bool bottom = false;
        if (j0 > y) {
            bottom = true;
#pragma unroll
            for (int u = 0; u < WMC; ++u)
                if (u == (j0 >> 6) && ((U[u] >> (j0 & 63)) & 1ull)) bottom = false;
        }
        // canonical tests: thread r takes member r of U (ascending j)
        const int r = tid;
        const bool active = r < nU;
        const int j = active ? select_words<WMC>(U, wm, r) : 0;
        const int wj = j >> 6, bj = j & 63;
        uint64_t bad = 0;
        if (active) {
#pragma unroll
            for (int u = 0; u < WMC; ++u) {
                if (u < wm && u <= wj) {
                    const uint64_t extra = s_d[r * WMC + u] & ~Bx[u];
                    bad |= (u < wj) ? extra : (extra & below_mask(bj));
                }
            }
        }
        const bool pass = active && bad == 0;
        const uint32_t cnt = pass ? s_c[r] : 0u;
        const uint64_t bal = __ballot(pass);
        next_mid += (uint32_t)__popcll(__ballot(pass && cnt > (uint32_t)kSmallMax));
        const uint32_t before = (uint32_t)__popcll(bal & below_mask(lane));
        const uint32_t ex = wave_excl_scan(cnt);
        const uint32_t wobj = wave_sum(cnt);
        if (lane == 0) {
            s_wsum[0][wv] = (uint32_t)__popcll(bal);
            s_wsum[1][wv] = wobj;
        }
        __syncthreads();
        uint32_t pbase = bottom ? 1u : 0u, obase = 0, npass = pbase, nobj = 0;
        for (int w = 0; w < kWideWaves; ++w) {
            const uint32_t a = s_wsum[0][w], o = s_wsum[1][w];
            if (w < wv) {
                pbase += a;
                obase += o;
            }
            npass += a;
            nobj += o;
        }
        if (tid == 0) {
            // (one counter: a level has a few thousand wide parents at most)
            uint64_t base = 0;
            if (npass) base = atomicAdd((unsigned long long *)&A.counters[CNT_WIDEREC], (unsigned long long)npass);
            if (base + npass > A.wrec_cap) {
                A.counters[CNT_OVERFLOW] = 1;
                base = ~0ull;  // nothing is written
            }
            s_base = base;
            A.nchild[p] = npass;
            A.nobj[p] = nobj;
        }
        __syncthreads();
        const uint64_t base = s_base;
        if (base != ~0ull) {
            if (bottom && tid == 0) {
                uint64_t *rec = A.wrec + base * rstride;
                rec[0] = p | ((uint64_t)j0 << 32);
                rec[1] = 0;
                rec[2] = 0;
                rec[3] = 0;
                for (int u = 0; u < wm; ++u) rec[4 + u] = (u == wm - 1) ? A.tail_m : ~0ull;
            }
            if (pass) {
                const uint32_t rank = pbase + before;
                uint64_t *rec = A.wrec + (base + rank) * rstride;
                rec[0] = p | ((uint64_t)j << 32);
                rec[1] = (uint64_t)rank | ((uint64_t)cnt << 32);
                rec[2] = obase + ex;
                rec[3] = 0;
#pragma unroll
                for (int u = 0; u < WMC; ++u)
                    if (u < wm) rec[4 + u] = (u == wm - 1) ? (s_d[r * WMC + u] & A.tail_m) : s_d[r * WMC + u];
            }
        }
        __syncthreads();  // the table, s_u and s_base are reused by the next parent
    }
    if (next_mid && lane == 0) atomicAdd((unsigned long long *)&A.counters[CNT_NEXT_MID], (unsigned long long)next_mid);
}

constexpr int kMidRun = 16;  // records per item of the narrow mid writer (4, 8, 16, 32: ctx20000x256 writer 18.1, 13.7, 12.1, 11.9 ms)
constexpr int kWideRun = 4;  // of the wide one (1, 2, 4, 8 records: ctx50000x400 level loop 5.06, 4.69, 4.56, 4.63 ms)

// One item of the mid parents' child records: nr <= kMidRun consecutive
// records at rec0 (a parent's records are consecutive, in rank order).  Their
// intents, cursors and list bounds come from the records, and every run of
// records with the same parent shares one pass over the parent's object list,
// in which each object's row is read once per needed intent word and tested
// for the attribute j of every record of the run (the objects of C_j,
// ascending).
template <int WMC>
__device__ __forceinline__ void mid_write_item(const LevelArgs &A, const uint64_t *rec0, int nr)
{
    const int lane = lane_id();
    const int wm = words_of<WMC>(A.wm);
    const uint64_t rstride = 4 + (uint64_t)A.wm;
    // lane r < nr: record r's header, child and list start
    uint64_t w0 = 0, w1 = 0, w2 = 0;
    if (lane < nr) {
        const uint64_t *rec = rec0 + (uint64_t)lane * rstride;
        w0 = rec[0];
        w1 = rec[1];
        w2 = rec[2];
    }
    const uint64_t pl = w0 & 0xFFFFFFFFull;
    uint64_t child = 0, qo = 0;
    if (lane < nr) {
        child = A.child_lo + A.cbase[pl] + (w1 & 0xFFFFFFFFull);
        qo = A.child_obj_lo + A.obase[pl] + w2;
    }
    // intents: one lane per (record, word)
    for (int x0 = 0; x0 < nr * wm; x0 += kWave) {
        const int x = x0 + lane;
        int r = x / wm;
        r = r < nr ? r : nr - 1;
        const uint64_t ch = __shfl(child, r);
        if (x < nr * wm) A.intents[ch * A.wm + (x - r * wm)] = rec0[(uint64_t)r * rstride + 4 + (x - r * wm)];
    }
    if (lane < nr) {
        const uint32_t cnt = (uint32_t)(w1 >> 32);
        A.cursor[child] = (int32_t)(w0 >> 32);
        A.loff[child] = qo;
        A.loff[child + 1] = qo + cnt;
    }
    // extent lists, one pass over each parent's list per run of records
    for (int r = 0; r < nr;) {
        const uint64_t p = lane_value64(w0, r) & 0xFFFFFFFFull;
        int r1 = r + 1;
        while (r1 < nr && (lane_value64(w0, r1) & 0xFFFFFFFFull) == p) ++r1;
        const uint64_t c0 = A.lo + p;
        const uint64_t l0 = A.loff[c0], l1 = A.loff[c0 + 1];
        // intent words holding the attributes of the run (C non-empty)
        uint32_t need = 0;
        for (int ri = r; ri < r1; ++ri)
            if ((lane_value64(w1, ri) >> 32) != 0) need |= 1u << ((lane_value64(w0, ri) >> 32) >> 6);
        // four chunks of 64 objects per step, so that their loads overlap;
        // per needed intent word, that word of the four rows, then the
        // records whose attribute lies in it (each record's objects still
        // come out in list order)
        for (uint64_t o = l0; o < l1; o += 4 * kWave) {
            uint32_t g[4];
            bool valid[4];
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const uint64_t idx = o + (uint64_t)(c4 * kWave + lane);
                valid[c4] = idx < l1;
                g[c4] = valid[c4] ? A.objs[idx] : 0u;
            }
            for (uint32_t nm = need; nm; nm &= nm - 1u) {
                const int u = __ffs(nm) - 1;
                uint64_t row[4];
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) row[c4] = valid[c4] ? A.rows[(uint64_t)g[c4] * A.wm + u] : 0ull;
                for (int ri = r; ri < r1; ++ri) {
                    if ((lane_value64(w1, ri) >> 32) == 0) continue;  // C empty (the bottom child)
                    const int j = (int)(lane_value64(w0, ri) >> 32);
                    if ((j >> 6) != u) continue;
#pragma unroll
                    for (int c4 = 0; c4 < 4; ++c4) {
                        const bool in = (row[c4] >> (j & 63)) & 1ull;
                        const uint64_t bal = __ballot(in);
                        const uint64_t at = lane_value64(qo, ri);
                        if (in) A.objs[at + __popcll(bal & below_mask(lane))] = g[c4];
                        if (lane == ri) qo += (uint64_t)__popcll(bal);
                    }
                }
            }
        }
        r = r1;
    }
}

// Children of the narrow mid parents: a wavefront takes kMidRun consecutive
// records of a stripe at a time (mid_write_item).
template <int WMC>
__global__ void __launch_bounds__(kBlock) k_mid_write(LevelArgs A)
{
    const int lane = lane_id();
    if (A.counters[CNT_OVERFLOW] || !store_has_room(A)) return;
    const uint64_t rstride = 4 + (uint64_t)A.wm;
    const uint64_t nw = (uint64_t)gridDim.x * kWavesPerBlock;
    const uint64_t w = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
    // the stripe counts, one per lane, loaded together
    const uint64_t counts = lane < kRecStripes ? A.counters[CNT_MIDREC + lane * kCntPad] : 0ull;
    uint64_t kmax = 0;
    for (int st = 0; st < kRecStripes; ++st) kmax = max(kmax, lane_value64(counts, st));
    // Items of kMidRun records, walked interleaved over the stripes (item i of
    // every stripe before item i + 1 of any: roughly the order of reservation).
    const uint64_t items = (kmax + kMidRun - 1) / kMidRun;
    for (uint64_t f = w; f < items * kRecStripes; f += nw) {
        const int st = __builtin_amdgcn_readfirstlane((int)(f % kRecStripes));  // f is per wavefront
        const uint64_t k0 = (f / kRecStripes) * kMidRun;
        const uint64_t nst = lane_value64(counts, st);
        if (k0 >= nst) continue;
        const int nr = (int)(nst - k0 < (uint64_t)kMidRun ? nst - k0 : (uint64_t)kMidRun);
        mid_write_item<WMC>(A, A.mrec + ((uint64_t)st * A.mrec_region + k0) * rstride, nr);
    }
}

// Children of the wide mid parents: their records (one block of consecutive
// records per parent, in rank order) taken kWideRun at a time as in k_mid_write,
// so the records of a parent share the passes over its long list.
template <int WMC>
__global__ void __launch_bounds__(kBlock) k_mid_write_wide(LevelArgs A)
{
    if (A.counters[CNT_OVERFLOW] || !store_has_room(A)) return;
    const uint64_t nrec = A.counters[CNT_WIDEREC];
    const uint64_t rstride = 4 + (uint64_t)A.wm;
    const uint64_t items = (nrec + kWideRun - 1) / kWideRun;
    for (uint64_t f = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; f < items;
         f += (uint64_t)gridDim.x * kWavesPerBlock) {
        const uint64_t k0 = f * kWideRun;
        const int nr = (int)(nrec - k0 < (uint64_t)kWideRun ? nrec - k0 : (uint64_t)kWideRun);
        mid_write_item<WMC>(A, A.wrec + k0 * rstride, nr);
    }
}

// Closure tests of huge parents through their object lists, one wavefront per
// task: an object is in C when its bit in col[j] is set, and its row is ANDed
// into the lane's partial D (page 1, section 4.2: the extent's set bits are
// walked, rows ANDed, then a wavefront AND-reduction).
template <int WMC>
__global__ void __launch_bounds__(kBlock) k_big_test_list(LevelArgs A)
{
    const BigSet &S = A.huge;
    const int lane = lane_id();
    const int wm = words_of<WMC>(A.wm);
    if (A.counters[CNT_OVERFLOW]) return;
    const uint64_t tset = S.off[A.counters[S.cnt_slot]];
    for (uint64_t t = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; t < tset;
         t += (uint64_t)gridDim.x * kWavesPerBlock) {
        const uint64_t task = S.tasks[t];
        const uint64_t bi = task >> 16;
        const int j = (int)(task & 0xFFFFu);
        const uint64_t p = S.idx[bi];
        const uint64_t c0 = A.lo + p;
        const int wj = j >> 6, bj = j & 63;
        uint64_t D[WMC];
#pragma unroll
        for (int u = 0; u < WMC; ++u) D[u] = ~0ull;
        uint32_t cnt = 0;
        scan_list_for_attr(A, A.loff[c0], A.loff[c0 + 1], j, [&](bool in, uint32_t g, uint64_t bal) {
            cnt += (uint32_t)__popcll(bal);
            if (in) {
#pragma unroll
                for (int u = 0; u < WMC; ++u)
                    if (u < wm) D[u] &= A.rows[(uint64_t)g * A.wm + u];
            }
        });
        uint64_t bad = 0;
#pragma unroll
        for (int u = 0; u < WMC; ++u) {
            if (u < wm && u <= wj) {
                uint64_t bx = A.intents[c0 * A.wm + u];
                if (u == wm - 1) bx |= ~A.tail_m;
                const uint64_t extra = wave_and(D[u]) & ~bx;
                bad |= (u < wj) ? extra : (extra & below_mask(bj));
            }
        }
        const bool pass = bad == 0;
        if (lane == 0) {
            S.size[t] = pass ? cnt : 0u;
            if (pass) big_record_pass(A, S, t, bi, p, j, cnt);
        }
    }
}

// Children of huge parents through their object lists, one wavefront per
// passing task.  The child's rank among its siblings is the number of passing
// attributes below j; its list offset comes from the scan of the passing
// tasks' |C|.
template <int WMC>
__global__ void __launch_bounds__(kBlock) k_big_write_list(LevelArgs A)
{
    const BigSet &S = A.huge;
    const int lane = lane_id();
    const int wm = words_of<WMC>(A.wm);
    if (A.counters[CNT_OVERFLOW] || !store_has_room(A)) return;
    const uint64_t npass = A.counters[S.pass_slot];
    for (uint64_t i = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; i < npass;
         i += (uint64_t)gridDim.x * kWavesPerBlock) {
        const uint64_t t = S.plist[i];
        const uint64_t task = S.tasks[t];
        const uint64_t bi = task >> 16;
        const int j = (int)(task & 0xFFFFu);
        const uint64_t p = S.idx[bi];
        const uint64_t c0 = A.lo + p;
        const uint64_t child = A.child_lo + A.cbase[p] + (uint64_t)pass_rank<WMC>(A, bi, j);
        const uint64_t obeg = A.child_obj_lo + A.obase[p] + (S.sscan[t] - S.sscan[S.off[bi]]);
        uint64_t D[WMC];
#pragma unroll
        for (int u = 0; u < WMC; ++u) D[u] = ~0ull;
        uint64_t qo = obeg;
        scan_list_for_attr(A, A.loff[c0], A.loff[c0 + 1], j, [&](bool in, uint32_t g, uint64_t bal) {
            if (in) {
                A.objs[qo + __popcll(bal & below_mask(lane))] = g;
#pragma unroll
                for (int u = 0; u < WMC; ++u)
                    if (u < wm) D[u] &= A.rows[(uint64_t)g * A.wm + u];
            }
            qo += __popcll(bal);
        });
#pragma unroll
        for (int u = 0; u < WMC; ++u) {
            if (u < wm) {
                uint64_t d = wave_and(D[u]);
                if (u == wm - 1) d &= A.tail_m;
                if (lane == 0) A.intents[child * A.wm + u] = d;
            }
        }
        if (lane == 0) {
            A.cursor[child] = j;
            A.loff[child] = obeg;
            A.loff[child + 1] = qo;
        }
    }
}

// --- extent bitmaps, one work item per (test, 64-word chunk) (huge set) ------------
//
// A closure test of a huge parent is split over the 64-word chunks of the
// extent bitmap: each item forms its part of C = A AND col[j] with one
// coalesced load per lane, ANDs the rows of its objects and folds the partial
// D and |C| into the test's accumulators.  Every item is short, so levels with
// a handful of huge parents (the root: every object) still fill the chip.

template <int WMC>
__global__ void __launch_bounds__(kBlock) k_huge_partial(LevelArgs A)
{
    const BigSet &S = A.huge;
    const int lane = lane_id();
    const int wm = words_of<WMC>(A.wm);
    if (A.counters[CNT_OVERFLOW]) return;
    const uint64_t items = S.off[A.counters[S.cnt_slot]] * (uint64_t)A.nchunk;
    for (uint64_t it = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; it < items;
         it += (uint64_t)gridDim.x * kWavesPerBlock) {
        const uint64_t t = it / (uint64_t)A.nchunk;
        const int k = (int)(it - t * (uint64_t)A.nchunk);
        const uint64_t task = S.tasks[t];
        const uint64_t bi = task >> 16;
        const int j = (int)(task & 0xFFFFu);
        const int w = kWave * k + lane;
        uint64_t c = 0;
        if (w < A.wn) c = S.bmp[bi * (uint64_t)A.wn + w] & A.cols[(uint64_t)j * A.wn + w];
        const uint32_t tot = wave_sum((uint32_t)__popcll(c));
        if (lane == 0) A.icnt[it] = tot;
        if (tot == 0) continue;
        uint64_t D[WMC];
#pragma unroll
        for (int u = 0; u < WMC; ++u) D[u] = ~0ull;
        const uint64_t base = (uint64_t)w * 64;
        while (c) {
            const uint64_t g0 = base + (uint64_t)(__ffsll((unsigned long long)c) - 1);
            c &= c - 1ull;
            uint64_t g1 = g0;
            if (c) {
                g1 = base + (uint64_t)(__ffsll((unsigned long long)c) - 1);
                c &= c - 1ull;
            }
#pragma unroll
            for (int u = 0; u < WMC; ++u)
                if (u < wm) D[u] &= A.rows[g0 * A.wm + u] & A.rows[g1 * A.wm + u];
        }
#pragma unroll
        for (int u = 0; u < WMC; ++u) {
            if (u < wm) {
                const uint64_t d = wave_and(D[u]);
                if (lane == 0 && d != ~0ull) atomicAnd((unsigned long long *)&A.dt[t * A.wm + u], (unsigned long long)d);
            }
        }
        if (lane == 0) atomicAdd(&A.tcnt[t], tot);
    }
}

// One thread per huge test: the canonical test on the accumulated D (all of M
// when C is empty); a passing test turns its chunk counts into offsets inside
// the child's list.
__global__ void __launch_bounds__(kBlock) k_huge_finalize(LevelArgs A)
{
    const BigSet &S = A.huge;
    if (A.counters[CNT_OVERFLOW]) return;
    const uint64_t tset = S.off[A.counters[S.cnt_slot]];
    for (uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; t < tset; t += (uint64_t)gridDim.x * blockDim.x) {
        const uint64_t task = S.tasks[t];
        const uint64_t bi = task >> 16;
        const int j = (int)(task & 0xFFFFu);
        const uint64_t p = S.idx[bi];
        const uint64_t c0 = A.lo + p;
        const int wj = j >> 6, bj = j & 63;
        uint64_t bad = 0;
        for (int u = 0; u <= wj; ++u) {
            uint64_t bx = A.intents[c0 * A.wm + u];
            if (u == A.wm - 1) bx |= ~A.tail_m;
            const uint64_t extra = A.dt[t * A.wm + u] & ~bx;
            bad |= (u < wj) ? extra : (extra & below_mask(bj));
        }
        const uint32_t cnt = A.tcnt[t];
        const bool pass = bad == 0;
        S.size[t] = pass ? cnt : 0u;
        if (!pass) continue;
        big_record_pass(A, S, t, bi, p, j, cnt);
        uint32_t run = 0;
        for (int k = 0; k < A.nchunk; ++k) {
            const uint32_t v = A.icnt[t * A.nchunk + k];
            A.icnt[t * A.nchunk + k] = run;
            run += v;
        }
    }
}

// Children of huge parents, one item per (passing test, chunk): the chunk's
// objects go to their place in the child's list (ascending); chunk 0 also
// writes the intent (the accumulated D), cursor and list bounds.
template <int WMC>
__global__ void __launch_bounds__(kBlock) k_huge_write(LevelArgs A)
{
    const BigSet &S = A.huge;
    const int lane = lane_id();
    if (A.counters[CNT_OVERFLOW] || !store_has_room(A)) return;
    const uint64_t items = A.counters[S.pass_slot] * (uint64_t)A.nchunk;
    for (uint64_t it = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; it < items;
         it += (uint64_t)gridDim.x * kWavesPerBlock) {
        const uint64_t pi = it / (uint64_t)A.nchunk;
        const int k = (int)(it - pi * (uint64_t)A.nchunk);
        const uint64_t t = S.plist[pi];
        const uint64_t task = S.tasks[t];
        const uint64_t bi = task >> 16;
        const int j = (int)(task & 0xFFFFu);
        const uint64_t p = S.idx[bi];
        const uint64_t obeg = A.child_obj_lo + A.obase[p] + (S.sscan[t] - S.sscan[S.off[bi]]);
        const int w = kWave * k + lane;
        uint64_t c = 0;
        if (w < A.wn) c = S.bmp[bi * (uint64_t)A.wn + w] & A.cols[(uint64_t)j * A.wn + w];
        uint64_t q = obeg + A.icnt[t * A.nchunk + k] + wave_excl_scan((uint32_t)__popcll(c));
        const uint32_t base = (uint32_t)w * 64u;
        while (c) {
            A.objs[q++] = base + (uint32_t)(__ffsll((unsigned long long)c) - 1);
            c &= c - 1ull;
        }
        if (k == 0 && lane == 0) {
            const uint64_t child = A.child_lo + A.cbase[p] + (uint64_t)pass_rank<WMC>(A, bi, j);
            for (int u = 0; u < A.wm; ++u) {
                uint64_t d = A.dt[t * A.wm + u];
                if (u == A.wm - 1) d &= A.tail_m;
                A.intents[child * A.wm + u] = d;
            }
            A.cursor[child] = j;
            A.loff[child] = obeg;
            A.loff[child + 1] = obeg + A.tcnt[t];
        }
    }
}

// ---------------------------------------------------------------------------
// exclusive scan of a u32 array (and optionally a u64 one) into u64 offsets, n read from the
// device (n_dev, clamped to n_cap) or given by the host (n_dev == nullptr).
// out[n] receives the total; *tot (optional) too.

__device__ __forceinline__ uint64_t scan_count(const uint64_t *n_dev, uint64_t n_host, uint64_t n_cap)
{
    uint64_t n = n_dev ? *n_dev : n_host;
    return n < n_cap ? n : n_cap;
}

__global__ void __launch_bounds__(kBlock) k_scan_up(const uint32_t *__restrict__ a, const uint64_t *__restrict__ b,
                                                     const uint64_t *n_dev, uint64_t n_host, uint64_t n_cap,
                                                     uint64_t *part)
{
    __shared__ uint64_t s_red[2][kWavesPerBlock];
    const uint64_t n = scan_count(n_dev, n_host, n_cap);
    const uint64_t per = (n + gridDim.x - 1) / gridDim.x;
    const uint64_t s = (uint64_t)blockIdx.x * per;
    const uint64_t e = s + per < n ? s + per : n;
    uint64_t sa = 0, sb = 0;
    for (uint64_t i = s + threadIdx.x; i < e; i += blockDim.x) {
        sa += a[i];
        if (b) sb += b[i];
    }
    sa = wave_sum64(sa);
    sb = wave_sum64(sb);
    if (lane_id() == 0) {
        s_red[0][threadIdx.x / kWave] = sa;
        s_red[1][threadIdx.x / kWave] = sb;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t ta = 0, tb = 0;
        for (int w = 0; w < kWavesPerBlock; ++w) {
            ta += s_red[0][w];
            tb += s_red[1][w];
        }
        part[blockIdx.x] = ta;
        part[kScanBlocks + blockIdx.x] = tb;
    }
}

// One block of kScanBlocks threads: exclusive scan of the block partials.
__global__ void __launch_bounds__(kScanBlocks) k_scan_mid(uint64_t *part, int nblocks, const uint64_t *n_dev,
                                                          uint64_t n_host, uint64_t n_cap, uint64_t *out_a,
                                                          uint64_t *out_b, uint64_t *tot_a, uint64_t *tot_b,
                                                          uint32_t *fch, uint64_t fbase)
{
    __shared__ uint64_t s_w[2][kScanBlocks / kWave];
    const int t = threadIdx.x, lane = lane_id(), wv = t / kWave;
    uint64_t va = t < nblocks ? part[t] : 0, vb = t < nblocks ? part[kScanBlocks + t] : 0;
    const uint64_t xa = wave_incl_scan64(va), xb = wave_incl_scan64(vb);
    if (lane == kWave - 1) {
        s_w[0][wv] = xa;
        s_w[1][wv] = xb;
    }
    __syncthreads();
    uint64_t ba = 0, bb = 0, ta = 0, tb = 0;
    for (int w = 0; w < kScanBlocks / kWave; ++w) {
        if (w < wv) {
            ba += s_w[0][w];
            bb += s_w[1][w];
        }
        ta += s_w[0][w];
        tb += s_w[1][w];
    }
    if (t < nblocks) {
        part[t] = ba + xa - va;
        part[kScanBlocks + t] = bb + xb - vb;
    }
    if (t == 0) {
        const uint64_t n = scan_count(n_dev, n_host, n_cap);
        out_a[n] = ta;
        if (out_b) out_b[n] = tb;
        if (tot_a) *tot_a = ta;
        if (tot_b) *tot_b = tb;
        if (fch) fch[n] = (uint32_t)(fbase + ta);
    }
}

__global__ void __launch_bounds__(kBlock) k_scan_down(const uint32_t *__restrict__ a, const uint64_t *__restrict__ b,
                                                       const uint64_t *n_dev, uint64_t n_host, uint64_t n_cap,
                                                       const uint64_t *part, uint64_t *out_a, uint64_t *out_b,
                                                       uint32_t *fch, uint64_t fbase)
{
    __shared__ uint64_t s_wave[kWavesPerBlock];
    const uint64_t n = scan_count(n_dev, n_host, n_cap);
    const uint64_t per = (n + gridDim.x - 1) / gridDim.x;
    const uint64_t s = (uint64_t)blockIdx.x * per;
    const uint64_t e = s + per < n ? s + per : n;
    uint64_t carry_a = part[blockIdx.x], carry_b = part[kScanBlocks + blockIdx.x];
    for (uint64_t base = s; base < e; base += blockDim.x) {
        const uint64_t i = base + threadIdx.x;
        const bool ok = i < e;
        uint64_t tot;
        const uint64_t xa = block_excl_scan(ok ? (uint64_t)a[i] : 0ull, s_wave, tot);
        if (ok) {
            out_a[i] = carry_a + xa;
            if (fch) fch[i] = (uint32_t)(fbase + carry_a + xa);
        }
        carry_a += tot;
        if (b) {
            const uint64_t xb = block_excl_scan(ok ? (uint64_t)b[i] : 0ull, s_wave, tot);
            if (ok) out_b[i] = carry_b + xb;
            carry_b += tot;
        }
    }
}

// The same scan in one workgroup of kScanBlocks threads, for short arrays
// whose length the host knows.
__global__ void __launch_bounds__(kScanBlocks) k_scan_small(const uint32_t *__restrict__ a,
                                                            const uint64_t *__restrict__ b, const uint64_t *n_dev,
                                                            uint64_t n_arg, uint64_t *out_a, uint64_t *out_b,
                                                            uint64_t *tot_a, uint64_t *tot_b, uint32_t *fch,
                                                            uint64_t fbase)
{
    // n_dev: the length in device memory, at most n_arg; else n_arg itself
    const uint64_t n = n_dev ? (*n_dev < n_arg ? *n_dev : n_arg) : n_arg;
    __shared__ uint64_t s_w[kScanBlocks / kWave];
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    auto block_scan = [&](uint64_t v, uint64_t &total) -> uint64_t {
        const uint64_t x = wave_incl_scan64(v);
        if (lane == kWave - 1) s_w[wv] = x;
        __syncthreads();
        uint64_t before = 0, all = 0;
        for (int w = 0; w < kScanBlocks / kWave; ++w) {
            const uint64_t sw = s_w[w];
            before += (w < wv) ? sw : 0ull;
            all += sw;
        }
        __syncthreads();
        total = all;
        return before + x - v;
    };
    uint64_t carry_a = 0, carry_b = 0;
    for (uint64_t base = 0; base < n; base += kScanBlocks) {
        const uint64_t i = base + threadIdx.x;
        const bool ok = i < n;
        uint64_t tot;
        const uint64_t xa = block_scan(ok ? (uint64_t)a[i] : 0ull, tot);
        if (ok) {
            out_a[i] = carry_a + xa;
            if (fch) fch[i] = (uint32_t)(fbase + carry_a + xa);
        }
        carry_a += tot;
        if (b) {
            const uint64_t xb = block_scan(ok ? (uint64_t)b[i] : 0ull, tot);
            if (ok) out_b[i] = carry_b + xb;
            carry_b += tot;
        }
    }
    if (threadIdx.x == 0) {
        out_a[n] = carry_a;
        if (out_b) out_b[n] = carry_b;
        if (tot_a) *tot_a = carry_a;
        if (tot_b) *tot_b = carry_b;
        if (fch) fch[n] = (uint32_t)(fbase + carry_a);
    }
}

// ---------------------------------------------------------------------------
// output order.  Concepts are listed in lexicographic order of the intent read
// as a bit string over attributes 0..M-1 (of two intents, the one holding the
// smallest attribute where they differ comes later; page 1, section 6.2 asks
// for a lexicographic intent key).  In the CbO tree this order is a pre-order
// walk that visits the children of a node by descending generating attribute:
//   * a child D of B (generated at j) agrees with B below j and holds j, which
//     B lacks, so it follows B;
//   * children D_j, D_k with j < k agree below j, and only D_j holds j, so D_j
//     follows D_k; every descendant of D_k agrees with D_k below k, so the
//     whole subtree of D_k precedes D_j.
// Hence the position of a concept is its parent's position, plus one, plus the
// subtree sizes of its siblings with a larger attribute.  Children of a concept
// are stored contiguously by ascending attribute, as [fchild[c], fchild[c+1]).

// Subtree sizes of the concepts [lo, lo + P); their children's sizes are final.
// With the task pool, desc (when given) adds the concepts the pool found below
// each task.
__global__ void __launch_bounds__(kBlock) k_subtree_size(const uint32_t *__restrict__ fchild, uint64_t lo,
                                                          uint64_t P, uint32_t *__restrict__ rank,
                                                          const uint32_t *__restrict__ desc)
{
    for (uint64_t p = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; p < P; p += (uint64_t)gridDim.x * blockDim.x) {
        const uint64_t c = lo + p;
        const uint32_t k0 = fchild[c], k1 = fchild[c + 1];
        uint32_t s = 1 + (desc ? desc[c] : 0u);
#pragma unroll 4
        for (uint32_t k = k0; k < k1; ++k) s += rank[k];
        rank[c] = s;
    }
}

// Positions of the children of the concepts [lo, lo + P), whose own positions
// are final (the root's is 0); a child's size is replaced by its position.
__global__ void __launch_bounds__(kBlock) k_child_position(const uint32_t *__restrict__ fchild, uint64_t lo,
                                                            uint64_t P, uint32_t *__restrict__ rank)
{
    for (uint64_t p = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; p < P; p += (uint64_t)gridDim.x * blockDim.x) {
        const uint64_t c = lo + p;
        const uint32_t k0 = fchild[c], k1 = fchild[c + 1];
        uint32_t run = (c == 0 ? 0u : rank[c]) + 1u;
        for (uint32_t k = k1; k > k0; --k) {
            const uint32_t sz = rank[k - 1];
            rank[k - 1] = run;
            run += sz;
        }
    }
}

// The same two passes for levels whose concepts have many children (the top
// of the tree): one wavefront per concept.  Sizes are summed across the
// lanes; positions come from an exclusive scan of the sizes taken in
// descending child order, 64 children a step.
__global__ void __launch_bounds__(kBlock) k_subtree_size_wave(const uint32_t *__restrict__ fchild, uint64_t lo,
                                                               uint64_t P, uint32_t *__restrict__ rank,
                                                               const uint32_t *__restrict__ desc)
{
    const int lane = lane_id();
    for (uint64_t p = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; p < P;
         p += (uint64_t)gridDim.x * kWavesPerBlock) {
        const uint64_t c = lo + p;
        const uint32_t k0 = fchild[c], k1 = fchild[c + 1];
        uint32_t s = 0;
        for (uint32_t k = k0 + (uint32_t)lane; k < k1; k += kWave) s += rank[k];
        s = wave_sum(s);
        if (lane == 0) rank[c] = s + 1u + (desc ? desc[c] : 0u);
    }
}

__global__ void __launch_bounds__(kBlock) k_child_position_wave(const uint32_t *__restrict__ fchild, uint64_t lo,
                                                                 uint64_t P, uint32_t *__restrict__ rank)
{
    const int lane = lane_id();
    for (uint64_t p = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; p < P;
         p += (uint64_t)gridDim.x * kWavesPerBlock) {
        const uint64_t c = lo + p;
        const uint32_t k0 = fchild[c], k1 = fchild[c + 1];
        uint32_t run = (c == 0 ? 0u : rank[c]) + 1u;
        for (uint32_t top = k1; top > k0;) {
            const uint32_t n = top - k0 < (uint32_t)kWave ? top - k0 : (uint32_t)kWave;
            const bool ok = (uint32_t)lane < n;
            const uint32_t k = top - 1u - (uint32_t)lane;  // lane 0 takes the last child
            const uint32_t sz = ok ? rank[k] : 0u;
            const uint32_t ex = wave_excl_scan(sz);
            if (ok) rank[k] = run + ex;
            run += wave_sum(sz);
            top -= n;
        }
    }
}

// perm[position] = concept
__global__ void __launch_bounds__(kBlock) k_invert(const uint32_t *__restrict__ rank, uint64_t K,
                                                    uint32_t *__restrict__ perm)
{
    for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < K; c += (uint64_t)gridDim.x * blockDim.x)
        perm[c == 0 ? 0 : rank[c]] = (uint32_t)c;
}

// ---------------------------------------------------------------------------
// output: sorted intents and extent bitmaps into the caller's buffers.  One
// wavefront per output row; the extent is assembled in LDS tile by tile from
// its sorted object list and streamed out with coalesced stores.

__global__ void __launch_bounds__(kBlock) k_output(const uint64_t *__restrict__ intents,
                                                    const uint64_t *__restrict__ loff,
                                                    const uint32_t *__restrict__ objs,
                                                    const uint32_t *__restrict__ perm, uint64_t K, int wm, int wn,
                                                    uint64_t *__restrict__ intents_out,
                                                    uint64_t *__restrict__ extents_out)
{
    __shared__ uint64_t s_tile[kWavesPerBlock][kOutTileWords];
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    uint64_t *T = s_tile[wv];
    for (uint64_t i = (uint64_t)blockIdx.x * kWavesPerBlock + wv; i < K; i += (uint64_t)gridDim.x * kWavesPerBlock) {
        const uint64_t src = perm[i];
        if (intents_out)
            for (int u = lane; u < wm; u += kWave) intents_out[i * wm + u] = intents[src * wm + u];
        if (!extents_out) continue;
        uint64_t o = loff[src];
        const uint64_t o1 = loff[src + 1];
        uint64_t *row = extents_out + i * (uint64_t)wn;
        for (int w0 = 0; w0 < wn; w0 += kOutTileWords) {
            const int tw = (wn - w0) < kOutTileWords ? (wn - w0) : kOutTileWords;
            for (int w = lane; w < tw; w += kWave) T[w] = 0;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const uint64_t gend = (uint64_t)(w0 + tw) * 64;
            while (o < o1) {
                bool in = false;
                uint32_t g = 0;
                if (o + lane < o1) {
                    g = objs[o + lane];
                    in = (uint64_t)g < gend;
                }
                if (in) atomicOr((unsigned long long *)&T[(g >> 6) - w0], (unsigned long long)(1ull << (g & 63)));
                const uint64_t bal = __ballot(in);
                o += __popcll(bal);
                if (bal != ~0ull) break;  // the list is sorted: the rest lies past this tile
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            for (int w = lane; w < tw; w += kWave) __builtin_nontemporal_store(T[w], &row[w0 + w]);
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// The ordered intents: output row r is intent perm[r].  A workgroup writes
// kBlock / wm consecutive rows a step, one word per thread (whole consecutive
// lines); the reads gather W_M words a row.  W_M <= 64 < kBlock.
__global__ void __launch_bounds__(kBlock) k_output_intents(const uint64_t *__restrict__ intents,
                                                           const uint32_t *__restrict__ perm, uint64_t K, int wm,
                                                           uint64_t *__restrict__ intents_out)
{
    const int rows = kBlock / wm;  // rows a step
    const int row = (int)threadIdx.x / wm, word = (int)threadIdx.x - row * wm;
    if (row >= rows) return;
    for (uint64_t r = (uint64_t)blockIdx.x * rows + row; r < K; r += (uint64_t)gridDim.x * rows)
        intents_out[r * wm + word] = intents[(uint64_t)perm[r] * wm + word];
}

typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

// Row-block output kernel: largest LDS tile in bytes, the tile size it aims
// for, threads per workgroup (512 measured best on MI355X against 256, 384 and
// 1024), and the words of a cache line its regions are aligned to.
constexpr int kOutBlockBytes = 65536;
constexpr int kOutTargetBytes = 40960;
constexpr int kOutThreads = 512;
constexpr int kOutWaves = kOutThreads / kWave;
constexpr int kOutLineWords = 128 / 8;

// Entries of slack after the last extent list, so that the output kernel can
// read object ids sixteen at a time past a list's end.
constexpr uint64_t kObjSlack = 16;

// Workgroup barrier for LDS only: the waves' LDS operations are done and
// visible after it, while their global stores stay in flight (a full barrier
// waits for those too).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// k_output_block: one workgroup writes R consecutive output rows.  Their extent
// bitmaps are assembled together in one dynamic LDS tile of R*wn words (the
// object lists OR-ed in with LDS atomics), then the tile goes out as a single
// contiguous region of the extent array: each wavefront stores 1 KiB runs, so
// when R*wn*8 is a multiple of 128 bytes every store covers whole, aligned cache
// lines.  The tile is cleared as it is read.  The intent rows are written by
// k_output_intents.  The grid is persistent: a workgroup walks blocks with the
// grid stride.
//
// The stores of one block and the assembly of the next overlap: gfx950 counts
// vector loads and stores on one in-order counter, so a vector load issued
// after a block's stores can only be waited for once those stores are done.
// The row sources (permutation entry, list bounds) and lists of up to 256
// objects are therefore read with scalar loads (a counter of their own, the
// ids sixteen at a time, uniform per wavefront), and the barriers wait for LDS
// work only.  Longer lists (a few large extents) use vector loads.
constexpr int kOutScalarList = 256;

__global__ void __launch_bounds__(kOutThreads) k_output_block(const uint64_t *__restrict__ loff,
                                                          const uint32_t *__restrict__ objs,
                                                          const uint32_t *__restrict__ perm, uint64_t K, int wn,
                                                          int R, uint64_t *__restrict__ extents_out)
{
    extern __shared__ __attribute__((aligned(16))) uint64_t s_rows[];
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int words = R * wn;
    for (int w = threadIdx.x; w < words; w += kOutThreads) s_rows[w] = 0;
    // stores of two words at a time need a 16-byte aligned region start
    const bool pairs = ((reinterpret_cast<uintptr_t>(extents_out) & 15) == 0) && (words & 1) == 0;
    const uint64_t nblk = (K + R - 1) / R;
    lds_barrier();
    for (uint64_t b = blockIdx.x; b < nblk; b += gridDim.x) {
        const uint64_t r0 = b * (uint64_t)R;
        const int nr = (int)((K - r0) < (uint64_t)R ? (K - r0) : (uint64_t)R);
        for (int rr = wv; rr < nr; rr += kOutWaves) {
            const uint32_t src = perm[r0 + rr];
            const uint64_t o = loff[src], e = loff[src + 1];
            uint64_t *T = s_rows + rr * wn;
            if (e - o <= (uint64_t)kOutScalarList) {
                for (uint64_t p = o; p < e; p += 16) {
                    uint32_t v[16];
#pragma unroll
                    for (int k = 0; k < 16; ++k) v[k] = objs[p + k];  // kObjSlack entries follow the last list
                    uint32_t g = 0;
#pragma unroll
                    for (int k = 0; k < 16; ++k) g = lane == k ? v[k] : g;
                    if (lane < 16 && (uint64_t)lane < e - p)
                        atomicOr((unsigned long long *)&T[g >> 6], (unsigned long long)(1ull << (g & 63)));
                }
            } else {
                for (uint64_t p = o + lane; p < e; p += kWave) {
                    const uint32_t g = objs[p];
                    atomicOr((unsigned long long *)&T[g >> 6], (unsigned long long)(1ull << (g & 63)));
                }
            }
        }
        lds_barrier();
        const uint64_t base = r0 * (uint64_t)wn;
        const int cnt = nr * wn;
        if (pairs) {
            u64x2 *S = reinterpret_cast<u64x2 *>(s_rows);
            u64x2 *D = reinterpret_cast<u64x2 *>(extents_out + base);
            const u64x2 z = {0, 0};
            for (int e = threadIdx.x; e < (cnt >> 1); e += kOutThreads) {
                const u64x2 v = S[e];
                S[e] = z;
                __builtin_nontemporal_store(v, &D[e]);
            }
            if ((cnt & 1) && threadIdx.x == 0) {
                extents_out[base + cnt - 1] = s_rows[cnt - 1];
                s_rows[cnt - 1] = 0;
            }
        } else {
            for (int e = threadIdx.x; e < cnt; e += kOutThreads) {
                const uint64_t v = s_rows[e];
                s_rows[e] = 0;
                __builtin_nontemporal_store(v, &extents_out[base + e]);
            }
        }
        lds_barrier();
    }
}

}  // namespace fcbo

namespace fcbo {

// ---------------------------------------------------------------------------
// Lattice cover edges.  The concepts ordered by extent inclusion form the
// concept lattice; the lower covers of (A, B) are the concepts right below it
// (page "hnwysp.cn/news/97538", section 4.4 and page "hotelren.com/news/5603750",
// section 3.4 rebuild these edges after the enumeration).
//
// For an attribute n outside B let c_n = A AND col[n] (the objects of A having
// n) and D_n = c_n' = (B + {n})''.  Every lower cover is some D_n, and D_n is a
// lower cover exactly when no c_k (k outside B) strictly contains c_n.  The
// attributes k of D_n outside B are exactly those with c_n inside c_k, so:
//     D_n is a lower cover  <=>  |c_k| = |c_n| for every k in D_n \ B.
// Each cover is generated by all of its attributes outside B; it is emitted
// once, by the smallest of them (n = the first attribute of D_n outside B, the
// form of the canonical test).  Of two covers the one emitted by the smaller
// attribute holds it and the other does not, while both agree with B below it,
// so it comes later in the output order: emitters in descending order give the
// covers' output positions in ascending order.
//
// Output, per concept at output position i: its lower covers' positions,
// ascending, at [offsets[i], offsets[i + 1]).  Two passes over the concepts:
// counting, then (after a scan) writing.

// Concepts are located by intent through an open-addressing hash table (linear
// probing, at most half full) of concept indices.  The hash folds the intent
// words with multiply-xorshift steps and finishes with the 64-bit finalizer of
// MurmurHash3 (Appleby).
constexpr uint32_t kCoverEmpty = 0xFFFFFFFFu;

template <int WMC>
__device__ __forceinline__ uint64_t intent_slot_hash(const uint64_t (&d)[WMC], int wm)
{
    uint64_t h = 0x2545F4914F6CDD1Dull;
#pragma unroll
    for (int u = 0; u < WMC; ++u) {
        if (u < wm) {
            h ^= d[u];
            h *= 0xFF51AFD7ED558CCDull;
            h ^= h >> 32;
        }
    }
    h ^= h >> 33;
    h *= 0xFF51AFD7ED558CCDull;
    h ^= h >> 33;
    h *= 0xC4CEB9FE1A85EC53ull;
    h ^= h >> 33;
    return h;
}

struct CoverArgs {
    const uint64_t *rows;     // N x wm
    const uint64_t *intents;  // generation order
    const int32_t *cursor;    // generation order
    const uint32_t *fchild;   // first child of every concept (children contiguous, ascending cursor)
    const uint32_t *rank;     // output position of every concept but the root
    const uint64_t *loff;
    const uint32_t *objs;
    const uint32_t *perm;     // output position -> concept
    uint32_t *table;          // concept index by intent (open addressing), kCoverEmpty when free
    uint64_t table_mask;      // slots - 1 (a power of two, at least 2K slots)
    uint64_t K;
    int m, wm;
    int64_t small_max;        // concepts with at most this many objects take the wavefront kernel
    uint64_t tail_m;
    uint32_t *big;            // output positions of the other concepts
    uint64_t *ctr;            // [0]: their number, [1]: covers not found among the intents (stays 0),
                              // [2]: scratch entries handed out, [3]: set when the scratch ran out
    uint32_t *count;          // passes 1 and 3: covers per output position
    const uint64_t *offsets;  // pass 2: their exclusive scan
    uint32_t *targets;        // pass 2: output positions of the covers
    uint32_t *scratch;        // pass 3: every concept's covers' positions, one run per concept
    uint64_t scratch_cap;     // entries
    uint64_t *sstart;         // pass 3: start of each concept's run in scratch
};

// The passes of the cover kernels: 1 counts the covers of every concept; 2
// (after the scan of the counts) writes their positions to the caller's
// targets; 3 counts them and keeps their positions in the scratch buffer, one
// run per concept, which k_cover_copy_runs moves to the targets after the scan.
constexpr int kCoverCount = 1, kCoverWrite = 2, kCoverKeep = 3;
// Scratch entries a wavefront of k_cover_local takes at a time (concepts with
// more covers reserve their run alone).
constexpr uint32_t kCoverChunk = 128;

// Every concept into the table, keyed by its intent.
template <int WMC>
__global__ void __launch_bounds__(kBlock) k_cover_table(CoverArgs C)
{
    for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < C.K; c += (uint64_t)gridDim.x * blockDim.x) {
        constexpr int DW = WMC <= 8 ? WMC : 64;
        uint64_t d[DW];
#pragma unroll
        for (int u = 0; u < DW; ++u) d[u] = u < C.wm ? C.intents[c * C.wm + u] : 0ull;
        uint64_t h = intent_slot_hash<DW>(d, C.wm) & C.table_mask;
        // the table has at least twice as many slots as concepts: a free slot is
        // reached within K probes
        for (uint64_t probe = 0; probe <= C.K; ++probe) {
            if (atomicCAS(&C.table[h], kCoverEmpty, (uint32_t)c) == kCoverEmpty) break;
            h = (h + 1) & C.table_mask;
        }
    }
}

// The output positions whose concept has more than small_max objects.
__global__ void __launch_bounds__(kBlock) k_cover_list_big(CoverArgs C)
{
    const uint64_t nt = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i0 = (uint64_t)blockIdx.x * blockDim.x; i0 < C.K; i0 += nt) {
        const uint64_t i = i0 + threadIdx.x;
        bool big = false;
        if (i < C.K) {
            const uint64_t c = C.perm[i];
            big = (int64_t)(C.loff[c + 1] - C.loff[c]) > C.small_max;
        }
        wave_append(big, (uint32_t)i, C.big, &C.ctr[0]);
    }
}

// Output position of the lower cover D (wm words) of concept c, emitted by n.
// When n lies above c's cursor, D is c's CbO child made at n (it passes the
// canonical test: D agrees with B below n), already placed by the order pass;
// otherwise the table gives the concept with intent D.
template <int WMC>
__device__ __forceinline__ uint32_t cover_position(const CoverArgs &C, uint64_t c, int n, const uint64_t (&D)[WMC])
{
    if (n > C.cursor[c]) {
        uint32_t lo = C.fchild[c], hi = C.fchild[c + 1];
        while (lo < hi) {
            const uint32_t mid = lo + (hi - lo) / 2;
            const int cm = C.cursor[mid];
            if (cm == n) return C.rank[mid];
            if (cm < n) lo = mid + 1;
            else hi = mid;
        }
    }
    uint64_t h = intent_slot_hash<WMC>(D, C.wm) & C.table_mask;
    for (uint64_t probe = 0; probe <= C.K; ++probe) {
        const uint32_t e = C.table[h];
        if (e == kCoverEmpty) break;
        bool same = true;
#pragma unroll
        for (int u = 0; u < WMC; ++u)
            if (u < C.wm) same = same && C.intents[(uint64_t)e * C.wm + u] == D[u];
        if (same) return e == 0 ? 0u : C.rank[e];
        h = (h + 1) & C.table_mask;
    }
    atomicAdd((unsigned long long *)&C.ctr[1], 1ull);  // not a concept: cannot happen
    return kCoverEmpty;
}

// 1 when any of the lane's flags is set
template <int N>
__device__ __forceinline__ uint32_t live_any(const bool (&f)[N])
{
    uint32_t r = 0;
#pragma unroll
    for (int u = 0; u < N; ++u) r |= f[u] ? 1u : 0u;
    return r;
}

// 64 x 64 bit transpose across the wavefront: lane l holds row l on entry and
// column l on return (bit o of the result is bit l of row o).  Six butterfly
// stages; in the stage of distance j, lanes l and l ^ j exchange the half
// blocks that cross the diagonal (the recursive block transpose, done with
// one lane per row).
__device__ __forceinline__ uint64_t wave_transpose64(uint64_t x)
{
    const int lane = lane_id();
#pragma unroll
    for (int s = 0; s < 6; ++s) {
        const int j = 32 >> s;
        // bits whose index has the bit j clear
        const uint64_t m = s == 0 ? 0x00000000FFFFFFFFull : s == 1 ? 0x0000FFFF0000FFFFull
                         : s == 2 ? 0x00FF00FF00FF00FFull : s == 3 ? 0x0F0F0F0F0F0F0F0Full
                         : s == 4 ? 0x3333333333333333ull : 0x5555555555555555ull;
        const uint64_t p = __shfl_xor(x, j);
        x = (lane & j) ? ((x & ~m) | ((p >> j) & m)) : ((x & m) | ((p << j) & ~m));
    }
    return x;
}

// Concepts with at most 64 objects, one wavefront each.  The object rows are
// staged in LDS; lane b gets, for every intent word u, the mask of the objects
// having attribute 64u + b: a transpose of the wavefront's rows (one object a
// lane), or for a few objects broadcast reads of the staged rows.
// When no object carries an attribute outside B the one lower cover is the
// bottom (for every concept but the bottom itself).
template <int WMC>
__global__ void __launch_bounds__(kBlock) k_cover_local(CoverArgs C, int pass)
{
    static_assert(WMC <= 8, "the wavefront cover kernel keeps rows of at most 8 words in LDS");
    __shared__ uint64_t s_rows[kWavesPerBlock][kWave * WMC];
    __shared__ uint32_t s_pos[kWavesPerBlock][64 * WMC];  // passes 2, 3: position of the cover emitted by n
    __shared__ uint64_t s_cmax[kWavesPerBlock][kWave];    // passes 2, 3: a batch of covers' objects
    __shared__ uint16_t s_emit[kWavesPerBlock][kWave];    // and their emitters
    const int lane = lane_id();
    const int wv = threadIdx.x / kWave;
    const int wm = words_of<WMC>(C.wm);
    uint64_t *R = s_rows[wv];
    uint32_t *POS = s_pos[wv];
    uint64_t *CMX = s_cmax[wv];
    uint16_t *EMT = s_emit[wv];
    uint64_t chunk = 0;             // pass 3: the wavefront's scratch chunk
    uint32_t used = kCoverChunk;    // entries of it taken
    for (uint64_t i = (uint64_t)blockIdx.x * kWavesPerBlock + wv; i < C.K; i += (uint64_t)gridDim.x * kWavesPerBlock) {
        const uint64_t c = C.perm[i];
        const uint64_t o0 = C.loff[c], a64 = C.loff[c + 1] - o0;
        if ((int64_t)a64 > C.small_max) continue;  // the workgroup kernel's
        const int a = (int)a64;
        uint64_t B[WMC];
        bool full = true;  // B = M: the bottom, no lower cover
#pragma unroll
        for (int u = 0; u < WMC; ++u) {
            B[u] = ~0ull;
            if (u < wm) {
                B[u] = C.intents[c * C.wm + u];
                if (u == wm - 1) B[u] |= ~C.tail_m;  // attributes past M count as in B
                full = full && B[u] == ~0ull;
            }
        }
        const bool mine = lane < a;
        const uint64_t g = mine ? C.objs[o0 + lane] : 0;
        uint64_t cand[WMC];  // attributes outside B carried by some object
        uint64_t row[WMC];   // this lane's object's row (zero past the last object)
        uint64_t any = 0;
#pragma unroll
        for (int u = 0; u < WMC; ++u) {
            row[u] = (mine && u < wm) ? C.rows[g * C.wm + u] : 0ull;
            R[lane * WMC + u] = row[u];
            cand[u] = (u < wm) ? (wave_or(row[u]) & ~B[u]) : 0ull;
            any |= cand[u];
        }
        // with no attribute outside B carried, every one gives the bottom, the
        // one lower cover (none when B is already every attribute)
        uint32_t ncov = any ? 0u : (full ? 0u : 1u);
        if (any) {
            wave_sync();
            // lane b: cm[u] = c_n, the objects having attribute n = 64u + b (the
            // transpose costs about as much as ten objects' broadcast reads)
            uint64_t cm[WMC];
#pragma unroll
            for (int u = 0; u < WMC; ++u) cm[u] = 0;
            if (a > 10) {
#pragma unroll
                for (int u = 0; u < WMC; ++u)
                    if (u < wm && cand[u]) cm[u] = wave_transpose64(row[u]);
            } else {
                for (int o = 0; o < a; ++o) {
#pragma unroll
                    for (int u = 0; u < WMC; ++u)
                        if (u < wm && cand[u]) cm[u] |= ((R[o * WMC + u] >> lane) & 1ull) << o;
                }
            }
            // Every extent strictly inside A lies in some c_n (n an attribute of
            // its intent outside B), and (B + {n})'' = c_n' adds exactly the k
            // with c_n inside c_k.  So the lower covers are the concepts (c_n,
            // c_n') of the maximal c_n, each emitted by the smallest n with that
            // c_n (the first attribute of c_n' outside B).  Taken largest first:
            // the largest live c_n is maximal (a strict superset would be larger
            // and would have taken it out); it takes out every live c_k inside
            // it, equal ones included; and ties go to the smallest attribute,
            // which for equal sets is the emitter.  The covers' intents and
            // positions are then found a lane each, 64 covers at a time, so
            // that their lookups overlap.
            bool live[WMC];
            uint32_t cnt[WMC];
#pragma unroll
            for (int u = 0; u < WMC; ++u) {
                live[u] = u < wm && ((cand[u] >> lane) & 1ull);
                cnt[u] = (uint32_t)__popcll(cm[u]);
                if (pass != kCoverCount && u < wm) POS[u * 64 + lane] = kCoverEmpty;
            }
            wave_sync();
            for (;;) {
                uint32_t key = 0;  // count, then the smaller attribute
#pragma unroll
                for (int u = 0; u < WMC; ++u) {
                    const uint32_t ku = (cnt[u] << 13) | 4096u | (uint32_t)(4095 - (64 * u + lane));
                    if (live[u] && ku > key) key = ku;
                }
                key = lane_value(wave_incl_scan_op<uint32_t>(key, 0u, [](uint32_t x, uint32_t y) { return x > y ? x : y; }),
                                 kWave - 1);
                if (!key) break;
                const int n = 4095 - (int)(key & 4095u);
                uint64_t pick = 0;
#pragma unroll
                for (int u = 0; u < WMC; ++u)
                    if (u == (n >> 6)) pick = cm[u];
                const uint64_t cmax = lane_value64(pick, n & 63);
#pragma unroll
                for (int u = 0; u < WMC; ++u)
                    if (live[u] && (cm[u] & ~cmax) == 0) live[u] = false;
                const uint32_t slot = ncov & (kWave - 1);
                if (pass != kCoverCount && lane == 0) {
                    CMX[slot] = cmax;
                    EMT[slot] = (uint16_t)n;
                }
                ++ncov;
                // a full batch, or the last covers: lane k finds cover k's
                // intent (the AND of its objects' rows) and position
                const bool last = __ballot(live_any(live) != 0u) == 0ull;
                if (pass != kCoverCount && (slot == kWave - 1 || last)) {
                    wave_sync();
                    if ((uint32_t)lane <= slot) {
                        const uint64_t cx = CMX[lane];
                        const int ne = (int)EMT[lane];
                        uint64_t D[WMC];
#pragma unroll
                        for (int v = 0; v < WMC; ++v) D[v] = ~0ull;
                        for (uint64_t x = cx; x; x &= x - 1ull) {
                            const int o = __ffsll((unsigned long long)x) - 1;
#pragma unroll
                            for (int v = 0; v < WMC; ++v)
                                if (v < wm) D[v] &= R[o * WMC + v];
                        }
                        D[wm - 1] &= C.tail_m;
                        POS[ne] = cover_position<WMC>(C, c, ne, D);
                    }
                    wave_sync();
                }
                if (last) break;
            }
        }
        if (pass != kCoverWrite && lane == 0) C.count[i] = ncov;
        if (pass != kCoverCount && ncov) {
            // the positions by descending emitter (ascending position): to the
            // targets, or (pass 3) to a run in the wavefront's scratch chunk (a
            // new chunk when it does not fit; a run longer than a chunk is
            // reserved on its own)
            uint32_t *out = C.targets;
            uint64_t at = 0;
            bool fits = true;
            if (pass == kCoverWrite) {
                at = C.offsets[i];
            } else {
                out = C.scratch;
                if (ncov > kCoverChunk) {
                    if (lane == 0) at = atomicAdd((unsigned long long *)&C.ctr[2], (unsigned long long)ncov);
                    at = uniform64(at);
                } else {
                    if (used + ncov > kCoverChunk) {
                        uint64_t b = 0;
                        if (lane == 0) b = atomicAdd((unsigned long long *)&C.ctr[2], (unsigned long long)kCoverChunk);
                        chunk = uniform64(b);
                        used = 0;
                    }
                    at = chunk + used;
                    used += ncov;
                }
                fits = at + ncov <= C.scratch_cap;
                if (lane == 0) {
                    C.sstart[i] = at;
                    if (!fits) C.ctr[3] = 1;
                }
            }
            if (fits) {
                if (!any) {
                    if (lane == 0) out[at] = (uint32_t)(C.K - 1);
                } else {
                    wave_sync();  // POS written by the batches above
                    uint32_t k0 = 0;
#pragma unroll
                    for (int u = WMC - 1; u >= 0; --u) {
                        if (u >= wm) continue;
                        const uint32_t p = POS[u * 64 + lane];
                        const bool e = p != kCoverEmpty;
                        const uint64_t bal = __ballot(e);
                        if (e) out[at + k0 + (uint32_t)__popcll(bal & ~upto_mask(lane))] = p;
                        k0 += (uint32_t)__popcll(bal);
                    }
                }
            }
        }
        wave_sync();
    }
}

// Pass 3's runs to the caller's targets: concept i's run of count[i] positions
// from scratch[sstart[i]] to targets[offsets[i]], one thread per concept.
__global__ void __launch_bounds__(kBlock) k_cover_copy_runs(CoverArgs C)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < C.K; i += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t n = C.count[i];
        if (!n) continue;
        const uint32_t *src = C.scratch + C.sstart[i];
        uint32_t *dst = C.targets + C.offsets[i];
        for (uint32_t k = 0; k < n; ++k) dst[k] = src[k];
    }
}

// Concepts with more objects, one workgroup each (from the list): object
// counts of all attributes by incidence (LDS atomics); the carried candidates
// listed in ascending order; then slices of kCoverSlice of them, each slice's
// D_n accumulated in one pass over the extent list (LDS AND atomics) and tested
// one per thread.  The covers' positions go to an LDS table indexed by emitter
// and leave in descending emitter order.
constexpr int kCoverThreads = 256;
constexpr int kCoverSlice = 64;
constexpr int kCoverMaxM = 4096;

// Exclusive scan over a kCoverThreads-thread workgroup; returns the total.
__device__ __forceinline__ uint32_t cover_block_scan(uint32_t v, uint32_t &excl, uint32_t *s_sum)
{
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    const uint32_t ex = wave_excl_scan(v);
    if (lane == kWave - 1) s_sum[wv] = ex + v;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int w = 0; w < kCoverThreads / kWave; ++w) {
        before += w < wv ? s_sum[w] : 0u;
        all += s_sum[w];
    }
    __syncthreads();
    excl = before + ex;
    return all;
}

// LDS of k_cover_big for M attributes (dynamic, so that small M leaves room
// for more workgroups per compute unit): D slice, slice mask, counts,
// positions, candidates, slots.
template <int WMC>
constexpr size_t cover_big_lds(int m)
{
    constexpr int WS = WMC <= 8 ? WMC : 64;
    const size_t mm = ((size_t)m + 7) / 8 * 8;
    return (size_t)kCoverSlice * WS * 8 + WS * 8 + mm * (4 + 4 + 2 + 2);
}

template <int WMC>
__global__ void __launch_bounds__(kCoverThreads) k_cover_big(CoverArgs C, int pass)
{
    constexpr int WS = WMC <= 8 ? WMC : 64;  // words of a D entry kept in LDS
    extern __shared__ __attribute__((aligned(16))) uint64_t s_big[];
    const size_t mm = ((size_t)C.m + 7) / 8 * 8;
    uint64_t *s_d = s_big;                                          // kCoverSlice x WS
    uint64_t *s_mask = s_d + kCoverSlice * WS;                      // WS: the current slice's attributes
    uint32_t *s_cnt = (uint32_t *)(s_mask + WS);                    // mm: |c_n|
    uint32_t *s_pos = s_cnt + mm;                                   // mm: position of the cover emitted by n, else ~0
    uint16_t *s_cand = (uint16_t *)(s_pos + mm);                    // mm: the carried candidates, ascending
    int16_t *s_slot = (int16_t *)(s_cand + mm);                     // mm: slot of n in the current slice, else -1
    __shared__ uint32_t s_sum[kCoverThreads / kWave];
    const int tid = threadIdx.x;
    const int wm = words_of<WMC>(C.wm);
    const int per = (C.m + kCoverThreads - 1) / kCoverThreads;  // attributes per thread, in blocks
    const uint64_t nbig = C.ctr[0];
    for (uint64_t it = blockIdx.x; it < nbig; it += gridDim.x) {
        const uint64_t i = C.big[it];
        const uint64_t c = C.perm[i];
        const uint64_t o0 = C.loff[c], o1 = C.loff[c + 1];
        const uint64_t *Bp = C.intents + c * C.wm;
        auto in_b = [&](int n) -> bool { return ((Bp[n >> 6] >> (n & 63)) & 1ull) != 0; };
        for (int n = tid; n < C.m; n += kCoverThreads) {
            s_cnt[n] = 0;
            s_pos[n] = 0xFFFFFFFFu;
            s_slot[n] = -1;
        }
        __syncthreads();
        for (uint64_t o = o0 + tid; o < o1; o += kCoverThreads) {
            const uint64_t g = C.objs[o];
            for (int u = 0; u < wm; ++u) {
                uint64_t x = C.rows[g * C.wm + u] & ~Bp[u];
                while (x) {
                    const int b = __ffsll((unsigned long long)x) - 1;
                    x &= x - 1ull;
                    atomicAdd(&s_cnt[64 * u + b], 1u);
                }
            }
        }
        __syncthreads();
        // the carried candidates in ascending order: thread t lists the block of
        // attributes [t * per, (t + 1) * per)
        const int lo_a = tid * per, hi_a = lo_a + per < C.m ? lo_a + per : C.m;
        uint32_t mine = 0;
        for (int n = lo_a; n < hi_a; ++n) mine += (!in_b(n) && s_cnt[n]) ? 1u : 0u;
        uint32_t at;
        const uint32_t ncand = cover_block_scan(mine, at, s_sum);
        for (int n = lo_a; n < hi_a; ++n)
            if (!in_b(n) && s_cnt[n]) s_cand[at++] = (uint16_t)n;
        uint32_t found = 0;
        if (ncand == 0) {
            // nothing outside B is carried: the bottom is the one lower cover
            // (none when B is already every attribute)
            bool full = true;
            for (int u = 0; u < wm; ++u) full = full && (Bp[u] == (u == wm - 1 ? C.tail_m : ~0ull));
            found = full ? 0u : 1u;
            if (pass == kCoverWrite && found && tid == 0) C.targets[C.offsets[i]] = (uint32_t)(C.K - 1);
            if (pass == kCoverKeep && tid == 0) {
                uint64_t at = 0;
                if (found) at = atomicAdd((unsigned long long *)&C.ctr[2], 1ull);
                const bool fits = at + found <= C.scratch_cap;
                if (found && fits) C.scratch[at] = (uint32_t)(C.K - 1);
                C.sstart[i] = at;
                if (!fits) C.ctr[3] = 1;
            }
        } else {
            __syncthreads();
            for (uint32_t s0 = 0; s0 < ncand; s0 += kCoverSlice) {
                const uint32_t nc = ncand - s0 < (uint32_t)kCoverSlice ? ncand - s0 : (uint32_t)kCoverSlice;
                if (tid < WS) s_mask[tid] = 0;
                for (uint32_t x = tid; x < nc * WS; x += kCoverThreads) s_d[x] = ~0ull;
                __syncthreads();
                if ((uint32_t)tid < nc) {
                    const uint32_t n = s_cand[s0 + tid];
                    s_slot[n] = (int16_t)tid;
                    atomicOr((unsigned long long *)&s_mask[n >> 6], (unsigned long long)(1ull << (n & 63)));
                }
                __syncthreads();
                for (uint64_t o = o0 + tid; o < o1; o += kCoverThreads) {
                    const uint64_t *row = C.rows + C.objs[o] * (uint64_t)C.wm;
                    for (int u = 0; u < wm; ++u) {
                        uint64_t x = row[u] & s_mask[u];
                        while (x) {
                            const int r = s_slot[64 * u + __ffsll((unsigned long long)x) - 1];
                            x &= x - 1ull;
                            for (int v = 0; v < wm; ++v)
                                atomicAnd((unsigned long long *)&s_d[r * WS + v], (unsigned long long)row[v]);
                        }
                    }
                }
                __syncthreads();
                if ((uint32_t)tid < nc) {
                    const int n = (int)s_cand[s0 + tid];
                    const uint64_t *D = s_d + tid * WS;
                    const uint32_t cnt_n = s_cnt[n];
                    bool ok = true, first = true;
                    for (int v = 0; v < wm && ok; ++v) {
                        uint64_t x = D[v] & ~Bp[v];
                        if (v == wm - 1) x &= C.tail_m;
                        if (first && x) {
                            ok = (64 * v + __ffsll((unsigned long long)x) - 1) == n;
                            first = false;
                        }
                        while (x && ok) {
                            const int k = 64 * v + __ffsll((unsigned long long)x) - 1;
                            x &= x - 1ull;
                            if (s_cnt[k] != cnt_n) ok = false;
                        }
                    }
                    if (ok) {
                        uint32_t pos = 0;
                        if (pass != kCoverCount) {
                            uint64_t d[WS];
                            for (int v = 0; v < wm; ++v) d[v] = (v == wm - 1) ? (D[v] & C.tail_m) : D[v];
                            pos = cover_position<WS>(C, c, n, d);
                        }
                        s_pos[n] = pos;
                    }
                    s_slot[n] = -1;
                }
                __syncthreads();
            }
            // covers in descending emitter order: thread t takes the t-th block
            // of attributes from the top down
            const int hi = C.m - tid * per, lo = hi - per > 0 ? hi - per : 0;
            uint32_t nmine = 0;
            for (int n = hi - 1; n >= lo; --n) nmine += s_pos[n] != 0xFFFFFFFFu ? 1u : 0u;
            uint32_t before;
            found = cover_block_scan(nmine, before, s_sum);
            uint64_t w = 0;
            bool fits = true;
            if (pass == kCoverWrite) {
                w = C.offsets[i] + before;
            } else if (pass == kCoverKeep) {
                // the concept's run: one reservation for the workgroup
                if (tid == 0) s_sum[0] = 0;
                __syncthreads();
                if (tid == 0 && found) {
                    const uint64_t at = atomicAdd((unsigned long long *)&C.ctr[2], (unsigned long long)found);
                    s_sum[0] = (uint32_t)at;
                    s_sum[1] = (uint32_t)(at >> 32);
                    C.sstart[i] = at;
                    if (at + found > C.scratch_cap) C.ctr[3] = 1;
                }
                __syncthreads();
                const uint64_t at = found ? ((uint64_t)s_sum[0] | ((uint64_t)s_sum[1] << 32)) : 0ull;
                fits = at + found <= C.scratch_cap;
                w = at + before;
            }
            if (pass != kCoverCount && fits) {
                uint32_t *out = pass == kCoverWrite ? C.targets : C.scratch;
                for (int n = hi - 1; n >= lo; --n)
                    if (s_pos[n] != 0xFFFFFFFFu) out[w++] = s_pos[n];
            }
        }
        if (pass != kCoverWrite && tid == 0) C.count[i] = found;
        __syncthreads();
    }
}


// ---------------------------------------------------------------------------
// task pool (page 1 sections 3.2 and 5.3: workers take tasks from a shared
// pool as they free up; page 4 section 4.3: a kernel of its own for one class
// of parents)
//
// With the pool the level loop expands only the parents with more than
// task_max objects (at most 64), and every concept of the store with at most
// task_max objects is a task whose whole subtree one wavefront enumerates
// depth-first.  A task of a objects has at most 2^a concepts below it, so a
// small task_max keeps the tasks short and many, and the wavefronts evenly
// loaded; the larger concepts stay with the level loop's packed kernels.  Every concept
// below a task has its objects among the task's (extents only shrink down the
// tree), so the wavefront keeps the task's rows in LDS and in registers (lane
// g: object g of the task's list) and every extent below as a 64-bit mask over
// them.  Wavefronts take the tasks in turn from an atomic counter until none
// are left; the pool is fixed before the launch, so no wavefront waits for
// another.
//
// A node's candidates are the task's candidates (above the task's cursor,
// outside its intent) that lie above the node's cursor and outside its
// intent; they are tested 64 at a time, one per lane, from the largest
// attribute down, and the passing ones visited in that order, so concepts come
// out in the output order of the task's subtree (pre-order, children by
// descending attribute).  The descent keeps one frame per depth in LDS; a
// child's extent is a proper subset of its parent's (j is outside the parent's
// intent, so some object lacks it), so the depth stays within the task's
// object count.
//
// Concepts go to pool slots, reserved 64 at a time per wavefront: the intent,
// and a record {object mask, task, offset in the task's subtree, cursor, depth
// below the task}.  Slots a wavefront reserved but did not use keep owner
// kPoolFree.  If the slots run out, the kernel raises the overflow flag and
// every wavefront stops; the host grows the slots and runs it again.

constexpr int kPoolWaves = 2;              // wavefronts per block
constexpr int kPoolStripes = 64;           // task claim counters
// Concepts with at most this many objects are tasks (measured against 8, 32
// and 64: best on the 2,000 x 64 context, 1.10 against 1.14 to 1.41 ms a
// step, and within 4% of the best on the 50,000 x 400 one).
constexpr int kPoolTaskMax = 16;
constexpr int kPoolDepth = kPoolTaskMax + 1;  // frames: the task and up to kPoolTaskMax levels below
constexpr uint32_t kPoolFree = 0xFFFFFFFFu;
// pool counters (word offsets, each in a 128-byte line of its own)
enum { POOL_NTASKS = 0, POOL_SLOTS = 16, POOL_OVERFLOW = 32, POOL_ERROR = 48, POOL_TOT_N = 64, POOL_TOT_OBJ = 80,
       POOL_CTR_N = 96 };

struct PoolRec {
    uint64_t mask;   // the concept's objects: bit g = object g of the task's list
    uint32_t owner;  // the task (store index); kPoolFree for a slot not used
    uint32_t off;    // position in the task's subtree, the task itself excluded
    int32_t cursor;  // the attribute that generated the concept
    uint32_t depth;  // levels below the task (1 = a child of the task)
};

struct PoolArgs {
    const uint64_t *rows;
    const uint64_t *intents;
    const int32_t *cursor;
    const uint64_t *loff;
    const uint32_t *objs;
    uint64_t K;       // store concepts
    const uint32_t *tasks;  // the tasks: store concepts with at most kPoolTaskMax objects
    uint64_t n_tasks;
    uint64_t *task_ctr;     // kPoolStripes claim counters, kCntPad words apart
    int m, wm;
    uint64_t tail_m;
    uint64_t *ctr;    // POOL_* counters
    uint64_t cap;     // pool slots
    uint64_t *p_int;  // cap x wm
    PoolRec *p_rec;   // cap
    uint32_t *desc;   // K: concepts below each task (0 for the other concepts)
};

template <int WMC>
__global__ void __launch_bounds__(kWave * kPoolWaves) k_pool(PoolArgs P)
{
    static_assert(WMC <= 8, "the pool keeps intents of at most 8 words");
    constexpr int kMaxCand = kWave * WMC;
    __shared__ uint64_t s_rows[kPoolWaves][kPoolTaskMax * WMC];  // the task's rows
    __shared__ uint64_t s_cm[kPoolWaves][kMaxCand];           // object mask of each task candidate
    __shared__ uint16_t s_cand[kPoolWaves][kMaxCand];         // the task's candidates, ascending
    __shared__ uint64_t s_fb[kPoolWaves][kPoolDepth * WMC];   // frame: intent
    __shared__ uint64_t s_fc[kPoolWaves][kPoolDepth];         // frame: object mask
    __shared__ uint64_t s_fp[kPoolWaves][kPoolDepth];         // frame: passing candidates of its round not yet visited
    __shared__ uint16_t s_flo[kPoolWaves][kPoolDepth];        // frame: first candidate above its cursor
    __shared__ uint16_t s_fhi[kPoolWaves][kPoolDepth];        // frame: candidates [lo, hi) not yet tested
    __shared__ uint16_t s_fbase[kPoolWaves][kPoolDepth];      // frame: candidate of bit 0 of the round
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = words_of<WMC>(P.wm);
    uint64_t *R = s_rows[wv];
    uint64_t *CM = s_cm[wv];
    uint16_t *CAND = s_cand[wv];
    uint64_t *FB = s_fb[wv];
    uint64_t *FC = s_fc[wv];
    uint64_t *FP = s_fp[wv];
    uint16_t *FLO = s_flo[wv], *FHI = s_fhi[wv], *FBASE = s_fbase[wv];
    uint64_t slot = 0, slot_end = 0;  // the wavefront's reserved slots not yet used
    bool stop = false;
    // Tasks are claimed one at a time from kPoolStripes counters (task i from
    // counter i mod kPoolStripes, each on a line of its own: atomics on one
    // address serialise); a wavefront starts on its own counter and moves to
    // the next one when that is used up, until every counter is.
    const int wid = (int)((blockIdx.x * (unsigned)kPoolWaves + (unsigned)wv) % (unsigned)kPoolStripes);
    int stripes_left = kPoolStripes, stripe = wid;
    while (!stop) {
        uint64_t k = 0;
        if (lane == 0) k = atomicAdd((unsigned long long *)&P.task_ctr[stripe * kCntPad], 1ull);
        const uint64_t ti = lane_value64(k, 0) * kPoolStripes + (uint64_t)stripe;
        if (ti >= P.n_tasks) {
            if (--stripes_left == 0) break;
            stripe = stripe + 1 == kPoolStripes ? 0 : stripe + 1;
            continue;
        }
        if (__hip_atomic_load(&P.ctr[POOL_OVERFLOW], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
        const uint64_t t = P.tasks[ti];
        const uint64_t o0 = P.loff[t];
        const int a = (int)(P.loff[t + 1] - o0);
        if (a > kPoolTaskMax) {  // not a task (the list holds none): never stage past the rows
            if (lane == 0) atomicOr((unsigned long long *)&P.ctr[POOL_ERROR], 1ull);
            break;
        }
        const int y0 = __builtin_amdgcn_readfirstlane(P.cursor[t]);
        // the task's rows: lane g < a holds object g's row, the others all ones
        // (neutral for the AND below)
        uint64_t row[WMC];
        {
            const uint64_t g = lane < a ? (uint64_t)P.objs[o0 + lane] : 0ull;
#pragma unroll
            for (int u = 0; u < WMC; ++u) {
                row[u] = ~0ull;
                if (u < wm && lane < a) {
                    row[u] = P.rows[g * P.wm + u];
                    R[lane * WMC + u] = row[u];
                }
            }
        }
        if (lane < wm) FB[lane] = P.intents[t * P.wm + lane];
        wave_sync();
        // the task's candidates and, for each, the objects of the task having it
        int nc = 0;
        for (int u = 0; u < wm; ++u) {
            uint64_t cm = ~uniform64(FB[u]) & above_mask(y0, u);
            if (u == wm - 1) cm &= P.tail_m;
            const bool has = ((cm >> lane) & 1ull) != 0;
            const uint64_t bal = __ballot(has);
            if (has) CAND[nc + __popcll(bal & below_mask(lane))] = (uint16_t)(64 * u + lane);
            nc += __popcll(bal);
        }
        wave_sync();
        for (int i = lane; i < nc; i += kWave) {
            const int j = CAND[i];
            const int u = j >> 6, b = j & 63;
            uint64_t msk = 0;
            for (int g = 0; g < a; ++g) msk |= ((R[g * WMC + u] >> b) & 1ull) << g;
            CM[i] = msk;
        }
        if (lane == 0) {
            FC[0] = a == 64 ? ~0ull : ((1ull << a) - 1ull);
            FP[0] = 0;
            FLO[0] = 0;
            FHI[0] = (uint16_t)nc;
        }
        wave_sync();
        uint32_t off = 0;  // concepts of the task's subtree written so far
        int d = 0;
        while (d >= 0) {
            const uint64_t pend = uniform64(FP[d]);
            if (!pend) {
                const int lo = __builtin_amdgcn_readfirstlane(FLO[d]);
                const int hi = __builtin_amdgcn_readfirstlane(FHI[d]);
                if (hi <= lo) {
                    --d;
                    continue;
                }
                // the next round: the highest untested candidates, one per lane
                const int base = hi - kWave > lo ? hi - kWave : lo;
                const int i = base + lane;
                bool pass = false;
                if (i < hi) {
                    const int j = CAND[i];
                    const int ju = j >> 6;
                    const uint64_t *Bd = FB + d * WMC;
                    if (!((Bd[ju] >> (j & 63)) & 1ull)) {
                        // C = the node's objects having j; D = AND of their rows
                        // (all attributes when C is empty); canonical: D agrees
                        // with the node's intent below j
                        const uint64_t c = FC[d] & CM[i];
                        uint64_t D[WMC];
#pragma unroll
                        for (int u = 0; u < WMC; ++u) D[u] = ~0ull;
                        for (uint64_t cc = c; cc; cc &= cc - 1ull) {
                            const int g = __ffsll((unsigned long long)cc) - 1;
#pragma unroll
                            for (int u = 0; u < WMC; ++u)
                                if (u < wm) D[u] &= R[g * WMC + u];
                        }
                        bool ok = true;
#pragma unroll
                        for (int u = 0; u < WMC; ++u) {
                            if (u < ju) ok = ok && D[u] == Bd[u];
                            if (u == ju) ok = ok && ((D[u] ^ Bd[u]) & below_mask(j & 63)) == 0;
                        }
                        pass = ok;
                    }
                }
                const uint64_t bal = __ballot(pass);
                if (lane == 0) {
                    FP[d] = bal;
                    FBASE[d] = (uint16_t)base;
                    FHI[d] = (uint16_t)base;
                }
                wave_sync();
                continue;
            }
            // the largest passing candidate not yet visited is the next child
            const int b = 63 - __clzll((long long)pend);
            const int i = __builtin_amdgcn_readfirstlane(FBASE[d]) + b;
            const int j = __builtin_amdgcn_readfirstlane(CAND[i]);
            const uint64_t c = uniform64(FC[d] & CM[i]);
            if (d + 1 >= kPoolDepth) {  // cannot happen for a closed intent; never write past the frames
                if (lane == 0) atomicOr((unsigned long long *)&P.ctr[POOL_ERROR], 1ull);
                stop = true;
                break;
            }
            // the child's intent: AND of the rows of its objects over the lanes
            const bool mine = ((c >> lane) & 1ull) != 0;
            uint64_t word = 0;  // lane u < wm: word u of the intent
#pragma unroll
            for (int u = 0; u < WMC; ++u) {
                if (u < wm) {
                    uint64_t w = wave_and(mine ? row[u] : ~0ull);
                    if (u == wm - 1) w &= P.tail_m;
                    if (lane == u) word = w;
                }
            }
            if (slot == slot_end) {
                uint64_t s0 = 0;
                if (lane == 0) s0 = atomicAdd((unsigned long long *)&P.ctr[POOL_SLOTS], (unsigned long long)kWave);
                s0 = lane_value64(s0, 0);
                if (s0 + kWave > P.cap) {
                    if (lane == 0) atomicOr((unsigned long long *)&P.ctr[POOL_OVERFLOW], 1ull);
                    stop = true;
                    break;
                }
                slot = s0;
                slot_end = s0 + kWave;
            }
            if (lane < wm) P.p_int[slot * P.wm + lane] = word;
            if (lane == 0) {
                PoolRec r;
                r.mask = c;
                r.owner = (uint32_t)t;
                r.off = off;
                r.cursor = j;
                r.depth = (uint32_t)(d + 1);
                P.p_rec[slot] = r;
                FP[d] = pend & ~(1ull << b);
                FC[d + 1] = c;
                FP[d + 1] = 0;
                FLO[d + 1] = (uint16_t)(i + 1);
                FHI[d + 1] = (uint16_t)nc;
            }
            if (lane < wm) FB[(d + 1) * WMC + lane] = word;
            ++slot;
            ++off;
            ++d;
            wave_sync();
        }
        if (stop) break;
        if (lane == 0) P.desc[t] = off;
    }
    // slots reserved but not used stay free
    for (uint64_t s = slot + (uint64_t)lane; s < slot_end; s += kWave) {
        P.p_rec[s].owner = kPoolFree;
        P.p_rec[s].mask = 0;
    }
}

// Per chunk of 64 pool slots (the unit a wavefront reserves): its used slots
// and their objects, for the scans that place the pool's concepts in the
// store.  One wavefront per chunk, a lane per slot.
__global__ void __launch_bounds__(kBlock) k_pool_chunk_counts(const PoolRec *__restrict__ rec, uint64_t n_chunks,
                                                              uint32_t *__restrict__ used, uint64_t *__restrict__ nobj)
{
    const int lane = lane_id();
    for (uint64_t c = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; c < n_chunks;
         c += (uint64_t)gridDim.x * kWavesPerBlock) {
        const PoolRec r = rec[c * kWave + (uint64_t)lane];
        const bool u = r.owner != kPoolFree;
        const uint32_t pc = u ? (uint32_t)__popcll(r.mask) : 0u;
        const uint64_t bal = __ballot(u);
        const uint32_t objs = wave_sum(pc);
        if (lane == 0) {
            used[c] = (uint32_t)__popcll(bal);
            nobj[c] = objs;
        }
    }
}

// Store concepts [0, K): 1 for a task (at most task_max objects); every
// concept's descendant count starts at 0 (the pool sets the tasks').
__global__ void __launch_bounds__(kBlock) k_pool_task_flags(const uint64_t *__restrict__ loff, uint64_t K,
                                                            int task_max, uint32_t *__restrict__ flag,
                                                            uint32_t *__restrict__ desc)
{
    for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < K; c += (uint64_t)gridDim.x * blockDim.x) {
        flag[c] = loff[c + 1] - loff[c] <= (uint64_t)task_max ? 1u : 0u;
        desc[c] = 0;
    }
}

// The tasks in store order (shallow levels first, whose subtrees are the
// larger ones), at the places the scan of the flags gives.
__global__ void __launch_bounds__(kBlock) k_pool_task_list(const uint32_t *__restrict__ flag,
                                                           const uint64_t *__restrict__ at, uint64_t K,
                                                           uint32_t *__restrict__ tasks)
{
    for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < K; c += (uint64_t)gridDim.x * blockDim.x)
        if (flag[c]) tasks[at[c]] = (uint32_t)c;
}

struct PoolCommitArgs {
    const PoolRec *rec;
    const uint64_t *p_int;
    const uint64_t *dense;  // per chunk of 64 slots: exclusive scan of its used slots
    const uint64_t *ooff;   // per chunk: exclusive scan of its objects
    uint64_t n_chunks;
    uint64_t K0, obj0;      // the store's concepts and list entries before the pool's
    uint64_t n_pool, n_obj; // the pool's concepts and list entries
    int wm;
    uint64_t *intents;
    int32_t *cursor;
    uint64_t *loff;
    uint32_t *objs;
    uint32_t *t_owner, *t_off;  // per pool concept (index - K0): task, offset in its subtree
    uint8_t *t_depth;           // levels below the task
};

// The used slots, in slot order, become store concepts K0, K0 + 1, ...: the
// intent, the cursor, and the object list (the task's list entries at the
// mask's bits, ascending) after the store's last list.  One wavefront per
// chunk of 64 slots, a lane per slot.
__global__ void __launch_bounds__(kBlock) k_pool_commit(PoolCommitArgs A)
{
    const int lane = lane_id();
    for (uint64_t c = (uint64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; c < A.n_chunks;
         c += (uint64_t)gridDim.x * kWavesPerBlock) {
        const uint64_t s = c * kWave + (uint64_t)lane;
        const PoolRec r = A.rec[s];
        const bool u = r.owner != kPoolFree;
        const uint32_t pc = u ? (uint32_t)__popcll(r.mask) : 0u;
        const uint64_t bal = __ballot(u);
        const uint32_t before = wave_excl_scan(pc);
        if (u) {
            const uint64_t i = A.dense[c] + (uint64_t)lanes_below(bal), k = A.K0 + i;
            for (int w = 0; w < A.wm; ++w) A.intents[k * A.wm + w] = A.p_int[s * A.wm + w];
            A.cursor[k] = r.cursor;
            const uint64_t o = A.obj0 + A.ooff[c] + before;
            A.loff[k] = o;
            const uint64_t to = A.loff[r.owner];
            uint64_t q = 0;
            for (uint64_t m = r.mask; m; m &= m - 1ull)
                A.objs[o + q++] = A.objs[to + (uint64_t)(__ffsll((unsigned long long)m) - 1)];
            A.t_owner[i] = r.owner;
            A.t_off[i] = r.off;
            A.t_depth[i] = (uint8_t)r.depth;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) A.loff[A.K0 + A.n_pool] = A.obj0 + A.n_obj;
}

// p[0, n) = v for 32-bit words.
__global__ void __launch_bounds__(kBlock) k_fill_u32(uint32_t *p, uint64_t n, uint32_t v)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// Output positions of the pool's concepts: the task's position, plus one, plus
// the concept's offset in the task's subtree (the subtree is written in output
// order).  The root's own position is 0 (its rank entry holds its size).
__global__ void __launch_bounds__(kBlock) k_tail_position(const uint32_t *__restrict__ owner,
                                                          const uint32_t *__restrict__ off, uint64_t n, uint64_t K0,
                                                          uint32_t *__restrict__ rank)
{
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t o = owner[i];
        rank[K0 + i] = (o == 0 ? 0u : rank[o]) + 1u + off[i];
    }
}

// Per-level and total counts of an enumeration whose store holds the level
// loop's concepts [0, K0) (level l: [lev_lo[l], lev_lo[l + 1])) and the pool's
// [K0, K): every concept is a parent that tests the attributes above its
// cursor outside its intent, so the counts follow from the store alone.
struct PoolStatsArgs {
    const uint64_t *intents;
    const int32_t *cursor;
    const uint64_t *loff;
    uint64_t K, K0;
    int m, wm, nlev, nbins, mid_max;
    uint64_t tail_m;
    const uint64_t *lev_lo;    // nlev + 1
    const uint32_t *t_owner;   // pool concepts
    const uint8_t *t_depth;
    uint64_t *out;             // [2 * nbins]: concepts, tests per level; then POOLSTAT_* sums
};
enum { POOLSTAT_TESTS = 0, POOLSTAT_PAIRS, POOLSTAT_SUMC, POOLSTAT_LOCAL, POOLSTAT_LOCAL_OBJS, POOLSTAT_MID,
       POOLSTAT_MID_OBJS, POOLSTAT_N };

__device__ __forceinline__ int level_of(const uint64_t *lev_lo, int nlev, uint64_t c)
{
    int lo = 0, hi = nlev - 1;  // the last l with lev_lo[l] <= c
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (lev_lo[mid] <= c) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__global__ void __launch_bounds__(kBlock) k_pool_stats(PoolStatsArgs S)
{
    extern __shared__ unsigned long long s_bins[];  // 2 * nbins
    __shared__ uint64_t s_part[POOLSTAT_N][kWavesPerBlock];
    for (int i = threadIdx.x; i < 2 * S.nbins; i += blockDim.x) s_bins[i] = 0;
    __syncthreads();
    uint64_t sum[POOLSTAT_N] = {0, 0, 0, 0, 0, 0, 0};
    for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < S.K; c += (uint64_t)gridDim.x * blockDim.x) {
        int l;
        if (c < S.K0) {
            l = level_of(S.lev_lo, S.nlev, c);
        } else {
            const uint64_t i = c - S.K0;
            l = level_of(S.lev_lo, S.nlev, S.t_owner[i]) + (int)S.t_depth[i];
        }
        const int y = S.cursor[c];
        uint64_t tests = 0;
        for (int u = 0; u < S.wm; ++u) {
            uint64_t x = ~S.intents[c * S.wm + u] & above_mask(y, u);
            if (u == S.wm - 1) x &= S.tail_m;
            tests += (uint64_t)__popcll(x);
        }
        const uint64_t a = S.loff[c + 1] - S.loff[c];
        if (l >= S.nbins) l = S.nbins - 1;  // cannot happen: a level adds an attribute
        atomicAdd(&s_bins[l], 1ull);
        atomicAdd(&s_bins[S.nbins + l], (unsigned long long)tests);
        sum[POOLSTAT_TESTS] += tests;
        sum[POOLSTAT_PAIRS] += (uint64_t)(S.m - 1 - y);
        if (c != 0) sum[POOLSTAT_SUMC] += a;
        if (a <= (uint64_t)kSmallMax) {
            sum[POOLSTAT_LOCAL] += 1;
            sum[POOLSTAT_LOCAL_OBJS] += a;
        } else if (a <= (uint64_t)S.mid_max) {
            sum[POOLSTAT_MID] += 1;
            sum[POOLSTAT_MID_OBJS] += a;
        }
    }
    const int lane = lane_id(), w = threadIdx.x / kWave;
#pragma unroll
    for (int k = 0; k < POOLSTAT_N; ++k) {
        const uint64_t v = wave_sum64(sum[k]);
        if (lane == 0) s_part[k][w] = v;
    }
    __syncthreads();
    if (threadIdx.x < POOLSTAT_N) {
        uint64_t v = 0;
        for (int i = 0; i < kWavesPerBlock; ++i) v += s_part[threadIdx.x][i];
        if (v) atomicAdd((unsigned long long *)&S.out[2 * S.nbins + threadIdx.x], (unsigned long long)v);
    }
    for (int i = threadIdx.x; i < 2 * S.nbins; i += blockDim.x)
        if (s_bins[i]) atomicAdd((unsigned long long *)&S.out[i], s_bins[i]);
}

}  // namespace fcbo
