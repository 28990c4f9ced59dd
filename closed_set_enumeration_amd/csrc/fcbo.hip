// libfcbo host runtime: context, concept store, level loop, sort, output.
// The C ABI is declared in include/fcbo.h.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <chrono>
#include <mutex>
#include <numeric>
#include <new>
#include <vector>

#include "fcbo.h"
#include "fcbo_device.h"

using namespace fcbo;

namespace {

// Error propagation inside the library: every HIP call goes through CK.
struct HipError {
    int code;
};

inline int map_error(hipError_t e)
{
    if (e == hipSuccess) return FCBO_OK;
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) return FCBO_ERR_OUT_OF_MEMORY;
    return FCBO_ERR_DEVICE;
}

#define CK(expr)                                                   \
    do {                                                           \
        hipError_t e_ = (expr);                                    \
        if (e_ != hipSuccess) throw HipError{map_error(e_)};       \
    } while (0)

#define CK_LAUNCH() CK(hipGetLastError())

// An allocation that fails is reported by the call that made it; its error
// must not stay behind as the thread's last error, where the next launch check
// (of this or any other context) would read it as its own failure.
#define CK_ALLOC(expr)                                             \
    do {                                                           \
        hipError_t e_ = (expr);                                    \
        if (e_ != hipSuccess) {                                    \
            (void)hipGetLastError();                               \
            throw HipError{map_error(e_)};                         \
        }                                                          \
    } while (0)

inline uint64_t div_up(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

// Where the enumeration buffers come from: hipMalloc, optionally under a cap
// on the bytes held together (fcbo_set_memory_limit); or, for the entry point
// that allocates nothing, consecutive pieces of a fixed device region that are
// never handed back (the region is reused from its start by the next call).
struct DeviceMemory {
    uint64_t limit = 0;  // bytes the buffers may hold together; 0 = no cap
    uint64_t held = 0;   // bytes they hold now
    uint64_t peak = 0;   // most bytes held at once since the last reset of peak
    char *region = nullptr;  // the fixed region, or null
    uint64_t region_size = 0, region_used = 0;

    void *get(uint64_t bytes)
    {
        if (region) {
            const uint64_t at = (region_used + 255) & ~255ull;
            if (at > region_size || bytes > region_size - at) throw HipError{FCBO_ERR_SCRATCH};
            region_used = at + bytes;
            return region + at;
        }
        if (limit && held + bytes > limit) throw HipError{FCBO_ERR_OUT_OF_MEMORY};
        void *q = nullptr;
        CK_ALLOC(hipMalloc(&q, bytes));
        held += bytes;
        peak = std::max(peak, held);
        return q;
    }
    void put(void *p, uint64_t bytes)
    {
        if (!p || region) return;
        (void)hipFree(p);
        held -= std::min(held, bytes);
    }
};

template <typename T>
void dfree(DeviceMemory &dm, T *&p, uint64_t &cap)
{
    dm.put((void *)p, cap * sizeof(T));
    p = nullptr;
    cap = 0;
}

// Grow a device array to hold at least `need` elements, keeping the first
// `keep` elements.  Capacity grows at least by half to amortise copies.
template <typename T>
void ensure(DeviceMemory &dm, T *&p, uint64_t &cap, uint64_t need, uint64_t keep, hipStream_t s,
            uint64_t min_cap = 1024)
{
    if (need <= cap && p) return;
    // (pieces of the fixed region are not reused: grow faster there)
    uint64_t ncap = std::max<uint64_t>(need, dm.region ? 2 * cap : cap + cap / 2);
    ncap = std::max<uint64_t>(ncap, min_cap);
    T *q = (T *)dm.get(ncap * sizeof(T));
    if (p && keep) {
        hipError_t e = hipMemcpyAsync(q, p, keep * sizeof(T), hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) {
            dm.put(q, ncap * sizeof(T));
            throw HipError{map_error(e)};
        }
    }
    dfree(dm, p, cap);
    p = q;
    cap = ncap;
}

// Per-level counts of an enumeration.  Every level adds an attribute to the
// intent, so there are at most M + 1 <= 4097 levels.
struct LevelLog {
    static constexpr size_t kMax = 4098;
    uint64_t concepts[kMax];  // concepts generated on level k
    uint64_t tests[kMax];     // closure tests made by them
    uint64_t lo[kMax + 1];    // index of level k's first concept (generation order)
    size_t n = 0;
    void clear() { n = 0; lo[0] = 0; }
    void truncate(size_t k) { n = std::min(n, k); }
    size_t size() const { return n; }
    void push(uint64_t c, uint64_t t)
    {
        if (n == kMax) throw HipError{FCBO_ERR_DEVICE};
        concepts[n] = c;
        tests[n] = t;
        lo[n + 1] = lo[n] + c;
        ++n;
    }
};

// Work counts of an enumeration, summed over its levels.
struct Totals {
    uint64_t tests = 0, pairs = 0, sum_c = 0, redos = 0;
    uint64_t local_parents = 0, local_objs = 0, med_parents = 0, med_objs = 0;
    uint64_t big_parents = 0, big_tests = 0, big_scan = 0, big_nzw = 0, big_cobjs = 0;
};

// Where the level loop stands: parents [lo, lo + P) of the store, objects
// used up to obj_hi, and the mid / huge parents expected among them.
struct LevelCursor {
    uint64_t lo = 0, P = 0, obj_hi = 0, next_mid = 0, next_huge = 0;
};

constexpr int kGridCap = 4096;  // blocks for grid-stride wave kernels
// Average children per concept from which the order passes take a wavefront
// per concept (measured: 8 against 4 and 16 on both full-size workloads).
constexpr uint64_t kOrderWaveFanout = 8;

// Device storage of one BigSet (see fcbo_device.h).
struct BigStore {
    uint64_t cap_idx = 0, cap_n = 0, cap_off = 0, cap_t = 0, cap_s = 0, cap_ss = 0, cap_p = 0, cap_bmp = 0;
    uint32_t *idx = nullptr, *n = nullptr, *size = nullptr;
    uint64_t *off = nullptr, *tasks = nullptr, *sscan = nullptr, *plist = nullptr, *bmp = nullptr;

    void free_all(DeviceMemory &dm)
    {
        dfree(dm, idx, cap_idx); dfree(dm, n, cap_n); dfree(dm, size, cap_s); dfree(dm, off, cap_off);
        dfree(dm, tasks, cap_t); dfree(dm, sscan, cap_ss); dfree(dm, plist, cap_p); dfree(dm, bmp, cap_bmp);
    }
    void ensure_members(DeviceMemory &dm, uint64_t P, hipStream_t s, uint64_t mc)
    {
        ensure(dm, idx, cap_idx, P, 0, s, mc);
        ensure(dm, n, cap_n, P, 0, s, mc);
        ensure(dm, off, cap_off, P + 1, 0, s, mc);
    }
    void ensure_tests(DeviceMemory &dm, uint64_t need, hipStream_t s, uint64_t mc)
    {
        ensure(dm, tasks, cap_t, need, 0, s, mc);
        ensure(dm, size, cap_s, need, 0, s, mc);
        ensure(dm, sscan, cap_ss, need + 1, 0, s, mc);
        ensure(dm, plist, cap_p, need, 0, s, mc);
    }
    uint64_t test_cap() const { return std::min(std::min(cap_t, cap_s), std::min(cap_ss ? cap_ss - 1 : 0, cap_p)); }
    BigSet view(int cnt_slot, int tot_slot, int pass_slot, bool bitmaps) const
    {
        BigSet S;
        S.idx = idx; S.n = n; S.off = off; S.tasks = tasks; S.size = size; S.sscan = sscan; S.plist = plist;
        S.cap = test_cap();
        S.bmp = bitmaps ? bmp : nullptr;
        S.bmp_cap = cap_bmp;
        S.cnt_slot = cnt_slot; S.tot_slot = tot_slot; S.pass_slot = pass_slot;
        return S;
    }
};

// A run of sibling concepts kept aside by a bounded enumeration, the seeds of
// its batches: intents, cursors (ascending), extent-list offsets as they were
// in the store, and the lists, which started at store object obj_base.
struct SeedSet {
    uint64_t count = 0, level = 0, obj_base = 0;
    uint64_t hi = 0, B = 0;  // seeds [0, hi) remain; the next batch takes up to B, ending at hi
    uint64_t B_cap = 0;      // no batch larger than this (half of a size that did not fit)
    std::vector<double> wsum;  // prefix sums of the seeds' weights (see enumerate_bounded)
    uint64_t cap_int = 0, cap_cur = 0, cap_loff = 0, cap_obj = 0;
    uint64_t *ints = nullptr;
    int32_t *cur = nullptr;
    uint64_t *loff = nullptr;
    uint32_t *objs = nullptr;
    std::vector<uint64_t> h_loff;
    void free_all(DeviceMemory &dm)
    {
        dfree(dm, ints, cap_int);
        dfree(dm, cur, cap_cur);
        dfree(dm, loff, cap_loff);
        dfree(dm, objs, cap_obj);
    }
};

}  // namespace

struct fcbo_context {
    int device = 0;
    int n_cu = 256;                // compute units of the device
    hipStream_t stream = nullptr;
    int64_t n = 0, m = 0;
    int wn = 0, wm = 0;
    uint64_t tail_m = 0, tail_n = 0;
    bool tiny = false;  // FCBO_TINY_BUFFERS: every buffer starts at its minimum size
    bool fixed = false; // buffers from the static scratch region: no allocation, no events,
                        // no side streams
    DeviceMemory dmem;  // source of the enumeration buffers below
    uint64_t *rows = nullptr;  // n x wm (+1 padding row)
    uint64_t *cols = nullptr;  // m x wn

    // concept store
    uint64_t cap_int = 0, cap_cur = 0, cap_loff = 0, cap_o = 0, cap_fch = 0;
    uint64_t *intents = nullptr;
    int32_t *cursor = nullptr;
    uint64_t *loff = nullptr;
    uint32_t *objs = nullptr;
    uint32_t *fchild = nullptr;  // K + 1: first child of each concept (children are contiguous)

    // level scratch
    uint64_t cap_pass = 0, cap_nch = 0, cap_nob = 0, cap_cb = 0, cap_ob = 0, cap_mid = 0, cap_mrec = 0;
    uint64_t *pass = nullptr, *cbase = nullptr, *obase = nullptr;
    uint32_t *nchild = nullptr, *mid_idx = nullptr;
    uint64_t *nobj = nullptr;
    uint64_t *mrec = nullptr;  // child records of the narrow mid parents (words)
    uint64_t *wrec = nullptr;  // child records of the wide mid parents (words)
    uint64_t cap_wrec = 0;
    uint64_t cap_lrec = 0, cap_lfill = 0;
    uint64_t *lrec = nullptr;  // child records of the local parents (words)
    uint32_t *lfill = nullptr; // records per 64-slot chunk
    BigStore huge;
    uint64_t cap_dt = 0, cap_tcnt = 0, cap_icnt = 0;
    uint64_t *dt = nullptr;                     // huge tests: D accumulators
    uint32_t *tcnt = nullptr, *icnt = nullptr;  // huge tests: |C|, per-chunk counts
    uint64_t *scan_part = nullptr;  // 2 x kScanBlocks
    uint64_t *counters = nullptr;   // 2 x CNT_N: levels alternate between the halves
    int ctr = 0;                    // half of the current level
    uint64_t *h_counters = nullptr; // pinned, CNT_N (h_counters_own when fixed)
    uint64_t h_counters_own[CNT_N];

    // output order
    uint64_t cap_rank = 0, cap_perm = 0;
    uint32_t *rank = nullptr;  // subtree size, then position, of every concept
    uint32_t *perm = nullptr;  // concept at every output position

    // staging buffers of fcbo_copy_to_host (two of each)
    uint64_t cap_hs_int[2] = {0, 0}, cap_hs_ext[2] = {0, 0};
    uint64_t *hs_int[2] = {nullptr, nullptr}, *hs_ext[2] = {nullptr, nullptr};
    hipEvent_t hs_written[2] = {nullptr, nullptr}, hs_copied[2] = {nullptr, nullptr};

    // cover edges
    uint64_t cap_ctable = 0, cap_ccount = 0, cap_coff = 0, cap_cbig = 0, cap_cctr = 0;
    uint32_t *ctable = nullptr;   // concept index by intent (open addressing)
    uint32_t *ccount = nullptr;   // covers per output position
    uint64_t *coff = nullptr;     // their exclusive scan
    uint32_t *cbig = nullptr;     // positions of the concepts with more than 64 objects
    uint64_t *cctr = nullptr;     // [0] their number, [1] covers not found, [2] scratch used, [3] scratch short
    bool have_cover_counts = false;  // ccount / coff / cbig hold the last result's
    uint64_t cover_total = 0;
    // with the counts: the table of concepts by intent is built, and the covers'
    // positions are kept in cscratch (one run per concept, starting at csstart)
    bool cover_table_ok = false, cover_kept = false;
    uint64_t cap_cscratch = 0, cap_csstart = 0;
    uint32_t *cscratch = nullptr;
    uint64_t *csstart = nullptr;

    // seed sets of a bounded enumeration, the deepest last
    std::vector<SeedSet> seeds;

    // task pool: the subtrees of the concepts with at most kPoolTaskMax objects
    bool pool_active = false;  // the level loop leaves such parents to the pool
    bool pool_result = false;  // the last result came from the level loop and the pool
    uint64_t K_sync = 0, n_pool = 0;  // concepts from the level loop, from the pool
    uint64_t pool_cap = 0;            // pool slots of the last run
    LevelLog lev_sync;                // the level loop's levels, walked by the order pass
    uint64_t cap_pint = 0, cap_prec = 0, cap_desc = 0, cap_towner = 0, cap_toff = 0, cap_tdepth = 0;
    uint64_t cap_pctr = 0, cap_levlo = 0, cap_pstat = 0;
    uint64_t *p_int = nullptr;        // pool slots: intents
    PoolRec *p_rec = nullptr;         // pool slots: records
    uint32_t *desc = nullptr;         // concepts below each task
    uint32_t *t_owner = nullptr, *t_off = nullptr;  // per pool concept: task, offset in its subtree
    uint8_t *t_depth = nullptr;       // per pool concept: levels below the task
    uint64_t *pool_ctr = nullptr;     // POOL_* counters
    uint64_t *task_ctr = nullptr;     // the pool's claim counters
    uint32_t *ptasks = nullptr;       // the pool's tasks
    uint64_t cap_tctr = 0, cap_ptasks = 0;
    uint64_t *d_levlo = nullptr;      // the level loop's level starts, for the counts
    uint64_t *pstat = nullptr;        // per-level and total counts

    // result of the last enumeration
    bool have_levels = false;  // lev holds the per-level counts of a complete enumeration
    bool have_result = false;
    bool have_perm = false;
    uint64_t K = 0, order_launches = 0;
    uint64_t store_rows_seen = 0;  // concepts the store was being sized for, last seen by the level loop
    Totals tot;
    LevelLog lev;

    // profiling
    bool profile = false;
    std::vector<hipEvent_t> ev_pool;
    hipEvent_t ev_counts = nullptr;  // a level's counters have reached the host
    size_t ev_used = 0;
    std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> marks;

    hipEvent_t ev_get()
    {
        if (ev_used == ev_pool.size()) {
            hipEvent_t e;
            CK(hipEventCreate(&e));
            ev_pool.push_back(e);
        }
        return ev_pool[ev_used++];
    }
    hipEvent_t prof_begin(hipStream_t s = nullptr)
    {
        if (!profile) return nullptr;
        hipEvent_t e = ev_get();
        CK(hipEventRecord(e, s ? s : stream));
        return e;
    }
    void prof_end(int cls, hipEvent_t b, hipStream_t s = nullptr)
    {
        if (!profile) return;
        hipEvent_t e = ev_get();
        CK(hipEventRecord(e, s ? s : stream));
        marks.push_back({cls, {b, e}});
    }

    // Side streams for work of a level that is independent of the main
    // stream's (different parents, different counters: the huge and the wide
    // mid parents' tests beside the narrow ones, the writers of the classes
    // beside each other); forked from and joined back to the main stream
    // through events.  Default priority, like the caller's stream.
    static constexpr int kSide = 2;
    hipStream_t aux[kSide] = {nullptr, nullptr};
    hipEvent_t ev_fork[kSide] = {nullptr, nullptr}, ev_join[kSide] = {nullptr, nullptr};
    hipStream_t fork(int i)
    {
        if (!aux[i]) CK(hipStreamCreateWithFlags(&aux[i], hipStreamNonBlocking));
        if (!ev_fork[i]) CK(hipEventCreateWithFlags(&ev_fork[i], hipEventDisableTiming));
        if (!ev_join[i]) CK(hipEventCreateWithFlags(&ev_join[i], hipEventDisableTiming));
        CK(hipEventRecord(ev_fork[i], stream));
        CK(hipStreamWaitEvent(aux[i], ev_fork[i], 0));
        return aux[i];
    }
    void join(int i)
    {
        CK(hipEventRecord(ev_join[i], aux[i]));
        CK(hipStreamWaitEvent(stream, ev_join[i], 0));
    }

    uint64_t min_cap() const { return tiny ? 1 : 1024; }
    // first size of a buffer that normally starts at `normal` elements of
    // elem_bytes bytes; under a memory limit none starts above 1/64 of it
    uint64_t start_size(uint64_t normal, uint64_t elem_bytes = 8) const
    {
        if (tiny) return 1;
        if (fixed) return std::max<uint64_t>(64, normal / 64);
        if (dmem.limit) return std::max<uint64_t>(64, std::min<uint64_t>(normal, dmem.limit / 64 / elem_bytes));
        return normal;
    }
    void clear_words(uint64_t *p, uint64_t n)
    {
        const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(1024, div_up(n, kBlock)));
        hipLaunchKernelGGL(k_fill_u64, dim3(g), dim3(kBlock), 0, stream, p, n, 0ull);
        CK_LAUNCH();
    }
    void setup(const uint64_t *rows_in, int64_t n_objects, int64_t n_attrs, int64_t row_stride_words,
               bool rows_on_device);

    bool use_bitmaps() const { return wn <= kBmpMaxWords; }
    int nchunk() const { return (int)div_up((uint64_t)wn, kWave); }

    // the per-level scratch of the level loop (the concept store and the
    // output order stay): released where later work needs the memory, grown
    // again by the next enumeration
    void free_level_scratch()
    {
        dfree(dmem, pass, cap_pass); dfree(dmem, cbase, cap_cb); dfree(dmem, obase, cap_ob);
        dfree(dmem, nchild, cap_nch); dfree(dmem, nobj, cap_nob); dfree(dmem, mid_idx, cap_mid);
        dfree(dmem, mrec, cap_mrec); dfree(dmem, wrec, cap_wrec); dfree(dmem, lrec, cap_lrec);
        dfree(dmem, lfill, cap_lfill);
        huge.free_all(dmem);
        dfree(dmem, dt, cap_dt); dfree(dmem, tcnt, cap_tcnt); dfree(dmem, icnt, cap_icnt);
    }

    // the enumeration's buffers (the context's rows, columns and counters stay)
    void free_buffers()
    {
        dfree(dmem, intents, cap_int); dfree(dmem, cursor, cap_cur); dfree(dmem, loff, cap_loff);
        dfree(dmem, objs, cap_o); dfree(dmem, fchild, cap_fch);
        dfree(dmem, pass, cap_pass); dfree(dmem, cbase, cap_cb); dfree(dmem, obase, cap_ob);
        dfree(dmem, nchild, cap_nch); dfree(dmem, nobj, cap_nob); dfree(dmem, mid_idx, cap_mid);
        dfree(dmem, mrec, cap_mrec); dfree(dmem, wrec, cap_wrec); dfree(dmem, lrec, cap_lrec);
        dfree(dmem, lfill, cap_lfill);
        huge.free_all(dmem);
        dfree(dmem, dt, cap_dt); dfree(dmem, tcnt, cap_tcnt); dfree(dmem, icnt, cap_icnt);
        dfree(dmem, rank, cap_rank); dfree(dmem, perm, cap_perm);
        dfree(dmem, ctable, cap_ctable); dfree(dmem, ccount, cap_ccount); dfree(dmem, coff, cap_coff);
        dfree(dmem, cbig, cap_cbig); dfree(dmem, cctr, cap_cctr);
        dfree(dmem, cscratch, cap_cscratch); dfree(dmem, csstart, cap_csstart);
        release_seeds();
        release_pool();
        for (int b = 0; b < 2; ++b) {
            dfree(dmem, hs_int[b], cap_hs_int[b]);
            dfree(dmem, hs_ext[b], cap_hs_ext[b]);
        }
        have_result = have_perm = have_cover_counts = have_levels = pool_result = false;
    }

    void free_all()
    {
        free_buffers();
        for (void *q : {(void *)rows, (void *)cols, (void *)scan_part, (void *)counters})
            if (q) (void)hipFree(q);
        rows = cols = scan_part = counters = nullptr;
        if (h_counters && h_counters != h_counters_own) (void)hipHostFree(h_counters);
        h_counters = nullptr;
        for (hipEvent_t e : ev_pool) (void)hipEventDestroy(e);
        ev_pool.clear();
        if (ev_counts) (void)hipEventDestroy(ev_counts);
        ev_counts = nullptr;
        for (int b = 0; b < 2; ++b) {
            if (hs_written[b]) (void)hipEventDestroy(hs_written[b]);
            if (hs_copied[b]) (void)hipEventDestroy(hs_copied[b]);
            hs_written[b] = hs_copied[b] = nullptr;
        }
        for (int i = 0; i < kSide; ++i) {
            if (ev_fork[i]) (void)hipEventDestroy(ev_fork[i]);
            if (ev_join[i]) (void)hipEventDestroy(ev_join[i]);
            if (aux[i]) (void)hipStreamDestroy(aux[i]);
            ev_fork[i] = ev_join[i] = nullptr;
            aux[i] = nullptr;
        }
    }

    // per-test buffers of the huge set (its BigStore plus the accumulators)
    void ensure_huge_tests(uint64_t need)
    {
        huge.ensure_tests(dmem, need, stream, min_cap());
        ensure(dmem, dt, cap_dt, need * wm, 0, stream, min_cap());
        ensure(dmem, tcnt, cap_tcnt, need, 0, stream, min_cap());
        ensure(dmem, icnt, cap_icnt, need * nchunk(), 0, stream, min_cap());
    }

    LevelArgs level_args(uint64_t lo, uint64_t P, uint64_t obj_hi) const
    {
        LevelArgs A;
        memset(&A, 0, sizeof(A));
        A.rows = rows; A.cols = cols;
        A.n = (int)n; A.m = (int)m; A.wn = wn; A.wm = wm; A.tail_m = tail_m; A.tail_n = tail_n;
        A.intents = intents; A.cursor = cursor; A.loff = loff; A.objs = objs;
        A.lo = lo; A.P = P; A.child_lo = lo + P; A.child_obj_lo = obj_hi;
        A.pass = pass; A.pass_cap = cap_pass / (uint64_t)wm; A.nchild = nchild; A.nobj = nobj; A.cbase = cbase; A.obase = obase;
        A.mid_idx = mid_idx;
        A.mid_max = wm <= 8 ? kMidMax : kSmallMax;
        A.mrec = mrec;
        A.mrec_region = cap_mrec / (4 + (uint64_t)wm) / kRecStripes;
        A.wrec = wrec;
        A.wrec_cap = cap_wrec / (4 + (uint64_t)wm);
        A.lrec = lrec;
        A.lfill = lfill;
        A.lrec_region = std::min(cap_lrec / (4 + (uint64_t)wm), cap_lfill * kWave) / kRecStripes / kWave * kWave;
        const bool bm = use_bitmaps();
        A.huge = huge.view(CNT_HUGE, CNT_THUGE, CNT_HUGEPASS, bm);
        if (bm) A.huge.cap = std::min(A.huge.cap, std::min(std::min(cap_dt / wm, cap_tcnt), cap_icnt / nchunk()));
        A.dt = dt; A.tcnt = tcnt; A.icnt = icnt;
        A.nchunk = nchunk();
        A.counters = counters + (uint64_t)ctr * CNT_N;
        A.counters_next = counters + (uint64_t)(1 - ctr) * CNT_N;
        A.child_cap = std::min(std::min(cap_int / (uint64_t)wm, cap_cur), cap_loff ? cap_loff - 1 : 0);
        A.obj_cap = cap_o > kObjSlack ? cap_o - kObjSlack : 0;  // the output kernel reads past the last list
        A.pool_max = pool_active ? kPoolTaskMax : -1;
        return A;
    }

    // exclusive scan (see k_scan_*): a (and b) -> out_a (and out_b), n from the
    // device or the host; fch (optional) receives fbase + out_a as u32.
    void scan(const uint32_t *a, const uint64_t *b, const uint64_t *n_dev, uint64_t n_host, uint64_t n_cap,
              uint64_t *out_a, uint64_t *out_b, uint64_t *tot_a, uint64_t *tot_b, uint32_t *fch = nullptr,
              uint64_t fbase = 0, hipStream_t s = nullptr, bool small = false)
    {
        // One workgroup when the length is known to be small, or expected to
        // be (`small`, with the length in device memory: correct for any
        // length, only slower if the expectation fails).
        const hipStream_t stream = s ? s : this->stream;
        if ((!n_dev && n_host <= kScanSmallMax) || (n_dev && small)) {
            hipLaunchKernelGGL(k_scan_small, dim3(1), dim3(kScanBlocks), 0, stream, a, b, n_dev,
                               n_dev ? n_cap : std::min(n_host, n_cap), out_a, out_b, tot_a, tot_b, fch, fbase);
            CK_LAUNCH();
            return;
        }
        int nb = kScanBlocks;
        if (!n_dev) nb = (int)std::min<uint64_t>(kScanBlocks, std::max<uint64_t>(1, div_up(n_host, 4 * kBlock)));
        hipLaunchKernelGGL(k_scan_up, dim3(nb), dim3(kBlock), 0, stream, a, b, n_dev, n_host, n_cap, scan_part);
        CK_LAUNCH();
        hipLaunchKernelGGL(k_scan_mid, dim3(1), dim3(kScanBlocks), 0, stream, scan_part, nb, n_dev, n_host, n_cap,
                           out_a, out_b, tot_a, tot_b, fch, fbase);
        CK_LAUNCH();
        hipLaunchKernelGGL(k_scan_down, dim3(nb), dim3(kBlock), 0, stream, a, b, n_dev, n_host, n_cap,
                           (const uint64_t *)scan_part, out_a, out_b, fch, fbase);
        CK_LAUNCH();
    }

    // local child records: `slots` rounded up to whole 64-slot chunks
    void ensure_local_records(uint64_t slots)
    {
        const uint64_t chunks = div_up(slots, kWave) + 1;
        ensure(dmem, lrec, cap_lrec, chunks * kWave * (4 + (uint64_t)wm), 0, stream, 1);
        ensure(dmem, lfill, cap_lfill, chunks, 0, stream, 1);
    }
    void start_root(LevelCursor &s);
    void run_levels(LevelCursor &s, uint64_t max_levels);
    void enumerate_levels(bool pool = false);
    // the task pool's buffers (its slots, task list and per-concept arrays)
    void release_pool()
    {
        drain_quiet();
        dfree(dmem, p_int, cap_pint); dfree(dmem, p_rec, cap_prec); dfree(dmem, desc, cap_desc);
        dfree(dmem, t_owner, cap_towner); dfree(dmem, t_off, cap_toff); dfree(dmem, t_depth, cap_tdepth);
        dfree(dmem, pool_ctr, cap_pctr); dfree(dmem, d_levlo, cap_levlo); dfree(dmem, pstat, cap_pstat);
        dfree(dmem, task_ctr, cap_tctr); dfree(dmem, ptasks, cap_ptasks);
        pool_cap = 0;
        pool_result = false;
    }
    // wait for the context's streams, ignoring errors (before freeing after a failure)
    void drain_quiet()
    {
        for (int i = 0; i < kSide; ++i)
            if (aux[i]) (void)hipStreamSynchronize(aux[i]);
        (void)hipStreamSynchronize(stream);
    }
    void run_pool(uint64_t K0, uint64_t obj0);
    void enumerate_bounded(uint64_t *intents_buf, uint64_t *extents_buf, uint64_t piece_rows, fcbo_sink_fn sink,
                           void *user, uint32_t flags, fcbo_stats &st);
    void capture_seeds(uint64_t first, uint64_t count, uint64_t obj_lo, uint64_t obj_hi, uint64_t level);
    void release_seeds();
    LevelCursor load_seeds(const SeedSet &S, uint64_t a, uint64_t B, bool announce_classes = true);
    void harvest_marks(fcbo_stats &st);
    void drain();
    void order_concepts();
    void write_output(uint64_t *intents_out, uint64_t *extents_out, uint64_t first, uint64_t count);
    uint64_t model_bytes(uint64_t k) const;  // of an enumeration of k concepts with the totals in tot
    void fill_counts(fcbo_stats &st, uint64_t k) const;
    uint64_t cover_edges(uint64_t *offsets_out, uint32_t *targets_out, uint64_t capacity);
    void copy_to_host(uint64_t first, uint64_t count, uint64_t *host_intents, uint64_t *host_extents,
                      uint64_t staging_rows);
};

namespace {

// Which parent classes a level has: the local test kernel always runs (it also
// counts and classifies); the mid and huge kernels only when the level holds
// such parents.
enum { kLevelMid = 1, kLevelHuge = 2, kLevelSide = 4 };
// A level runs independent parts on the side streams only when it has huge
// parents (the shallow levels, whose huge and wide tests under-fill the
// device): a fork and join cost the main stream some 20 us of idle time, more
// than the overlap gains on the deeper levels.

template <int WMC>
void launch_level_tests(fcbo_context *c, const LevelArgs &A, uint64_t P, unsigned classes, uint64_t n_huge)
{
    // n_huge: the huge parents expected on the level (the previous level's
    // count of such children); their scans take one workgroup when few
    const bool huge_small = n_huge <= kScanSmallMax;
    const bool tests_small = n_huge * (uint64_t)c->m <= kScanSmallMax;
    const unsigned gm = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(1024, div_up(P, kWavesPerBlock)));
    const bool bm = A.huge.bmp != nullptr;
    // local tests; the same pass counts every parent's tests and lists the mid
    // and huge parents
    hipEvent_t b = c->prof_begin();
    {
        constexpr int kW = LocalCfg<WMC>::kWaves;
        LevelArgs L = A;
        L.chunk = LocalCfg<WMC>::kChunk;
        const uint64_t want = (uint64_t)c->n_cu * kLocalChunksPerCu;
        while (L.chunk / 2 >= kLocalMinChunk && div_up(P, (uint64_t)L.chunk) < want) L.chunk /= 2;
        const uint64_t chunks = div_up(P, (uint64_t)L.chunk);
        const uint64_t per_block = (uint64_t)kW * LocalCfg<WMC>::kChunksPerWave;
        const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(65535, div_up(chunks, per_block)));
        hipLaunchKernelGGL(k_local_test<WMC>, dim3(g), dim3(LocalCfg<WMC>::kThreads), 0, c->stream, L);
    }
    CK_LAUNCH();
    c->prof_end(FCBO_K_TEST_LOCAL, b);
    // With mid parents on the level too, the huge parents' tests (a few
    // under-filled launches) run on the second stream beside the mid tests:
    // the two touch different parents and different counters.
    const bool mid = (classes & kLevelMid) && WMC <= 8;
    const bool use_side = (classes & kLevelSide) != 0;
    const bool side = (classes & kLevelHuge) && mid && use_side;
    const hipStream_t hs = side ? c->fork(0) : c->stream;
    if (classes & kLevelHuge) {
        // test offsets of the huge parents; total -> counters
        b = c->prof_begin(hs);
        c->scan(c->huge.n, nullptr, A.counters + CNT_HUGE, 0, P, c->huge.off, nullptr, A.counters + CNT_THUGE,
                nullptr, nullptr, 0, hs, huge_small);
        c->prof_end(FCBO_K_SCAN, b, hs);
        b = c->prof_begin(hs);
        hipLaunchKernelGGL(k_huge_tasks<WMC>, dim3(gm), dim3(kBlock), 0, hs, A);
        CK_LAUNCH();
        c->prof_end(FCBO_K_TEST_BIG, b, hs);
    }
    if constexpr (WMC <= 8) {
        if (classes & kLevelMid) {
            // wide parents on a side stream, narrow ones on the main stream
            const hipStream_t ws = use_side ? c->fork(1) : c->stream;
            b = c->prof_begin(ws);
            const unsigned gw = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(P, 4 * (uint64_t)c->n_cu));
            hipLaunchKernelGGL(k_mid_test_wide<WMC>, dim3(gw), dim3(kWideThreads), 0, ws, A);
            CK_LAUNCH();
            c->prof_end(FCBO_K_TEST_MEDIUM, b, ws);
            b = c->prof_begin();
            const unsigned gmid = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(2048, div_up(P, kMidWaves)));
            hipLaunchKernelGGL(k_mid_test<WMC>, dim3(gmid), dim3(kWave * kMidWaves), 0, c->stream, A);
            CK_LAUNCH();
            c->prof_end(FCBO_K_TEST_MEDIUM, b);
            if (use_side) c->join(1);
        }
    }
    if (!(classes & kLevelHuge)) return;
    b = c->prof_begin(hs);
    if (bm) {
        hipLaunchKernelGGL(k_huge_partial<WMC>, dim3(kGridCap), dim3(kBlock), 0, hs, A);
        CK_LAUNCH();
        hipLaunchKernelGGL(k_huge_finalize, dim3(1024), dim3(kBlock), 0, hs, A);
    } else {
        hipLaunchKernelGGL(k_big_test_list<WMC>, dim3(kGridCap), dim3(kBlock), 0, hs, A);
    }
    CK_LAUNCH();
    c->prof_end(FCBO_K_TEST_BIG, b, hs);
    // sibling offsets of the passing huge tests
    b = c->prof_begin(hs);
    c->scan(c->huge.size, nullptr, A.counters + CNT_THUGE, 0, A.huge.cap, c->huge.sscan, nullptr, nullptr, nullptr,
            nullptr, 0, hs, tests_small);
    c->prof_end(FCBO_K_SCAN, b, hs);
    if (side) c->join(0);
}

template <int WMC>
void launch_level_writes(fcbo_context *c, const LevelArgs &A, uint64_t P, unsigned classes, uint64_t)
{
    // the local writer: four threads per parent (a thread walks record slots
    // through a chain of dependent loads; more of them in flight measured
    // best at 4x, 58 -> 57 ms on ctx20000x256)
    const unsigned gl = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(4 * kGridCap, div_up(4 * P, kBlock)));
    // the mid parents' writers run beside the local one (different children)
    const bool mid = (classes & kLevelMid) && WMC <= 8;
    const bool use_side = mid && (classes & kLevelSide) != 0;
    hipStream_t s0 = c->stream, s1 = c->stream;
    if (use_side) {
        s0 = c->fork(0);
        s1 = c->fork(1);
    }
    hipEvent_t b = c->prof_begin();
    hipLaunchKernelGGL(k_local_write<WMC>, dim3(gl), dim3(kBlock), 0, c->stream, A);
    CK_LAUNCH();
    c->prof_end(FCBO_K_WRITE_LOCAL, b);
    if (classes & kLevelHuge) {  // main stream, beside the mid writers
        b = c->prof_begin();
        if (A.huge.bmp)
            hipLaunchKernelGGL(k_huge_write<WMC>, dim3(kGridCap), dim3(kBlock), 0, c->stream, A);
        else
            hipLaunchKernelGGL(k_big_write_list<WMC>, dim3(kGridCap), dim3(kBlock), 0, c->stream, A);
        CK_LAUNCH();
        c->prof_end(FCBO_K_WRITE_BIG, b);
    }
    if constexpr (WMC <= 8) {
        if (mid) {
            b = c->prof_begin(s0);
            hipLaunchKernelGGL(k_mid_write<WMC>, dim3(kGridCap), dim3(kBlock), 0, s0, A);
            CK_LAUNCH();
            c->prof_end(FCBO_K_WRITE_MEDIUM, b, s0);
            b = c->prof_begin(s1);
            hipLaunchKernelGGL(k_mid_write_wide<WMC>, dim3(kGridCap), dim3(kBlock), 0, s1, A);
            CK_LAUNCH();
            c->prof_end(FCBO_K_WRITE_MEDIUM, b, s1);
            if (use_side) {
                c->join(0);
                c->join(1);
            }
        }
    }
}

typedef void (*level_fn)(fcbo_context *, const LevelArgs &, uint64_t, unsigned, uint64_t);

struct LevelFns {
    level_fn tests, writes;
};

LevelFns pick_level_fns(int wm)
{
    switch (wm) {
    case 1: return {launch_level_tests<1>, launch_level_writes<1>};
    case 2: return {launch_level_tests<2>, launch_level_writes<2>};
    case 3: return {launch_level_tests<3>, launch_level_writes<3>};
    case 4: return {launch_level_tests<4>, launch_level_writes<4>};
    case 5: return {launch_level_tests<5>, launch_level_writes<5>};
    case 6: return {launch_level_tests<6>, launch_level_writes<6>};
    case 7: return {launch_level_tests<7>, launch_level_writes<7>};
    case 8: return {launch_level_tests<8>, launch_level_writes<8>};
    default:
        if (wm <= 16) return {launch_level_tests<16>, launch_level_writes<16>};
        if (wm <= 32) return {launch_level_tests<32>, launch_level_writes<32>};
        return {launch_level_tests<64>, launch_level_writes<64>};
    }
}

static_assert(POOL_CTR_N <= CNT_N, "the pool's counters are read through the level counters' host buffer");
static_assert(kPoolTaskMax <= kSmallMax, "pool tasks keep their objects in one wavefront");

typedef void (*pool_fn)(fcbo_context *, const PoolArgs &);

template <int WMC>
void launch_pool(fcbo_context *c, const PoolArgs &PA)
{
    // as many workgroups as are resident at once: the tasks are taken from a
    // counter, so more would only queue behind them
    int per_cu = 1;
    CK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_pool<WMC>, kWave * kPoolWaves, 0));
    const uint64_t resident = (uint64_t)c->n_cu * std::max(1, per_cu);
    const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(resident, div_up(PA.n_tasks, kPoolWaves)));
    hipLaunchKernelGGL(k_pool<WMC>, dim3(g), dim3(kWave * kPoolWaves), 0, c->stream, PA);
    CK_LAUNCH();
}

pool_fn pick_pool_fn(int wm)
{
    switch (wm) {
    case 1: return launch_pool<1>;
    case 2: return launch_pool<2>;
    case 3: return launch_pool<3>;
    case 4: return launch_pool<4>;
    case 5: return launch_pool<5>;
    case 6: return launch_pool<6>;
    case 7: return launch_pool<7>;
    default: return launch_pool<8>;
    }
}

}  // namespace

// Reset the result and run the root: its intent G' and extent G at store
// index 0; s is left at the root level.
void fcbo_context::start_root(LevelCursor &s)
{
    const uint64_t mc = min_cap();
    const bool bm = use_bitmaps();
    // nothing of an earlier result survives a failure part-way through
    have_result = have_perm = have_cover_counts = have_levels = pool_result = false;
    K = 0;
    // the last result's cover runs (their room goes to the enumeration)
    dfree(dmem, cscratch, cap_cscratch);
    dfree(dmem, csstart, cap_csstart);
    ensure(dmem, intents, cap_int, (uint64_t)wm * 1024, 0, stream, mc);
    ensure(dmem, cursor, cap_cur, 1024, 0, stream, mc);
    ensure(dmem, loff, cap_loff, 1025, 0, stream, mc);
    ensure(dmem, objs, cap_o, (uint64_t)n + kObjSlack, 0, stream, mc);
    {
        uint64_t t = std::max<uint64_t>((uint64_t)n, (uint64_t)wm);
        hipLaunchKernelGGL(k_root_init, dim3((unsigned)div_up(t, kBlock)), dim3(kBlock), 0, stream, intents, cursor,
                           loff, objs, (int)n, wm, tail_m);
        CK_LAUNCH();
        unsigned gx = (unsigned)std::min<uint64_t>(256, div_up((uint64_t)n, kBlock));
        hipLaunchKernelGGL(k_root_and, dim3(gx, wm), dim3(kBlock), 0, stream, (const uint64_t *)rows, intents,
                           (int)n, wm);
        CK_LAUNCH();
    }
    lev.clear();
    tot = Totals{};
    const uint64_t rstride = 4 + (uint64_t)wm;
    if (!huge.tasks) {
        if (bm) ensure_huge_tests(start_size(1u << 16, 8 * (4 + (uint64_t)wm + (uint64_t)nchunk())));
        else huge.ensure_tests(dmem, start_size(1u << 20, 32), stream, mc);
    }
    if (bm && !huge.bmp) ensure(dmem, huge.bmp, huge.cap_bmp, (uint64_t)wn * start_size(64, 8 * (uint64_t)wn), 0, stream, 1);
    if (!mrec) ensure(dmem, mrec, cap_mrec, rstride * start_size(1u << 18, 8 * rstride), 0, stream, 1);
    if (!wrec) ensure(dmem, wrec, cap_wrec, rstride * start_size(1u << 16, 8 * rstride), 0, stream, 1);
    if (!lrec) ensure_local_records(tiny ? kWave : start_size(1u << 21, 8 * rstride));
    s = LevelCursor{};
    s.P = 1;
    s.obj_hi = (uint64_t)n;
    // parents of each class on the level about to run (the root: N objects);
    // later levels learn them from the children counted by the test kernels
    const uint64_t mid_max = wm <= 8 ? (uint64_t)kMidMax : (uint64_t)kSmallMax;
    s.next_mid = ((uint64_t)n > (uint64_t)kSmallMax && (uint64_t)n <= mid_max) ? 1 : 0;
    s.next_huge = (uint64_t)n > mid_max ? 1 : 0;
    ctr = 0;
    clear_words(counters, 2 * CNT_N);
}

// Expand up to max_levels levels from s (parents [s.lo, s.lo + s.P)): test,
// count, grow the store, write the children; s moves to the children.
void fcbo_context::run_levels(LevelCursor &s, uint64_t max_levels)
{
    const LevelFns fns = pick_level_fns(wm);
    const uint64_t mc = min_cap();
    const bool bm = use_bitmaps();
    const uint64_t rstride = 4 + (uint64_t)wm;
    uint64_t lo = s.lo, P = s.P, obj_hi = s.obj_hi, next_mid = s.next_mid, next_huge = s.next_huge;
    for (uint64_t done = 0; P > 0 && done < max_levels; ++done) {
        store_rows_seen = lo + P;
        if (lo + P >= (1ull << 32)) throw HipError{FCBO_ERR_LIMIT};  // concept indices are 32-bit
        // every level adds an attribute to the intent, so there are at most M + 1
        if (lev.size() > (size_t)m + 1) throw HipError{FCBO_ERR_DEVICE};
        ensure(dmem, pass, cap_pass, std::max<uint64_t>(1, next_huge) * wm, 0, stream, mc);
        ensure(dmem, nchild, cap_nch, P, 0, stream, mc);
        ensure(dmem, nobj, cap_nob, P, 0, stream, mc);
        ensure(dmem, cbase, cap_cb, P + 1, 0, stream, mc);
        ensure(dmem, obase, cap_ob, P + 1, 0, stream, mc);
        ensure(dmem, mid_idx, cap_mid, P, 0, stream, mc);
        ensure(dmem, fchild, cap_fch, lo + P + 1, lo + 1, stream, mc);
        huge.ensure_members(dmem, P, stream, mc);
        unsigned classes = (next_mid ? kLevelMid : 0u) | (next_huge ? kLevelHuge : 0u) |
                           (next_huge && !fixed ? kLevelSide : 0u);
        bool redo;
        int redos = 0;
        uint64_t huge_seen = next_huge;  // huge parents counted by the last attempt
        uint64_t n_children = 0, n_objs = 0;
        do {
            redo = false;
            // a grown buffer always fits the redo; a class miss turns every kernel on
            if (redos > 3) throw HipError{FCBO_ERR_DEVICE};
            LevelArgs A = level_args(lo, P, obj_hi);
            if (redos) clear_words(A.counters, CNT_N);
            fns.tests(this, A, P, classes, redos ? huge_seen : next_huge);
            hipEvent_t b = prof_begin();
            // child offsets per parent, and the first child of every parent
            scan(nchild, nobj, nullptr, P, P, cbase, obase, A.counters + CNT_CHILDREN, A.counters + CNT_OBJS,
                 fchild + lo, lo + P);
            prof_end(FCBO_K_SCAN, b);
            CK(hipMemcpyAsync(h_counters, A.counters, CNT_N * sizeof(uint64_t), hipMemcpyDeviceToHost, stream));
            if (!fixed) {
                if (!ev_counts) CK(hipEventCreateWithFlags(&ev_counts, hipEventDisableTiming));
                CK(hipEventRecord(ev_counts, stream));
            }
            // The children are written before the host has read the counts, so the
            // device works on while the host prepares the next level.  The write
            // kernels do nothing when the level overflowed or the store has no
            // room; both cases are handled below.
            fns.writes(this, A, P, classes, 0);
            if (fixed) CK(hipStreamSynchronize(stream));
            else CK(hipEventSynchronize(ev_counts));
            const uint64_t n_mid = h_counters[CNT_MID] + h_counters[CNT_MIDW];
            const unsigned found = (n_mid ? kLevelMid : 0u) | (h_counters[CNT_HUGE] ? kLevelHuge : 0u);
            huge_seen = h_counters[CNT_HUGE];
            if (found & ~classes) {  // parents of a class whose kernels did not run
                classes |= found;
                ensure(dmem, pass, cap_pass, std::max<uint64_t>(1, h_counters[CNT_HUGE]) * wm, 0, stream, mc);
                redo = true;
                ++redos;
                ++tot.redos;
                continue;
            }
            if (h_counters[CNT_OVERFLOW]) {
                if (bm) {
                    ensure_huge_tests(h_counters[CNT_THUGE]);
                    ensure(dmem, huge.bmp, huge.cap_bmp, h_counters[CNT_HUGE] * (uint64_t)wn, 0, stream, 1);
                } else {
                    huge.ensure_tests(dmem, h_counters[CNT_THUGE], stream, mc);
                }
                uint64_t stripe_max = 0;
                for (int t = 0; t < kRecStripes; ++t)
                    stripe_max = std::max<uint64_t>(stripe_max, h_counters[CNT_MIDREC + t * kCntPad]);
                // headroom: the split of records over stripes varies from run to run
                ensure(dmem, mrec, cap_mrec, stripe_max * kRecStripes * rstride / 4 * 5, 0, stream, 1);
                ensure(dmem, wrec, cap_wrec, h_counters[CNT_WIDEREC] * rstride, 0, stream, 1);
                ensure(dmem, pass, cap_pass, std::max<uint64_t>(1, h_counters[CNT_HUGE]) * wm, 0, stream, mc);
                uint64_t lstripe_max = 0;
                for (int t = 0; t < kRecStripes; ++t)
                    lstripe_max = std::max<uint64_t>(lstripe_max, h_counters[CNT_LOCREC + t * kCntPad]);
                ensure_local_records(lstripe_max * kRecStripes / 4 * 5);
                redo = true;
                ++redos;
                ++tot.redos;
                continue;
            }
            n_children = h_counters[CNT_CHILDREN];
            n_objs = h_counters[CNT_OBJS];
            next_mid = h_counters[CNT_NEXT_MID];
            next_huge = h_counters[CNT_NEXT_HUGE];
            lev.push(P, h_counters[CNT_TESTS]);
            tot.tests += h_counters[CNT_TESTS];
            tot.pairs += h_counters[CNT_PAIRS];
            tot.sum_c += n_objs;
            tot.big_parents += h_counters[CNT_HUGE];
            tot.med_parents += n_mid;
            tot.local_parents += P - h_counters[CNT_HUGE] - n_mid;
            tot.local_objs += h_counters[CNT_SMALL_OBJS];
            tot.med_objs += h_counters[CNT_MID_OBJS];
            tot.big_tests += h_counters[CNT_THUGE];
            tot.big_scan += h_counters[CNT_BIG_SCAN];
            tot.big_nzw += h_counters[CNT_HUGE_NZW];
            tot.big_cobjs += h_counters[CNT_HUGE_COBJS];
            // room for the children in the store; the writes issued above did
            // nothing if it had to grow
            const uint64_t k_end = lo + P + n_children;
            const uint64_t keep_k = lo + P;
            store_rows_seen = k_end;
            // first-child offsets (u32) of this level already wrapped if so
            if (k_end >= (1ull << 32)) throw HipError{FCBO_ERR_LIMIT};
            const bool had_room = k_end <= A.child_cap && obj_hi + n_objs <= A.obj_cap;
            ensure(dmem, intents, cap_int, k_end * wm, keep_k * wm, stream, mc);
            ensure(dmem, cursor, cap_cur, k_end, keep_k, stream, mc);
            ensure(dmem, loff, cap_loff, k_end + 1, keep_k + 1, stream, mc);
            ensure(dmem, objs, cap_o, obj_hi + n_objs + kObjSlack, obj_hi, stream, mc);
            ensure(dmem, fchild, cap_fch, k_end + 1, keep_k + 1, stream, mc);
            if (n_children && !had_room) fns.writes(this, level_args(lo, P, obj_hi), P, classes, 0);
        } while (redo);
        ctr ^= 1;
        lo += P;
        P = n_children;
        obj_hi += n_objs;
        s.lo = lo;
        s.P = P;
        s.obj_hi = obj_hi;
        s.next_mid = next_mid;
        s.next_huge = next_huge;
    }
}

void fcbo_context::enumerate_levels(bool pool)
{
    if (pool && wm > 8) throw HipError{FCBO_ERR_INVALID_ARGUMENT};  // the pool keeps intents of <= 8 words
    LevelCursor s;
    pool_active = pool;
    pool_result = false;
    try {
        start_root(s);
        run_levels(s, ~0ull);
    } catch (...) {
        pool_active = false;
        throw;
    }
    pool_active = false;
    K = s.lo;
    if (pool) {
        try {
            run_pool(s.lo, s.obj_hi);
        } catch (...) {
            // a failed pool run keeps none of its memory (its commit grew the
            // level scratch to the pool's slots)
            release_pool();
            free_level_scratch();
            throw;
        }
    }
    have_result = have_levels = true;
    have_perm = false;
}

// The task pool: every concept of the store [0, K0) with at most kPoolTaskMax objects is
// a task whose subtree k_pool enumerates; the pool's concepts then join the
// store after it (lists from obj0 on), and the counts are taken over the whole
// store.
void fcbo_context::run_pool(uint64_t K0, uint64_t obj0)
{
    const uint64_t mc = min_cap();
    pool_fn fn = pick_pool_fn(wm);
    ensure(dmem, desc, cap_desc, K0, 0, stream, mc);
    ensure(dmem, pool_ctr, cap_pctr, POOL_CTR_N, 0, stream, 1);
    ensure(dmem, task_ctr, cap_tctr, (uint64_t)kPoolStripes * kCntPad, 0, stream, 1);
    // the task list: the store's concepts with at most kPoolTaskMax objects
    ensure(dmem, nchild, cap_nch, K0, 0, stream, mc);
    ensure(dmem, cbase, cap_cb, K0 + 1, 0, stream, mc);
    clear_words(pool_ctr, POOL_CTR_N);
    {
        const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(65535, div_up(K0, kBlock)));
        hipLaunchKernelGGL(k_pool_task_flags, dim3(g), dim3(kBlock), 0, stream, (const uint64_t *)loff, K0,
                           kPoolTaskMax, nchild, desc);
        CK_LAUNCH();
        scan(nchild, nullptr, nullptr, K0, K0, cbase, nullptr, pool_ctr + POOL_NTASKS, nullptr);
        CK(hipMemcpyAsync(h_counters, pool_ctr, POOL_CTR_N * sizeof(uint64_t), hipMemcpyDeviceToHost, stream));
        CK(hipStreamSynchronize(stream));
    }
    const uint64_t n_tasks = h_counters[POOL_NTASKS];
    ensure(dmem, ptasks, cap_ptasks, std::max<uint64_t>(1, n_tasks), 0, stream, mc);
    {
        const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(65535, div_up(K0, kBlock)));
        hipLaunchKernelGGL(k_pool_task_list, dim3(g), dim3(kBlock), 0, stream, (const uint32_t *)nchild,
                           (const uint64_t *)cbase, K0, ptasks);
        CK_LAUNCH();
    }
    // Slots the device can hold beside what it holds now (the slots being
    // replaced included), leaving room for the commit, which adds about as
    // many bytes per concept to the store again.
    const uint64_t slot_bytes = 8 * (uint64_t)wm + sizeof(PoolRec);
    const uint64_t commit_bytes = 8 * (uint64_t)wm + 4 + 8 + 4 + 9 + 2 * (uint64_t)kPoolTaskMax;
    auto affordable = [&]() -> uint64_t {
        size_t free_b = 0, total_b = 0;
        CK(hipMemGetInfo(&free_b, &total_b));
        const double room = (double)(free_b + cap_pint * 8 + cap_prec * sizeof(PoolRec)) * 0.85;
        return (uint64_t)(room / (double)(slot_bytes + commit_bytes));
    };
    uint64_t cap = pool_cap;
    if (!cap) cap = tiny ? (uint64_t)kWave : std::min(std::max<uint64_t>(start_size(1u << 22, slot_bytes), 8 * K0),
                                                       std::max<uint64_t>(kWave, affordable()));
    uint64_t slots = 0;
    for (int attempt = 0;; ++attempt) {
        if (attempt > 48) throw HipError{FCBO_ERR_DEVICE};
        ensure(dmem, p_int, cap_pint, cap * wm, 0, stream, mc);
        ensure(dmem, p_rec, cap_prec, cap, 0, stream, mc);
        clear_words(pool_ctr, POOL_CTR_N);
        clear_words(task_ctr, (uint64_t)kPoolStripes * kCntPad);
        PoolArgs PA;
        PA.rows = rows;
        PA.intents = intents;
        PA.cursor = cursor;
        PA.loff = loff;
        PA.objs = objs;
        PA.K = K0;
        PA.tasks = ptasks;
        PA.n_tasks = n_tasks;
        PA.task_ctr = task_ctr;
        PA.m = (int)m;
        PA.wm = wm;
        PA.tail_m = tail_m;
        PA.ctr = pool_ctr;
        PA.cap = cap;
        PA.p_int = p_int;
        PA.p_rec = p_rec;
        PA.desc = desc;
        hipEvent_t b = prof_begin();
        if (n_tasks) fn(this, PA);
        prof_end(FCBO_K_TEST_LOCAL, b);
        CK(hipMemcpyAsync(h_counters, pool_ctr, POOL_CTR_N * sizeof(uint64_t), hipMemcpyDeviceToHost, stream));
        CK(hipStreamSynchronize(stream));
        if (h_counters[POOL_ERROR]) throw HipError{FCBO_ERR_DEVICE};
        if (!h_counters[POOL_OVERFLOW]) {
            slots = h_counters[POOL_SLOTS];
            break;
        }
        // The slots ran out: everything again, with room for the slots used so
        // far scaled by the share of the tasks claimed (the tasks go largest
        // first, so this overestimates), and at least half as many again.
        const uint64_t reserved = h_counters[POOL_SLOTS];
        std::vector<uint64_t> claims((size_t)kPoolStripes * kCntPad);
        CK(hipMemcpyAsync(claims.data(), task_ctr, claims.size() * sizeof(uint64_t), hipMemcpyDeviceToHost, stream));
        CK(hipStreamSynchronize(stream));
        uint64_t started = 0;
        for (int st = 0; st < kPoolStripes; ++st) {
            const uint64_t in_stripe = n_tasks > (uint64_t)st ? div_up(n_tasks - st, kPoolStripes) : 0;
            started += std::min(claims[(size_t)st * kCntPad], in_stripe);
        }
        const double share = std::max(1e-3, (double)started / (double)std::max<uint64_t>(1, n_tasks));
        const uint64_t guess = (uint64_t)((double)reserved / share * 1.1) + kWave;
        const uint64_t want = std::min(std::max(cap + cap / 2, guess), affordable());
        if (want <= cap) throw HipError{FCBO_ERR_OUT_OF_MEMORY};
        cap = want;
    }
    pool_cap = cap;
    // dense store indices and list offsets of the used slots, per chunk of 64
    const uint64_t n_chunks = slots / kWave;  // reservations are whole chunks
    ensure(dmem, nchild, cap_nch, std::max<uint64_t>(1, n_chunks), 0, stream, mc);
    ensure(dmem, nobj, cap_nob, std::max<uint64_t>(1, n_chunks), 0, stream, mc);
    ensure(dmem, cbase, cap_cb, n_chunks + 1, 0, stream, mc);
    ensure(dmem, obase, cap_ob, n_chunks + 1, 0, stream, mc);
    hipEvent_t b = prof_begin();
    {
        const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(65535, div_up(n_chunks, kWavesPerBlock)));
        hipLaunchKernelGGL(k_pool_chunk_counts, dim3(g), dim3(kBlock), 0, stream, (const PoolRec *)p_rec, n_chunks,
                           nchild, nobj);
        CK_LAUNCH();
    }
    scan(nchild, nobj, nullptr, n_chunks, n_chunks, cbase, obase, pool_ctr + POOL_TOT_N, pool_ctr + POOL_TOT_OBJ);
    prof_end(FCBO_K_SCAN, b);
    CK(hipMemcpyAsync(h_counters, pool_ctr, POOL_CTR_N * sizeof(uint64_t), hipMemcpyDeviceToHost, stream));
    CK(hipStreamSynchronize(stream));
    const uint64_t np = h_counters[POOL_TOT_N], nob = h_counters[POOL_TOT_OBJ];
    const uint64_t kt = K0 + np;
    if (kt >= (1ull << 32)) throw HipError{FCBO_ERR_LIMIT};
    ensure(dmem, intents, cap_int, kt * wm, K0 * wm, stream, mc);
    ensure(dmem, cursor, cap_cur, kt, K0, stream, mc);
    ensure(dmem, loff, cap_loff, kt + 1, K0 + 1, stream, mc);
    ensure(dmem, objs, cap_o, obj0 + nob + kObjSlack, obj0, stream, mc);
    ensure(dmem, fchild, cap_fch, kt + 1, K0 + 1, stream, mc);
    ensure(dmem, t_owner, cap_towner, std::max<uint64_t>(1, np), 0, stream, mc);
    ensure(dmem, t_off, cap_toff, std::max<uint64_t>(1, np), 0, stream, mc);
    ensure(dmem, t_depth, cap_tdepth, std::max<uint64_t>(1, np), 0, stream, mc);
    b = prof_begin();
    {
        PoolCommitArgs C;
        C.rec = p_rec;
        C.p_int = p_int;
        C.dense = cbase;
        C.ooff = obase;
        C.n_chunks = n_chunks;
        C.K0 = K0;
        C.obj0 = obj0;
        C.n_pool = np;
        C.n_obj = nob;
        C.wm = wm;
        C.intents = intents;
        C.cursor = cursor;
        C.loff = loff;
        C.objs = objs;
        C.t_owner = t_owner;
        C.t_off = t_off;
        C.t_depth = t_depth;
        const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(65535, div_up(n_chunks, kWavesPerBlock)));
        hipLaunchKernelGGL(k_pool_commit, dim3(g), dim3(kBlock), 0, stream, C);
        CK_LAUNCH();
        // the pool's concepts have no children in the store (empty ranges)
        if (np) {
            const unsigned gf = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(65535, div_up(np, kBlock)));
            hipLaunchKernelGGL(k_fill_u32, dim3(gf), dim3(kBlock), 0, stream, fchild + K0 + 1, np, (uint32_t)K0);
            CK_LAUNCH();
        }
    }
    prof_end(FCBO_K_WRITE_LOCAL, b);
    K_sync = K0;
    n_pool = np;
    K = kt;
    // counts over the whole store; the level loop's levels stay for the order pass
    lev_sync = lev;
    const int nlev = (int)lev_sync.size();
    const int nbins = (int)m + 2;
    ensure(dmem, d_levlo, cap_levlo, (uint64_t)nlev + 1, 0, stream, 1);
    ensure(dmem, pstat, cap_pstat, 2 * (uint64_t)nbins + POOLSTAT_N, 0, stream, 1);
    std::vector<uint64_t> h_lo(lev_sync.lo, lev_sync.lo + nlev + 1);
    CK(hipMemcpyAsync(d_levlo, h_lo.data(), (nlev + 1) * sizeof(uint64_t), hipMemcpyHostToDevice, stream));
    clear_words(pstat, 2 * (uint64_t)nbins + POOLSTAT_N);
    {
        PoolStatsArgs S;
        S.intents = intents;
        S.cursor = cursor;
        S.loff = loff;
        S.K = kt;
        S.K0 = K0;
        S.m = (int)m;
        S.wm = wm;
        S.nlev = nlev;
        S.nbins = nbins;
        S.mid_max = kMidMax;
        S.tail_m = tail_m;
        S.lev_lo = d_levlo;
        S.t_owner = t_owner;
        S.t_depth = t_depth;
        S.out = pstat;
        const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(4096, div_up(kt, kBlock)));
        hipLaunchKernelGGL(k_pool_stats, dim3(g), dim3(kBlock), 2 * (size_t)nbins * sizeof(uint64_t), stream, S);
        CK_LAUNCH();
    }
    std::vector<uint64_t> h_stat(2 * (size_t)nbins + POOLSTAT_N);
    CK(hipMemcpyAsync(h_stat.data(), pstat, h_stat.size() * sizeof(uint64_t), hipMemcpyDeviceToHost, stream));
    CK(hipStreamSynchronize(stream));
    int last = 0;
    for (int l = 0; l < nbins; ++l)
        if (h_stat[l]) last = l;
    lev.clear();
    for (int l = 0; l <= last; ++l) lev.push(h_stat[l], h_stat[nbins + l]);
    const uint64_t *sums = h_stat.data() + 2 * nbins;
    tot.tests = sums[POOLSTAT_TESTS];
    tot.pairs = sums[POOLSTAT_PAIRS];
    tot.sum_c = sums[POOLSTAT_SUMC];
    tot.local_parents = sums[POOLSTAT_LOCAL];
    tot.local_objs = sums[POOLSTAT_LOCAL_OBJS];
    tot.med_parents = sums[POOLSTAT_MID];
    tot.med_objs = sums[POOLSTAT_MID_OBJS];
    pool_result = true;
}

// Add the kernel times recorded since the last harvest to st (after the
// stream has finished) and recycle their events.
void fcbo_context::harvest_marks(fcbo_stats &st)
{
    float ms = 0;
    for (auto &mk : marks) {
        CK(hipEventElapsedTime(&ms, mk.second.first, mk.second.second));
        st.kernel_ms[mk.first] += ms;
        st.kernel_launches[mk.first] += 1;
    }
    marks.clear();
    ev_used = 0;
}

// Wait for everything issued on the context's streams (after a failed batch,
// whose work may still be running).
void fcbo_context::drain()
{
    for (int i = 0; i < kSide; ++i)
        if (aux[i]) CK(hipStreamSynchronize(aux[i]));
    CK(hipStreamSynchronize(stream));
}

// Keep the store's concepts [first, first + count) (siblings, ascending
// attribute, lists at store objects [obj_lo, obj_hi)) aside as the seeds of
// later batches; their concepts sit on the given level of the CbO tree.
void fcbo_context::capture_seeds(uint64_t first, uint64_t count, uint64_t obj_lo, uint64_t obj_hi, uint64_t level)
{
    const uint64_t mc = min_cap();
    seeds.emplace_back();
    SeedSet &S = seeds.back();
    S.count = S.hi = S.B = S.B_cap = count;
    S.level = level;
    S.obj_base = obj_lo;
    ensure(dmem, S.ints, S.cap_int, count * wm, 0, stream, mc);
    ensure(dmem, S.cur, S.cap_cur, count, 0, stream, mc);
    ensure(dmem, S.loff, S.cap_loff, count + 1, 0, stream, mc);
    ensure(dmem, S.objs, S.cap_obj, std::max<uint64_t>(1, obj_hi - obj_lo), 0, stream, mc);
    CK(hipMemcpyAsync(S.ints, intents + first * wm, count * wm * 8, hipMemcpyDeviceToDevice, stream));
    CK(hipMemcpyAsync(S.cur, cursor + first, count * 4, hipMemcpyDeviceToDevice, stream));
    CK(hipMemcpyAsync(S.loff, loff + first, (count + 1) * 8, hipMemcpyDeviceToDevice, stream));
    if (obj_hi > obj_lo)
        CK(hipMemcpyAsync(S.objs, objs + obj_lo, (obj_hi - obj_lo) * 4, hipMemcpyDeviceToDevice, stream));
    S.h_loff.resize(count + 1);
    std::vector<int32_t> h_cur(count);
    CK(hipMemcpyAsync(S.h_loff.data(), S.loff, (count + 1) * 8, hipMemcpyDeviceToHost, stream));
    CK(hipMemcpyAsync(h_cur.data(), S.cur, count * 4, hipMemcpyDeviceToHost, stream));
    CK(hipStreamSynchronize(stream));
    // a parent's children are stored by ascending attribute and listed in the
    // output by descending attribute: batches are taken from the end
    for (uint64_t i = 1; i < count; ++i)
        if (h_cur[i] <= h_cur[i - 1]) throw HipError{FCBO_ERR_DEVICE};
    if (S.h_loff[0] != obj_lo || S.h_loff[count] != obj_hi) throw HipError{FCBO_ERR_DEVICE};
    // A seed's weight, the size of the context its subtree is searched in
    // (its objects times the attributes above its cursor), stands in for the
    // subtree's size when batches are sized.
    S.wsum.assign(count + 1, 0.0);
    for (uint64_t i = 0; i < count; ++i) {
        const double objs_i = (double)std::max<uint64_t>(1, S.h_loff[i + 1] - S.h_loff[i]);
        S.wsum[i + 1] = S.wsum[i] + objs_i * (double)(m - h_cur[i]);
    }
}

void fcbo_context::release_seeds()
{
    for (SeedSet &S : seeds) S.free_all(dmem);
    seeds.clear();
}

// Seeds [a, a + B) of S become level 1 of the store under a stand-in root at
// index 0 (its first-child link stays 1; the level loop rewrites the rest).
LevelCursor fcbo_context::load_seeds(const SeedSet &S, uint64_t a, uint64_t B, bool announce_classes)
{
    const uint64_t mc = min_cap();
    const uint64_t o0 = S.h_loff[a], o1 = S.h_loff[a + B];
    ensure(dmem, intents, cap_int, (1 + B) * wm, wm, stream, mc);
    ensure(dmem, cursor, cap_cur, 1 + B, 1, stream, mc);
    ensure(dmem, loff, cap_loff, 2 + B, 1, stream, mc);
    ensure(dmem, objs, cap_o, (uint64_t)n + (o1 - o0) + kObjSlack, (uint64_t)n, stream, mc);
    ensure(dmem, fchild, cap_fch, 2 + B, 1, stream, mc);
    CK(hipMemcpyAsync(intents + wm, S.ints + a * wm, B * wm * 8, hipMemcpyDeviceToDevice, stream));
    CK(hipMemcpyAsync(cursor + 1, S.cur + a, B * 4, hipMemcpyDeviceToDevice, stream));
    const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(1024, div_up(B + 1, kBlock)));
    hipLaunchKernelGGL(k_shift_offsets, dim3(g), dim3(kBlock), 0, stream, (const uint64_t *)S.loff + a, B + 1, o0,
                       (uint64_t)n, loff + 1);
    CK_LAUNCH();
    if (o1 > o0)
        CK(hipMemcpyAsync(objs + n, S.objs + (o0 - S.obj_base), (o1 - o0) * 4, hipMemcpyDeviceToDevice, stream));
    LevelCursor bs;
    bs.lo = 1;
    bs.P = B;
    bs.obj_hi = (uint64_t)n + (o1 - o0);
    // the seeds' classes, so the level loop launches the kernels they need
    // (without them it finds the classes on the level and runs it again)
    const uint64_t mid_max = wm <= 8 ? (uint64_t)kMidMax : (uint64_t)kSmallMax;
    for (uint64_t i = a; i < a + B && announce_classes; ++i) {
        const uint64_t sz = S.h_loff[i + 1] - S.h_loff[i];
        bs.next_huge += sz > mid_max;
        bs.next_mid += sz > (uint64_t)kSmallMax && sz <= mid_max;
    }
    lev.truncate(1);
    ctr = 0;
    clear_words(counters, 2 * CNT_N);
    return bs;
}

void fcbo_context::enumerate_bounded(uint64_t *intents_buf, uint64_t *extents_buf, uint64_t piece_rows,
                                     fcbo_sink_fn sink, void *user, uint32_t flags, fcbo_stats &st)
{
    const bool one_per_batch = (flags & FCBO_ONE_SUBTREE_PER_BATCH) != 0;
    const bool split_root_children = (flags & FCBO_SPLIT_ROOT_CHILDREN) != 0;
    const auto t_start = std::chrono::steady_clock::now();
    const uint64_t mc = min_cap();
    const bool out = intents_buf || extents_buf;
    release_seeds();
    dmem.peak = dmem.held;
    marks.clear();
    ev_used = 0;
    float ms = 0;
    double loop_ms = 0, order_ms = 0, out_ms = 0;
    uint64_t pos = 0;  // output positions handed out so far
    // store positions [p0, p1) of the current order to the sink, piece by piece
    auto emit = [&](uint64_t p0, uint64_t p1) {
        if (!out) {
            pos += p1 - p0;
            return;
        }
        hipEvent_t w0 = ev_get(), w1 = ev_get();
        for (uint64_t p = p0; p < p1;) {
            const uint64_t cnt = std::min(piece_rows, p1 - p);
            CK(hipEventRecord(w0, stream));
            write_output(intents_buf, extents_buf, p, cnt);
            CK(hipEventRecord(w1, stream));
            CK(hipStreamSynchronize(stream));
            CK(hipEventElapsedTime(&ms, w0, w1));
            out_ms += ms;
            if (sink && sink(user, pos, cnt, intents_buf, extents_buf)) throw HipError{FCBO_ERR_STOPPED};
            pos += cnt;
            p += cnt;
        }
    };
    // the one concept at store index idx, without an order pass
    auto emit_concept = [&](uint32_t idx) {
        if (out) {
            ensure(dmem, perm, cap_perm, 1, 0, stream, mc);
            hipLaunchKernelGGL(k_set_u32, dim3(1), dim3(1), 0, stream, perm, idx);
            CK_LAUNCH();
            have_perm = false;
        }
        emit(0, 1);
    };
    // per-level counts of the whole tree: level l >= 1 of a batch is level
    // base + l - 1 of the tree
    std::vector<uint64_t> lev_c, lev_t;
    auto add_levels = [&](uint64_t base) {
        for (size_t l = 1; l < lev.size(); ++l) {
            const size_t at = base + l - 1;
            if (at >= lev_c.size()) {
                lev_c.resize(at + 1, 0);
                lev_t.resize(at + 1, 0);
            }
            lev_c[at] += lev.concepts[l];
            lev_t[at] += lev.tests[l];
        }
    };

    // the root, its row, and its children as the first seed set
    LevelCursor s;
    {
        hipEvent_t e0 = ev_get(), e1 = ev_get();
        CK(hipEventRecord(e0, stream));
        start_root(s);
        run_levels(s, 1);
        CK(hipEventRecord(e1, stream));
        CK(hipStreamSynchronize(stream));
        CK(hipEventElapsedTime(&ms, e0, e1));
        loop_ms += ms;
        lev_c.assign(1, 1);
        lev_t.assign(1, lev.tests[0]);
        emit_concept(0);
        harvest_marks(st);
    }
    uint64_t total = 1, batches = 0, retries = 0, splits = 0;
    // Batch sizing, once a batch has failed: concepts per unit of seed weight,
    // measured on the last batch that fitted, predicts a batch's concepts, and
    // a batch aims at 70% of the smallest store size at which one failed.
    double k_per_w = 0;
    uint64_t k_fail = ~0ull;
    auto predict = [&](SeedSet &S) {
        if (k_per_w <= 0 || k_fail == ~0ull || S.hi == 0) return;
        const double budget = 0.7 * (double)k_fail;
        uint64_t lo = 1, hi = std::min(S.hi, S.B_cap);
        while (lo < hi) {  // the largest batch within the budget
            const uint64_t mid = (lo + hi + 1) / 2;
            if ((S.wsum[S.hi] - S.wsum[S.hi - mid]) * k_per_w <= budget) lo = mid;
            else hi = mid - 1;
        }
        S.B = lo;
    };
    if (s.P) capture_seeds(1, s.P, (uint64_t)n, s.obj_hi, 1);
    while (!seeds.empty()) {
        const size_t si = seeds.size() - 1;
        if (seeds[si].hi == 0) {
            seeds[si].free_all(dmem);
            seeds.pop_back();
            continue;
        }
        const bool force_split = split_root_children && seeds[si].level == 1;
        const uint64_t B = std::min(one_per_batch || force_split ? 1 : seeds[si].B, seeds[si].hi);
        const uint64_t a = seeds[si].hi - B;
        const Totals saved = tot;
        hipEvent_t b0 = ev_get(), b1 = ev_get(), b2 = ev_get();
        bool fits = !force_split;
        if (fits) try {
            CK(hipEventRecord(b0, stream));
            LevelCursor bs = load_seeds(seeds[si], a, B, !one_per_batch);
            run_levels(bs, ~0ull);
            K = bs.lo;
            have_result = true;
            have_perm = false;
            CK(hipEventRecord(b1, stream));
            if (out) order_concepts();
            CK(hipEventRecord(b2, stream));
            CK(hipStreamSynchronize(stream));
        } catch (const HipError &e) {
            if (e.code != FCBO_ERR_OUT_OF_MEMORY && e.code != FCBO_ERR_LIMIT) throw;
            drain();
            harvest_marks(st);
            tot = saved;
            have_result = have_perm = false;
            ++retries;
            fits = false;
        }
        if (!fits) {
            k_fail = std::min(k_fail, store_rows_seen);
            if (B > 1) {
                seeds[si].B = seeds[si].B_cap = (B + 1) / 2;
                predict(seeds[si]);
                continue;
            }
            // A single seed whose subtree does not fit: its own row goes out and
            // its children become the next seed set (in the output a subtree is
            // its root, then its children's subtrees by descending attribute).
            // Should this one level not fit either, the call fails.
            hipEvent_t x0 = ev_get(), x1 = ev_get();
            CK(hipEventRecord(x0, stream));
            LevelCursor bs = load_seeds(seeds[si], a, 1);
            const uint64_t child_obj_lo = bs.obj_hi;
            run_levels(bs, 1);
            CK(hipEventRecord(x1, stream));
            CK(hipStreamSynchronize(stream));
            CK(hipEventElapsedTime(&ms, x0, x1));
            loop_ms += ms;
            add_levels(seeds[si].level);
            const uint64_t level = seeds[si].level;
            seeds[si].hi = a;
            ++splits;
            ++total;
            emit_concept(1);
            harvest_marks(st);
            if (bs.P) {
                capture_seeds(2, bs.P, child_obj_lo, bs.obj_hi, level + 1);
                predict(seeds.back());
            }
            continue;
        }
        CK(hipEventElapsedTime(&ms, b0, b1));
        loop_ms += ms;
        CK(hipEventElapsedTime(&ms, b1, b2));
        order_ms += ms;
        add_levels(seeds[si].level);
        emit(1, K);  // the stand-in root at position 0 is not part of the batch
        harvest_marks(st);
        total += K - 1;
        ++batches;
        seeds[si].hi = a;
        k_per_w = (double)(K - 1) / std::max(1e-9, seeds[si].wsum[a + B] - seeds[si].wsum[a]);
        predict(seeds[si]);
    }
    // the level log of the whole enumeration; the store holds only the last batch
    lev.clear();
    for (size_t l = 0; l < lev_c.size(); ++l) lev.push(lev_c[l], lev_t[l]);
    have_result = have_perm = have_cover_counts = false;
    have_levels = true;
    K = 0;
    fill_counts(st, total);
    st.closure_kernel_ms = loop_ms;
    st.sort_ms = order_ms;
    st.output_ms = out_ms;
    st.output_bytes = out ? total * 8 * ((intents_buf ? (uint64_t)wm : 0) + (extents_buf ? (uint64_t)wn : 0)) : 0;
    st.batches = batches;
    st.batch_retries = retries;
    st.batch_splits = splits;
    st.peak_device_bytes = dmem.peak;
    st.enumerate_ms =
        std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t_start).count();
}

void fcbo_context::order_concepts()
{
    if (K >= (1ull << 32)) throw HipError{FCBO_ERR_LIMIT};
    const uint64_t mc = min_cap();
    ensure(dmem, rank, cap_rank, K, 0, stream, mc);
    ensure(dmem, perm, cap_perm, K, 0, stream, mc);
    // with the task pool the levels are the level loop's; the pool's concepts
    // are placed after them from their tasks' positions
    const LevelLog &L = pool_result ? lev_sync : lev;
    const uint32_t *dsc = pool_result ? desc : nullptr;
    const size_t nlev = L.size();
    const uint64_t *lev_concepts = L.concepts, *lev_lo = L.lo;
    auto grid = [](uint64_t n) { return (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(65535, div_up(n, kBlock))); };
    auto wgrid = [](uint64_t n) {
        return (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(65535, div_up(n, kWavesPerBlock)));
    };
    // levels whose concepts average many children take a wavefront per concept
    auto wide_level = [&](size_t l) { return l + 1 < nlev && lev_concepts[l + 1] >= kOrderWaveFanout * lev_concepts[l]; };
    hipEvent_t b = prof_begin();
    order_launches = 0;
    for (size_t l = nlev; l-- > 0;) {  // sizes, deepest level first
        if (wide_level(l))
            hipLaunchKernelGGL(k_subtree_size_wave, dim3(wgrid(lev_concepts[l])), dim3(kBlock), 0, stream,
                               (const uint32_t *)fchild, lev_lo[l], lev_concepts[l], rank, dsc);
        else
            hipLaunchKernelGGL(k_subtree_size, dim3(grid(lev_concepts[l])), dim3(kBlock), 0, stream,
                               (const uint32_t *)fchild, lev_lo[l], lev_concepts[l], rank, dsc);
        CK_LAUNCH();
        ++order_launches;
    }
    for (size_t l = 0; l + 1 < nlev; ++l) {  // positions, root level first
        if (wide_level(l))
            hipLaunchKernelGGL(k_child_position_wave, dim3(wgrid(lev_concepts[l])), dim3(kBlock), 0, stream,
                               (const uint32_t *)fchild, lev_lo[l], lev_concepts[l], rank);
        else
            hipLaunchKernelGGL(k_child_position, dim3(grid(lev_concepts[l])), dim3(kBlock), 0, stream,
                               (const uint32_t *)fchild, lev_lo[l], lev_concepts[l], rank);
        CK_LAUNCH();
        ++order_launches;
    }
    if (pool_result && n_pool) {
        hipLaunchKernelGGL(k_tail_position, dim3(grid(n_pool)), dim3(kBlock), 0, stream, (const uint32_t *)t_owner,
                           (const uint32_t *)t_off, n_pool, K_sync, rank);
        CK_LAUNCH();
        ++order_launches;
    }
    hipLaunchKernelGGL(k_invert, dim3(grid(K)), dim3(kBlock), 0, stream, (const uint32_t *)rank, K, perm);
    CK_LAUNCH();
    ++order_launches;
    prof_end(FCBO_K_ORDER, b);
    have_perm = true;
}

// Output rows [first, first + count): row r of the buffers gets the concept at
// output position first + r.  Either buffer may be null.
void fcbo_context::write_output(uint64_t *intents_out, uint64_t *extents_out, uint64_t first, uint64_t count)
{
    hipEvent_t b = prof_begin();
    const uint32_t *pm = perm + first;
    const uint64_t row_bytes = (uint64_t)wn * 8;
    if (extents_out && row_bytes > (uint64_t)kOutBlockBytes) {
        // rows wider than the LDS tile: one wavefront per row, tile by tile
        const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(8192, div_up(count, kWavesPerBlock)));
        hipLaunchKernelGGL(k_output, dim3(g), dim3(kBlock), 0, stream, (const uint64_t *)intents,
                           (const uint64_t *)loff, (const uint32_t *)objs, pm, count, wm, wn, intents_out,
                           extents_out);
        CK_LAUNCH();
        prof_end(FCBO_K_OUTPUT, b);
        return;
    }
    // the ordered intents, then (with an extent buffer) the extent row blocks
    if (intents_out) {
        hipLaunchKernelGGL(k_output_intents, dim3(kGridCap), dim3(kBlock), 0, stream, (const uint64_t *)intents, pm,
                           count, wm, intents_out);
        CK_LAUNCH();
    }
    if (extents_out) {
        // Rows per block: a multiple of L/gcd(wn, L), L the words of a cache
        // line, makes the block's region a whole number of lines; aim for
        // kOutTargetBytes of LDS per block.
        const int al = kOutLineWords / std::gcd(wn, kOutLineWords);
        const uint64_t al_bytes = (uint64_t)al * row_bytes;
        int R;
        if (al_bytes <= (uint64_t)kOutBlockBytes)
            R = al * (int)std::max<uint64_t>(1, (uint64_t)kOutTargetBytes / al_bytes);
        else
            R = (int)(kOutBlockBytes / row_bytes);
        R = std::min(R, kWave);
        const size_t lds = (size_t)R * wn * 8;
        int per_cu = 1;
        CK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_output_block, kOutThreads, lds));
        const uint64_t nblk = div_up(count, (uint64_t)R);
        const uint64_t slots = (uint64_t)n_cu * std::max(1, per_cu);
        const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(nblk, slots));
        hipLaunchKernelGGL(k_output_block, dim3(g), dim3(kOutThreads), lds, stream, (const uint64_t *)loff,
                           (const uint32_t *)objs, pm, count, wn, R, extents_out);
        CK_LAUNCH();
    }
    prof_end(FCBO_K_OUTPUT, b);
}

// Algorithmic bytes of the last enumeration (the formula in fcbo.h, with the
// row-local threshold of the class split: 4096 objects up to eight intent
// words, else 64).
uint64_t fcbo_context::model_bytes(uint64_t k) const
{
    if (!k) return 0;
    const uint64_t W_M = (uint64_t)wm, W_N = (uint64_t)wn;
    uint64_t b = k * (8 * W_M + 4 + 16);             // every concept read once as a parent
    b += (tot.local_objs + tot.med_objs) * (4 + 8 * W_M);   // row-local parents: list entries and rows
    b += tot.big_parents * 8 * W_N;                      // larger parents: extent bitmap
    b += tot.big_nzw * 8;                                // their tests: non-zero column words
    b += tot.big_cobjs * 8 * W_M;                        // their children: rows of C
    b += (k - 1) * (8 * W_M + 4 + 8) + 4 * tot.sum_c;    // children written
    b += (uint64_t)n * (8 * W_M + 4);                // the root
    return b;
}

// The counts of the last enumeration (K, tests, levels, classes, bytes).
void fcbo_context::fill_counts(fcbo_stats &st, uint64_t k) const
{
    st.n_concepts = k;
    st.model_bytes = model_bytes(k);
    st.closure_tests = tot.tests;
    st.item_pairs = tot.pairs;
    st.n_levels = lev.size();
    st.sum_child_objects = tot.sum_c;
    st.local_parents = tot.local_parents;
    st.local_parent_objects = tot.local_objs;
    st.medium_parents = tot.med_parents;
    st.medium_parent_objects = tot.med_objs;
    st.big_parents = tot.big_parents;
    st.big_tests = tot.big_tests;
    st.big_scanned_objects = tot.big_scan;
    st.big_nonzero_words = tot.big_nzw;
    st.big_child_objects = tot.big_cobjs;
    st.order_launches = order_launches;
    st.level_redos = tot.redos;
}

// The context on the device: rows copied and masked, columns transposed.
// Fixed contexts take these buffers from the static region too and keep the
// counters' host copy in the context itself.
void fcbo_context::setup(const uint64_t *rows_in, int64_t n_objects, int64_t n_attrs, int64_t row_stride_words,
                         bool rows_on_device)
{
    CK(hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, device));
    n = n_objects;
    m = n_attrs;
    wn = (int)((n_objects + 63) / 64);
    wm = (int)((n_attrs + 63) / 64);
    tail_m = (n_attrs & 63) ? ((1ull << (n_attrs & 63)) - 1ull) : ~0ull;
    tail_n = (n_objects & 63) ? ((1ull << (n_objects & 63)) - 1ull) : ~0ull;
    const uint64_t row_words = ((uint64_t)n_objects + 1) * wm;  // a zero row after the last
    const uint64_t col_words = (uint64_t)n_attrs * wn;
    if (fixed) {
        rows = (uint64_t *)dmem.get(row_words * sizeof(uint64_t));
        cols = (uint64_t *)dmem.get(col_words * sizeof(uint64_t));
        scan_part = (uint64_t *)dmem.get(2 * kScanBlocks * sizeof(uint64_t));
        counters = (uint64_t *)dmem.get(2 * CNT_N * sizeof(uint64_t));
        h_counters = h_counters_own;
    } else {
        CK_ALLOC(hipMalloc((void **)&rows, row_words * sizeof(uint64_t)));
        CK_ALLOC(hipMalloc((void **)&cols, col_words * sizeof(uint64_t)));
        CK_ALLOC(hipMalloc((void **)&scan_part, 2 * kScanBlocks * sizeof(uint64_t)));
        CK_ALLOC(hipMalloc((void **)&counters, 2 * CNT_N * sizeof(uint64_t)));
        CK_ALLOC(hipHostMalloc((void **)&h_counters, CNT_N * sizeof(uint64_t), hipHostMallocDefault));
    }
    clear_words(rows, row_words);
    const hipMemcpyKind kind = rows_on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;
    CK(hipMemcpy2DAsync(rows, (size_t)wm * sizeof(uint64_t), rows_in, (size_t)row_stride_words * sizeof(uint64_t),
                        (size_t)wm * sizeof(uint64_t), (size_t)n_objects, kind, stream));
    hipLaunchKernelGGL(k_mask_rows, dim3((unsigned)div_up((uint64_t)n_objects, kBlock)), dim3(kBlock), 0, stream, rows,
                       (int)n_objects, wm, tail_m);
    CK_LAUNCH();
    const uint64_t waves = (uint64_t)wn * wm;
    hipLaunchKernelGGL(k_transpose, dim3((unsigned)div_up(waves, kWavesPerBlock)), dim3(kBlock), 0, stream,
                       (const uint64_t *)rows, cols, (int)n_objects, (int)n_attrs, wn, wm);
    CK_LAUNCH();
    CK(hipStreamSynchronize(stream));
}

namespace {

typedef void (*cover_fn)(const CoverArgs &, int, hipStream_t, int);

template <int WMC>
void launch_cover(const CoverArgs &C, int pass, hipStream_t s, int n_cu)
{
    if (pass == 0) {
        const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(16384, div_up(C.K, kBlock)));
        hipLaunchKernelGGL(k_cover_table<WMC>, dim3(g), dim3(kBlock), 0, s, C);
        CK_LAUNCH();
        return;
    }
    if constexpr (WMC <= 8) {
        const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(16384, div_up(C.K, kWavesPerBlock)));
        hipLaunchKernelGGL(k_cover_local<WMC>, dim3(g), dim3(kBlock), 0, s, C, pass);
        CK_LAUNCH();
    }
    // as many workgroups as fit the compute units (the big concepts are few
    // and their passes wait on memory)
    const size_t lds = cover_big_lds<WMC>(C.m);
    int per_cu = 1;
    CK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_cover_big<WMC>, kCoverThreads, lds));
    hipLaunchKernelGGL(k_cover_big<WMC>, dim3((unsigned)(std::max(1, per_cu) * n_cu)), dim3(kCoverThreads), lds, s, C,
                       pass);
    CK_LAUNCH();
}

cover_fn pick_cover_fn(int wm)
{
    switch (wm) {
    case 1: return launch_cover<1>;
    case 2: return launch_cover<2>;
    case 3: return launch_cover<3>;
    case 4: return launch_cover<4>;
    case 5: return launch_cover<5>;
    case 6: return launch_cover<6>;
    case 7: return launch_cover<7>;
    case 8: return launch_cover<8>;
    default:
        if (wm <= 16) return launch_cover<16>;
        if (wm <= 32) return launch_cover<32>;
        return launch_cover<64>;
    }
}

}  // namespace

// Lower covers of every concept (see k_cover_local): the large concepts listed,
// a counting pass, the scan, and (when the caller's buffer holds all E edges)
// the table of concepts by intent and the writing pass.  Returns E.
uint64_t fcbo_context::cover_edges(uint64_t *offsets_out, uint32_t *targets_out, uint64_t capacity)
{
    if (!have_perm) order_concepts();
    CK(hipStreamSynchronize(stream));
    free_level_scratch();  // the cover buffers of 10^9 concepts need that room
    const uint64_t mc = min_cap();
    CoverArgs C;
    memset(&C, 0, sizeof(C));
    C.rows = rows; C.intents = intents; C.cursor = cursor; C.fchild = fchild; C.rank = rank;
    C.loff = loff; C.objs = objs; C.perm = perm;
    C.K = K; C.m = (int)m; C.wm = wm; C.tail_m = tail_m;
    C.small_max = wm <= 8 ? kSmallMax : -1;
    const cover_fn fn = pick_cover_fn(wm);
    uint64_t slots = 1024;
    while (slots < 2 * K) slots *= 2;
    auto build_table = [&]() {
        ensure(dmem, ctable, cap_ctable, slots, 0, stream, mc);
        const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(16384, div_up(slots, kBlock)));
        hipLaunchKernelGGL(k_fill_u64, dim3(g), dim3(kBlock), 0, stream, (uint64_t *)ctable, slots / 2, ~0ull);
        CK_LAUNCH();
        C.table = ctable;
        C.table_mask = slots - 1;
        fn(C, 0, stream, n_cu);
        cover_table_ok = true;
    };
    if (!have_cover_counts) {
        cover_table_ok = cover_kept = false;
        ensure(dmem, ccount, cap_ccount, K, 0, stream, mc);
        ensure(dmem, coff, cap_coff, K + 1, 0, stream, mc);
        ensure(dmem, cbig, cap_cbig, K, 0, stream, mc);
        ensure(dmem, cctr, cap_cctr, 4, 0, stream, 4);
        clear_words(cctr, 4);
    }
    C.big = cbig; C.ctr = cctr; C.count = ccount; C.offsets = coff; C.targets = targets_out;
    if (cover_table_ok) {
        C.table = ctable;
        C.table_mask = slots - 1;
    }
    if (!have_cover_counts) {
        // Counts kept until the next enumeration: a count call and the call
        // that writes take one counting pass together.  When the room is
        // there (and the result is large), that pass also keeps every cover's
        // position (one run per concept), so the writing call only moves the
        // runs; the room is
        // guessed (8 covers a concept on average, plus the wavefronts' part-used
        // chunks) and the writing call falls back to a second pass over the
        // concepts if it ran out.
        const unsigned gl = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(4096, div_up(K, kBlock)));
        hipLaunchKernelGGL(k_cover_list_big, dim3(gl), dim3(kBlock), 0, stream, C);
        CK_LAUNCH();
        const uint64_t local_waves = std::min<uint64_t>(16384, div_up(K, kWavesPerBlock)) * kWavesPerBlock;
        // (FCBO_TINY_BUFFERS: two chunks, so the fallback runs on any input)
        const uint64_t entries = tiny ? 2 * kCoverChunk : 8 * K + kCoverChunk * local_waves + 4096;
        const uint64_t need = entries * 4 + K * 8 + (cap_ctable >= slots ? 0 : slots * 4);
        size_t free_b = 0, total_b = 0;
        CK(hipMemGetInfo(&free_b, &total_b));
        // (below 2^20 concepts the second pass costs less than the scratch and
        // the copy: 1.0 against 1.5 ms at 1.7 * 10^5 concepts)
        bool keep = !fixed && (tiny || K >= (1ull << 20)) && need + need / 4 < (uint64_t)free_b &&
                    (!dmem.limit || dmem.held + need <= dmem.limit);
        if (keep) {
            try {
                ensure(dmem, cscratch, cap_cscratch, entries, 0, stream, mc);
                ensure(dmem, csstart, cap_csstart, K, 0, stream, mc);
                build_table();
            } catch (const HipError &e) {
                if (e.code != FCBO_ERR_OUT_OF_MEMORY) throw;
                dfree(dmem, cscratch, cap_cscratch);
                dfree(dmem, csstart, cap_csstart);
                keep = false;
            }
        }
        if (keep) {
            C.scratch = cscratch;
            C.scratch_cap = cap_cscratch;
            C.sstart = csstart;
        }
        fn(C, keep ? kCoverKeep : kCoverCount, stream, n_cu);
        scan(ccount, nullptr, nullptr, K, K, coff, nullptr, nullptr, nullptr);
        uint64_t h[3] = {0, 0, 0};  // covers not found, scratch entries used, scratch short
        CK(hipMemcpyAsync(&cover_total, coff + K, sizeof(uint64_t), hipMemcpyDeviceToHost, stream));
        CK(hipMemcpyAsync(h, cctr + 1, sizeof(h), hipMemcpyDeviceToHost, stream));
        CK(hipStreamSynchronize(stream));
        if (h[0]) throw HipError{FCBO_ERR_DEVICE};  // a cover that is not a concept: cannot happen
        cover_kept = keep && !h[2];
        if (keep && !cover_kept) {  // the runs are of no use
            dfree(dmem, cscratch, cap_cscratch);
            dfree(dmem, csstart, cap_csstart);
        }
        have_cover_counts = true;
    }
    const uint64_t e = cover_total;
    if (!offsets_out || !targets_out || capacity < e) return e;
    if (cover_kept) {
        C.scratch = cscratch;
        C.scratch_cap = cap_cscratch;
        C.sstart = csstart;
        const unsigned g = (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(16384, div_up(K, kBlock)));
        hipLaunchKernelGGL(k_cover_copy_runs, dim3(g), dim3(kBlock), 0, stream, C);
        CK_LAUNCH();
        CK(hipMemcpyAsync(offsets_out, coff, (K + 1) * sizeof(uint64_t), hipMemcpyDeviceToDevice, stream));
        CK(hipStreamSynchronize(stream));
        return e;
    }
    clear_words(cctr + 1, 1);
    if (!cover_table_ok) build_table();
    fn(C, kCoverWrite, stream, n_cu);
    CK(hipMemcpyAsync(offsets_out, coff, (K + 1) * sizeof(uint64_t), hipMemcpyDeviceToDevice, stream));
    uint64_t missing = 0;
    CK(hipMemcpyAsync(&missing, cctr + 1, sizeof(uint64_t), hipMemcpyDeviceToHost, stream));
    CK(hipStreamSynchronize(stream));
    if (missing) throw HipError{FCBO_ERR_DEVICE};  // a cover that is not a concept: cannot happen
    return e;
}

// Output rows [first, first + count) into host memory, staging_rows at a time
// through two device buffers: the output kernels fill one buffer on the
// context's stream while the other is copied to the host on the side stream
// (events order a buffer's reuse after its copy).
void fcbo_context::copy_to_host(uint64_t first, uint64_t count, uint64_t *host_intents, uint64_t *host_extents,
                                uint64_t staging_rows)
{
    if (!have_perm) order_concepts();
    const uint64_t rows_per = std::min(staging_rows, count);
    for (int b = 0; b < 2; ++b) {
        if (host_intents) ensure(dmem, hs_int[b], cap_hs_int[b], rows_per * (uint64_t)wm, 0, stream, 1);
        if (host_extents) ensure(dmem, hs_ext[b], cap_hs_ext[b], rows_per * (uint64_t)wn, 0, stream, 1);
        if (!hs_written[b]) CK(hipEventCreateWithFlags(&hs_written[b], hipEventDisableTiming));
        if (!hs_copied[b]) CK(hipEventCreateWithFlags(&hs_copied[b], hipEventDisableTiming));
    }
    if (!aux[0]) CK(hipStreamCreateWithFlags(&aux[0], hipStreamNonBlocking));
    hipStream_t cs = aux[0];
    // the copy stream starts after what the caller's stream holds
    if (!ev_fork[0]) CK(hipEventCreateWithFlags(&ev_fork[0], hipEventDisableTiming));
    CK(hipEventRecord(ev_fork[0], stream));
    CK(hipStreamWaitEvent(cs, ev_fork[0], 0));
    bool used[2] = {false, false};
    uint64_t i = 0;
    for (uint64_t at = 0; at < count; at += rows_per, ++i) {
        const int b = (int)(i & 1);
        const uint64_t n = std::min(rows_per, count - at);
        if (used[b]) CK(hipStreamWaitEvent(stream, hs_copied[b], 0));  // its last copy is done
        write_output(host_intents ? hs_int[b] : nullptr, host_extents ? hs_ext[b] : nullptr, first + at, n);
        CK(hipEventRecord(hs_written[b], stream));
        CK(hipStreamWaitEvent(cs, hs_written[b], 0));
        if (host_intents)
            CK(hipMemcpyAsync(host_intents + at * (uint64_t)wm, hs_int[b], n * (uint64_t)wm * sizeof(uint64_t),
                              hipMemcpyDeviceToHost, cs));
        if (host_extents)
            CK(hipMemcpyAsync(host_extents + at * (uint64_t)wn, hs_ext[b], n * (uint64_t)wn * sizeof(uint64_t),
                              hipMemcpyDeviceToHost, cs));
        CK(hipEventRecord(hs_copied[b], cs));
        used[b] = true;
    }
    CK(hipStreamSynchronize(cs));
    CK(hipStreamSynchronize(stream));
}

// ---------------------------------------------------------------------------
// Static device scratch of fcbo_enumerate_static: one copy per GPU, held until
// the process ends.  Host code never takes its name as an address (that is a
// host-side stand-in): the device address comes from hipGetSymbolAddress, once
// per device with that device current, and is kept per device.

namespace {

static __device__ __align__(256) unsigned char scratch[FCBO_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
char *g_scratch_ptr[kMaxDevices] = {};

char *scratch_on_device(int device)
{
    if (device < 0 || device >= kMaxDevices) throw HipError{FCBO_ERR_DEVICE};
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[device]) {
        void *p = nullptr;
        CK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) throw HipError{FCBO_ERR_DEVICE};
        g_scratch_ptr[device] = (char *)p;
    }
    return g_scratch_ptr[device];
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI

extern "C" {

const char *fcbo_error_string(int code)
{
    switch (code) {
    case FCBO_OK: return "ok";
    case FCBO_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FCBO_ERR_OUT_OF_MEMORY: return "device out of memory";
    case FCBO_ERR_DEVICE: return "HIP device error";
    case FCBO_ERR_CAPACITY: return "output capacity too small";
    case FCBO_ERR_LIMIT: return "2^32 concepts or more (beyond the 32-bit concept indices)";
    case FCBO_ERR_SCRATCH: return "the work does not fit the static scratch of fcbo_enumerate_static";
    case FCBO_ERR_STOPPED: return "the sink stopped the enumeration";
    default: return "unknown error";
    }
}

namespace {

bool valid_context_args(const uint64_t *rows, int64_t n_objects, int64_t n_attrs, int64_t row_stride_words)
{
    return rows && n_objects >= 1 && n_objects <= INT32_MAX && n_attrs >= 1 && n_attrs <= 4096 &&
           row_stride_words >= (n_attrs + 63) / 64;
}

}  // namespace

int fcbo_context_create(const uint64_t *rows, int64_t n_objects, int64_t n_attrs, int64_t row_stride_words,
                        uint32_t flags, void *hip_stream, fcbo_context **out)
{
    if (!out) return FCBO_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    if (!valid_context_args(rows, n_objects, n_attrs, row_stride_words) ||
        (flags & ~(FCBO_ROWS_ON_DEVICE | FCBO_TINY_BUFFERS)))
        return FCBO_ERR_INVALID_ARGUMENT;
    fcbo_context *c = new (std::nothrow) fcbo_context();
    if (!c) return FCBO_ERR_OUT_OF_MEMORY;
    try {
        CK(hipGetDevice(&c->device));
        (void)hipGetLastError();  // an error left by earlier, unrelated work is not this call's
        c->stream = (hipStream_t)hip_stream;
        c->tiny = (flags & FCBO_TINY_BUFFERS) != 0;
        c->setup(rows, n_objects, n_attrs, row_stride_words, (flags & FCBO_ROWS_ON_DEVICE) != 0);
    } catch (const HipError &e) {
        c->free_all();
        delete c;
        return e.code;
    } catch (const std::bad_alloc &) {
        c->free_all();
        delete c;
        return FCBO_ERR_OUT_OF_MEMORY;
    }
    *out = c;
    return FCBO_OK;
}

int fcbo_enumerate(fcbo_context *ctx, uint64_t *intents_out, uint64_t *extents_out, uint64_t capacity,
                   uint32_t flags, uint64_t *n_concepts_out, fcbo_stats *stats_out)
{
    if (!ctx || (flags & ~(FCBO_REUSE_RESULT | FCBO_PROFILE | FCBO_TASK_POOL))) return FCBO_ERR_INVALID_ARGUMENT;
    if ((flags & FCBO_TASK_POOL) && ctx->m > 512) return FCBO_ERR_INVALID_ARGUMENT;
    fcbo_stats st;
    memset(&st, 0, sizeof(st));
    hipEvent_t e0 = nullptr, e1 = nullptr, e2 = nullptr, e3 = nullptr;
    int rc = FCBO_OK;
    try {
        CK(hipSetDevice(ctx->device));
        (void)hipGetLastError();  // an error left by earlier, unrelated work is not this call's
        ctx->profile = (flags & FCBO_PROFILE) != 0;
        ctx->ev_used = 0;
        ctx->marks.clear();
        e0 = ctx->ev_get();
        e1 = ctx->ev_get();
        e2 = ctx->ev_get();
        e3 = ctx->ev_get();
        CK(hipEventRecord(e0, ctx->stream));
        const bool reuse = (flags & FCBO_REUSE_RESULT) && ctx->have_result;
        ctx->dmem.peak = ctx->dmem.held;
        if (!reuse) ctx->enumerate_levels((flags & FCBO_TASK_POOL) != 0);
        CK(hipEventRecord(e1, ctx->stream));
        if (n_concepts_out) *n_concepts_out = ctx->K;
        if (!intents_out || capacity < ctx->K) {
            rc = FCBO_ERR_CAPACITY;
            CK(hipStreamSynchronize(ctx->stream));
        } else {
            if (!(reuse && ctx->have_perm)) ctx->order_concepts();
            CK(hipEventRecord(e2, ctx->stream));
            ctx->write_output(intents_out, extents_out, 0, ctx->K);
            CK(hipEventRecord(e3, ctx->stream));
            CK(hipStreamSynchronize(ctx->stream));
            float ms = 0;
            CK(hipEventElapsedTime(&ms, e0, e3));
            st.enumerate_ms = ms;
            CK(hipEventElapsedTime(&ms, e1, e2));
            st.sort_ms = ms;
            CK(hipEventElapsedTime(&ms, e2, e3));
            st.output_ms = ms;
        }
        float ms = 0;
        CK(hipEventElapsedTime(&ms, e0, e1));
        st.closure_kernel_ms = ms;
        for (auto &mk : ctx->marks) {
            CK(hipEventElapsedTime(&ms, mk.second.first, mk.second.second));
            st.kernel_ms[mk.first] += ms;
            st.kernel_launches[mk.first] += 1;
        }
    } catch (const HipError &e) {
        ctx->have_result = ctx->have_perm = false;
        if (e.code == FCBO_ERR_OUT_OF_MEMORY) {
            // give back what the failed run grew beyond the store, so the
            // next call has the room
            ctx->release_pool();  // waits for the streams first
            ctx->free_level_scratch();
        }
        return e.code;
    } catch (const std::bad_alloc &) {
        ctx->have_result = ctx->have_perm = false;
        return FCBO_ERR_OUT_OF_MEMORY;
    }
    ctx->fill_counts(st, ctx->have_result ? ctx->K : 0);
    st.batches = 1;
    st.peak_device_bytes = ctx->dmem.peak;
    if (rc == FCBO_OK)
        st.output_bytes = ctx->K * (uint64_t)ctx->wm * 8 + (extents_out ? ctx->K * (uint64_t)ctx->wn * 8 : 0);
    if (stats_out) *stats_out = st;
    return rc;
}

int fcbo_enumerate_static(const uint64_t *rows, int64_t n_objects, int64_t n_attrs, int64_t row_stride_words,
                          uint32_t flags, void *hip_stream, uint64_t *intents_out, uint64_t *extents_out,
                          uint64_t capacity, uint64_t *n_concepts_out, fcbo_stats *stats_out)
{
    if (!valid_context_args(rows, n_objects, n_attrs, row_stride_words) || (flags & ~FCBO_ROWS_ON_DEVICE))
        return FCBO_ERR_INVALID_ARGUMENT;
    {
        // the context alone (rows with the zero row, columns, scan partials,
        // counters) must leave at least half of the scratch to the enumeration
        const uint64_t wn = ((uint64_t)n_objects + 63) / 64, wm = ((uint64_t)n_attrs + 63) / 64;
        const uint64_t words = ((uint64_t)n_objects + 1) * wm + (uint64_t)n_attrs * wn + 2 * kScanBlocks + 2 * CNT_N;
        if (words * 8 + 4 * 256 > (uint64_t)FCBO_STATIC_SCRATCH_BYTES / 2) return FCBO_ERR_SCRATCH;
    }
    fcbo_stats st;
    memset(&st, 0, sizeof(st));
    hipStream_t stream = (hipStream_t)hip_stream;
    int rc = FCBO_OK;
    try {
        fcbo_context c;
        CK(hipGetDevice(&c.device));
        (void)hipGetLastError();  // an error left by earlier, unrelated work is not this call's
        c.stream = stream;
        c.fixed = true;
        c.dmem.region = scratch_on_device(c.device);
        c.dmem.region_size = FCBO_STATIC_SCRATCH_BYTES;
        c.setup(rows, n_objects, n_attrs, row_stride_words, (flags & FCBO_ROWS_ON_DEVICE) != 0);
        c.enumerate_levels();
        if (n_concepts_out) *n_concepts_out = c.K;
        if (!intents_out || capacity < c.K) {
            rc = FCBO_ERR_CAPACITY;
        } else {
            c.order_concepts();
            c.write_output(intents_out, extents_out, 0, c.K);
        }
        CK(hipStreamSynchronize(stream));
        c.fill_counts(st, c.have_result ? c.K : 0);
        st.batches = 1;
        st.peak_device_bytes = c.dmem.region_used;
        if (rc == FCBO_OK)
            st.output_bytes = c.K * (uint64_t)c.wm * 8 + (extents_out ? c.K * (uint64_t)c.wn * 8 : 0);
    } catch (const HipError &e) {
        (void)hipStreamSynchronize(stream);  // nothing of this call runs on after it returns
        return e.code;
    } catch (const std::bad_alloc &) {
        (void)hipStreamSynchronize(stream);
        return FCBO_ERR_OUT_OF_MEMORY;
    }
    if (stats_out) *stats_out = st;
    return rc;
}

int fcbo_enumerate_bounded(fcbo_context *ctx, uint64_t *intents_buf, uint64_t *extents_buf, uint64_t piece_rows,
                           fcbo_sink_fn sink, void *user, uint32_t flags, uint64_t *n_concepts_out,
                           fcbo_stats *stats_out)
{
    if (!ctx || (flags & ~(FCBO_PROFILE | FCBO_ONE_SUBTREE_PER_BATCH | FCBO_SPLIT_ROOT_CHILDREN)) ||
        ((intents_buf || extents_buf) && piece_rows == 0))
        return FCBO_ERR_INVALID_ARGUMENT;
    fcbo_stats st;
    memset(&st, 0, sizeof(st));
    int rc = FCBO_OK;
    try {
        CK(hipSetDevice(ctx->device));
        (void)hipGetLastError();  // an error left by earlier, unrelated work is not this call's
        ctx->profile = (flags & FCBO_PROFILE) != 0;
        ctx->enumerate_bounded(intents_buf, extents_buf, piece_rows, sink, user, flags, st);
    } catch (const HipError &e) {
        rc = e.code;
    } catch (const std::bad_alloc &) {
        rc = FCBO_ERR_OUT_OF_MEMORY;
    }
    if (rc != FCBO_OK) {
        // nothing half-done stays: no result, no level counts, no work in flight
        ctx->have_result = ctx->have_perm = ctx->have_cover_counts = ctx->have_levels = false;
        ctx->K = 0;
        for (int i = 0; i < fcbo_context::kSide; ++i)
            if (ctx->aux[i]) (void)hipStreamSynchronize(ctx->aux[i]);
        (void)hipStreamSynchronize(ctx->stream);
        ctx->release_seeds();
        ctx->marks.clear();
        ctx->ev_used = 0;
        return rc;
    }
    if (n_concepts_out) *n_concepts_out = st.n_concepts;
    if (stats_out) *stats_out = st;
    return FCBO_OK;
}

int fcbo_write_range(fcbo_context *ctx, uint64_t first, uint64_t count, uint64_t *intents_out,
                     uint64_t *extents_out)
{
    if (!ctx || (!intents_out && !extents_out) || !ctx->have_result || first > ctx->K || count > ctx->K - first)
        return FCBO_ERR_INVALID_ARGUMENT;
    try {
        CK(hipSetDevice(ctx->device));
        (void)hipGetLastError();  // an error left by earlier, unrelated work is not this call's
        ctx->profile = false;
        ctx->ev_used = 0;
        ctx->marks.clear();
        if (!ctx->have_perm) ctx->order_concepts();
        if (count) ctx->write_output(intents_out, extents_out, first, count);
        CK(hipStreamSynchronize(ctx->stream));
    } catch (const HipError &e) {
        return e.code;
    } catch (const std::bad_alloc &) {
        return FCBO_ERR_OUT_OF_MEMORY;
    }
    return FCBO_OK;
}

int fcbo_cover_edges(fcbo_context *ctx, uint64_t *offsets_out, uint32_t *targets_out, uint64_t capacity,
                     uint64_t *n_edges_out, double *elapsed_ms)
{
    if (!ctx || !ctx->have_result) return FCBO_ERR_INVALID_ARGUMENT;
    if (ctx->m > kCoverMaxM) return FCBO_ERR_INVALID_ARGUMENT;
    int rc = FCBO_OK;
    try {
        CK(hipSetDevice(ctx->device));
        (void)hipGetLastError();  // an error left by earlier, unrelated work is not this call's
        ctx->profile = false;
        ctx->ev_used = 0;
        ctx->marks.clear();
        hipEvent_t e0 = ctx->ev_get(), e1 = ctx->ev_get();
        CK(hipEventRecord(e0, ctx->stream));
        const uint64_t e = ctx->cover_edges(offsets_out, targets_out, capacity);
        CK(hipEventRecord(e1, ctx->stream));
        CK(hipStreamSynchronize(ctx->stream));
        if (n_edges_out) *n_edges_out = e;
        if (!offsets_out || !targets_out || capacity < e) rc = FCBO_ERR_CAPACITY;
        if (elapsed_ms) {
            float ms = 0;
            CK(hipEventElapsedTime(&ms, e0, e1));
            *elapsed_ms = ms;
        }
    } catch (const HipError &err) {
        return err.code;
    } catch (const std::bad_alloc &) {
        return FCBO_ERR_OUT_OF_MEMORY;
    }
    return rc;
}

int fcbo_copy_to_host(fcbo_context *ctx, uint64_t first, uint64_t count, uint64_t *host_intents,
                      uint64_t *host_extents, uint64_t staging_rows, double *elapsed_ms)
{
    if (!ctx || (!host_intents && !host_extents) || !ctx->have_result || first > ctx->K ||
        count > ctx->K - first || staging_rows == 0)
        return FCBO_ERR_INVALID_ARGUMENT;
    try {
        CK(hipSetDevice(ctx->device));
        (void)hipGetLastError();  // an error left by earlier, unrelated work is not this call's
        ctx->profile = false;
        ctx->ev_used = 0;
        ctx->marks.clear();
        hipEvent_t e0 = ctx->ev_get(), e1 = ctx->ev_get();
        CK(hipEventRecord(e0, ctx->stream));
        if (count) ctx->copy_to_host(first, count, host_intents, host_extents, staging_rows);
        CK(hipEventRecord(e1, ctx->stream));
        CK(hipStreamSynchronize(ctx->stream));
        if (elapsed_ms) {
            float ms = 0;
            CK(hipEventElapsedTime(&ms, e0, e1));
            *elapsed_ms = ms;
        }
    } catch (const HipError &e) {
        return e.code;
    } catch (const std::bad_alloc &) {
        return FCBO_ERR_OUT_OF_MEMORY;
    }
    return FCBO_OK;
}

int fcbo_set_memory_limit(fcbo_context *ctx, uint64_t bytes)
{
    if (!ctx) return FCBO_ERR_INVALID_ARGUMENT;
    ctx->dmem.limit = bytes;
    if (bytes && ctx->dmem.held > bytes) {
        // the cap holds from now on: the buffers (and the result in them) go
        hipError_t e = hipSetDevice(ctx->device);
        if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
        if (e != hipSuccess) return map_error(e);
        ctx->free_buffers();
    }
    return FCBO_OK;
}

int fcbo_level_counts(const fcbo_context *ctx, uint64_t *concepts_per_level, uint64_t *tests_per_level,
                      uint64_t max_levels, uint64_t *n_levels_out)
{
    if (!ctx || !ctx->have_levels) return FCBO_ERR_INVALID_ARGUMENT;
    const uint64_t nl = ctx->lev.size();
    if (n_levels_out) *n_levels_out = nl;
    for (uint64_t i = 0; i < nl && i < max_levels; ++i) {
        if (concepts_per_level) concepts_per_level[i] = ctx->lev.concepts[i];
        if (tests_per_level) tests_per_level[i] = ctx->lev.tests[i];
    }
    return FCBO_OK;
}

int fcbo_copy_columns(const fcbo_context *ctx, uint64_t *host_cols, uint64_t capacity_words)
{
    if (!ctx || !host_cols) return FCBO_ERR_INVALID_ARGUMENT;
    const uint64_t words = (uint64_t)ctx->m * ctx->wn;
    if (capacity_words < words) return FCBO_ERR_CAPACITY;
    hipError_t e = hipSetDevice(ctx->device);
    if (e == hipSuccess) e = hipMemcpyAsync(host_cols, ctx->cols, words * sizeof(uint64_t), hipMemcpyDeviceToHost, ctx->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
    return map_error(e);
}

void fcbo_destroy(fcbo_context *ctx)
{
    if (!ctx) return;
    (void)hipSetDevice(ctx->device);
    if (ctx->stream) (void)hipStreamSynchronize(ctx->stream);
    else (void)hipDeviceSynchronize();
    ctx->free_all();
    delete ctx;
}

}  // extern "C"
