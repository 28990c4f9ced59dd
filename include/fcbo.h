/*
 * fcbo.h - C ABI of the MI355X formal-concept enumeration library (libfcbo.so).
 *
 * The library lists every formal concept (extent, intent) of a 0/1 formal
 * context with Close-by-One: starting from the root (all objects, the
 * attributes they share) every concept (A, B) with cursor y tries each
 * attribute j > y that is not in B, forms C = A AND col[j] and D = C', and keeps
 * (C, D) with cursor j iff D and B agree on the attributes below j.
 *   - concept, derivation and closure: page "hnwysp.cn/news/97538", sections
 *     1.1-1.2, and page "hotelren.com/news/5603750", section 1.1;
 *   - the CbO step, canonical test and attribute-saturation skip: page 1,
 *     sections 2.1-2.3 and 4.3; page 4, sections 1.2 and 3.2;
 *   - the two bitmap layouts kept on the device: page 1 section 3.1, page 4
 *     section 2.3;
 *   - the sorted, deterministic output: page 1 section 6.2.
 *
 * Bit layout everywhere: element e of a set is bit (e & 63) of 64-bit word
 * (e >> 6), least significant bit first.  Bits past the last object or the
 * last attribute are zero in everything the library writes.
 *
 * Output order: concepts are listed in lexicographic order of the intent read
 * as a bit string over the attributes 0, 1, ..., M-1: of two intents, the one
 * holding the smallest attribute in which they differ comes later (so the
 * root, whose intent is contained in every other, is first).  Intents are
 * pairwise distinct, so the order is total and the output is byte-for-byte
 * unique.  "Output position" below means the index of a concept in this order.
 *
 * Errors are reported only by return code; no call aborts or throws.  A HIP
 * failure maps to FCBO_ERR_DEVICE (FCBO_ERR_OUT_OF_MEMORY for allocation) and
 * leaves the context safe to destroy.  After any error from fcbo_enumerate the
 * context holds no result (a later FCBO_REUSE_RESULT call enumerates again).
 * A context must not be used from two host threads at once.
 *
 * Limits: 1 <= N <= 2^31 - 1 objects, 1 <= M <= 4096 attributes, fewer than
 * 2^32 concepts (concept indices are 32-bit on the device).
 */
#ifndef FCBO_H
#define FCBO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fcbo_context fcbo_context; /* opaque, owned by the library */

enum {
    FCBO_OK = 0,
    FCBO_ERR_INVALID_ARGUMENT = -1, /* null pointer, bad size, bad flag, no result yet */
    FCBO_ERR_OUT_OF_MEMORY = -2,    /* a device allocation failed or the memory limit was hit */
    FCBO_ERR_DEVICE = -3,           /* any other HIP runtime failure */
    FCBO_ERR_CAPACITY = -4,         /* output buffers hold fewer rows than concepts (or edges) */
    FCBO_ERR_LIMIT = -5,            /* 2^32 concepts or more: beyond the 32-bit concept indices */
    FCBO_ERR_SCRATCH = -6,          /* fcbo_enumerate_static: the work does not fit the static scratch */
    FCBO_ERR_STOPPED = -7           /* fcbo_enumerate_bounded: the sink asked to stop */
};

/* Bytes of the static device scratch of fcbo_enumerate_static (one per GPU). */
#define FCBO_STATIC_SCRATCH_BYTES (64u << 20)

/* fcbo_context_create flags */
#define FCBO_ROWS_ON_DEVICE 1u /* rows is a device pointer (else host memory) */
#define FCBO_TINY_BUFFERS 2u   /* test hook: start every device buffer at its minimum size, so
                                  growth and the level redo run on any input */

/* fcbo_enumerate flags */
#define FCBO_REUSE_RESULT 1u /* reuse the concepts of the previous call if any */
#define FCBO_PROFILE 2u      /* time every kernel class with HIP events (fills kernel_ms) */
#define FCBO_TASK_POOL 16u   /* schedule the search as a task pool (M <= 512): the level loop
                                expands only the parents with more than 16 objects, and the
                                subtree of every concept with at most 16 objects is one task,
                                enumerated depth-first by one wavefront; wavefronts claim tasks
                                from shared counters as they free up (page 1 sections 3.2 and
                                5.3; page 4 section 4.3) */

/* fcbo_enumerate_bounded flags (besides FCBO_PROFILE) */
#define FCBO_ONE_SUBTREE_PER_BATCH 4u /* test hook: every batch takes a single subtree, so the
                                         batch path runs on any input; its seeds' parent classes
                                         are not announced to the level loop, which then finds
                                         them on the level and runs the level again */
#define FCBO_SPLIT_ROOT_CHILDREN 8u   /* test hook: every child of the root is split one level
                                         down as if its subtree did not fit */

/* Kernel classes reported in fcbo_stats.kernel_ms / kernel_launches. */
enum {
    FCBO_K_COUNT = 0,        /* reserved: the per-parent counts and classes are made by the
                                local test kernel and timed under FCBO_K_TEST_LOCAL */
    FCBO_K_TEST_LOCAL = 1,   /* closure tests of parents with <= 64 objects */
    FCBO_K_TEST_MEDIUM = 2,  /* closure tests of parents with 65..4096 objects (M <= 512 only) */
    FCBO_K_TEST_BIG = 3,     /* closure tests of the larger parents (tasks + tests) */
    FCBO_K_SCAN = 4,         /* exclusive scans (children, objects, big tests) */
    FCBO_K_WRITE_LOCAL = 5,  /* child write, parents with <= 64 objects */
    FCBO_K_WRITE_MEDIUM = 6, /* child write, parents of the medium class */
    FCBO_K_WRITE_BIG = 7,    /* child write, larger parents */
    FCBO_K_ORDER = 8,        /* output positions from the CbO tree (sizes, positions, inverse) */
    FCBO_K_OUTPUT = 9,       /* ordered intents + extent bitmaps to the caller */
    FCBO_K_NUM_CLASSES = 10
};

/*
 * Statistics of one fcbo_enumerate call.  The first eight fields are the
 * measurement record of the method (concept count, closure tests, item pairs,
 * levels, times, algorithmic bytes); the rest break the work down by the
 * library's parent classes.
 *
 * A closure test is one (parent, j) with j > cursor and j not in B (page 1,
 * section 2.1; saturated j in B are skipped without a test, section 2.3); an
 * item pair is one (parent, j) with j > cursor (page 4, section 2.1 counts
 * parents x attributes).
 *
 * model_bytes: the algorithmic bytes of the enumeration (root to last level),
 * independent of how the kernels are scheduled.  Parents whose extent has at
 * most T objects are tested row-locally (T = 4096 when M <= 512, else 64):
 *     K * (8 W_M + 4 + 16)                  every concept read once as a parent:
 *                                           intent, cursor, extent-list bounds
 *   + S_rl * (4 + 8 W_M)                    row-local parents: each object's list
 *                                           entry and row, once
 *   + P_col * 8 W_N                         larger parents: extent bitmap, once
 *   + Z_col * 8                             their tests: the words of col[j] where
 *                                           the extent is non-zero (page 1 section
 *                                           4.2 skips the zero words)
 *   + C_col * 8 W_M                         their children: the rows of C
 *   + (K - 1) * (8 W_M + 4 + 8) + 4 sum|C|  every child written: intent, cursor,
 *                                           list offset, extent list
 *   + N * (8 W_M + 4)                       the root: all rows read, its list
 * with W_N = ceil(N/64), W_M = ceil(M/64), S_rl the objects of the row-local
 * parents' extents, P_col the larger parents, Z_col the sum over their tests
 * of the non-zero words of their extent, C_col the objects of their children.
 */
typedef struct {
    uint64_t n_concepts;        /* K */
    uint64_t closure_tests;     /* (parent, j) with j > cursor and j not in B */
    uint64_t item_pairs;        /* (parent, j) with j > cursor */
    uint64_t n_levels;          /* levels of the CbO tree, root level included */
    double enumerate_ms;        /* whole call on the device stream (HIP events) */
    double closure_kernel_ms;   /* the level loop: root to last level, closure tests, scans,
                                   child writes and the per-level host wait (HIP events) */
    double sort_ms;             /* output order: positions from the CbO tree */
    uint64_t model_bytes;       /* algorithmic bytes of the level loop (formula above) */
    double output_ms;           /* writing the caller's buffers */
    uint64_t sum_child_objects; /* sum of |C| over all concepts except the root */
    uint64_t output_bytes;      /* bytes written to the caller's buffers */
    uint64_t local_parents;     /* parents with <= 64 objects (packed local test kernel) */
    uint64_t local_parent_objects;  /* objects in their extents (rows staged) */
    uint64_t medium_parents;    /* parents of the medium class (tests by incidence) */
    uint64_t medium_parent_objects; /* objects in their extents */
    uint64_t big_parents;       /* larger parents (tests split in 64-word extent chunks or list scans) */
    uint64_t big_tests;         /* closure tests made by them */
    uint64_t big_scanned_objects;   /* extent-list entries read by those tests */
    uint64_t big_nonzero_words; /* Z_col above: sum over their tests of the extent's non-zero words */
    uint64_t big_child_objects; /* C_col above: objects of their children */
    uint64_t order_launches;    /* kernel launches of the last output ordering */
    double kernel_ms[FCBO_K_NUM_CLASSES];       /* with FCBO_PROFILE only */
    uint64_t kernel_launches[FCBO_K_NUM_CLASSES];
    uint64_t batches;           /* batches of sibling subtrees enumerated (1 for fcbo_enumerate) */
    uint64_t batch_retries;     /* batches that hit the memory limit and were run again smaller */
    uint64_t batch_splits;      /* single subtrees that did not fit and were split one level down */
    uint64_t peak_device_bytes; /* most device memory the enumeration buffers held at once during
                                   the call (buffers kept from earlier calls included) */
    uint64_t level_redos;       /* levels run again: a record buffer overflowed, or parents of a
                                   class the level loop was not told about turned up */
} fcbo_stats;

/*
 * Build a context from the 0/1 object x attribute table (page 1 section 1.1,
 * page 4 section 1.1), kept on the device as rows and as their transpose, the
 * columns (page 1 section 3.1, page 4 sections 2.3 and 3.1).
 *   rows              row g (the attributes of object g) starts at
 *                     rows + g * row_stride_words; host memory, or device
 *                     memory on the current HIP device with FCBO_ROWS_ON_DEVICE.
 *                     The library copies it; the caller keeps ownership.  Bits
 *                     past n_attrs in the last word are ignored.
 *   n_objects         N, 1 <= N <= 2^31 - 1
 *   n_attrs           M, 1 <= M <= 4096
 *   row_stride_words  >= ceil(M / 64)
 *   flags             FCBO_ROWS_ON_DEVICE, FCBO_TINY_BUFFERS
 *   hip_stream        hipStream_t the calls are ordered on, or NULL for the null
 *                     stream.  Independent parts of a level also run on two
 *                     internal streams of the context (default priority) that
 *                     fork from and join back to this one through events.
 *   out               receives the context
 * The device holds the rows (N x ceil(M/64) words) and the columns
 * (M x ceil(N/64) words, column j = objects having attribute j).
 * Returns FCBO_OK, FCBO_ERR_INVALID_ARGUMENT (bad sizes or flags, null
 * pointers), FCBO_ERR_OUT_OF_MEMORY or FCBO_ERR_DEVICE; *out is NULL on error.
 */
int fcbo_context_create(const uint64_t *rows, int64_t n_objects, int64_t n_attrs,
                        int64_t row_stride_words, uint32_t flags, void *hip_stream,
                        fcbo_context **out);

/*
 * Enumerate all concepts with Close-by-One (page 1 sections 2.1-2.3 and
 * 4.2-4.4; page 4 sections 1.2, 2.1 and 3.2; level by level as page 4 section
 * 2.1 expands the tree, with page 1's canonical test so no concept repeats)
 * and write them in the output order (page 1 section 6.2) to caller-owned
 * device buffers on the context's device.
 *   intents_out   K x ceil(M/64) words, row i = intent of concept i
 *   extents_out   K x ceil(N/64) words in the same order, or NULL to skip
 *   capacity      rows available in the output buffers
 *   flags         FCBO_REUSE_RESULT, FCBO_PROFILE, FCBO_TASK_POOL (M <= 512, else
 *                 FCBO_ERR_INVALID_ARGUMENT); the result is the same either way
 *   n_concepts_out receives K (also on FCBO_ERR_CAPACITY); may be NULL
 *   stats_out     optional statistics, or NULL
 * If intents_out is NULL or capacity < K the call returns FCBO_ERR_CAPACITY,
 * stores K and writes nothing; the concepts stay in the context, so a second
 * call with FCBO_REUSE_RESULT and large enough buffers only orders and writes.
 * Device buffers grow as the levels need (page 4 section 4.1); a failed
 * allocation or the memory limit gives FCBO_ERR_OUT_OF_MEMORY, 2^32 concepts
 * or more FCBO_ERR_LIMIT.  The call returns after the stream has finished.
 */
int fcbo_enumerate(fcbo_context *ctx, uint64_t *intents_out, uint64_t *extents_out,
                   uint64_t capacity, uint32_t flags, uint64_t *n_concepts_out,
                   fcbo_stats *stats_out);

/*
 * Write the output rows [first, first + count) of the last enumeration: row r
 * of intents_out / extents_out receives the concept at output position
 * first + r.  Either buffer may be NULL (not both).  With it a caller pages
 * the output through bounded device buffers (page 1 section 6.1 moves
 * concepts off the device in batches when they do not fit at once), e.g. the
 * extent bitmaps of a context whose K x N/8 bytes exceed device memory.
 * FCBO_ERR_INVALID_ARGUMENT if nothing was enumerated or first + count > K.
 * Returns after the stream has finished.
 */
int fcbo_write_range(fcbo_context *ctx, uint64_t first, uint64_t count, uint64_t *intents_out,
                     uint64_t *extents_out);

/*
 * Output rows [first, first + count) of the last enumeration into host memory
 * (row r of host_intents / host_extents = output position first + r; either may
 * be NULL, not both), staging_rows rows at a time through two device buffers:
 * the output kernels fill one on the context's stream while the other is copied
 * to the host on an internal stream, so writing and copying overlap (page 1
 * section 6.1 moves concepts to the host in batches with copy and compute
 * staggered; page 4 section 5.2 overlaps transfers with streams).  Device
 * memory for the output stays bounded by 2 x staging_rows rows, whatever K is.
 * Pinned host memory (hipHostMalloc) lets the copies run asynchronously;
 * pageable memory works but the runtime then stages each copy.
 * elapsed_ms (optional) receives the call's time on the context's stream.
 * FCBO_ERR_INVALID_ARGUMENT if nothing was enumerated, first + count > K or
 * staging_rows is 0.  Returns after the copies have finished.
 */
int fcbo_copy_to_host(fcbo_context *ctx, uint64_t first, uint64_t count, uint64_t *host_intents,
                      uint64_t *host_extents, uint64_t staging_rows, double *elapsed_ms);

/*
 * Lattice cover edges of the last enumeration (page 1 section 4.4 and page 4
 * section 3.4 rebuild them after the concepts are found): for the concept at
 * output position i, the output positions of its lower covers (the concepts
 * right below it in the lattice: extent strictly inside, nothing between), in
 * ascending order, at targets_out[offsets_out[i] .. offsets_out[i + 1]).
 *   offsets_out   K + 1 words, device
 *   targets_out   E 32-bit positions, device
 *   capacity      entries available in targets_out
 *   n_edges_out   receives E (also on FCBO_ERR_CAPACITY); may be NULL
 *   elapsed_ms    device time of the call (HIP events), or NULL
 * If either buffer is NULL or capacity < E the call returns FCBO_ERR_CAPACITY,
 * stores E and writes nothing.  FCBO_ERR_INVALID_ARGUMENT if nothing was
 * enumerated.  Returns after the stream has finished.
 * The first call on a result finds every concept's covers and keeps the
 * counts, and for 2^20 concepts or more (when device memory allows: about 4
 * bytes a cover and 8 a concept) the covers' positions too, until the next
 * enumeration; a later call with large enough buffers then only copies them
 * out.
 */
int fcbo_cover_edges(fcbo_context *ctx, uint64_t *offsets_out, uint32_t *targets_out, uint64_t capacity,
                     uint64_t *n_edges_out, double *elapsed_ms);

/*
 * Receiver of the pieces of a bounded enumeration: rows [0, count) of the
 * device buffers hold the concepts at output positions [first, first + count)
 * (intents, and extents unless that buffer is NULL).  Pieces arrive in
 * ascending order of first and cover every position once.  The context's
 * stream has finished when the sink is called and the library touches neither
 * buffer until it returns; the sink may read or copy them on any stream, but
 * must be done with them when it returns.  Return 0 to go on, anything else to
 * stop the enumeration.
 */
typedef int (*fcbo_sink_fn)(void *user, uint64_t first, uint64_t count, const uint64_t *intents,
                            const uint64_t *extents);

/*
 * Enumerate like fcbo_enumerate in bounded device memory, handing the output
 * to a sink piece by piece (page 1 section 6.1: when the concepts do not fit
 * the device, move finished ones off it in batches while the search goes on;
 * section 3.4 bounds the task memory).  In the output order every subtree of
 * the CbO tree is one run of consecutive positions: a concept, then its
 * children's subtrees by descending attribute.  So the root's children are
 * taken in batches, largest attribute first; a batch's subtrees are
 * enumerated level by level, ordered and written out, and the store is reused
 * by the next batch.  A batch that hits the memory limit
 * (fcbo_set_memory_limit) or a full device runs again with half as many
 * subtrees; a single subtree that does not fit is split one level down (its
 * root's row goes out, its children become the next run of batches).  Once a
 * batch has failed, batches are sized from the concepts per unit of seed
 * weight (objects times the attributes above the cursor) of the last batch
 * that fitted, aiming at 70% of the smallest store size at which one failed,
 * and never above half a size that failed in the same run.  Device memory thus stays within the limit as
 * long as one concept's children (one level) fit; the total concept count may
 * exceed 2^32, the concepts of one batch may not.
 *   intents_buf   piece_rows x ceil(M/64) words, device, or NULL
 *   extents_buf   piece_rows x ceil(N/64) words, device, or NULL
 *   piece_rows    rows per piece (>= 1 when a buffer is given)
 *   sink, user    called once per piece; may be NULL.  With both buffers NULL
 *                 nothing is ordered or written and the sink is not called
 *                 (counts and statistics only).
 *   flags         FCBO_PROFILE, FCBO_ONE_SUBTREE_PER_BATCH, FCBO_SPLIT_ROOT_CHILDREN
 *   n_concepts_out receives K; may be NULL
 *   stats_out     optional: counts as for fcbo_enumerate, summed over the
 *                 batches; enumerate_ms = the call's host wall time (sink
 *                 included), closure_kernel_ms / sort_ms / output_ms = device
 *                 time of the level loops / order passes / output kernels;
 *                 batches, batch_retries, batch_splits, peak_device_bytes
 * Returns FCBO_OK, FCBO_ERR_INVALID_ARGUMENT, FCBO_ERR_OUT_OF_MEMORY (one
 * concept's children do not fit), FCBO_ERR_STOPPED (the sink returned
 * non-zero) or FCBO_ERR_DEVICE.  Afterwards the context holds no result
 * (write_range, copy_to_host and cover_edges return FCBO_ERR_INVALID_ARGUMENT
 * until the next fcbo_enumerate); fcbo_level_counts reports the whole
 * enumeration.  After an error it reports nothing either.
 */
int fcbo_enumerate_bounded(fcbo_context *ctx, uint64_t *intents_buf, uint64_t *extents_buf, uint64_t piece_rows,
                           fcbo_sink_fn sink, void *user, uint32_t flags, uint64_t *n_concepts_out,
                           fcbo_stats *stats_out);

/*
 * Cap the device memory the context's enumeration buffers may hold (bytes;
 * 0 = no cap).  An enumeration that would need more fails with
 * FCBO_ERR_OUT_OF_MEMORY at the allocation that crosses the cap, as a full
 * device would (page 4 section 4.1: pool overflow; page 1 section 6.1: device
 * memory budget).  If the buffers already hold more than the new cap they are
 * released, and the last result with them.  The rows and columns built at
 * creation are not counted.
 */
int fcbo_set_memory_limit(fcbo_context *ctx, uint64_t bytes);

/*
 * Diagnostic: per-level counts of the last enumeration, concepts generated on
 * level k (level 0 is the root) and closure tests made by the concepts of
 * level k (page 4 section 6 checks exactly these against a serial run).
 * Copies min(n_levels, max_levels) entries; *n_levels_out gets n_levels.
 * Either array may be NULL.  FCBO_ERR_INVALID_ARGUMENT if nothing was
 * enumerated yet.
 */
int fcbo_level_counts(const fcbo_context *ctx, uint64_t *concepts_per_level,
                      uint64_t *tests_per_level, uint64_t max_levels, uint64_t *n_levels_out);

/*
 * Test hook: copy the device column bitmap (M x ceil(N/64) words, column j =
 * objects having attribute j; page 1 section 3.1) into a host buffer of at
 * least that many words, so tests can check the transpose.
 * FCBO_ERR_CAPACITY if capacity_words is too small.
 */
int fcbo_copy_columns(const fcbo_context *ctx, uint64_t *host_cols, uint64_t capacity_words);

/*
 * For callers that cannot allocate device memory (tight serving loops,
 * harnesses that forbid hipMalloc): the whole of fcbo_context_create +
 * fcbo_enumerate + fcbo_destroy in one call that allocates nothing.  Every
 * device buffer of the enumeration (rows, columns, concept store, level
 * buffers, output order) is carved from a static device array of
 * FCBO_STATIC_SCRATCH_BYTES (64 MiB), one per GPU, held until the process
 * ends; no hipMalloc, hipFree, pinned host memory, event or stream is created,
 * and the per-level wait synchronises the caller's stream.
 *   rows ... row_stride_words, flags   as for fcbo_context_create (flags:
 *                                      FCBO_ROWS_ON_DEVICE only)
 *   hip_stream                         the stream the work runs on (NULL: the
 *                                      null stream)
 *   intents_out ... stats_out          as for fcbo_enumerate (stats without
 *                                      times)
 * Returns FCBO_ERR_SCRATCH if the context or its enumeration needs more than
 * the scratch (up front when the rows and columns alone take more than half
 * of it), FCBO_ERR_CAPACITY with K if the outputs are too small (nothing is
 * kept: a second call enumerates again).  All calls on one GPU share its
 * scratch: calls that overlap on one GPU (two host threads, or two streams
 * not ordered with each other) race.  The scratch keeps the last call's
 * contents; a call clears or writes everything it reads first.  Returns after
 * the stream has finished.
 */
int fcbo_enumerate_static(const uint64_t *rows, int64_t n_objects, int64_t n_attrs, int64_t row_stride_words,
                          uint32_t flags, void *hip_stream, uint64_t *intents_out, uint64_t *extents_out,
                          uint64_t capacity, uint64_t *n_concepts_out, fcbo_stats *stats_out);

/* Free the context and everything it owns.  NULL is allowed. */
void fcbo_destroy(fcbo_context *ctx);

/* Static text for an error code. */
const char *fcbo_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* FCBO_H */
