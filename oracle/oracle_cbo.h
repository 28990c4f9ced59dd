/*
 * Serial CbO oracle interface.  TEST INFRASTRUCTURE ONLY: used by the test
 * suite, the smoke check and the CPU-baseline leg of the benchmark, never by
 * the GPU library (which has its own header and shares nothing with this).
 */
#ifndef ORACLE_CBO_H
#define ORACLE_CBO_H

#include <stdint.h>

/* oracle_cbo flags */
#define ORACLE_KEEP_EXTENTS 1 /* return every extent bitmap */
#define ORACLE_HASH_EXTENTS 2 /* return every extent's 64-bit hash g(A) (cbo.c) */

typedef struct {
    int64_t n_concepts;            /* concepts found (all of them unless truncated) */
    int64_t tests;                 /* closure tests: (node, j) with j > cursor, j not in B */
    int64_t pairs;                 /* (node, j) with j > cursor */
    int64_t sum_nzw;               /* sum over tests of the non-zero words of the parent extent */
    int64_t sum_c;                 /* sum over kept children of |C| */
    int64_t saturation_violations; /* j not in B although A inside col[j]; 0 for closed B */
    /* the byte-model split by the row-local threshold T (rowlocal_max) */
    int64_t sum_rl_objs;           /* objects of the parents with |A| <= T */
    int64_t col_parents;           /* parents with |A| > T */
    int64_t col_nzw;               /* sum over their tests of the non-zero words of A */
    int64_t col_child_objs;        /* sum over their kept children of |C| */
    int32_t n_levels;              /* deepest level + 1 (root is level 0) */
    int32_t truncated;             /* stopped early at max_tests */
    int64_t *level_concepts;       /* [M + 2] concepts per level */
    int64_t *level_tests;          /* [M + 2] tests made by the nodes of each level */
    uint64_t *intents;             /* n_concepts x wm, lexicographic over attributes 0..M-1 */
    uint64_t *extents;             /* n_concepts x wn in the same order, or NULL */
    uint64_t *extent_hashes;       /* n_concepts g(A) in the same order, or NULL */
    int64_t wn, wm;                /* words per extent / per intent */
    double seconds_enum;           /* enumeration wall time */
    double seconds_sort;           /* final sort wall time */
} oracle_result;

/* Enumerate all concepts of the context whose row g (attributes of object g)
 * starts at rows + g * row_stride.  max_tests < 0 means no limit; otherwise the
 * search stops after that many closure tests and sets truncated.
 * rowlocal_max is the threshold T of the byte-model split.  Returns 0 on
 * success, -1 on bad arguments, -2 when memory runs out. */
int oracle_cbo(const uint64_t *rows, int64_t n_objects, int64_t n_attrs, int64_t row_stride,
               int flags, int64_t max_tests, int64_t rowlocal_max, oracle_result *out);

void oracle_free(oracle_result *r);

/* A subtree of the CbO tree in output order, its root at local position 0:
 * size, sum of intent hashes h, sum of local position x h, and the same two
 * sums for the extent hashes g (mod 2^64). */
typedef struct {
    int64_t size;
    uint64_t hi0, hi1, he0, he1;
} oracle_subtree;

/* Counters and digests of the same search without storing concepts
 * (cbo_digest.c). */
typedef struct {
    int64_t n_concepts;
    int64_t tests;
    int64_t pairs;
    int64_t sum_c;
    int32_t n_levels;
    int32_t threads;               /* worker threads that ran */
    int64_t *level_concepts;       /* [M + 2] */
    int64_t *level_tests;          /* [M + 2] */
    uint64_t digest;               /* sum of intent hashes, counted per concept */
    int64_t subtree_size;          /* concepts in the combined summary (= n_concepts) */
    uint64_t intent_digest;        /* sum of intent hashes from the summaries (= digest) */
    uint64_t intent_positional;    /* sum over output positions i of i x h(intent_i) */
    uint64_t extent_digest;        /* sum of extent hashes */
    uint64_t extent_positional;    /* sum over output positions i of i x g(extent_i) */
    int32_t n_root_children;
    int32_t *root_child_attr;      /* attribute of each child of the root, descending (output order) */
    oracle_subtree *root_child;    /* their subtrees' summaries, in the same order */
    double seconds;                /* search wall time */
} oracle_digest;

/* Returns 0, -1 on bad arguments, -2 when memory runs out. */
int oracle_cbo_digest(const uint64_t *rows, int64_t n_objects, int64_t n_attrs, int64_t row_stride, int threads,
                      oracle_digest *out);

void oracle_digest_free(oracle_digest *d);

/* Lower covers of every concept of a complete concept list (cover.c): the
 * intents, K x wm words, in the output order of oracle_cbo.  offsets gets
 * K + 1 entries; *targets_out (free with oracle_cover_free) the positions of
 * the lower covers of concept i at [offsets[i], offsets[i + 1]), ascending.
 * Returns 0, -1 on bad arguments, -2 when memory runs out, -3 if a closure is
 * missing from the list. */
int oracle_cover_edges(const uint64_t *rows, int64_t n_objects, int64_t n_attrs, int64_t row_stride,
                       const uint64_t *intents, int64_t k, int64_t *offsets, int64_t **targets_out,
                       int64_t *n_edges_out);

void oracle_cover_free(int64_t *targets);

#endif
