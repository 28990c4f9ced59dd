/*
 * Serial CbO oracle interface.  TEST INFRASTRUCTURE ONLY: used by the test
 * suite, the smoke check and the CPU-baseline leg of the benchmark, never by
 * the GPU library (which has its own header and shares nothing with this).
 */
#ifndef ORACLE_CBO_H
#define ORACLE_CBO_H

#include <stdint.h>

typedef struct {
    int64_t n_concepts;            /* concepts found (all of them unless truncated) */
    int64_t tests;                 /* closure tests: (node, j) with j > cursor, j not in B */
    int64_t pairs;                 /* (node, j) with j > cursor */
    int64_t sum_nzw;               /* sum over tests of the non-zero words of the parent extent */
    int64_t sum_c;                 /* sum over kept children of |C| */
    int64_t saturation_violations; /* j not in B although A inside col[j]; 0 for closed B */
    int32_t n_levels;              /* deepest level + 1 (root is level 0) */
    int32_t truncated;             /* stopped early at max_tests */
    int64_t *level_concepts;       /* [M + 2] concepts per level */
    int64_t *level_tests;          /* [M + 2] tests made by the nodes of each level */
    uint64_t *intents;             /* n_concepts x wm, lexicographic over attributes 0..M-1 */
    uint64_t *extents;             /* n_concepts x wn in the same order, or NULL */
    int64_t wn, wm;                /* words per extent / per intent */
    double seconds_enum;           /* enumeration wall time */
    double seconds_sort;           /* final sort wall time */
} oracle_result;

/* Enumerate all concepts of the context whose row g (attributes of object g)
 * starts at rows + g * row_stride.  max_tests < 0 means no limit; otherwise the
 * search stops after that many closure tests and sets truncated.  Returns 0 on
 * success, -1 on bad arguments, -2 when memory runs out. */
int oracle_cbo(const uint64_t *rows, int64_t n_objects, int64_t n_attrs, int64_t row_stride,
               int keep_extents, int64_t max_tests, oracle_result *out);

void oracle_free(oracle_result *r);

/* Counters and intent digest of the same search without storing concepts
 * (cbo_digest.c): digest = sum over concepts of the SplitMix64 chain of the
 * intent words, mod 2^64. */
typedef struct {
    int64_t n_concepts;
    int64_t tests;
    int64_t pairs;
    int64_t sum_c;
    int32_t n_levels;
    int32_t threads;               /* worker threads that ran */
    int64_t *level_concepts;       /* [M + 2] */
    int64_t *level_tests;          /* [M + 2] */
    uint64_t digest;
    double seconds;                /* search wall time */
} oracle_digest;

/* Returns 0, -1 on bad arguments, -2 when memory runs out. */
int oracle_cbo_digest(const uint64_t *rows, int64_t n_objects, int64_t n_attrs, int64_t row_stride, int threads,
                      oracle_digest *out);

void oracle_digest_free(oracle_digest *d);

#endif
