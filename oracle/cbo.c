/*
 * Serial Close-by-One concept enumeration: the CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, single-threaded
 * reference that the GPU library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark load it; the GPU
 * library never links, includes or calls it, and it shares no code with it.
 *
 * What it computes (page "hnwysp.cn/news/97538", sections 1.1-1.2; page
 * "hotelren.com/news/5603750", section 1.1): for a formal context of N objects
 * and M attributes, every formal concept (A, B) with A' = B and B' = A, where
 * X' of an object set is the AND of its rows and Y' of an attribute set is the
 * AND of its columns.  The empty object set derives to all of M.
 *
 * How (page 1, sections 2.1 and 2.3; page 4, section 1.2): depth-first CbO
 * from the root (G, G'), cursor -1.  For a node (A, B, y) and every attribute
 * j > y in ascending order:
 *   - j in B: attribute saturation; A is inside col[j] already, no child.
 *   - otherwise one closure test: C = A AND col[j]; D = C' (AND of the rows of
 *     the objects in C); the child (C, D, j) is kept iff D and B agree on the
 *     attributes 0..j-1 (bit j itself excluded, page 1 section 4.3), and the
 *     search recurses into it.
 * Afterwards the concepts are sorted by intent in lexicographic order of the
 * intent read as a bit string over the attributes 0, 1, ..., M-1: of two
 * intents, the one holding the smallest attribute in which they differ comes
 * later (page 1 section 6.2 asks for a lexicographic intent key; reading the
 * intent as its characteristic string in attribute index order is the reading
 * taken here).
 *
 * Bit layout: element e of a set is bit (e & 63) of 64-bit word (e >> 6);
 * bits past N or M in the last word are always zero.
 *
 * Besides the concepts it counts what the byte model of the GPU path needs:
 * closure tests, item pairs, concepts and tests per depth, the sum over tests
 * of the non-zero words of the parent extent, and the sum over kept children
 * of |C|; and the same split by a threshold T on the parent's extent size:
 * the objects of the parents with |A| <= T, the number of parents with
 * |A| > T, the sum over their tests of the non-zero words of A, and the
 * objects of their children.
 *
 * On request every concept's extent is also reduced to a 64-bit hash,
 *     g(A) = sum over words k of f(a_k XOR f(k)) mod 2^64,
 * with a_k the 64-bit words of the extent bitmap and f the SplitMix64 output
 * function (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014; constants as in Vigna's public splitmix64.c),
 * and the hashes follow the concepts through the final sort.  They let a test
 * compare extents of contexts whose K x N/8 bytes do not fit in memory.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include "oracle_cbo.h"

typedef struct {
    int64_t n, m, wn, wm;
    uint64_t *rows;    /* n x wm, row g = attributes of object g */
    uint64_t *cols;    /* m x wn, col j = objects having attribute j */
    uint64_t tail_n;   /* valid bits of the last extent word */
    uint64_t tail_m;   /* valid bits of the last intent word */
    uint64_t *stack;   /* per-depth storage for C and D */
    /* concept store */
    int64_t count, cap;
    uint64_t *intents, *extents;
    int keep_extents, hash_extents;
    uint64_t *ehash;   /* extent hash of every stored concept (hash_extents) */
    uint64_t *wkey;    /* f(k) for every extent word k */
    /* counters */
    int64_t tests, pairs, sum_nzw, sum_c, violations;
    int64_t rowlocal_max, sum_rl_objs, col_parents, col_nzw, col_child_objs;
    int64_t *level_concepts, *level_tests;
    int32_t max_depth;
    int64_t max_tests;
    int truncated, oom;
} cbo_state;

static double now_seconds(void)
{
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

static uint64_t splitmix64_f(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* g(A) of an extent bitmap (see the file comment). */
static uint64_t extent_hash(const cbo_state *s, const uint64_t *a)
{
    uint64_t h = 0;
    for (int64_t k = 0; k < s->wn; ++k)
        h += splitmix64_f(a[k] ^ s->wkey[k]);
    return h;
}

static int has_bit(const uint64_t *set, int64_t e)
{
    return (int)((set[e >> 6] >> (e & 63)) & 1u);
}

static int64_t popcount_words(const uint64_t *set, int64_t nw)
{
    int64_t c = 0;
    for (int64_t w = 0; w < nw; ++w)
        c += __builtin_popcountll(set[w]);
    return c;
}

static int64_t nonzero_words(const uint64_t *set, int64_t nw)
{
    int64_t c = 0;
    for (int64_t w = 0; w < nw; ++w)
        c += set[w] != 0;
    return c;
}

/* X' for an object set X: start from all attributes and AND the row of every
 * object of X, found by scanning the set bits of X word by word (page 1,
 * section 4.2: the extent's set bits are walked, zero words skipped). */
static void derive_objects(const cbo_state *s, const uint64_t *x, uint64_t *out)
{
    for (int64_t w = 0; w < s->wm; ++w)
        out[w] = ~(uint64_t)0;
    out[s->wm - 1] = s->tail_m;
    for (int64_t xw = 0; xw < s->wn; ++xw) {
        uint64_t bits = x[xw];
        while (bits) {
            int64_t g = xw * 64 + __builtin_ctzll(bits);
            bits &= bits - 1u;
            const uint64_t *row = s->rows + g * s->wm;
            for (int64_t w = 0; w < s->wm; ++w)
                out[w] &= row[w];
        }
    }
}

/* D and B agree on attributes 0..j-1 (bit j itself is not compared). */
static int same_prefix(const uint64_t *d, const uint64_t *b, int64_t j)
{
    int64_t word = j >> 6, bit = j & 63;
    for (int64_t w = 0; w < word; ++w)
        if (d[w] != b[w])
            return 0;
    uint64_t mask = bit ? (((uint64_t)1 << bit) - 1u) : 0u;
    return (d[word] & mask) == (b[word] & mask);
}

static int store(cbo_state *s, const uint64_t *a, const uint64_t *b, int32_t depth)
{
    if (s->count == s->cap) {
        int64_t ncap = s->cap ? 2 * s->cap : 1024;
        uint64_t *ni = realloc(s->intents, (size_t)ncap * s->wm * sizeof(uint64_t));
        if (!ni) { s->oom = 1; return 0; }
        s->intents = ni;
        if (s->hash_extents) {
            uint64_t *nh = realloc(s->ehash, (size_t)ncap * sizeof(uint64_t));
            if (!nh) { s->oom = 1; return 0; }
            s->ehash = nh;
        }
        if (s->keep_extents) {
            uint64_t *ne = realloc(s->extents, (size_t)ncap * s->wn * sizeof(uint64_t));
            if (!ne) { s->oom = 1; return 0; }
            s->extents = ne;
        }
        s->cap = ncap;
    }
    memcpy(s->intents + s->count * s->wm, b, (size_t)s->wm * sizeof(uint64_t));
    if (s->keep_extents)
        memcpy(s->extents + s->count * s->wn, a, (size_t)s->wn * sizeof(uint64_t));
    if (s->hash_extents)
        s->ehash[s->count] = extent_hash(s, a);
    s->count += 1;
    s->level_concepts[depth] += 1;
    if (depth > s->max_depth)
        s->max_depth = depth;
    return 1;
}

/* One CbO node (A, B) with cursor y at the given depth.  B may be widened by
 * the saturation fold, so it is writable. */
static void generate(cbo_state *s, const uint64_t *a, uint64_t *b, int64_t y, int32_t depth)
{
    uint64_t *c = s->stack + (size_t)(depth + 1) * (s->wn + s->wm);
    uint64_t *d = c + s->wn;
    /* the byte-model class of this node as a parent */
    const int64_t size_a = popcount_words(a, s->wn);
    const int col_class = size_a > s->rowlocal_max;
    const int64_t nzw_a = nonzero_words(a, s->wn);
    if (col_class)
        s->col_parents += 1;
    else
        s->sum_rl_objs += size_a;
    for (int64_t j = y + 1; j < s->m; ++j) {
        if (s->truncated || s->oom)
            return;
        s->pairs += 1;
        if (has_bit(b, j))
            continue; /* saturated: A is already inside col[j] */
        if (s->max_tests >= 0 && s->tests >= s->max_tests) {
            s->truncated = 1;
            return;
        }
        s->tests += 1;
        s->level_tests[depth] += 1;
        s->sum_nzw += nzw_a;
        if (col_class)
            s->col_nzw += nzw_a;
        const uint64_t *col = s->cols + j * s->wn;
        int shrinks = 0;
        for (int64_t w = 0; w < s->wn; ++w) {
            c[w] = a[w] & col[w];
            shrinks |= c[w] != a[w];
        }
        if (!shrinks) {
            /* A inside col[j] although j is not in B: fold j into B.  With B
             * closed this cannot happen; it is counted so tests can insist. */
            s->violations += 1;
            b[j >> 6] |= (uint64_t)1 << (j & 63);
            continue;
        }
        derive_objects(s, c, d);
        if (!same_prefix(d, b, j))
            continue;
        const int64_t size_c = popcount_words(c, s->wn);
        s->sum_c += size_c;
        if (col_class)
            s->col_child_objs += size_c;
        if (!store(s, c, d, depth + 1))
            return;
        generate(s, c, d, j, depth + 1);
    }
}

static const cbo_state *g_sort_state;

static int cmp_intent(const void *pa, const void *pb)
{
    int64_t ia = *(const int64_t *)pa, ib = *(const int64_t *)pb;
    const uint64_t *x = g_sort_state->intents + ia * g_sort_state->wm;
    const uint64_t *y = g_sort_state->intents + ib * g_sort_state->wm;
    /* attributes in index order: word by word, bit 0 of a word first */
    for (int64_t w = 0; w < g_sort_state->wm; ++w) {
        uint64_t diff = x[w] ^ y[w];
        if (diff) {
            int e = __builtin_ctzll(diff);  /* smallest differing attribute in this word */
            return ((x[w] >> e) & 1u) ? 1 : -1;
        }
    }
    return 0;
}

static int sort_concepts(cbo_state *s)
{
    int64_t k = s->count;
    if (k < 2)
        return 1;
    int64_t *perm = malloc((size_t)k * sizeof(int64_t));
    uint64_t *ni = malloc((size_t)k * s->wm * sizeof(uint64_t));
    uint64_t *ne = s->keep_extents ? malloc((size_t)k * s->wn * sizeof(uint64_t)) : NULL;
    uint64_t *nh = s->hash_extents ? malloc((size_t)k * sizeof(uint64_t)) : NULL;
    if (!perm || !ni || (s->keep_extents && !ne) || (s->hash_extents && !nh)) {
        free(perm); free(ni); free(ne); free(nh);
        return 0;
    }
    for (int64_t i = 0; i < k; ++i)
        perm[i] = i;
    g_sort_state = s;
    qsort(perm, (size_t)k, sizeof(int64_t), cmp_intent);
    g_sort_state = NULL;
    for (int64_t i = 0; i < k; ++i) {
        memcpy(ni + i * s->wm, s->intents + perm[i] * s->wm, (size_t)s->wm * sizeof(uint64_t));
        if (ne)
            memcpy(ne + i * s->wn, s->extents + perm[i] * s->wn, (size_t)s->wn * sizeof(uint64_t));
        if (nh)
            nh[i] = s->ehash[perm[i]];
    }
    free(perm);
    free(s->intents);
    s->intents = ni;
    if (ne) {
        free(s->extents);
        s->extents = ne;
    }
    if (nh) {
        free(s->ehash);
        s->ehash = nh;
    }
    return 1;
}

int oracle_cbo(const uint64_t *rows, int64_t n_objects, int64_t n_attrs, int64_t row_stride,
               int flags, int64_t max_tests, int64_t rowlocal_max, oracle_result *out)
{
    if (!rows || !out || n_objects < 1 || n_attrs < 1 || row_stride < (n_attrs + 63) / 64)
        return -1;
    memset(out, 0, sizeof(*out));
    cbo_state s;
    memset(&s, 0, sizeof(s));
    s.n = n_objects;
    s.m = n_attrs;
    s.wn = (n_objects + 63) / 64;
    s.wm = (n_attrs + 63) / 64;
    s.tail_n = (n_objects & 63) ? (((uint64_t)1 << (n_objects & 63)) - 1u) : ~(uint64_t)0;
    s.tail_m = (n_attrs & 63) ? (((uint64_t)1 << (n_attrs & 63)) - 1u) : ~(uint64_t)0;
    s.keep_extents = (flags & ORACLE_KEEP_EXTENTS) != 0;
    s.hash_extents = (flags & ORACLE_HASH_EXTENTS) != 0;
    s.max_tests = max_tests;
    s.rowlocal_max = rowlocal_max;

    s.rows = calloc((size_t)s.n * s.wm, sizeof(uint64_t));
    s.cols = calloc((size_t)s.m * s.wn, sizeof(uint64_t));
    s.stack = calloc((size_t)(s.m + 2) * (s.wn + s.wm), sizeof(uint64_t));
    s.level_concepts = calloc((size_t)s.m + 2, sizeof(int64_t));
    s.level_tests = calloc((size_t)s.m + 2, sizeof(int64_t));
    s.wkey = calloc((size_t)s.wn, sizeof(uint64_t));
    uint64_t *a0 = calloc((size_t)s.wn, sizeof(uint64_t));
    uint64_t *b0 = calloc((size_t)s.wm, sizeof(uint64_t));
    int rc = -2;
    if (!s.rows || !s.cols || !s.stack || !s.level_concepts || !s.level_tests || !s.wkey || !a0 || !b0)
        goto fail;
    for (int64_t k = 0; k < s.wn; ++k)
        s.wkey[k] = splitmix64_f((uint64_t)k);

    /* The context in both layouts; bits past M are dropped. */
    for (int64_t g = 0; g < s.n; ++g) {
        for (int64_t w = 0; w < s.wm; ++w)
            s.rows[g * s.wm + w] = rows[g * row_stride + w];
        s.rows[g * s.wm + s.wm - 1] &= s.tail_m;
    }
    for (int64_t g = 0; g < s.n; ++g)
        for (int64_t j = 0; j < s.m; ++j)
            if (has_bit(s.rows + g * s.wm, j))
                s.cols[j * s.wn + (g >> 6)] |= (uint64_t)1 << (g & 63);

    double t0 = now_seconds();
    /* Root: all objects and the attributes they share (page 4 section 1.2). */
    for (int64_t w = 0; w < s.wn; ++w)
        a0[w] = ~(uint64_t)0;
    a0[s.wn - 1] = s.tail_n;
    derive_objects(&s, a0, b0);
    if (!store(&s, a0, b0, 0))
        goto fail;
    generate(&s, a0, b0, -1, 0);
    if (s.oom)
        goto fail;
    double t1 = now_seconds();
    if (!sort_concepts(&s))
        goto fail;
    double t2 = now_seconds();

    out->n_concepts = s.count;
    out->tests = s.tests;
    out->pairs = s.pairs;
    out->sum_nzw = s.sum_nzw;
    out->sum_c = s.sum_c;
    out->saturation_violations = s.violations;
    out->n_levels = s.max_depth + 1;
    out->truncated = s.truncated;
    out->level_concepts = s.level_concepts;
    out->level_tests = s.level_tests;
    out->intents = s.intents;
    out->extents = s.extents;
    out->extent_hashes = s.ehash;
    out->sum_rl_objs = s.sum_rl_objs;
    out->col_parents = s.col_parents;
    out->col_nzw = s.col_nzw;
    out->col_child_objs = s.col_child_objs;
    out->wn = s.wn;
    out->wm = s.wm;
    out->seconds_enum = t1 - t0;
    out->seconds_sort = t2 - t1;
    free(s.rows);
    free(s.cols);
    free(s.stack);
    free(s.wkey);
    free(a0);
    free(b0);
    return 0;

fail:
    free(s.rows);
    free(s.cols);
    free(s.stack);
    free(s.level_concepts);
    free(s.level_tests);
    free(s.intents);
    free(s.extents);
    free(s.ehash);
    free(s.wkey);
    free(a0);
    free(b0);
    return rc;
}

void oracle_free(oracle_result *r)
{
    if (!r)
        return;
    free(r->level_concepts);
    free(r->level_tests);
    free(r->intents);
    free(r->extents);
    free(r->extent_hashes);
    memset(r, 0, sizeof(*r));
}
