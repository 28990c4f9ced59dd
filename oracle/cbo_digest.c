/*
 * Close-by-One without a concept store: the CPU oracle for contexts whose
 * concepts do not fit in host memory.
 *
 * TEST INFRASTRUCTURE ONLY.  Like cbo.c this is reference code for the test
 * suite and never part of the GPU library; the two share no code.
 *
 * The search is the one of cbo.c (page "hnwysp.cn/news/97538", sections 2.1
 * and 2.3; page "hotelren.com/news/5603750", section 1.2): from the root
 * (G, G'), cursor -1, every node (A, B, y) tries each attribute j > y; j in B
 * is skipped (saturation), otherwise C = the objects of A having j, D = C' (the
 * AND of their rows, all of M when C is empty), and (C, D, j) is a child iff D
 * and B agree on attributes 0..j-1 (page 1, section 4.3).  Only the
 * representation differs: an extent is the ascending list of its objects
 * rather than a bitmap, which is what makes contexts with 10^9 concepts
 * tractable (page 1, section 4.2 walks the set bits of the extent for the same
 * reason).
 *
 * Nothing is stored.  Per concept the search adds to the counters of cbo.c
 * (tests, item pairs, sum of |C|, concepts and tests per level) and to an
 * order-independent digest of the intents:
 *     digest = sum over concepts of h(B) mod 2^64,
 *     h(B)   = f(... f(f(0 ^ w_0) ^ w_1) ... ^ w_{W-1}),
 * with w_k the 64-bit words of B (bit layout of cbo.c) and f the SplitMix64
 * output function (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014; constants as in Vigna's public splitmix64.c).
 *
 * The subtrees below the root's children are independent (canonicity is a
 * property of a node and its parent only, page 1 section 2.2), so they are
 * handed out to worker threads one at a time; counters are summed at the end.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include "oracle_cbo.h"

static uint64_t splitmix64_mix(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static uint64_t intent_hash(const uint64_t *b, int64_t wm)
{
    uint64_t h = 0;
    for (int64_t k = 0; k < wm; ++k)
        h = splitmix64_mix(h ^ b[k]);
    return h;
}

typedef struct {
    int64_t n, m, wm;
    const uint64_t *rows; /* n x wm */
    uint64_t tail_m;
} context;

typedef struct {
    int64_t concepts, tests, pairs, sum_c;
    int64_t *level_concepts, *level_tests; /* [m + 2] */
    int32_t max_depth;
    uint64_t digest;
    int oom;
} counters;

static int has_attr(const context *x, int64_t g, int64_t j)
{
    return (int)((x->rows[g * x->wm + (j >> 6)] >> (j & 63)) & 1u);
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

static void count_concept(const context *x, counters *c, const uint64_t *b, int32_t depth)
{
    c->concepts += 1;
    c->level_concepts[depth] += 1;
    if (depth > c->max_depth)
        c->max_depth = depth;
    c->digest += intent_hash(b, x->wm);
}

/* The children of node (A, B, y): C as an object list, D = C'.  With `only_j`
 * >= 0 just that attribute is tried (the root's children are split this way
 * between threads); `count_node` says whether this call also counts the
 * node's own tests and pairs (every attribute of the node is tried by
 * exactly one call). */
static void expand(const context *x, counters *c, const int32_t *a, int64_t na, const uint64_t *b, int64_t y,
                   int32_t depth, int64_t only_j)
{
    int64_t j_lo = y + 1, j_hi = x->m;
    if (only_j >= 0) {
        j_lo = only_j;
        j_hi = only_j + 1;
    }
    int32_t *cl = NULL;
    uint64_t *d = malloc((size_t)x->wm * sizeof(uint64_t));
    if (na > 0)
        cl = malloc((size_t)na * sizeof(int32_t));
    if (!d || (na > 0 && !cl)) {
        c->oom = 1;
        free(d);
        free(cl);
        return;
    }
    for (int64_t j = j_lo; j < j_hi && !c->oom; ++j) {
        c->pairs += 1;
        if ((b[j >> 6] >> (j & 63)) & 1u)
            continue; /* saturated: A is already inside col[j] */
        c->tests += 1;
        c->level_tests[depth] += 1;
        int64_t nc = 0;
        for (int64_t i = 0; i < na; ++i)
            if (has_attr(x, a[i], j))
                cl[nc++] = a[i];
        for (int64_t w = 0; w < x->wm; ++w)
            d[w] = ~(uint64_t)0;
        d[x->wm - 1] = x->tail_m;
        for (int64_t i = 0; i < nc; ++i)
            for (int64_t w = 0; w < x->wm; ++w)
                d[w] &= x->rows[(int64_t)cl[i] * x->wm + w];
        if (!same_prefix(d, b, j))
            continue;
        c->sum_c += nc;
        count_concept(x, c, d, depth + 1);
        expand(x, c, cl, nc, d, j, depth + 1, -1);
    }
    free(d);
    free(cl);
}

typedef struct {
    const context *x;
    const int32_t *a0;
    int64_t n0;
    const uint64_t *b0;
    int64_t next_j; /* next root attribute to hand out */
    pthread_mutex_t lock;
    counters part;  /* summed results of finished workers */
    int oom;
} pool;

static int counters_init(counters *c, int64_t m)
{
    memset(c, 0, sizeof(*c));
    c->level_concepts = calloc((size_t)m + 2, sizeof(int64_t));
    c->level_tests = calloc((size_t)m + 2, sizeof(int64_t));
    return c->level_concepts && c->level_tests;
}

static void counters_free(counters *c)
{
    free(c->level_concepts);
    free(c->level_tests);
}

static void counters_add(counters *to, const counters *from, int64_t m)
{
    to->concepts += from->concepts;
    to->tests += from->tests;
    to->pairs += from->pairs;
    to->sum_c += from->sum_c;
    to->digest += from->digest;
    to->oom |= from->oom;
    if (from->max_depth > to->max_depth)
        to->max_depth = from->max_depth;
    for (int64_t l = 0; l < m + 2; ++l) {
        to->level_concepts[l] += from->level_concepts[l];
        to->level_tests[l] += from->level_tests[l];
    }
}

static void *worker(void *arg)
{
    pool *p = arg;
    counters c;
    if (!counters_init(&c, p->x->m)) {
        pthread_mutex_lock(&p->lock);
        p->oom = 1;
        pthread_mutex_unlock(&p->lock);
        counters_free(&c);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&p->lock);
        int64_t j = p->next_j++;
        pthread_mutex_unlock(&p->lock);
        if (j >= p->x->m)
            break;
        expand(p->x, &c, p->a0, p->n0, p->b0, -1, 0, j);
    }
    pthread_mutex_lock(&p->lock);
    counters_add(&p->part, &c, p->x->m);
    pthread_mutex_unlock(&p->lock);
    counters_free(&c);
    return NULL;
}

int oracle_cbo_digest(const uint64_t *rows, int64_t n_objects, int64_t n_attrs, int64_t row_stride, int threads,
                      oracle_digest *out)
{
    if (!rows || !out || n_objects < 1 || n_objects > INT32_MAX || n_attrs < 1 ||
        row_stride < (n_attrs + 63) / 64 || threads < 1)
        return -1;
    memset(out, 0, sizeof(*out));
    context x;
    x.n = n_objects;
    x.m = n_attrs;
    x.wm = (n_attrs + 63) / 64;
    x.tail_m = (n_attrs & 63) ? (((uint64_t)1 << (n_attrs & 63)) - 1u) : ~(uint64_t)0;
    uint64_t *r = malloc((size_t)x.n * x.wm * sizeof(uint64_t));
    int32_t *a0 = malloc((size_t)x.n * sizeof(int32_t));
    uint64_t *b0 = malloc((size_t)x.wm * sizeof(uint64_t));
    pool p;
    memset(&p, 0, sizeof(p));
    int rc = -2;
    if (!r || !a0 || !b0 || !counters_init(&p.part, x.m))
        goto done;
    for (int64_t g = 0; g < x.n; ++g) {
        for (int64_t w = 0; w < x.wm; ++w)
            r[g * x.wm + w] = rows[g * row_stride + w];
        r[g * x.wm + x.wm - 1] &= x.tail_m; /* bits past M are dropped */
    }
    x.rows = r;

    struct timespec t0, t1;
    clock_gettime(CLOCK_MONOTONIC, &t0);
    /* Root: all objects and the attributes they share (page 4 section 1.2). */
    for (int64_t g = 0; g < x.n; ++g)
        a0[g] = (int32_t)g;
    for (int64_t w = 0; w < x.wm; ++w)
        b0[w] = ~(uint64_t)0;
    b0[x.wm - 1] = x.tail_m;
    for (int64_t g = 0; g < x.n; ++g)
        for (int64_t w = 0; w < x.wm; ++w)
            b0[w] &= r[g * x.wm + w];
    count_concept(&x, &p.part, b0, 0);

    p.x = &x;
    p.a0 = a0;
    p.n0 = x.n;
    p.b0 = b0;
    p.next_j = 0;
    pthread_mutex_init(&p.lock, NULL);
    pthread_t *th = malloc((size_t)threads * sizeof(pthread_t));
    int started = 0;
    if (th)
        for (; started < threads; ++started)
            if (pthread_create(&th[started], NULL, worker, &p) != 0)
                break;
    if (started == 0) {
        worker(&p); /* no thread could be started: search on this one */
    }
    for (int i = 0; i < started; ++i)
        pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&p.lock);
    clock_gettime(CLOCK_MONOTONIC, &t1);
    if (p.oom || p.part.oom)
        goto done;

    out->n_concepts = p.part.concepts;
    out->tests = p.part.tests;
    out->pairs = p.part.pairs;
    out->sum_c = p.part.sum_c;
    out->n_levels = p.part.max_depth + 1;
    out->level_concepts = p.part.level_concepts;
    out->level_tests = p.part.level_tests;
    p.part.level_concepts = NULL;
    p.part.level_tests = NULL;
    out->digest = p.part.digest;
    out->threads = started ? started : 1;
    out->seconds = (double)(t1.tv_sec - t0.tv_sec) + 1e-9 * (double)(t1.tv_nsec - t0.tv_nsec);
    rc = 0;

done:
    counters_free(&p.part);
    free(r);
    free(a0);
    free(b0);
    return rc;
}

void oracle_digest_free(oracle_digest *d)
{
    if (!d)
        return;
    free(d->level_concepts);
    free(d->level_tests);
    d->level_concepts = NULL;
    d->level_tests = NULL;
}
