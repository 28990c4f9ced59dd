/*
 * Close-by-One without a concept store: the CPU oracle for contexts whose
 * concepts do not fit in host memory.
 *
 * TEST INFRASTRUCTURE ONLY.  Like cbo.c this is reference code for the test
 * suite and never part of the GPU library; the two share no code.
 *
 * The search is the one of cbo.c (page "hnwysp.cn/news/97538", sections 2.1
 * and 2.3; page "hotelren.com/news/5603750", section 1.2): from the root
 * (G, G'), cursor -1, every node (A, B, y) tries each attribute j > y in
 * ascending order; j in B is skipped (saturation), otherwise C = the objects
 * of A having j, D = C' (the AND of their rows, all of M when C is empty), and
 * (C, D, j) is a child iff D and B agree on attributes 0..j-1 (page 1,
 * section 4.3).  Only the representation differs: an extent is the ascending
 * list of its objects rather than a bitmap, which is what makes contexts with
 * 10^9 concepts tractable (page 1, section 4.2 walks the set bits of the
 * extent for the same reason).
 *
 * Nothing is stored.  Per concept the search adds to the counters of cbo.c
 * (tests, item pairs, sum of |C|, concepts and tests per level) and hashes the
 * concept:
 *     h(B) = f(... f(f(0 ^ w_0) ^ w_1) ... ^ w_{W_M-1})   (intent words w_k)
 *     g(A) = sum over k < W_N of f(a_k ^ f(k)) mod 2^64  (extent bitmap words a_k)
 * with f the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014; constants as in
 * Vigna's public splitmix64.c).  g is computed from the list: the words that
 * hold no object contribute f(f(k)) each, so
 *     g(A) = Z + sum over the non-zero words k of (f(a_k ^ f(k)) - f(f(k))),
 * Z = sum over all k of f(f(k)).
 *
 * Digests (all mod 2^64):
 *     digest            = sum over concepts of h(B)          (order-free)
 *     intent_positional = sum over concepts of i * h(B_i)
 *     extent_positional = sum over concepts of i * g(A_i)
 * where i is the concept's position in the output order: intents in
 * lexicographic order over the attributes 0..M-1, the one holding the
 * smallest attribute where two differ coming later.  In that order the CbO
 * tree is listed in pre-order with the children of a node taken by
 * descending generating attribute (a child agrees with its parent below its
 * attribute and adds it; of two children the one made at the smaller
 * attribute holds it and the other does not, so it and its whole subtree come
 * later).  The search walks children by ascending attribute, as the pages do,
 * so positions are not known on the way down; instead every subtree returns
 * (size, sum of hashes, sum of local position x hash) with its root at local
 * position 0, and a node places its children's subtrees after itself in
 * descending attribute order: a child subtree starting at offset o adds
 * o x (its hash sum) to the node's position-weighted sum.
 *
 * The subtrees below the root's children are independent (canonicity is a
 * property of a node and its parent only, page 1 section 2.2), so they are
 * handed out to worker threads one at a time; their summaries are combined in
 * the output order at the end.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#include "oracle_cbo.h"

static uint64_t splitmix64_f(uint64_t z)
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
        h = splitmix64_f(h ^ b[k]);
    return h;
}

typedef struct {
    int64_t n, m, wm, wn;
    const uint64_t *rows; /* n x wm */
    uint64_t tail_m;
    uint64_t *wkey;       /* f(k) for every extent word k */
    uint64_t zero_sum;    /* Z: g of the empty extent */
} context;

/* g(A) of an ascending object list (see the file comment). */
static uint64_t extent_hash(const context *x, const int32_t *a, int64_t na)
{
    uint64_t h = x->zero_sum;
    int64_t i = 0;
    while (i < na) {
        const int64_t k = a[i] >> 6;
        uint64_t word = 0;
        for (; i < na && (a[i] >> 6) == k; ++i)
            word |= (uint64_t)1 << (a[i] & 63);
        h += splitmix64_f(word ^ x->wkey[k]) - splitmix64_f(x->wkey[k]);
    }
    return h;
}

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

/* Place the subtree `kid` after the `off` concepts already in `to`. */
static void append_subtree(oracle_subtree *to, const oracle_subtree *kid)
{
    const uint64_t off = (uint64_t)to->size;
    to->hi1 += kid->hi1 + off * kid->hi0;
    to->he1 += kid->he1 + off * kid->he0;
    to->hi0 += kid->hi0;
    to->he0 += kid->he0;
    to->size += kid->size;
}

typedef struct {
    int64_t j;
    oracle_subtree sub;
} child_summary;

static oracle_subtree subtree(const context *x, counters *c, const int32_t *a, int64_t na, const uint64_t *b,
                              int64_t y, int32_t depth);

/* The children of node (A, B) at `depth` made at the attributes j in [j_lo,
 * j_hi) (ascending), each with its subtree searched; their summaries go to
 * kids[] in ascending j.  The node's tests and item pairs for these j are
 * counted here.  Returns the number of children. */
static int64_t children(const context *x, counters *c, const int32_t *a, int64_t na, const uint64_t *b, int32_t depth,
                        int64_t j_lo, int64_t j_hi, child_summary *kids)
{
    int64_t nk = 0;
    int32_t *cl = NULL;
    uint64_t *d = malloc((size_t)x->wm * sizeof(uint64_t));
    if (na > 0)
        cl = malloc((size_t)na * sizeof(int32_t));
    if (!d || (na > 0 && !cl)) {
        c->oom = 1;
        free(d);
        free(cl);
        return 0;
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
        kids[nk].j = j;
        kids[nk].sub = subtree(x, c, cl, nc, d, j, depth + 1);
        ++nk;
    }
    free(d);
    free(cl);
    return nk;
}

/* Count the node (A, B) with cursor y at `depth` and search its subtree;
 * returns the subtree's summary with the node at local position 0. */
static oracle_subtree subtree(const context *x, counters *c, const int32_t *a, int64_t na, const uint64_t *b,
                              int64_t y, int32_t depth)
{
    const uint64_t hi = intent_hash(b, x->wm), he = extent_hash(x, a, na);
    c->concepts += 1;
    c->level_concepts[depth] += 1;
    if (depth > c->max_depth)
        c->max_depth = depth;
    c->digest += hi;
    oracle_subtree s = {1, hi, 0, he, 0};
    const int64_t span = x->m - (y + 1);
    if (span <= 0)
        return s;
    child_summary *kids = malloc((size_t)span * sizeof(child_summary));
    if (!kids) {
        c->oom = 1;
        return s;
    }
    const int64_t nk = children(x, c, a, na, b, depth, y + 1, x->m, kids);
    for (int64_t k = nk; k-- > 0;) /* descending attribute: the output order */
        append_subtree(&s, &kids[k].sub);
    free(kids);
    return s;
}

typedef struct {
    const context *x;
    const int32_t *a0;
    int64_t n0;
    const uint64_t *b0;
    int64_t next_j;          /* next root attribute to hand out */
    pthread_mutex_t lock;
    counters part;           /* summed results of finished workers */
    child_summary *slot;     /* [m]: the root's child made at j, if any */
    unsigned char *has_slot; /* [m] */
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
        child_summary kid;
        if (children(p->x, &c, p->a0, p->n0, p->b0, 0, j, j + 1, &kid) == 1) {
            p->slot[j] = kid; /* each j is handed to one worker only */
            p->has_slot[j] = 1;
        }
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
    x.wn = (n_objects + 63) / 64;
    x.tail_m = (n_attrs & 63) ? (((uint64_t)1 << (n_attrs & 63)) - 1u) : ~(uint64_t)0;
    uint64_t *r = malloc((size_t)x.n * x.wm * sizeof(uint64_t));
    int32_t *a0 = malloc((size_t)x.n * sizeof(int32_t));
    uint64_t *b0 = malloc((size_t)x.wm * sizeof(uint64_t));
    x.wkey = malloc((size_t)x.wn * sizeof(uint64_t));
    pool p;
    memset(&p, 0, sizeof(p));
    p.slot = malloc((size_t)x.m * sizeof(child_summary));
    p.has_slot = calloc((size_t)x.m, 1);
    int32_t *child_attr = NULL;
    oracle_subtree *child_sub = NULL;
    int rc = -2;
    if (!r || !a0 || !b0 || !x.wkey || !p.slot || !p.has_slot || !counters_init(&p.part, x.m))
        goto done;
    for (int64_t g = 0; g < x.n; ++g) {
        for (int64_t w = 0; w < x.wm; ++w)
            r[g * x.wm + w] = rows[g * row_stride + w];
        r[g * x.wm + x.wm - 1] &= x.tail_m; /* bits past M are dropped */
    }
    x.rows = r;
    x.zero_sum = 0;
    for (int64_t k = 0; k < x.wn; ++k) {
        x.wkey[k] = splitmix64_f((uint64_t)k);
        x.zero_sum += splitmix64_f(x.wkey[k]);
    }

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
    const uint64_t root_hi = intent_hash(b0, x.wm), root_he = extent_hash(&x, a0, x.n);
    p.part.concepts = 1;
    p.part.level_concepts[0] = 1;
    p.part.digest = root_hi;

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

    /* the root, then its children's subtrees by descending attribute */
    oracle_subtree whole = {1, root_hi, 0, root_he, 0};
    int32_t nroot = 0;
    for (int64_t j = 0; j < x.m; ++j)
        nroot += p.has_slot[j];
    child_attr = malloc((size_t)(nroot ? nroot : 1) * sizeof(int32_t));
    child_sub = malloc((size_t)(nroot ? nroot : 1) * sizeof(oracle_subtree));
    if (!child_attr || !child_sub)
        goto done;
    int32_t k = 0;
    for (int64_t j = x.m; j-- > 0;) {
        if (!p.has_slot[j])
            continue;
        child_attr[k] = (int32_t)j;
        child_sub[k] = p.slot[j].sub;
        append_subtree(&whole, &p.slot[j].sub);
        ++k;
    }

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
    out->subtree_size = whole.size;
    out->intent_digest = whole.hi0;
    out->intent_positional = whole.hi1;
    out->extent_digest = whole.he0;
    out->extent_positional = whole.he1;
    out->n_root_children = nroot;
    out->root_child_attr = child_attr;
    out->root_child = child_sub;
    child_attr = NULL;
    child_sub = NULL;
    out->threads = started ? started : 1;
    out->seconds = (double)(t1.tv_sec - t0.tv_sec) + 1e-9 * (double)(t1.tv_nsec - t0.tv_nsec);
    rc = 0;

done:
    counters_free(&p.part);
    free(child_attr);
    free(child_sub);
    free(p.slot);
    free(p.has_slot);
    free(x.wkey);
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
    free(d->root_child_attr);
    free(d->root_child);
    d->level_concepts = NULL;
    d->level_tests = NULL;
    d->root_child_attr = NULL;
    d->root_child = NULL;
}
