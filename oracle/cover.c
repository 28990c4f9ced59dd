/*
 * Lattice cover edges of a concept list: the CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY, like cbo.c: used by the tests, never by the GPU
 * library, sharing no code with it.
 *
 * The concepts of a context, ordered by extent inclusion, form the concept
 * lattice; (A2, B2) covers (A1, B1) when A1 is a proper subset of A2 and no
 * concept lies strictly between (page "hnwysp.cn/news/97538", section 4.4
 * rebuilds these edges after the enumeration, by extent inclusion, and warns
 * that the generation tree's parent edges are not cover edges; page
 * "hotelren.com/news/5603750", section 3.4 rebuilds parent links by searching
 * the sorted concept array).
 *
 * For a concept (A, B), every concept below it has an intent D that strictly
 * contains B; the smallest such D containing a given m outside B is the
 * closure (B + {m})'' = ((A AND col[m]))'.  Every lower cover is such a
 * closure (take any m of D outside B), and a closure is a lower cover exactly
 * when no other of these closures lies strictly inside it.  So per concept:
 * compute D_m for every m outside B, keep the distinct ones that are minimal
 * under inclusion among them, and find each one's position in the sorted
 * concept list by binary search.  (Lindig, "Fast concept analysis", 2000,
 * computes the upper neighbours of a concept the same way from the other
 * side.)
 *
 * Positions are indices into the given intent list, which is in the output
 * order of cbo.c: lexicographic over the attributes 0..M-1, the intent holding
 * the smallest attribute where two differ coming later.  Edges of concept i
 * are its lower covers, in ascending position.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle_cbo.h"

typedef struct {
    int64_t n, m, wn, wm;
    uint64_t *rows, *cols;
    uint64_t tail_n, tail_m;
} lattice_ctx;

static int in_set(const uint64_t *s, int64_t e)
{
    return (int)((s[e >> 6] >> (e & 63)) & 1u);
}

/* -1 if x comes before y in the output order, 1 if after, 0 if equal. */
static int order_cmp(const uint64_t *x, const uint64_t *y, int64_t wm)
{
    for (int64_t w = 0; w < wm; ++w) {
        uint64_t diff = x[w] ^ y[w];
        if (diff) {
            int e = __builtin_ctzll(diff);
            return ((x[w] >> e) & 1u) ? 1 : -1;
        }
    }
    return 0;
}

/* x strictly inside y */
static int proper_subset(const uint64_t *x, const uint64_t *y, int64_t wm)
{
    int equal = 1;
    for (int64_t w = 0; w < wm; ++w) {
        if (x[w] & ~y[w])
            return 0;
        if (x[w] != y[w])
            equal = 0;
    }
    return !equal;
}

static int64_t find(const uint64_t *intents, int64_t k, int64_t wm, const uint64_t *d)
{
    int64_t lo = 0, hi = k;
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        int c = order_cmp(intents + mid * wm, d, wm);
        if (c == 0)
            return mid;
        if (c < 0)
            lo = mid + 1;
        else
            hi = mid;
    }
    return -1;
}

static int cmp_i64(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

int oracle_cover_edges(const uint64_t *rows, int64_t n_objects, int64_t n_attrs, int64_t row_stride,
                       const uint64_t *intents, int64_t k, int64_t *offsets, int64_t **targets_out,
                       int64_t *n_edges_out)
{
    if (!rows || !intents || !offsets || !targets_out || !n_edges_out || n_objects < 1 || n_attrs < 1 || k < 1 ||
        row_stride < (n_attrs + 63) / 64)
        return -1;
    lattice_ctx x;
    x.n = n_objects;
    x.m = n_attrs;
    x.wn = (n_objects + 63) / 64;
    x.wm = (n_attrs + 63) / 64;
    x.tail_n = (n_objects & 63) ? (((uint64_t)1 << (n_objects & 63)) - 1u) : ~(uint64_t)0;
    x.tail_m = (n_attrs & 63) ? (((uint64_t)1 << (n_attrs & 63)) - 1u) : ~(uint64_t)0;
    x.rows = calloc((size_t)x.n * x.wm, sizeof(uint64_t));
    x.cols = calloc((size_t)x.m * x.wn, sizeof(uint64_t));
    uint64_t *a = malloc((size_t)x.wn * sizeof(uint64_t));
    uint64_t *e = malloc((size_t)x.wn * sizeof(uint64_t));
    uint64_t *cand = malloc((size_t)x.m * x.wm * sizeof(uint64_t)); /* the closures D_m of one concept */
    int64_t *pos = malloc((size_t)x.m * sizeof(int64_t));
    int64_t cap = 1024, ne = 0;
    int64_t *tg = malloc((size_t)cap * sizeof(int64_t));
    int rc = -2;
    if (!x.rows || !x.cols || !a || !e || !cand || !pos || !tg)
        goto done;
    for (int64_t g = 0; g < x.n; ++g) {
        for (int64_t w = 0; w < x.wm; ++w)
            x.rows[g * x.wm + w] = rows[g * row_stride + w];
        x.rows[g * x.wm + x.wm - 1] &= x.tail_m;
    }
    for (int64_t g = 0; g < x.n; ++g)
        for (int64_t j = 0; j < x.m; ++j)
            if (in_set(x.rows + g * x.wm, j))
                x.cols[j * x.wn + (g >> 6)] |= (uint64_t)1 << (g & 63);

    for (int64_t i = 0; i < k; ++i) {
        const uint64_t *b = intents + i * x.wm;
        offsets[i] = ne;
        /* A = B': the objects having every attribute of B */
        for (int64_t w = 0; w < x.wn; ++w)
            a[w] = ~(uint64_t)0;
        a[x.wn - 1] = x.tail_n;
        for (int64_t j = 0; j < x.m; ++j)
            if (in_set(b, j))
                for (int64_t w = 0; w < x.wn; ++w)
                    a[w] &= x.cols[j * x.wn + w];
        /* the closures D_m = (A AND col[m])' for m outside B, distinct */
        int64_t nc = 0;
        for (int64_t j = 0; j < x.m; ++j) {
            if (in_set(b, j))
                continue;
            uint64_t *d = cand + nc * x.wm;
            for (int64_t w = 0; w < x.wm; ++w)
                d[w] = ~(uint64_t)0;
            d[x.wm - 1] = x.tail_m;
            for (int64_t w = 0; w < x.wn; ++w) {
                e[w] = a[w] & x.cols[j * x.wn + w];
                uint64_t bits = e[w];
                while (bits) {
                    int64_t g = w * 64 + __builtin_ctzll(bits);
                    bits &= bits - 1u;
                    for (int64_t v = 0; v < x.wm; ++v)
                        d[v] &= x.rows[g * x.wm + v];
                }
            }
            int dup = 0;
            for (int64_t q = 0; q < nc && !dup; ++q)
                dup = memcmp(cand + q * x.wm, d, (size_t)x.wm * sizeof(uint64_t)) == 0;
            if (!dup)
                ++nc;
        }
        /* the minimal ones are the lower covers */
        int64_t np = 0;
        for (int64_t q = 0; q < nc; ++q) {
            int minimal = 1;
            for (int64_t r = 0; r < nc && minimal; ++r)
                if (r != q && proper_subset(cand + r * x.wm, cand + q * x.wm, x.wm))
                    minimal = 0;
            if (!minimal)
                continue;
            int64_t p = find(intents, k, x.wm, cand + q * x.wm);
            if (p < 0) {
                rc = -3; /* a closure missing from the list: not a complete concept list */
                goto done;
            }
            pos[np++] = p;
        }
        qsort(pos, (size_t)np, sizeof(int64_t), cmp_i64);
        if (ne + np > cap) {
            while (ne + np > cap)
                cap *= 2;
            int64_t *t2 = realloc(tg, (size_t)cap * sizeof(int64_t));
            if (!t2)
                goto done;
            tg = t2;
        }
        memcpy(tg + ne, pos, (size_t)np * sizeof(int64_t));
        ne += np;
    }
    offsets[k] = ne;
    *targets_out = tg;
    *n_edges_out = ne;
    tg = NULL;
    rc = 0;

done:
    free(x.rows);
    free(x.cols);
    free(a);
    free(e);
    free(cand);
    free(pos);
    free(tg);
    return rc;
}

void oracle_cover_free(int64_t *targets)
{
    free(targets);
}
