/*
 * Seeded synthetic-graph helpers: R-MAT edge generation and an edge-list to
 * symmetric, deduplicated, row-sorted int32 CSR builder.  Input preparation
 * only: no BFS arithmetic lives here.  Shared by the oracle tests and the HIP
 * tests/benchmark; it includes nothing from either side.
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  Its i-th output for seed s
 * is mix64(s + (i + 1) * 0x9E3779B97F4A7C15), so every edge can draw its own
 * slice of the stream independently of thread count.
 *
 * R-MAT: Chakrabarti, Zhan and Faloutsos, "R-MAT: A Recursive Model for Graph
 * Mining", SDM 2004 -- each edge picks one of four quadrants per bit level with
 * probabilities (a, b, c, d), without noise.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* i-th output (0-based) of SplitMix64 seeded with `seed`. */
static inline uint64_t sm64_at(uint64_t seed, uint64_t i)
{
    return mix64(seed + (i + 1) * GOLDEN);
}

/* Uniform integer in [0, bound) from a 64-bit draw (multiply-shift). */
static inline uint64_t bounded(uint64_t r, uint64_t bound)
{
    return (uint64_t)(((unsigned __int128)r * bound) >> 64);
}

/*
 * Fisher-Yates permutation of [0, n) driven by the SplitMix64 stream of
 * `seed` (draw number n-1-i for position i).
 */
void gen_permutation(int32_t n, uint64_t seed, int32_t *perm)
{
    for (int32_t i = 0; i < n; ++i) perm[i] = i;
    uint64_t k = 0;
    for (int32_t i = n - 1; i > 0; --i) {
        int32_t j = (int32_t)bounded(sm64_at(seed, k++), (uint64_t)i + 1);
        int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
}

/*
 * R-MAT edges: nedges pairs over 2^scale vertices.  Edge e uses draws
 * [e*W, e*W + W) of the seed's stream, W = ceil(scale/2); each 64-bit draw
 * gives two 32-bit uniforms, one per bit level, most significant level first.
 * perm (may be NULL) relabels both endpoints.
 */
void gen_rmat_edges(int32_t scale, int64_t nedges, double a, double b, double c,
                    uint64_t seed, const int32_t *perm, int32_t *src, int32_t *dst)
{
    const uint64_t ta = (uint64_t)(a * 4294967296.0);
    const uint64_t tab = (uint64_t)((a + b) * 4294967296.0);
    const uint64_t tabc = (uint64_t)((a + b + c) * 4294967296.0);
    const int32_t W = (scale + 1) / 2;
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < nedges; ++e) {
        uint32_t u = 0, v = 0;
        uint64_t base = (uint64_t)e * (uint64_t)W;
        for (int32_t j = 0; j < W; ++j) {
            uint64_t r64 = sm64_at(seed, base + (uint64_t)j);
            for (int32_t h = 0; h < 2 && 2 * j + h < scale; ++h) {
                /* level 2j+h: high half first; quadrants a=(0,0) b=(0,1) c=(1,0) d=(1,1) */
                uint64_t r = h ? (r64 & 0xffffffffULL) : (r64 >> 32);
                uint32_t ub = r >= tab;
                uint32_t vb = (r >= ta) & ((r < tab) | (r >= tabc));
                u = (u << 1) | ub;
                v = (v << 1) | vb;
            }
        }
        if (perm) { u = (uint32_t)perm[u]; v = (uint32_t)perm[v]; }
        src[e] = (int32_t)u;
        dst[e] = (int32_t)v;
    }
}

static void insertion_sort(int32_t *a, int64_t len)
{
    for (int64_t i = 1; i < len; ++i) {
        int32_t x = a[i];
        int64_t j = i - 1;
        while (j >= 0 && a[j] > x) { a[j + 1] = a[j]; --j; }
        a[j + 1] = x;
    }
}

/* In-place quicksort (median of three, insertion sort below 24 elements). */
static void sort_i32(int32_t *a, int64_t len)
{
    while (len > 24) {
        int32_t x = a[0], y = a[len / 2], z = a[len - 1];
        int32_t piv = x < y ? (y < z ? y : (x < z ? z : x)) : (x < z ? x : (y < z ? z : y));
        int64_t i = 0, j = len - 1;
        for (;;) {
            while (a[i] < piv) ++i;
            while (a[j] > piv) --j;
            if (i >= j) break;
            int32_t t = a[i]; a[i] = a[j]; a[j] = t;
            ++i; --j;
        }
        /* recurse into the smaller half, loop on the larger */
        int64_t left = j + 1;
        if (left < len - left) { sort_i32(a, left); a += left; len -= left; }
        else { sort_i32(a + left, len - left); len = left; }
    }
    insertion_sort(a, len);
}

typedef struct {
    int32_t n;
    int32_t *tmp;
    int64_t *start;
    int32_t *deg;
    const int32_t *row_ptr;
} csr_build_t;

/*
 * Builds the symmetric closure of an edge list as CSR: self-loops dropped,
 * both directions added, each row sorted ascending and deduplicated.
 * Two calls: csr_build fills row_ptr (n+1 entries) and *m_out and returns a
 * handle; csr_finish writes the m column indices into col_out and frees it.
 * Streaming two-pass bucket partition by source vertex (buckets of 2^13
 * vertices, per-thread slices so the layout is deterministic), then a local
 * counting sort, a sort and a dedup per row.
 * *err: 0, -1 on bad input (endpoint out of range), -2 on allocation failure,
 * -3 if the result does not fit int32 offsets; the handle is NULL on error.
 */
void *csr_build(int32_t n, int64_t nedges, const int32_t *src, const int32_t *dst,
                int32_t *row_ptr, int64_t *m_out, int32_t *err)
{
    const int shift = 13;
    const int64_t nb = ((int64_t)n + (1 << shift) - 1) >> shift;
    const int T = omp_get_max_threads();
    int64_t *cnt = (int64_t *)calloc((size_t)T * (size_t)nb, sizeof(int64_t));
    int64_t *bbase = (int64_t *)calloc((size_t)nb + 1, sizeof(int64_t));
    if (!cnt || !bbase) { free(cnt); free(bbase); *err = -2; return NULL; }
    int bad = 0;
#pragma omp parallel num_threads(T) reduction(|:bad)
    {
        int t = omp_get_thread_num(), nt = omp_get_num_threads();
        int64_t e0 = nedges * t / nt, e1 = nedges * (t + 1) / nt;
        int64_t *c = cnt + (int64_t)t * nb;
        for (int64_t e = e0; e < e1; ++e) {
            int32_t u = src[e], v = dst[e];
            if (u < 0 || u >= n || v < 0 || v >= n) { bad |= 1; continue; }
            if (u == v) continue;
            c[u >> shift]++;
            c[v >> shift]++;
        }
    }
    if (bad) { free(cnt); free(bbase); *err = -1; return NULL; }
    /* exclusive positions: bucket-major, thread-minor */
    int64_t run = 0;
    for (int64_t b = 0; b < nb; ++b) {
        bbase[b] = run;
        for (int t = 0; t < T; ++t) {
            int64_t x = cnt[(int64_t)t * nb + b];
            cnt[(int64_t)t * nb + b] = run;
            run += x;
        }
    }
    bbase[nb] = run;
    const int64_t total = run;
    uint64_t *packed = (uint64_t *)malloc((size_t)(total > 0 ? total : 1) * sizeof(uint64_t));
    int32_t *tmp = (int32_t *)malloc((size_t)(total > 0 ? total : 1) * sizeof(int32_t));
    int64_t *start = (int64_t *)malloc(((size_t)n + 1) * sizeof(int64_t));
    int32_t *deg = (int32_t *)malloc((size_t)n * sizeof(int32_t));
    if (!packed || !tmp || !start || !deg) {
        free(cnt); free(bbase); free(packed); free(tmp); free(start); free(deg);
        { *err = -2; return NULL; }
    }
#pragma omp parallel num_threads(T)
    {
        int t = omp_get_thread_num(), nt = omp_get_num_threads();
        int64_t e0 = nedges * t / nt, e1 = nedges * (t + 1) / nt;
        int64_t *pos = cnt + (int64_t)t * nb;
        for (int64_t e = e0; e < e1; ++e) {
            uint32_t u = (uint32_t)src[e], v = (uint32_t)dst[e];
            if (u == v) continue;
            packed[pos[u >> shift]++] = ((uint64_t)u << 32) | v;
            packed[pos[v >> shift]++] = ((uint64_t)v << 32) | u;
        }
    }
    free(cnt);
    /* per bucket: counting sort by source, then sort + dedup each row */
#pragma omp parallel num_threads(T)
    {
        int64_t *loc = (int64_t *)malloc(((size_t)(1 << shift) + 1) * sizeof(int64_t));
#pragma omp for schedule(dynamic, 1)
        for (int64_t b = 0; b < nb; ++b) {
            int32_t v0 = (int32_t)(b << shift);
            int32_t nv = (int32_t)((n - v0) < (1 << shift) ? (n - v0) : (1 << shift));
            for (int32_t i = 0; i <= nv; ++i) loc[i] = 0;
            for (int64_t k = bbase[b]; k < bbase[b + 1]; ++k)
                loc[(int32_t)(packed[k] >> 32) - v0 + 1]++;
            for (int32_t i = 0; i < nv; ++i) loc[i + 1] += loc[i];
            for (int32_t i = 0; i < nv; ++i) start[v0 + i] = bbase[b] + loc[i];
            for (int64_t k = bbase[b]; k < bbase[b + 1]; ++k) {
                int32_t lu = (int32_t)(packed[k] >> 32) - v0;
                tmp[bbase[b] + loc[lu]++] = (int32_t)(packed[k] & 0xffffffffULL);
            }
            for (int32_t i = 0; i < nv; ++i) {
                int32_t *r = tmp + start[v0 + i];
                int64_t len = (i + 1 < nv ? start[v0 + i + 1] : bbase[b + 1]) - start[v0 + i];
                sort_i32(r, len);
                int64_t w = 0;
                for (int64_t j = 0; j < len; ++j)
                    if (w == 0 || r[j] != r[w - 1]) r[w++] = r[j];
                deg[v0 + i] = (int32_t)w;
            }
        }
        free(loc);
    }
    free(packed);
    int64_t m = 0;
    for (int32_t i = 0; i < n; ++i) m += deg[i];
    if (m > INT32_MAX) { free(bbase); free(tmp); free(start); free(deg); *err = -3; return NULL; }
    row_ptr[0] = 0;
    for (int32_t i = 0; i < n; ++i) row_ptr[i + 1] = row_ptr[i] + deg[i];
    free(bbase);
    csr_build_t *h = (csr_build_t *)malloc(sizeof(csr_build_t));
    if (!h) { free(tmp); free(start); free(deg); *err = -2; return NULL; }
    h->n = n; h->tmp = tmp; h->start = start; h->deg = deg; h->row_ptr = row_ptr;
    *m_out = m;
    *err = 0;
    return h;
}

void csr_finish(void *handle, int32_t *col_out)
{
    csr_build_t *h = (csr_build_t *)handle;
#pragma omp parallel for schedule(dynamic, 4096)
    for (int32_t i = 0; i < h->n; ++i)
        memcpy(col_out + h->row_ptr[i], h->tmp + h->start[i], (size_t)h->deg[i] * sizeof(int32_t));
    free(h->tmp); free(h->start); free(h->deg); free(h);
}
