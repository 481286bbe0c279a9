/*
 * Reference oracle for level-synchronous BFS over an int32 CSR graph.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link
 * or call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes (a plain serial FIFO-queue BFS, no blocking or reordering):
 *   - "Chapter 22: The Frontier Model for Parallel Breadth-First Search",
 *     section 22.1, the sequential CPU baseline: a vertex is enqueued when it
 *     is first discovered and expanded when dequeued; unvisited is -1.
 *   - bfs.cu of "Day 38 - Graph traversal on a GPU", function bfsCpu: the
 *     FIFO order sliced by level gives the exact per-level frontiers.
 *   - PMPP ch.15 notes ("graph traversal"), section 15.1: CSR layout,
 *     neighbours of u are col_idx[row_ptr[u] .. row_ptr[u+1]).
 *
 * Readings taken where the pages leave a point open:
 *   - unreached vertices hold -1 (the sentinel of bfs.cu and Chapter 22);
 *   - parent[source] = source, parent of an unreached vertex = -1, and the
 *     parent of a reached vertex is the vertex that first discovered it in
 *     FIFO order (any same-level predecessor is an equally valid parent);
 *   - the level count L is the number of non-empty frontiers (= max dist + 1);
 *   - edges are followed in CSR direction, so directed graphs are allowed;
 *   - self-loops and duplicate entries are accepted (they change nothing).
 *
 * Parity pins (in tests, against things other than this code): the values
 * Chapter 22 prints for its 6-vertex graph, the 4-vertex graph of PMPP
 * section 15.1 checked by brute force, Floyd-Warshall all-pairs distances on
 * tiny random graphs, closed forms (paths, stars, complete graphs, full grids)
 * and the checker's own negative cases.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/*
 * ORACLE_MUTANT plants one deliberate mistake (test builds only, never the
 * default build): the mutation tests compile each mutant and check that the
 * pins reject it.  0 = the real oracle.
 *   1 dist[v] = dist[u] (dropped +1)      2 last neighbour of each row skipped
 *   3 parent[v] = v                       4 L one short
 *   5 neighbours scanned in reverse       6 checker skips the adjacency test
 *   7 checker skips the last vertex's dist
 *   8 walk adds (c + r) instead of (c ^ r)  9 walk starts at r = 1
 *  10 walk sums entry indices, not neighbour ids
 */
#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* ---------------------------------------------------------------- BFS --- */

/*
 * Serial FIFO BFS from `source`.
 *   dist[n]        out: hop count or -1
 *   parent[n]      out (may be NULL): discovering vertex, source for source
 *   level_sizes[n] out (may be NULL): |{v : dist[v] = k}| for k < L
 *   order[n]       out (may be NULL): the FIFO dequeue order (reached vertices)
 * Returns L >= 1, or -1 on invalid arguments, -2 on allocation failure.
 */
int32_t oracle_bfs(int32_t n, const int32_t *row_ptr, const int32_t *col_idx,
                   int32_t source, int32_t *dist, int32_t *parent,
                   int32_t *level_sizes, int32_t *order)
{
    if (n <= 0 || !row_ptr || !col_idx || !dist || source < 0 || source >= n)
        return -1;
    int32_t *queue = order;
    int own = 0;
    if (!queue) {
        queue = (int32_t *)malloc((size_t)n * sizeof(int32_t));
        if (!queue) return -2;
        own = 1;
    }
    for (int32_t v = 0; v < n; ++v) dist[v] = -1;
    if (parent)
        for (int32_t v = 0; v < n; ++v) parent[v] = -1;

    int64_t head = 0, tail = 0;
    dist[source] = 0;
    if (parent) parent[source] = source;
    queue[tail++] = source;
    while (head < tail) {
        int32_t u = queue[head++];
#if ORACLE_MUTANT == 2
        for (int32_t e = row_ptr[u]; e < row_ptr[u + 1] - 1; ++e) {
#elif ORACLE_MUTANT == 5
        for (int32_t r = row_ptr[u + 1] - 1; r >= row_ptr[u]; --r) {
            int32_t e = r;
#else
        for (int32_t e = row_ptr[u]; e < row_ptr[u + 1]; ++e) {
#endif
            int32_t v = col_idx[e];
            if (dist[v] < 0) {
#if ORACLE_MUTANT == 1
                dist[v] = dist[u];
                if (dist[v] < 0) dist[v] = 0;
#else
                dist[v] = dist[u] + 1;
#endif
#if ORACLE_MUTANT == 3
                if (parent) parent[v] = v;
#else
                if (parent) parent[v] = u;
#endif
                queue[tail++] = v;
            }
        }
    }
    /* FIFO order is sorted by dist, so the last dequeued vertex has the
     * largest distance; levels are the runs of equal dist in the queue. */
    int32_t L = dist[queue[tail - 1]] + 1;
#if ORACLE_MUTANT == 4
    L -= 1;
#endif
    if (level_sizes) {
        for (int32_t k = 0; k < L; ++k) level_sizes[k] = 0;
        for (int64_t i = 0; i < tail; ++i) level_sizes[dist[queue[i]]]++;
    }
    if (own) free(queue);
    return L;
}

/*
 * Many sources, one after another (used for the CPU-baseline timing and for
 * eccentricity checks).  Writes L per source into levels_out[s_i] and the
 * count of reached vertices into reached_out (either may be NULL).  dist is
 * scratch of n entries.  Returns 0 or a negative error.
 */
int32_t oracle_bfs_many(int32_t n, const int32_t *row_ptr, const int32_t *col_idx,
                        int32_t nsrc, const int32_t *sources, int32_t *dist,
                        int32_t *levels_out, int64_t *reached_out)
{
    int32_t *queue = (int32_t *)malloc((size_t)n * sizeof(int32_t));
    if (!queue) return -2;
    for (int32_t i = 0; i < nsrc; ++i) {
        int32_t L = oracle_bfs(n, row_ptr, col_idx, sources[i], dist, NULL, NULL, queue);
        if (L < 0) { free(queue); return L; }
        if (levels_out) levels_out[i] = L;
        if (reached_out) {
            int64_t r = 0;
            for (int32_t v = 0; v < n; ++v) r += dist[v] >= 0;
            reached_out[i] = r;
        }
    }
    free(queue);
    return 0;
}

/* ------------------------------------------------------------ checker --- */

/* Is v among col_idx[b..e)?  Binary search when the slice is sorted. */
__attribute__((unused)) static int in_row(const int32_t *col_idx, int32_t b, int32_t e, int32_t v, int sorted)
{
    if (sorted) {
        int32_t lo = b, hi = e;
        while (lo < hi) {
            int32_t mid = lo + (hi - lo) / 2;
            if (col_idx[mid] < v) lo = mid + 1; else hi = mid;
        }
        return lo < e && col_idx[lo] == v;
    }
    for (int32_t i = b; i < e; ++i)
        if (col_idx[i] == v) return 1;
    return 0;
}

/* Failure codes of oracle_check. */
enum {
    CHK_OK = 0,
    CHK_DIST = 1,          /* dist differs from the oracle's             */
    CHK_LEVELS = 2,        /* L differs from the oracle's                */
    CHK_SIZES = 3,         /* level_sizes[k] differs                     */
    CHK_SIZE_SUM = 4,      /* sum of level sizes != reached count        */
    CHK_PARENT_SRC = 5,    /* parent[source] != source                   */
    CHK_PARENT_LEVEL = 6,  /* dist[parent[v]] != dist[v] - 1             */
    CHK_PARENT_EDGE = 7,   /* v not in adj(parent[v])                    */
    CHK_PARENT_UNREACHED = 8, /* unreached vertex with parent != -1      */
    CHK_EDGE_SYM = 9,      /* |dist[u]-dist[v]| > 1 or reached~unreached */
    CHK_EDGE_DIR = 10,     /* dist[u] >= 0 but dist[v] not in [0,dist[u]+1] */
    CHK_ARGS = 11,
    CHK_NOMEM = 12
};

/*
 * Checks a BFS result (dist, parent, L, level_sizes) for `source`.
 *   ref_dist / ref_L / ref_sizes: the oracle's result (exact comparison, the
 *     gates of bfs.cu's main: distances equal, level count equal, frontier
 *     sizes sum to the number reached).
 *   parent may be NULL (not checked); sizes may be NULL (not checked).
 *   symmetric != 0 selects the undirected edge invariant.
 * Returns CHK_OK or the first failing code; *bad gets the offending vertex
 * (or level) index.
 */
int32_t oracle_check(int32_t n, const int32_t *row_ptr, const int32_t *col_idx,
                     int32_t source, const int32_t *ref_dist, int32_t ref_L,
                     const int32_t *ref_sizes, const int32_t *dist,
                     const int32_t *parent, int32_t L, const int32_t *sizes,
                     int32_t symmetric, int64_t *bad)
{
    int64_t dummy;
    if (!bad) bad = &dummy;
    *bad = -1;
    if (n <= 0 || !row_ptr || !col_idx || !ref_dist || !dist || source < 0 || source >= n)
        return CHK_ARGS;

    /* V1: dist equal to the oracle's, vertex by vertex. */
#if ORACLE_MUTANT == 7
    for (int32_t v = 0; v < n - 1; ++v)
#else
    for (int32_t v = 0; v < n; ++v)
#endif
        if (dist[v] != ref_dist[v]) { *bad = v; return CHK_DIST; }

    /* V2: level count and per-level sizes; the sizes add up to #reached. */
    if (L != ref_L) { *bad = L; return CHK_LEVELS; }
    int64_t reached = 0;
    for (int32_t v = 0; v < n; ++v) reached += dist[v] >= 0;
    if (sizes) {
        int64_t sum = 0;
        for (int32_t k = 0; k < L; ++k) {
            if (ref_sizes && sizes[k] != ref_sizes[k]) { *bad = k; return CHK_SIZES; }
            sum += sizes[k];
        }
        if (sum != reached) { *bad = sum; return CHK_SIZE_SUM; }
    }

    /* V3: parents are valid BFS parents (any same-level candidate is fine). */
    if (parent) {
        if (parent[source] != source) { *bad = source; return CHK_PARENT_SRC; }
        /* per-row sortedness, so membership tests can binary search */
        unsigned char *sorted = (unsigned char *)malloc((size_t)n);
        if (!sorted) return CHK_NOMEM;
        for (int32_t u = 0; u < n; ++u) {
            int ok = 1;
            for (int32_t e = row_ptr[u] + 1; e < row_ptr[u + 1]; ++e)
                if (col_idx[e - 1] > col_idx[e]) { ok = 0; break; }
            sorted[u] = (unsigned char)ok;
        }
        for (int32_t v = 0; v < n; ++v) {
            if (v == source) continue;
            int32_t p = parent[v];
            if (dist[v] < 0) {
                if (p != -1) { free(sorted); *bad = v; return CHK_PARENT_UNREACHED; }
                continue;
            }
            if (p < 0 || p >= n || dist[p] != dist[v] - 1) {
                free(sorted); *bad = v; return CHK_PARENT_LEVEL;
            }
#if ORACLE_MUTANT == 6
            if (0) {
#else
            if (!in_row(col_idx, row_ptr[p], row_ptr[p + 1], v, sorted[p])) {
#endif
                free(sorted); *bad = v; return CHK_PARENT_EDGE;
            }
        }
        free(sorted);
    }

    /* V4: edge invariants of a BFS layering. */
    for (int32_t u = 0; u < n; ++u) {
        for (int32_t e = row_ptr[u]; e < row_ptr[u + 1]; ++e) {
            int32_t v = col_idx[e];
            if (symmetric) {
                if ((dist[u] < 0) != (dist[v] < 0)) { *bad = u; return CHK_EDGE_SYM; }
                if (dist[u] >= 0) {
                    int32_t d = dist[u] - dist[v];
                    if (d > 1 || d < -1) { *bad = u; return CHK_EDGE_SYM; }
                }
            } else if (dist[u] >= 0) {
                if (dist[v] < 0 || dist[v] > dist[u] + 1) { *bad = u; return CHK_EDGE_DIR; }
            }
        }
    }
    return CHK_OK;
}

/*
 * Neighbour-walk checksum of one level ("Day 38 - Graph traversal on a GPU",
 * "Measuring the mapping without measuring the launch"): for every listed
 * vertex u, the wrapping unsigned 32-bit sum over repeats r = 0 .. repeats-1
 * and over u's CSR entries of (neighbour id XOR r).  Unsigned arithmetic wraps
 * by definition, so every correct walk returns the same value whatever order
 * it adds in.  Returns 0, or -1 on bad arguments.
 */
int32_t oracle_walk_checksum(int32_t n, const int32_t *row_ptr, const int32_t *col_idx,
                             int32_t count, const int32_t *vertices, int32_t repeats,
                             uint32_t *out)
{
    if (n < 0 || count < 0 || repeats < 0 || (count > 0 && (!vertices || !out))) return -1;
    for (int32_t i = 0; i < count; ++i) {
        const int32_t u = vertices[i];
        if (u < 0 || u >= n) return -1;
        uint32_t acc = 0u;
#if ORACLE_MUTANT == 9
        for (int32_t r = 1; r < repeats; ++r)
#else
        for (int32_t r = 0; r < repeats; ++r)
#endif
            for (int32_t e = row_ptr[u]; e < row_ptr[u + 1]; ++e)
#if ORACLE_MUTANT == 8
                acc += (uint32_t)col_idx[e] + (uint32_t)r;
#elif ORACLE_MUTANT == 10
                acc += (uint32_t)e ^ (uint32_t)r;
#else
                acc += (uint32_t)col_idx[e] ^ (uint32_t)r;
#endif
        out[i] = acc;
    }
    return 0;
}


/*
 * Single-source shortest paths with non-negative integer edge weights, the
 * second workload the Gunrock reading guide (step 2) says the same atomic-min
 * lambda serves, and the next chapter "Chapter 22" points to.  weights[e] is
 * the weight of CSR entry e (row u, neighbour col_idx[e]).
 *
 * Distances: Dijkstra's algorithm with a binary min-heap of (distance,
 * vertex) pairs and lazy deletion (a popped pair whose distance is above the
 * vertex's current one is skipped).  dist[v] = -1 when v is unreachable.
 * Predecessor: among the entries u -> v that are tight (dist[u] + w = dist[v],
 * u reached), the smallest u; pred[source] = source, -1 when unreachable.
 * That choice is a property of the distances alone, so every correct solver
 * that settles ties by the smaller id agrees with it exactly.
 * Returns 0, -1 on bad arguments, -2 when out of memory.
 */
typedef struct { int64_t d; int32_t v; } HeapItem;

static void heap_push(HeapItem *h, int64_t *len, HeapItem x)
{
    int64_t i = (*len)++;
    while (i > 0) {
        const int64_t p = (i - 1) / 2;
        if (h[p].d <= x.d) break;
        h[i] = h[p];
        i = p;
    }
    h[i] = x;
}

static HeapItem heap_pop(HeapItem *h, int64_t *len)
{
    const HeapItem top = h[0];
    const HeapItem x = h[--(*len)];
    int64_t i = 0;
    for (;;) {
        int64_t c = 2 * i + 1;
        if (c >= *len) break;
        if (c + 1 < *len && h[c + 1].d < h[c].d) ++c;
        if (h[c].d >= x.d) break;
        h[i] = h[c];
        i = c;
    }
    if (*len > 0) h[i] = x;
    return top;
}

int32_t oracle_sssp(int32_t n, const int32_t *row_ptr, const int32_t *col_idx, const uint32_t *weights,
                    int32_t source, int64_t *dist, int32_t *pred)
{
    if (n <= 0 || source < 0 || source >= n || !row_ptr || !dist || !pred) return -1;
    const int64_t m = row_ptr[n];
    if (m > 0 && (!col_idx || !weights)) return -1;
    for (int32_t v = 0; v < n; ++v) { dist[v] = -1; pred[v] = -1; }
    /* every entry pushes at most one pair, plus the source */
    HeapItem *h = (HeapItem *)malloc(sizeof(HeapItem) * (size_t)(m + 1));
    if (!h) return -2;
    int64_t len = 0;
    dist[source] = 0;
    heap_push(h, &len, (HeapItem){0, source});
    while (len > 0) {
        const HeapItem it = heap_pop(h, &len);
        if (it.d > dist[it.v]) continue;          /* stale */
        const int32_t u = it.v;
        for (int64_t e = row_ptr[u]; e < row_ptr[u + 1]; ++e) {
            const int32_t v = col_idx[e];
#if ORACLE_MUTANT == 11
            const int64_t nd = it.d + 1;
#else
            const int64_t nd = it.d + (int64_t)weights[e];
#endif
            if (dist[v] < 0 || nd < dist[v]) {
                dist[v] = nd;
                heap_push(h, &len, (HeapItem){nd, v});
            }
        }
    }
    free(h);
    /* predecessors: the smallest tight in-neighbour */
    pred[source] = source;
    for (int32_t u = 0; u < n; ++u) {
        if (dist[u] < 0) continue;
        for (int64_t e = row_ptr[u]; e < row_ptr[u + 1]; ++e) {
            const int32_t v = col_idx[e];
            if (v == source) continue;
#if ORACLE_MUTANT == 11
            const int64_t w = 1;
#else
            const int64_t w = (int64_t)weights[e];
#endif
#if ORACLE_MUTANT == 13
            /* reads the entry backwards: v as the predecessor of u */
            if (dist[v] >= 0 && dist[v] + w == dist[u] && u != source && (pred[u] < 0 || v < pred[u])) pred[u] = v;
#else
            if (dist[u] + w == dist[v]) {
#if ORACLE_MUTANT == 12
                if (pred[v] < 0 || u > pred[v]) pred[v] = u;
#else
                if (pred[v] < 0 || u < pred[v]) pred[v] = u;
#endif
            }
#endif
        }
    }
    return 0;
}
