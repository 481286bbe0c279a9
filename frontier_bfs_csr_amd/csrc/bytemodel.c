/*
 * Algorithmic byte model of one BFS (host, OpenMP): the bytes the method
 * itself must move -- CSR reads, frontier reads and writes, outputs -- per
 * level, given the graph, the result dist and the direction each level ran in.
 * Random status probes (visited tests in top-down, frontier-bit tests in
 * bottom-up) and the mapping's own overhead (bins, scans, conversions) are not
 * counted, so a fraction of the roofline computed from it is conservative.
 *
 *   init:      4n (dist) + 4n (parent, if written) + n/8 (visited bitmap)
 *   top-down k:  4|F_k| (queue) + 8|F_k| (row_ptr pair) + 4*sum deg(F_k)
 *                + |F_k+1| * (4 dist + 4 parent + 4 queue)
 *   bottom-up k: n/8 (visited words) + 8|U_k| (row_ptr pairs) + 4*S_k
 *                + |F_k+1| * (4 dist + 4 parent) + n/8 (next bitmap)
 * Bottom-up levels scan in-edge lists (in_row_ptr/in_col_idx: the CSR itself
 * for a symmetric graph, its transpose otherwise).  U_k = vertices with
 * in-edges still unreached when level k starts; S_k = entries a scan of the
 * in-lists reads: up to and including the first in-neighbour at distance k
 * for vertices found at level k+1, the whole list otherwise.  With no parent
 * output the 4-byte parent terms are dropped.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

int32_t bfs_alg_bytes(int32_t n, const int32_t *row_ptr, const int32_t *col_idx,
                      const int32_t *in_row_ptr, const int32_t *in_col_idx,
                      const int32_t *dist, int32_t L, const int8_t *dir,
                      int32_t with_parent, int64_t *init_bytes, int64_t *level_bytes)
{
    if (n <= 0 || L <= 0) return -1;
    int64_t *fsz = (int64_t *)calloc((size_t)L + 1, sizeof(int64_t));
    int64_t *fdeg = (int64_t *)calloc((size_t)L + 1, sizeof(int64_t));
    int64_t *uge = (int64_t *)calloc((size_t)L + 2, sizeof(int64_t)); /* with in-edges, dist >= k or unreached */
    if (!fsz || !fdeg || !uge) { free(fsz); free(fdeg); free(uge); return -2; }
    int64_t unreached_noniso = 0;
    for (int32_t v = 0; v < n; ++v) {
        int32_t d = dist[v];
        int64_t deg = row_ptr[v + 1] - row_ptr[v];
        int64_t indeg = in_row_ptr[v + 1] - in_row_ptr[v];
        if (d >= 0) {
            if (d >= L) { free(fsz); free(fdeg); free(uge); return -3; }
            fsz[d] += 1;
            fdeg[d] += deg;
            if (indeg > 0) uge[d] += 1;
        } else if (indeg > 0) {
            unreached_noniso += 1;
        }
    }
    /* suffix sums: uge[k] = nonisolated vertices with dist >= k, plus unreached */
    uge[L] = unreached_noniso;
    for (int32_t k = L - 1; k >= 0; --k) uge[k] += uge[k + 1];
    const int64_t bm = ((int64_t)n + 7) / 8;
    const int64_t per_new_td = with_parent ? 12 : 8;
    const int64_t per_new_bu = with_parent ? 8 : 4;
    *init_bytes = 4LL * n + (with_parent ? 4LL * n : 0) + bm;
    for (int32_t k = 0; k < L; ++k) {
        const int64_t fnext = (k + 1 < L) ? fsz[k + 1] : 0;
        if (dir[k] == 0) {
            level_bytes[k] = 12 * fsz[k] + 4 * fdeg[k] + per_new_td * fnext;
        } else {
            /* U_k: unreached at the start of level k = dist > k or unreached,
             * i.e. dist >= k+1; the frontier F_k itself is already visited */
            const int64_t U = uge[k + 1];
            int64_t S = 0;
#pragma omp parallel for reduction(+:S) schedule(dynamic, 4096)
            for (int32_t v = 0; v < n; ++v) {
                const int32_t d = dist[v];
                const int32_t b = in_row_ptr[v], e = in_row_ptr[v + 1];
                if (e == b || (d >= 0 && d <= k)) continue;
                if (d == k + 1) {
                    int32_t j = b;
                    while (j < e && dist[in_col_idx[j]] != k) ++j;
                    S += (j < e) ? (j - b + 1) : (e - b);
                } else {
                    S += e - b;
                }
            }
            level_bytes[k] = bm + 8 * U + 4 * S + per_new_bu * fnext + bm;
        }
    }
    free(fsz); free(fdeg); free(uge);
    return 0;
}
