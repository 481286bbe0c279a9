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
 *
 * Where the search stores dist elsewhere, the per-level flags (the library's
 * BFS_LF_* bits; NULL: every level stores its own) move those bytes:
 *   queue-free top-down level: its new vertices cost 4 (parent) each plus the
 *     next bitmap n/8, instead of dist, parent and queue entry;
 *   finds kept: a bottom-up level's new vertices cost 4 (parent) each plus
 *     the kept bitmap n/8; frontier kept: + n/8; frontier dist: + 4|F_k|;
 *   finishing pass (bit 16 of level 0): the init writes no dist, and the
 *     finishing launch (finish_bytes) reads the visited bitmap and template
 *     (n/8 each) and every kept bitmap (n/8 each) and writes 4 bytes of dist
 *     for every vertex no level stored: kept, unreached, not the source.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { LF_QUEUE_FREE = 1, LF_FINDS_KEPT = 2, LF_FRONTIER_KEPT = 4, LF_FRONTIER_DIST = 8, LF_FINISHING = 16 };

int32_t bfs_alg_bytes(int32_t n, const int32_t *row_ptr, const int32_t *col_idx,
                      const int32_t *in_row_ptr, const int32_t *in_col_idx,
                      const int32_t *dist, int32_t L, const int8_t *dir, const uint8_t *flags,
                      int32_t with_parent, int64_t *init_bytes, int64_t *level_bytes,
                      int64_t *finish_bytes)
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
    const int64_t par = with_parent ? 4 : 0;
    const int64_t per_new_td = 8 + par;
    const int64_t per_new_bu = 4 + par;
    const int finishing = flags && (flags[0] & LF_FINISHING);
    *init_bytes = (finishing ? 0 : 4LL * n) + par * (int64_t)n + bm;
    *finish_bytes = 0;
    int64_t kept_maps = 0;
    for (int32_t k = 0; k < L; ++k) {
        const int64_t fnext = (k + 1 < L) ? fsz[k + 1] : 0;
        const uint8_t f = flags ? flags[k] : 0;
        int64_t extra = 0;   /* the frontier's kept bitmap or dist, left by the level before */
        if (f & LF_FRONTIER_KEPT) { extra += bm; kept_maps += 1; }
        if (f & LF_FRONTIER_DIST) extra += 4 * fsz[k];
        if (dir[k] == 0) {
            if (f & LF_QUEUE_FREE)
                level_bytes[k] = 12 * fsz[k] + 4 * fdeg[k] + par * fnext + bm + extra;
            else
                level_bytes[k] = 12 * fsz[k] + 4 * fdeg[k] + per_new_td * fnext + extra;
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
            if (f & LF_FINDS_KEPT) {
                level_bytes[k] = bm + 8 * U + 4 * S + par * fnext + bm + bm + extra;
                kept_maps += 1;
            } else {
                level_bytes[k] = bm + 8 * U + 4 * S + per_new_bu * fnext + bm + extra;
            }
        }
    }
    if (finishing) {
        /* dist of the kept levels' vertices, of the unreached and of nothing
         * else (the source and the vertices of levels that stored their own) */
        int64_t stored = 0;
        for (int32_t k = 0; k < L; ++k) {
            const uint8_t f = flags[k];
            const int finds_kept = dir[k] != 0 && (f & LF_FINDS_KEPT);
            if (k + 1 < L && finds_kept) stored += fsz[k + 1];
            if (f & LF_FRONTIER_KEPT) stored += fsz[k];
        }
        int64_t reached = 0;
        for (int32_t k = 0; k < L; ++k) reached += fsz[k];
        const int64_t writes = stored + ((int64_t)n - reached);
        *finish_bytes = 2 * bm + kept_maps * bm + 4 * writes;
    }
    free(fsz); free(fdeg); free(uge);
    return 0;
}
