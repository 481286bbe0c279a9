// The whole search in one workgroup, for graphs of at most ONE_N vertices
// (the word-graph scale of the "Day 38" page).  On such a graph every level
// of the multi-workgroup path is a chain of device round trips (decision,
// queue, flush reservation, barrier) around a few hundred edges; here the
// visited bits, both frontier queues and the frontier's degree offsets sit in
// LDS, a claim is an LDS atomicOr, and a level costs the row-pointer reads,
// the adjacency reads and three workgroup barriers.  Same level-synchronous
// method: the frontier's edges are dealt out edge-balanced (owner by the last
// offset not above the edge, as in the edge-balanced advance), every neighbour
// is claimed once, and the winner writes dist and parent and joins the next
// frontier.  Top-down only: on graphs this small a bottom-up pass has nothing
// to save.  When the graph has at most ONE_M CSR entries and 16-byte aligned
// arrays, the row pointers and the adjacency (as 16-bit ids: n <= ONE_N) are
// first copied into LDS (16-byte loads, all in flight at once), and the
// levels then read no global memory (their only global accesses are the
// dist, parent and per-level stores).
#include <type_traits>

#include "bfs_internal.h"
#include "frontier_bfs.h"

namespace fbfs {

namespace {

constexpr int ONE_BLOCK = 1024;
constexpr int ONE_WAVES = ONE_BLOCK / WAVE;
constexpr int ONE_PER = (ONE_N + ONE_BLOCK - 1) / ONE_BLOCK;   // frontier entries per thread in the scan
constexpr int ONE_CB = 8;                                        // edges per thread per pass, loaded together

struct OneLds {
    uint32_t vis[ONE_N / 32];       // visited bits
    int32_t q[2][ONE_N];            // frontier of this level and of the next
    int32_t off[ONE_N + 1];         // exclusive scan of the frontier's degrees
    int32_t beg[ONE_N];             // the frontier vertices' first CSR entries
    uint32_t wsum[ONE_WAVES];       // per-wavefront degree totals
    int32_t ncount;                 // next-frontier length
    int32_t bad;                    // the LDS copy of the graph failed its checks
};

// ... and, for the LDS-resident variant, the graph itself
constexpr int ONE_LD = 10;                         // 16-byte loads per thread in the copy
static_assert(ONE_BLOCK * ONE_LD * 4 >= ONE_M, "one pass of loads copies the adjacency");
struct OneGraphLds {
    int32_t rp[ONE_N + 1];          // row pointers
    uint16_t col[ONE_M];            // adjacency, 16-bit ids
};
struct OneNoGraph {                 // its stand-in elsewhere (never read)
    int32_t rp[1];
    uint16_t col[2];
};
static_assert(ONE_N % 32 == 0, "whole visited words");

template <bool RES>
__global__ __launch_bounds__(ONE_BLOCK) void bfs_one_kernel(Params P) {
    __shared__ OneLds sh;
    __shared__ std::conditional_t<RES, OneGraphLds, OneNoGraph> gr;   // (a stub unless resident)
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int wv = tid / WAVE;
    const int n = P.n;
    const int s = P.source;
    for (int i = tid; i < n; i += ONE_BLOCK) {
        P.dist[i] = (i == s) ? 0 : -1;
        if (P.parent) P.parent[i] = (i == s) ? s : -1;
#ifdef FBFS_COUNT_ENQUEUES
        if (P.enq) P.enq[i] = 0;
#endif
    }
    for (int w = tid; w < ONE_N / 32; w += ONE_BLOCK) sh.vis[w] = (w == (s >> 5)) ? (1u << (s & 31)) : 0u;
    if (tid == 0) {
        sh.q[0][0] = s;
        sh.bad = 0;
        P.ctl->err = 0;
        P.ctl->err_info = 0;
    }
    if constexpr (RES) {
        // the graph into LDS: ONE_LD 16-byte loads per thread issued before
        // any is stored (both arrays are 16-byte aligned: the host checks);
        // an id outside [0, n) or a row pointer out of [0, m] (a graph
        // changed after its checks) ends the search with an error
        const int m = P.m;
        const int4 *c4 = reinterpret_cast<const int4 *>(P.col_idx);
        const int nc4 = (m + 3) / 4;
        int4 x[ONE_LD];
#pragma unroll
        for (int j = 0; j < ONE_LD; ++j) {
            const int i = j * ONE_BLOCK + tid;
            x[j] = (i < nc4 && 4 * i + 3 < m) ? c4[i] : make_int4(0, 0, 0, 0);
            if (i < nc4 && 4 * i + 3 >= m) {   // the ragged tail, entry by entry
                x[j].x = P.col_idx[4 * i];
                if (4 * i + 1 < m) x[j].y = P.col_idx[4 * i + 1];
                if (4 * i + 2 < m) x[j].z = P.col_idx[4 * i + 2];
            }
        }
        for (int i = tid; i <= n; i += ONE_BLOCK) {
            const int r = P.row_ptr[i];
            gr.rp[i] = r;
            if (r < 0 || r > m || (i == 0 && r != 0) || (i == n && r != m)) sh.bad = 1;
        }
#pragma unroll
        for (int j = 0; j < ONE_LD; ++j) {
            const int i = j * ONE_BLOCK + tid;
            if (i < nc4) {
                const int e = 4 * i;
                bool ok = (uint32_t)x[j].x < (uint32_t)n;
                gr.col[e] = (uint16_t)x[j].x;
                if (e + 1 < m) { ok = ok && (uint32_t)x[j].y < (uint32_t)n; gr.col[e + 1] = (uint16_t)x[j].y; }
                if (e + 2 < m) { ok = ok && (uint32_t)x[j].z < (uint32_t)n; gr.col[e + 2] = (uint16_t)x[j].z; }
                if (e + 3 < m) { ok = ok && (uint32_t)x[j].w < (uint32_t)n; gr.col[e + 3] = (uint16_t)x[j].w; }
                if (!ok) sh.bad = 1;
            }
        }
    }
    __syncthreads();
    if constexpr (RES) {
        for (int i = tid; i < n; i += ONE_BLOCK)
            if (gr.rp[i] > gr.rp[i + 1]) sh.bad = 1;
        __syncthreads();
        if (sh.bad) {
            if (tid == 0) { P.ctl->err = ERR_BAD_VERTEX; P.ctl->err_info = -1; P.ctl->L = 0; P.ctl->done = 1; }
            return;
        }
    }
    int F = 1, cur = 0, k = 0;
    while (F > 0 && k < n) {
        // the frontier's first entries and degrees, and the exclusive scan of
        // the degrees (ONE_PER consecutive entries per thread)
        int d[ONE_PER];
        uint32_t tot = 0;
#pragma unroll
        for (int j = 0; j < ONE_PER; ++j) {
            const int i = tid * ONE_PER + j;
            d[j] = 0;
            if (i < F) {
                const int v = sh.q[cur][i];
                const int b = RES ? gr.rp[v] : P.row_ptr[v];
                d[j] = (RES ? gr.rp[v + 1] : P.row_ptr[v + 1]) - b;
                sh.beg[i] = b;
            }
            tot += (uint32_t)d[j];
        }
        const uint32_t incl = wave_incl_scan_u32(tot);
        if (lane == WAVE - 1) sh.wsum[wv] = incl;
        __syncthreads();
        uint32_t base = incl - tot, E = 0;
        for (int w = 0; w < ONE_WAVES; ++w) {
            if (w < wv) base += sh.wsum[w];
            E += sh.wsum[w];
        }
#pragma unroll
        for (int j = 0; j < ONE_PER; ++j) {
            const int i = tid * ONE_PER + j;
            if (i < F) sh.off[i] = (int)base;
            base += (uint32_t)d[j];
        }
        if (tid == 0) {
            sh.off[F] = (int)E;
            sh.ncount = 0;   // every thread read last level's count before the barrier above
            if (P.level_sizes) P.level_sizes[k] = F;
            if (k < P.st_cap) {
                P.st_dir[k] = 0;
                P.st_fdeg[k] = E;
            }
        }
        __syncthreads();
        // every frontier edge: its owner, its neighbour, one claim per neighbour
        const int nxt = cur ^ 1;
        for (int e0 = 0; e0 < (int)E; e0 += ONE_CB * ONE_BLOCK) {
            // ONE_CB consecutive edges per thread: one binary search for the
            // owner of the first, then a walk forward (an owner's edges are
            // consecutive, so the walk mostly stays put)
            int u[ONE_CB], o[ONE_CB];
            const int ea = e0 + tid * ONE_CB;
            int lo = 0;
            if (ea < (int)E) {
                int hi = F;   // last frontier entry whose offset is <= ea
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (sh.off[mid] <= ea) lo = mid; else hi = mid;
                }
            }
#pragma unroll
            for (int q = 0; q < ONE_CB; ++q) {
                const int e = ea + q;
                u[q] = -1;
                o[q] = 0;
                if (e < (int)E) {
                    while (sh.off[lo + 1] <= e) ++lo;   // off[F] = E > e ends it
                    o[q] = lo;
                    const int ce = sh.beg[lo] + (e - sh.off[lo]);
                    u[q] = RES ? (int)gr.col[ce] : P.col_idx[ce];
                }
            }
#pragma unroll
            for (int q = 0; q < ONE_CB; ++q) {
                if (u[q] < 0) continue;
                if (u[q] >= n) {   // a graph changed after its checks: reported, never stored
                    if (P.ctl->err == 0) { P.ctl->err = ERR_BAD_VERTEX; P.ctl->err_info = u[q]; }
                    continue;
                }
                const uint32_t bit = 1u << (u[q] & 31);
                if (atomicOr(&sh.vis[u[q] >> 5], bit) & bit) continue;
                P.dist[u[q]] = k + 1;
                if (P.parent) P.parent[u[q]] = sh.q[cur][o[q]];
                FBFS_ENQ(P, u[q]);
                sh.q[nxt][atomicAdd(&sh.ncount, 1)] = u[q];
            }
        }
        __syncthreads();
        F = sh.ncount;
        cur = nxt;
        ++k;
    }
    if (tid == 0) {
        P.ctl->L = k;
        P.ctl->done = 1;
    }
}

}  // namespace

hipError_t launch_one(const Params &P, hipStream_t s) {
    const bool aligned = (reinterpret_cast<uintptr_t>(P.col_idx) & 15) == 0;
    if (P.m <= ONE_M && aligned)
        hipLaunchKernelGGL(bfs_one_kernel<true>, dim3(1), dim3(ONE_BLOCK), 0, s, P);
    else
        hipLaunchKernelGGL(bfs_one_kernel<false>, dim3(1), dim3(ONE_BLOCK), 0, s, P);
    return hipGetLastError();
}

}  // namespace fbfs
