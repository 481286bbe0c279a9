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
// to save.
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
};
static_assert(ONE_N % 32 == 0, "whole visited words");

__global__ __launch_bounds__(ONE_BLOCK) void bfs_one_kernel(Params P) {
    __shared__ OneLds sh;
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
        P.ctl->err = 0;
        P.ctl->err_info = 0;
    }
    __syncthreads();
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
                const int b = P.row_ptr[v];
                d[j] = P.row_ptr[v + 1] - b;
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
            int u[ONE_CB], o[ONE_CB];
#pragma unroll
            for (int q = 0; q < ONE_CB; ++q) {
                const int e = e0 + q * ONE_BLOCK + tid;
                u[q] = -1;
                o[q] = 0;
                if (e < (int)E) {
                    int lo = 0, hi = F;   // last frontier entry whose offset is <= e
                    while (hi - lo > 1) {
                        const int mid = (lo + hi) >> 1;
                        if (sh.off[mid] <= e) lo = mid; else hi = mid;
                    }
                    o[q] = lo;
                    u[q] = P.col_idx[sh.beg[lo] + (e - sh.off[lo])];
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
    hipLaunchKernelGGL(bfs_one_kernel, dim3(1), dim3(ONE_BLOCK), 0, s, P);
    return hipGetLastError();
}

}  // namespace fbfs
