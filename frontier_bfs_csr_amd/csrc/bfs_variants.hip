// Alternative claim and compaction primitives for the top-down level, as the
// pages describe them beside the direction-optimising path:
//
//   claim      BFS_CLAIM_BITMAP  one atomicOr on the visited bitmap picks the
//                                winner, which writes dist (the main path's);
//              BFS_CLAIM_MIN     atomicMin on dist itself, the winner being the
//                                caller that saw a larger old value (Gunrock
//                                reading guide, step 2: the search lambda with
//                                atomic::min; unreached dist is -1, the largest
//                                value read as unsigned)
//   compaction BFS_COMPACT_ATOMIC wave-aggregated atomic append of the winners
//                                ("Day 38" page: claimVertex with an atomic
//                                counter standing in for the scan)
//              BFS_COMPACT_PADDED idempotent advance: every frontier edge writes
//                                its neighbour if it won, else a -1 sentinel,
//                                at its own position; the padded array is the
//                                next frontier (Gunrock step 2, filter off)
//              BFS_COMPACT_FILTER the padded array compacted by flag, scan and
//                                scatter (the filter on)
//              BFS_COMPACT_FLAGS flag every vertex with dist = k + 1, scan the
//                                flags over all n vertices, scatter: a
//                                deterministic frontier in id order for O(n)
//                                per level ("Day 38" page, day 33's compaction)
//
// The level loop is the pages' own: one read of two counters per level on the
// host.  Each level: the frontier's degrees, their exclusive scan, one
// edge-balanced advance over all frontier edges (short runs per lane, owner
// by binary search), the compaction.
#include "bfs_internal.h"
#include "frontier_bfs.h"

namespace fbfs {

namespace {

constexpr int VAR_K = 4;   // longest run of frontier edges per lane in the advance

__device__ __forceinline__ int owner_in(const int32_t *offs, int lo, int hi, int64_t e) {
    // last i in [lo, hi) with offs[i] <= e (offs[lo] <= e < offs[hi] on entry)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offs[mid] <= e) lo = mid; else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(BLOCK) void var_seed_kernel(int32_t *F, int32_t source, int32_t *level_sizes,
                                                        VarCtl *vc) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        F[0] = source;
        if (level_sizes) level_sizes[0] = 1;
        vc->winners = 0ull;
        vc->edges = 0;
    }
}

__global__ __launch_bounds__(256) void var_degrees_kernel(const int32_t *row_ptr, const int32_t *F, int32_t len,
                                                          int32_t *deg) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < len; i += nth) {
        const int v = F[i];
        deg[i] = v >= 0 ? row_ptr[v + 1] - row_ptr[v] : 0;
    }
}

__global__ __launch_bounds__(BLOCK) void var_advance_kernel(VarAdvance A) {
    const int64_t E = A.offs[A.len];
    const int64_t nth = (int64_t)gridDim.x * BLOCK;
    int64_t K = (E + nth - 1) / nth;
    K = K < 1 ? 1 : (K > VAR_K ? VAR_K : K);
    const int64_t runs = (E + K - 1) / K;
    const int lane = (int)__lane_id();
    const uint32_t lvl = (uint32_t)A.next_level;
    unsigned long long wins = 0ull;
    // per wavefront (t0 is lane 0's run): every lane takes part in the ballots
    for (int64_t t0 = (int64_t)blockIdx.x * BLOCK + (threadIdx.x & ~(WAVE - 1)); t0 < runs; t0 += nth) {
        const int64_t t = t0 + lane;
        const bool has = t < runs;
        const int64_t e0 = has ? t * K : E;
        const int64_t e1 = e0 + K < E ? e0 + K : E;
        const int64_t wl = ((t0 + WAVE) * K < E ? (t0 + WAVE) * K : E) - 1;
        const int lo_w = owner_in(A.offs, 0, A.len, t0 * K);
        const int hi_w = owner_in(A.offs, lo_w, A.len, wl) + 1;
        int i = has ? owner_in(A.offs, lo_w, hi_w, e0) : 0;
        for (int q = 0; q < VAR_K; ++q) {
            const int64_t e = e0 + q;
            const bool valid = has && e < e1;
            int u = -1;
            bool won = false;
            if (valid) {
                while (A.offs[i + 1] <= e) ++i;   // frontier entries without edges are skipped
                const int v = A.F[i];
                u = A.col_idx[A.row_ptr[v] + (int)(e - A.offs[i])];
                if (A.claim == BFS_CLAIM_MIN) {
                    const uint32_t old = atomicMin(reinterpret_cast<unsigned int *>(A.dist + u), lvl);
                    won = lvl < old;
                } else {
                    const uint32_t bit = 1u << (u & 31);
                    won = !(atomicOr(A.visited + (u >> 5), bit) & bit);
                    if (won) A.dist[u] = (int32_t)lvl;
                }
                if (won && A.parent) A.parent[u] = v;
                if (A.padded) A.padded[e] = won ? u : -1;
            }
            if (A.compact) {
                const uint64_t m = __ballot(won);
                if (m) {
                    const int leader = __ffsll((unsigned long long)m) - 1;
                    unsigned long long base = 0ull;
                    if (lane == leader) base = atomicAdd(&A.vc->winners, (unsigned long long)__popcll(m));
                    base = __shfl(base, leader, WAVE);
                    if (won) A.compact[base + __popcll(m & ((1ull << lane) - 1))] = u;
                }
            } else {
                wins += won ? 1ull : 0ull;
            }
        }
    }
    if (!A.compact) {
#pragma unroll
        for (int d = WAVE / 2; d > 0; d >>= 1) wins += __shfl_xor(wins, d, WAVE);
        if (lane == 0 && wins) atomicAdd(&A.vc->winners, wins);
    }
}

// Level k's bookkeeping after its advance: stats, level size, and the two
// counters the host reads ({frontier edges, winners}); the winner count is
// cleared for the next level.
__global__ void var_record_kernel(const int32_t *offs_end, int32_t k, int8_t *st_dir, int64_t *st_fdeg,
                                  int32_t st_cap, int32_t *level_sizes, VarCtl *vc, VarCtl *out) {
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        const int64_t E = *offs_end;
        const unsigned long long w = vc->winners;
        if (k < st_cap) {
            st_dir[k] = 0;
            st_fdeg[k] = E;
        }
        if (level_sizes && w > 0) level_sizes[k + 1] = (int32_t)w;
        out->edges = E;
        out->winners = w;
        vc->winners = 0ull;
    }
}

// Flag / scan / scatter, the scan done between the two kernels: entry t of x
// is kept when it is not a sentinel (padded frontier), or vertex v is kept
// when dist[v] = level (all vertices).
__global__ __launch_bounds__(256) void var_flags_padded_kernel(const int32_t *x, int64_t len, int32_t *flag) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < len; t += nth) flag[t] = x[t] >= 0;
}

__global__ __launch_bounds__(256) void var_flags_level_kernel(const int32_t *dist, int32_t n, int32_t level,
                                                              int32_t *flag) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n; v += nth) flag[v] = dist[v] == level;
}

// out[offs[t]] = x ? x[t] : t wherever offs rises at t (the flag was set)
__global__ __launch_bounds__(256) void var_scatter_kernel(const int32_t *x, const int32_t *offs, int64_t len,
                                                          int32_t *out) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < len; t += nth)
        if (offs[t + 1] > offs[t]) out[offs[t]] = x ? x[t] : (int32_t)t;
}

int var_grid(int64_t work, int per_block) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (int)g;
}

}  // namespace

hipError_t launch_var_seed(int32_t *F, int32_t source, int32_t *level_sizes, VarCtl *vc, hipStream_t s) {
    hipLaunchKernelGGL(var_seed_kernel, dim3(1), dim3(BLOCK), 0, s, F, source, level_sizes, vc);
    return hipGetLastError();
}

hipError_t launch_var_degrees(const int32_t *row_ptr, const int32_t *F, int32_t len, int32_t *deg, hipStream_t s) {
    if (len == 0) return hipSuccess;
    hipLaunchKernelGGL(var_degrees_kernel, dim3(var_grid(len, 256 * 4)), dim3(256), 0, s, row_ptr, F, len, deg);
    return hipGetLastError();
}

hipError_t launch_var_advance(const VarAdvance &A, int grid, hipStream_t s) {
    hipLaunchKernelGGL(var_advance_kernel, dim3(grid), dim3(BLOCK), 0, s, A);
    return hipGetLastError();
}

hipError_t launch_var_record(const int32_t *offs_end, int32_t k, int8_t *st_dir, int64_t *st_fdeg, int32_t st_cap,
                             int32_t *level_sizes, VarCtl *vc, VarCtl *out, hipStream_t s) {
    hipLaunchKernelGGL(var_record_kernel, dim3(1), dim3(64), 0, s, offs_end, k, st_dir, st_fdeg, st_cap,
                       level_sizes, vc, out);
    return hipGetLastError();
}

hipError_t launch_var_compact_padded(const int32_t *x, int64_t len, int32_t *flag, int32_t *offs, int32_t *tmp,
                                     int32_t *out, hipStream_t s) {
    if (len > 0) {
        hipLaunchKernelGGL(var_flags_padded_kernel, dim3(var_grid(len, 256 * 4)), dim3(256), 0, s, x, len, flag);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipError_t e = exclusive_scan(flag, offs, len, tmp, s);
    if (e != hipSuccess || len == 0) return e;
    hipLaunchKernelGGL(var_scatter_kernel, dim3(var_grid(len, 256 * 4)), dim3(256), 0, s, x, offs, len, out);
    return hipGetLastError();
}

hipError_t launch_var_compact_level(const int32_t *dist, int32_t n, int32_t level, int32_t *flag, int32_t *offs,
                                    int32_t *tmp, int32_t *out, hipStream_t s) {
    hipLaunchKernelGGL(var_flags_level_kernel, dim3(var_grid(n, 256 * 4)), dim3(256), 0, s, dist, n, level, flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = exclusive_scan(flag, offs, n, tmp, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(var_scatter_kernel, dim3(var_grid(n, 256 * 4)), dim3(256), 0, s, nullptr, offs, (int64_t)n,
                       out);
    return hipGetLastError();
}

}  // namespace fbfs
