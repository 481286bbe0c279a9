// Single-source shortest paths on the frontier machinery: the atomic-min
// relaxation the Gunrock reading guide (step 2) carries over from BFS, where
// the winning condition becomes a strictly smaller distance.
//
// Each vertex holds one 64-bit key, (distance << 32) | predecessor, and every
// relaxation of an entry v -> u with weight w is one 64-bit atomicMin of
// ((dist(v) + w) << 32) | v into u's key.  Distance and predecessor therefore
// change together, and among the entries that reach u's shortest distance the
// smallest v stays: every v relaxes its entries again whenever its own
// distance drops, so each tight in-neighbour offers its final key.  A
// relaxation that lowers u's distance sets u's bit in the next-frontier
// bitmap; the bitmap is compacted by word popcounts, their exclusive scan and
// a scatter (the frontier in id order), each word cleared as it is read.  The
// rounds end when no distance dropped.  Distances stay below 2^32 - 1 (the
// caller bounds the weights so), and the all-ones key means unreached.
#include "bfs_internal.h"
#include "frontier_bfs.h"

namespace fbfs {

namespace {

constexpr int SSSP_K = 4;   // longest run of frontier edges per lane

__device__ __forceinline__ int owner_at(const int32_t *offs, int lo, int hi, int64_t e) {
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offs[mid] <= e) lo = mid; else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(256) void sssp_init_kernel(unsigned long long *key, uint32_t *nbm, int32_t n,
                                                        int32_t nwords, int32_t source, int32_t *F, SsspCtl *sc) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t v = tid; v < n; v += nth) key[v] = (v == source) ? (unsigned long long)source : ~0ull;
    for (int64_t w = tid; w < nwords; w += nth) nbm[w] = 0u;
    if (tid == 0) {
        F[0] = source;
        sc->err = 0;
        sc->len = 1;
    }
}

__global__ __launch_bounds__(BLOCK) void sssp_relax_kernel(SsspRelax R) {
    const int64_t E = R.offs[R.len];
    const int64_t nth = (int64_t)gridDim.x * BLOCK;
    int64_t K = (E + nth - 1) / nth;
    K = K < 1 ? 1 : (K > SSSP_K ? SSSP_K : K);
    const int64_t runs = (E + K - 1) / K;
    const int lane = (int)__lane_id();
    if (blockIdx.x == 0 && threadIdx.x == 0 && R.round < R.st_cap) {
        R.st_dir[R.round] = 0;
        R.st_fdeg[R.round] = E;
    }
    bool bad = false;
    for (int64_t t0 = (int64_t)blockIdx.x * BLOCK + (threadIdx.x & ~(WAVE - 1)); t0 < runs; t0 += nth) {
        const int64_t t = t0 + lane;
        if (t >= runs) continue;
        const int64_t e0 = t * K;
        const int64_t e1 = e0 + K < E ? e0 + K : E;
        const int64_t wl = ((t0 + WAVE) * K < E ? (t0 + WAVE) * K : E) - 1;
        const int lo_w = owner_at(R.offs, 0, R.len, t0 * K);
        const int hi_w = owner_at(R.offs, lo_w, R.len, wl) + 1;
        int i = owner_at(R.offs, lo_w, hi_w, e0);
        for (int64_t e = e0; e < e1; ++e) {
            while (R.offs[i + 1] <= e) ++i;
            const int v = R.F[i];
            const int64_t j = R.row_ptr[v] + (e - R.offs[i]);
            const int u = R.col_idx[j];
            const uint32_t w = R.weights[j];
            if (w > R.max_weight) {
                bad = true;
                continue;
            }
            if (u == R.source) continue;   // the source keeps itself as predecessor
            const uint32_t dv = (uint32_t)(R.key[v] >> 32);
            const uint32_t nd = dv + w;
            const unsigned long long nk = ((unsigned long long)nd << 32) | (uint32_t)v;
            // a plain read first: most relaxations of a heavy round lose, and
            // keys only fall, so a key already at or below nk stays so
            if (nk >= R.key[u]) continue;
            const unsigned long long old = atomicMin(R.key + u, nk);
            if (nd < (uint32_t)(old >> 32)) atomicOr(R.nbm + (u >> 5), 1u << (u & 31));
        }
    }
    if (bad) atomicOr(&R.sc->err, 1);
}

// next frontier from the bitmap: popcounts, (scan), scatter + clear
__global__ __launch_bounds__(256) void sssp_count_kernel(const uint32_t *nbm, int32_t nwords, int32_t *cnt) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwords; w += nth) cnt[w] = __popc(nbm[w]);
}

__global__ __launch_bounds__(256) void sssp_scatter_kernel(uint32_t *nbm, int32_t nwords, const int32_t *offs,
                                                           int32_t *F, SsspCtl *sc) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t w = tid; w < nwords; w += nth) {
        uint32_t bits = nbm[w];
        if (!bits) continue;
        int32_t p = offs[w];
        while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1;
            F[p++] = (int32_t)(w * 32 + b);
        }
        nbm[w] = 0u;
    }
    if (tid == 0) sc->len = offs[nwords];
}

__global__ __launch_bounds__(256) void sssp_output_kernel(const unsigned long long *key, int32_t n, int64_t *dist,
                                                          int32_t *pred) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n; v += nth) {
        const unsigned long long k = key[v];
        const bool reached = k != ~0ull;
        dist[v] = reached ? (int64_t)(k >> 32) : -1;
        if (pred) pred[v] = reached ? (int32_t)(uint32_t)(k & 0xffffffffull) : -1;
    }
}

int sssp_grid(int64_t work, int per_block) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (int)g;
}

}  // namespace

hipError_t launch_sssp_init(unsigned long long *key, uint32_t *nbm, int32_t n, int32_t nwords, int32_t source,
                            int32_t *F, SsspCtl *sc, hipStream_t s) {
    hipLaunchKernelGGL(sssp_init_kernel, dim3(sssp_grid(n > nwords ? n : nwords, 256 * 4)), dim3(256), 0, s, key,
                       nbm, n, nwords, source, F, sc);
    return hipGetLastError();
}

hipError_t launch_sssp_relax(const SsspRelax &R, int grid, hipStream_t s) {
    hipLaunchKernelGGL(sssp_relax_kernel, dim3(grid), dim3(BLOCK), 0, s, R);
    return hipGetLastError();
}

hipError_t launch_sssp_compact(uint32_t *nbm, int32_t nwords, int32_t *cnt, int32_t *offs, int32_t *tmp,
                               int32_t *F, SsspCtl *sc, hipStream_t s) {
    hipLaunchKernelGGL(sssp_count_kernel, dim3(sssp_grid(nwords, 256 * 4)), dim3(256), 0, s, nbm, nwords, cnt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = exclusive_scan(cnt, offs, nwords, tmp, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sssp_scatter_kernel, dim3(sssp_grid(nwords, 256 * 4)), dim3(256), 0, s, nbm, nwords, offs,
                       F, sc);
    return hipGetLastError();
}

hipError_t launch_sssp_output(const unsigned long long *key, int32_t n, int64_t *dist, int32_t *pred,
                              hipStream_t s) {
    hipLaunchKernelGGL(sssp_output_kernel, dim3(sssp_grid(n, 256 * 4)), dim3(256), 0, s, key, n, dist, pred);
    return hipGetLastError();
}

}  // namespace fbfs
