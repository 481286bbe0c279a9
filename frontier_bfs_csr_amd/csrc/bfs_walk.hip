// Isolated neighbour walk of one level on gfx950: the measurement the "Day 38 -
// Graph traversal on a GPU" page uses to compare thread-to-work mappings
// without the atomics, the frontier build and the distance writes of a real
// level ("Measuring the mapping without measuring the launch").  For every
// listed vertex u the walk returns the wrapping unsigned sum, over repeats r
// and over u's CSR entries, of (neighbour id XOR r); the XOR keeps the inner
// sum from being loop invariant, and unsigned wrap makes every addition order
// give the same value, so each mapping is checked bit-exactly.
//
// Mappings (the degree classes of the PMPP chapter 15 notes, section 15.7, and
// of the Gunrock reading guide, step 4; the edge-balanced partition of its
// step 5):
//   lane     one lane walks a whole list;
//   wave     a 64-lane wavefront strides a list and reduces with shuffles;
//   binned   the level's lists are first sorted into three bins by degree
//            (under T_LANE entries, under T_WG, longer); then a lane walks
//            each list of the first bin, a wavefront each of the second and a
//            whole workgroup each of the third;
//   merge    the exclusive scan of the listed degrees splits all entries into
//            short runs of consecutive entries (one per lane on thin levels, up
//            to WALK_MERGE_K on heavy ones), handed to lanes in order
//            (grid-stride), so the runs of one wavefront sit side by side and
//            stay in L1 across the repeats; a lane finds the owner of its first
//            entry by binary search ("the last scan entry not greater than e")
//            inside the bracket of its wavefront's first and last owners; the
//            first pieces of the lanes' runs are summed per owner across the
//            wavefront (a segmented shuffle reduction), and every other piece
//            goes to its owner's sum with one atomic.
#include "bfs_internal.h"
#include "frontier_bfs.h"

namespace fbfs {

namespace {

__device__ __forceinline__ int lane_of() { return (int)__lane_id(); }

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
#pragma unroll
    for (int d = WAVE / 2; d > 0; d >>= 1) x += __shfl_xor(x, d, WAVE);
    return x;
}

// The walk of one list piece [b, e) for every repeat, from one lane.  The
// entry loop is unrolled by four so that a lane keeps four loads in flight
// (rolled, it waits out each load's latency before issuing the next).
__device__ __forceinline__ uint32_t walk_run(const int32_t *col_idx, int b, int e, int stride,
                                             int repeats) {
    uint32_t acc = 0u;
    for (int r = 0; r < repeats; ++r) {
#pragma unroll 4
        for (int j = b; j < e; j += stride) acc += (uint32_t)col_idx[j] ^ (uint32_t)r;
    }
    return acc;
}

// Adjacency bounds of listed vertex i; an id outside [0, n) walks nothing and
// raises the error flag.
__device__ __forceinline__ void bounds_of(const int32_t *row_ptr, const int32_t *vs, int64_t i,
                                          int32_t n, int32_t *bad, int &b, int &e) {
    const int u = vs[i];
    if (u < 0 || u >= n) {
        atomicOr(bad, 1);
        b = e = 0;
        return;
    }
    b = row_ptr[u];
    e = row_ptr[u + 1];
}

__global__ __launch_bounds__(BLOCK) void walk_lane_kernel(const int32_t *row_ptr,
                                                          const int32_t *col_idx, int32_t n,
                                                          const int32_t *vs, int32_t count,
                                                          int32_t repeats, uint32_t *out,
                                                          int32_t *bad) {
    const int64_t nth = (int64_t)gridDim.x * BLOCK;
    for (int64_t i = (int64_t)blockIdx.x * BLOCK + threadIdx.x; i < count; i += nth) {
        int b, e;
        bounds_of(row_ptr, vs, i, n, bad, b, e);
        out[i] = walk_run(col_idx, b, e, 1, repeats);
    }
}

__global__ __launch_bounds__(BLOCK) void walk_wave_kernel(const int32_t *row_ptr,
                                                          const int32_t *col_idx, int32_t n,
                                                          const int32_t *vs, int32_t count,
                                                          int32_t repeats, uint32_t *out,
                                                          int32_t *bad) {
    const int lane = lane_of();
    const int64_t nw = (int64_t)gridDim.x * WAVES;
    // the loop bound is the same for every lane of a wavefront: the loads are
    // guarded, the shuffle reduction never is
    for (int64_t i = (int64_t)blockIdx.x * WAVES + threadIdx.x / WAVE; i < count; i += nw) {
        int b, e;
        bounds_of(row_ptr, vs, i, n, bad, b, e);
        const uint32_t acc = wave_sum_u32(walk_run(col_idx, b + lane, e, WAVE, repeats));
        if (lane == 0) out[i] = acc;
    }
}

// Degree bins of the whole level: listed vertex i goes to the lane bin
// (degree < T_LANE), the wavefront bin (< T_WG) or the workgroup bin, each a
// compact list of indexes (cnt[0..2] entries).  Appends are aggregated per
// wavefront: one atomic per bin and wavefront.  An id outside [0, n) walks
// nothing: its sum is written as 0 here and it joins no bin.
__global__ __launch_bounds__(BLOCK) void walk_bin_kernel(const int32_t *row_ptr, int32_t n,
                                                         const int32_t *vs, int32_t count,
                                                         int32_t *bins, int32_t *cnt, uint32_t *out,
                                                         int32_t *bad) {
    const int lane = lane_of();
    const int64_t nth = (int64_t)gridDim.x * BLOCK;
    // the loop runs per wavefront, so every lane takes part in the ballots
    for (int64_t i0 = (int64_t)blockIdx.x * BLOCK + (threadIdx.x & ~(WAVE - 1)); i0 < count; i0 += nth) {
        const int64_t i = i0 + lane;
        int bin = -1;
        if (i < count) {
            int b, e;
            bounds_of(row_ptr, vs, i, n, bad, b, e);
            const int u = vs[i];
            if (u < 0 || u >= n) out[i] = 0u;
            else bin = e - b < T_LANE ? 0 : (e - b < T_WG ? 1 : 2);
        }
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const uint64_t mm = __ballot(bin == k);
            if (!mm) continue;
            int base = 0;
            if (lane == __ffsll((unsigned long long)mm) - 1) base = atomicAdd(&cnt[k], __popcll(mm));
            base = __shfl(base, __ffsll((unsigned long long)mm) - 1, WAVE);
            if (bin == k)
                bins[(int64_t)k * count + base + __popcll(mm & ((1ull << lane) - 1))] = (int32_t)i;
        }
    }
}

// Walk of the three bins, each with its own mapping across the whole grid:
// a workgroup per list of the workgroup bin, then a wavefront per list of the
// wavefront bin, then a lane per list of the lane bin.  Every list has one
// owner, so each sum is written once, without atomics.
__global__ __launch_bounds__(BLOCK) void walk_binned_kernel(const int32_t *row_ptr,
                                                            const int32_t *col_idx,
                                                            const int32_t *vs, int32_t count,
                                                            const int32_t *bins, const int32_t *cnt,
                                                            int32_t repeats, uint32_t *out) {
    __shared__ uint32_t red[WAVES];
    const int lane = lane_of();
    const int wv = threadIdx.x / WAVE;
    const int32_t *lane_bin = bins, *wave_bin = bins + count, *wg_bin = bins + 2 * (int64_t)count;
    const int n_lane = cnt[0], n_wave = cnt[1], n_wg = cnt[2];
    for (int k = blockIdx.x; k < n_wg; k += gridDim.x) {
        const int i = wg_bin[k];
        const int u = vs[i];
        const uint32_t acc = wave_sum_u32(walk_run(col_idx, row_ptr[u] + (int)threadIdx.x, row_ptr[u + 1],
                                                   BLOCK, repeats));
        if (lane == 0) red[wv] = acc;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t t = 0u;
            for (int w = 0; w < WAVES; ++w) t += red[w];
            out[i] = t;
        }
        __syncthreads();
    }
    const int64_t gw = (int64_t)blockIdx.x * WAVES + wv, nw = (int64_t)gridDim.x * WAVES;
    for (int64_t k = gw; k < n_wave; k += nw) {
        const int i = wave_bin[k];
        const int u = vs[i];
        const uint32_t acc = wave_sum_u32(walk_run(col_idx, row_ptr[u] + lane, row_ptr[u + 1], WAVE, repeats));
        if (lane == 0) out[i] = acc;
    }
    const int64_t nth = (int64_t)gridDim.x * BLOCK;
    for (int64_t k = (int64_t)blockIdx.x * BLOCK + threadIdx.x; k < n_lane; k += nth) {
        const int i = lane_bin[k];
        const int u = vs[i];
        out[i] = walk_run(col_idx, row_ptr[u], row_ptr[u + 1], 1, repeats);
    }
}

// Degrees of the listed vertices, for the scan of the merge mapping; the
// output is cleared for its atomics on the way.
__global__ __launch_bounds__(256) void walk_degrees_kernel(const int32_t *row_ptr, int32_t n,
                                                           const int32_t *vs, int32_t count,
                                                           int32_t *deg, uint32_t *out,
                                                           int32_t *bad) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += nth) {
        int b, e;
        bounds_of(row_ptr, vs, i, n, bad, b, e);
        deg[i] = e - b;
        out[i] = 0u;
    }
}

// Owner of entry e among listed vertices [lo, hi): the last one whose scan
// entry is not greater than e (offs[lo] <= e < offs[hi] on entry).
__device__ __forceinline__ int owner_of(const int32_t *offs, int lo, int hi, int64_t e) {
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offs[mid] <= e) lo = mid; else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(BLOCK) void walk_merge_kernel(const int32_t *row_ptr,
                                                           const int32_t *col_idx, int32_t n,
                                                           const int32_t *vs, int32_t count,
                                                           const int32_t *offs, int32_t repeats,
                                                           uint32_t *out) {
    const int64_t E = offs[count];
    const int64_t nth = (int64_t)gridDim.x * BLOCK;
    // run length: one entry per lane while the level is thinner than the
    // grid, longer runs (at most WALK_MERGE_K) on heavier levels
    int64_t K = (E + nth - 1) / nth;
    K = K < 1 ? 1 : (K > WALK_MERGE_K ? WALK_MERGE_K : K);
    const int64_t runs = (E + K - 1) / K;
    const int lane = lane_of();
    // the loop runs per wavefront (t0 is lane 0's run), so the shuffles below
    // always see all 64 lanes; lanes past the last run carry no entries
    for (int64_t t0 = (int64_t)blockIdx.x * BLOCK + (threadIdx.x & ~(WAVE - 1)); t0 < runs; t0 += nth) {
        const int64_t t = t0 + lane;
        const bool has = t < runs;
        const int64_t e0 = has ? t * K : E;
        const int64_t e1 = e0 + K < E ? e0 + K : E;
        // the wavefront's runs are consecutive: bracket them by the owners of
        // the wavefront's first and last entries, then search inside
        const int64_t wl = ((t0 + WAVE) * K < E ? (t0 + WAVE) * K : E) - 1;
        const int lo_w = owner_of(offs, 0, count, t0 * K);
        const int hi_w = owner_of(offs, lo_w, count, wl) + 1;
        int i = has ? owner_of(offs, lo_w, hi_w, e0) : -1;
        // first segment of the run: summed over the lanes that share its owner
        // (owners never decrease across the lanes), one atomic per owner
        const int own = i;
        uint32_t first = 0u;
        int64_t e = e0;
        if (has) {
            const int64_t seg_end = offs[i + 1] < e1 ? offs[i + 1] : e1;
            const int u = vs[i];
            if (u >= 0 && u < n) {
                const int b = row_ptr[u] + (int)(e - offs[i]);
                first = walk_run(col_idx, b, b + (int)(seg_end - e), 1, repeats);
            }
            e = seg_end;
            ++i;
        }
#pragma unroll
        for (int d = 1; d < WAVE; d <<= 1) {
            const uint32_t v = __shfl_down(first, d, WAVE);
            const int o = __shfl_down(own, d, WAVE);
            if (lane + d < WAVE && o == own) first += v;
        }
        const int prev = __shfl_up(own, 1, WAVE);
        if (has && (lane == 0 || prev != own) && first) atomicAdd(&out[own], first);
        // the rest of the run: whole lists and the head of the next one
        while (e < e1) {
            const int64_t seg_end = offs[i + 1] < e1 ? offs[i + 1] : e1;
            const int u = vs[i];
            if (u >= 0 && u < n && seg_end > e) {
                const int b = row_ptr[u] + (int)(e - offs[i]);
                atomicAdd(&out[i], walk_run(col_idx, b, b + (int)(seg_end - e), 1, repeats));
            }
            e = seg_end;
            ++i;
        }
    }
}

int walk_grid(int64_t work, int per_block) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (int)g;
}

}  // namespace

// merge: degrees (count), scan (count + 1), scan temporaries; binned: three
// bins of count entries and their counters
int64_t walk_scratch_ints(int64_t count) { return 3 * count + 4 + scan_tmp_ints(count); }

hipError_t launch_walk(const Params &P, const int32_t *vs, int32_t count, int32_t mapping,
                       int32_t repeats, uint32_t *out, int32_t *scratch, int32_t *bad,
                       int lanes_grid, hipStream_t s) {
    if (count == 0) return hipSuccess;
    switch (mapping) {
    case BFS_WALK_LANE:
        hipLaunchKernelGGL(walk_lane_kernel, dim3(walk_grid(count, BLOCK)), dim3(BLOCK), 0, s, P.row_ptr,
                           P.col_idx, P.n, vs, count, repeats, out, bad);
        break;
    case BFS_WALK_WAVE:
        hipLaunchKernelGGL(walk_wave_kernel, dim3(walk_grid(count, WAVES)), dim3(BLOCK), 0, s, P.row_ptr,
                           P.col_idx, P.n, vs, count, repeats, out, bad);
        break;
    case BFS_WALK_BINNED: {
        int32_t *bins = scratch, *cnt = scratch + 3 * (int64_t)count;
        hipError_t e = hipMemsetAsync(cnt, 0, 3 * sizeof(int32_t), s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(walk_bin_kernel, dim3(walk_grid(count, BLOCK)), dim3(BLOCK), 0, s, P.row_ptr, P.n,
                           vs, count, bins, cnt, out, bad);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(walk_binned_kernel, dim3(lanes_grid), dim3(BLOCK), 0, s, P.row_ptr, P.col_idx, vs,
                           count, bins, cnt, repeats, out);
        break;
    }
    case BFS_WALK_MERGE: {
        // scratch: degrees (count), scan (count + 1), scan temporaries
        int32_t *deg = scratch, *offs = scratch + count, *tmp = scratch + 2 * (int64_t)count + 1;
        hipLaunchKernelGGL(walk_degrees_kernel, dim3(walk_grid(count, 256)), dim3(256), 0, s, P.row_ptr,
                           P.n, vs, count, deg, out, bad);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = exclusive_scan(deg, offs, count, tmp, s);
        if (e != hipSuccess) return e;
        // the run count is known on the device only: a grid that fills the
        // chip, and the loop over runs takes the rest
        hipLaunchKernelGGL(walk_merge_kernel, dim3(lanes_grid), dim3(BLOCK), 0, s, P.row_ptr, P.col_idx,
                           P.n, vs, count, offs, repeats, out);
        break;
    }
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fbfs
