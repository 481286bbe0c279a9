// C ABI of the gfx950 BFS library: graph handle, validation, workspace and
// the device-resident level loop.  The interface is documented in
// include/frontier_bfs.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "bfs_internal.h"
#include "frontier_bfs.h"

using namespace fbfs;

namespace {

thread_local std::string g_err;
thread_local int32_t g_err_code = 0;

void set_error(const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
}

// bfs_last_error text for an error word the kernels recorded
void set_device_error(int32_t err, int32_t info, uint32_t barrier_ticks) {
    if (err == ERR_BARRIER_TIMEOUT)
        set_error("small-frontier barrier wait exceeded its limit (%u ticks)", barrier_ticks);
    else if (err == ERR_BAD_VERTEX)
        set_error("vertex id %d outside [0, n) met in the graph (changed after it was checked?)", info);
    else
        set_error("device reported internal error %d (info %d)", err, info);
}

struct HostCtl {
    int32_t done, L, err, err_info;
    uint8_t ran[RAN_CAP];   // the device's record of the launches that ran a level or found the end
};

}  // namespace

struct bfs_graph {
    int device = 0;
    int32_t n = 0;
    int32_t m = 0;
    const int32_t *row_ptr = nullptr;
    const int32_t *col_idx = nullptr;
    int32_t sorted = 0, symmetric = 0, max_degree = 0;
    int grid = 0;      // init and top-down launches: one full wave of workgroups
    int grid_bu = 0;   // bottom-up launches
    uint32_t *visited = nullptr, *vis_init = nullptr, *fbm0 = nullptr, *fbm1 = nullptr;
    uint32_t *cf = nullptr;        // 3 coarse frontier maps
    int32_t *pnb = nullptr;        // in-neighbour of highest out-degree of each vertex
    int4 *sreg = nullptr;          // small-frontier regions
    unsigned long long *sslot = nullptr;   // small-frontier words
    int32_t *snb = nullptr;        // ... and of second highest
    uint8_t *deg8 = nullptr;       // in-degrees in a byte (255: 255 or more)
    int32_t *in_row_ptr = nullptr, *in_col = nullptr;   // transpose (directed graphs)
    int32_t can_pull = 0;          // in-edges available
    int32_t cf_sh = 0, cf_words = 0;
    Seg *q0 = nullptr, *q1 = nullptr, *t0 = nullptr, *t1 = nullptr;
    int32_t *ts0 = nullptr, *ts1 = nullptr;
    int64_t tcap = 0, tscap = 0;
    unsigned long long *qtab = nullptr;   // queue chunk tables
    int4 *adj4 = nullptr;                 // inline short adjacencies
    uint64_t *lvbm = nullptr;             // kept per-level found bitmaps (KCAP x nwp words)
    int32_t *wscr = nullptr;              // walk scratch (binned, merge), grown on demand
    int64_t wscr_ints = 0;
    unsigned long long *ctr = nullptr;
    Ctl *ctl = nullptr;
    int8_t *st_dir = nullptr;
    int64_t *st_fdeg = nullptr;
    int32_t st_cap = 0;
    HostCtl *host_ctl = nullptr;   // pinned
    int32_t *enq = nullptr;        // debug builds: per-vertex enqueue counts of the last run
    GraphFacts *facts = nullptr;   // device, create only
    int32_t pol_dir = BFS_DIR_AUTO, pol_adv = BFS_ADV_AUTO, pol_loop = BFS_LOOP_DEVICE;
    int32_t pol_claim = BFS_CLAIM_BITMAP, pol_compact = BFS_COMPACT_DEFAULT;
    // launch kinds (1 top-down, 2 bottom-up) that cover the working launches
    // of the searches on this handle: each search's sequence of working
    // launches is a subsequence of it.  The next search enqueues it first.
    std::vector<uint8_t> plan;
    // buffers of the alternative compactions (allocated when one is chosen):
    // two frontiers, flags/degrees, their scan, scan temporaries
    int32_t *va = nullptr, *vb = nullptr, *vs = nullptr, *vo = nullptr, *vt = nullptr;
    int64_t var_cap = 0;
    VarCtl *vctl = nullptr;        // device: running counters, then the copy the host reads
    VarCtl *hvctl = nullptr;       // pinned host mirror
    // shortest-path buffers (allocated on the first bfs_sssp call)
    unsigned long long *skey = nullptr;
    uint32_t *snbm = nullptr;
    int32_t *sf0 = nullptr, *sf1 = nullptr, *scnt = nullptr, *soffs = nullptr, *stmp = nullptr;
    SsspCtl *sctl = nullptr, *hsctl = nullptr;
    int32_t alpha = ALPHA, beta = BETA;
    uint32_t barrier_ticks = 200000000u;   // 2 s at 100 MHz
    int64_t finish_min_n = FINISH_MIN_N;   // kept bitmaps and the finishing pass from this size
    int32_t last_L = 0;
    // timing hook
    int32_t timing = 0;
    int32_t last_timed = 0;
    float last_init_ms = 0.f, last_level_ms = 0.f;
    int32_t last_launches = 0;
    float last_kind_ms[2] = {0.f, 0.f};       // top-down, bottom-up launches
    int32_t last_kind_launches[2] = {0, 0};
    std::vector<hipEvent_t> events;   // [0,1] init, then one before and one after each
                                      // launch of a batch
    std::vector<float> launch_ms;     // each level launch of the last timed run
    std::vector<uint8_t> launch_ran;  // ... and the device's record of its work
};

namespace {

// a failed HIP call returns `code`, or BFS_ENOMEM when the device ran out of memory
#define HIP_TRY(expr, code)                                                              \
    do {                                                                                 \
        hipError_t e_ = (expr);                                                          \
        if (e_ != hipSuccess) {                                                          \
            set_error("%s failed: %s", #expr, hipGetErrorString(e_));                   \
            return e_ == hipErrorOutOfMemory ? BFS_ENOMEM : (code);                      \
        }                                                                                \
    } while (0)

template <typename T>
hipError_t dalloc(T **p, size_t count) {
    if (count == 0) count = 1;
    return hipMalloc(reinterpret_cast<void **>(p), count * sizeof(T));
}

void free_all(bfs_graph *g) {
    void *ptrs[] = {g->visited, g->vis_init, g->fbm0, g->fbm1, g->cf, g->pnb, g->snb, g->deg8, g->in_row_ptr, g->in_col, g->q0, g->q1, g->t0, g->t1,
                    g->ts0, g->ts1, g->ctr, g->ctl, g->st_dir, g->st_fdeg, g->facts, g->enq, g->sreg, g->sslot,
                    g->qtab, g->wscr, g->adj4, g->lvbm};
    for (void *p : ptrs)
        if (p) (void)hipFree(p);
    void *vptrs[] = {g->va, g->vb, g->vs, g->vo, g->vt, g->vctl};
    for (void *p : vptrs)
        if (p) (void)hipFree(p);
    if (g->hvctl) (void)hipHostFree(g->hvctl);
    void *sptrs[] = {g->skey, g->snbm, g->sf0, g->sf1, g->scnt, g->soffs, g->stmp, g->sctl};
    for (void *p : sptrs)
        if (p) (void)hipFree(p);
    if (g->hsctl) (void)hipHostFree(g->hsctl);
    if (g->host_ctl) (void)hipHostFree(g->host_ctl);
    for (hipEvent_t e : g->events) (void)hipEventDestroy(e);
    g->events.clear();
}

hipError_t ensure_events(bfs_graph *g, size_t count) {
    while (g->events.size() < count) {
        hipEvent_t e;
        hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) return r;
        g->events.push_back(e);
    }
    return hipSuccess;
}

int alloc_workspace(bfs_graph *g) {
    const int64_t n = g->n, m = g->m;
    const int64_t nwp = (n + 63) / 64;
    g->tcap = tile_cap(m);
    g->tscap = tstart_cap(m);
    g->st_cap = (int32_t)stats_cap(n);
    // coarse frontier map: the finest power-of-two grain that fits CF_WORDS words
    g->cf_sh = 0;
    while (((n + (1LL << g->cf_sh) - 1) >> g->cf_sh) > (int64_t)CF_WORDS * 32) ++g->cf_sh;
    g->cf_words = (int32_t)((((n + (1LL << g->cf_sh) - 1) >> g->cf_sh) + 31) / 32);
    struct {
        hipError_t e;
        const char *what;
    } r[] = {
        {dalloc(&g->visited, 2 * nwp), "visited bitmap"},
        {dalloc(&g->vis_init, 2 * nwp), "visited template"},
        {dalloc(&g->fbm0, 2 * nwp), "frontier bitmap"},
        {dalloc(&g->fbm1, 2 * nwp), "frontier bitmap"},
        {dalloc(&g->cf, 3 * (int64_t)CF_WORDS), "coarse frontier maps"},
        {dalloc(&g->pnb, n), "probe-neighbour index"},
        {dalloc(&g->snb, n), "probe-neighbour index"},
        {dalloc(&g->deg8, n), "byte degrees"},
        {dalloc(&g->adj4, n), "inline adjacencies"},
        {dalloc(&g->lvbm, n >= g->finish_min_n ? (size_t)KCAP * nwp : 1), "kept level bitmaps"},
        {dalloc(&g->q0, (size_t)queue_segs(n)), "frontier queue"},
        {dalloc(&g->q1, (size_t)queue_segs(n)), "frontier queue"},
        {dalloc(&g->qtab, (size_t)queue_tab(n)), "queue chunk tables"},
        {dalloc(&g->t0, (size_t)STRIPES * g->tcap), "tile queue"},
        {dalloc(&g->t1, (size_t)STRIPES * g->tcap), "tile queue"},
        {dalloc(&g->ts0, (size_t)NLISTS * STRIPES * g->tscap), "tile start table"},
        {dalloc(&g->ts1, (size_t)NLISTS * STRIPES * g->tscap), "tile start table"},
        {dalloc(&g->sreg, (size_t)2 * SMALL_G * SREG_CAP), "small-frontier regions"},
        {dalloc(&g->sslot, (size_t)2 * SMALL_G), "small-frontier words"},
        {dalloc(&g->ctr, (size_t)NSLOTS * NCTR * CTR_STRIDE), "counters"},
        {dalloc(&g->ctl, 1), "control block"},
        {dalloc(&g->st_dir, (size_t)g->st_cap), "level stats"},
        {dalloc(&g->st_fdeg, (size_t)g->st_cap), "level stats"},
    };
    for (auto &x : r) {
        if (x.e != hipSuccess) {
            // a failed allocation leaves HIP's last-error state set: clear it,
            // or the next launch check (this handle's or another's) reads it
            (void)hipGetLastError();
            set_error("allocating the %s for n=%d m=%d failed: %s", x.what, g->n, g->m,
                      hipGetErrorString(x.e));
            return x.e == hipErrorOutOfMemory ? BFS_ENOMEM : BFS_EHIP;
        }
    }
#ifdef FBFS_COUNT_ENQUEUES
    if (dalloc(&g->enq, n) != hipSuccess) {
        (void)hipGetLastError();
        set_error("allocating the enqueue counts for n=%d failed", g->n);
        return BFS_ENOMEM;
    }
#endif
    HIP_TRY(hipMemset(g->ctr, 0, (size_t)NSLOTS * NCTR * CTR_STRIDE * sizeof(unsigned long long)),
            BFS_EHIP);
    HIP_TRY(hipMemset(g->ctl, 0, sizeof(Ctl)), BFS_EHIP);
    HIP_TRY(hipHostMalloc(reinterpret_cast<void **>(&g->host_ctl), sizeof(HostCtl), hipHostMallocDefault),
            BFS_EHIP);
    return 0;
}

int validate_and_classify(bfs_graph *g) {
    const int32_t n = g->n;
    int32_t rp0 = -1, rpn = -1;
    HIP_TRY(hipMemcpy(&rp0, g->row_ptr, sizeof(int32_t), hipMemcpyDeviceToHost), BFS_EHIP);
    HIP_TRY(hipMemcpy(&rpn, g->row_ptr + n, sizeof(int32_t), hipMemcpyDeviceToHost), BFS_EHIP);
    if (rp0 != 0) {
        set_error("invalid CSR: row_ptr[0] = %d, expected 0", rp0);
        return BFS_EINVAL;
    }
    if (rpn < 0) {
        set_error("invalid CSR: row_ptr[%d] = %d is negative", n, rpn);
        return BFS_EINVAL;
    }
    g->m = rpn;
    if (g->m > 0 && !g->col_idx) {
        set_error("col_idx must be a device pointer when row_ptr[n] = %d > 0", g->m);
        return BFS_EINVAL;
    }
    if (dalloc(&g->facts, 1) != hipSuccess) {
        (void)hipGetLastError();
        set_error("allocating the graph facts failed");
        return BFS_ENOMEM;
    }
    GraphFacts h;
    std::memset(&h, 0, sizeof(h));
    h.bad_row = ~0ull;
    h.bad_col = ~0ull;
    HIP_TRY(hipMemcpy(g->facts, &h, sizeof(h), hipMemcpyHostToDevice), BFS_EHIP);
    HIP_TRY(launch_check_rows(g->row_ptr, n, g->facts, 0), BFS_EHIP);
    HIP_TRY(hipMemcpy(&h, g->facts, sizeof(h), hipMemcpyDeviceToHost), BFS_EHIP);
    if (h.bad_row != ~0ull) {
        set_error("invalid CSR: row_ptr is decreasing at index %llu (row_ptr[i] > row_ptr[i+1])",
                  (unsigned long long)h.bad_row);
        return BFS_EINVAL;
    }
    g->max_degree = h.max_degree;
    if (g->m > 0) {
        HIP_TRY(launch_check_cols(g->row_ptr, g->col_idx, n, g->facts, 0), BFS_EHIP);
        HIP_TRY(hipMemcpy(&h, g->facts, sizeof(h), hipMemcpyDeviceToHost), BFS_EHIP);
        if (h.bad_col != ~0ull) {
            set_error("invalid CSR: col_idx[%llu] is outside [0, %d)", (unsigned long long)h.bad_col, n);
            return BFS_EINVAL;
        }
    }
    g->sorted = h.unsorted ? 0 : 1;
    g->symmetric = 0;
    if (g->sorted) {
        if (g->m > 0) {
            HIP_TRY(launch_check_symmetry(g->row_ptr, g->col_idx, n, g->facts, 0), BFS_EHIP);
            HIP_TRY(hipMemcpy(&h, g->facts, sizeof(h), hipMemcpyDeviceToHost), BFS_EHIP);
        }
        g->symmetric = h.asymmetric ? 0 : 1;
    }
    return 0;
}

}  // namespace

// In-edges for the bottom-up pass: the CSR itself when symmetric; else its
// transpose, built on the device.  If the transpose does not fit in device
// memory the graph stays push-only (can_pull = 0) instead of failing.
hipError_t build_in_edges(bfs_graph *g) {
    if (g->symmetric) {
        g->can_pull = 1;
        return hipSuccess;
    }
    const int64_t n = g->n, m = g->m;
    int32_t *tmp = nullptr, *cnt = nullptr;
    const int64_t tmp_n = scan_tmp_ints(n);
    if (dalloc(&g->in_row_ptr, n + 1) != hipSuccess || dalloc(&g->in_col, m > 0 ? m : 1) != hipSuccess ||
        dalloc(&cnt, n) != hipSuccess || dalloc(&tmp, tmp_n) != hipSuccess) {
        (void)hipGetLastError();
        if (g->in_row_ptr) (void)hipFree(g->in_row_ptr);
        if (g->in_col) (void)hipFree(g->in_col);
        if (cnt) (void)hipFree(cnt);
        if (tmp) (void)hipFree(tmp);
        g->in_row_ptr = g->in_col = nullptr;
        g->can_pull = 0;
        return hipSuccess;
    }
    hipError_t e = hipMemset(cnt, 0, sizeof(int32_t) * n);
    if (e == hipSuccess && m > 0) e = launch_in_degree(g->col_idx, g->m, cnt, 0);
    if (e == hipSuccess) e = exclusive_scan(cnt, g->in_row_ptr, n, tmp, 0);
    // the counts become the append cursors: cnt = in_row_ptr[0, n)
    if (e == hipSuccess)
        e = hipMemcpy(cnt, g->in_row_ptr, sizeof(int32_t) * n, hipMemcpyDeviceToDevice);
    if (e == hipSuccess && m > 0) e = launch_transpose_fill(g->row_ptr, g->col_idx, g->n, cnt, g->in_col, 0);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    (void)hipFree(cnt);
    (void)hipFree(tmp);
    if (e == hipSuccess) g->can_pull = 1;
    return e;
}

// The shortest sequence holding both a and b as subsequences (a shortest
// common supersequence, by the textbook dynamic programme); b alone when that
// is more than 4 longer than b, so a plan stays close to recent searches.
std::vector<uint8_t> merge_plan(const std::vector<uint8_t> &a, const std::vector<uint8_t> &b) {
    const size_t p = a.size(), q = b.size();
    if (p == 0) return b;
    // len[i][j]: shortest supersequence of a[i..] and b[j..]
    std::vector<std::vector<int32_t>> len(p + 1, std::vector<int32_t>(q + 1, 0));
    for (size_t i = p + 1; i-- > 0;)
        for (size_t j = q + 1; j-- > 0;) {
            if (i == p) len[i][j] = (int32_t)(q - j);
            else if (j == q) len[i][j] = (int32_t)(p - i);
            else if (a[i] == b[j]) len[i][j] = 1 + len[i + 1][j + 1];
            else len[i][j] = 1 + std::min(len[i + 1][j], len[i][j + 1]);
        }
    if (len[0][0] > (int32_t)q + 4) return b;
    std::vector<uint8_t> out;
    size_t i = 0, j = 0;
    while (i < p || j < q) {
        if (i == p) out.push_back(b[j++]);
        else if (j == q) out.push_back(a[i++]);
        else if (a[i] == b[j]) { out.push_back(a[i]); ++i; ++j; }
        else if (len[i + 1][j] <= len[i][j + 1]) out.push_back(a[i++]);
        else out.push_back(b[j++]);
    }
    return out;
}

// Buffers of the alternative compactions: frontiers of up to max(n, m)
// entries (a padded frontier holds one entry per frontier edge).
int alloc_variant_buffers(bfs_graph *g) {
    if (g->va) return 0;
    const int64_t cap = (g->m > g->n ? g->m : (int64_t)g->n) + 1;
    hipError_t e = dalloc(&g->va, cap);
    if (e == hipSuccess) e = dalloc(&g->vb, cap);
    if (e == hipSuccess) e = dalloc(&g->vs, cap);
    if (e == hipSuccess) e = dalloc(&g->vo, cap + 1);
    if (e == hipSuccess) e = dalloc(&g->vt, scan_tmp_ints(cap));
    if (e == hipSuccess) e = dalloc(&g->vctl, 2);
    if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void **>(&g->hvctl), sizeof(VarCtl));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        void *vptrs[] = {g->va, g->vb, g->vs, g->vo, g->vt, g->vctl};
        for (void *p : vptrs)
            if (p) (void)hipFree(p);
        if (g->hvctl) (void)hipHostFree(g->hvctl);
        g->va = g->vb = g->vs = g->vo = g->vt = nullptr;
        g->vctl = nullptr;
        g->hvctl = nullptr;
        set_error("device allocation of the compaction buffers (5 x %lld ints) failed", (long long)cap);
        return BFS_ENOMEM;
    }
    g->var_cap = cap;
    return 0;
}

// Top-down search with the chosen claim and compaction primitives; the host
// reads {frontier edges, winners} once per level.
int32_t run_variant(bfs_graph *g, const Params &P, hipStream_t stream) {
    const bool timing = g->timing != 0;
    if (timing) {
        HIP_TRY(ensure_events(g, 3), BFS_EHIP);
        HIP_TRY(hipEventRecord(g->events[0], stream), BFS_EHIP);
    }
    {
        Params Q = P;
        Q.fill_dist = 1;   // this path has no finishing pass
        Q.l0_init = 0;     // ... and seeds level 0 itself
        HIP_TRY(launch_init(Q, g->grid, stream), BFS_EHIP);
    }
    HIP_TRY(launch_var_seed(g->va, P.source, P.level_sizes, g->vctl, stream), BFS_EHIP);
    if (timing) HIP_TRY(hipEventRecord(g->events[1], stream), BFS_EHIP);
    const int32_t mode = g->pol_compact;
    int32_t *F = g->va, *Fn = g->vb;
    int64_t len = 1;
    int32_t L = 0;
    for (int32_t k = 0;; ++k) {
        if (k >= g->n) {
            set_error("search did not terminate after %d levels", k);
            return BFS_EDEVICE;
        }
        HIP_TRY(launch_var_degrees(P.row_ptr, F, (int32_t)len, g->vs, stream), BFS_EHIP);
        HIP_TRY(exclusive_scan(g->vs, g->vo, len, g->vt, stream), BFS_EHIP);
        VarAdvance A;
        A.row_ptr = P.row_ptr;
        A.col_idx = P.col_idx;
        A.F = F;
        A.len = (int32_t)len;
        A.offs = g->vo;
        A.next_level = k + 1;
        A.claim = g->pol_claim;
        A.dist = P.dist;
        A.parent = P.parent;
        A.visited = P.visited;
        A.padded = (mode == BFS_COMPACT_PADDED || mode == BFS_COMPACT_FILTER) ? Fn : nullptr;
        A.compact = (mode == BFS_COMPACT_ATOMIC) ? Fn : nullptr;
        A.vc = g->vctl;
        HIP_TRY(launch_var_advance(A, g->grid, stream), BFS_EHIP);
        HIP_TRY(launch_var_record(g->vo + len, k, P.st_dir, P.st_fdeg, P.st_cap, P.level_sizes, g->vctl,
                                  g->vctl + 1, stream),
                BFS_EHIP);
        if (mode == BFS_COMPACT_FLAGS)
            HIP_TRY(launch_var_compact_level(P.dist, g->n, k + 1, g->vs, g->vo, g->vt, Fn, stream), BFS_EHIP);
        HIP_TRY(hipMemcpyAsync(g->hvctl, g->vctl + 1, sizeof(VarCtl), hipMemcpyDeviceToHost, stream), BFS_EHIP);
        HIP_TRY(hipStreamSynchronize(stream), BFS_EHIP);
        const int64_t E = g->hvctl->edges;
        const int64_t w = (int64_t)g->hvctl->winners;
        if (w == 0) {
            L = k + 1;
            break;
        }
        if (mode == BFS_COMPACT_FILTER) {
            // the padded frontier in Fn, compacted into the spent frontier F
            HIP_TRY(launch_var_compact_padded(Fn, E, g->vs, g->vo, g->vt, F, stream), BFS_EHIP);
            len = w;
        } else {
            len = (mode == BFS_COMPACT_PADDED) ? E : w;
            int32_t *t = F;
            F = Fn;
            Fn = t;
        }
    }
    g->last_L = L;
    g->last_timed = 0;
    if (timing) {
        HIP_TRY(hipEventRecord(g->events[2], stream), BFS_EHIP);
        HIP_TRY(hipEventSynchronize(g->events[2]), BFS_EHIP);
        float ms = 0.f;
        HIP_TRY(hipEventElapsedTime(&ms, g->events[0], g->events[1]), BFS_EHIP);
        g->last_init_ms = ms;
        HIP_TRY(hipEventElapsedTime(&ms, g->events[1], g->events[2]), BFS_EHIP);
        g->last_level_ms = ms;
        g->last_launches = L;
        g->last_kind_ms[0] = ms;
        g->last_kind_ms[1] = 0.f;
        g->last_kind_launches[0] = L;
        g->last_kind_launches[1] = 0;
        g->launch_ms.clear();
        g->launch_ran.clear();
        g->last_timed = 1;
    }
    return L;
}

int alloc_sssp_buffers(bfs_graph *g) {
    if (g->skey) return 0;
    const int64_t n = g->n, nwords = (n + 31) / 32;
    hipError_t e = dalloc(&g->skey, n);
    if (e == hipSuccess) e = dalloc(&g->snbm, nwords);
    if (e == hipSuccess) e = dalloc(&g->sf0, n);
    if (e == hipSuccess) e = dalloc(&g->sf1, n);
    if (e == hipSuccess) e = dalloc(&g->scnt, n + 1);
    if (e == hipSuccess) e = dalloc(&g->soffs, n + 1);
    if (e == hipSuccess) e = dalloc(&g->stmp, scan_tmp_ints(n + 1));
    if (e == hipSuccess) e = dalloc(&g->sctl, 1);
    if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void **>(&g->hsctl), sizeof(SsspCtl));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        void *sptrs[] = {g->skey, g->snbm, g->sf0, g->sf1, g->scnt, g->soffs, g->stmp, g->sctl};
        for (void *p : sptrs)
            if (p) (void)hipFree(p);
        if (g->hsctl) (void)hipHostFree(g->hsctl);
        g->skey = nullptr;
        g->snbm = nullptr;
        g->sf0 = g->sf1 = g->scnt = g->soffs = g->stmp = nullptr;
        g->sctl = g->hsctl = nullptr;
        set_error("device allocation of the shortest-path buffers failed");
        return BFS_ENOMEM;
    }
    return 0;
}

// ---- allocation-free search: fixed scratch in a file-scope device array ----
//
// bfs_run_noalloc searches a graph of at most NA_N vertices and NA_M CSR
// entries without a handle: its workspace (graph facts, control block,
// counters, bitmaps, probe-neighbour index, queues, tile tables, per-level
// record) is carved out of `scratch`, one array per device that lives until
// the process ends.  Host code never passes `scratch` itself to a kernel: the
// array's device address comes from hipGetSymbolAddress, once per device.
namespace {

constexpr int64_t NA_N = 1 << 16;          // most vertices
constexpr int64_t NA_M = 1 << 21;          // most CSR entries
constexpr int64_t NA_NWP = (NA_N + 63) / 64;

constexpr int64_t na_round(int64_t b) { return (b + 255) / 256 * 256; }
// byte offsets of the pieces of the scratch array
constexpr int64_t NA_FACTS = 0;
constexpr int64_t NA_CTL = NA_FACTS + na_round(sizeof(GraphFacts));
constexpr int64_t NA_CTR = NA_CTL + na_round(sizeof(Ctl));
constexpr int64_t NA_VIS = NA_CTR + na_round((int64_t)NSLOTS * NCTR * CTR_STRIDE * 8);
constexpr int64_t NA_VIS_INIT = NA_VIS + na_round(2 * NA_NWP * 4);
constexpr int64_t NA_FBM0 = NA_VIS_INIT + na_round(2 * NA_NWP * 4);
constexpr int64_t NA_FBM1 = NA_FBM0 + na_round(2 * NA_NWP * 4);
constexpr int64_t NA_CF = NA_FBM1 + na_round(2 * NA_NWP * 4);
constexpr int64_t NA_PNB = NA_CF + na_round(3 * (int64_t)CF_WORDS * 4);
constexpr int64_t NA_SNB = NA_PNB + na_round(NA_N * 4);
constexpr int64_t NA_DEG8 = NA_SNB + na_round(NA_N * 4);
constexpr int64_t NA_ADJ4 = NA_DEG8 + na_round(NA_N);
constexpr int64_t NA_Q0 = NA_ADJ4 + na_round(NA_N * 16);
constexpr int64_t NA_Q1 = NA_Q0 + na_round(queue_segs(NA_N) * (int64_t)sizeof(Seg));
constexpr int64_t NA_QTAB = NA_Q1 + na_round(queue_segs(NA_N) * (int64_t)sizeof(Seg));
constexpr int64_t NA_T0 = NA_QTAB + na_round(queue_tab(NA_N) * 8);
constexpr int64_t NA_T1 = NA_T0 + na_round(STRIPES * tile_cap(NA_M) * (int64_t)sizeof(Seg));
constexpr int64_t NA_TS0 = NA_T1 + na_round(STRIPES * tile_cap(NA_M) * (int64_t)sizeof(Seg));
constexpr int64_t NA_TS1 = NA_TS0 + na_round((int64_t)NLISTS * STRIPES * tstart_cap(NA_M) * 4);
constexpr int64_t NA_SREG = NA_TS1 + na_round((int64_t)NLISTS * STRIPES * tstart_cap(NA_M) * 4);
constexpr int64_t NA_SSLOT = NA_SREG + na_round((int64_t)2 * SMALL_G * SREG_CAP * 16);
constexpr int64_t NA_STDIR = NA_SSLOT + na_round((int64_t)2 * SMALL_G * 8);
constexpr int64_t NA_STFDEG = NA_STDIR + na_round(stats_cap(NA_N));
constexpr int64_t NA_BYTES = NA_STFDEG + na_round(stats_cap(NA_N) * 8);

}  // namespace

static __device__ __align__(256) unsigned char scratch[NA_BYTES];

namespace {

constexpr int NA_MAX_DEV = 64;
struct NaDevice {
    int ready = 0;
    unsigned char *ptr = nullptr;   // this device's copy of `scratch`
    int grid = 0, grid_bu = 0;
};
NaDevice g_na[NA_MAX_DEV];
std::mutex g_na_mu;

// Set-up on the current device, once: the scratch array's device address and
// the level kernels' grids.
int na_setup(int dev, NaDevice **out) {
    if (dev < 0 || dev >= NA_MAX_DEV) {
        set_error("device %d is beyond the %d devices the allocation-free search supports", dev, NA_MAX_DEV);
        return BFS_EINVAL;
    }
    std::lock_guard<std::mutex> lock(g_na_mu);
    NaDevice &d = g_na[dev];
    if (!d.ready) {
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            set_error("hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
            return BFS_EHIP;
        }
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        d.ptr = static_cast<unsigned char *>(p);
        d.grid = cus * level_kernel_blocks_per_cu(false);
        d.grid_bu = cus * level_kernel_blocks_per_cu(true);
        d.ready = 1;
    }
    *out = &d;
    return 0;
}

}  // namespace

extern "C" {

const char *bfs_last_error(void) { return g_err.c_str(); }

int32_t bfs_last_error_code(void) { return g_err_code; }

bfs_graph *bfs_graph_create(int32_t n, const int32_t *row_ptr, const int32_t *col_idx) {
    g_err.clear();
    g_err_code = 0;
    if (n < 1) {
        set_error("n = %d: need at least one vertex", n);
        g_err_code = BFS_EINVAL;
        return nullptr;
    }
    if (!row_ptr) {
        set_error("row_ptr must be a device pointer (got NULL)");
        g_err_code = BFS_EINVAL;
        return nullptr;
    }
    bfs_graph *g = new (std::nothrow) bfs_graph();
    if (!g) {
        set_error("host allocation failed");
        g_err_code = BFS_ENOMEM;
        return nullptr;
    }
    g->n = n;
    g->row_ptr = row_ptr;
    g->col_idx = col_idx;
    if (hipGetDevice(&g->device) != hipSuccess) {
        set_error("no HIP device");
        g_err_code = BFS_EHIP;
        delete g;
        return nullptr;
    }
    // tests lower the size from which levels keep bitmaps and a finishing
    // pass writes dist, to run that path on small graphs
    if (const char *t = getenv("FBFS_FINISH_MIN_N")) {
        const long long v = atoll(t);
        if (v >= 0) g->finish_min_n = v;
    }
    int rc = validate_and_classify(g);
    if (rc == 0) rc = alloc_workspace(g);
    if (rc == 0) {
        hipError_t e = build_in_edges(g);
        const int32_t *irp = g->symmetric ? row_ptr : g->in_row_ptr;
        const int32_t *icol = g->symmetric ? col_idx : g->in_col;
        // with in-edges at hand, vertices without any are unreachable (but for
        // the source) and start out visited
        if (e == hipSuccess) e = launch_build_vis_init(g->can_pull ? irp : row_ptr, n, g->can_pull, g->vis_init, 0);
        if (e == hipSuccess && g->can_pull) e = launch_build_probe_nb(row_ptr, irp, icol, n, g->pnb, g->snb, 0);
        if (e == hipSuccess && g->can_pull) e = launch_build_deg8(irp, n, g->deg8, 0);
        if (e == hipSuccess) e = launch_build_adj4(row_ptr, col_idx, n, g->adj4, 0);
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) {
            set_error("building the visited template, in-edges and probe-neighbour index failed: %s",
                      hipGetErrorString(e));
            rc = BFS_EHIP;
        }
    }
    if (const char *t = getenv("FBFS_BARRIER_TIMEOUT_US")) {
        const long long us = atoll(t);
        if (us >= 0) g->barrier_ticks = (uint32_t)(us * 100 < 4000000000LL ? us * 100 : 4000000000LL);
    }
    if (rc == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, g->device) != hipSuccess ||
            cus <= 0)
            cus = 256;
        g->grid = cus * level_kernel_blocks_per_cu(false);
        g->grid_bu = cus * level_kernel_blocks_per_cu(true);
    }
    if (rc != 0) {
        g_err_code = rc;
        free_all(g);
        delete g;
        return nullptr;
    }
    return g;
}

void bfs_graph_destroy(bfs_graph *g) {
    if (!g) return;
    (void)hipSetDevice(g->device);
    (void)hipDeviceSynchronize();
    free_all(g);
    delete g;
}

int32_t bfs_set_policy(bfs_graph *g, int32_t direction, int32_t advance, int32_t loop) {
    if (!g) {
        set_error("NULL graph handle");
        return BFS_EINVAL;
    }
    if (direction < BFS_DIR_AUTO || direction > BFS_DIR_PULL || advance < BFS_ADV_AUTO ||
        advance > BFS_ADV_EDGE || loop < BFS_LOOP_DEVICE || loop > BFS_LOOP_CHAIN) {
        set_error("unknown policy (direction %d, advance %d, loop %d)", direction, advance, loop);
        return BFS_EINVAL;
    }
    if (direction == BFS_DIR_PULL && !g->can_pull) {
        set_error("pull-only needs in-edges: a symmetric graph, or room for its transpose");
        return BFS_EINVAL;
    }
    g->pol_dir = direction;
    g->pol_adv = advance;
    g->pol_loop = loop;
    g->plan.clear();
    return 0;
}

int32_t bfs_set_primitives(bfs_graph *g, int32_t claim, int32_t compaction) {
    if (!g) {
        set_error("NULL graph handle");
        return BFS_EINVAL;
    }
    if (claim < BFS_CLAIM_BITMAP || claim > BFS_CLAIM_MIN || compaction < BFS_COMPACT_DEFAULT ||
        compaction > BFS_COMPACT_FLAGS) {
        set_error("unknown claim %d or compaction %d", claim, compaction);
        return BFS_EINVAL;
    }
    if (compaction == BFS_COMPACT_DEFAULT && claim != BFS_CLAIM_BITMAP) {
        set_error("the direction-optimising path claims with the visited bitmap");
        return BFS_EINVAL;
    }
    if (compaction != BFS_COMPACT_DEFAULT) {
        HIP_TRY(hipSetDevice(g->device), BFS_EHIP);
        const int rc = alloc_variant_buffers(g);
        if (rc) return rc;
    }
    g->pol_claim = claim;
    g->pol_compact = compaction;
    g->plan.clear();
    return 0;
}

int32_t bfs_set_switch(bfs_graph *g, int32_t alpha, int32_t beta) {
    if (!g) {
        set_error("NULL graph handle");
        return BFS_EINVAL;
    }
    if (alpha < 1 || alpha > 1000000 || beta < 1 || beta > 1000000) {
        set_error("switch parameters out of range (alpha %d, beta %d; each must be in [1, 1e6])",
                  alpha, beta);
        return BFS_EINVAL;
    }
    g->alpha = alpha;
    g->beta = beta;
    g->plan.clear();
    return 0;
}

int32_t bfs_run(bfs_graph *g, int32_t source, int32_t *dist_out, int32_t *parent_out,
                int32_t *level_sizes_out, hipStream_t stream) {
    g_err.clear();
    if (!g) {
        set_error("NULL graph handle");
        return BFS_EINVAL;
    }
    if (!dist_out) {
        set_error("dist_out is required");
        return BFS_EINVAL;
    }
    if (source < 0 || source >= g->n) {
        set_error("source %d is outside [0, %d)", source, g->n);
        return BFS_EINVAL;
    }
    HIP_TRY(hipSetDevice(g->device), BFS_EHIP);
    Params P;
    std::memset(&P, 0, sizeof(P));
    P.row_ptr = g->row_ptr;
    P.col_idx = g->col_idx;
    P.n = g->n;
    P.m = g->m;
    P.nwp = (int32_t)(((int64_t)g->n + 63) / 64);
    P.source = source;
    P.dist = dist_out;
    P.parent = parent_out;
    P.level_sizes = level_sizes_out;
    P.visited = g->visited;
    P.vis_init = g->vis_init;
    P.pnb = g->pnb;
    P.snb = g->snb;
    P.deg8 = g->deg8;
    P.adj4 = g->adj4;
    P.lvbm = g->lvbm;
    P.fill_dist = (g->n < g->finish_min_n) ? 1 : 0;   // else the finishing pass writes dist
    P.l0_init = g->sorted;   // level 0 may run in the init kernel (it needs sorted rows)
    P.in_row_ptr = g->symmetric ? g->row_ptr : g->in_row_ptr;
    P.in_col_idx = g->symmetric ? g->col_idx : g->in_col;
    P.can_pull = g->can_pull;
    P.fbm0 = g->fbm0;
    P.fbm1 = g->fbm1;
    P.cf = g->cf;
    P.cf_sh = g->cf_sh;
    P.cf_words = g->cf_words;
    P.q0 = g->q0;
    P.q1 = g->q1;
    P.t0 = g->t0;
    P.t1 = g->t1;
    P.ts0 = g->ts0;
    P.ts1 = g->ts1;
    P.qk_sh = qk_shift(g->n);
    P.qpool = (int32_t)queue_pool(g->n);
    P.qtab = g->qtab;
    P.tcap = g->tcap;
    P.tscap = g->tscap;
    P.ctr = g->ctr;
    P.ctl = g->ctl;
    P.st_dir = g->st_dir;
    P.st_fdeg = g->st_fdeg;
    P.st_cap = g->st_cap;
    P.symmetric = g->symmetric;
    P.col_vec = (reinterpret_cast<uintptr_t>(g->col_idx) % 16) == 0;
    P.in_col_vec = (reinterpret_cast<uintptr_t>(P.in_col_idx) % 16) == 0;
    P.pol_dir = g->pol_dir;
    P.pol_adv = g->pol_adv;
    P.small_mode = g->pol_loop == BFS_LOOP_DEVICE;
    P.alpha = g->alpha;
    P.max_deg = g->max_degree;
    P.beta = g->beta;
    P.barrier_ticks = g->barrier_ticks;
    P.enq = g->enq;
    P.sreg = g->sreg;
    P.sslot = g->sslot;

    if (g->pol_compact != BFS_COMPACT_DEFAULT) return run_variant(g, P, stream);
    const bool timing = g->timing != 0;
    g->last_timed = 0;
    if (g->n <= ONE_N && g->pol_dir == BFS_DIR_AUTO && g->pol_adv == BFS_ADV_AUTO &&
        g->pol_loop == BFS_LOOP_DEVICE) {
        // a graph this small is searched by one workgroup in one launch (its
        // timing counts as one top-down launch; the launch plan is untouched)
        if (timing) {
            HIP_TRY(ensure_events(g, 3), BFS_EHIP);
            HIP_TRY(hipEventRecord(g->events[0], stream), BFS_EHIP);
        }
        HIP_TRY(launch_one(P, stream), BFS_EHIP);
        if (timing) HIP_TRY(hipEventRecord(g->events[1], stream), BFS_EHIP);
        HIP_TRY(hipMemcpyAsync(g->host_ctl, g->ctl, sizeof(HostCtl), hipMemcpyDeviceToHost, stream), BFS_EHIP);
        HIP_TRY(hipStreamSynchronize(stream), BFS_EHIP);
        if (g->host_ctl->err) {
            set_device_error(g->host_ctl->err, g->host_ctl->err_info, g->barrier_ticks);
            return BFS_EDEVICE;
        }
        const int32_t L = g->host_ctl->L;
        g->last_L = L;
        if (timing) {
            float ms = 0.f;
            HIP_TRY(hipEventElapsedTime(&ms, g->events[0], g->events[1]), BFS_EHIP);
            g->last_init_ms = 0.f;
            g->last_level_ms = ms;
            g->last_launches = 1;
            g->last_kind_ms[0] = ms;
            g->last_kind_ms[1] = 0.f;
            g->last_kind_launches[0] = 1;
            g->last_kind_launches[1] = 0;
            g->launch_ms.assign(1, ms);
            g->launch_ran.assign(1, 1);
            g->last_timed = 1;
        }
        return L;
    }
    if (timing) HIP_TRY(ensure_events(g, 4), BFS_EHIP);
    HIP_TRY(launch_init(P, g->grid, stream, timing ? g->events[0] : nullptr, timing ? g->events[1] : nullptr),
            BFS_EHIP);
    const bool host_loop = g->pol_loop == BFS_LOOP_HOST;
    int64_t k = 0;
    // Launch kinds: searches on one graph tend to repeat their pattern of
    // directions, so the first batch is the plan (a shortest sequence that
    // holds the working launches of the recent searches in order: those that
    // ran a level or found the empty frontier; a search whose last level ran
    // in the small-frontier mode finds its end in that same launch); without
    // a plan, a batch of 12 that alternates top-down and bottom-up, which
    // covers most searches of under ten levels.  Later batches alternate.  A
    // launch whose level belongs to the other direction passes it on, so the
    // order only costs time, never results.
    const std::vector<uint8_t> plan = host_loop ? std::vector<uint8_t>() : g->plan;
    const int64_t prefix = (int64_t)plan.size();
    int64_t batch = host_loop ? 1 : (prefix ? prefix : 12);
    bool prev_bu = true;   // so that alternation starts top-down
    std::vector<uint8_t> kinds;
    float level_ms = 0.f, kind_ms[2] = {0.f, 0.f}, finish_ms = 0.f;
    int32_t kind_launches[2] = {0, 0};
    g->launch_ms.clear();
    g->launch_ran.clear();
    // outside the prefix, launches alternate top-down and bottom-up; each pair
    // runs at least one level or finds the empty frontier, and L <= n, so
    // launch prefix + 2n + 1 has found it
    const int64_t kmax = 2 * (int64_t)g->n + 2 + prefix;
    for (;;) {
        const int64_t k0 = k;
        kinds.clear();
        // timing: launch i of the batch records events 2+2i and 3+2i as its
        // kernel begins and ends, the finishing pass the next two
        if (timing) HIP_TRY(ensure_events(g, 2 + 2 * (size_t)batch + 2), BFS_EHIP);
        for (int64_t i = 0; i < batch && k <= kmax; ++i, ++k) {
            const bool bu = k < prefix ? (k < (int64_t)plan.size() && plan[k] == 2) : !prev_bu;
            prev_bu = bu;
            kinds.push_back(bu ? 1 : 0);
            HIP_TRY(launch_level(P, (int32_t)k, bu, bu ? g->grid_bu : g->grid, stream,   // k = launch index
                                 timing ? g->events[2 + 2 * i] : nullptr, timing ? g->events[3 + 2 * i] : nullptr),
                    BFS_EHIP);
        }
        // the finishing pass writes dist once the search is done (it does
        // nothing after a batch that leaves the search running)
        if (!P.fill_dist) {
            const int64_t j = k - k0;
            HIP_TRY(launch_finish(P, stream, timing ? g->events[2 + 2 * j] : nullptr,
                                  timing ? g->events[3 + 2 * j] : nullptr),
                    BFS_EHIP);
        }
        HIP_TRY(hipMemcpyAsync(g->host_ctl, g->ctl, sizeof(HostCtl), hipMemcpyDeviceToHost, stream),
                BFS_EHIP);
        HIP_TRY(hipStreamSynchronize(stream), BFS_EHIP);
        if (timing) {
            for (int64_t i = 0; i < k - k0; ++i) {
                float ms = 0.f;
                HIP_TRY(hipEventElapsedTime(&ms, g->events[2 + 2 * i], g->events[3 + 2 * i]), BFS_EHIP);
                level_ms += ms;
                kind_ms[kinds[i]] += ms;
                kind_launches[kinds[i]] += 1;
                g->launch_ms.push_back(ms);
            }
            if (!P.fill_dist) {
                float ms = 0.f;
                HIP_TRY(hipEventElapsedTime(&ms, g->events[2 + 2 * (k - k0)], g->events[3 + 2 * (k - k0)]), BFS_EHIP);
                finish_ms += ms;
            }
        }
        const HostCtl &h = *g->host_ctl;
        if (h.err) {
            g->plan.clear();
            set_device_error(h.err, h.err_info, g->barrier_ticks);
            return BFS_EDEVICE;
        }
        if (h.done) {
            g->last_L = h.L;
            // this search's working launches, merged into the plan
            if (host_loop || k > RAN_CAP) {
                g->plan.clear();
            } else {
                std::vector<uint8_t> seq;
                for (int64_t i = 0; i < k; ++i)
                    if (h.ran[i]) seq.push_back(h.ran[i]);
                g->plan = merge_plan(g->plan, seq);
            }
            if (timing) {
                float ms = 0.f;
                HIP_TRY(hipEventElapsedTime(&ms, g->events[0], g->events[1]), BFS_EHIP);
                g->last_init_ms = ms + finish_ms;   // the init kernel and the finishing pass
                g->last_level_ms = level_ms;
                g->last_launches = (int32_t)k;
                for (int t = 0; t < 2; ++t) {
                    g->last_kind_ms[t] = kind_ms[t];
                    g->last_kind_launches[t] = kind_launches[t];
                }
                for (int64_t i = 0; i < k; ++i) g->launch_ran.push_back(i < RAN_CAP ? h.ran[i] : 0);
                g->last_timed = 1;
            }
            return h.L;
        }
        if (k > kmax) {
            g->plan.clear();
            set_error("search did not terminate after %lld level launches", (long long)k);
            return BFS_EDEVICE;
        }
        if (!host_loop && batch < 1024) batch = batch < 12 ? 12 : batch * 2;
    }
}

int32_t bfs_run_noalloc(int32_t n, const int32_t *row_ptr, const int32_t *col_idx, int32_t source,
                        int32_t *dist_out, int32_t *parent_out, int32_t *level_sizes_out, hipStream_t stream) {
    g_err.clear();
    if (n < 1 || n > NA_N) {
        set_error("n = %d is outside [1, %lld], the allocation-free search's limit", n, (long long)NA_N);
        return BFS_EINVAL;
    }
    if (!row_ptr || !dist_out) {
        set_error("row_ptr and dist_out must be device pointers");
        return BFS_EINVAL;
    }
    if (source < 0 || source >= n) {
        set_error("source %d is outside [0, %d)", source, n);
        return BFS_EINVAL;
    }
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev), BFS_EHIP);
    NaDevice *d = nullptr;
    {
        const int rc = na_setup(dev, &d);
        if (rc) return rc;
    }
    unsigned char *base = d->ptr;
    GraphFacts *facts = reinterpret_cast<GraphFacts *>(base + NA_FACTS);
    // the graph, checked as bfs_graph_create checks it
    int32_t ends[2] = {-1, -1};
    HIP_TRY(hipMemcpyAsync(&ends[0], row_ptr, sizeof(int32_t), hipMemcpyDeviceToHost, stream), BFS_EHIP);
    HIP_TRY(hipMemcpyAsync(&ends[1], row_ptr + n, sizeof(int32_t), hipMemcpyDeviceToHost, stream), BFS_EHIP);
    HIP_TRY(hipStreamSynchronize(stream), BFS_EHIP);
    if (ends[0] != 0) {
        set_error("invalid CSR: row_ptr[0] = %d, expected 0", ends[0]);
        return BFS_EINVAL;
    }
    if (ends[1] < 0 || ends[1] > NA_M) {
        set_error("row_ptr[%d] = %d: the allocation-free search takes 0 to %lld CSR entries", n, ends[1],
                  (long long)NA_M);
        return BFS_EINVAL;
    }
    const int32_t m = ends[1];
    if (m > 0 && !col_idx) {
        set_error("col_idx must be a device pointer when row_ptr[n] = %d > 0", m);
        return BFS_EINVAL;
    }
    GraphFacts h;
    HIP_TRY(launch_facts_reset(facts, stream), BFS_EHIP);
    HIP_TRY(launch_check_rows(row_ptr, n, facts, stream), BFS_EHIP);
    HIP_TRY(hipMemcpyAsync(&h, facts, sizeof(h), hipMemcpyDeviceToHost, stream), BFS_EHIP);
    HIP_TRY(hipStreamSynchronize(stream), BFS_EHIP);
    if (h.bad_row != ~0ull) {
        set_error("invalid CSR: row_ptr is decreasing at index %llu (row_ptr[i] > row_ptr[i+1])",
                  (unsigned long long)h.bad_row);
        return BFS_EINVAL;
    }
    if (m > 0) {
        HIP_TRY(launch_check_cols(row_ptr, col_idx, n, facts, stream), BFS_EHIP);
        HIP_TRY(hipMemcpyAsync(&h, facts, sizeof(h), hipMemcpyDeviceToHost, stream), BFS_EHIP);
        HIP_TRY(hipStreamSynchronize(stream), BFS_EHIP);
        if (h.bad_col != ~0ull) {
            set_error("invalid CSR: col_idx[%llu] is outside [0, %d)", (unsigned long long)h.bad_col, n);
            return BFS_EINVAL;
        }
        if (!h.unsorted) {
            HIP_TRY(launch_check_symmetry(row_ptr, col_idx, n, facts, stream), BFS_EHIP);
            HIP_TRY(hipMemcpyAsync(&h, facts, sizeof(h), hipMemcpyDeviceToHost, stream), BFS_EHIP);
            HIP_TRY(hipStreamSynchronize(stream), BFS_EHIP);
        }
    }
    // pull needs in-edges: a symmetric graph is its own; any other graph is
    // searched push-only here (no room for a transpose)
    const int32_t symmetric = (!h.unsorted && !h.asymmetric) ? 1 : 0;
    const int64_t nwp = ((int64_t)n + 63) / 64;
    Params P;
    std::memset(&P, 0, sizeof(P));
    P.row_ptr = row_ptr;
    P.col_idx = col_idx;
    P.n = n;
    P.m = m;
    P.nwp = (int32_t)nwp;
    P.source = source;
    P.dist = dist_out;
    P.parent = parent_out;
    P.level_sizes = level_sizes_out;
    P.visited = reinterpret_cast<uint32_t *>(base + NA_VIS);
    P.vis_init = reinterpret_cast<uint32_t *>(base + NA_VIS_INIT);
    P.pnb = reinterpret_cast<int32_t *>(base + NA_PNB);
    P.snb = reinterpret_cast<int32_t *>(base + NA_SNB);
    P.deg8 = reinterpret_cast<uint8_t *>(base + NA_DEG8);
    P.adj4 = reinterpret_cast<int4 *>(base + NA_ADJ4);
    // graphs this small keep no level bitmaps: the init kernel fills dist
    static_assert(NA_N < FINISH_MIN_N, "the allocation-free search has no kept bitmaps");
    P.lvbm = nullptr;
    P.fill_dist = 1;
    P.l0_init = h.unsorted ? 0 : 1;
    P.in_row_ptr = symmetric ? row_ptr : nullptr;
    P.in_col_idx = symmetric ? col_idx : nullptr;
    P.can_pull = symmetric;
    P.fbm0 = reinterpret_cast<uint32_t *>(base + NA_FBM0);
    P.fbm1 = reinterpret_cast<uint32_t *>(base + NA_FBM1);
    P.cf = reinterpret_cast<uint32_t *>(base + NA_CF);
    P.cf_sh = 0;
    while ((((int64_t)n + (1LL << P.cf_sh) - 1) >> P.cf_sh) > (int64_t)CF_WORDS * 32) ++P.cf_sh;
    P.cf_words = (int32_t)(((((int64_t)n + (1LL << P.cf_sh) - 1) >> P.cf_sh) + 31) / 32);
    P.q0 = reinterpret_cast<Seg *>(base + NA_Q0);
    P.q1 = reinterpret_cast<Seg *>(base + NA_Q1);
    P.t0 = reinterpret_cast<Seg *>(base + NA_T0);
    P.t1 = reinterpret_cast<Seg *>(base + NA_T1);
    P.ts0 = reinterpret_cast<int32_t *>(base + NA_TS0);
    P.ts1 = reinterpret_cast<int32_t *>(base + NA_TS1);
    P.qk_sh = qk_shift(n);
    P.qpool = (int32_t)queue_pool(n);
    P.qtab = reinterpret_cast<unsigned long long *>(base + NA_QTAB);
    P.tcap = tile_cap(m);
    P.tscap = tstart_cap(m);
    P.ctr = reinterpret_cast<unsigned long long *>(base + NA_CTR);
    P.ctl = reinterpret_cast<Ctl *>(base + NA_CTL);
    P.sreg = reinterpret_cast<int4 *>(base + NA_SREG);
    P.sslot = reinterpret_cast<unsigned long long *>(base + NA_SSLOT);
    P.st_dir = reinterpret_cast<int8_t *>(base + NA_STDIR);
    P.st_fdeg = reinterpret_cast<int64_t *>(base + NA_STFDEG);
    P.st_cap = (int32_t)stats_cap(n);
    P.symmetric = symmetric;
    P.col_vec = (reinterpret_cast<uintptr_t>(col_idx) % 16) == 0;
    P.in_col_vec = symmetric && P.col_vec;
    P.pol_dir = BFS_DIR_AUTO;
    P.pol_adv = BFS_ADV_AUTO;
    P.small_mode = 1;
    P.alpha = ALPHA;
    P.beta = BETA;
    P.max_deg = h.max_degree;
    P.barrier_ticks = 200000000u;   // 2 s at 100 MHz, as a handle's default
    // the graph-derived tables a handle builds at creation
    HIP_TRY(launch_build_vis_init(row_ptr, n, symmetric, reinterpret_cast<uint32_t *>(base + NA_VIS_INIT),
                                  stream), BFS_EHIP);
    if (symmetric) {
        HIP_TRY(launch_build_probe_nb(row_ptr, row_ptr, col_idx, n, reinterpret_cast<int32_t *>(base + NA_PNB),
                                      reinterpret_cast<int32_t *>(base + NA_SNB), stream), BFS_EHIP);
        HIP_TRY(launch_build_deg8(row_ptr, n, reinterpret_cast<uint8_t *>(base + NA_DEG8), stream), BFS_EHIP);
    }
    HIP_TRY(launch_build_adj4(row_ptr, col_idx, n, reinterpret_cast<int4 *>(base + NA_ADJ4), stream), BFS_EHIP);
    int32_t hc[4] = {0, 0, 0, 0};   // done, L, err, err_info
    if (n <= ONE_N) {
        HIP_TRY(launch_one(P, stream), BFS_EHIP);
        HIP_TRY(hipMemcpyAsync(hc, P.ctl, sizeof(hc), hipMemcpyDeviceToHost, stream), BFS_EHIP);
        HIP_TRY(hipStreamSynchronize(stream), BFS_EHIP);
        if (hc[2]) {
            set_device_error(hc[2], hc[3], P.barrier_ticks);
            return BFS_EDEVICE;
        }
        return hc[1];
    }
    HIP_TRY(launch_init(P, d->grid, stream), BFS_EHIP);
    // the level launches as in bfs_run's default loop, without a learnt plan:
    // batches that alternate top-down and bottom-up (top-down only when the
    // graph cannot pull), growing from 12 to 1024 launches
    const int64_t kmax = 2 * (int64_t)n + 2;
    int64_t k = 0, batch = 12;
    bool prev_bu = true;
    for (;;) {
        for (int64_t i = 0; i < batch && k <= kmax; ++i, ++k) {
            const bool bu = symmetric ? !prev_bu : false;
            prev_bu = bu;
            HIP_TRY(launch_level(P, (int32_t)k, bu, bu ? d->grid_bu : d->grid, stream), BFS_EHIP);
        }
        HIP_TRY(hipMemcpyAsync(hc, P.ctl, sizeof(hc), hipMemcpyDeviceToHost, stream), BFS_EHIP);
        HIP_TRY(hipStreamSynchronize(stream), BFS_EHIP);
        if (hc[2]) {
            set_device_error(hc[2], hc[3], P.barrier_ticks);
            return BFS_EDEVICE;
        }
        if (hc[0]) return hc[1];
        if (k > kmax) {
            set_error("search did not terminate after %lld level launches", (long long)k);
            return BFS_EDEVICE;
        }
        if (batch < 1024) batch *= 2;
    }
}

int32_t bfs_walk_level(bfs_graph *g, const int32_t *vertices, int32_t count, int32_t mapping,
                       int32_t repeats, uint32_t *out, hipStream_t stream) {
    g_err.clear();
    if (!g) {
        set_error("NULL graph handle");
        return BFS_EINVAL;
    }
    if (count < 0 || repeats < 0) {
        set_error("count (%d) and repeats (%d) must not be negative", count, repeats);
        return BFS_EINVAL;
    }
    if (mapping < BFS_WALK_LANE || mapping > BFS_WALK_MERGE) {
        set_error("unknown walk mapping %d", mapping);
        return BFS_EINVAL;
    }
    if (count > 0 && (!vertices || !out)) {
        set_error("vertices and out must be device pointers");
        return BFS_EINVAL;
    }
    if ((int64_t)count > 8 * (int64_t)g->n) {
        set_error("count %d is above the walk's limit of 8n = %lld", count, 8LL * g->n);
        return BFS_EINVAL;
    }
    HIP_TRY(hipSetDevice(g->device), BFS_EHIP);
    // the binned and merge mappings' scratch: a buffer of the handle, grown on demand
    if ((mapping == BFS_WALK_BINNED || mapping == BFS_WALK_MERGE) && walk_scratch_ints(count) > g->wscr_ints) {
        HIP_TRY(hipDeviceSynchronize(), BFS_EHIP);   // a walk still running may use the old one
        if (g->wscr) (void)hipFree(g->wscr);
        g->wscr = nullptr;
        g->wscr_ints = 0;
        if (dalloc(&g->wscr, (size_t)walk_scratch_ints(count)) != hipSuccess) {
            (void)hipGetLastError();
            g->wscr = nullptr;
            set_error("allocating the walk scratch for count %d failed", count);
            return BFS_ENOMEM;
        }
        g->wscr_ints = walk_scratch_ints(count);
    }
    Params P;
    std::memset(&P, 0, sizeof(P));
    P.row_ptr = g->row_ptr;
    P.col_idx = g->col_idx;
    P.n = g->n;
    P.m = g->m;
    int32_t *bad = &g->ctl->err;
    const bool timing = g->timing != 0;
    g->last_timed = 0;
    HIP_TRY(hipMemsetAsync(bad, 0, sizeof(int32_t), stream), BFS_EHIP);
    if (timing) {
        HIP_TRY(ensure_events(g, 2), BFS_EHIP);
        HIP_TRY(hipEventRecord(g->events[0], stream), BFS_EHIP);
    }
    HIP_TRY(launch_walk(P, vertices, count, mapping, repeats, out, g->wscr, bad,
                        g->grid, stream),
            BFS_EHIP);
    if (timing) HIP_TRY(hipEventRecord(g->events[1], stream), BFS_EHIP);
    HIP_TRY(hipMemcpyAsync(g->host_ctl, g->ctl, sizeof(HostCtl), hipMemcpyDeviceToHost, stream), BFS_EHIP);
    HIP_TRY(hipStreamSynchronize(stream), BFS_EHIP);
    if (g->host_ctl->err) {
        set_error("a listed vertex is outside [0, %d)", g->n);
        return BFS_EINVAL;
    }
    if (timing) {
        float ms = 0.f;
        HIP_TRY(hipEventElapsedTime(&ms, g->events[0], g->events[1]), BFS_EHIP);
        g->last_init_ms = 0.f;
        g->last_level_ms = ms;
        g->last_launches = 1;
        g->last_kind_ms[0] = g->last_kind_ms[1] = 0.f;
        g->last_kind_launches[0] = g->last_kind_launches[1] = 0;
        g->launch_ms.clear();
        g->launch_ran.clear();
        g->last_timed = 1;
    }
    return 0;
}

int32_t bfs_sssp(bfs_graph *g, int32_t source, const uint32_t *weights, uint32_t max_weight,
                 int64_t *dist_out, int32_t *pred_out, hipStream_t stream) {
    g_err.clear();
    if (!g) {
        set_error("NULL graph handle");
        return BFS_EINVAL;
    }
    if (!dist_out || (g->m > 0 && !weights)) {
        set_error("dist_out and weights must be device pointers");
        return BFS_EINVAL;
    }
    if (source < 0 || source >= g->n) {
        set_error("source %d is outside [0, %d)", source, g->n);
        return BFS_EINVAL;
    }
    if ((uint64_t)g->n * (uint64_t)max_weight >= 0xffffffffull) {
        set_error("n * max_weight = %llu does not stay below 2^32 - 1",
                  (unsigned long long)g->n * (unsigned long long)max_weight);
        return BFS_EINVAL;
    }
    HIP_TRY(hipSetDevice(g->device), BFS_EHIP);
    {
        const int rc = alloc_sssp_buffers(g);
        if (rc) return rc;
    }
    const int32_t n = g->n, nwords = (int32_t)(((int64_t)n + 31) / 32);
    const bool timing = g->timing != 0;
    g->last_timed = 0;
    if (timing) {
        HIP_TRY(ensure_events(g, 2), BFS_EHIP);
        HIP_TRY(hipEventRecord(g->events[0], stream), BFS_EHIP);
    }
    HIP_TRY(launch_sssp_init(g->skey, g->snbm, n, nwords, source, g->sf0, g->sctl, stream), BFS_EHIP);
    int32_t *F = g->sf0, *Fn = g->sf1;
    int64_t len = 1;
    int32_t rounds = 0;
    for (;;) {
        if (rounds > n) {
            set_error("shortest paths did not settle after %d rounds", rounds);
            return BFS_EDEVICE;
        }
        ++rounds;
        HIP_TRY(launch_var_degrees(g->row_ptr, F, (int32_t)len, g->scnt, stream), BFS_EHIP);
        HIP_TRY(exclusive_scan(g->scnt, g->soffs, len, g->stmp, stream), BFS_EHIP);
        SsspRelax R;
        R.row_ptr = g->row_ptr;
        R.col_idx = g->col_idx;
        R.weights = weights;
        R.max_weight = max_weight;
        R.source = source;
        R.F = F;
        R.len = (int32_t)len;
        R.offs = g->soffs;
        R.key = g->skey;
        R.nbm = g->snbm;
        R.sc = g->sctl;
        R.round = rounds - 1;
        R.st_dir = g->st_dir;
        R.st_fdeg = g->st_fdeg;
        R.st_cap = g->st_cap;
        HIP_TRY(launch_sssp_relax(R, g->grid, stream), BFS_EHIP);
        HIP_TRY(launch_sssp_compact(g->snbm, nwords, g->scnt, g->soffs, g->stmp, Fn, g->sctl, stream), BFS_EHIP);
        HIP_TRY(hipMemcpyAsync(g->hsctl, g->sctl, sizeof(SsspCtl), hipMemcpyDeviceToHost, stream), BFS_EHIP);
        HIP_TRY(hipStreamSynchronize(stream), BFS_EHIP);
        if (g->hsctl->err) {
            set_error("an edge weight is above max_weight = %u", max_weight);
            return BFS_EINVAL;
        }
        len = g->hsctl->len;
        if (len == 0) break;
        int32_t *t = F;
        F = Fn;
        Fn = t;
    }
    HIP_TRY(launch_sssp_output(g->skey, n, dist_out, pred_out, stream), BFS_EHIP);
    g->last_L = rounds;   // bfs_last_run_stats: the frontier edges of each round
    if (timing) {
        HIP_TRY(hipEventRecord(g->events[1], stream), BFS_EHIP);
        HIP_TRY(hipEventSynchronize(g->events[1]), BFS_EHIP);
        float ms = 0.f;
        HIP_TRY(hipEventElapsedTime(&ms, g->events[0], g->events[1]), BFS_EHIP);
        g->last_init_ms = 0.f;
        g->last_level_ms = ms;
        g->last_launches = rounds;
        g->last_kind_ms[0] = ms;
        g->last_kind_ms[1] = 0.f;
        g->last_kind_launches[0] = rounds;
        g->last_kind_launches[1] = 0;
        g->launch_ms.clear();
        g->launch_ran.clear();
        g->last_timed = 1;
    }
    HIP_TRY(hipStreamSynchronize(stream), BFS_EHIP);
    return rounds;
}

int32_t bfs_last_run_stats(const bfs_graph *g, int32_t cap, int8_t *dir, int64_t *frontier_edges) {
    if (!g || cap < 0) {
        set_error("NULL graph handle or negative capacity");
        return BFS_EINVAL;
    }
    int64_t cnt = g->last_L;
    if (cnt > cap) cnt = cap;
    if (cnt > g->st_cap) cnt = g->st_cap;
    if (cnt > 0 && dir) {
        HIP_TRY(hipMemcpy(dir, g->st_dir, (size_t)cnt, hipMemcpyDeviceToHost), BFS_EHIP);
        for (int64_t k = 0; k < cnt; ++k) dir[k] &= 1;   // the level flags sit above bit 0
    }
    if (cnt > 0 && frontier_edges)
        HIP_TRY(hipMemcpy(frontier_edges, g->st_fdeg, (size_t)cnt * sizeof(int64_t), hipMemcpyDeviceToHost),
                BFS_EHIP);
    return g->last_L;
}

int32_t bfs_last_run_level_flags(const bfs_graph *g, int32_t cap, uint8_t *flags) {
    if (!g || cap < 0) {
        set_error("NULL graph handle or negative capacity");
        return BFS_EINVAL;
    }
    int64_t cnt = g->last_L;
    if (cnt > cap) cnt = cap;
    if (cnt > g->st_cap) cnt = g->st_cap;
    if (cnt > 0 && flags) {
        HIP_TRY(hipMemcpy(flags, g->st_dir, (size_t)cnt, hipMemcpyDeviceToHost), BFS_EHIP);
        for (int64_t k = 0; k < cnt; ++k) flags[k] = (uint8_t)((flags[k] >> 1) & 31);
    }
    return g->last_L;
}

int32_t bfs_set_timing(bfs_graph *g, int32_t on) {
    if (!g) {
        set_error("NULL graph handle");
        return BFS_EINVAL;
    }
    g->timing = on ? 1 : 0;
    return 0;
}

int32_t bfs_last_run_kernel_timing(const bfs_graph *g, float *td_ms, int32_t *td_launches,
                                   float *bu_ms, int32_t *bu_launches) {
    if (!g || !g->last_timed) {
        set_error(g ? "the last run was not timed (bfs_set_timing)" : "NULL graph handle");
        return BFS_EINVAL;
    }
    if (td_ms) *td_ms = g->last_kind_ms[0];
    if (td_launches) *td_launches = g->last_kind_launches[0];
    if (bu_ms) *bu_ms = g->last_kind_ms[1];
    if (bu_launches) *bu_launches = g->last_kind_launches[1];
    return 0;
}

int32_t bfs_debug_enqueue_counts(const bfs_graph *g, int32_t *counts_out) {
    if (!g || !counts_out) {
        set_error("NULL graph handle or output");
        return BFS_EINVAL;
    }
#ifdef FBFS_COUNT_ENQUEUES
    HIP_TRY(hipSetDevice(g->device), BFS_EHIP);
    HIP_TRY(hipMemcpy(counts_out, g->enq, sizeof(int32_t) * (size_t)g->n, hipMemcpyDeviceToDevice), BFS_EHIP);
    return 0;
#else
    set_error("this build does not count enqueues (build with -DFBFS_COUNT_ENQUEUES)");
    return BFS_EINVAL;
#endif
}

int32_t bfs_last_run_launch_timing(const bfs_graph *g, int32_t cap, float *ms, uint8_t *ran) {
    if (!g || !g->last_timed || cap < 0) {
        set_error(g ? (cap < 0 ? "negative capacity" : "the last run was not timed (bfs_set_timing)")
                    : "NULL graph handle");
        return BFS_EINVAL;
    }
    const int64_t cnt = (int64_t)g->launch_ms.size();
    for (int64_t i = 0; i < cnt && i < cap; ++i) {
        if (ms) ms[i] = g->launch_ms[i];
        if (ran) ran[i] = i < (int64_t)g->launch_ran.size() ? g->launch_ran[i] : 0;
    }
    return (int32_t)cnt;
}

int32_t bfs_last_run_timing(const bfs_graph *g, float *init_ms, float *level_ms,
                            int32_t *level_launches) {
    if (!g || !g->last_timed) {
        set_error(g ? "the last run was not timed (bfs_set_timing)" : "NULL graph handle");
        return BFS_EINVAL;
    }
    if (init_ms) *init_ms = g->last_init_ms;
    if (level_ms) *level_ms = g->last_level_ms;
    if (level_launches) *level_launches = g->last_launches;
    return 0;
}

int32_t bfs_graph_info(const bfs_graph *g, int64_t *m, int32_t *sorted_rows, int32_t *symmetric,
                       int32_t *max_degree, int32_t *pull_ready) {
    if (!g) {
        set_error("NULL graph handle");
        return BFS_EINVAL;
    }
    if (m) *m = g->m;
    if (sorted_rows) *sorted_rows = g->sorted;
    if (symmetric) *symmetric = g->symmetric;
    if (max_degree) *max_degree = g->max_degree;
    if (pull_ready) *pull_ready = g->can_pull;
    return 0;
}

}  // extern "C"
