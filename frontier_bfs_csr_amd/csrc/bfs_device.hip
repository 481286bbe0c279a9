// gfx950 kernels for level-synchronous, frontier-based BFS over an int32 CSR
// graph.  One launch initialises a search; then one launch of
// bfs_level_kernel runs one level.  Every level launch reads the frontier
// counters left in device memory by the previous launch, decides the
// direction itself and exits at once after the search has ended, so the host
// can enqueue launches ahead without learning anything per level (the per-level
// launch plus device-to-host count copy of bfs.cu's runBfs, in "Day 38 - Graph
// traversal on a GPU", is what this removes).
//
// Per level, every workgroup computes the same decision from the counters:
//   * top-down (push): expand every frontier vertex's adjacency list; a
//     neighbour is claimed by atomicOr on the visited bitmap (exactly one
//     winner), and the winner writes dist/parent (Chapter 22, sections 22.1
//     and 22.2: a compare-and-swap style claim gives one discovery per vertex);
//   * bottom-up (pull): every unvisited vertex scans its list for a neighbour
//     in the frontier bitmap (PMPP ch.15 notes, sections 15.3 and 15.7; Gunrock
//     reading guide, step 6: dense frontier, no atomics, no duplicates).
// The PMPP ch.15 notes (section 15.7) switch to pull when |F| * (m/n) > |U|.
// Counting vertices misjudges power-law frontiers, whose few hubs carry most
// of the edges, so the switch here counts edges, which the frontier counters
// give exactly: pull when sum deg(F) > (edges of unvisited vertices) / ALPHA,
// back to push when |F| < n / BETA and shrinking (Beamer, Asanovic and
// Patterson, "Direction-Optimizing Breadth-First Search", SC 2012).
//
// Top-down advance (PMPP ch.15 notes, section 15.7 and Gunrock reading guide,
// step 4: degree classes of one thread / one warp / one block):
//   degree < T_LANE          one lane walks the list,
//   T_LANE <= degree < T_WG  one 64-lane wavefront strides the list (coalesced),
//   degree >= T_WG           the list is cut into TILE-edge pieces when the
//                            vertex enters the frontier, one workgroup per
//                            piece, so a hub spreads over many workgroups.
// Edge-balanced variant (Gunrock reading guide, steps 4 and 5; Day 38 page,
// exercise): every frontier segment carries its offset in the frontier-degree
// exclusive scan, and the start segment of every EB_TE-edge tile is recorded
// when the frontier is built; a workgroup takes a tile, stages the tile's
// segment offsets in LDS and each lane finds the owner of its edge by binary
// search ("the last scan entry not greater than e").
//
// New frontier vertices are staged in LDS with wavefront ballot / mbcnt ranks
// and written out with one global atomic per workgroup flush per list (PMPP
// ch.15 notes, section 15.6, privatised queue -- without its overflow drop:
// a full LDS buffer spills to a direct global append instead).
#include "bfs_internal.h"
#include "frontier_bfs.h"

namespace fbfs {

// --------------------------------------------------------------- helpers ----

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x / WAVE); }

__device__ __forceinline__ int mbcnt64(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ int readlane_i(int x, int lane) {
    return __builtin_amdgcn_readlane(x, lane);
}

__device__ __forceinline__ unsigned long long *ctr_at(const Params &P, int slot, int idx) {
    return P.ctr + ((size_t)slot * NCTR + (size_t)idx) * CTR_STRIDE;
}

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
        uint64_t y = __shfl_up(x, (unsigned)d, WAVE);
        if (lane >= d) x += y;
    }
    return x;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T x) {
#pragma unroll
    for (int d = WAVE / 2; d > 0; d >>= 1) x += __shfl_xor(x, d, WAVE);
    return x;
}

// ---------------------------------------------------------- LDS layout -----

// Shared state of one level launch.  The work area is used by one pass at a
// time: the frontier list of the from-bitmap pass or the segment table of the
// edge-balanced pass.
constexpr int WORK_INTS = 3 * (EB_TE + 1);
constexpr int FLIST_CAP = 4 * BLOCK;     // from-bitmap pass: 4 word pairs per wave per round
static_assert(FLIST_CAP <= WORK_INTS, "work area too small");

struct LevelShared {
    union {
        struct {                          // top-down passes
            int32_t buf[CAP];             // staged new frontier vertices
            int32_t work[WORK_INTS];
            int32_t big_v[BLOCK], big_beg[BLOCK], big_len[BLOCK];
            int32_t tstart[CAP], toff[CAP];   // flush: piece start / edge offset of each staged slot
        };
        struct {                          // bottom-up pass, per wavefront
            int32_t bu_lst[WAVES][BU_GP * 64];     // unvisited vertices of the group
            unsigned long long bu_fm[WAVES][BU_GP];  // found masks per word pair
            unsigned long long bu_vis[WAVES][BU_GP]; // visited words per word pair
        };
    };
    int32_t ntiles;
    uint64_t scan_tmp[3][WAVES];
    unsigned long long list_base[NLISTS];
    int32_t cnt;                      // staged count (may exceed CAP: overflow spilled)
    int32_t nbig;
    int32_t fcnt;                     // from-bitmap list count
    // decision, identical in every workgroup
    int32_t mode;                     // 0 exit, 1 finish, 2 run
    int32_t dir, input_bm, wbits, clear_bm, adv_eb, small;
    int32_t fsize;
    int64_t fdeg, reached_before, edges_before;
    int32_t lcount[NLISTS * STRIPES];  // segments per (list, stripe)
    int32_t ledges[NLISTS * STRIPES];  // edges per (list, stripe)
    int32_t uprefix[NLISTS * STRIPES + 1];  // unit prefix (binned or edge-balanced)
};

// Per-thread context of one level launch.
struct Ctx {
    const Params *P;
    LevelShared *sh;
    int32_t level;          // k: new vertices get k+1
    int32_t wg, G;          // this workgroup's index among the G taking part
    int32_t stripe;         // counter / queue stripe of this workgroup
    int32_t nslot;          // slot of level k+1
    int32_t wbits;
    uint32_t *nbm;          // bitmap of level k+1 (top-down with wbits)
    Seg *nq, *nt;           // queues of level k+1
    int32_t *nts;
    // per-thread tallies of new frontier vertices
    int32_t fcnt;
    int64_t fdeg;
};

// --------------------------------------------------------- emission --------

// Where segment `idx` of list `l`, stripe `s` lives.
__device__ __forceinline__ Seg *seg_slot(const Params &P, Seg *q, Seg *t, int l, int s, int64_t idx) {
    if (l == L_SMALL) return q + (size_t)s * P.qcap + idx;
    if (l == L_MID) return q + (size_t)s * P.qcap + (P.qcap - 1 - idx);
    return t + (size_t)s * P.tcap + idx;
}

__device__ __forceinline__ void set_err(const Params &P, int code, int info) {
    atomicCAS(&P.ctl->err, 0, code);
    P.ctl->err_info = info;
}

// Writes one segment (vertex v, adjacency piece [pb, pb+pl), edge offset po)
// at index si of list l and records the edge-balanced tiles whose first edge
// falls inside it.
__device__ __forceinline__ void write_piece(const Ctx &c, int l, int64_t si, int v, int pb, int pl,
                                            int64_t po) {
    const Params &P = *c.P;
    const int64_t cap = (l == L_TILE) ? P.tcap : P.qcap;
    if (si >= cap) { set_err(P, l == L_TILE ? ERR_TILE_OVERFLOW : ERR_QUEUE_OVERFLOW, (int)l); return; }
    Seg sg;
    sg.v = v; sg.beg = pb; sg.len = pl; sg.off = (int32_t)po;
    *seg_slot(P, c.nq, c.nt, l, c.stripe, si) = sg;
    int32_t *ts = c.nts + (size_t)(l * STRIPES + c.stripe) * P.tscap;
    int64_t t0 = (po + EB_TE - 1) / EB_TE;
    const int64_t t1 = (po + pl - 1) / EB_TE;
    for (; t0 <= t1; ++t0) {
        if (t0 >= P.tscap) { set_err(P, ERR_TSTART_OVERFLOW, (int)l); return; }
        ts[t0] = (int32_t)si;
    }
}

// Writes the segments of one new frontier vertex v (adjacency [beg, beg+len),
// cut into TILE pieces for list L_TILE) at segment index `idx` and edge
// offset `eoff` of list l.
__device__ __forceinline__ void write_vertex_segments(const Ctx &c, int l, int v, int beg, int len,
                                                      int64_t idx, int64_t eoff) {
    const int nseg = (l == L_TILE) ? (len + TILE - 1) / TILE : 1;
    for (int j = 0; j < nseg; ++j) {
        const int pb = (l == L_TILE) ? beg + j * TILE : beg;
        const int pl = (l == L_TILE) ? min(TILE, len - j * TILE) : len;
        write_piece(c, l, idx + j, v, pb, pl, eoff + (int64_t)j * TILE);
    }
}

__device__ __forceinline__ int list_of(int len) {
    return len <= 0 ? -1 : (len < T_LANE ? L_SMALL : (len < T_WG ? L_MID : L_TILE));
}

// One vertex, one lane: used when the LDS staging buffer is full (the
// expansion loops flush often enough that this is rare).
__device__ __forceinline__ void emit_single(Ctx &c, int v) {
    const Params &P = *c.P;
    const int beg = P.row_ptr[v];
    const int len = P.row_ptr[v + 1] - beg;
    c.fcnt += 1;
    c.fdeg += len;
    const int l = list_of(len);
    if (l < 0) return;
    const int nseg = (l == L_TILE) ? (len + TILE - 1) / TILE : 1;
    unsigned long long add = ((unsigned long long)nseg << 32) | (unsigned)len;
    unsigned long long base = atomicAdd(ctr_at(P, c.nslot, l * STRIPES + c.stripe), add);
    write_vertex_segments(c, l, v, beg, len, (int64_t)(base >> 32), (int64_t)(base & 0xffffffffull));
}

// Stage a winner in LDS (wave-aggregated LDS atomic, rank by mbcnt).
__device__ __forceinline__ void stage(Ctx &c, bool win, int v) {
    const uint64_t m = __ballot(win);
    if (m == 0) return;
    const int leader = __ffsll((unsigned long long)m) - 1;
    int base = 0;
    if (lane_id() == leader) base = atomicAdd(&c.sh->cnt, __popcll(m));
    base = readlane_i(base, leader);
    bool spill = false;
    if (win) {
        const int slot = base + mbcnt64(m);
        if (slot < CAP) c.sh->buf[slot] = v;
        else spill = true;
    }
    // the lanes that found the buffer full append their vertex directly
    if (spill) emit_single(c, v);
}

// Claim up to N targets (v[q] valid where ok[q], reached from u[q]) for
// level k+1: filter on plain loads of the visited words, then one atomicOr per
// remaining target decides its single winner.  The N loads and the N atomics
// are each issued before any result is used, so a lane keeps N claims in
// flight instead of one.
constexpr int CB = 4;

template <int N>
__device__ __forceinline__ void claim_batch(Ctx &c, const int (&v)[N], const bool (&ok)[N],
                                            const int (&u)[N]) {
    constexpr int CB = N;
    const Params &P = *c.P;
    uint32_t w[CB];
#pragma unroll
    for (int q = 0; q < CB; ++q) w[q] = ok[q] ? P.visited[v[q] >> 5] : ~0u;
    bool tryq[CB];
#pragma unroll
    for (int q = 0; q < CB; ++q) tryq[q] = ok[q] && !((w[q] >> (v[q] & 31)) & 1u);
    uint32_t old[CB];
#pragma unroll
    for (int q = 0; q < CB; ++q)
        old[q] = tryq[q] ? atomicOr(P.visited + (v[q] >> 5), 1u << (v[q] & 31)) : ~0u;
    bool win[CB];
#pragma unroll
    for (int q = 0; q < CB; ++q) {
        win[q] = tryq[q] && !((old[q] >> (v[q] & 31)) & 1u);
        if (win[q]) {
            P.dist[v[q]] = c.level + 1;
            if (P.parent) P.parent[v[q]] = u[q];
            if (c.wbits) atomicOr(c.nbm + (v[q] >> 5), 1u << (v[q] & 31));
        }
    }
#pragma unroll
    for (int q = 0; q < CB; ++q) stage(c, win[q], v[q]);
}

// Claims for entries e0, e0+stride, ... (N of them) of col_idx below `end`.
template <int N = CB>
__device__ __forceinline__ void claim_run(Ctx &c, int e0, int stride, int end, int u) {
    constexpr int CB = N;
    const Params &P = *c.P;
    int v[CB], uu[CB];
    bool ok[CB];
#pragma unroll
    for (int q = 0; q < CB; ++q) {
        const int e = e0 + q * stride;
        ok[q] = e < end;
        v[q] = ok[q] ? P.col_idx[e] : 0;
        uu[q] = u;
    }
    claim_batch(c, v, ok, uu);
}

// Workgroup flush of the staged vertices: one global atomic per list per
// flush (exclusive scans of (segments, edges) give every vertex its place).
// Two passes over the thread's staged slots -- tally, then write -- keep
// few registers live; the second pass re-reads row_ptr entries the first one
// just loaded.
__device__ __forceinline__ void flush(Ctx &c) {
    LevelShared &sh = *c.sh;
    const Params &P = *c.P;
    __syncthreads();
    const int cnt = min(sh.cnt, CAP);
    constexpr int EPT = CAP / BLOCK;
    const int i0 = threadIdx.x * EPT;
    uint64_t tot0 = 0, tot1 = 0, tot2 = 0;
    for (int i = i0; i < min(i0 + EPT, cnt); ++i) {
        const int v = sh.buf[i];
        const int beg = P.row_ptr[v];
        const int len = P.row_ptr[v + 1] - beg;
        c.fcnt += 1;
        c.fdeg += len;
        const int l = list_of(len);
        if (l == L_SMALL) tot0 += (1ull << 32) | (uint32_t)len;
        else if (l == L_MID) tot1 += (1ull << 32) | (uint32_t)len;
        else if (l == L_TILE) tot2 += ((uint64_t)((len + TILE - 1) / TILE) << 32) | (uint32_t)len;
    }
    // exclusive scans of the per-thread totals, one per list
    const uint64_t in0 = wave_incl_scan_u64(tot0);
    const uint64_t in1 = wave_incl_scan_u64(tot1);
    const uint64_t in2 = wave_incl_scan_u64(tot2);
    if (lane_id() == WAVE - 1) {
        sh.scan_tmp[0][wave_id()] = in0;
        sh.scan_tmp[1][wave_id()] = in1;
        sh.scan_tmp[2][wave_id()] = in2;
    }
    __syncthreads();
    uint64_t ex0 = in0 - tot0, ex1 = in1 - tot1, ex2 = in2 - tot2;
    for (int w = 0; w < wave_id(); ++w) {
        ex0 += sh.scan_tmp[0][w];
        ex1 += sh.scan_tmp[1][w];
        ex2 += sh.scan_tmp[2][w];
    }
    if (threadIdx.x < NLISTS) {
        const int l = threadIdx.x;
        uint64_t all = 0;
        for (int w = 0; w < WAVES; ++w) all += sh.scan_tmp[l][w];
        if (all != 0)
            sh.list_base[l] = atomicAdd(ctr_at(P, c.nslot, l * STRIPES + c.stripe), (unsigned long long)all);
        if (l == L_TILE) sh.ntiles = (int32_t)(all >> 32);
    }
    __syncthreads();
    // small and mid vertices: one segment each, written by their thread; big
    // vertices: record where their pieces start, then the whole workgroup
    // writes the pieces (a hub can have hundreds)
    const uint64_t b0 = sh.list_base[L_SMALL], b1 = sh.list_base[L_MID];
    for (int i = i0; i < min(i0 + EPT, cnt); ++i) {
        const int v = sh.buf[i];
        const int beg = P.row_ptr[v];
        const int len = P.row_ptr[v + 1] - beg;
        const int l = list_of(len);
        sh.tstart[i] = (int32_t)(ex2 >> 32);
        sh.toff[i] = (int32_t)(ex2 & 0xffffffffull);
        if (l == L_SMALL) {
            write_piece(c, l, (int64_t)((b0 >> 32) + (ex0 >> 32)), v, beg, len,
                        (int64_t)((b0 & 0xffffffffull) + (ex0 & 0xffffffffull)));
            ex0 += (1ull << 32) | (uint32_t)len;
        } else if (l == L_MID) {
            write_piece(c, l, (int64_t)((b1 >> 32) + (ex1 >> 32)), v, beg, len,
                        (int64_t)((b1 & 0xffffffffull) + (ex1 & 0xffffffffull)));
            ex1 += (1ull << 32) | (uint32_t)len;
        } else if (l == L_TILE) {
            ex2 += ((uint64_t)((len + TILE - 1) / TILE) << 32) | (uint32_t)len;
        }
    }
    __syncthreads();
    const int ntiles = sh.ntiles;
    if (ntiles > 0) {
        const uint64_t base = sh.list_base[L_TILE];
        const int64_t tbase = (int64_t)(base >> 32);
        const int64_t ebase = (int64_t)(base & 0xffffffffull);
        for (int gt = threadIdx.x; gt < ntiles; gt += BLOCK) {
            // last staged slot whose pieces start at or before gt
            int lo = 0, hi = cnt;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (sh.tstart[mid] <= gt) lo = mid; else hi = mid;
            }
            const int v = sh.buf[lo];
            const int beg = P.row_ptr[v];
            const int len = P.row_ptr[v + 1] - beg;
            const int pcs = gt - sh.tstart[lo];
            write_piece(c, L_TILE, tbase + gt, v, beg + pcs * TILE, min(TILE, len - pcs * TILE),
                        ebase + sh.toff[lo] + (int64_t)pcs * TILE);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) sh.cnt = 0;
    __syncthreads();
}

__device__ __forceinline__ void maybe_flush(Ctx &c) {
    // callers reach this from uniform control flow, after a barrier; every
    // thread reads the count before any thread can stage more vertices
    const int cnt = c.sh->cnt;
    __syncthreads();
    if (cnt >= CAP / 2) flush(c);
}

// -------------------------------------------------------- top-down ---------

// Expand the segments held by the threads of the workgroup (at most one per
// thread): lane, wavefront or workgroup mapping by length.  Ends with a barrier.
__device__ __forceinline__ void expand_segments(Ctx &c, bool has, int v, int beg, int len) {
    LevelShared &sh = *c.sh;
    // lane bin: CB consecutive entries per step
    if (has && len < T_LANE) {
        for (int e = beg; e < beg + len; e += CB) claim_run(c, e, 1, beg + len, v);
    }
    // wavefront bin: lanes stride the list, CB entries per lane per step
    uint64_t mm = __ballot(has && len >= T_LANE && len < T_WG);
    while (mm) {
        const int src = __ffsll((unsigned long long)mm) - 1;
        mm &= mm - 1;
        const int sv = readlane_i(v, src), sb = readlane_i(beg, src), sl = readlane_i(len, src);
        for (int e = lane_id(); e < sl; e += CB * WAVE) claim_run(c, sb + e, WAVE, sb + sl, sv);
    }
    // workgroup bin
    if (has && len >= T_WG) {
        const int i = atomicAdd(&sh.nbig, 1);
        sh.big_v[i] = v; sh.big_beg[i] = beg; sh.big_len[i] = len;
    }
    __syncthreads();
    const int nbig = sh.nbig;
    for (int i = 0; i < nbig; ++i) {
        const int bv = sh.big_v[i], bb = sh.big_beg[i], bl = sh.big_len[i];
        // steps of STEP_CLAIMS entries, each followed by a flush check: a
        // hub cannot overfill the staging buffer
        for (int e0 = 0; e0 < bl; e0 += STEP_CLAIMS) {
            __syncthreads();    // the previous step's staging is done
            maybe_flush(c);
            claim_run<STEP_CLAIMS / BLOCK>(c, bb + e0 + (int)threadIdx.x, BLOCK, bb + bl, bv);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) sh.nbig = 0;
    __syncthreads();
}

// Top-down from the queue lists, degree-binned: tiles (one per unit), then
// mid segments (one per wavefront, WAVES per unit), then small segments (one
// per lane, BLOCK per unit); units are dealt round-robin to workgroups.
__device__ __forceinline__ void td_binned(Ctx &c, const Seg *cq, const Seg *ct, uint32_t *cbm) {
    const Params &P = *c.P;
    LevelShared &sh = *c.sh;
    const int total = sh.uprefix[NLISTS * STRIPES];
    for (int u = c.wg; u < total; u += c.G) {
        // find (list, stripe) region of unit u
        int r = 0;
        while (sh.uprefix[r + 1] <= u) ++r;
        const int l = r / STRIPES, s = r % STRIPES;
        const int ui = u - sh.uprefix[r];
        const int nseg = sh.lcount[r];
        bool has = false;
        int64_t si = -1;
        if (l == L_TILE) {
            if (threadIdx.x == 0) si = ui;
        } else if (l == L_MID) {
            if (lane_id() == 0) si = (int64_t)ui * WAVES + wave_id();
        } else {
            si = (int64_t)ui * BLOCK + threadIdx.x;
        }
        int v = 0, beg = 0, len = 0;
        if (si >= 0 && si < nseg) {
            const Seg sg = *seg_slot(P, const_cast<Seg *>(cq), const_cast<Seg *>(ct), l, s, si);
            v = sg.v; beg = sg.beg; len = sg.len;
            has = true;
            if (c.sh->clear_bm) cbm[v >> 5] = 0u;
        }
        expand_segments(c, has, v, beg, len);
        maybe_flush(c);
    }
}

// Top-down, edge-balanced: tiles of EB_TE edges over each (list, stripe)
// region's edge range; the region's frontier-degree scan (Seg::off) and tile
// start table locate the segments; each lane binary-searches its edge's owner.
__device__ __forceinline__ void td_edge_balanced(Ctx &c, const Seg *cq, const Seg *ct, const int32_t *cts,
                                 uint32_t *cbm) {
    const Params &P = *c.P;
    LevelShared &sh = *c.sh;
    int32_t *s_off = sh.work;
    int32_t *s_v = sh.work + (EB_TE + 1);
    int32_t *s_beg = sh.work + 2 * (EB_TE + 1);
    const int total = sh.uprefix[NLISTS * STRIPES];
    for (int u = c.wg; u < total; u += c.G) {
        int r = 0;
        while (sh.uprefix[r + 1] <= u) ++r;
        const int l = r / STRIPES, s = r % STRIPES;
        const int t = u - sh.uprefix[r];
        const int E = sh.ledges[r];
        const int N = sh.lcount[r];
        const int a = t * EB_TE;
        const int b = min(a + EB_TE, E);   // at most STEP_CLAIMS winners
        const int32_t *ts = cts + (size_t)r * P.tscap;
        const int i0 = ts[t];
        const int i1 = (a + EB_TE < E) ? ts[t + 1] : N - 1;
        int ns = i1 - i0 + 1;   // <= EB_TE + 1: every segment has an edge
        if (ns > EB_TE + 1 || ns < 1) {
            if (threadIdx.x == 0) set_err(P, ERR_TSTART_OVERFLOW, ns);
            ns = max(1, min(ns, EB_TE + 1));
        }
        for (int j = threadIdx.x; j < ns; j += BLOCK) {
            const Seg sg = *seg_slot(P, const_cast<Seg *>(cq), const_cast<Seg *>(ct), l, s, i0 + j);
            s_off[j] = sg.off; s_v[j] = sg.v; s_beg[j] = sg.beg;
            if (sh.clear_bm) cbm[sg.v >> 5] = 0u;
        }
        __syncthreads();
        static_assert(EB_TE % BLOCK == 0 && EB_TE <= STEP_CLAIMS, "one step per tile");
        constexpr int NB = EB_TE / BLOCK;
        {
            const int e0 = a + (int)threadIdx.x;
            int tv[NB], owner[NB];
            bool ok[NB];
#pragma unroll
            for (int q = 0; q < NB; ++q) {
                const int e = e0 + q * BLOCK;
                ok[q] = e < b;
                // last j with s_off[j] <= e
                int lo = 0, hi = ns;
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (s_off[mid] <= e) lo = mid; else hi = mid;
                }
                owner[q] = s_v[lo];
                tv[q] = ok[q] ? P.col_idx[s_beg[lo] + (e - s_off[lo])] : 0;
            }
            claim_batch(c, tv, ok, owner);
        }
        __syncthreads();
        maybe_flush(c);
    }
}

// Top-down from a bitmap frontier (the level after a bottom-up level): each
// workgroup scans its range of bitmap words, lists the frontier vertices in
// LDS and expands them as segments.  Both frontier bitmaps are zeroed on the
// way (this level writes no bitmap).
__device__ __forceinline__ void td_from_bitmap(Ctx &c, uint32_t *cbm, uint32_t *obm) {
    const Params &P = *c.P;
    LevelShared &sh = *c.sh;
    int32_t *flist = sh.work;
    const int per = (P.nwp + c.G - 1) / c.G;
    const int start = c.wg * per;
    const int end = min(P.nwp, start + per);
    constexpr int R = FLIST_CAP / BLOCK;   // word pairs per wave per round
    for (int base = start; base < end; base += WAVES * R) {
        for (int j = 0; j < R; ++j) {
            const int wp = base + wave_id() * R + j;
            if (wp < end) {
                uint64_t *cw = reinterpret_cast<uint64_t *>(cbm) + wp;
                const uint64_t word = *cw;
                const bool in = (word >> lane_id()) & 1ull;
                const uint64_t m = __ballot(in);
                if (m) {
                    const int leader = __ffsll((unsigned long long)m) - 1;
                    int b0 = 0;
                    if (lane_id() == leader) b0 = atomicAdd(&sh.fcnt, __popcll(m));
                    b0 = readlane_i(b0, leader);
                    if (in) flist[b0 + mbcnt64(m)] = wp * 64 + lane_id();
                }
                if (lane_id() == 0) {
                    *cw = 0ull;
                    reinterpret_cast<uint64_t *>(obm)[wp] = 0ull;
                }
            }
        }
        __syncthreads();
        const int nf = sh.fcnt;
        for (int c0 = 0; c0 < nf; c0 += BLOCK) {
            const int i = c0 + (int)threadIdx.x;
            const bool has = i < nf && flist[i] < P.n;
            int v = 0, beg = 0, len = 0;
            if (has) {
                v = flist[i];
                beg = P.row_ptr[v];
                len = P.row_ptr[v + 1] - beg;
            }
            expand_segments(c, has && len > 0, v, beg, len);
            maybe_flush(c);
        }
        if (threadIdx.x == 0) sh.fcnt = 0;
        __syncthreads();
    }
}

// -------------------------------------------------------- bottom-up --------

// Every unvisited vertex looks for a parent in the frontier bitmap, in CSR
// order; a wavefront owns 64 consecutive vertices, so __ballot(found) is the
// next bitmap's 64-bit word and the visited word update needs no atomics.
__device__ __forceinline__ void wave_lds_sync() {
    // order this wavefront's LDS traffic between lanes (no workgroup barrier)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ void bottom_up(Ctx &c, const uint32_t *cbm, uint32_t *nbm) {
    const Params &P = *c.P;
    LevelShared &sh = *c.sh;
    const int per = (P.nwp + c.G - 1) / c.G;
    const int start = c.wg * per;
    const int end = min(P.nwp, start + per);
    const int lane = lane_id();
    const int wv = wave_id();
    uint64_t *vis64 = reinterpret_cast<uint64_t *>(P.visited);
    uint64_t *nbm64 = reinterpret_cast<uint64_t *>(nbm);
    int32_t *lst = sh.bu_lst[wv];
    // a wavefront takes BU_GP word pairs (BU_GP*64 vertices) at a time,
    // gathers their unvisited vertices into a dense LDS list, and scans them
    // 64 at a time: every lane has a vertex whatever share is visited
    for (int g0 = start + wv * BU_GP; g0 < end; g0 += WAVES * BU_GP) {
        const int ng = min(BU_GP, end - g0);
        int cnt = 0;
        for (int j = 0; j < ng; ++j) {
            const uint64_t vis = vis64[g0 + j];
            const bool act = !((vis >> lane) & 1ull);   // padding bits are set
            const uint64_t m = __ballot(act);
            if (act) lst[cnt + mbcnt64(m)] = (g0 + j) * 64 + lane;
            if (lane == 0) { sh.bu_vis[wv][j] = vis; sh.bu_fm[wv][j] = 0ull; }
            cnt += __popcll(m);
        }
        wave_lds_sync();
        for (int b0 = 0; b0 < cnt; b0 += WAVE) {
            const bool act = b0 + lane < cnt;
            const int v = act ? lst[b0 + lane] : 0;
            const int beg = act ? P.row_ptr[v] : 0;
            const int eend = act ? P.row_ptr[v + 1] : 0;
            const int lim = min(eend, beg + BU_LANE_SCAN);
            int e = beg, par = -1;
            bool fnd = false;
            // lane scan: each step covers the aligned 8-entry block holding
            // the scan position, fetched as two 16-byte loads, then probes the
            // block's entries inside [e, lim); the first hit in CSR order wins
            for (int step = 0; step <= BU_LANE_SCAN / 8; ++step) {
                const bool go = act && e < lim;
                if (!__ballot(go)) break;
                const int blk = e & ~7;
                int x[8];
                if (go && P.col_vec && blk + 8 <= P.m) {
                    const int4 a = *reinterpret_cast<const int4 *>(P.col_idx + blk);
                    const int4 b = *reinterpret_cast<const int4 *>(P.col_idx + blk + 4);
                    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
                    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
                } else {
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        x[q] = (go && blk + q >= e && blk + q < lim) ? P.col_idx[blk + q] : -1;
                }
                uint32_t w[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    if (!(go && blk + q >= e && blk + q < lim)) x[q] = -1;
                    w[q] = (x[q] >= 0) ? cbm[x[q] >> 5] : 0u;
                }
#pragma unroll
                for (int q = 7; q >= 0; --q)
                    if (x[q] >= 0 && ((w[q] >> (x[q] & 31)) & 1u)) { fnd = true; par = x[q]; }
                if (go) e = fnd ? lim : min(blk + 8, lim);
            }
            if (!fnd) e = lim;
            // long lists: the whole wavefront scans 64 entries at a time; the
            // first hit in CSR order is the lowest set lane of the first chunk
            uint64_t pm = __ballot(act && !fnd && e < eend);
            while (pm) {
                const int src = __ffsll((unsigned long long)pm) - 1;
                pm &= pm - 1;
                const int sb = readlane_i(e, src), se = readlane_i(eend, src);
                for (int c0 = sb; c0 < se; c0 += WAVE) {
                    const int ee = c0 + lane;
                    int u = 0;
                    bool hit = false;
                    if (ee < se) {
                        u = P.col_idx[ee];
                        hit = (cbm[u >> 5] >> (u & 31)) & 1u;
                    }
                    const uint64_t hm = __ballot(hit);
                    if (hm) {
                        const int first = __ffsll((unsigned long long)hm) - 1;
                        const int pu = readlane_i(u, first);
                        if (lane == src) { fnd = true; par = pu; }
                        break;
                    }
                }
            }
            if (fnd) {
                P.dist[v] = c.level + 1;
                if (P.parent) P.parent[v] = par;
                atomicOr(&sh.bu_fm[wv][(v >> 6) - g0], 1ull << (v & 63));
                c.fcnt += 1;
                c.fdeg += eend - beg;
            }
        }
        wave_lds_sync();
        // the group's next-bitmap words (every word written) and visited words
        if (lane < ng) {
            const uint64_t fm = sh.bu_fm[wv][lane];
            nbm64[g0 + lane] = fm;
            if (fm) vis64[g0 + lane] = sh.bu_vis[wv][lane] | fm;
        }
        wave_lds_sync();
    }
}

// ---------------------------------------------------------- kernels -------

__global__ __launch_bounds__(BLOCK) void bfs_init_kernel(Params P) {
    const int tid = blockIdx.x * BLOCK + threadIdx.x;
    const int nth = gridDim.x * BLOCK;
    const int s = P.source;
    for (int i = tid; i < P.n; i += nth) {
        P.dist[i] = (i == s) ? 0 : -1;
        if (P.parent) P.parent[i] = (i == s) ? s : -1;
    }
    uint64_t *vis64 = reinterpret_cast<uint64_t *>(P.visited);
    const uint64_t *init64 = reinterpret_cast<const uint64_t *>(P.vis_init);
    uint64_t *b0 = reinterpret_cast<uint64_t *>(P.fbm0);
    uint64_t *b1 = reinterpret_cast<uint64_t *>(P.fbm1);
    for (int wp = tid; wp < P.nwp; wp += nth) {
        const uint64_t sbit = (wp == (s >> 6)) ? (1ull << (s & 63)) : 0ull;
        vis64[wp] = init64[wp] | sbit;
        b0[wp] = sbit;
        b1[wp] = 0ull;
    }
    if (blockIdx.x == 0) {
        // every counter of every slot, then the source as the level-0 frontier
        for (int i = threadIdx.x; i < NSLOTS * NCTR; i += BLOCK)
            P.ctr[(size_t)i * CTR_STRIDE] = 0ull;
        if (threadIdx.x == 0) {
            P.ctl->done = 0; P.ctl->L = 0; P.ctl->err = 0; P.ctl->err_info = 0;
            P.ctl->lvl[0] = 0; P.ctl->lvl[1] = 0;
            P.ctl->bar_count = 0; P.ctl->bar_gen = 0;
            for (int k = 0; k < NSLOTS; ++k) {
                P.ctl->slot[k].dir = 0; P.ctl->slot[k].wbits = 0;
                P.ctl->slot[k].input_bm = 0; P.ctl->slot[k].fsize = 0;
                P.ctl->slot[k].reached_before = 0; P.ctl->slot[k].edges_before = 0;
            }
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            Ctx c;
            c.P = &P; c.sh = nullptr; c.level = -1; c.wg = 0; c.G = 1; c.stripe = 0; c.nslot = 0; c.wbits = 0;
            c.nbm = nullptr; c.nq = P.q0; c.nt = P.t0; c.nts = P.ts0; c.fcnt = 0; c.fdeg = 0;
            const int beg = P.row_ptr[s];
            const int len = P.row_ptr[s + 1] - beg;
            const int l = list_of(len);
            if (l >= 0) {
                const int nseg = (l == L_TILE) ? (len + TILE - 1) / TILE : 1;
                P.ctr[(size_t)(l * STRIPES) * CTR_STRIDE] =
                    ((unsigned long long)nseg << 32) | (unsigned)len;
                write_vertex_segments(c, l, s, beg, len, 0, 0);
            }
            P.ctr[(size_t)VC_BASE * CTR_STRIDE] = (1ull << 32) | (unsigned)len;
        }
    }
}

// Decision for level k, taken by wavefront 0 of every workgroup from the
// counters the previous level left (identical in every workgroup); the
// caller synchronises before reading it.
__device__ __forceinline__ void decide(const Params &P, LevelShared &sh, int k) {
    const int lane = lane_id();
    const int slot = k % NSLOTS;
    const int done = P.ctl->done;
    unsigned long long cv = 0;
    if (lane < NCTR) cv = *ctr_at(P, slot, lane);
    const bool is_vc = lane >= VC_BASE && lane < NCTR;
    const int64_t fsize = wave_sum<int64_t>(is_vc ? (int64_t)(cv >> 32) : 0);
    const int64_t fdeg = wave_sum<int64_t>(is_vc ? (int64_t)(cv & 0xffffffffull) : 0);
    if (lane < VC_BASE) {
        sh.lcount[lane] = (int32_t)(cv >> 32);
        sh.ledges[lane] = (int32_t)(cv & 0xffffffffull);
    }
    if (lane == 0) {
        sh.cnt = 0; sh.nbig = 0; sh.fcnt = 0;
        sh.fsize = (int32_t)fsize; sh.fdeg = fdeg;
        sh.small = 0;
        if (done || P.ctl->err) {
            sh.mode = 0;
        } else if (fsize == 0) {
            sh.mode = 1;
        } else {
            sh.mode = 2;
            const SlotInfo prev = (k > 0) ? P.ctl->slot[(k + NSLOTS - 1) % NSLOTS] : SlotInfo{0, 0, 0, 0, 0, 0};
            const int64_t reached_before = (k > 0) ? P.ctl->slot[slot].reached_before : 0;
            const int64_t edges_before = (k > 0) ? P.ctl->slot[slot].edges_before : 0;
            const bool has_queue = (k == 0) || prev.dir == DIR_TD;
            const bool has_bm = (k == 0) || prev.dir == DIR_BU || prev.wbits;
            bool want_pull;
            if (P.pol_dir == BFS_DIR_PULL) {
                want_pull = true;
            } else if (P.pol_dir == BFS_DIR_PUSH) {
                want_pull = false;
            } else if (k == 0 || prev.dir == DIR_TD) {
                // edges still to be explored from unvisited vertices
                const int64_t m_u = (int64_t)P.m - edges_before - fdeg;
                want_pull = fdeg * ALPHA > m_u;
            } else {
                want_pull = !(fsize * BETA < (int64_t)P.n && fsize < prev.fsize);
            }
            const int dir = (want_pull && P.symmetric && has_bm) ? DIR_BU : DIR_TD;
            sh.dir = dir;
            sh.reached_before = reached_before;
            sh.edges_before = edges_before;
            sh.input_bm = (dir == DIR_TD) && !has_queue;
            sh.clear_bm = (dir == DIR_TD) && has_queue && has_bm;
            // a top-down level from a queue also sets its new vertices in the
            // next bitmap whenever the next level may pull
            sh.wbits = (dir == DIR_TD) && has_queue && P.symmetric && P.pol_dir == BFS_DIR_AUTO;
            // edge-balanced unless the binned advance is forced: its tiles
            // spread even a small frontier over several workgroups and
            // bound the winners between flushes
            sh.adv_eb = (dir == DIR_TD) && has_queue && P.pol_adv != BFS_ADV_BINNED;
            sh.small = P.small_mode && (dir == DIR_TD) && has_queue && fsize <= SMALL_F && fdeg <= SMALL_E;
        }
    }
}

// Barrier among the G workgroups of the small-frontier mode (all resident:
// the others exit at once).  Release before arriving, acquire after leaving,
// both at device scope so queues, bitmaps and counters written before it are
// seen after it.  The wait is bounded: past the limit it records
// ERR_BARRIER_TIMEOUT and returns, and every workgroup then leaves its loop.
__device__ __forceinline__ void small_barrier(const Params &P, int G) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const uint32_t gen = __hip_atomic_load(&P.ctl->bar_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t arrived = atomicAdd(&P.ctl->bar_count, 1u);
        if (arrived == (uint32_t)G - 1) {
            __hip_atomic_store(&P.ctl->bar_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&P.ctl->bar_gen, gen + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while (__hip_atomic_load(&P.ctl->bar_gen, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == gen) {
                __builtin_amdgcn_s_sleep(2);
                if (__builtin_amdgcn_s_memrealtime() - t0 > P.barrier_ticks) {
                    atomicCAS(&P.ctl->err, 0, ERR_BARRIER_TIMEOUT);
                    break;
                }
            }
        }
        __threadfence();
    }
    __syncthreads();
}

// One level on the G workgroups taking part (this one is number wg).
__device__ __forceinline__ void run_level(const Params &P, LevelShared &sh, int k, int wg, int G) {
    const int lane = lane_id();
    const int slot = k % NSLOTS;
    // unit prefix tables
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int r = 0; r < NLISTS * STRIPES; ++r) {
            sh.uprefix[r] = acc;
            const int l = r / STRIPES;
            int units;
            if (sh.adv_eb) units = (sh.ledges[r] + EB_TE - 1) / EB_TE;
            else if (l == L_TILE) units = sh.lcount[r];
            else if (l == L_MID) units = (sh.lcount[r] + WAVES - 1) / WAVES;
            else units = (sh.lcount[r] + BLOCK - 1) / BLOCK;
            acc += units;
        }
        sh.uprefix[NLISTS * STRIPES] = acc;
    }
    // bookkeeping of level k by workgroup 0
    if (wg == 0) {
        if (threadIdx.x == 0) {
            if (P.level_sizes) P.level_sizes[k] = sh.fsize;
            if (k < P.st_cap) { P.st_dir[k] = (int8_t)sh.dir; P.st_fdeg[k] = sh.fdeg; }
            P.ctl->slot[slot].dir = sh.dir;
            P.ctl->slot[slot].wbits = sh.wbits;
            P.ctl->slot[slot].input_bm = sh.input_bm;
            P.ctl->slot[slot].fsize = sh.fsize;
            P.ctl->slot[(k + 1) % NSLOTS].reached_before = sh.reached_before + sh.fsize;
            P.ctl->slot[(k + 1) % NSLOTS].edges_before = sh.edges_before + sh.fdeg;
        }
        if (threadIdx.x < NCTR) *ctr_at(P, (k + 2) % NSLOTS, threadIdx.x) = 0ull;
    }
    __syncthreads();

    Ctx c;
    c.P = &P;
    c.sh = &sh;
    c.level = k;
    c.wg = wg;
    c.G = G;
    c.stripe = wg % STRIPES;
    c.nslot = (k + 1) % NSLOTS;
    c.wbits = sh.wbits;
    const int cur = k & 1;
    uint32_t *cbm = cur ? P.fbm1 : P.fbm0;
    uint32_t *obm = cur ? P.fbm0 : P.fbm1;
    c.nbm = obm;
    c.nq = cur ? P.q0 : P.q1;
    c.nt = cur ? P.t0 : P.t1;
    c.nts = cur ? P.ts0 : P.ts1;
    c.fcnt = 0;
    c.fdeg = 0;
    const Seg *cq = cur ? P.q1 : P.q0;
    const Seg *ct = cur ? P.t1 : P.t0;
    const int32_t *cts = cur ? P.ts1 : P.ts0;

    if (sh.dir == DIR_BU) {
        bottom_up(c, cbm, obm);
    } else if (sh.input_bm) {
        td_from_bitmap(c, cbm, obm);
        if (sh.cnt > 0) flush(c);
    } else if (sh.adv_eb) {
        td_edge_balanced(c, cq, ct, cts, cbm);
        if (sh.cnt > 0) flush(c);
    } else {
        td_binned(c, cq, ct, cbm);
        if (sh.cnt > 0) flush(c);
    }

    // workgroup tallies -> one striped atomic
    const int64_t wc = wave_sum<int64_t>((int64_t)c.fcnt);
    const int64_t wd = wave_sum<int64_t>(c.fdeg);
    __syncthreads();
    if (lane == 0) { sh.scan_tmp[0][wave_id()] = (uint64_t)wc; sh.scan_tmp[1][wave_id()] = (uint64_t)wd; }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t tc = 0, td = 0;
        for (int w = 0; w < WAVES; ++w) { tc += sh.scan_tmp[0][w]; td += sh.scan_tmp[1][w]; }
        if (tc) atomicAdd(ctr_at(P, c.nslot, VC_BASE + c.stripe), (unsigned long long)((tc << 32) | td));
    }
}

// One launch: runs the level lvl[launch & 1] on the whole grid, or, when that
// level is small, runs levels on the first SMALL_G workgroups until one is
// not small; then records where the next launch starts.
__global__ __launch_bounds__(BLOCK, 4) void bfs_level_kernel(Params P, int32_t launch) {
    __shared__ LevelShared sh;
    int k = P.ctl->lvl[launch & 1];
    if (threadIdx.x < WAVE) decide(P, sh, k);
    __syncthreads();
    if (sh.mode == 0) return;
    if (sh.mode == 1) {
        if (blockIdx.x == 0 && threadIdx.x == 0) { P.ctl->L = k; P.ctl->done = 1; }
        return;
    }
    const bool small = sh.small;
    if (small && blockIdx.x >= SMALL_G) return;
    const int G = small ? min((int)gridDim.x, SMALL_G) : (int)gridDim.x;
    for (;;) {
        run_level(P, sh, k, blockIdx.x, G);
        ++k;
        if (!small) break;
        small_barrier(P, G);
        if (threadIdx.x < WAVE) decide(P, sh, k);
        __syncthreads();
        if (sh.mode == 0) return;    // an error was recorded
        if (sh.mode == 1) {
            if (blockIdx.x == 0 && threadIdx.x == 0) { P.ctl->L = k; P.ctl->done = 1; }
            return;
        }
        if (!sh.small) break;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) P.ctl->lvl[(launch + 1) & 1] = k;
}

// ------------------------------------------------- graph validation --------

__global__ __launch_bounds__(256) void check_rows_kernel(const int32_t *row_ptr, int32_t n,
                                                         GraphFacts *f) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    int32_t maxd = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += nth) {
        const int32_t a = row_ptr[i], b = row_ptr[i + 1];
        if (a > b) atomicMin(&f->bad_row, (unsigned long long)i);
        else maxd = max(maxd, b - a);
    }
    maxd = max(maxd, __shfl_xor(maxd, 1, WAVE));
    for (int d = 2; d < WAVE; d <<= 1) maxd = max(maxd, __shfl_xor(maxd, d, WAVE));
    if (lane_id() == 0) atomicMax(&f->max_degree, maxd);
}

// one wavefront per row: every entry in range, rows ascending
__global__ __launch_bounds__(256) void check_cols_kernel(const int32_t *row_ptr,
                                                         const int32_t *col_idx, int32_t n,
                                                         GraphFacts *f) {
    const int64_t wid = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / WAVE;
    const int64_t nw = (int64_t)gridDim.x * blockDim.x / WAVE;
    const int lane = lane_id();
    bool unsorted = false;
    for (int64_t u = wid; u < n; u += nw) {
        const int32_t b = row_ptr[u], e = row_ptr[u + 1];
        for (int32_t i = b + lane; i < e; i += WAVE) {
            const int32_t x = col_idx[i];
            if (x < 0 || x >= n) atomicMin(&f->bad_col, (unsigned long long)i);
            if (i + 1 < e && col_idx[i + 1] < x) unsorted = true;
        }
    }
    if (__ballot(unsorted) && lane == 0) atomicOr(&f->unsorted, 1u);
}

// sorted rows only: every entry u->v has v->u (binary search in row v)
__global__ __launch_bounds__(256) void check_symmetry_kernel(const int32_t *row_ptr,
                                                             const int32_t *col_idx, int32_t n,
                                                             GraphFacts *f) {
    const int64_t wid = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / WAVE;
    const int64_t nw = (int64_t)gridDim.x * blockDim.x / WAVE;
    const int lane = lane_id();
    bool asym = false;
    for (int64_t u = wid; u < n; u += nw) {
        const int32_t b = row_ptr[u], e = row_ptr[u + 1];
        for (int32_t i = b + lane; i < e; i += WAVE) {
            const int32_t v = col_idx[i];
            int32_t lo = row_ptr[v], hi = row_ptr[v + 1];
            while (lo < hi) {
                const int32_t mid = lo + ((hi - lo) >> 1);
                if (col_idx[mid] < (int32_t)u) lo = mid + 1; else hi = mid;
            }
            if (!(lo < row_ptr[v + 1] && col_idx[lo] == (int32_t)u)) asym = true;
        }
        if (__ballot(asym)) break;
    }
    if (__ballot(asym) && lane == 0) atomicOr(&f->asymmetric, 1u);
}

// visited-bitmap template: padding bits past n, and (symmetric graphs)
// isolated vertices, which no search can reach
__global__ __launch_bounds__(256) void vis_init_kernel(const int32_t *row_ptr, int32_t n,
                                                       int32_t mark_isolated, uint32_t *out,
                                                       int32_t nwords) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwords; w += nth) {
        uint32_t word = 0;
        for (int b = 0; b < 32; ++b) {
            const int64_t v = w * 32 + b;
            if (v >= n) word |= 1u << b;
            else if (mark_isolated && row_ptr[v + 1] == row_ptr[v]) word |= 1u << b;
        }
        out[w] = word;
    }
}

// ------------------------------------------------------ host helpers -------

hipError_t launch_init(const Params &P, int grid, hipStream_t s) {
    hipLaunchKernelGGL(bfs_init_kernel, dim3(grid), dim3(BLOCK), 0, s, P);
    return hipGetLastError();
}

hipError_t launch_level(const Params &P, int32_t launch_index, int grid, hipStream_t s) {
    hipLaunchKernelGGL(bfs_level_kernel, dim3(grid), dim3(BLOCK), 0, s, P, launch_index);
    return hipGetLastError();
}

int level_kernel_blocks_per_cu() {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void *)bfs_level_kernel, BLOCK, 0) !=
        hipSuccess)
        return 1;
    return nb > 0 ? nb : 1;
}

static int grid_for(int64_t work, int per_block) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (int)g;
}

hipError_t launch_check_rows(const int32_t *row_ptr, int32_t n, GraphFacts *f, hipStream_t s) {
    hipLaunchKernelGGL(check_rows_kernel, dim3(grid_for(n, 256 * 4)), dim3(256), 0, s, row_ptr, n, f);
    return hipGetLastError();
}

hipError_t launch_check_cols(const int32_t *row_ptr, const int32_t *col_idx, int32_t n,
                             GraphFacts *f, hipStream_t s) {
    hipLaunchKernelGGL(check_cols_kernel, dim3(grid_for((int64_t)n * WAVE, 256 * 8)), dim3(256), 0, s,
                       row_ptr, col_idx, n, f);
    return hipGetLastError();
}

hipError_t launch_check_symmetry(const int32_t *row_ptr, const int32_t *col_idx, int32_t n,
                                 GraphFacts *f, hipStream_t s) {
    hipLaunchKernelGGL(check_symmetry_kernel, dim3(grid_for((int64_t)n * WAVE, 256 * 8)), dim3(256), 0,
                       s, row_ptr, col_idx, n, f);
    return hipGetLastError();
}

hipError_t launch_build_vis_init(const int32_t *row_ptr, int32_t n, int32_t mark_isolated,
                                 uint32_t *vis_init, hipStream_t s) {
    const int64_t nwp = ((int64_t)n + 63) / 64;
    const int32_t nwords = (int32_t)(2 * nwp);
    hipLaunchKernelGGL(vis_init_kernel, dim3(grid_for(nwords, 256 * 4)), dim3(256), 0, s, row_ptr, n,
                       mark_isolated, vis_init, nwords);
    return hipGetLastError();
}

}  // namespace fbfs
