// gfx950 kernels for level-synchronous, frontier-based BFS over an int32 CSR
// graph.  One launch initialises a search; then launches of two level kernels
// alternate: bfs_td_kernel (even launch indexes) runs top-down levels and
// bfs_bu_kernel (odd indexes) runs bottom-up levels.  Every launch reads the
// level it stands at and the frontier counters left in device memory by the
// previous launch, decides the direction itself, runs the level if the
// direction is its own (else passes it on) and exits at once after the
// search has ended, so the host can enqueue launches ahead without learning
// anything per level (the per-level launch plus device-to-host count copy of
// bfs.cu's runBfs, in "Day 38 - Graph traversal on a GPU", is what this
// removes).  The two directions live in separate kernels so that each gets
// its own register allocation.
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
// give exactly: pull when sum deg(F) > (edges of unvisited vertices) / alpha,
// back to push when |F| < n / beta and shrinking (Beamer, Asanovic and
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
#include <type_traits>

#include <hip/hip_ext.h>

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

// The same over a pair of 32-bit counts packed in 64 bits (high: items, low:
// edges): callers keep each field's wavefront total below 2^32, so the
// halves are scanned apart with no carry between them.
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t x) {
    const uint32_t lo = wave_incl_scan_u32((uint32_t)x);
    const uint32_t hi = wave_incl_scan_u32((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}


// ---------------------------------------------------------- LDS layout -----

constexpr int WORK_INTS = 3 * (EB_TE + 1);
constexpr int FLIST_CAP = 4 * BLOCK;     // from-bitmap pass: 4 word pairs per wave per round
static_assert(FLIST_CAP <= WORK_INTS, "work area too small");

// Shared state of one level launch: the decision (identical in every
// workgroup) and the bookkeeping common to both directions ...
struct LevelCommon {
    uint64_t scan_tmp[3][WAVES];
    // decision
    int32_t mode;                     // 0 exit, 1 finish, 2 run
    int32_t dir, input_bm, wbits, wcf, clear_bm, adv_eb, small, use_cf, cf_clear, noq;
    int32_t dfr;                      // the level before was queue-free: this level writes its frontier's dist
    int32_t keep_in;                  // ... and this level records its frontier in the kept bitmap instead
    int32_t keep_out;                 // a bottom-up level recording its finds in the kept bitmap, no dist stores
    int32_t fsize;
    int32_t prev_wcf;                 // the level before set the coarse map of this one
    int64_t prev_fdeg;                // the level before's frontier edges
    int64_t fdeg, reached_before, edges_before;
    int32_t lcount[NLISTS * STRIPES];  // segments per (list, stripe)
    int32_t ledges[NLISTS * STRIPES];  // edges per (list, stripe)
    int32_t uprefix[NLISTS * STRIPES + 1];  // unit prefix (binned or edge-balanced)
};

// ... then the top-down kernel's work areas (one pass at a time uses the work
// area: the frontier lists of the from-bitmap pass or the segment table of
// the edge-balanced pass) ...
struct TdLds : LevelCommon {
    int32_t buf[CAP];                 // staged new frontier vertices
    int32_t sbeg[CAP], slen[CAP];     // their adjacency start and degree
    int32_t work[WORK_INTS];
    int32_t big_v[BLOCK], big_beg[BLOCK], big_len[BLOCK];
    int32_t tstart[CAP], toff[CAP];   // flush: piece start / edge offset of each staged slot
    int32_t ntiles;
    unsigned long long list_base[NLISTS];
    int32_t qsplit[2], qd[2][2];      // flush: per list, the first index of its second chunk and
                                      // storage - index for either chunk (QD_NONE: missing)
    int32_t qbad;                     // a queue chunk of the level's input is missing (error recorded)
    int32_t cnt;                      // staged count (may exceed CAP: overflow spilled)
    int32_t spilled;                  // some lane appended directly this level (its tallies are per thread)
    int32_t nbig;
    int32_t fl_cnt[WAVES], fl_more[WAVES];   // from-bitmap lists: count, words left
    int32_t vfilter;                  // claims first load the visited words
    // small-frontier mode
    unsigned long long rpack[2];      // this workgroup's winners of a level (by its parity) in
                                      // its region (bits 40-63) and their edges (bits 0-39, each
                                      // winner's at most SMALL_E + 1)
    int32_t rbig[2];                  // ... one of them has at least T_WG edges
    int32_t inl[2];                   // ... all of them have their targets in itgt / iown
    int32_t itgt[2][BLOCK];           // own mode: a level's winners' targets by edge offset (those
    int32_t iown[2][BLOCK];           //   of degree <= ADJ_INLINE within BLOCK edges) and owners
    int32_t spre[SMALL_G + 1];        // exclusive prefix of the workgroups' winners
    int32_t s_total, s_err, s_big;    // winners of all workgroups; an error was recorded; a big one
    int32_t s_own;                    // each workgroup expands its own winners (kept in buf, sbeg, slen)
    unsigned long long s_edges;       // their edges (saturating per workgroup at 2^24 - 1)
};

// ... and the bottom-up kernel's, per wavefront; kept small so that several
// workgroups share a compute unit.
struct BuLds : LevelCommon {
    int32_t bu_lst[WAVES][BU_GSZ];   // listed unvisited vertices
    int32_t bu_deg[WAVES][BU_GSZ];   // their degrees
    int32_t bu_hit[WAVES][BU_GSZ];   // entry of the first hit, BU_NOHIT if none
    int32_t bu_pi[WAVES][BU_GSZ];    // pending vertices: index into bu_lst,
    int32_t bu_pn[WAVES][BU_GSZ];    //   next entry to probe,
    int32_t bu_pe[WAVES][BU_GSZ];    //   end of the list,
    int32_t bu_ps[WAVES][BU_GSZ];    //   exclusive scan of this round's probes
    unsigned long long bu_fm[WAVES][WAVE];  // found masks of the 64 words in hand
    uint32_t bu_cf[CF_WORDS];        // coarse frontier map (when use_cf)
};

// Per-thread context of one level launch (S: the kernel's LDS layout).
template <class S>
struct CtxT {
    const Params *P;
    S *sh;
    int32_t level;          // k: new vertices get k+1
    int32_t wg, G;          // this workgroup's index among the G taking part
    int32_t stripe;         // counter / queue stripe of this workgroup
    int32_t nslot;          // slot of level k+1
    int32_t wbits;
    uint32_t *nbm;          // bitmap of level k+1 (top-down with wbits)
    uint32_t *ncf;          // coarse map of level k+1 (top-down with wcf)
    int32_t wcf;
    int32_t noq;            // no queue: winners are tallied per thread, not staged
    Seg *nq, *nt;           // queues of level k+1
    int32_t *nts;
    int4 *region;           // small-frontier mode: winners go to this region (else staged)
    int32_t converting;     // the flush converts a region already counted (enqueue counts)
    // per-thread tallies of new frontier vertices
    int32_t fcnt;
    int64_t fdeg;
};
using Ctx = CtxT<TdLds>;
using BuCtx = CtxT<BuLds>;

// --------------------------------------------------------- emission --------

__device__ __forceinline__ void set_err(const Params &P, int code, int info) {
    atomicCAS(&P.ctl->err, 0, code);
    P.ctl->err_info = info;
}

constexpr int32_t QD_NONE = (int32_t)0x80000000;

// Table entry of chunk j >= 1 of region (list l < L_TILE, stripe s) in the
// chunk table of level slot `slot`.
__device__ __forceinline__ unsigned long long *qtab_at(const Params &P, int slot, int l, int s, int64_t j) {
    return P.qtab + (((size_t)slot * 2 + l) * STRIPES + s) * P.qpool + (size_t)(j - 1);
}

// Where segment `idx` of list l, stripe s of the queue of level k (tables of
// slot k % NSLOTS, tag k + 1) lives; null (the error recorded) when a chunk
// table entry is missing or out of range.
__device__ __forceinline__ Seg *seg_slot(const Params &P, Seg *q, Seg *t, int l, int s, int64_t idx, int k) {
    if (l == L_TILE) return t + (size_t)s * P.tcap + idx;
    const int64_t j = idx >> P.qk_sh;
    const int64_t off = idx & ((1LL << P.qk_sh) - 1);
    if (__builtin_expect(j == 0, 1)) return q + ((size_t)(l * STRIPES + s) << P.qk_sh) + off;
    if (j > P.qpool) { set_err(P, ERR_QUEUE_OVERFLOW, l); return nullptr; }
    const unsigned long long e = *qtab_at(P, k % NSLOTS, l, s, j);
    const uint32_t id = (uint32_t)e;
    if ((uint32_t)(e >> 32) != (uint32_t)(k + 1) || id >= (uint32_t)P.qpool) {
        set_err(P, ERR_QUEUE_OVERFLOW, l);
        return nullptr;
    }
    return q + ((size_t)(2 * STRIPES + id) << P.qk_sh) + off;
}

// Start (a segment offset into the queue being written) of chunk j of this
// workgroup's region of list l < L_TILE in the queue of level c.level + 1,
// for a reservation of segments from index b on: chunk 0 is fixed; a chunk
// whose first segment lies in the reservation is taken from the pool here
// and recorded (tagged c.level + 2) in the level's table; any other chunk was
// taken by the earlier reservation holding its first segment, whose entry
// is awaited (bounded).  -1, the error recorded, when the pool or the wait
// runs out.
// The pool chunk behind table entry e (tag: the writing level's): taken from
// the pool counter and recorded (take), or awaited until recorded (bounded
// by `ticks`).  -1 when the pool is used up or the wait runs out, the error
// recorded in ctl.  Lanes of one wavefront may need the same chunk, one
// taking it and others awaiting it, so every lane that takes a chunk has
// recorded it before any lane starts to wait (an if / else here could run
// the waiting side first, with the taking lane masked off).  Kept out of
// line: the expansion loops inline the queue writes in many places, and this
// rare path would weigh on all of them.
__device__ __noinline__ int32_t queue_chunk_slow(unsigned long long *e, unsigned long long *pool, uint32_t tag,
                                                 int32_t qpool, bool take, uint32_t ticks, Ctl *ctl) {
    uint32_t id = 0xffffffffu;
    int code = ERR_QUEUE_OVERFLOW;
    if (take) {
        id = (uint32_t)atomicAdd(pool, 1ull);
        if (id < (uint32_t)qpool)
            __hip_atomic_store(e, ((unsigned long long)tag << 32) | id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // keeps the records ahead of the waits
    if (!take) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (;;) {
            const unsigned long long x = __hip_atomic_load(e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((uint32_t)(x >> 32) == tag) {
                id = (uint32_t)x;
                break;
            }
            if (__builtin_amdgcn_s_memrealtime() - t0 > ticks) {
                code = ERR_BARRIER_TIMEOUT;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    if (id >= (uint32_t)qpool) {
        atomicCAS(&ctl->err, 0, code);
        return -1;
    }
    return (int32_t)id;
}

__device__ __forceinline__ int64_t queue_chunk(const Ctx &c, int l, int64_t j, int64_t b) {
    const Params &P = *c.P;
    if (__builtin_expect(j == 0, 1)) return (int64_t)(l * STRIPES + c.stripe) << P.qk_sh;
    if (j > P.qpool) { set_err(P, ERR_QUEUE_OVERFLOW, l); return -1; }
    const int32_t id = queue_chunk_slow(qtab_at(P, c.nslot, l, c.stripe, j), ctr_at(P, c.nslot, QPOOL_CTR),
                                        (uint32_t)(c.level + 2), P.qpool, (j << P.qk_sh) >= b,
                                        P.barrier_ticks, P.ctl);
    return id < 0 ? -1 : (int64_t)(2 * STRIPES + id) << P.qk_sh;
}

// Writes one segment (vertex v, adjacency piece [pb, pb+pl), edge offset po)
// at index si of list l (stored at dst; null: its chunk is missing, the error
// already recorded) and records the edge-balanced tiles whose first edge
// falls inside it.
__device__ __forceinline__ void write_piece(const Ctx &c, int l, int64_t si, int v, int pb, int pl,
                                            int64_t po, Seg *dst) {
    const Params &P = *c.P;
    // a region of the queue holds at most n segments (one per vertex)
    const int64_t cap = (l == L_TILE) ? P.tcap : (int64_t)P.n;
    if (si >= cap) { set_err(P, l == L_TILE ? ERR_TILE_OVERFLOW : ERR_QUEUE_OVERFLOW, (int)l); return; }
    if (!dst) return;
    Seg sg;
    sg.v = v; sg.beg = pb; sg.len = pl; sg.off = (int32_t)po;
    *dst = sg;
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
    const Params &P = *c.P;
    if (l != L_TILE) {
        // one segment: its chunk, for a reservation of this index alone
        Seg *dst = nullptr;
        if (idx < (int64_t)P.n) {
            const int64_t cb = queue_chunk(c, l, idx >> P.qk_sh, idx);
            if (cb >= 0) dst = c.nq + cb + (idx & ((1LL << P.qk_sh) - 1));
        }
        write_piece(c, l, idx, v, beg, len, eoff, dst);
        return;
    }
    const int nseg = (len + TILE - 1) / TILE;
    for (int j = 0; j < nseg; ++j) {
        const int64_t si = idx + j;
        write_piece(c, l, si, v, beg + j * TILE, min(TILE, len - j * TILE), eoff + (int64_t)j * TILE,
                    si < P.tcap ? c.nt + (size_t)c.stripe * P.tcap + si : nullptr);
    }
}

__device__ __forceinline__ int list_of(int len) {
    return len <= 0 ? -1 : (len < T_LANE ? L_SMALL : (len < T_WG ? L_MID : L_TILE));
}

// One vertex (adjacency [beg, beg+len)), one lane: used when the LDS staging
// buffer is full (the expansion loops flush often enough that this is rare).
__device__ __forceinline__ void emit_single(Ctx &c, int v, int beg, int len) {
    const Params &P = *c.P;
    FBFS_ENQ(P, v);
    c.fcnt += 1;
    c.fdeg += len;
    c.sh->spilled = 1;
    const int l = list_of(len);
    if (l < 0) return;
    const int nseg = (l == L_TILE) ? (len + TILE - 1) / TILE : 1;
    unsigned long long add = ((unsigned long long)nseg << 32) | (unsigned)len;
    unsigned long long base = atomicAdd(ctr_at(P, c.nslot, l * STRIPES + c.stripe), add);
    write_vertex_segments(c, l, v, beg, len, (int64_t)(base >> 32), (int64_t)(base & 0xffffffffull));
}

// Stage a winner (adjacency [beg, beg+len)) in LDS (wave-aggregated LDS
// atomic, rank by mbcnt).
__device__ __forceinline__ void stage(Ctx &c, bool win, int v, int beg, int len) {
    const uint64_t m = __ballot(win);
    if (m == 0) return;
    const int leader = __ffsll((unsigned long long)m) - 1;
    int base = 0;
    if (lane_id() == leader) base = atomicAdd(&c.sh->cnt, __popcll(m));
    base = readlane_i(base, leader);
    bool spill = false;
    if (win) {
        const int slot = base + mbcnt64(m);
        if (slot < CAP) {
            c.sh->buf[slot] = v;
            c.sh->sbeg[slot] = beg;
            c.sh->slen[slot] = len;
        } else {
            spill = true;
        }
    }
    // the lanes that found the buffer full append their vertex directly
    if (spill) emit_single(c, v, beg, len);
}

// Small-frontier mode: a winner (adjacency [beg, beg+len)) goes straight to
// this workgroup's region; one LDS atomic per winner on the packed (count,
// edges) word gives its place and the edge offset of its list (per lane:
// callers may be in divergent control flow).  The first OWN_CAP winners are
// also kept in LDS (vertex, adjacency start, edge offset), in the half of
// buf / sbeg / toff that belongs to their level's parity, for the next
// level's own-mode expansion.
constexpr int OWN_CAP = CAP / 2;
constexpr int ADJ_NONE = (int)0x80000000;   // an inline adjacency record that was not read
constexpr unsigned long long RP_EDGES = (1ull << 40) - 1;

__device__ __forceinline__ void stage_region(Ctx &c, bool win, int v, int beg, int len, int4 a4) {
    if (win) {
        // each degree counts at most SMALL_E + 1: the sum only needs to be
        // exact up to SMALL_E (the published edges saturate above it)
        const int par = (c.level + 1) & 1;
        const unsigned long long old =
            atomicAdd(&c.sh->rpack[par], (1ull << 40) | (unsigned long long)min(len, SMALL_E + 1));
        const int slot = (int)(old >> 40);
        if (len >= T_WG) c.sh->rbig[par] = 1;
        if (slot < SREG_CAP) {
            c.region[slot] = make_int4(v, beg, len, 0);
            FBFS_ENQ(*c.P, v);
            if (slot < OWN_CAP) {
                const int o = par * OWN_CAP + slot;
                c.sh->buf[o] = v;
                c.sh->sbeg[o] = beg;
                c.sh->toff[o] = (int32_t)(old & RP_EDGES);   // exact while the level's edges are few
            }
            // the targets themselves, by edge offset, when the adjacency came
            // inline and fits the first BLOCK edges
            const unsigned long long off = old & RP_EDGES;
            if (a4.x != ADJ_NONE && len <= ADJ_INLINE && off + (unsigned long long)len <= (unsigned long long)BLOCK) {
                int32_t *tg = c.sh->itgt[par] + off, *ow = c.sh->iown[par] + off;
                if (len > 0) { tg[0] = a4.x; ow[0] = v; }
                if (len > 1) { tg[1] = a4.y; ow[1] = v; }
                if (len > 2) { tg[2] = a4.z; ow[2] = v; }
                if (len > 3) { tg[3] = a4.w; ow[3] = v; }
            } else if (len > 0) {
                c.sh->inl[par] = 0;
            }
        } else {
            set_err(*c.P, ERR_QUEUE_OVERFLOW, slot);
        }
    }
}

// Claim up to N targets (v[q] valid where ok[q], reached from u[q]) for
// level k+1: one atomicOr per target on the visited bitmap decides its single
// winner.  On wide levels (vfilter) a plain load of the visited words first
// drops the targets already visited, sparing their atomics; on narrow levels
// that load would only lengthen the chain.  The loads and atomics of the N
// targets are each issued before any result is used, so a lane keeps N
// claims in flight; a winner's adjacency bounds are fetched at once for the
// flush.
constexpr int CB = 4;

template <int N>
__device__ __forceinline__ void claim_batch(Ctx &c, const int (&v)[N], const bool (&ok)[N],
                                            const int (&u)[N]) {
    constexpr int CB = N;
    const Params &P = *c.P;
    bool tryq[CB];
    // an id outside [0, n) (a graph changed after its checks) is reported,
    // never used as an index
    bool okq[CB];
#pragma unroll
    for (int q = 0; q < CB; ++q) {
        okq[q] = ok[q] && (uint32_t)v[q] < (uint32_t)P.n;
        if (ok[q] && !okq[q]) set_err(P, ERR_BAD_VERTEX, v[q]);
    }
    if (c.sh->vfilter) {
        uint32_t w[CB];
#pragma unroll
        for (int q = 0; q < CB; ++q) w[q] = okq[q] ? P.visited[v[q] >> 5] : ~0u;
#pragma unroll
        for (int q = 0; q < CB; ++q) tryq[q] = okq[q] && !((w[q] >> (v[q] & 31)) & 1u);
    } else {
#pragma unroll
        for (int q = 0; q < CB; ++q) tryq[q] = okq[q];
    }
    uint32_t old[CB];
#pragma unroll
    for (int q = 0; q < CB; ++q)
        old[q] = tryq[q] ? atomicOr(P.visited + (v[q] >> 5), 1u << (v[q] & 31)) : ~0u;
    bool win[CB];
    int beg[CB], len[CB];
    int4 a4[CB];
    if (c.region) {
        // small levels wait on each round trip: the adjacency bounds of every
        // candidate, and the adjacency itself when it is short, are read
        // beside its claim, not after it
#pragma unroll
        for (int q = 0; q < CB; ++q) {
            beg[q] = tryq[q] ? P.row_ptr[v[q]] : 0;
            len[q] = tryq[q] ? P.row_ptr[v[q] + 1] : 0;
            // (with one claim per lane, as own mode has: more would cost
            // registers the wider loops spill; ADJ_NONE marks a record not read)
            if constexpr (CB == 1) a4[q] = tryq[q] ? P.adj4[v[q]] : make_int4(-1, -1, -1, -1);
            else a4[q] = make_int4(ADJ_NONE, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < CB; ++q) win[q] = tryq[q] && !((old[q] >> (v[q] & 31)) & 1u);
    } else if (c.noq && P.symmetric) {
        // a queue-free level needs a winner's degree only for the tallies:
        // its degree byte (in-degree = out-degree here), and the row
        // pointers only past 254
#pragma unroll
        for (int q = 0; q < CB; ++q) {
            win[q] = tryq[q] && !((old[q] >> (v[q] & 31)) & 1u);
            beg[q] = 0;
            len[q] = win[q] ? (int)P.deg8[v[q]] : 0;
        }
#pragma unroll
        for (int q = 0; q < CB; ++q) {
            if (len[q] == 255) {
                beg[q] = P.row_ptr[v[q]];
                len[q] = P.row_ptr[v[q] + 1];
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < CB; ++q) {
            win[q] = tryq[q] && !((old[q] >> (v[q] & 31)) & 1u);
            beg[q] = win[q] ? P.row_ptr[v[q]] : 0;
            len[q] = win[q] ? P.row_ptr[v[q] + 1] : 0;
        }
    }
    if (c.noq) {
        // a queue-free level: its winners are the next level's frontier
        // bitmap, and their dist is left to that level, which writes it in
        // vertex order beside its own (a hub level's winners are spread over
        // the whole array, and a scattered 4-byte store costs a line).  The
        // parent, known only here, is a streaming store
#pragma unroll
        for (int q = 0; q < CB; ++q) {
            if (win[q]) {
                if (P.parent) __builtin_nontemporal_store(u[q], P.parent + v[q]);
                if (c.wbits) atomicOr(c.nbm + (v[q] >> 5), 1u << (v[q] & 31));
                if (c.wcf) {
                    const uint32_t cb = (uint32_t)v[q] >> P.cf_sh;
                    atomicOr(c.ncf + (cb >> 5), 1u << (cb & 31));
                }
                FBFS_ENQ(P, v[q]);
            }
            c.fcnt += win[q] ? 1 : 0;
            c.fdeg += win[q] ? len[q] - beg[q] : 0;
        }
        return;
    }
#pragma unroll
    for (int q = 0; q < CB; ++q) {
        if (win[q]) {
            P.dist[v[q]] = c.level + 1;
            if (P.parent) P.parent[v[q]] = u[q];
            if (c.wbits) atomicOr(c.nbm + (v[q] >> 5), 1u << (v[q] & 31));
            if (c.wcf) {
                const uint32_t cb = (uint32_t)v[q] >> P.cf_sh;
                atomicOr(c.ncf + (cb >> 5), 1u << (cb & 31));
            }
        }
    }
    if (c.region) {
#pragma unroll
        for (int q = 0; q < CB; ++q) stage_region(c, win[q], v[q], beg[q], len[q] - beg[q], a4[q]);
        return;
    }
#pragma unroll
    for (int q = 0; q < CB; ++q) stage(c, win[q], v[q], beg[q], len[q] - beg[q]);
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
// few registers live; both read the staged adjacency bounds from LDS.
__device__ __forceinline__ void flush(Ctx &c) {
    auto &sh = *c.sh;
    const Params &P = *c.P;
    __syncthreads();
    const int cnt = min(sh.cnt, CAP);
    constexpr int EPT = CAP / BLOCK;
    const int i0 = threadIdx.x * EPT;
    uint64_t tot0 = 0, tot1 = 0, tot2 = 0;
    for (int i = i0; i < min(i0 + EPT, cnt); ++i) {
        const int len = sh.slen[i];
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
        if (all != 0) {
            const unsigned long long base =
                atomicAdd(ctr_at(P, c.nslot, l * STRIPES + c.stripe), (unsigned long long)all);
            sh.list_base[l] = base;
            if (l != L_TILE) {
                // the chunks holding this flush's segments [b, b + cnt) of list l
                // (cnt <= min(CAP, n) <= 2^qk_sh: at most two), as the
                // difference storage - index for the indexes below and from
                // the second chunk's first one
                // Chunks whose first segment lies in the range are taken
                // before any wait for a chunk an earlier reservation holds:
                // the lists' threads share a wavefront, so a wait ahead of a
                // take would hold that take back, and two workgroups could
                // each wait for the other's
                const int64_t b = (int64_t)(base >> 32), e = b + (int64_t)(all >> 32) - 1;
                const int64_t j0 = b >> P.qk_sh, j1 = e >> P.qk_sh;
                const bool own0 = j0 == 0 || (j0 << P.qk_sh) >= b;
                int64_t c0 = -1, c1 = -1;
                if (b < (int64_t)P.n && own0) c0 = queue_chunk(c, l, j0, b);
                if (j1 != j0 && e < (int64_t)P.n) c1 = queue_chunk(c, l, j1, b);
                if (b < (int64_t)P.n && !own0) c0 = queue_chunk(c, l, j0, b);
                if (j1 == j0) c1 = c0;
                sh.qsplit[l] = (int32_t)((j0 + 1) << P.qk_sh);
                sh.qd[l][0] = (c0 >= 0) ? (int32_t)(c0 - (j0 << P.qk_sh)) : QD_NONE;
                sh.qd[l][1] = (c1 >= 0) ? (int32_t)(c1 - (j1 << P.qk_sh)) : QD_NONE;
            }
        }
        if (l == L_TILE) sh.ntiles = (int32_t)(all >> 32);
    } else if (threadIdx.x == NLISTS) {
        // the flushed vertices and their edges go straight into the level
        // tallies (the staged vertices of every list, whole or in pieces)
        uint64_t edges = 0;
        for (int l = 0; l < NLISTS; ++l)
            for (int w = 0; w < WAVES; ++w) edges += sh.scan_tmp[l][w] & 0xffffffffull;
        atomicAdd(ctr_at(P, c.nslot, VC_BASE + c.stripe), ((unsigned long long)cnt << 32) | edges);
    }
    __syncthreads();
    // small and mid vertices: one segment each, written by their thread; big
    // vertices: record where their pieces start, then the whole workgroup
    // writes the pieces (a hub can have hundreds)
    const uint64_t b0 = sh.list_base[L_SMALL], b1 = sh.list_base[L_MID];
    // where segment si of the small (mid) list of this flush is stored
    const int32_t sp0 = sh.qsplit[L_SMALL], d00 = sh.qd[L_SMALL][0], d01 = sh.qd[L_SMALL][1];
    const int32_t sp1 = sh.qsplit[L_MID], d10 = sh.qd[L_MID][0], d11 = sh.qd[L_MID][1];
    auto qdst = [&](int64_t si, int32_t sp, int32_t da, int32_t db) -> Seg * {
        const int32_t d = (si < sp) ? da : db;
        return d != QD_NONE ? c.nq + (si + d) : nullptr;
    };
    for (int i = i0; i < min(i0 + EPT, cnt); ++i) {
        const int v = sh.buf[i];
        const int beg = sh.sbeg[i];
        const int len = sh.slen[i];
        const int l = list_of(len);
        if (!c.converting) FBFS_ENQ(P, v);   // every staged vertex joins the tally above once
        sh.tstart[i] = (int32_t)(ex2 >> 32);
        sh.toff[i] = (int32_t)(ex2 & 0xffffffffull);
        if (l == L_SMALL) {
            const int64_t si = (int64_t)((b0 >> 32) + (ex0 >> 32));
            write_piece(c, l, si, v, beg, len, (int64_t)((b0 & 0xffffffffull) + (ex0 & 0xffffffffull)),
                        qdst(si, sp0, d00, d01));
            ex0 += (1ull << 32) | (uint32_t)len;
        } else if (l == L_MID) {
            const int64_t si = (int64_t)((b1 >> 32) + (ex1 >> 32));
            write_piece(c, l, si, v, beg, len, (int64_t)((b1 & 0xffffffffull) + (ex1 & 0xffffffffull)),
                        qdst(si, sp1, d10, d11));
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
            const int beg = sh.sbeg[lo];
            const int len = sh.slen[lo];
            const int pcs = gt - sh.tstart[lo];
            const int64_t si = tbase + gt;
            write_piece(c, L_TILE, si, v, beg + pcs * TILE, min(TILE, len - pcs * TILE),
                        ebase + sh.toff[lo] + (int64_t)pcs * TILE,
                        si < P.tcap ? c.nt + (size_t)c.stripe * P.tcap + si : nullptr);
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
    auto &sh = *c.sh;
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
    auto &sh = *c.sh;
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
            const Seg *sp = seg_slot(P, const_cast<Seg *>(cq), const_cast<Seg *>(ct), l, s, si, c.level);
            if (sp) {
                const Seg sg = *sp;
                v = sg.v; beg = sg.beg; len = sg.len;
                has = true;
                if (c.sh->clear_bm) cbm[v >> 5] = 0u;
            }
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
    auto &sh = *c.sh;
    int32_t *s_off = sh.work;
    int32_t *s_v = sh.work + (EB_TE + 1);
    int32_t *s_beg = sh.work + 2 * (EB_TE + 1);
    const int tiles = sh.uprefix[NLISTS * STRIPES];
    // fewer tiles than workgroups: each tile is cut into 2 or 4 parts, each
    // part one workgroup's unit (all parts stage the tile's segments)
    const int spl = (4 * tiles <= c.G) ? 4 : ((2 * tiles <= c.G) ? 2 : 1);
    const int total = tiles * spl;
    for (int u = c.wg; u < total; u += c.G) {
        const int ut = u / spl, part = u % spl;
        int r = 0;
        while (sh.uprefix[r + 1] <= ut) ++r;
        const int l = r / STRIPES, s = r % STRIPES;
        const int t = ut - sh.uprefix[r];
        const int E = sh.ledges[r];
        const int N = sh.lcount[r];
        const int a = t * EB_TE;
        const int pa = a + part * (EB_TE / spl);                 // this part's edges
        const int pb = min(pa + EB_TE / spl, E);                  // (at most STEP_CLAIMS winners)
        const int32_t *ts = cts + (size_t)r * P.tscap;
        // tile 0 starts at segment 0 (segments and edges are reserved together
        // from one counter, so the segment at index 0 holds edge offset 0): a
        // list with one tile needs no table read
        const int i0 = t ? ts[t] : 0;
        const int i1 = (a + EB_TE < E) ? ts[t + 1] : N - 1;
        int ns = i1 - i0 + 1;   // <= EB_TE + 1: every segment has an edge
        if (ns > EB_TE + 1 || ns < 1) {
            if (threadIdx.x == 0) set_err(P, ERR_TSTART_OVERFLOW, ns);
            ns = max(1, min(ns, EB_TE + 1));
        }
        for (int j = threadIdx.x; j < ns; j += BLOCK) {
            const Seg *sp = seg_slot(P, const_cast<Seg *>(cq), const_cast<Seg *>(ct), l, s, i0 + j, c.level);
            if (sp) {
                const Seg sg = *sp;
                s_off[j] = sg.off; s_v[j] = sg.v; s_beg[j] = sg.beg;
                if (sh.clear_bm) cbm[sg.v >> 5] = 0u;
            } else {
                sh.qbad = 1;   // a missing chunk (error recorded): the tile is skipped
            }
        }
        __syncthreads();
        if (sh.qbad) continue;   // uniform: every thread reads it after the barrier
        static_assert(EB_TE % BLOCK == 0 && EB_TE <= STEP_CLAIMS, "one step per tile");
        constexpr int NB = EB_TE / BLOCK;
        {
            const int e0 = pa + (int)threadIdx.x;
            int tv[NB], owner[NB];
            bool ok[NB];
#pragma unroll
            for (int q = 0; q < NB; ++q) {
                const int e = e0 + q * BLOCK;
                ok[q] = e < pb;
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
// wavefront reads 64 of the workgroup's bitmap words at a time (one per lane),
// lists the frontier vertices of its words in its own LDS region (up to
// FL_WAVE; the words that do not fit wait for the next round), and the
// workgroup expands the listed vertices as segments.  Both frontier bitmaps
// are zeroed on the way (this level writes no bitmap).
constexpr int FL_WAVE = FLIST_CAP / WAVES;

__device__ __forceinline__ void td_from_bitmap(Ctx &c, uint32_t *cbm, uint32_t *obm) {
    const Params &P = *c.P;
    auto &sh = *c.sh;
    const int lane = lane_id();
    const int wv = wave_id();
    int32_t *flist = sh.work + wv * FL_WAVE;
    uint64_t *cb64 = reinterpret_cast<uint64_t *>(cbm);
    uint64_t *ob64 = reinterpret_cast<uint64_t *>(obm);
    const int dfr = sh.dfr;
    uint64_t *lvi = sh.keep_in ? P.lvbm + (size_t)c.level * P.nwp : nullptr;
    const int per = (P.nwp + c.G - 1) / c.G;
    const int start = min(P.nwp, c.wg * per);
    const int end = min(P.nwp, start + per);
    for (int base = start; base < end; base += WAVES * WAVE) {
        const int w0 = base + wv * WAVE;
        const int wp = w0 + lane;
        uint64_t word = 0;
        if (wp < end) {
            word = cb64[wp];
            cb64[wp] = 0ull;
            ob64[wp] = 0ull;
            if (lvi) lvi[wp] = word;   // the frontier a queue-free level left, kept
        }
        uint64_t todo = __ballot(word != 0);
        for (;;) {
            // list the vertices of this wavefront's words, word by word, while they fit
            int cnt = 0;
            while (todo) {
                const int j = __ffsll((unsigned long long)todo) - 1;
                const uint32_t lo = (uint32_t)readlane_i((int)(uint32_t)word, j);
                const uint32_t hi = (uint32_t)readlane_i((int)(uint32_t)(word >> 32), j);
                const uint64_t wj = ((uint64_t)hi << 32) | lo;
                const int bits = __popcll(wj);
                if (cnt + bits > FL_WAVE) break;
                const bool in = (wj >> lane) & 1ull;
                const uint64_t m = __ballot(in);
                if (in) flist[cnt + mbcnt64(m)] = (w0 + j) * 64 + lane;
                // the frontier's dist, left by a queue-free level before
                if (in && dfr && (w0 + j) * 64 + lane < P.n) P.dist[(w0 + j) * 64 + lane] = c.level;
                cnt += bits;
                todo &= todo - 1;
            }
            if (lane == 0) { sh.fl_cnt[wv] = cnt; sh.fl_more[wv] = todo != 0; }
            __syncthreads();
            int maxc = 0, more = 0;
            for (int w = 0; w < WAVES; ++w) { maxc = max(maxc, sh.fl_cnt[w]); more |= sh.fl_more[w]; }
            // expand: pass p takes entry p*64 + lane of every wavefront's region
            for (int p0 = 0; p0 < maxc; p0 += WAVE) {
                const int i = p0 + lane;
                const bool has = i < sh.fl_cnt[wv] && flist[i] < P.n;
                int v = 0, beg = 0, len = 0;
                if (has) {
                    v = flist[i];
                    beg = P.row_ptr[v];
                    len = P.row_ptr[v + 1] - beg;
                }
                expand_segments(c, has && len > 0, v, beg, len);
                maybe_flush(c);
            }
            __syncthreads();
            if (!more) break;
        }
    }
}

// -------------------------------------------------------- bottom-up --------

// Every unvisited vertex looks for a parent: its first in-neighbour, in CSR
// order of the in-edge lists (the graph itself when symmetric, else its
// transpose), that is in the frontier bitmap.  Each wavefront owns a contiguous
// range of 64-vertex words and walks it 64 words at a time: it reads their
// visited words (one per lane), skips the fully visited ones and lists the
// unvisited vertices in LDS, BU_GSZ at a time.  Round 0 loads the aligned
// 8-entry block that holds every listed vertex's first entry and probes the
// first entry, then the rest of the block for the vertices still searching.  Each later
// round gives every vertex still without a parent its next min(W, rest)
// entries (W = 8, 32, 128, ... per round) and
// lays those probes out densely, 64 per instruction whatever the mix of list
// lengths: an exclusive scan of the counts and a binary search over it give
// each lane its (vertex, entry).  The first hit in CSR order is kept by an LDS
// atomicMin on the entry index.  When the frontier is a small share of the
// vertices, a coarse copy of it (one bit per 2^cf_sh vertices, set by the
// previous level's claims) sits in LDS and answers most probes without a
// memory access.  A wavefront owns whole 64-vertex words, so the next
// frontier's bitmap words and the visited words are plain stores: no global
// atomics and no duplicates.
__device__ __forceinline__ void wave_lds_sync() {
    // order this wavefront's LDS traffic between lanes (no workgroup barrier)
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int wave_incl_scan_i32(int x) {
    return (int)wave_incl_scan_u32((uint32_t)x);
}

constexpr int BU_NOHIT = 0x7fffffff;

// Can u be in the frontier?  (false only when its coarse bit is clear)
__device__ __forceinline__ bool cf_maybe(const BuLds &sh, int use_cf, int cf_sh, int u) {
    if (!use_cf) return true;
    const uint32_t b = (uint32_t)u >> cf_sh;
    return (sh.bu_cf[b >> 5] >> (b & 31)) & 1u;
}

// Entries of the aligned 8-entry block of col_idx that holds entry e, as x[q]
// = col_idx[blk + q]; entries outside [lo, hi) (or all, when !go) read as -1.
__device__ __forceinline__ void load_block8(const Params &P, bool go, int e, int lo, int hi,
                                            int (&x)[8]) {
    const int blk = e & ~7;
    if (go && P.in_col_vec && blk + 8 <= P.m) {
        const int4 a = *reinterpret_cast<const int4 *>(P.in_col_idx + blk);
        const int4 b = *reinterpret_cast<const int4 *>(P.in_col_idx + blk + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            x[q] = (go && blk + q >= lo && blk + q < hi) ? P.in_col_idx[blk + q] : -1;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
        if (!(go && blk + q >= lo && blk + q < hi)) x[q] = -1;
}

// The first entry of x (in order) that is in the frontier, else -1.  All
// probes are issued before any result is used.
__device__ __forceinline__ int probe_first(const BuLds &sh, const uint32_t *cbm, int use_cf,
                                           int cf_sh, const int (&x)[8]) {
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        w[q] = (x[q] >= 0 && cf_maybe(sh, use_cf, cf_sh, x[q])) ? cbm[x[q] >> 5] : 0u;
    int hit = -1;
#pragma unroll
    for (int q = 7; q >= 0; --q)
        if (x[q] >= 0 && ((w[q] >> (x[q] & 31)) & 1u)) hit = x[q];
    return hit;
}

// Records that listed vertex v found parent u (d = its in-degree; the
// frontier tally counts out-degrees, which differ on a directed graph).
__device__ __forceinline__ void bu_found(BuCtx &c, int wbase, int v, int u, int d, bool dstore) {
    const Params &P = *c.P;
    // v comes from this wavefront's own words [wbase, wbase + 64): anything
    // else is reported, never stored
    if ((uint32_t)v >= (uint32_t)P.n || (v >> 6) - wbase < 0 || (v >> 6) - wbase >= WAVE) {
        set_err(P, ERR_BAD_VERTEX, v);
        return;
    }
    if (!P.symmetric) d = P.row_ptr[v + 1] - P.row_ptr[v];
    FBFS_ENQ(P, v);
    // streaming, as in the word pass (dstore: dist is neither kept as a
    // bitmap nor written per word at the end after a queue-free level)
    if (dstore) __builtin_nontemporal_store(c.level + 1, P.dist + v);
    if (P.parent) __builtin_nontemporal_store(u, P.parent + v);
    atomicOr(&c.sh->bu_fm[wave_id()][(v >> 6) - wbase], 1ull << (v & 63));
    c.fcnt += 1;
    c.fdeg += d;
}

// Searches parents for the listed vertices lst[0, cnt) of this wavefront
// (all inside words [wbase, wbase + 64)).
__device__ __forceinline__ void bu_list(BuCtx &c, const uint32_t *cbm, int cnt, int wbase, bool dstore) {
    const Params &P = *c.P;
    auto &sh = *c.sh;
    const int lane = lane_id();
    const int wv = wave_id();
    const int use_cf = sh.use_cf, cf_sh = P.cf_sh;
    int32_t *lst = sh.bu_lst[wv], *deg = sh.bu_deg[wv], *hit = sh.bu_hit[wv];
    int32_t *pi = sh.bu_pi[wv], *pn = sh.bu_pn[wv], *pe = sh.bu_pe[wv], *ps = sh.bu_ps[wv];
    constexpr int R0 = BU_GSZ / WAVE;   // listed vertices per lane in round 0
    // round 0: every listed vertex's probe neighbour (its in-neighbour of
    // highest out-degree), from the probe-neighbour index read in vertex
    // order beside row_ptr, so no scattered adjacency line is fetched for the
    // vertices that stop there (entries with bit 31 set were probed there
    // already, in the word walk); then, for the vertices still searching with
    // more than one entry, the aligned 8-entry block of the list holding its
    // first entry (two 16-byte loads).  R0 vertices per lane with their loads
    // overlapped; a hit is recorded at once
    int npend = 0;
    {
        int v[R0], beg[R0], en[R0], par[R0];
        int x[R0][8];
        bool probed[R0];
#pragma unroll
        for (int j = 0; j < R0; ++j) {
            const int i = j * WAVE + lane;
            const int raw = (i < cnt) ? lst[i] : 0;
            probed[j] = i < cnt && raw < 0;
            v[j] = (i < cnt) ? (raw & 0x7fffffff) : -1;
        }
        {
            int f[R0];
            uint32_t w[R0];
#pragma unroll
            for (int j = 0; j < R0; ++j) {
                beg[j] = (v[j] >= 0) ? P.in_row_ptr[v[j]] : 0;
                en[j] = (v[j] >= 0) ? P.in_row_ptr[v[j] + 1] : 0;
                f[j] = (v[j] >= 0 && !probed[j]) ? P.pnb[v[j]] : -1;
            }
#pragma unroll
            for (int j = 0; j < R0; ++j)
                w[j] = (f[j] >= 0 && cf_maybe(sh, use_cf, cf_sh, f[j])) ? cbm[f[j] >> 5] : 0u;
#pragma unroll
            for (int j = 0; j < R0; ++j) par[j] = (f[j] >= 0 && ((w[j] >> (f[j] & 31)) & 1u)) ? f[j] : -1;
        }
        bool more = false;
#pragma unroll
        for (int j = 0; j < R0; ++j) more |= par[j] < 0 && beg[j] + 1 < en[j];
        if (__ballot(more)) {
#pragma unroll
            for (int j = 0; j < R0; ++j)
                load_block8(P, par[j] < 0 && beg[j] + 1 < en[j], beg[j], beg[j], en[j], x[j]);
#pragma unroll
            for (int j = 0; j < R0; ++j)
                if (par[j] < 0) par[j] = probe_first(sh, cbm, use_cf, cf_sh, x[j]);
        }
#pragma unroll
        for (int j = 0; j < R0; ++j) {
            const int i = j * WAVE + lane;
            const bool found = par[j] >= 0;
            if (found) bu_found(c, wbase, v[j], par[j], en[j] - beg[j], dstore);
            if (v[j] >= 0) {
                hit[i] = BU_NOHIT;
                deg[i] = en[j] - beg[j];
            }
            const int nx = (beg[j] | 7) + 1;   // first entry after the block
            const bool keep = v[j] >= 0 && !found && nx < en[j];
            const uint64_t m = __ballot(keep);
            if (keep) {
                const int p = npend + mbcnt64(m);
                pi[p] = i; pn[p] = nx; pe[p] = en[j];
            }
            npend += __popcll(m);
        }
    }
    if (npend == 0) return;
    // later rounds, dense
    for (int W = BU_W1; npend > 0; W = min(4 * W, BU_WMAX)) {
        wave_lds_sync();
        int T = 0;
        for (int b = 0; b < npend; b += WAVE) {
            const int i = b + lane;
            const int cc = (i < npend) ? min(pe[i] - pn[i], W) : 0;
            const int incl = wave_incl_scan_i32(cc);
            if (i < npend) ps[i] = T + incl - cc;
            T += readlane_i(incl, WAVE - 1);
        }
        wave_lds_sync();
        for (int t0 = 0; t0 < T; t0 += BU_U * WAVE) {
            int e[BU_U], own[BU_U], u[BU_U];
            uint32_t w[BU_U];
#pragma unroll
            for (int q = 0; q < BU_U; ++q) {
                const int slot = t0 + q * WAVE + lane;
                e[q] = -1;
                own[q] = 0;
                if (slot < T) {
                    // the pending vertex owning this slot: last p with ps[p] <= slot
                    // (every pending vertex has at least one entry left, so ps rises)
                    int lo = 0, hi = npend;
                    while (hi - lo > 1) {
                        const int mid = (lo + hi) >> 1;
                        if (ps[mid] <= slot) lo = mid; else hi = mid;
                    }
                    e[q] = pn[lo] + (slot - ps[lo]);
                    own[q] = pi[lo];
                }
            }
#pragma unroll
            for (int q = 0; q < BU_U; ++q) u[q] = (e[q] >= 0) ? P.in_col_idx[e[q]] : -1;
#pragma unroll
            for (int q = 0; q < BU_U; ++q)
                w[q] = (u[q] >= 0 && cf_maybe(sh, use_cf, cf_sh, u[q])) ? cbm[u[q] >> 5] : 0u;
#pragma unroll
            for (int q = 0; q < BU_U; ++q)
                if (u[q] >= 0 && ((w[q] >> (u[q] & 31)) & 1u)) atomicMin(&hit[own[q]], e[q]);
        }
        wave_lds_sync();
        // keep the vertices without a hit whose lists go on (in place: a
        // chunk reads its entries before writing at or below them)
        int nn = 0;
        for (int b = 0; b < npend; b += WAVE) {
            const int i = b + lane;
            bool keep = false;
            int a = 0, nx = 0, ee = 0;
            if (i < npend) {
                a = pi[i];
                ee = pe[i];
                nx = pn[i] + min(ee - pn[i], W);
                keep = hit[a] == BU_NOHIT && nx < ee;
            }
            const uint64_t m = __ballot(keep);
            if (keep) {
                const int p = nn + mbcnt64(m);
                pi[p] = a; pn[p] = nx; pe[p] = ee;
            }
            nn += __popcll(m);
        }
        npend = nn;
    }
    wave_lds_sync();
    // the vertices found in the later rounds: the neighbour at the first hit
    // (bit 31 of a list entry is the word walk's mark, not part of the id)
#pragma unroll
    for (int j = 0; j < R0; ++j) {
        const int i = j * WAVE + lane;
        const int h = (i < cnt) ? hit[i] : BU_NOHIT;
        if (h != BU_NOHIT) bu_found(c, wbase, lst[i] & 0x7fffffff, P.in_col_idx[h], deg[i], dstore);
    }
}

__device__ __forceinline__ void bottom_up(BuCtx &c, const uint32_t *cbm, uint32_t *nbm) {
    const Params &P = *c.P;
    auto &sh = *c.sh;
    const int lane = lane_id();
    const int wv = wave_id();
    if (sh.use_cf) {
        // the coarse frontier map, into LDS
        const uint32_t *cf = P.cf + (size_t)(c.level % 3) * CF_WORDS;
        for (int i = threadIdx.x; i < P.cf_words; i += BLOCK) sh.bu_cf[i] = cf[i];
        __syncthreads();
    }
    // this workgroup's words, then this wavefront's share of them
    const int per = (P.nwp + c.G - 1) / c.G;
    const int start = min(P.nwp, c.wg * per);
    const int end = min(P.nwp, start + per);
    const int wper = (end - start + WAVES - 1) / WAVES;
    const int ws = min(end, start + wv * wper);
    const int we = min(end, ws + wper);
    uint64_t *vis64 = reinterpret_cast<uint64_t *>(P.visited);
    uint64_t *nbm64 = reinterpret_cast<uint64_t *>(nbm);
    int32_t *lst = sh.bu_lst[wv];
    const int use_cf = sh.use_cf, cf_sh = P.cf_sh;
    const int dfr = sh.dfr, keep_out = sh.keep_out;
    const uint64_t *cb64 = reinterpret_cast<const uint64_t *>(cbm);
    // kept bitmaps: this level's finds (distance level + 1) and its frontier
    // when a queue-free level left it (distance level)
    uint64_t *lvo = keep_out ? P.lvbm + (size_t)(c.level + 1) * P.nwp : nullptr;
    uint64_t *lvi = sh.keep_in ? P.lvbm + (size_t)c.level * P.nwp : nullptr;
    constexpr int FW = 4;   // words probed together
    for (int cw = ws; cw < we; cw += WAVE) {
        const int nw = min(WAVE, we - cw);
        const uint64_t myvis = (lane < nw) ? vis64[cw + lane] : ~0ull;
        sh.bu_fm[wv][lane] = 0ull;
        // pass 1, over the words with at least BU_DENSE unvisited vertices,
        // FW words at a time with lane l on vertex l of each: the probe
        // neighbour and the in-list bounds (consecutive ids, coalesced), then
        // the frontier probe; a hit is recorded here, a miss with one
        // in-neighbour is settled.  Lane j keeps in myrest the vertices of
        // word j still to be listed: those left by pass 1 in a dense word,
        // every unvisited one in a sparse word
        const bool dense = lane < nw && __popcll(~myvis) >= BU_DENSE;
        uint64_t myrest = dense ? 0ull : ~myvis;
        // issue priority falls as the wavefront gets through its words (3 and
        // 2 over the halves of pass 1, 1 and 0 over those of pass 2): a
        // compute unit otherwise issues for its oldest wavefronts first, and
        // the workgroups placed last on it end the level well after the others
        const int nd_it = (__popcll(__ballot(dense)) + FW - 1) / FW;
        int d_it = 0;
        __builtin_amdgcn_s_setprio(3);
        for (uint64_t todo = __ballot(dense); todo;) {
            if (++d_it == nd_it / 2 + 1) __builtin_amdgcn_s_setprio(2);
            int jw[FW], v[FW], f[FW], dg[FW];
            uint32_t w[FW];
#pragma unroll
            for (int q = 0; q < FW; ++q) {
                jw[q] = todo ? __ffsll((unsigned long long)todo) - 1 : -1;
                todo &= todo - 1;
                bool act = false;
                if (jw[q] >= 0) {
                    const uint32_t lo = (uint32_t)readlane_i((int)(uint32_t)myvis, jw[q]);
                    const uint32_t hi = (uint32_t)readlane_i((int)(uint32_t)(myvis >> 32), jw[q]);
                    act = !(((((uint64_t)hi << 32) | lo) >> lane) & 1ull);   // padding bits are set
                }
                v[q] = act ? (cw + jw[q]) * 64 + lane : -1;
            }
#pragma unroll
            for (int q = 0; q < FW; ++q) {
                f[q] = (v[q] >= 0) ? P.pnb[v[q]] : -1;
                dg[q] = (v[q] >= 0) ? (int)P.deg8[v[q]] : 0;   // in-degree, 255 meaning 255 or more
            }
#pragma unroll
            for (int q = 0; q < FW; ++q)
                w[q] = (f[q] >= 0 && cf_maybe(sh, use_cf, cf_sh, f[q])) ? cbm[f[q] >> 5] : 0u;
            // a miss with more in-neighbours tries its second probe neighbour
            bool h1[FW];
            int f2[FW];
#pragma unroll
            for (int q = 0; q < FW; ++q) {
                h1[q] = f[q] >= 0 && ((w[q] >> (f[q] & 31)) & 1u);
                f2[q] = (!h1[q] && v[q] >= 0 && dg[q] > 1) ? P.snb[v[q]] : -1;
            }
#pragma unroll
            for (int q = 0; q < FW; ++q)
                w[q] = (f2[q] >= 0 && cf_maybe(sh, use_cf, cf_sh, f2[q])) ? cbm[f2[q] >> 5] : 0u;
#pragma unroll
            for (int q = 0; q < FW; ++q) {
                const int par = h1[q] ? f[q] : ((f2[q] >= 0 && ((w[q] >> (f2[q] & 31)) & 1u)) ? f2[q] : -1);
                const bool hitq = par >= 0 && v[q] < P.n;   // padding bits past n are set visited
                if (hitq) {
                    FBFS_ENQ(P, v[q]);
                    // outputs are never read back: streaming stores keep them
                    // out of the caches the pass reads through (dist is
                    // written per word at the end after a queue-free level,
                    // and not at all when the finds are kept as a bitmap)
                    if (!dfr && !keep_out) __builtin_nontemporal_store(c.level + 1, P.dist + v[q]);
                    if (P.parent) __builtin_nontemporal_store(par, P.parent + v[q]);
                    c.fcnt += 1;
                    c.fdeg += (P.symmetric && dg[q] < 255) ? dg[q] : P.row_ptr[v[q] + 1] - P.row_ptr[v[q]];
                }
                const uint64_t hm = __ballot(hitq);
                // two probes settle a vertex with two in-neighbours
                const uint64_t rm = __ballot(v[q] >= 0 && !hitq && dg[q] > 2);
                if (lane == jw[q]) {
                    myrest = rm;
                    if (hm) sh.bu_fm[wv][lane] = hm;
                }
            }
        }
        // pass 2: the vertices left, listed 128 at a time for bu_list (bit 31
        // marks those already probed at their probe neighbour)
        int cnt = 0;
        const uint64_t denses = __ballot(dense);
        const int n2 = readlane_i(wave_incl_scan_i32(__popcll(myrest)), WAVE - 1);
        int d2 = 0;
        __builtin_amdgcn_s_setprio(1);
        for (uint64_t tm = __ballot(myrest != 0ull); tm; tm &= tm - 1) {
            const int j = __ffsll((unsigned long long)tm) - 1;
            const uint32_t lo = (uint32_t)readlane_i((int)(uint32_t)myrest, j);
            const uint32_t hi = (uint32_t)readlane_i((int)(uint32_t)(myrest >> 32), j);
            const bool act = ((((uint64_t)hi << 32) | lo) >> lane) & 1ull;
            const uint64_t m = __ballot(act);
            if (cnt + __popcll(m) > BU_GSZ) {
                wave_lds_sync();
                bu_list(c, cbm, cnt, cw, !dfr && !keep_out);
                wave_lds_sync();
                d2 += cnt;
                if (2 * d2 >= n2) __builtin_amdgcn_s_setprio(0);
                cnt = 0;
            }
            if (act)
                lst[cnt + mbcnt64(m)] = ((cw + j) * 64 + lane) | (((denses >> j) & 1ull) ? (int)0x80000000 : 0);
            cnt += __popcll(m);
        }
        if (cnt > 0) {
            wave_lds_sync();
            bu_list(c, cbm, cnt, cw, !dfr && !keep_out);
        }
        wave_lds_sync();
        // the next-bitmap words (every word written) and visited words
        const uint64_t fm = (lane < nw) ? sh.bu_fm[wv][lane] : 0ull;
        if (lane < nw) {
            nbm64[cw + lane] = fm;
            if (fm) vis64[cw + lane] = myvis | fm;
        }
        if (lane < nw) {
            if (lvo) lvo[cw + lane] = fm;
            if (lvi) lvi[cw + lane] = cb64[cw + lane];
        }
        // past KCAP, after a queue-free level, dist in one store per word with
        // a change: the vertices found here and this level's frontier, which
        // that level left (its finds are spread thin, and this level's are
        // most of the rest: per word, each line is written once)
        const uint64_t fr = (dfr && lane < nw) ? cb64[cw + lane] : 0ull;
        for (uint64_t t = __ballot(dfr && (fm | fr) != 0ull); t; t &= t - 1) {
            const int j = __ffsll((unsigned long long)t) - 1;
            const uint32_t alo = (uint32_t)readlane_i((int)(uint32_t)fm, j);
            const uint32_t ahi = (uint32_t)readlane_i((int)(uint32_t)(fm >> 32), j);
            const uint32_t blo = (uint32_t)readlane_i((int)(uint32_t)fr, j);
            const uint32_t bhi = (uint32_t)readlane_i((int)(uint32_t)(fr >> 32), j);
            const bool hit = (((((uint64_t)ahi << 32) | alo) >> lane) & 1ull) != 0;
            const bool fro = (((((uint64_t)bhi << 32) | blo) >> lane) & 1ull) != 0;
            const int v = (cw + j) * 64 + lane;
            if ((hit || fro) && v < P.n) __builtin_nontemporal_store(hit ? c.level + 1 : c.level, P.dist + v);
        }
        wave_lds_sync();
    }
}

// ---------------------------------------------------------- kernels -------

// A top-down level whose frontier has fewer edges than this never turns to
// pull: a pull level passes over every vertex, which costs more than pushing
// a few edges, even when the edges left unexplored are fewer still (the last
// levels of a long search; on the grid they flipped direction every level).
__device__ __forceinline__ int64_t pull_floor(const Params &P) { return (int64_t)P.n >> 14; }

// Level 0 in the init kernel: a source of at most L0_MAX entries whose level
// is top-down.  Its winners are its distinct out-neighbours other than
// itself, known without a claim when the rows are sorted.  The fill
// workgroups write everything as for a search from level 0; then each one
// rewrites, in place, the entries it wrote that level 0 changes (dist and
// parent of the winners, their visited and next-frontier words, the coarse
// map of level 1), after a barrier, so those stores land after its own fill
// stores.  The last workgroup of the grid does no fill: it writes the control
// block and counters and either the source's queue entry or level 1's queue
// lists, counters and level 0's record.  The first level launch then starts
// at level 1, and the search has one launch fewer.
constexpr int L0_MAX = BLOCK;   // one entry per thread of the control workgroup

struct Level0 {
    int on;        // level 0 runs here
    int wb, wcf;   // it sets level 1's frontier bitmap / coarse map
};

// The decision decide() takes for level 0 (the same in every thread).
__device__ __forceinline__ Level0 level0_here(const Params &P, int d) {
    Level0 r{0, 0, 0};
    if (!P.l0_init || d < 0 || d > L0_MAX || (int64_t)d > (1LL << P.qk_sh) || P.pol_dir == BFS_DIR_PULL)
        return r;
    const bool pull = P.pol_dir == BFS_DIR_AUTO && (int64_t)d * P.alpha > (int64_t)P.m - d && d >= pull_floor(P);
    if (pull && P.can_pull) return r;
    r.on = 1;
    const double m_left = (double)((int64_t)P.m - d);
    r.wb = (P.can_pull && P.pol_dir == BFS_DIR_AUTO &&
            (double)P.max_deg * (double)d * (double)(P.alpha + 1) > m_left) ? 1 : 0;
    r.wcf = (r.wb && ((int64_t)d << P.cf_sh) <= 2 * (int64_t)P.n) ? 1 : 0;
    return r;
}

__global__ __launch_bounds__(BLOCK) void bfs_init_kernel(Params P) {
    __shared__ int32_t nsrc[L0_MAX];
    __shared__ uint64_t l0_tot[3][WAVES];
    __shared__ int32_t l0_cnt[WAVES];
    __shared__ int32_t l0_ts[L0_MAX], l0_beg[L0_MAX], l0_len[L0_MAX], l0_eo[L0_MAX];
    const int G = (int)gridDim.x - 1;   // fill workgroups (the launch adds the control one)
    const int s = P.source;
    // the source's row bounds: the fill below does not wait for them
    const int sb = P.row_ptr[s];
    const int d = P.row_ptr[s + 1] - sb;
    if ((int)blockIdx.x == G) {
        const Level0 l0 = level0_here(P, d);
        // control workgroup: every counter of every slot, the control block,
        // then level 0's output queue (the source's entry) or level 1's
        for (int i = threadIdx.x; i < NSLOTS * NCTR; i += BLOCK) P.ctr[(size_t)i * CTR_STRIDE] = 0ull;
        if (threadIdx.x == 0) {
            P.ctl->done = 0; P.ctl->L = 0; P.ctl->err = 0; P.ctl->err_info = 0;
            for (int i = 0; i < RAN_CAP; ++i) P.ctl->ran[i] = 0;
            P.ctl->lvl[0] = l0.on ? 1 : 0; P.ctl->lvl[1] = 0;
            P.ctl->kmask = 0u;
            for (int k = 0; k < NSLOTS; ++k) {
                P.ctl->slot[k].dir = 0; P.ctl->slot[k].wbits = 0; P.ctl->slot[k].wcf = 0;
                P.ctl->slot[k].input_bm = 0; P.ctl->slot[k].fsize = 0; P.ctl->slot[k].noq = 0;
                P.ctl->slot[k].reached_before = 0; P.ctl->slot[k].edges_before = 0;
            }
        }
        if (!l0.on) {
            __syncthreads();
            if (threadIdx.x == 0) {
                Ctx c;
                c.P = &P; c.sh = nullptr; c.level = -1; c.wg = 0; c.G = 1; c.stripe = 0; c.nslot = 0; c.wbits = 0;
                c.nbm = nullptr; c.ncf = nullptr; c.wcf = 0; c.noq = 0; c.nq = P.q0; c.nt = P.t0; c.nts = P.ts0;
                c.fcnt = 0; c.fdeg = 0; c.region = nullptr; c.converting = 0;
                const int l = list_of(d);
                if (l >= 0) {
                    const int nseg = (l == L_TILE) ? (d + TILE - 1) / TILE : 1;
                    P.ctr[(size_t)(l * STRIPES) * CTR_STRIDE] = ((unsigned long long)nseg << 32) | (unsigned)d;
                    write_vertex_segments(c, l, s, sb, d, 0, 0);
                }
                P.ctr[(size_t)VC_BASE * CTR_STRIDE] = (1ull << 32) | (unsigned)d;
            }
            return;
        }
        // level 1's queue lists (stripe 0) and counters, and level 0's record,
        // as run_level and flush leave them: thread t takes entry t of the
        // row, a winner when it is in [0, n) and neither the source nor the
        // entry before it (sorted row)
        const int t = threadIdx.x;
        if (t < d) nsrc[t] = P.col_idx[sb + t];
        __syncthreads();
        const int v = (t < d) ? nsrc[t] : -1;
        const bool win = t < d && v != s && (t == 0 || nsrc[t - 1] != v) && (uint32_t)v < (uint32_t)P.n;
        const int beg = win ? P.row_ptr[v] : 0;
        const int len = win ? P.row_ptr[v + 1] - beg : 0;
        const int l = win ? list_of(len) : -1;
        const uint64_t one = (l < 0) ? 0ull
                             : ((uint64_t)(l == L_TILE ? (len + TILE - 1) / TILE : 1) << 32) | (uint32_t)len;
        uint64_t in[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            in[q] = wave_incl_scan_u64(l == q ? one : 0ull);
            if (lane_id() == WAVE - 1) l0_tot[q][wave_id()] = in[q];
        }
        const int cin = wave_incl_scan_i32(win ? 1 : 0);
        if (lane_id() == WAVE - 1) l0_cnt[wave_id()] = cin;
        __syncthreads();
        uint64_t ex[3], all[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            ex[q] = in[q] - (l == q ? one : 0ull);
            all[q] = 0ull;
            for (int w = 0; w < WAVES; ++w) {
                if (w < wave_id()) ex[q] += l0_tot[q][w];
                all[q] += l0_tot[q][w];
            }
        }
        Ctx c;
        c.P = &P; c.sh = nullptr; c.level = 0; c.wg = 0; c.G = 1; c.stripe = 0; c.nslot = 1; c.wbits = l0.wb;
        c.nbm = nullptr; c.ncf = nullptr; c.wcf = l0.wcf; c.noq = 0; c.nq = P.q1; c.nt = P.t1; c.nts = P.ts1;
        c.fcnt = 0; c.fdeg = 0; c.region = nullptr; c.converting = 0;
        if (win && !P.fill_dist) P.dist[v] = 1;   // (with the fill, its rewrite stores it)
        if (l == L_SMALL || l == L_MID)
            write_vertex_segments(c, l, v, beg, len, (int64_t)(ex[l] >> 32), (int64_t)(ex[l] & 0xffffffffull));
        // hubs: their pieces, written by the whole workgroup (where each
        // entry's pieces start, then a search for the entry of piece gt)
        if (t < d) {
            l0_ts[t] = (int32_t)(ex[L_TILE] >> 32);
            l0_beg[t] = beg;
            l0_len[t] = (l == L_TILE) ? len : 0;
            l0_eo[t] = (int32_t)(ex[L_TILE] & 0xffffffffull);
        }
        __syncthreads();
        const int ntiles = (int)(all[L_TILE] >> 32);
        for (int gt = t; gt < ntiles; gt += BLOCK) {
            int lo = 0, hi = d;   // last entry whose pieces start at or before gt
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (l0_ts[mid] <= gt) lo = mid; else hi = mid;
            }
            const int pcs = gt - l0_ts[lo];
            const int64_t si = gt;
            write_piece(c, L_TILE, si, nsrc[lo], l0_beg[lo] + pcs * TILE, min(TILE, l0_len[lo] - pcs * TILE),
                        (int64_t)l0_eo[lo] + (int64_t)pcs * TILE, si < P.tcap ? c.nt + si : nullptr);
        }
        if (t == 0) {
            uint64_t winners = 0ull, edges = 0ull;
            for (int w = 0; w < WAVES; ++w) winners += (uint64_t)l0_cnt[w];
            for (int q = 0; q < 3; ++q) {
                *ctr_at(P, 1, q * STRIPES) = all[q];
                edges += all[q] & 0xffffffffull;
            }
            *ctr_at(P, 1, VC_BASE) = (winners << 32) | edges;
            if (P.level_sizes) P.level_sizes[0] = 1;
            if (P.st_cap > 0) { P.st_dir[0] = (int8_t)DIR_TD; P.st_fdeg[0] = d; }
            P.ctl->slot[0].dir = DIR_TD;
            P.ctl->slot[0].wbits = l0.wb;
            P.ctl->slot[0].wcf = l0.wcf;
            P.ctl->slot[0].fsize = 1;
            P.ctl->slot[1].reached_before = 1;
            P.ctl->slot[1].edges_before = d;
        }
        return;
    }
    const int tid = blockIdx.x * BLOCK + threadIdx.x;
    const int nth = G * BLOCK;
    // parent, and dist unless the finishing pass writes it: 16-byte
    // streaming stores (no level kernel reads them, and 8n bytes left in the
    // caches would evict what the levels read), entry by entry when the
    // caller's arrays are not 16-byte aligned.  Without the fill, the
    // source's dist is the one entry written here
    typedef int v4i __attribute__((ext_vector_type(4)));
    const int fill = P.fill_dist;
    const bool al = (((fill ? reinterpret_cast<uintptr_t>(P.dist) : 0) |
                      (P.parent ? reinterpret_cast<uintptr_t>(P.parent) : 0)) & 15) == 0;
    const int lim = (fill || P.parent) && al ? (P.n >> 2) : 0;
    {
        v4i *d4 = reinterpret_cast<v4i *>(P.dist);
        v4i *p4 = reinterpret_cast<v4i *>(P.parent);
        for (int i = tid; i < lim; i += nth) {
            v4i a = {-1, -1, -1, -1};
            v4i b = a;
            if ((s >> 2) == i) { a[s & 3] = 0; b[s & 3] = s; }
            if (fill) __builtin_nontemporal_store(a, d4 + i);
            if (P.parent) __builtin_nontemporal_store(b, p4 + i);
        }
        if (fill || P.parent) {
            for (int i = 4 * lim + tid; i < P.n; i += nth) {
                if (fill) P.dist[i] = (i == s) ? 0 : -1;
                if (P.parent) P.parent[i] = (i == s) ? s : -1;
            }
        }
        if (!fill && tid == 0) P.dist[s] = 0;
    }
    uint64_t *vis64 = reinterpret_cast<uint64_t *>(P.visited);
    const uint64_t *init64 = reinterpret_cast<const uint64_t *>(P.vis_init);
    uint64_t *b0 = reinterpret_cast<uint64_t *>(P.fbm0);
    uint64_t *b1 = reinterpret_cast<uint64_t *>(P.fbm1);
    for (int i = tid; i < 3 * CF_WORDS; i += nth) P.cf[i] = 0u;
    // queue chunk tables: entries of an earlier search must not match a tag
    for (int64_t i = tid; i < (int64_t)NSLOTS * 2 * STRIPES * P.qpool; i += nth) P.qtab[i] = 0ull;
    for (int i = tid; i < 2 * SMALL_G; i += nth) P.sslot[i] = 0ull;
#ifdef FBFS_COUNT_ENQUEUES
    if (P.enq)
        for (int i = tid; i < P.n; i += nth) P.enq[i] = 0;
#endif
    for (int wp = tid; wp < P.nwp; wp += nth) {
        const uint64_t sbit = (wp == (s >> 6)) ? (1ull << (s & 63)) : 0ull;
        vis64[wp] = init64[wp] | sbit;
        b0[wp] = sbit;
        b1[wp] = 0ull;
    }
    const Level0 l0 = level0_here(P, d);
    if (!l0.on) return;
    // level 0's changes to what this workgroup wrote: an entry is rewritten
    // by the workgroup of the thread that wrote it (entry e of a grid-stride
    // loop: thread e % nth), once its own stores are ordered before by the
    // barrier (each thread's fill stores complete before it)
    for (int j = threadIdx.x; j < d; j += BLOCK) nsrc[j] = P.col_idx[sb + j];
    // (a wait for this thread's stores, not an agent-scope release: that
    // would write back the whole L2 of the workgroup's die)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int me = blockIdx.x;
    auto mine = [&](int64_t e) { return (int)((e % nth) / BLOCK) == me; };
    for (int j = threadIdx.x; j < d; j += BLOCK) {
        const int v = nsrc[j];
        if ((uint32_t)v >= (uint32_t)P.n) continue;
        const int pv = j > 0 ? nsrc[j - 1] : -1;
        if (v != s && pv != v) {
            // dist and parent: quad v/4 of the vector loop, else entry v - 4*lim of the scalar one
            const int64_t e = ((v >> 2) < lim) ? (int64_t)(v >> 2) : (int64_t)v - 4LL * lim;
            if ((fill || P.parent) && mine(e)) {
                if (fill) P.dist[v] = 1;
                if (P.parent) P.parent[v] = s;
            }
#ifdef FBFS_COUNT_ENQUEUES
            if (P.enq && mine(v)) P.enq[v] = 1;   // level 0's winner, enqueued once
#endif
        }
        // the visited and next-frontier word of v, from the first entry in it
        const int wp = v >> 6;
        if ((j == 0 || (pv >> 6) != wp || pv < 0) && mine(wp)) {
            uint64_t nb = 0ull;
            for (int jj = j; jj < d && nsrc[jj] >= 0 && (nsrc[jj] >> 6) == wp; ++jj)
                if (nsrc[jj] != s && nsrc[jj] < P.n) nb |= 1ull << (nsrc[jj] & 63);
            const uint64_t sbit = (wp == (s >> 6)) ? (1ull << (s & 63)) : 0ull;
            vis64[wp] = init64[wp] | sbit | nb;
            if (l0.wb) b1[wp] = nb;
        }
        // level 1's coarse map word (map 1), from the first entry in it
        if (l0.wcf) {
            const int cw = (int)(((uint32_t)v >> P.cf_sh) >> 5);
            const bool first = j == 0 || pv < 0 || (int)(((uint32_t)pv >> P.cf_sh) >> 5) != cw;
            if (first && mine(CF_WORDS + cw)) {
                uint32_t w = 0u;
                for (int jj = j; jj < d && nsrc[jj] >= 0 && (int)(((uint32_t)nsrc[jj] >> P.cf_sh) >> 5) == cw; ++jj)
                    if (nsrc[jj] != s && nsrc[jj] < P.n) w |= 1u << (((uint32_t)nsrc[jj] >> P.cf_sh) & 31u);
                P.cf[CF_WORDS + cw] = w;
            }
        }
    }
    // level 0's frontier bitmap is read only when level 0 pulls: the source's bit goes
    if (threadIdx.x == 0 && mine(s >> 6)) b0[s >> 6] = 0ull;
}

// Decision for level k, taken by wavefront 0 of every workgroup from the
// counters the previous level left (identical in every workgroup); the
// caller synchronises before reading it.

__device__ __forceinline__ void decide(const Params &P, LevelCommon &sh, int k) {
    const int lane = lane_id();
    const int slot = k % NSLOTS;
    // every word the decision reads is loaded here, before any is used, so
    // the wavefront waits out one memory round trip instead of a chain of them
    unsigned long long cv = 0;
    if (lane < NCTR) cv = *ctr_at(P, slot, lane);
    int done = 0, err = 0, cf_prev2 = 0;
    SlotInfo prev{0, 0, 0, 0, 0, 0, 0};
    int64_t reached_before = 0, edges_before = 0;
    if (lane == 0) {
        done = P.ctl->done;
        err = P.ctl->err;
        // the coarse map of level k+2 was written by level k-2 if it set wcf
        // (the slot ring still holds level k-2's record at level k)
        if (k >= 2) cf_prev2 = P.ctl->slot[(k + NSLOTS - 2) % NSLOTS].wcf;
        if (k > 0) {
            prev = P.ctl->slot[(k + NSLOTS - 1) % NSLOTS];
            reached_before = P.ctl->slot[slot].reached_before;
            edges_before = P.ctl->slot[slot].edges_before;
        }
    }
    const bool is_vc = lane >= VC_BASE && lane < VC_BASE + STRIPES;
    // |F| <= n and deg(F) <= m, both below 2^31: 32-bit sums, read from the
    // last lane of the scans
    const int64_t fsize = (uint32_t)readlane_i(
        (int)wave_incl_scan_u32(is_vc ? (uint32_t)(cv >> 32) : 0u), WAVE - 1);
    const int64_t fdeg = (uint32_t)readlane_i(
        (int)wave_incl_scan_u32(is_vc ? (uint32_t)(cv & 0xffffffffull) : 0u), WAVE - 1);
    if (lane < VC_BASE) {
        sh.lcount[lane] = (int32_t)(cv >> 32);
        sh.ledges[lane] = (int32_t)(cv & 0xffffffffull);
    }
    if (lane == 0) {
        sh.fsize = (int32_t)fsize; sh.fdeg = fdeg;
        sh.prev_wcf = prev.wcf;
        sh.prev_fdeg = (k > 0) ? edges_before - prev.edges_before : 0;
        sh.small = 0;
        sh.use_cf = 0;
        sh.noq = 0;
        // the frontier a queue-free level left: kept as a bitmap below KCAP,
        // else its dist is written by this level
        sh.keep_in = (!P.fill_dist && k > 0 && prev.noq && k < KCAP) ? 1 : 0;
        sh.dfr = (k > 0 && prev.noq && !sh.keep_in) ? 1 : 0;
        sh.keep_out = 0;
        sh.cf_clear = cf_prev2;
        if (done || err) {
            sh.mode = 0;
        } else if (fsize == 0) {
            sh.mode = 1;
        } else {
            sh.mode = 2;
            const bool has_queue = (k == 0) || (prev.dir == DIR_TD && !prev.noq);
            const bool has_bm = (k == 0) || prev.dir == DIR_BU || prev.wbits;
            bool want_pull;
            if (P.pol_dir == BFS_DIR_PULL) {
                want_pull = true;
            } else if (P.pol_dir == BFS_DIR_PUSH) {
                want_pull = false;
            } else if (k == 0 || prev.dir == DIR_TD) {
                // edges still to be explored from unvisited vertices
                const int64_t m_u = (int64_t)P.m - edges_before - fdeg;
                want_pull = fdeg * P.alpha > m_u && fdeg >= pull_floor(P);
            } else {
                want_pull = !(fsize * P.beta < (int64_t)P.n && fsize < prev.fsize);
            }
            const int dir = (want_pull && P.can_pull && has_bm) ? DIR_BU : DIR_TD;
            sh.dir = dir;
            sh.keep_out = (!P.fill_dist && dir == DIR_BU && k + 1 < KCAP) ? 1 : 0;
            sh.reached_before = reached_before;
            sh.edges_before = edges_before;
            sh.input_bm = (dir == DIR_TD) && !has_queue;
            sh.clear_bm = (dir == DIR_TD) && has_queue && has_bm;
            // a top-down level from a queue also sets its new vertices in the
            // next bitmap whenever the next level may pull.  The next level
            // pulls when alpha*deg(F') > m - (edges reached so far) - deg(F'),
            // and deg(F') <= max_deg*|F'| <= max_deg*deg(F), so levels for
            // which even that bound cannot tip the rule skip the bit writes.
            const int64_t m_left = (int64_t)P.m - edges_before - fdeg;
            const bool may_pull = (double)P.max_deg * (double)fdeg * (double)(P.alpha + 1) > (double)m_left;
            sh.wbits = (dir == DIR_TD) && has_queue && P.can_pull && P.pol_dir == BFS_DIR_AUTO && may_pull;
            // edge-balanced unless the binned advance is forced: its tiles
            // spread even a small frontier over several workgroups and
            // bound the winners between flushes
            sh.adv_eb = (dir == DIR_TD) && has_queue && P.pol_adv != BFS_ADV_BINNED;
            sh.small = P.small_mode && (dir == DIR_TD) && has_queue && fsize <= SMALL_F && fdeg <= SMALL_E;
            // the coarse frontier map exists when the previous level set it (a
            // top-down level with wcf); it filters well while the frontier
            // covers under about two vertices per coarse bit
            sh.use_cf = (dir == DIR_BU) && k > 0 && prev.dir == DIR_TD && prev.wcf &&
                        (fsize << P.cf_sh) <= 2 * (int64_t)P.n;
            // a top-down level sets the next coarse map only when its edges (a
            // bound on the next frontier) are few enough for the map to filter
            sh.wcf = sh.wbits && (fdeg << P.cf_sh) <= 2 * (int64_t)P.n;
            // a wide level whose next level may pull writes its new vertices
            // to the next bitmap only: the pull needs no queue, and should
            // the next level stay top-down it reads the bitmap, as after a
            // bottom-up level
            sh.noq = sh.wbits && !sh.small && fdeg >= NOQ_EDGES;
        }
    }
}

// This workgroup's per-thread tallies of new frontier vertices (and their
// edges) into one striped atomic of the next level's vertex counters.
template <class S>
__device__ __forceinline__ void add_tallies(CtxT<S> &c) {
    auto &sh = *c.sh;
    const int lane = lane_id();
    // a workgroup's vertices and their edges number below 2^31: 32-bit scans
    const int64_t wc = (uint32_t)readlane_i((int)wave_incl_scan_u32((uint32_t)c.fcnt), WAVE - 1);
    const int64_t wd = (uint32_t)readlane_i((int)wave_incl_scan_u32((uint32_t)c.fdeg), WAVE - 1);
    __syncthreads();
    if (lane == 0) { sh.scan_tmp[0][wave_id()] = (uint64_t)wc; sh.scan_tmp[1][wave_id()] = (uint64_t)wd; }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t tc = 0, td = 0;
        for (int w = 0; w < WAVES; ++w) { tc += sh.scan_tmp[0][w]; td += sh.scan_tmp[1][w]; }
        if (tc) atomicAdd(ctr_at(*c.P, c.nslot, VC_BASE + c.stripe), (unsigned long long)((tc << 32) | td));
    }
}

// Will a small level's winners make a small frontier again?  The next
// frontier's edges are predicted as this level's edges times their growth
// since the level before: a level that grows out of the small-frontier mode
// writes the queue lists at once and ends the launch, instead of its
// workgroups publishing regions and converting them afterwards.
__device__ __forceinline__ bool grows_out(int64_t fdeg, int64_t fprev) {
    const double g = (double)fdeg / (double)(fprev > 0 ? fprev : 1);
    return (double)fdeg * (g > 1.0 ? g : 1.0) > (double)SMALL_E;
}

// Unit prefix tables of a level read from the queue lists: one lane per
// (list, stripe) and a wavefront scan (a serial loop here waits out one LDS
// round trip per entry).  The caller synchronises before using them.
__device__ __forceinline__ void unit_prefix(LevelCommon &sh) {
    if (threadIdx.x < WAVE) {
        const int r = threadIdx.x;
        int units = 0;
        if (r < NLISTS * STRIPES) {
            const int l = r / STRIPES;
            if (sh.adv_eb) units = (sh.ledges[r] + EB_TE - 1) / EB_TE;
            else if (l == L_TILE) units = sh.lcount[r];
            else if (l == L_MID) units = (sh.lcount[r] + WAVES - 1) / WAVES;
            else units = (sh.lcount[r] + BLOCK - 1) / BLOCK;
        }
        const int incl = wave_incl_scan_i32(units);
        if (r < NLISTS * STRIPES) sh.uprefix[r] = incl - units;
        if (r == NLISTS * STRIPES - 1) sh.uprefix[NLISTS * STRIPES] = incl;
    }
}

// One level on the G workgroups taking part (this one is number wg); BU
// selects the direction's code (the decision in sh must agree).
template <bool BU, class S>
__device__ __forceinline__ void run_level(const Params &P, S &sh, int k, int wg, int G, bool to_region = false) {
    const int lane = lane_id();
    const int slot = k % NSLOTS;
    if constexpr (!BU) {
        if (threadIdx.x == 0) {
            sh.cnt = 0;
            sh.spilled = 0;
            sh.nbig = 0;
            sh.rpack[(k + 1) & 1] = 0ull;
            sh.rbig[(k + 1) & 1] = 0;
            sh.inl[(k + 1) & 1] = 1;
            sh.qbad = 0;
            // a visited-word load before each claim pays on levels with many
            // edges (it spares the atomics of targets already reached)
            sh.vfilter = sh.fdeg >= VFILTER_EDGES;
        }
    }
    unit_prefix(sh);
    // bookkeeping of level k by workgroup 0
    if (wg == 0) {
        if (threadIdx.x == 0) {
            if (P.level_sizes) P.level_sizes[k] = sh.fsize;
            if (k < P.st_cap) {
                // direction in bit 0; above it where the level's dist stores went
                // (the level flags of the host interface)
                const int fl = (sh.noq ? 1 : 0) | (sh.keep_out ? 2 : 0) | (sh.keep_in ? 4 : 0) | (sh.dfr ? 8 : 0);
                P.st_dir[k] = (int8_t)(sh.dir | (fl << 1));
                P.st_fdeg[k] = sh.fdeg;
            }
            P.ctl->slot[slot].dir = sh.dir;
            P.ctl->slot[slot].wbits = sh.wbits;
            P.ctl->slot[slot].wcf = sh.wcf;
            P.ctl->slot[slot].input_bm = sh.input_bm;
            P.ctl->slot[slot].fsize = sh.fsize;
            P.ctl->slot[slot].noq = sh.noq;
            if (sh.keep_in || sh.keep_out)
                atomicOr(&P.ctl->kmask, (sh.keep_in ? 1u << k : 0u) | (sh.keep_out ? 1u << (k + 1) : 0u));
            P.ctl->slot[(k + 1) % NSLOTS].reached_before = sh.reached_before + sh.fsize;
            P.ctl->slot[(k + 1) % NSLOTS].edges_before = sh.edges_before + sh.fdeg;
        }
        if (threadIdx.x < NCTR) *ctr_at(P, (k + 2) % NSLOTS, threadIdx.x) = 0ull;
    }
    __syncthreads();

    CtxT<S> c;
    c.P = &P;
    c.sh = &sh;
    c.level = k;
    c.wg = wg;
    c.G = G;
    c.stripe = wg % STRIPES;
    c.nslot = (k + 1) % NSLOTS;
    c.wbits = sh.wbits;
    c.wcf = sh.wcf;
    c.noq = sh.noq;
    // the small-frontier mode's first level: winners to this workgroup's region
    c.region = to_region ? P.sreg + ((size_t)((k + 1) & 1) * SMALL_G + wg) * SREG_CAP : nullptr;
    c.converting = 0;
    const int cur = k & 1;
    uint32_t *cbm = cur ? P.fbm1 : P.fbm0;
    uint32_t *obm = cur ? P.fbm0 : P.fbm1;
    c.nbm = obm;
    c.ncf = P.cf + (size_t)((k + 1) % 3) * CF_WORDS;
    if (sh.cf_clear) {
        // clear the coarse map of level k+2: level k-2 wrote it (when its
        // wcf was set), level k-1 was its last reader and level k+1 is its
        // first writer
        uint32_t *z = P.cf + (size_t)((k + 2) % 3) * CF_WORDS;
        for (int i = wg * BLOCK + (int)threadIdx.x; i < P.cf_words; i += G * BLOCK) z[i] = 0u;
    }
    c.nq = cur ? P.q0 : P.q1;
    c.nt = cur ? P.t0 : P.t1;
    c.nts = cur ? P.ts0 : P.ts1;
    c.fcnt = 0;
    c.fdeg = 0;
    const Seg *cq = cur ? P.q1 : P.q0;
    const Seg *ct = cur ? P.t1 : P.t0;
    const int32_t *cts = cur ? P.ts1 : P.ts0;

    if constexpr (BU) {
        bottom_up(c, cbm, obm);
    } else {
        if (sh.input_bm) td_from_bitmap(c, cbm, obm);
        else if (sh.adv_eb) td_edge_balanced(c, cq, ct, cts, cbm);
        else td_binned(c, cq, ct, cbm);
        if (sh.cnt > 0) flush(c);
    }

    // workgroup tallies -> one striped atomic (a top-down level's flushes
    // added theirs already; only direct appends are left)
    if constexpr (!BU) {
        if (!sh.spilled && !sh.noq) return;
    }
    add_tallies(c);
}

// Small-frontier mode: top-down levels k, k+1, ... on the first G
// workgroups while they stay small (at most SMALL_F vertices and SMALL_E
// edges) and top-down, so that a long thin search needs few launches.  Per
// level, each workgroup appends the vertices it wins to its own region (no
// shared reservation), then publishes one 64-bit word {level, count, edges}
// after a release; every workgroup waits for all G words of the level with
// an acquire.  Those words are the barrier, and they also give the next
// level's size and work split: each workgroup takes an equal share of the
// frontier's entries, located from the prefix of the counts, and expands them
// lane, wavefront or workgroup per entry by degree.  Level k itself reads
// the queue lists the launch started from.  When the next level is not small
// (or pulls), each workgroup converts its region into that level's queue
// lists and counters with the usual flush, and the next launch takes over.
// The wait for the words is bounded: past the limit the search ends with
// ERR_BARRIER_TIMEOUT.  Returns the level the next launch starts at, or -1
// when this launch found the empty frontier or an error was recorded.
// word layout: bits 40-63 level + 1 (24 bits), 25-39 winners (at most
// SMALL_E), 24 a winner has at least T_WG edges, 0-23 their edges
// (saturating at 2^24 - 1, far above SMALL_E)
constexpr uint32_t SW_SEQ_MASK = 0xffffffu;
constexpr unsigned long long SW_EDGE_MAX = 0xffffffull;

__device__ __forceinline__ int run_small(const Params &P, TdLds &sh, int k, int launch, int G) {
    const int wg = blockIdx.x;
    const int lane = lane_id();
    // level k has run (run_level, its winners in the regions); the level
    // state as decide() left it, carried in registers from level to level
    // (uniform in the workgroup)
    int fsize = sh.fsize, wbits = sh.wbits, wcf = sh.wcf, prev_wcf = sh.prev_wcf;
    int64_t fdeg = sh.fdeg, reached_before0 = sh.reached_before, edges_before0 = sh.edges_before;
    for (;;) {
        const int cur = k & 1;
        // publish this workgroup's winners of level k+1
        const uint32_t want = (uint32_t)(k + 1) & SW_SEQ_MASK;
        unsigned long long *words = P.sslot + (size_t)((k + 1) & 1) * SMALL_G;
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned long long rp = sh.rpack[(k + 1) & 1];
            const unsigned long long cnt = min(rp >> 40, (unsigned long long)SREG_CAP);
            const unsigned long long ed = min(rp & RP_EDGES, SW_EDGE_MAX);
            const unsigned long long big = sh.rbig[(k + 1) & 1] ? 1ull : 0ull;
            // the counts of level k's winners are read (published, and
            // taken as own-mode entries) by now: cleared for level k+2's,
            // which the next expansion stages after the barrier below
            sh.rpack[k & 1] = 0ull;
            sh.rbig[k & 1] = 0;
            sh.inl[k & 1] = 1;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __hip_atomic_store(words + wg, ((unsigned long long)want << 40) | (cnt << 25) | (big << 24) | ed,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // wait for every workgroup's word: lane w polls workgroup w's
        if (threadIdx.x < WAVE) {
            const bool mine = lane < G;
            unsigned long long word = 0ull;
            int errv = 0;
            bool late = false;
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            for (;;) {
                // lane G reads the error word beside the others' words (G <= SMALL_G < WAVE)
                if (mine) word = __hip_atomic_load(words + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                else if (lane == G) errv = __hip_atomic_load(&P.ctl->err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const bool ok = !mine || (uint32_t)(word >> 40) == want;
                if (__ballot(!ok) == 0ull) break;
                __builtin_amdgcn_s_sleep(1);
                if (__builtin_amdgcn_s_memrealtime() - t0 > P.barrier_ticks) {
                    late = true;
                    break;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            const int cnt = mine ? (int)((word >> 25) & 0x7fffull) : 0;
            const bool anybig = __ballot(mine && ((word >> 24) & 1ull)) != 0ull;
            const uint32_t ed = mine ? (uint32_t)(word & SW_EDGE_MAX) : 0u;   // G * 2^24 < 2^32
            // every workgroup's winners have at most one edge per thread:
            // each expands its own (a workgroup with two claims per thread
            // took over 2 us longer on the grid, more than the region read
            // an equal split costs)
            const bool own = __ballot(mine && (cnt > OWN_CAP || ed > (uint32_t)BLOCK)) == 0ull;
            const bool err_seen = readlane_i(errv, G) != 0;
            const int incl = wave_incl_scan_i32(cnt);
            const uint32_t eincl = wave_incl_scan_u32(ed);
            // cross-lane reads in uniform control flow: inside a branch on
            // the lane, the scans' last steps may be left to that lane only
            const int total = readlane_i(incl, WAVE - 1);
            const uint32_t etotal = (uint32_t)readlane_i((int)eincl, WAVE - 1);
            if (mine) sh.spre[lane] = incl - cnt;
            if (lane == 0) {
                if (late) atomicCAS(&P.ctl->err, 0, ERR_BARRIER_TIMEOUT);
                sh.spre[G] = total;
                sh.s_total = total;
                sh.s_edges = etotal;
                sh.s_big = anybig;
                sh.s_own = own;
                sh.s_err = late || err_seen;
            }
        }
        __syncthreads();
        if (sh.s_err) return -1;
        const int F1 = sh.s_total;
        const int64_t E1 = (int64_t)sh.s_edges;
        const int64_t reached_before = reached_before0 + fsize;
        const int64_t edges_before = edges_before0 + fdeg;
        if (F1 == 0) {
            if (wg == 0 && threadIdx.x == 0) {
                P.ctl->L = k + 1;
                P.ctl->done = 1;
                if (launch < RAN_CAP) P.ctl->ran[launch] = 1;
            }
            return -1;
        }
        // the direction of level k+1, as decide() takes it after a top-down
        // level (edges saturate only above SMALL_E, where the next launch
        // decides again from the exact counters)
        const int64_t m_u = (int64_t)P.m - edges_before - E1;
        const bool want_pull = P.pol_dir == BFS_DIR_PULL ||
                               (P.pol_dir == BFS_DIR_AUTO && E1 * P.alpha > m_u && E1 >= pull_floor(P));
        const bool pull = want_pull && P.can_pull && wbits;   // level k set the next bitmap
        Ctx c;
        c.P = &P; c.sh = &sh; c.level = k; c.wg = wg; c.G = G; c.stripe = wg % STRIPES;
        c.nslot = (k + 1) % NSLOTS; c.wbits = wbits; c.wcf = wcf; c.noq = 0;
        c.nbm = cur ? P.fbm0 : P.fbm1;
        c.ncf = P.cf + (size_t)((k + 1) % 3) * CF_WORDS;
        c.nq = cur ? P.q0 : P.q1; c.nt = cur ? P.t0 : P.t1; c.nts = cur ? P.ts0 : P.ts1;
        c.fcnt = 0; c.fdeg = 0;
        // a vertex of T_WG or more edges in the next frontier: the regions
        // are dealt out by entries, which would leave its list to one
        // workgroup, so the next launch takes the level, edge-balanced
        if (pull || !P.small_mode || F1 > SMALL_F || E1 > SMALL_E || sh.s_big) {
            // level k+1's frontier into its queue lists and counters
            c.region = nullptr;
            c.converting = 1;
            const int4 *rg = P.sreg + ((size_t)((k + 1) & 1) * SMALL_G + wg) * SREG_CAP;
            const int total = (int)min(sh.rpack[(k + 1) & 1] >> 40, (unsigned long long)SREG_CAP);
            for (int b0 = 0; b0 < total; b0 += CAP) {
                const int nb = min(CAP, total - b0);
                for (int i = threadIdx.x; i < nb; i += BLOCK) {
                    const int4 e = rg[b0 + i];
                    sh.buf[i] = e.x; sh.sbeg[i] = e.y; sh.slen[i] = e.z;
                }
                if (threadIdx.x == 0) sh.cnt = nb;
                flush(c);   // begins with a barrier
            }
            return k + 1;
        }
        // level k+1: small and top-down; its winners go to the regions, or
        // to the queue lists when they are predicted not to be small (then
        // the launch ends after it)
        const bool to_queue = grows_out(E1, fdeg);
        const int64_t m_left = (int64_t)P.m - edges_before - E1;
        const bool may_pull = (double)P.max_deg * (double)E1 * (double)(P.alpha + 1) > (double)m_left;
        const int wbits1 = (P.can_pull && P.pol_dir == BFS_DIR_AUTO && may_pull) ? 1 : 0;
        const int clear_bm = wbits;    // level k's bits are level k+1's frontier bitmap
        const int cf_clear = prev_wcf;   // level k-1 wrote the coarse map of level k+3
        const int wcf1 = (wbits1 && (E1 << P.cf_sh) <= 2 * (int64_t)P.n) ? 1 : 0;
        ++k;
        const int nc = k & 1;
        uint32_t *cbm = nc ? P.fbm1 : P.fbm0;
        // bookkeeping of level k by workgroup 0 (as a full-grid level's)
        if (wg == 0) {
            if (threadIdx.x == 0) {
                const int slot = k % NSLOTS;
                if (P.level_sizes) P.level_sizes[k] = F1;
                if (k < P.st_cap) { P.st_dir[k] = (int8_t)DIR_TD; P.st_fdeg[k] = E1; }
                P.ctl->slot[slot].dir = DIR_TD;
                P.ctl->slot[slot].wbits = wbits1;
                P.ctl->slot[slot].wcf = wcf1;
                P.ctl->slot[slot].input_bm = 0;
                P.ctl->slot[slot].fsize = F1;
                P.ctl->slot[slot].noq = 0;
                P.ctl->slot[(k + 1) % NSLOTS].reached_before = reached_before + F1;
                P.ctl->slot[(k + 1) % NSLOTS].edges_before = edges_before + E1;
            }
            if (threadIdx.x < NCTR) *ctr_at(P, (k + 2) % NSLOTS, threadIdx.x) = 0ull;
        }
        if (cf_clear) {
            // the coarse map of level k+2: level k-2 wrote it, level k-1 read it
            uint32_t *z = P.cf + (size_t)((k + 2) % 3) * CF_WORDS;
            for (int i = wg * BLOCK + (int)threadIdx.x; i < P.cf_words; i += G * BLOCK) z[i] = 0u;
        }
        // own mode: this workgroup's winners of level k, in LDS (at most
        // OWN_CAP of them, with at most BLOCK edges); not when this
        // level's winners go to the queue lists, whose LDS staging would
        // overwrite them
        const bool own = sh.s_own && !to_queue;
        const int own_cnt = (int)min(sh.rpack[k & 1] >> 40, (unsigned long long)OWN_CAP);
        const int own_edges = (int)min(sh.rpack[k & 1] & RP_EDGES, (unsigned long long)STEP_CLAIMS);
        prev_wcf = wcf;
        wcf = wcf1;
        wbits = wbits1;
        fsize = F1;
        fdeg = E1;
        reached_before0 = reached_before;
        edges_before0 = edges_before;
        // (the staging count, spill flag and hub list stay 0 in region mode:
        // only a level that writes the queue lists stages into them, and the
        // launch ends after it)
        c.level = k;
        c.nslot = (k + 1) % NSLOTS;
        c.wbits = wbits1;
        c.wcf = wcf1;
        c.nbm = nc ? P.fbm0 : P.fbm1;
        c.ncf = P.cf + (size_t)((k + 1) % 3) * CF_WORDS;
        c.nq = nc ? P.q0 : P.q1; c.nt = nc ? P.t0 : P.t1; c.nts = nc ? P.ts0 : P.ts1;
        c.region = to_queue ? nullptr : P.sreg + ((size_t)((k + 1) & 1) * SMALL_G + wg) * SREG_CAP;
        c.converting = 0;
        // STEP_CLAIMS claims per step over the edges [0, Ew) of entries
        // [0, nloc) (vertex ev[j], adjacency start eb[j], edge offset eo[j],
        // ascending), each step followed by a flush check: the staging buffer
        // of a level into the queue lists never overfills
        // (NQ claims per thread per step: own mode has at most BLOCK edges and
        // takes one, whose claims also read the winners' inline adjacency)
        auto claim_steps = [&](auto nq, const int32_t *eo, const int32_t *ev, const int32_t *eb, int nloc, int Ew) {
            constexpr int NQ = decltype(nq)::value;
            const int t = (int)threadIdx.x;
            for (int e0 = 0; e0 < Ew; e0 += NQ * BLOCK) {
                int tv[NQ], ow[NQ];
                bool ok[NQ];
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const int e = e0 + q * BLOCK + t;
                    ok[q] = e < Ew;
                    int lo2 = 0, hi2 = nloc;   // last j with eo[j] <= e (skips degree-0 entries)
                    while (hi2 - lo2 > 1) {
                        const int mid = (lo2 + hi2) >> 1;
                        if (eo[mid] <= e) lo2 = mid; else hi2 = mid;
                    }
                    ow[q] = ev[lo2];
                    tv[q] = ok[q] ? P.col_idx[eb[lo2] + (e - eo[lo2])] : 0;
                }
                claim_batch(c, tv, ok, ow);
                if (!c.region) {   // uniform; region staging never fills the staging buffer
                    __syncthreads();
                    maybe_flush(c);
                }
            }
        };
        if (own) {
            // own mode: this workgroup's winners of level k, as staged in LDS
            // with their edge offsets (one step: at most BLOCK edges);
            // level k+1's winners go to the other half
            const int h = (k & 1) * OWN_CAP;
            if (clear_bm)
                for (int i = threadIdx.x; i < own_cnt; i += BLOCK) cbm[sh.buf[h + i] >> 5] = 0u;
            if (sh.inl[k & 1]) {
                // every target is in LDS: edge t of thread t, no adjacency read
                const int e = (int)threadIdx.x;
                const bool ok[1] = {e < own_edges};   // own_edges <= BLOCK
                const int tv[1] = {ok[0] ? sh.itgt[k & 1][e] : 0};
                const int ow[1] = {ok[0] ? sh.iown[k & 1][e] : 0};
                claim_batch(c, tv, ok, ow);
            } else {
                claim_steps(std::integral_constant<int, 1>{}, sh.toff + h, sh.buf + h, sh.sbeg + h, own_cnt, own_edges);
            }
        } else {
            // an equal share of all workgroups' entries of level k, from the
            // regions; the share's edges are dealt out over the whole
            // workgroup (an exclusive scan of the entries' degrees in LDS,
            // the owner of each edge by binary search), as in the
            // edge-balanced advance
            const int4 *rin = P.sreg + (size_t)nc * SMALL_G * SREG_CAP;
            int32_t *s_off = sh.work;
            int32_t *s_v = sh.work + (EB_TE + 1);
            int32_t *s_beg = sh.work + 2 * (EB_TE + 1);
            const int per = (F1 + G - 1) / G;
            const int lo = min(F1, wg * per), hi = min(F1, lo + per);
            for (int i0 = lo; i0 < hi; i0 += BLOCK) {
                const int nloc = min(BLOCK, hi - i0);
                const int t = (int)threadIdx.x;
                int v = 0, beg = 0, len = 0;
                if (t < nloc) {
                    const int i = i0 + t;
                    int a = 0, b = G;   // the region holding entry i: last a with spre[a] <= i
                    while (b - a > 1) {
                        const int mid = (a + b) >> 1;
                        if (sh.spre[mid] <= i) a = mid; else b = mid;
                    }
                    const int4 e = rin[(size_t)a * SREG_CAP + (i - sh.spre[a])];
                    v = e.x; beg = e.y; len = e.z;
                    if (clear_bm) cbm[v >> 5] = 0u;
                }
                const int incl = wave_incl_scan_i32(len);
                const int wsum = readlane_i(incl, WAVE - 1);
                if (lane == 0) sh.scan_tmp[0][wave_id()] = (uint64_t)(uint32_t)wsum;
                __syncthreads();
                int base = 0, Ew = 0;
                for (int w = 0; w < WAVES; ++w) {
                    const int x = (int)sh.scan_tmp[0][w];
                    if (w < wave_id()) base += x;
                    Ew += x;
                }
                if (t < nloc) { s_off[t] = base + incl - len; s_v[t] = v; s_beg[t] = beg; }
                __syncthreads();
                claim_steps(std::integral_constant<int, STEP_CLAIMS / BLOCK>{}, s_off, s_v, s_beg, nloc, Ew);
                __syncthreads();   // s_off and scan_tmp are reused
            }
        }
        if (wg == 0 && threadIdx.x == 0 && launch < RAN_CAP) P.ctl->ran[launch] = 1;
        if (to_queue) {
            if (sh.cnt > 0) flush(c);
            if (sh.spilled) add_tallies(c);
            return k + 1;
        }
    }
}

// Common start of a level launch: the level it stands at and the decision
// for it.  Returns that level, or -1 when the launch has nothing to do (the
// search is over, an error was recorded, or it has just found the empty
// frontier and recorded the end).
__device__ __forceinline__ int level_launch_start(const Params &P, LevelCommon &sh, int launch) {
    const int k = P.ctl->lvl[launch & 1];
    if (threadIdx.x < WAVE) decide(P, sh, k);
    __syncthreads();
    if (sh.mode == 0) return -1;
    if (sh.mode == 1) {
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            P.ctl->L = k;
            P.ctl->done = 1;
            if (launch < RAN_CAP) P.ctl->ran[launch] = 2;
        }
        return -1;
    }
    return k;
}

__device__ __forceinline__ void set_next_level(const Params &P, int launch, int k) {
    if (blockIdx.x == 0 && threadIdx.x == 0) P.ctl->lvl[(launch + 1) & 1] = k;
}

// Top-down launch: runs the level it stands at on the whole grid when that
// level is top-down, or, when the level is small, runs levels on the first
// SMALL_G workgroups until one is not small (or is bottom-up); a bottom-up
// level is passed on to the next launch.
__global__ __launch_bounds__(BLOCK, 4) void bfs_td_kernel(Params P, int32_t launch) {
    __shared__ TdLds sh;
    const int k = P.ctl->lvl[launch & 1];
    if (threadIdx.x < WAVE) decide(P, sh, k);
    __syncthreads();
    if (sh.mode == 0) return;    // over, or an error was recorded
    if (sh.mode == 1) {
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            P.ctl->L = k;
            P.ctl->done = 1;
            if (launch < RAN_CAP) P.ctl->ran[launch] = 1;
        }
        return;
    }
    if (sh.dir == DIR_BU) {      // for the bottom-up launch
        set_next_level(P, launch, k);
        return;
    }
    if (sh.small) {
        // the first SMALL_G workgroups; the first level writes the regions
        // unless its winners are predicted not to be small (no growth is
        // seen at the source level, which always writes the queue lists)
        if (blockIdx.x >= SMALL_G) return;
        const int G = min((int)gridDim.x, SMALL_G);
        const bool to_queue = k == 0 || grows_out(sh.fdeg, sh.prev_fdeg);
        run_level<false>(P, sh, k, blockIdx.x, G, !to_queue);
        if (blockIdx.x == 0 && threadIdx.x == 0 && launch < RAN_CAP) P.ctl->ran[launch] = 1;
        if (to_queue) {
            set_next_level(P, launch, k + 1);
            return;
        }
        const int kn = run_small(P, sh, k, launch, G);
        if (kn >= 0) set_next_level(P, launch, kn);
        return;
    }
    run_level<false>(P, sh, k, blockIdx.x, (int)gridDim.x);
    if (blockIdx.x == 0 && threadIdx.x == 0 && launch < RAN_CAP) P.ctl->ran[launch] = 1;
    set_next_level(P, launch, k + 1);
}

// Bottom-up launch: runs the level it stands at when that level is
// bottom-up, else passes it on.  The launch bounds hold it to 64 VGPRs, so
// that with its 35 KB of LDS four workgroups share a compute unit (the pass
// waits on scattered reads; a fourth workgroup hides more of that latency).
__global__ __launch_bounds__(BLOCK, 8) void bfs_bu_kernel(Params P, int32_t launch) {
    __shared__ BuLds sh;
    const int k = level_launch_start(P, sh, launch);
    if (k < 0) return;
    if (sh.dir != DIR_BU) {
        set_next_level(P, launch, k);
        return;
    }
    run_level<true>(P, sh, k, blockIdx.x, (int)gridDim.x);
    if (blockIdx.x == 0 && threadIdx.x == 0 && launch < RAN_CAP) P.ctl->ran[launch] = 2;
    set_next_level(P, launch, k + 1);
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

__global__ void facts_reset_kernel(GraphFacts *f) {
    if (threadIdx.x == 0) {
        f->bad_row = ~0ull;
        f->bad_col = ~0ull;
        f->unsorted = 0u;
        f->asymmetric = 0u;
        f->max_degree = 0;
        f->pad = 0;
    }
}

// ------------------------------------------------------ host helpers -------

hipError_t launch_facts_reset(GraphFacts *f, hipStream_t s) {
    hipLaunchKernelGGL(facts_reset_kernel, dim3(1), dim3(64), 0, s, f);
    return hipGetLastError();
}

hipError_t launch_init(const Params &P, int grid, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    // grid fill workgroups and the control one
    hipExtLaunchKernelGGL(bfs_init_kernel, dim3(grid + 1), dim3(BLOCK), 0, s, start, stop, 0, P);
    return hipGetLastError();
}

// The finishing pass, after the level launches: nothing unless the search is
// done (a search that needs another batch of launches finishes after it).  A
// lane takes four consecutive vertices (a wavefront, four 64-vertex words),
// and a wavefront FIN_U such groups at once with all their loads in flight:
// the distance of the kept bitmap holding a vertex, else -1 for a vertex
// never reached (not visited, or marked visited from the start for lack of
// in-edges), else nothing (a level stored it, as the init kernel stored the
// source's).  A lane whose four vertices all take a value writes them with
// one 16-byte streaming store (a wavefront, sixteen whole 64-byte lines):
// 4-byte stores issue four times the lane stores for the same bytes.  Each
// bitmap is read as the 32-bit half holding the lane's four bits.
constexpr int FIN_BLOCK = 256;
constexpr int FIN_U = 4;
__global__ __launch_bounds__(FIN_BLOCK) void bfs_finish_kernel(Params P) {
    const Ctl *ctl = P.ctl;
    if (!ctl->done || ctl->err) return;
    // the per-level record says the search ended here (level 0, bit 5:
    // above the direction bit and the level's own flags)
    if (blockIdx.x == 0 && threadIdx.x == 0 && P.st_cap > 0) P.st_dir[0] = (int8_t)(P.st_dir[0] | 32);
    const uint32_t km = ctl->kmask & ((1u << KCAP) - 1u);
    const uint32_t *lv32 = reinterpret_cast<const uint32_t *>(P.lvbm);
    typedef int v4i __attribute__((ext_vector_type(4)));
    v4i *d4 = reinterpret_cast<v4i *>(P.dist);
    const bool al = (reinterpret_cast<uintptr_t>(P.dist) & 15) == 0;
    const int lane = lane_id();
    const int sh = (lane & 15) * 4;   // this lane's first vertex within its word
    const int half = sh >> 5;         // the 32-bit half of the word holding it
    const int bit = sh & 31;
    const int64_t nquads = ((int64_t)P.nwp + 3) / 4;
    const int64_t nwaves = (int64_t)gridDim.x * (FIN_BLOCK / WAVE);
    for (int64_t q0 = ((int64_t)blockIdx.x * (FIN_BLOCK / WAVE) + threadIdx.x / WAVE) * FIN_U; q0 < nquads;
         q0 += nwaves * FIN_U) {
        int64_t w[FIN_U];
        bool ok[FIN_U];
        uint32_t rn[FIN_U];
        int d[FIN_U][4];
#pragma unroll
        for (int u = 0; u < FIN_U; ++u) {
            w[u] = (q0 + u) * 4 + (lane >> 4);
            ok[u] = q0 + u < nquads && w[u] < P.nwp;
            const size_t x = (size_t)w[u] * 2 + half;
            rn[u] = ok[u] ? ((P.visited[x] & ~P.vis_init[x]) >> bit) & 15u : 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) d[u][e] = -1;
        }
        // the kept bitmaps, four levels at a time (every load of a round in
        // flight before any is used)
        for (uint32_t t = km; t;) {
            int j[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                j[q] = t ? __ffs((int)t) - 1 : -1;
                if (t) t &= t - 1;
            }
            uint32_t kn[FIN_U][4];
#pragma unroll
            for (int u = 0; u < FIN_U; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    kn[u][q] = (ok[u] && j[q] >= 0)
                                   ? (lv32[((size_t)j[q] * P.nwp + w[u]) * 2 + half] >> bit) & 15u : 0u;
#pragma unroll
            for (int u = 0; u < FIN_U; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if ((kn[u][q] >> e) & 1u) d[u][e] = j[q];
        }
#pragma unroll
        for (int u = 0; u < FIN_U; ++u) {
            if (!ok[u]) continue;
            const int64_t v0 = w[u] * 64 + sh;
            bool wr[4];
            bool all = al;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t v = v0 + e;
                wr[e] = v < P.n && v != P.source && (d[u][e] >= 0 || !((rn[u] >> e) & 1u));
                all = all && wr[e];
            }
            if (all) {
                v4i xv = {d[u][0], d[u][1], d[u][2], d[u][3]};
                __builtin_nontemporal_store(xv, d4 + (v0 >> 2));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (wr[e]) __builtin_nontemporal_store(d[u][e], P.dist + v0 + e);
            }
        }
    }
}

hipError_t launch_finish(const Params &P, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
    const int64_t quads = ((int64_t)P.nwp + 3) / 4;
    const int64_t waves = (quads + FIN_U - 1) / FIN_U;
    const int64_t blocks = (waves + FIN_BLOCK / WAVE - 1) / (FIN_BLOCK / WAVE);
    hipExtLaunchKernelGGL(bfs_finish_kernel, dim3((unsigned)(blocks < 16384 ? blocks : 16384)), dim3(FIN_BLOCK), 0, s,
                          start, stop, 0, P);
    return hipGetLastError();
}

hipError_t launch_level(const Params &P, int32_t launch_index, bool bottom_up, int grid, hipStream_t s,
                        hipEvent_t start, hipEvent_t stop) {
    if (bottom_up)
        hipExtLaunchKernelGGL(bfs_bu_kernel, dim3(grid), dim3(BLOCK), 0, s, start, stop, 0, P, launch_index);
    else
        hipExtLaunchKernelGGL(bfs_td_kernel, dim3(grid), dim3(BLOCK), 0, s, start, stop, 0, P, launch_index);
    return hipGetLastError();
}

int level_kernel_blocks_per_cu(bool bottom_up) {
    int nb = 0;
    const void *fn = bottom_up ? (const void *)bfs_bu_kernel : (const void *)bfs_td_kernel;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, BLOCK, 0) != hipSuccess) return 1;
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

// ---------------------------------------------------- in-edge transpose -----
// A counting sort of the CSR entries by target: in-degree counts, an
// exclusive scan into in_row_ptr, then every entry u -> v is appended to v's
// in-list at a cursor taken with an atomic.  In-lists come out in no fixed
// order (any in-neighbour in the frontier is a valid parent).

__global__ __launch_bounds__(256) void in_degree_kernel(const int32_t *col_idx, int32_t m,
                                                        int32_t *cnt) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < m; e += nth)
        atomicAdd(&cnt[col_idx[e]], 1);
}

constexpr int SCAN_BLOCK = 256;
constexpr int SCAN_ITEMS = 4;
constexpr int SCAN_TILE = SCAN_BLOCK * SCAN_ITEMS;

// Exclusive scan of one tile of cnt into out; the tile's total goes to sums.
__global__ __launch_bounds__(SCAN_BLOCK) void scan_tile_kernel(const int32_t *cnt, int32_t *out,
                                                              int64_t n, int32_t *sums) {
    __shared__ int32_t wsum[SCAN_BLOCK / WAVE];
    const int64_t base = (int64_t)blockIdx.x * SCAN_TILE + (int64_t)threadIdx.x * SCAN_ITEMS;
    int32_t x[SCAN_ITEMS], t = 0;
#pragma unroll
    for (int i = 0; i < SCAN_ITEMS; ++i) {
        x[i] = (base + i < n) ? cnt[base + i] : 0;
        t += x[i];
    }
    // exclusive prefix of the per-thread totals over the block
    int32_t incl = t;
    for (int d = 1; d < WAVE; d <<= 1) {
        const int32_t y = __shfl_up(incl, (unsigned)d, WAVE);
        if (lane_id() >= d) incl += y;
    }
    if (lane_id() == WAVE - 1) wsum[threadIdx.x / WAVE] = incl;
    __syncthreads();
    int32_t before = 0;
    for (int w = 0; w < (int)(threadIdx.x / WAVE); ++w) before += wsum[w];
    int32_t run = before + incl - t;
#pragma unroll
    for (int i = 0; i < SCAN_ITEMS; ++i) {
        if (base + i < n) out[base + i] = run;
        run += x[i];
    }
    if (threadIdx.x == SCAN_BLOCK - 1) sums[blockIdx.x] = run;
}

__global__ __launch_bounds__(SCAN_BLOCK) void scan_add_kernel(int32_t *out, int64_t n,
                                                             const int32_t *offs) {
    const int64_t base = (int64_t)blockIdx.x * SCAN_TILE;
    for (int i = threadIdx.x; i < SCAN_TILE; i += SCAN_BLOCK)
        if (base + i < n) out[base + i] += offs[blockIdx.x];
}

// Every entry u -> v appended to v's in-list.
__global__ __launch_bounds__(256) void transpose_fill_kernel(const int32_t *row_ptr,
                                                             const int32_t *col_idx, int32_t n,
                                                             int32_t *cursor, int32_t *in_col) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < n; u += nth) {
        const int32_t b = row_ptr[u], e = row_ptr[u + 1];
        for (int32_t j = b; j < e; ++j) in_col[atomicAdd(&cursor[col_idx[j]], 1)] = (int32_t)u;
    }
}

// Probe-neighbour index: for every vertex v the in-neighbour of highest
// out-degree (the first in CSR order among equals), and the one after it
// (second highest), -1 where there is none.  Hubs are reached in the first
// levels, so these are the in-neighbours most likely to be in a bottom-up
// level's frontier.  One wavefront per vertex; each lane keeps its best two
// entries as keys (out-degree << 32 | ~entry), merged across the wavefront.
__device__ __forceinline__ void top2_insert(unsigned long long &k1, unsigned long long &k2, unsigned long long x) {
    if (x > k1) {
        k2 = k1;
        k1 = x;
    } else if (x > k2) {
        k2 = x;
    }
}

__global__ __launch_bounds__(256) void probe_nb_kernel(const int32_t *row_ptr, const int32_t *in_row_ptr,
                                                       const int32_t *in_col, int32_t n, int32_t *pnb,
                                                       int32_t *snb) {
    const int lane = lane_id();
    const int64_t nw = (int64_t)gridDim.x * (blockDim.x / WAVE);
    for (int64_t v = (int64_t)blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE; v < n; v += nw) {
        const int b = in_row_ptr[v], e = in_row_ptr[v + 1];
        unsigned long long k1 = 0ull, k2 = 0ull;   // 0: none (a real key has ~entry > 0)
        for (int j = b + lane; j < e; j += WAVE) {
            const int u = in_col[j];
            const uint32_t d = (uint32_t)(row_ptr[u + 1] - row_ptr[u]);
            top2_insert(k1, k2, ((unsigned long long)d << 32) | (uint32_t)(0x7fffffff - j));
        }
#pragma unroll
        for (int off = WAVE / 2; off > 0; off >>= 1) {
            const unsigned long long o1 = __shfl_xor(k1, off, WAVE);
            const unsigned long long o2 = __shfl_xor(k2, off, WAVE);
            top2_insert(k1, k2, o1);
            top2_insert(k1, k2, o2);
        }
        if (lane == 0) {
            pnb[v] = k1 ? in_col[0x7fffffff - (int)(uint32_t)(k1 & 0xffffffffull)] : -1;
            snb[v] = k2 ? in_col[0x7fffffff - (int)(uint32_t)(k2 & 0xffffffffull)] : -1;
        }
    }
}

__global__ __launch_bounds__(256) void deg8_kernel(const int32_t *in_row_ptr, int32_t n, uint8_t *deg8) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n; v += nth) {
        const int d = in_row_ptr[v + 1] - in_row_ptr[v];
        deg8[v] = (uint8_t)(d < 255 ? d : 255);
    }
}

__global__ __launch_bounds__(256) void adj4_kernel(const int32_t *row_ptr, const int32_t *col_idx, int32_t n,
                                                   int4 *adj4) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n; v += nth) {
        const int b = row_ptr[v], d = row_ptr[v + 1] - b;
        int4 a = make_int4(-1, -1, -1, -1);
        if (d <= ADJ_INLINE) {
            if (d > 0) a.x = col_idx[b];
            if (d > 1) a.y = col_idx[b + 1];
            if (d > 2) a.z = col_idx[b + 2];
            if (d > 3) a.w = col_idx[b + 3];
        }
        adj4[v] = a;
    }
}

hipError_t launch_build_adj4(const int32_t *row_ptr, const int32_t *col_idx, int32_t n, int4 *adj4, hipStream_t s) {
    hipLaunchKernelGGL(adj4_kernel, dim3(grid_for(n, 256 * 4)), dim3(256), 0, s, row_ptr, col_idx, n, adj4);
    return hipGetLastError();
}

hipError_t launch_build_deg8(const int32_t *in_row_ptr, int32_t n, uint8_t *deg8, hipStream_t s) {
    hipLaunchKernelGGL(deg8_kernel, dim3(grid_for(n, 256 * 4)), dim3(256), 0, s, in_row_ptr, n, deg8);
    return hipGetLastError();
}

hipError_t launch_build_probe_nb(const int32_t *row_ptr, const int32_t *in_row_ptr, const int32_t *in_col,
                                 int32_t n, int32_t *pnb, int32_t *snb, hipStream_t s) {
    hipLaunchKernelGGL(probe_nb_kernel, dim3(grid_for(n, 4 * 16)), dim3(256), 0, s, row_ptr, in_row_ptr,
                       in_col, n, pnb, snb);
    return hipGetLastError();
}

hipError_t launch_in_degree(const int32_t *col_idx, int32_t m, int32_t *cnt, hipStream_t s) {
    hipLaunchKernelGGL(in_degree_kernel, dim3(grid_for(m, 256 * 4)), dim3(256), 0, s, col_idx, m, cnt);
    return hipGetLastError();
}

int64_t scan_tmp_ints(int64_t n) {
    int64_t total = 0;
    for (int64_t len = n; len > 1;) {
        const int64_t tiles = (len + SCAN_TILE - 1) / SCAN_TILE;
        total += 2 * tiles + 1;   // tile sums and their scan (plus the grand total)
        len = tiles;
    }
    return total + 1;
}

hipError_t exclusive_scan(const int32_t *cnt, int32_t *out, int64_t n, int32_t *tmp, hipStream_t s) {
    // out[0, n) = exclusive prefix; out[n] = total.  Tiles of SCAN_TILE are
    // scanned alone, their totals are scanned the same way (recursively), and
    // the scanned totals are added back.
    if (n <= 0) {
        return hipMemsetAsync(out, 0, sizeof(int32_t), s);
    }
    const int64_t tiles = (n + SCAN_TILE - 1) / SCAN_TILE;
    if (tiles > 0x7fffffff) return hipErrorInvalidValue;
    int32_t *sums = tmp, *offs = tmp + tiles;
    hipLaunchKernelGGL(scan_tile_kernel, dim3((unsigned)tiles), dim3(SCAN_BLOCK), 0, s, cnt, out, n, sums);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (tiles == 1) return hipMemcpyAsync(out + n, sums, sizeof(int32_t), hipMemcpyDeviceToDevice, s);
    e = exclusive_scan(sums, offs, tiles, tmp + 2 * tiles + 1, s);   // offs[tiles] = total
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scan_add_kernel, dim3((unsigned)tiles), dim3(SCAN_BLOCK), 0, s, out, n, offs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return hipMemcpyAsync(out + n, offs + tiles, sizeof(int32_t), hipMemcpyDeviceToDevice, s);
}

hipError_t launch_transpose_fill(const int32_t *row_ptr, const int32_t *col_idx, int32_t n,
                                 int32_t *cursor, int32_t *in_col, hipStream_t s) {
    hipLaunchKernelGGL(transpose_fill_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, row_ptr,
                       col_idx, n, cursor, in_col);
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
