// Internal layout shared by the gfx950 kernels (bfs_device.hip) and the C ABI
// layer (bfs_api.hip).  Not installed; the public interface is
// include/frontier_bfs.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fbfs {

// ---- launch geometry and bin thresholds (gfx950: 64-lane wavefronts) -------
constexpr int WAVE = 64;
constexpr int BLOCK = 512;               // threads per workgroup
constexpr int WAVES = BLOCK / WAVE;      // wavefronts per workgroup
constexpr int STRIPES = 8;               // counter / queue stripes (spread atomics)
constexpr int T_LANE = 32;               // degree < T_LANE: one lane walks the list
constexpr int T_WG = BLOCK;              // T_LANE <= degree < T_WG: one wavefront
constexpr int TILE = 4 * BLOCK;          // degree >= T_WG: split into tiles of TILE edges,
                                         // one workgroup per tile
constexpr int CAP = 2048;                // LDS staging capacity for new frontier vertices
constexpr int STEP_CLAIMS = CAP / 2;     // claims between flush checks: a flush starts at
                                         // CAP / 2 staged, so a step never overfills
constexpr int EB_TE = 1024;              // edges per tile of the edge-balanced advance
constexpr int64_t NOQ_EDGES = 1 << 17;       // top-down levels with at least this many frontier
                                              // edges whose next level may pull skip the queue
constexpr int64_t VFILTER_EDGES = 1 << 20;  // top-down levels with at least this many
                                         // edges load the visited word before a claim
constexpr int BU_GSZ = 64;                // bottom-up: vertices a wavefront lists at a time
#ifndef BU_DENSE
#define BU_DENSE 16                      // bottom-up: a word with this many unvisited vertices
#endif                                   //   is probed lane per vertex before listing
constexpr int BU_W1 = 8;                 // bottom-up: entries per vertex in the round after
                                         // the first (x4 per round after that)
constexpr int BU_WMAX = 8192;            // bottom-up: cap of the per-round entries per vertex
constexpr int BU_U = 4;                  // bottom-up: probes a lane keeps in flight per step
constexpr int CF_WORDS = 4096;           // coarse frontier map: at most 4096 words (16 KB)
// direction switching (edge-based, as in Beamer et al. SC'12): go bottom-up
// when the frontier's edges exceed 1/alpha of the unexplored vertices' edges;
// come back top-down when the frontier is under n/beta and shrinking.  These
// are the defaults; bfs_set_switch changes them per handle.
constexpr int ALPHA = 40;
constexpr int BETA = 96;

// lists of a frontier queue
constexpr int L_SMALL = 0;               // degree in [1, T_LANE)
constexpr int L_MID = 1;                 // degree in [T_LANE, T_WG)
constexpr int L_TILE = 2;                // pieces of vertices with degree >= T_WG
constexpr int NLISTS = 3;

// counters of one level slot: NLISTS*STRIPES list counters, then STRIPES
// vertex counters; each 64-bit counter sits alone in 256 bytes.
constexpr int NCTR = 33;
constexpr int CTR_STRIDE = 32;           // in uint64 units
constexpr int VC_BASE = NLISTS * STRIPES;
constexpr int QPOOL_CTR = VC_BASE + STRIPES;   // pool chunks handed out for the level's queue
constexpr int NSLOTS = 4;                // ring of level slots

// direction codes stored per level
constexpr int DIR_TD = 0;
constexpr int DIR_BU = 1;

// One frontier segment: vertex v's adjacency piece col_idx[beg, beg+len), and
// off = the exclusive prefix of len over its list stripe (the frontier-degree
// scan used by the edge-balanced advance).
struct __align__(16) Seg {
    int32_t v, beg, len, off;
};

// Per-level scalars, written once per level by workgroup 0.
struct SlotInfo {
    int32_t dir;          // direction this level ran in
    int32_t wbits;        // this level's new vertices were also set in the next bitmap
    int32_t input_bm;     // this level's frontier came as a bitmap only
    int32_t fsize;        // this level's frontier size
    int32_t wcf;          // this level's new vertices were also set in the next coarse map
    int32_t noq;          // this level wrote its new vertices to the next bitmap only (no queue)
    int64_t reached_before;  // vertices in levels < this one
    int64_t edges_before;    // sum of degrees of the vertices in levels < this one
};

constexpr int RAN_CAP = 64;               // launches whose kind of work is recorded

struct Ctl {
    int32_t done;         // set by the kernel that finds an empty frontier
    int32_t L;            // number of non-empty levels
    int32_t err;          // nonzero: internal limit exceeded (see ERR_*)
    int32_t err_info;
    // ran[i]: launch i ran a level, or found the empty frontier, in the
    // top-down (1) or bottom-up (2) kernel, else 0; read by the host with the
    // status words, to order the next search's launches
    uint8_t ran[RAN_CAP];
    int32_t lvl[2];       // level the launch with index i starts at: lvl[i & 1]
    uint32_t kmask;       // bit j: level j's found set is in the kept bitmap lvbm[j]
    int32_t pad0;
    SlotInfo slot[NSLOTS];
    alignas(128) uint32_t pad1;
};

// Levels below KCAP found from or into a bitmap (bottom-up levels, and the
// frontier a queue-free top-down level leaves) keep their found set as a
// bitmap instead of storing dist vertex by vertex; dist is written at the end.
constexpr int KCAP = 16;
// ... on graphs of at least FINISH_MIN_N vertices: on smaller ones dist stays
// in the caches, its scattered stores cost little, and the finishing pass
// would only add its launch (C2, 2^20 vertices: +10 %; C3, 2^22: +1.5 %;
// C5, 2^24: -6.5 % per search)
constexpr int64_t FINISH_MIN_N = 1LL << 23;

constexpr int ERR_QUEUE_OVERFLOW = 1;
constexpr int ERR_TILE_OVERFLOW = 2;
constexpr int ERR_TSTART_OVERFLOW = 3;
constexpr int ERR_BARRIER_TIMEOUT = 4;
constexpr int ERR_BAD_VERTEX = 5;        // a vertex id outside [0, n) met before a store (info: the id)

// small-frontier mode: a top-down level whose frontier has at most SMALL_F
// vertices and SMALL_E edges runs on the first SMALL_G workgroups only, and
// those keep going level after level with a barrier among themselves.  One
// edge per thread of those workgroups: a level of 53K edges (an Erdos-Renyi
// search's fifth level) took 29 us there against 10 us on the whole grid
constexpr int SMALL_G = 32;
constexpr int SMALL_F = SMALL_G * BLOCK;
constexpr int SMALL_E = SMALL_F;
// In that mode each workgroup appends the vertices it wins to a region of
// its own (entries {v, beg, len}: a workgroup's winners are at most the
// level's edges, so SMALL_E entries always fit), one set of regions per level
// parity, and publishes {level, count, edges} in one 64-bit word; the words
// of all workgroups are the barrier and the next level's work split at once.
constexpr int SREG_CAP = SMALL_E;

// Inclusive prefix sum over the 64 lanes of a wavefront (all lanes active)
// with DPP moves, register to register: shifts right by 1, 2, 4 and 8 lanes
// within each row of 16 (a lane shifted in from outside its row reads 0),
// then lane 15 of each row added into the next row and lane 31 into the two
// upper rows.  A shuffle would take a round trip through the LDS crossbar
// per step.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1, 3
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2, 3
    return x;
}

struct Params {
    const int32_t *row_ptr;
    const int32_t *col_idx;
    int32_t n;
    int32_t m;
    int32_t nwp;              // 64-vertex word pairs: ceil(n / 64)
    int32_t source;
    int32_t *dist;
    int32_t *parent;          // may be null
    int32_t *level_sizes;     // may be null
    uint32_t *visited;        // 2*nwp words
    const uint32_t *vis_init; // 2*nwp words: isolated vertices (symmetric graphs) + padding
    // in-edges, read by the bottom-up pass: the CSR itself when it is
    // symmetric, else its transpose built at graph creation
    const int32_t *in_row_ptr;
    const int32_t *in_col_idx;
    const int32_t *pnb;       // n entries: in-neighbour of highest out-degree, -1 if none
    const int32_t *snb;       // n entries: in-neighbour of second highest out-degree, -1 if none
    const uint8_t *deg8;      // n entries: in-degree, 255 standing for 255 or more
    const int4 *adj4;         // n entries: the out-neighbours of a vertex of out-degree at most
                              // ADJ_INLINE (-1 padded), so a small level reads them beside the
                              // claim instead of after it; unused for larger degrees
    uint64_t *lvbm;           // KCAP bitmaps of nwp words: bitmap j holds the vertices at
                              // distance j when a level recorded them there (bit j of the
                              // control block's kmask) instead of storing their dist; the
                              // finishing pass then writes dist once, in vertex order
    int32_t fill_dist;        // the init kernel fills dist with -1 (paths without the finishing pass)
    int32_t l0_init;          // rows are sorted: the init kernel may run level 0 itself
    uint32_t *fbm0, *fbm1;    // frontier bitmaps, 2*nwp words each
    Seg *q0, *q1;             // queue storage, queue_segs(n) segments each (chunks of 2^qk_sh)
    Seg *t0, *t1;             // STRIPES regions of tcap tiles
    int32_t *ts0, *ts1;       // edge-balanced tile starts: NLISTS*STRIPES regions of tscap
    int64_t tcap, tscap;
    int32_t qk_sh;            // log2 of the segments per queue chunk
    int32_t qpool;            // pool chunks per queue
    unsigned long long *qtab; // chunk tables: NSLOTS x 2 lists x STRIPES x qpool entries,
                              // entry j-1 = (tag << 32) | pool chunk of chunk j >= 1
    unsigned long long *ctr;  // NSLOTS * NCTR counters, CTR_STRIDE apart
    Ctl *ctl;
    int8_t *st_dir;           // per-level stats, st_cap entries
    int64_t *st_fdeg;
    int32_t st_cap;
    int32_t symmetric;
    int32_t col_vec;          // col_idx is 16-byte aligned: 16-byte loads allowed
    int32_t in_col_vec;       // the same for in_col_idx
    int32_t can_pull;         // in-edges are available (symmetric, or transpose built)
    int32_t pol_dir;          // BFS_DIR_*
    int32_t pol_adv;          // BFS_ADV_*
    int32_t small_mode;       // allow the small-frontier mode
    int32_t alpha, beta;      // direction-switch parameters
    int32_t max_deg;          // largest degree of the graph
    uint32_t *cf;             // 3 coarse frontier maps of CF_WORDS words: bit b of map j
                              // says some vertex in [b << cf_sh, (b+1) << cf_sh) joined the
                              // frontier of a level l with l % 3 == j
    int32_t cf_sh, cf_words;  // vertices per coarse bit (log2); words in use per map
    uint32_t barrier_ticks;   // small-mode barrier wait limit (100 MHz ticks)
    int4 *sreg;               // small-frontier regions: 2 parities x SMALL_G x SREG_CAP entries
    unsigned long long *sslot;   // small-frontier words: 2 parities x SMALL_G
    int32_t *enq;             // debug builds (FBFS_COUNT_ENQUEUES): n per-vertex counts of
                              // writes into a next frontier, else null
};

// Debug builds count, per vertex, every write of it into a next frontier (a
// queue segment, a bitmap-only winner, a bottom-up find), so that a test can
// check each reached vertex joins exactly one frontier once: duplicates in
// the frontier leave dist right and are invisible to a dist check.
#ifdef FBFS_COUNT_ENQUEUES
#define FBFS_ENQ(P, v)                                  \
    do {                                                \
        if ((P).enq) atomicAdd((P).enq + (v), 1);       \
    } while (0)
#else
#define FBFS_ENQ(P, v) ((void)0)
#endif

// Workspace capacities (segments or entries per stripe region) for a graph of
// n vertices and m CSR entries; the handle's workspace and the fixed scratch
// of the allocation-free entry point both follow them.
//
// Queue storage.  A level puts at most n vertices into its queue, but how
// they split over the 2*STRIPES (small or mid list, stripe) regions is not
// known ahead, so a region's segments live in chunks of 2^qk_sh: chunk 0 of
// every region is fixed, and chunk j >= 1 comes from a pool on demand (the
// reservation holding the chunk's first segment takes it and records it in
// the level's table).  A region of c segments uses ceil(c / 2^qk_sh) - 1 pool
// chunks, so the level's regions together use at most n >> qk_sh of them.
constexpr int QK_MAX_SH = 14;             // chunks of at most 16384 segments
constexpr int qk_shift(int64_t n) {
    int s = 0;
    while ((1LL << s) < n && s < QK_MAX_SH) ++s;
    return s;
}
constexpr int64_t queue_pool(int64_t n) { return (n + (1LL << qk_shift(n)) - 1) >> qk_shift(n); }
constexpr int64_t queue_segs(int64_t n) { return (2 * STRIPES + queue_pool(n)) << qk_shift(n); }
constexpr int64_t queue_tab(int64_t n) { return (int64_t)NSLOTS * 2 * STRIPES * queue_pool(n); }
constexpr int64_t tile_cap(int64_t m) { return m / TILE + m / T_WG + 1; }
constexpr int64_t tstart_cap(int64_t m) { return m / EB_TE + 2; }
constexpr int64_t stats_cap(int64_t n) { return (n + 1) < (1 << 22) ? (n + 1) : (1 << 22); }

// host-side launch helpers (bfs_device.hip)
// Launch helpers.  start/stop (may be null): HIP events that the launch
// itself records when the kernel begins and ends (the timing hook), so a
// timed interval holds the kernel alone, not the gaps around it.
hipError_t launch_init(const Params &P, int grid, hipStream_t s, hipEvent_t start = nullptr,
                       hipEvent_t stop = nullptr);
// the finishing pass: once the search is done, dist of every vertex that no
// level stored directly (kept bitmaps, unreached) in one vertex-order pass
hipError_t launch_finish(const Params &P, hipStream_t s, hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// Graphs of at most ONE_N vertices are searched by one workgroup with the
// visited bits and both frontiers in LDS (bfs_small.hip).
constexpr int ONE_N = 3584;
constexpr int ONE_M = 40960;           // ... and with the graph itself in LDS when m <= ONE_M
hipError_t launch_one(const Params &P, hipStream_t s);
// launch `launch_index` of the level chain: even indexes run the top-down
// kernel, odd ones the bottom-up kernel
hipError_t launch_level(const Params &P, int32_t launch_index, bool bottom_up, int grid, hipStream_t s,
                        hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
// resident workgroups per compute unit of the top-down or bottom-up kernel
int level_kernel_blocks_per_cu(bool bottom_up);

// graph validation / classification (bfs_device.hip)
struct GraphFacts {
    unsigned long long bad_row;   // first index i with row_ptr[i] > row_ptr[i+1], or ~0
    unsigned long long bad_col;   // first entry e with col_idx[e] outside [0,n), or ~0
    uint32_t unsorted;            // some row is not ascending
    uint32_t asymmetric;          // some entry u->v has no v->u (sorted rows only)
    int32_t max_degree;
    int32_t pad;
};
// sets f to "no bad row, no bad column, sorted, symmetric, degree 0" (a fill
// kernel, so that nothing here records a memset)
hipError_t launch_facts_reset(GraphFacts *f, hipStream_t s);
hipError_t launch_check_rows(const int32_t *row_ptr, int32_t n, GraphFacts *f, hipStream_t s);
hipError_t launch_check_cols(const int32_t *row_ptr, const int32_t *col_idx, int32_t n,
                             GraphFacts *f, hipStream_t s);
hipError_t launch_check_symmetry(const int32_t *row_ptr, const int32_t *col_idx, int32_t n,
                                 GraphFacts *f, hipStream_t s);
hipError_t launch_build_vis_init(const int32_t *row_ptr, int32_t n, int32_t mark_isolated,
                                 uint32_t *vis_init, hipStream_t s);
hipError_t launch_build_deg8(const int32_t *in_row_ptr, int32_t n, uint8_t *deg8, hipStream_t s);
constexpr int ADJ_INLINE = 4;
hipError_t launch_build_adj4(const int32_t *row_ptr, const int32_t *col_idx, int32_t n, int4 *adj4, hipStream_t s);
hipError_t launch_build_probe_nb(const int32_t *row_ptr, const int32_t *in_row_ptr, const int32_t *in_col,
                                 int32_t n, int32_t *pnb, int32_t *snb, hipStream_t s);
// transpose (in-edge CSR) of a CSR: in-degree counts, exclusive scan, scatter
hipError_t launch_in_degree(const int32_t *col_idx, int32_t m, int32_t *cnt, hipStream_t s);
// exclusive scan of cnt[0, n) into out[0, n]; tmp holds scan_tmp_ints(n) ints
int64_t scan_tmp_ints(int64_t n);
hipError_t exclusive_scan(const int32_t *cnt, int32_t *out, int64_t n, int32_t *tmp, hipStream_t s);
hipError_t launch_transpose_fill(const int32_t *row_ptr, const int32_t *col_idx, int32_t n,
                                 int32_t *cursor, int32_t *in_col, hipStream_t s);

// alternative claim / compaction primitives (bfs_variants.hip)
struct VarCtl {
    int64_t edges;                 // frontier edges of the level just advanced
    unsigned long long winners;    // its new vertices (the append cursor when compacting by atomics)
};
struct VarAdvance {
    const int32_t *row_ptr, *col_idx;
    const int32_t *F;              // frontier (may hold -1 sentinels)
    int32_t len;
    const int32_t *offs;           // exclusive scan of the frontier's degrees (len + 1)
    int32_t next_level;
    int32_t claim;                 // BFS_CLAIM_*
    int32_t *dist, *parent;
    uint32_t *visited;
    int32_t *padded;               // non-null: neighbour or -1 at every edge position
    int32_t *compact;              // non-null: winners appended (atomic cursor in vc)
    VarCtl *vc;
};
hipError_t launch_var_seed(int32_t *F, int32_t source, int32_t *level_sizes, VarCtl *vc, hipStream_t s);
hipError_t launch_var_degrees(const int32_t *row_ptr, const int32_t *F, int32_t len, int32_t *deg, hipStream_t s);
hipError_t launch_var_advance(const VarAdvance &A, int grid, hipStream_t s);
hipError_t launch_var_record(const int32_t *offs_end, int32_t k, int8_t *st_dir, int64_t *st_fdeg, int32_t st_cap,
                             int32_t *level_sizes, VarCtl *vc, VarCtl *out, hipStream_t s);
hipError_t launch_var_compact_padded(const int32_t *x, int64_t len, int32_t *flag, int32_t *offs, int32_t *tmp,
                                     int32_t *out, hipStream_t s);
hipError_t launch_var_compact_level(const int32_t *dist, int32_t n, int32_t level, int32_t *flag, int32_t *offs,
                                    int32_t *tmp, int32_t *out, hipStream_t s);

// single-source shortest paths (bfs_sssp.hip)
struct SsspCtl {
    int32_t err;                   // a weight above the declared maximum was seen
    int32_t len;                   // length of the frontier just built
};
struct SsspRelax {
    const int32_t *row_ptr, *col_idx;
    const uint32_t *weights;
    uint32_t max_weight;
    int32_t source;
    const int32_t *F;              // frontier, id order
    int32_t len;
    const int32_t *offs;           // exclusive scan of the frontier's degrees (len + 1)
    unsigned long long *key;       // (distance << 32) | predecessor, all ones = unreached
    uint32_t *nbm;                 // next-frontier bitmap
    SsspCtl *sc;
    int32_t round;                 // this round's number, for the per-round stats
    int8_t *st_dir;
    int64_t *st_fdeg;              // frontier edges of each round (the relaxations it tries)
    int32_t st_cap;
};
hipError_t launch_sssp_init(unsigned long long *key, uint32_t *nbm, int32_t n, int32_t nwords, int32_t source,
                            int32_t *F, SsspCtl *sc, hipStream_t s);
hipError_t launch_sssp_relax(const SsspRelax &R, int grid, hipStream_t s);
hipError_t launch_sssp_compact(uint32_t *nbm, int32_t nwords, int32_t *cnt, int32_t *offs, int32_t *tmp,
                               int32_t *F, SsspCtl *sc, hipStream_t s);
hipError_t launch_sssp_output(const unsigned long long *key, int32_t n, int64_t *dist, int32_t *pred,
                              hipStream_t s);

// isolated neighbour walk of listed vertices (bfs_walk.hip); scratch holds
// walk_scratch_ints(count) ints, bad is raised for ids outside [0, n)
int64_t walk_scratch_ints(int64_t count);
#ifndef WALK_MERGE_K
#define WALK_MERGE_K 4   // longest run of entries per lane in the merge walk
#endif
hipError_t launch_walk(const Params &P, const int32_t *vs, int32_t count, int32_t mapping,
                       int32_t repeats, uint32_t *out, int32_t *scratch, int32_t *bad,
                       int lanes_grid, hipStream_t s);

}  // namespace fbfs
