/*
 * frontier_bfs.h -- level-synchronous, frontier-based BFS over an int32 CSR
 * graph on one MI355X (gfx950), behind a plain C ABI.
 *
 * What is computed.  Level 0 is {source}; level k+1 holds the vertices not yet
 * reached that are out-neighbours of level k; the search stops at the first
 * empty level ("Day 38 - Graph traversal on a GPU", section "What a
 * level-synchronous search actually launches"; PMPP ch.15 notes, section 15.2).
 * The graph is CSR: the neighbours of u are col_idx[row_ptr[u] .. row_ptr[u+1])
 * (PMPP ch.15 notes, section 15.1).  Edges are followed in CSR direction, so a
 * directed graph is allowed; self-loops and duplicate entries are allowed and
 * change nothing.
 *
 * Memory.  Every array argument is DEVICE memory of the current HIP device
 * (for example a torch tensor's data_ptr()), int32, contiguous.  The graph
 * arrays are borrowed: they must stay alive and unmodified until
 * bfs_graph_destroy.  The library owns its workspace (queues, bitmaps,
 * counters), allocated at bfs_graph_create and freed at bfs_graph_destroy.
 *
 * Streams.  bfs_run enqueues all its work on `stream` (0 = the null stream)
 * and returns after that work has finished.  One handle runs one search at a
 * time; separate handles may run concurrently on separate streams.
 *
 * Errors.  Functions never exit the process.  On failure they return NULL or a
 * negative code, and bfs_last_error() (thread-local) describes the first
 * problem found, naming the offending index where there is one.
 */
#ifndef FRONTIER_BFS_H
#define FRONTIER_BFS_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes of bfs_run / bfs_set_policy / bfs_last_run_stats. */
#define BFS_EINVAL  (-1)  /* bad argument: NULL handle/output, source out of range, bad policy */
#define BFS_EHIP    (-2)  /* a HIP call failed; the message carries hipGetErrorString      */
#define BFS_ENOMEM  (-3)  /* device allocation failed                                        */
#define BFS_EDEVICE (-4)  /* a kernel reported an internal limit or a corrupted graph        */

typedef struct bfs_graph bfs_graph;   /* opaque handle */

/*
 * Wraps a CSR graph for searching.
 *   n        number of vertices, 1 <= n < 2^31
 *   row_ptr  device, n+1 entries: row_ptr[0] = 0, non-decreasing,
 *            row_ptr[n] = number of CSR entries m < 2^31
 *   col_idx  device, m entries, each in [0, n) (may be NULL when m = 0)
 * The arrays are validated on the device (the first bad index is named in
 * bfs_last_error), and the graph is classified: rows sorted or not, and
 * symmetric or not.  The bottom-up (pull) pass needs in-edges (Gunrock reading
 * guide, question 3): a symmetric graph serves as its own; for any other
 * graph the transpose is built here on the device (a counting sort by target,
 * m + n + 1 more ints), and if it does not fit the graph stays push-only.
 * Returns NULL on invalid input or allocation failure.  Uses the current
 * device and the null stream; synchronises before returning.
 */
bfs_graph *bfs_graph_create(int32_t n, const int32_t *row_ptr, const int32_t *col_idx);

/*
 * One breadth-first search from `source`.
 *   dist_out         device, n entries, required: hop count from source, -1 if
 *                    unreached (the sentinel of Chapter 22 and bfs.cu).
 *   parent_out       device, n entries, or NULL to skip: parent[source] =
 *                    source; for a reached v, a vertex p with dist[p] =
 *                    dist[v]-1 and v in adj(p) (any such p: which one may
 *                    vary between runs); -1 if unreached.
 *   level_sizes_out  device, capacity n entries, or NULL: entry k = number of
 *                    vertices at distance k, for k < L; entries from L on are
 *                    left untouched.
 *   stream           HIP stream for all work (0 = null stream).
 * Returns L >= 1, the number of non-empty levels (= max dist + 1), or a
 * negative BFS_E* code.  On BFS_EINVAL the outputs are untouched; after
 * BFS_EHIP or BFS_EDEVICE their contents are unspecified (on large graphs
 * dist is completed only by the launch that follows a finished search).
 */
int32_t bfs_run(bfs_graph *g, int32_t source, int32_t *dist_out, int32_t *parent_out,
                int32_t *level_sizes_out, hipStream_t stream);

/*
 * bfs_run without a handle and without any device allocation, for callers
 * that cannot allocate (code under HIP graph capture of its neighbours, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments and
 * results as bfs_graph_create followed by bfs_run with the default policy,
 * for a graph of at most 65,536 vertices and 2,097,152 CSR entries: the graph
 * is validated as bfs_graph_create validates it (BFS_EINVAL, with the first
 * bad index in bfs_last_error), then searched by the same kernels, the
 * direction switching included when the graph is symmetric with sorted rows
 * (any other graph is searched push-only: dist, L and level sizes do not
 * change).  The workspace (about 30 MB) is one fixed device array per GPU,
 * created with the library's code object and held until the process ends;
 * nothing is allocated or freed on any call.  Every call on one GPU shares
 * that array and leaves its contents behind, so calls that overlap on one GPU
 * (other threads, other streams) race and must be serialised by the caller.
 * Reads a few words back to the host per call and synchronises `stream`
 * before returning.  Returns L >= 1, or BFS_EINVAL (a bound exceeded, an
 * invalid graph or argument; outputs untouched), BFS_EHIP or BFS_EDEVICE.
 */
int32_t bfs_run_noalloc(int32_t n, const int32_t *row_ptr, const int32_t *col_idx, int32_t source,
                        int32_t *dist_out, int32_t *parent_out, int32_t *level_sizes_out,
                        hipStream_t stream);

/*
 * Frees the handle's workspace (the counterpart of the frees at the end of
 * bfs.cu's main in the Day 38 program, which releases the device graph and
 * the search's buffers once the runs are done).  The caller's row_ptr,
 * col_idx and output arrays are not touched.  NULL is a no-op.  Synchronises
 * the device first, so work still queued on the handle finishes.
 */
void bfs_graph_destroy(bfs_graph *g);

/*
 * Thread-local description of the last failure on this thread ("" if none).
 * It names the first bad index where there is one: the Day 38 program's
 * loadGraph rejects a graph file at its first bad line, and its CUDA_CHECK
 * reports a failed call with the runtime's error text; here both come back
 * as text and a return code instead of an exit.
 */
const char *bfs_last_error(void);

/*
 * The BFS_E* code behind the last NULL that bfs_graph_create returned on this
 * thread (BFS_EINVAL: invalid graph or argument; BFS_ENOMEM: the workspace
 * did not fit; BFS_EHIP: a HIP call failed); 0 after a successful create.
 * Same sources as bfs_last_error.
 */
int32_t bfs_last_error_code(void);

/* ---- measurement and test hooks (results never depend on them) --------- */

/* Direction policy: automatic switching, push (top-down) only, pull
 * (bottom-up) only.  Pull needs in-edges (see bfs_graph_create). */
#define BFS_DIR_AUTO 0
#define BFS_DIR_PUSH 1
#define BFS_DIR_PULL 2
/* Top-down advance: automatic (currently edge-balanced for every top-down
 * level that starts from a queue), degree-binned (lane / wavefront /
 * workgroup, hubs split across workgroups), edge-balanced (frontier-degree
 * scan plus tile partition by search over the scan). */
#define BFS_ADV_AUTO   0
#define BFS_ADV_BINNED 1
#define BFS_ADV_EDGE   2

/* Level loop.  Level launches go to a top-down kernel or a bottom-up kernel;
 * each reads the level to run and the frontier from device memory, runs that
 * level if its direction is the kernel's own and otherwise leaves it to the
 * next launch.  Level 0 itself runs in the initialisation launch when the
 * graph's rows are sorted, the source has at most 512 entries and that level
 * is top-down under the policy (its winners are the source's distinct
 * out-neighbours, so no claim is needed); the first level launch then starts
 * at level 1.
 *   DEVICE (default): launches are enqueued ahead in batches and the host
 *     waits once per batch; the first batch follows the handle's record of
 *     its recent searches' launches (else 12 alternating launches), later
 *     batches alternate and grow.  A small top-down level (up to 16,384
 *     vertices and 16,384 edges) runs on 32 workgroups that carry on level
 *     after level with a barrier among themselves, so a long thin search is a
 *     handful of launches.
 *   HOST: the host waits for every launch before the next one, as bfs.cu's
 *     runBfs in the Day 38 program waits for every level.
 *   CHAIN: as DEVICE but at most one level per launch (no small-frontier mode).
 * The small-frontier barrier's wait is bounded (2 s; the environment variable
 * FBFS_BARRIER_TIMEOUT_US, read at bfs_graph_create, overrides it for tests):
 * past it bfs_run returns BFS_EDEVICE instead of waiting forever.
 * On graphs of at least 2^23 vertices the levels run from or into a bitmap
 * (bottom-up levels, and the level after a wide top-down level) keep their
 * found sets as bitmaps, and a finishing launch after each batch writes dist
 * in vertex order once the search is done; FBFS_FINISH_MIN_N, read at
 * bfs_graph_create, lowers that size for tests.  Results are the same. */
#define BFS_LOOP_DEVICE 0
#define BFS_LOOP_HOST   1
#define BFS_LOOP_CHAIN  2

/*
 * Forces a policy for later bfs_run calls on this handle.  dist, L and the
 * level sizes are the same under every policy; only speed differs.
 * Returns 0, or BFS_EINVAL (unknown value, or pull on a graph without
 * in-edges: see bfs_graph_create).
 */
int32_t bfs_set_policy(bfs_graph *g, int32_t direction, int32_t advance, int32_t loop);

/*
 * Direction-switch parameters of the automatic policy, for later bfs_run calls
 * on this handle (defaults 40 and 96: Beamer, Asanovic and Patterson, SC 2012,
 * use 14 and 24 on CPUs; the bottom-up pass here is cheap enough relative to
 * the top-down one that pulling earlier and pushing again later measured
 * best on the R-MAT and Erdos-Renyi graphs).  After a top-down level, the next level pulls when
 * alpha * (sum of degrees of the frontier) exceeds the degree sum of the
 * vertices not yet reached; after a bottom-up level, it pushes again when
 * beta * |frontier| < n and the frontier shrank.  The PMPP chapter 15 notes
 * (section 15.7) state the vertex-count form of this rule.  dist, L and the
 * level sizes do not depend on them.  Returns 0, or BFS_EINVAL when the handle
 * is NULL or either value is outside [1, 1e6].
 */
int32_t bfs_set_switch(bfs_graph *g, int32_t alpha, int32_t beta);

/*
 * Per-level record of the last bfs_run on this handle, for the byte model and
 * tests: the per-level table of the "Day 38 - Graph traversal on a GPU" page
 * (section "What a level-synchronous search actually launches": frontier
 * size and edges to walk per level), with the direction each level ran in
 * (PMPP ch.15 notes, section 15.7: push or pull per level).  The frontier
 * sizes themselves are level_sizes_out of bfs_run.
 * For k < min(L, cap): dir[k] = 0 for a top-down level, 1 for a
 * bottom-up level; frontier_edges[k] = sum of degrees of level k's vertices.
 * Either array may be NULL.  Host memory.  Returns L of that run (0 if none
 * yet), or a negative code.
 */
int32_t bfs_last_run_stats(const bfs_graph *g, int32_t cap, int8_t *dir,
                           int64_t *frontier_edges);

/*
 * Where each level of the last bfs_run stored its outputs, for the byte model
 * (the per-level table of the "Day 38 - Graph traversal on a GPU" page,
 * section "What a level-synchronous search actually launches", extended by
 * what each launch writes).  For k < min(L, cap), flags[k] ORs:
 *   BFS_LF_QUEUE_FREE     a wide top-down level: winners go to the next
 *                         bitmap only, and their dist is left to the next level
 *   BFS_LF_FINDS_KEPT     the level's finds are kept as a bitmap; the
 *                         finishing launch writes their dist
 *   BFS_LF_FRONTIER_KEPT  the level keeps its frontier (left by a queue-free
 *                         level) as a bitmap for the finishing launch
 *   BFS_LF_FRONTIER_DIST  the level writes its frontier's dist (left by a
 *                         queue-free level) beside its own
 *   BFS_LF_FINISHING      (level 0 only) the search ended with the finishing
 *                         launch, which wrote dist of every vertex that no
 *                         level stored; the initialisation wrote none
 * Levels of the small-frontier mode and of the other search paths read 0.
 * Host memory, may be NULL.  Returns L of that run (0 if none yet), or a
 * negative code.
 */
#define BFS_LF_QUEUE_FREE     1
#define BFS_LF_FINDS_KEPT     2
#define BFS_LF_FRONTIER_KEPT  4
#define BFS_LF_FRONTIER_DIST  8
#define BFS_LF_FINISHING      16
int32_t bfs_last_run_level_flags(const bfs_graph *g, int32_t cap, uint8_t *flags);

/*
 * Timing hook.  When on, bfs_run's initialisation, level and finishing
 * launches each record a pair of HIP events as their kernel begins and ends
 * (the launch records them itself, so an interval holds the kernel and not
 * the gaps between launches).
 * Returns 0 or BFS_EINVAL.
 */
int32_t bfs_set_timing(bfs_graph *g, int32_t on);

/*
 * Milliseconds of the last timed bfs_run (host memory, any may be NULL):
 * init_ms = the initialisation launch (with level 0 when it runs there, see
 * the level loop above) and the finishing passes (the launch
 * after each batch of level launches that writes dist from the levels' kept
 * bitmaps once the search is done); level_ms = the level launches, each
 * timed alone (host waits between batches excluded); level_launches = level
 * launches issued (including the one that found the empty frontier and any
 * that exited at once after it).  Returns 0, or BFS_EINVAL if the last run was
 * not timed.
 */
int32_t bfs_last_run_timing(const bfs_graph *g, float *init_ms, float *level_ms,
                            int32_t *level_launches);

/*
 * The level launches of the last timed bfs_run split by kernel (host memory,
 * any may be NULL): milliseconds and launches of the top-down kernel and of
 * the bottom-up kernel, each launch timed by the HIP events it records as its
 * kernel begins and ends.  The two sums make up level_ms of
 * bfs_last_run_timing.  Returns 0, or BFS_EINVAL if the last run was not timed.
 */
int32_t bfs_last_run_kernel_timing(const bfs_graph *g, float *td_ms, int32_t *td_launches,
                                   float *bu_ms, int32_t *bu_launches);

/*
 * The level launches of the last timed bfs_run one by one (host memory, either
 * may be NULL; the first min(cap, count) entries are written): ms[i] = launch
 * i's time between the HIP events it records as its kernel begins and ends on the
 * run's stream; ran[i] = the device's record of its work: 1 the top-down
 * kernel ran a level or found the empty frontier, 2 the bottom-up kernel did,
 * 0 it passed its level on or exited at once (launches from index 64 on are
 * not recorded and read 0).  A top-down launch in the small-frontier mode may
 * run several levels.  The per-level launch table of the "Day 38 - Graph
 * traversal on a GPU" page (section "What a level-synchronous search actually
 * launches") is what this reproduces.  Returns the number of launches, or
 * BFS_EINVAL if the last run was not timed or cap < 0.  The walk, shortest
 * paths and the non-default compactions record no launches (count 0).
 */
int32_t bfs_last_run_launch_timing(const bfs_graph *g, int32_t cap, float *ms, uint8_t *ran);

/*
 * Validator V5 of a debug build: copies to counts_out (device, n entries) how
 * many times each vertex was written into a next frontier during the last
 * bfs_run on this handle (a queue segment, a bitmap-only winner of a wide
 * top-down level, a bottom-up find, a level-0 winner written by the
 * initialisation launch); the source, the initial frontier, reads
 * 0.  On a correct search every other reached vertex reads exactly 1 and
 * every unreached vertex 0: a frontier with duplicates ("Day 38 - Graph
 * traversal on a GPU", Pitfalls; Chapter 22, section 22.1, where a naive
 * claim discovers a vertex twice) still gives the right dist, so only a count
 * shows it.  Runs of the default direction-optimising path only (not the
 * non-default compactions).  Returns 0; BFS_EINVAL for a NULL argument or a
 * library built without -DFBFS_COUNT_ENQUEUES (the normal build).
 */
int32_t bfs_debug_enqueue_counts(const bfs_graph *g, int32_t *counts_out);

/*
 * Claim and compaction primitives of the top-down level (Gunrock reading
 * guide, step 2; "Day 38 - Graph traversal on a GPU", on day 33's
 * compaction).  claim: BFS_CLAIM_BITMAP (an atomicOr on the visited bitmap
 * elects the one writer of dist and parent) or BFS_CLAIM_MIN (atomicMin on
 * dist: the caller that read a larger old value wins).  compaction:
 * BFS_COMPACT_DEFAULT, the direction-optimising path of bfs_run (claims with
 * the bitmap, so claim must be BFS_CLAIM_BITMAP); or a top-down-only search
 * whose level loop reads two counters per level on the host, with the next
 * frontier built by BFS_COMPACT_ATOMIC (winners appended at a
 * wavefront-aggregated atomic cursor; order varies), BFS_COMPACT_PADDED (the
 * idempotent advance: every frontier edge writes its neighbour, or -1 where
 * it lost, at its own position, and that padded array is the next
 * frontier, one entry per frontier edge of the level before),
 * BFS_COMPACT_FILTER (the padded array compacted by flag, exclusive scan and
 * scatter; order of the edges) or BFS_COMPACT_FLAGS (flag every vertex with
 * the new level, scan the flags over all n vertices, scatter: the frontier in
 * id order, at O(n) per level).  dist and level_sizes are those of bfs_run;
 * parent is a frontier neighbour.  A non-default compaction allocates its
 * buffers (five arrays of max(n, m) + 1 ints) on this call.  Returns 0;
 * BFS_EINVAL for a NULL handle or an unknown or unsupported pair;
 * BFS_ENOMEM if the buffers do not fit.
 */
#define BFS_CLAIM_BITMAP    0
#define BFS_CLAIM_MIN       1
#define BFS_COMPACT_DEFAULT 0
#define BFS_COMPACT_ATOMIC  1
#define BFS_COMPACT_PADDED  2
#define BFS_COMPACT_FILTER  3
#define BFS_COMPACT_FLAGS   4
int32_t bfs_set_primitives(bfs_graph *g, int32_t claim, int32_t compaction);

/*
 * Single-source shortest paths over the same CSR and frontier machinery: the
 * atomic-min relaxation that the Gunrock reading guide (step 2) extends the
 * BFS lambda to, where a neighbour wins only with a strictly smaller
 * distance.  weights (device, m entries, uint32) holds the weight of each CSR
 * entry (row u to col_idx[e]); every weight must be at most max_weight, and
 * n * max_weight must stay below 2^32 - 1 (distances are kept in 32 bits).
 * dist_out (device, n int64): the shortest distance, -1 if unreachable.
 * pred_out (device, n int32, or NULL): the smallest u with an entry u -> v
 * and dist[u] + w = dist[v]; the source's own id for the source; -1 if
 * unreachable.  Both are unique, so results compare exactly.  Rounds of
 * frontier relaxation run until no distance drops; the host reads one counter
 * per round; bfs_last_run_stats then reports the rounds, each with the
 * frontier edges it relaxed.  Uses the handle's SSSP buffers (about 24n bytes, allocated on
 * the first call); must not overlap other calls on the handle.  Returns the
 * number of rounds (>= 1); BFS_EINVAL for a NULL handle or buffer, a source
 * outside [0, n), a max_weight that breaks the bound, or a weight above
 * max_weight (then the outputs are unspecified); BFS_ENOMEM; BFS_EHIP.
 */
int32_t bfs_sssp(bfs_graph *g, int32_t source, const uint32_t *weights, uint32_t max_weight,
                 int64_t *dist_out, int32_t *pred_out, hipStream_t stream);

/*
 * Isolated neighbour walk of one level: the measurement the "Day 38 - Graph
 * traversal on a GPU" page uses to compare thread-to-work mappings without
 * the atomics, frontier build and distance writes of a real level (section
 * "Measuring the mapping without measuring the launch").  For listed vertex i
 * (vertices[i], device, count entries, each in [0, n)) out[i] (device, count
 * entries) becomes the wrapping unsigned 32-bit sum over r = 0 .. repeats-1
 * and over the vertex's CSR entries of (neighbour id XOR r).  mapping is one
 * of BFS_WALK_*: one lane per list; one 64-lane wavefront per list; degree
 * bins over the whole level (a lane per list under 32 entries, a wavefront
 * per list under 512, a workgroup per longer list); or the edge-balanced
 * split, where an exclusive scan of the listed degrees gives every lane an
 * equal short run of entries and the owner of its first entry by binary
 * search (Gunrock reading guide, steps 4 and 5).  Uses the handle's
 * workspace, so it must not overlap a bfs_run on the same handle; runs on
 * stream and returns after the work finished.  With the timing hook on,
 * bfs_last_run_timing reports the walk's kernels as level_ms.  Returns 0;
 * BFS_EINVAL for a NULL handle or buffer, negative count or repeats, an
 * unknown mapping, count above 8n, or a listed id outside [0, n) (then out is
 * unspecified); BFS_EHIP if a HIP call fails.
 */
#define BFS_WALK_LANE   0
#define BFS_WALK_WAVE   1
#define BFS_WALK_BINNED 2
#define BFS_WALK_MERGE  3
int32_t bfs_walk_level(bfs_graph *g, const int32_t *vertices, int32_t count, int32_t mapping,
                       int32_t repeats, uint32_t *out, hipStream_t stream);

/*
 * Graph facts found by bfs_graph_create (host memory, any may be NULL):
 * CSR entry count, rows-sorted flag, symmetric flag, maximum degree, and
 * whether the bottom-up (pull) pass is available: always on a symmetric
 * graph, and on any other graph once its transpose (the in-edges) was built,
 * which fails only when device memory runs short.  Returns 0 or BFS_EINVAL.
 */
int32_t bfs_graph_info(const bfs_graph *g, int64_t *m, int32_t *sorted_rows,
                       int32_t *symmetric, int32_t *max_degree, int32_t *pull_ready);

#ifdef __cplusplus
}
#endif

#endif /* FRONTIER_BFS_H */
