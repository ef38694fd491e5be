/*
 * pr.h -- C ABI of libpr, PageRank power iteration with dangling-node
 * redistribution on one AMD Instinct MI355X (gfx950), and the valued sparse
 * matrix-vector product its pull iteration generalizes (pr_spmv, below), and
 * breadth-first search and weakly connected components on the same CSR
 * (pr_bfs, pr_wcc).
 *
 * The method ("100 Days of GPU", Day 40 "PageRank on a real graph in CUDA",
 * section "One iteration, three shapes of work"):
 *
 *     x'[v] = (1 - d)/n + d * ( sum over in-neighbours u of x[u]/outdeg[u] + D/n )
 *
 * where D is the rank held by vertices with no out-edge (dangling vertices) in
 * the vector the iteration starts from.  One iteration is a pull-style sparse
 * matrix-vector product over the in-edge (transposed) graph plus two
 * full-array reductions: the dangling mass and the L1 distance between
 * successive vectors, which decides convergence.  The same page builds the
 * in-edge graph once with a counting sort (histogram, prefix sum, scatter).
 *
 * Conventions for every entry point:
 *   - Graphs are CSR with int32 indices: row_ptr[n+1], col_idx[nnz], and
 *     nnz <= INT32_MAX.  "Out-edge CSR" rows list the targets of each vertex;
 *     "in-edge CSR" rows list the sources pointing at each vertex.
 *   - Pointers named *_dev are device pointers (hipMalloc'd or torch CUDA
 *     tensors); the caller owns them and keeps them alive while any work that
 *     uses them is in flight.  Host pointers are named *_host.
 *   - Workspaces are caller-allocated device memory of at least the size the
 *     matching *_workspace_bytes() call returns, 256-byte aligned.  The
 *     library never allocates device memory and never uses the null stream.
 *   - `stream` is a hipStream_t (passed as void*); all device work is enqueued
 *     on it.  An entry point returns once its work is enqueued unless its
 *     description says it synchronizes.
 *   - Every entry point returns PR_OK (0) or a negative pr_status; no C++
 *     exception crosses the ABI.  pr_last_error() gives the calling thread's
 *     most recent error message.
 */
#ifndef PR_H
#define PR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pr_status {
    PR_OK = 0,
    PR_ERR_ARG = -1,       /* null pointer, n < 1, nnz < 0 or > INT32_MAX, d outside [0,1],
                              max_iter < 1, unknown flag bits */
    PR_ERR_WORKSPACE = -2, /* workspace too small or not 256-byte aligned */
    PR_ERR_GRAPH = -3,     /* malformed CSR found by PR_VALIDATE */
    PR_ERR_HIP = -4        /* a HIP runtime call or kernel launch failed */
} pr_status;

/* Flag for pr_transpose and pr_plan_create. */
#define PR_VALIDATE 0x1u /* check the input CSR on the device (row_ptr[0] == 0,
                            non-decreasing, row_ptr[n] == nnz, 0 <= col < n); this
                            synchronizes `stream` once to read the verdict.  Without
                            it malformed input cannot fault the GPU (every device
                            index is clamped) but the output is unspecified. */

/* Flags for pr_run. */
#define PR_X0_GIVEN 0x1u      /* x holds the start vector on entry (warm start, or a
                                 resume from a saved vector); otherwise 1/n */
#define PR_RECORD_EVENTS 0x2u /* record the plan's timing events around the
                                 iteration launches (see pr_plan_iteration_ms
                                 and pr_plan_kernel_ms) */

/* Device bytes pr_transpose needs as workspace.  Host-only, no device work. */
size_t pr_transpose_workspace_bytes(int32_t n, int64_t nnz);

/*
 * In-edge CSR of an out-edge CSR (Day 40, "One iteration, three shapes of
 * work": the counting-sort transpose).  Built on the device as a stable
 * least-significant-digit radix sort of the (target, source) pairs by target:
 * each 8-bit pass is a histogram, an exclusive scan and a scatter.
 * in_row_ptr[v] = number of edges whose target is below v (the exclusive scan
 * of the in-degree histogram), read off the sorted targets.
 *
 *   n, nnz                     vertices and edges
 *   out_row_ptr_dev[n+1]       out-edge CSR (read only)
 *   out_col_idx_dev[nnz]
 *   in_row_ptr_dev[n+1]        written: in_row_ptr[v+1]-in_row_ptr[v] = in-degree of v
 *   in_col_idx_dev[nnz]        written: the sources of each in-row in ascending id
 *                              order, parallel edges kept adjacent; bit-identical to
 *                              a sequential counting sort over sources in order
 *   ws_dev, ws_bytes           workspace, >= pr_transpose_workspace_bytes(n, nnz)
 *   flags                      0 or PR_VALIDATE
 *
 * Asynchronous on `stream` unless PR_VALIDATE is given.
 */
int pr_transpose(int32_t n, int64_t nnz, const int32_t* out_row_ptr_dev,
                 const int32_t* out_col_idx_dev, int32_t* in_row_ptr_dev,
                 int32_t* in_col_idx_dev, void* ws_dev, size_t ws_bytes, uint32_t flags,
                 void* stream);

/*
 * pr_transpose without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, output and errors as
 * pr_transpose; the workspace is instead a device array inside the library,
 * PR_NOALLOC_SCRATCH_BYTES bytes, of which every GPU the library runs on
 * holds one copy until the process ends.  The call allocates nothing (no
 * hipMalloc, no hipFree, no allocating library routine).
 *
 * Limit: graphs whose pr_transpose_workspace_bytes(n, nnz) exceeds
 * PR_NOALLOC_SCRATCH_BYTES (about 8 million edges) are rejected with
 * PR_ERR_WORKSPACE before any device work.
 * Calls on one GPU share its array: calls that overlap in time on the same
 * GPU (on different streams, or from different threads) race and give
 * unspecified output.  Every array entry a call reads is written earlier in
 * the same call, so nothing carries over from one call to the next.
 */
#define PR_NOALLOC_SCRATCH_BYTES (128u << 20)
int pr_transpose_noalloc(int32_t n, int64_t nnz, const int32_t* out_row_ptr_dev,
                         const int32_t* out_col_idx_dev, int32_t* in_row_ptr_dev,
                         int32_t* in_col_idx_dev, uint32_t flags, void* stream);

/* Opaque iteration plan. */
typedef struct pr_plan pr_plan;

/* Flag for pr_plan_create: iterate with the degree-bucketed row-per-lane /
 * group / wavefront pull kernels over the plan's in-edge CSR instead of the
 * default tiled pull (see pr_plan_create). */
#define PR_PLAN_BUCKETED 0x2u

/* Device bytes the plan keeps for its lifetime (pr_plan_create's ws_dev), and
 * the device bytes it needs only while pr_plan_create runs (scratch_dev).
 * Host-only, no device work; 0 for invalid sizes. */
size_t pr_plan_workspace_bytes(int32_t n, int64_t nnz);
size_t pr_plan_scratch_bytes(int32_t n, int64_t nnz);

/*
 * Build an iteration plan for one graph, all inside ws_dev:
 *   - a renumbering of the vertices ("plan order"): rows split into degree
 *     buckets by in-degree ("gpu-graph-study", PageRank T4 degree-bucketed
 *     load balancing), the longest-row bucket first, and inside each bucket
 *     by decreasing out-degree, ties by id.  Every bucket is a contiguous
 *     range of plan ids, and the sources read most often sit together at the
 *     start of each range;
 *   - inverse out-degrees: 1/outdeg[u], or 0 for a dangling vertex (Meerkat's
 *     PageRank section caches the per-vertex ratio x[u]/out[u]; the
 *     "gpu-graph-study" T3 tier precomputes 1/deg);
 *   - the in-edges in one of two layouts:
 *       default (tiled pull): each bucket cut into tiles of 2^k consecutive
 *         rows (k per bucket, so a tile holds about 2^22 in-edges, at most
 *         16384 rows), a tile's in-edges stored as (source, row offset) pairs
 *         in increasing source order; the iteration streams a tile's edges in
 *         that order and adds each contribution into the row's accumulator
 *         (64-bit fixed point in LDS, exact and order-free);
 *       PR_PLAN_BUCKETED: the in-edge CSR (rows and sources in plan ids, each
 *         row listing its sources in increasing plan id), iterated with one
 *         lane, a 4- or 16-lane group or a 64-lane wavefront per row by
 *         bucket, hub rows split in chunks;
 *     either built from the out-edge CSR on the device with the counting-sort
 *     machinery of pr_transpose;
 *   - the work list of the iteration kernel and the per-run scratch.
 *
 *   plan_out                   receives the plan (host memory owned by the
 *                              library; release with pr_plan_destroy)
 *   out_row_ptr_dev[n+1]       out-edge CSR (read only; not kept)
 *   out_col_idx_dev[nnz]
 *   ws_dev, ws_bytes           >= pr_plan_workspace_bytes(n, nnz) (enough for
 *                              either layout); must stay allocated and
 *                              untouched while the plan lives
 *   scratch_dev, scratch_bytes >= pr_plan_scratch_bytes(n, nnz); free for other
 *                              use once the call returns
 *   flags                      PR_VALIDATE | PR_PLAN_BUCKETED; the default
 *                              (tiled) layout takes n <= 2^30, PR_PLAN_BUCKETED
 *                              any n that the sizes allow
 *
 * Synchronizes `stream` (bucket sizes and the tiles' or hub rows' edge counts
 * are read back to build the work list).  The plan belongs to the device
 * current at creation.  Without PR_VALIDATE a malformed CSR cannot make the
 * library access memory outside the buffers (targets are clamped), but the
 * ranks are then unspecified.
 */
int pr_plan_create(pr_plan** plan_out, int32_t n, int64_t nnz, const int32_t* out_row_ptr_dev,
                   const int32_t* out_col_idx_dev, void* ws_dev, size_t ws_bytes,
                   void* scratch_dev, size_t scratch_bytes, uint32_t flags, void* stream);

/* Release a plan (host state and its events); NULL is allowed.  The caller
 * must make sure no pr_run on it is still in flight. */
int pr_plan_destroy(pr_plan* plan);

/*
 * Power iteration (Day 40 update; Meerkat's PageRank section gives the same
 * loop with max_iter and an L1 error margin).
 *
 *   d              damping factor in [0, 1] (0.85 on the pages); the device
 *                  arithmetic uses it rounded to float, the constant term
 *                  (1-d)/n + d*D/n is formed in double
 *   tol            tol > 0: stop after the first iteration t whose L1 distance
 *                  sum_v |x_t[v] - x_{t-1}[v]| is below tol (that iteration
 *                  counts and its vector is returned); tol <= 0: run exactly
 *                  max_iter iterations (the timed mode)
 *   max_iter       >= 1
 *   x_dev[n]       float; start vector on entry if PR_X0_GIVEN (else ignored and
 *                  1/n is used), ranks after the last iteration on exit
 *   l1_trace_dev   float[max_iter]; entry t-1 = L1 distance of iteration t;
 *                  entries after the stopping iteration are left untouched
 *   sum_trace_dev  float[max_iter] or NULL; entry t-1 = sum of x after iteration t
 *                  (the page's conserved quantity, which should stay 1)
 *   iterations_host  receives the number of iterations performed
 *   flags          PR_X0_GIVEN | PR_RECORD_EVENTS
 *
 * The dangling mass and the stop test stay on the device: no iteration waits
 * for the host.  With tol <= 0 the call only enqueues work and does not
 * synchronize.  With tol > 0 it enqueues iterations in chunks, reads the
 * device stop flag after each chunk while the next chunk runs, and
 * synchronizes `stream` before returning.  Calls on one plan must not
 * overlap in time (they share the plan's scratch).
 */
int pr_run(pr_plan* plan, double d, double tol, int32_t max_iter, float* x_dev,
           float* l1_trace_dev, float* sum_trace_dev, int32_t* iterations_host, uint32_t flags,
           void* stream);

/* Elapsed milliseconds between the timing events the last pr_run with
 * PR_RECORD_EVENTS recorded (first iteration launch to last), waiting for the
 * second event.  Divide by the iteration count for the mean per iteration. */
int pr_plan_iteration_ms(pr_plan* plan, float* ms_host);

/* Mean duration in milliseconds of the iteration's gather-and-update kernel
 * alone, over the launches the last pr_run with PR_RECORD_EVENTS timed (one
 * event pair around each of its first 64 iterations), waiting for them.
 * *launches_host receives the number of launches averaged.  This is the
 * kernel that moves almost all of an iteration's bytes; the rest of the
 * iteration is, when some tiles (or, bucketed, some in-rows) are cut into
 * pieces too many to finish inside it, the kernel that finishes their rows,
 * and in the bucketed layout the per-iteration reduction (one workgroup). */
int pr_plan_kernel_ms(pr_plan* plan, float* mean_ms_host, int32_t* launches_host);

/* Introspection for tests and benchmarks: the number of degree buckets and,
 * per bucket, its first row-length, row count and edge count (host arrays of
 * length at least pr_plan_num_buckets()). */
int pr_plan_num_buckets(void);
int pr_plan_buckets(const pr_plan* plan, int32_t* min_len_host, int32_t* rows_host,
                    int64_t* edges_host);

/* Introspection for tests: device pointers (inside the plan's workspace) to
 * the plan's in-edge CSR (n+1 row pointers, nnz sources; rows and sources in
 * plan ids; NULL for a tiled plan) and to new_id[n] (the plan id of each of
 * the caller's vertices).  Any output pointer may be NULL. */
int pr_plan_layout(const pr_plan* plan, const int32_t** in_row_ptr_dev,
                   const int32_t** in_col_idx_dev, const int32_t** new_id_dev);

/* Introspection for tests, tiled plans only (PR_ERR_ARG otherwise): device
 * pointers to tile_src[S], tile_row[S], tile_block[S/256] and
 * tile_ptr[n_tiles+1] (the first slot of each tile; S = tile_ptr[n_tiles]);
 * the tile count; and, into host arrays of n_tiles entries, each tile's first
 * plan id and row count.  Slots hold a tile's edges in increasing source
 * order, padded to a multiple of 256 (padding slots repeat the tile's last
 * source with row offset 16384, an accumulator that is never read), and each
 * block of 256 is stored transposed: edge 64*i + l of a block sits at slot
 * 4*l + i.  Block b is narrow when its sources span less than 2^16: then
 * tile_block[b] is its first source and slot k of the block holds
 * (source - tile_block[b]) | row_offset << 16 in tile_src; otherwise
 * tile_block[b] = -1, tile_src holds the source and tile_row the row offset
 * (tile_row is not kept up to date for narrow blocks).  Any output may be
 * NULL (call once with NULL arrays to learn n_tiles). */
int pr_plan_tiles(const pr_plan* plan, const int32_t** tile_src_dev, const uint16_t** tile_row_dev,
                  const int32_t** tile_block_dev, const int32_t** tile_ptr_dev, int32_t* n_tiles_host,
                  int32_t* row0_host, int32_t* rows_host);

/* ------------------------------------------------------------------------
 * Valued sparse product y = A x in double precision ("A Pedagogical
 * Introduction to Porting a Conjugate Gradient Solver to CUDA": the sparse
 * product that takes most of its CG solver's time, on the CSR arrays
 * row_offsets[n_rows+1], cols[nnz], vals[nnz]):
 *
 *     y[i] = sum over j in [row_ptr[i], row_ptr[i+1]) of vals[j] * x[col_idx[j]]
 *
 * A plan holds the row schedule of one sparsity pattern, built once on the
 * device: rows of at most 64 entries in streamed blocks (their products are
 * each rounded once and added in stored order from 0.0, so such rows come
 * out bit-identical to a sequential CPU loop without fused multiply-adds),
 * rows of 65..1024 entries one 64-lane wavefront each, longer rows in chunks
 * of 4096 entries whose sums are added in order.  Rows longer than 64 are
 * summed in a fixed tree order: deterministic, within the usual k-term
 * rounding bound of the exact sum.
 * ------------------------------------------------------------------------ */
typedef struct pr_spmv_plan pr_spmv_plan;

/* Device bytes a product plan keeps for its lifetime (ws_dev) and needs only
 * while pr_spmv_plan_create runs (scratch_dev).  Host-only; 0 for invalid sizes. */
size_t pr_spmv_workspace_bytes(int32_t n_rows, int64_t nnz);
size_t pr_spmv_scratch_bytes(int32_t n_rows, int64_t nnz);

/*
 * Build the row schedule of a CSR sparsity pattern.
 *
 *   plan_out                 receives the plan (host memory owned by the library;
 *                            release with pr_spmv_plan_destroy)
 *   n_rows, n_cols, nnz      n_rows >= 0, n_cols >= 0, 0 <= nnz <= INT32_MAX;
 *                            nnz > 0 needs n_rows >= 1 and n_cols >= 1
 *   row_ptr_dev[n_rows+1]    the pattern; BORROWED: the plan keeps both pointers,
 *   col_idx_dev[nnz]         and the caller keeps them allocated and unchanged
 *                            while the plan lives
 *   ws_dev, ws_bytes         >= pr_spmv_workspace_bytes(n_rows, nnz), 256-byte
 *                            aligned, untouched while the plan lives
 *   scratch_dev, scratch_bytes  >= pr_spmv_scratch_bytes(n_rows, nnz); free
 *                            again once the call returns
 *   flags                    0 or PR_VALIDATE (row_ptr[0] == 0, non-decreasing,
 *                            row_ptr[n_rows] == nnz, 0 <= col < n_cols; else
 *                            PR_ERR_GRAPH)
 *
 * Synchronizes `stream` (the block and row counts are read back, and the
 * schedule is complete when the call returns).
 * Without PR_VALIDATE a malformed pattern cannot make the product access
 * memory outside the arrays (offsets and columns are clamped) but y is then
 * unspecified; row pointers that describe more rows of a kind than nnz
 * allows are rejected with PR_ERR_GRAPH.
 */
int pr_spmv_plan_create(pr_spmv_plan** plan_out, int32_t n_rows, int32_t n_cols, int64_t nnz,
                        const int32_t* row_ptr_dev, const int32_t* col_idx_dev, void* ws_dev,
                        size_t ws_bytes, void* scratch_dev, size_t scratch_bytes, uint32_t flags,
                        void* stream);

/* Release a product plan; NULL is allowed.  No pr_spmv on it may be in flight. */
int pr_spmv_plan_destroy(pr_spmv_plan* plan);

/*
 * y = A x on `stream`, asynchronous.
 *
 *   vals_dev[nnz]     the values, in the order of the plan's col_idx (they may
 *                     change between calls; the pattern may not)
 *   x_dev[n_cols]     input vector (read only)
 *   y_dev[n_rows]     written; must not overlap x_dev or vals_dev
 *
 * The plan's device must be current.  Calls on one plan must not overlap in
 * time when it has rows longer than 1024 entries (their chunk sums share the
 * plan's workspace); otherwise calls may run concurrently.
 */
int pr_spmv(const pr_spmv_plan* plan, const double* vals_dev, const double* x_dev, double* y_dev,
            void* stream);

/* Introspection for tests and benchmarks: counts_host[4] receives the number
 * of streamed blocks, of 65..1024-entry rows, of longer rows, and of chunks. */
int pr_spmv_plan_items(const pr_spmv_plan* plan, int32_t* counts_host);

/* ---------------------------------------------------------------------------
 * Traversals on the same out-edge CSR ("gpu-graph-study", sections
 * "Traversal (BFS / WCC)" and "Traversal T4 -- degree-bucketed BFS / WCC"):
 * breadth-first levels from a source, and weakly connected components.  Both
 * schedule rows by out-degree: rows of fewer than 256 edges are walked 64 at
 * a time by one wavefront as one flattened edge list; longer rows are cut
 * into 2048-edge chunks dealt to whole workgroups.
 * ------------------------------------------------------------------------ */

/* Device bytes pr_bfs / pr_wcc need as workspace.  Host-only; 0 for invalid
 * sizes (n < 1, nnz < 0 or > INT32_MAX). */
size_t pr_bfs_workspace_bytes(int32_t n, int64_t nnz);
size_t pr_wcc_workspace_bytes(int32_t n, int64_t nnz);

/*
 * Breadth-first search over the out-edges from `source`, level by level.  A
 * level is expanded top-down (each frontier vertex's out-edges; a vertex is
 * claimed by the first edge that reaches it, with a compare-and-swap on its
 * level) or, when the in-edge CSR is given and the frontier is large,
 * bottom-up (each unvisited vertex looks through its in-edges for a source on
 * the current level), by the direction-optimizing rule: bottom-up once the
 * frontier's out-edges exceed 1/14 of the unexplored edges, top-down again
 * once the frontier holds fewer than n/24 vertices.  The levels do not
 * depend on the direction taken.
 *
 *   n, nnz                   n >= 1, 0 <= nnz <= INT32_MAX
 *   row_ptr_dev[n+1],        out-edge CSR (read only); duplicate edges and
 *   col_idx_dev[nnz]         self-loops are allowed
 *   in_row_ptr_dev[n+1],     the in-edge CSR of the same graph (pr_transpose's
 *   in_col_idx_dev[nnz]      output), or both NULL for top-down levels only
 *   source                   0 <= source < n, else PR_ERR_ARG
 *   level_dev[n]             out: level[v] = edges on a shortest directed path
 *                            source -> v, -1 if v is unreachable
 *   depth_host               out (may be NULL): the largest level reached
 *   edges_scanned_host       out (may be NULL): out-edges of the vertices
 *                            reached (the edges a top-down search scans)
 *   ws_dev, ws_bytes         >= pr_bfs_workspace_bytes(n, nnz), 256-byte aligned
 *   flags                    0 or PR_VALIDATE (both CSRs checked as for
 *                            pr_transpose; that the second is the transpose
 *                            of the first is the caller's promise)
 *
 * Synchronizes `stream`: levels are launched in batches (4, 8, ... up to 64)
 * and the next frontier's size is read back once per batch.  Without
 * PR_VALIDATE a malformed CSR cannot make a kernel leave its arrays (edge
 * offsets and columns are clamped) but the levels are then unspecified.
 */
int pr_bfs(int32_t n, int64_t nnz, const int32_t* row_ptr_dev, const int32_t* col_idx_dev,
           const int32_t* in_row_ptr_dev, const int32_t* in_col_idx_dev, int32_t source,
           int32_t* level_dev, int32_t* depth_host, int64_t* edges_scanned_host, void* ws_dev,
           size_t ws_bytes, uint32_t flags, void* stream);

/*
 * Weakly connected components (edge directions ignored): label_dev[v] = the
 * smallest vertex id in v's component, which is where the page's min-label
 * propagation settles.  Computed by linking trees (a tree's root is always
 * its smallest vertex): each vertex's first two out-edges, then every other
 * edge, then a pass that points every vertex at its root.  With the in-edge
 * CSR, the full pass skips the vertices already in the tree most of 1024
 * sampled vertices share and reads the in-edges of the rest instead.
 *
 *   n, nnz, row_ptr_dev, col_idx_dev, in_row_ptr_dev, in_col_idx_dev
 *                            as for pr_bfs (the in-edge CSR may be NULL)
 *   label_dev[n]             out
 *   n_components_host        out (may be NULL): number of components; when
 *                            given, the call synchronizes `stream`
 *   ws_dev, ws_bytes         >= pr_wcc_workspace_bytes(n, nnz), 256-byte aligned
 *   flags                    0 or PR_VALIDATE
 *
 * Asynchronous unless n_components_host or PR_VALIDATE is given.  Calls that
 * share a workspace must not overlap in time.
 */
int pr_wcc(int32_t n, int64_t nnz, const int32_t* row_ptr_dev, const int32_t* col_idx_dev,
           const int32_t* in_row_ptr_dev, const int32_t* in_col_idx_dev, int32_t* label_dev,
           int32_t* n_components_host, void* ws_dev, size_t ws_bytes, uint32_t flags,
           void* stream);

/* Human-readable name of a status code (static storage). */
const char* pr_status_string(int status);

/* Message of the calling thread's most recent failure (thread-local storage,
 * valid until the next call on the same thread). */
const char* pr_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PR_H */
