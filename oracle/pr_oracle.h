/*
 * PageRank power-iteration oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, sequential, double-precision CPU implementation of what the GPU
 * library computes, written from the method's definition.  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it; the
 * product path never calls it.  It shares no code, header or build step with
 * the GPU library.
 *
 * Sources of the method (cited by page title and section):
 *   "100 Days of GPU", Day 40 "PageRank on a real graph in CUDA":
 *     section "One iteration, three shapes of work" -- the update
 *       x'[v] = (1-d)/n + d * (sum_{u -> v} x[u]/outdeg[u] + D/n),
 *     d = 0.85, D = rank held by vertices with no out-edge, the host
 *     counting-sort transpose (histogram, prefix sum, scatter) from out-edges
 *     to in-edges, the L1 convergence distance, and the invariant that the
 *     ranks sum to 1 after every pass;
 *     section "Exercise" (Hint 2, Solution) -- the variant with the dangling
 *     term removed, whose total obeys S' = (1-d) + d (S - D).
 *   "A Pedagogical Introduction to Porting a Conjugate Gradient Solver to
 *     CUDA": the CSR arrays row_offsets / cols / vals and the product
 *     y[i] = sum over j in row i of vals[j] * x[cols[j]], in double, summed
 *     in stored order (the thread-per-row kernel and the CPU loop it ports).
 *   "gpu-graph-study", sections "Traversal (BFS / WCC)" and "Traversal T4 --
 *     degree-bucketed BFS / WCC": breadth-first levels from a source over the
 *     out-edges, and weakly connected components (edge directions ignored)
 *     labelled by label propagation, whose fixed point gives every vertex the
 *     smallest id of its component.
 *   "Meerkat: A Framework for Dynamic Graph Algorithms on GPUs", PageRank
 *     section -- static start 1/n, iteration i built from iteration i-1,
 *     teleport mass from the zero-out-degree vertices of iteration i-1, and
 *     delta = L1 distance between successive vectors bounded by max_iter.
 *
 * Return codes: 0 ok, -1 bad argument, -2 malformed CSR, -3 out of memory.
 */
#ifndef PR_ORACLE_H
#define PR_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Sequential counting-sort transpose of an out-edge CSR (n vertices, m edges)
 * into an in-edge CSR.  Within each in-row the sources appear in ascending
 * order (edges are visited source by source, in stored order).  All arrays are
 * host memory owned by the caller: in_row_ptr[n+1], in_col_idx[m]. */
int pro_transpose(int32_t n, int64_t m, const int32_t* out_row_ptr, const int32_t* out_col_idx,
                  int32_t* in_row_ptr, int32_t* in_col_idx);

/* Power iteration from x0 (or 1/n when x0 is NULL) on the out-edge CSR.
 *   d            damping factor in [0, 1]
 *   tol          stop after the first iteration t whose L1 distance is < tol;
 *                tol <= 0 runs exactly max_iter iterations
 *   flags        PRO_DROP_DANGLING: use D = 0 (the page's exercise variant)
 *   x            out: ranks after the last iteration performed, double[n]
 *   l1_trace     out (may be NULL): L1 distance of iteration t at [t-1]
 *   sum_trace    out (may be NULL): sum of the ranks after iteration t
 *   dmass_trace  out (may be NULL): dangling mass D used by iteration t
 *   iterations   out: iterations performed
 *   loop_seconds out (may be NULL): wall time of the iteration loop alone */
#define PRO_DROP_DANGLING 1u
int pro_pagerank(int32_t n, int64_t m, const int32_t* out_row_ptr, const int32_t* out_col_idx,
                 double d, double tol, int32_t max_iter, const double* x0, uint32_t flags,
                 double* x, double* l1_trace, double* sum_trace, double* dmass_trace,
                 int32_t* iterations, double* loop_seconds);

/* Sparse matrix-vector product y = A x of a valued CSR matrix with n_rows
 * rows, n_cols columns and nnz stored entries: y[i] = 0.0 + the products
 * vals[j] * x[col_idx[j]] added one at a time for j = row_ptr[i] ..
 * row_ptr[i+1]-1.  Each product and each sum is rounded on its own (the file
 * is built without contraction to fused multiply-adds).  Host arrays owned by
 * the caller: row_ptr[n_rows+1], col_idx[nnz], vals[nnz], x[n_cols], y[n_rows].
 * loop_seconds (may be NULL): wall time of the product loop. */
int pro_spmv(int32_t n_rows, int32_t n_cols, int64_t nnz, const int32_t* row_ptr,
             const int32_t* col_idx, const double* vals, const double* x, double* y,
             double* loop_seconds);

/* Breadth-first levels from `source` over the out-edges: level[v] = edges on a
 * shortest directed path source -> v, or -1 if v is unreachable.  Host arrays:
 * level[n].  Optional outputs: *depth = the largest level reached (the
 * search's depth; 0 when only the source is reached), *edges_scanned =
 * out-edges of the reached vertices,
 * *loop_seconds = wall time of the search. */
int pro_bfs(int32_t n, int64_t m, const int32_t* row_ptr, const int32_t* col_idx, int32_t source,
            int32_t* level, int32_t* depth, int64_t* edges_scanned, double* loop_seconds);

/* Weakly connected components: label[v] = smallest vertex id of the
 * component of v in the graph with edge directions ignored.  Host arrays:
 * label[n].  Optional: *n_components, *loop_seconds (the search alone, not
 * the transpose it builds first). */
int pro_wcc(int32_t n, int64_t m, const int32_t* row_ptr, const int32_t* col_idx, int32_t* label,
            int32_t* n_components, double* loop_seconds);

#ifdef __cplusplus
}
#endif

#endif
