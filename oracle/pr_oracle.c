/*
 * PageRank power-iteration oracle -- TEST INFRASTRUCTURE ONLY (see
 * pr_oracle.h for the sources it follows and who may call it).
 *
 * Deliberately plain: sequential loops, double precision, one division per
 * edge exactly as the update is written, no blocking, no fusion.
 */
#define _POSIX_C_SOURCE 199309L
#include "pr_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#define PRO_OK 0
#define PRO_ERR_ARG -1
#define PRO_ERR_CSR -2
#define PRO_ERR_NOMEM -3

/* A CSR is well formed when row_ptr starts at 0, never decreases, ends at m,
 * and every column lies in [0, n). */
static int check_csr(int32_t n, int64_t m, const int32_t* rp, const int32_t* ci) {
    if (n < 1 || m < 0 || m > INT32_MAX || !rp || (m > 0 && !ci)) return PRO_ERR_ARG;
    if (rp[0] != 0 || (int64_t)rp[n] != m) return PRO_ERR_CSR;
    for (int32_t u = 0; u < n; ++u)
        if (rp[u + 1] < rp[u]) return PRO_ERR_CSR;
    for (int64_t e = 0; e < m; ++e)
        if (ci[e] < 0 || ci[e] >= n) return PRO_ERR_CSR;
    return PRO_OK;
}

/* Day 40, "One iteration, three shapes of work": the host turns out-edges into
 * in-edges once with a counting sort -- a histogram of destinations, a prefix
 * sum over it, and a scatter. */
int pro_transpose(int32_t n, int64_t m, const int32_t* out_rp, const int32_t* out_ci,
                  int32_t* in_rp, int32_t* in_ci) {
    int rc = check_csr(n, m, out_rp, out_ci);
    if (rc) return rc;
    if (!in_rp || (m > 0 && !in_ci)) return PRO_ERR_ARG;

    /* histogram: in-degree of every vertex */
    int64_t* count = (int64_t*)calloc((size_t)n, sizeof(int64_t));
    if (!count) return PRO_ERR_NOMEM;
    for (int64_t e = 0; e < m; ++e) count[out_ci[e]] += 1;

    /* exclusive prefix sum -> in_row_ptr */
    int64_t run = 0;
    for (int32_t v = 0; v < n; ++v) {
        in_rp[v] = (int32_t)run;
        run += count[v];
    }
    in_rp[n] = (int32_t)run;

    /* scatter: sources in increasing order, so each in-row comes out sorted */
    for (int32_t v = 0; v < n; ++v) count[v] = in_rp[v];
    for (int32_t u = 0; u < n; ++u)
        for (int32_t e = out_rp[u]; e < out_rp[u + 1]; ++e) {
            int32_t v = out_ci[e];
            in_ci[count[v]] = u;
            count[v] += 1;
        }
    free(count);
    return PRO_OK;
}

static double now_seconds(void) {
    struct timespec t;
    clock_gettime(CLOCK_MONOTONIC, &t);
    return (double)t.tv_sec + 1e-9 * (double)t.tv_nsec;
}

/* Day 40 update, iterated (Meerkat's PageRank section gives the same loop:
 * start from 1/n, build iteration i from iteration i-1, stop on the L1 delta
 * or after max_iter super-steps). */
int pro_pagerank(int32_t n, int64_t m, const int32_t* out_rp, const int32_t* out_ci, double d,
                 double tol, int32_t max_iter, const double* x0, uint32_t flags, double* x,
                 double* l1_trace, double* sum_trace, double* dmass_trace, int32_t* iterations,
                 double* loop_seconds) {
    int rc = check_csr(n, m, out_rp, out_ci);
    if (rc) return rc;
    if (!x || !iterations || max_iter < 1 || !(d >= 0.0 && d <= 1.0)) return PRO_ERR_ARG;

    int32_t* in_rp = (int32_t*)malloc(sizeof(int32_t) * ((size_t)n + 1));
    int32_t* in_ci = (int32_t*)malloc(sizeof(int32_t) * (size_t)(m > 0 ? m : 1));
    int32_t* outdeg = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    double* xn = (double*)malloc(sizeof(double) * (size_t)n);
    if (!in_rp || !in_ci || !outdeg || !xn) {
        free(in_rp); free(in_ci); free(outdeg); free(xn);
        return PRO_ERR_NOMEM;
    }
    pro_transpose(n, m, out_rp, out_ci, in_rp, in_ci);
    for (int32_t u = 0; u < n; ++u) outdeg[u] = out_rp[u + 1] - out_rp[u];

    /* Meerkat, PageRank section: the static start is 1/n for every vertex. */
    for (int32_t v = 0; v < n; ++v) x[v] = x0 ? x0[v] : 1.0 / (double)n;

    const double t0 = now_seconds();
    int32_t t = 0;
    while (t < max_iter) {
        t += 1;
        /* Dangling mass D: rank held by out-degree-0 vertices in the vector
         * this iteration starts from (Day 40 reduces x before the combine;
         * Meerkat's teleport term uses iteration i-1). */
        double D = 0.0;
        if (!(flags & PRO_DROP_DANGLING))
            for (int32_t u = 0; u < n; ++u)
                if (outdeg[u] == 0) D += x[u];

        /* x'[v] = (1-d)/n + d * (sum over in-neighbours u of x[u]/outdeg[u] + D/n) */
        for (int32_t v = 0; v < n; ++v) {
            double s = 0.0;
            for (int32_t k = in_rp[v]; k < in_rp[v + 1]; ++k) {
                int32_t u = in_ci[k];
                s += x[u] / (double)outdeg[u];
            }
            xn[v] = (1.0 - d) / (double)n + d * (s + D / (double)n);
        }

        /* L1 distance between successive vectors, then the new vector. */
        double l1 = 0.0, sum = 0.0;
        for (int32_t v = 0; v < n; ++v) {
            l1 += fabs(xn[v] - x[v]);
            x[v] = xn[v];
            sum += x[v];
        }
        if (l1_trace) l1_trace[t - 1] = l1;
        if (sum_trace) sum_trace[t - 1] = sum;
        if (dmass_trace) dmass_trace[t - 1] = D;
        if (tol > 0.0 && l1 < tol) break;
    }
    if (loop_seconds) *loop_seconds = now_seconds() - t0;
    *iterations = t;
    free(in_rp); free(in_ci); free(outdeg); free(xn);
    return PRO_OK;
}

/* "A Pedagogical Introduction to Porting a Conjugate Gradient Solver to CUDA":
 * the sparse product of its CG loop, on the flattened CSR arrays -- for every
 * row, start from zero and add value times gathered x over the row's entries
 * in stored order. */
int pro_spmv(int32_t n_rows, int32_t n_cols, int64_t nnz, const int32_t* rp, const int32_t* ci,
             const double* vals, const double* x, double* y, double* loop_seconds) {
    if (n_rows < 0 || n_cols < 0 || nnz < 0 || nnz > INT32_MAX || !rp) return PRO_ERR_ARG;
    if (nnz > 0 && (!ci || !vals)) return PRO_ERR_ARG;
    if ((n_rows > 0 && !y) || (n_cols > 0 && !x)) return PRO_ERR_ARG;
    if (rp[0] != 0 || (int64_t)rp[n_rows] != nnz) return PRO_ERR_CSR;
    for (int32_t i = 0; i < n_rows; ++i)
        if (rp[i + 1] < rp[i]) return PRO_ERR_CSR;
    for (int64_t j = 0; j < nnz; ++j)
        if (ci[j] < 0 || ci[j] >= n_cols) return PRO_ERR_CSR;

    const double t0 = now_seconds();
    for (int32_t i = 0; i < n_rows; ++i) {
        double sum = 0.0;
        for (int32_t j = rp[i]; j < rp[i + 1]; ++j) sum += vals[j] * x[ci[j]];
        y[i] = sum;
    }
    if (loop_seconds) *loop_seconds = now_seconds() - t0;
    return PRO_OK;
}

/* "gpu-graph-study", section "Traversal (BFS / WCC)": breadth-first search
 * from one source over the out-edges.  level[v] = number of edges on a
 * shortest directed path source -> v, -1 when no path exists.  A plain FIFO
 * queue: every vertex enters it once, when it is first reached, with the
 * level of the vertex that reached it plus one. */
int pro_bfs(int32_t n, int64_t m, const int32_t* rp, const int32_t* ci, int32_t source,
            int32_t* level, int32_t* depth, int64_t* edges_scanned, double* loop_seconds) {
    int rc = check_csr(n, m, rp, ci);
    if (rc) return rc;
    if (!level || source < 0 || source >= n) return PRO_ERR_ARG;
    int32_t* queue = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    if (!queue) return PRO_ERR_NOMEM;
    const double t0 = now_seconds();
    for (int32_t v = 0; v < n; ++v) level[v] = -1;
    level[source] = 0;
    int64_t head = 0, tail = 0, scanned = 0;
    queue[tail++] = source;
    int32_t deepest = 0;
    while (head < tail) {
        const int32_t u = queue[head++];
        if (level[u] > deepest) deepest = level[u];
        for (int32_t e = rp[u]; e < rp[u + 1]; ++e) {
            const int32_t v = ci[e];
            scanned += 1;
            if (level[v] == -1) {
                level[v] = level[u] + 1;
                queue[tail++] = v;
            }
        }
    }
    if (loop_seconds) *loop_seconds = now_seconds() - t0;
    if (depth) *depth = deepest;
    if (edges_scanned) *edges_scanned = scanned;
    free(queue);
    return PRO_OK;
}

/* "gpu-graph-study", section "Traversal (BFS / WCC)": weakly connected
 * components, the components of the graph with edge directions ignored.
 * label[v] = the smallest vertex id in v's component (the value min-label
 * propagation settles on).  Computed by breadth-first search over the
 * undirected view (out-edges plus in-edges), starting a new search from each
 * vertex, in increasing id order, that no earlier search reached: that
 * vertex is the smallest of its component. */
int pro_wcc(int32_t n, int64_t m, const int32_t* rp, const int32_t* ci, int32_t* label,
            int32_t* n_components, double* loop_seconds) {
    int rc = check_csr(n, m, rp, ci);
    if (rc) return rc;
    if (!label) return PRO_ERR_ARG;
    int32_t* in_rp = (int32_t*)malloc(sizeof(int32_t) * ((size_t)n + 1));
    int32_t* in_ci = (int32_t*)malloc(sizeof(int32_t) * (size_t)(m > 0 ? m : 1));
    int32_t* queue = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    if (!in_rp || !in_ci || !queue) {
        free(in_rp); free(in_ci); free(queue);
        return PRO_ERR_NOMEM;
    }
    pro_transpose(n, m, rp, ci, in_rp, in_ci);
    const double t0 = now_seconds();
    for (int32_t v = 0; v < n; ++v) label[v] = -1;
    int32_t comps = 0;
    for (int32_t s = 0; s < n; ++s) {
        if (label[s] != -1) continue;
        comps += 1;
        int64_t head = 0, tail = 0;
        label[s] = s;
        queue[tail++] = s;
        while (head < tail) {
            const int32_t u = queue[head++];
            for (int32_t e = rp[u]; e < rp[u + 1]; ++e)  /* u -> v */
                if (label[ci[e]] == -1) {
                    label[ci[e]] = s;
                    queue[tail++] = ci[e];
                }
            for (int32_t e = in_rp[u]; e < in_rp[u + 1]; ++e)  /* w -> u */
                if (label[in_ci[e]] == -1) {
                    label[in_ci[e]] = s;
                    queue[tail++] = in_ci[e];
                }
        }
    }
    if (loop_seconds) *loop_seconds = now_seconds() - t0;
    if (n_components) *n_components = comps;
    free(in_rp); free(in_ci); free(queue);
    return PRO_OK;
}
