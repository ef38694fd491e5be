/*
 * Seeded synthetic graph generators (out-edge CSR, int32).
 *
 * This module produces INPUTS only: it holds none of PageRank's arithmetic
 * and no transpose.  Both the CPU oracle's tests and the GPU path's tests and
 * benchmark read their graphs from here.
 *
 * Every generator returns an out-edge CSR whose rows are sorted ascending by
 * target id, with no duplicate (u, v) pairs and no self-loops, which is the
 * cleanup the synthetic workloads ask for.
 *
 * Randomness is counter-based: draw k of stream `seed` is
 *     splitmix64_mix(splitmix64_mix(seed) + (k + 1) * 0x9E3779B97F4A7C15)
 * i.e. the output function of Steele, Lea and Flood's SplitMix64 ("Fast
 * splittable pseudorandom number generators", OOPSLA 2014) evaluated at
 * counter k.  Because a draw depends only on (seed, k), generation can be
 * split over threads and still give one graph per seed.
 *
 * Generators:
 *   gg_rmat       R-MAT recursive quadrant choice (Chakrabarti, Zhan and
 *                 Faloutsos, SDM 2004) with Graph500 parameters, one uniform
 *                 draw per edge per bit level, no per-level noise.
 *   gg_stencil27  27-point stencil on an nx*ny*nz grid, every point linked to
 *                 each in-grid point at Chebyshev distance 1.
 *   gg_citation   citation-like digraph: a seeded uniform sample of papers
 *                 cite nothing; every other paper cites a geometric number
 *                 (support 1, 2, ...) of distinct earlier-or-later papers,
 *                 each drawn with probability proportional to (in-degree+1).
 *
 * Memory: generators malloc their outputs; the caller copies them and hands
 * them back to gg_free().
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GG_OK 0
#define GG_ERR_ARG -1
#define GG_ERR_NOMEM -2

static const uint64_t GOLDEN = 0x9E3779B97F4A7C15ull;

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Draw k of stream `key` (key = mix64(seed)). */
static inline uint64_t draw_u64(uint64_t key, uint64_t k) {
    return mix64(key + (k + 1) * GOLDEN);
}

/* Uniform double in [0, 1) from the top 53 bits. */
static inline double draw_unif(uint64_t key, uint64_t k) {
    return (double)(draw_u64(key, k) >> 11) * (1.0 / 9007199254740992.0);
}

uint64_t gg_draw_u64(uint64_t seed, uint64_t k) { return draw_u64(mix64(seed), k); }
double gg_draw_unif(uint64_t seed, uint64_t k) { return draw_unif(mix64(seed), k); }

void gg_free(void* p) { free(p); }

int gg_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}


static int cmp_i32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

static void sort_row(int32_t* r, int64_t len) {
    if (len < 24) {
        for (int64_t i = 1; i < len; ++i) {
            int32_t v = r[i];
            int64_t j = i - 1;
            while (j >= 0 && r[j] > v) { r[j + 1] = r[j]; --j; }
            r[j + 1] = v;
        }
    } else {
        qsort(r, (size_t)len, sizeof(int32_t), cmp_i32);
    }
}

/* Sort every row, drop duplicates (self-loops were never stored), and compact
 * into freshly allocated arrays.  raw_rp[n+1] / raw_ci are consumed (freed). */
static int finish_csr(int32_t n, int64_t* raw_rp, int32_t* raw_ci, int32_t** rp_out,
                      int32_t** ci_out, int64_t* m_out) {
    int64_t* len = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
    if (!len) return GG_ERR_NOMEM;
#pragma omp parallel for schedule(dynamic, 1024)
    for (int32_t u = 0; u < n; ++u) {
        int32_t* r = raw_ci + raw_rp[u];
        int64_t l = raw_rp[u + 1] - raw_rp[u];
        sort_row(r, l);
        int64_t w = 0;
        for (int64_t i = 0; i < l; ++i)
            if (w == 0 || r[i] != r[w - 1]) r[w++] = r[i];
        len[u] = w;
    }
    int32_t* rp = (int32_t*)malloc(sizeof(int32_t) * ((size_t)n + 1));
    int64_t total = 0;
    for (int32_t u = 0; u < n; ++u) total += len[u];
    if (!rp || total > INT32_MAX) { free(rp); free(len); return rp ? GG_ERR_ARG : GG_ERR_NOMEM; }
    int32_t* ci = (int32_t*)malloc(sizeof(int32_t) * (size_t)(total > 0 ? total : 1));
    if (!ci) { free(rp); free(len); return GG_ERR_NOMEM; }
    int64_t acc = 0;
    for (int32_t u = 0; u < n; ++u) { rp[u] = (int32_t)acc; acc += len[u]; }
    rp[n] = (int32_t)acc;
#pragma omp parallel for schedule(dynamic, 1024)
    for (int32_t u = 0; u < n; ++u)
        memcpy(ci + rp[u], raw_ci + raw_rp[u], sizeof(int32_t) * (size_t)len[u]);
    free(len);
    free(raw_rp);
    free(raw_ci);
    *rp_out = rp;
    *ci_out = ci;
    *m_out = total;
    return GG_OK;
}

/* One R-MAT edge: for each bit level (most significant first) pick a quadrant
 * with probabilities a (u=0,v=0), b (u=0,v=1), c (u=1,v=0), 1-a-b-c (u=1,v=1).
 * The 53-bit uniform integer r is compared against the cumulative thresholds
 * ceil(p * 2^53), which is the same test as comparing r * 2^-53 with p. */
static inline void rmat_edge(uint64_t key, int scale, uint64_t e, uint64_t A, uint64_t AB,
                             uint64_t ABC, int32_t* u_out, int32_t* v_out) {
    uint32_t u = 0, v = 0;
    uint64_t k = e * (uint64_t)scale;
    for (int l = 0; l < scale; ++l) {
        uint64_t r = draw_u64(key, k + (uint64_t)l) >> 11;
        uint32_t ub = (uint32_t)(r >= AB);
        uint32_t vb = (uint32_t)(((r >= A) & (r < AB)) | (r >= ABC));
        u = (u << 1) | ub;
        v = (v << 1) | vb;
    }
    *u_out = (int32_t)u;
    *v_out = (int32_t)v;
}

static uint64_t threshold53(double p) {
    double t = ceil(p * 9007199254740992.0);
    return t >= 9007199254740992.0 ? (1ull << 53) : (uint64_t)t;
}

int gg_rmat(int scale, int64_t n_draws, double a, double b, double c, uint64_t seed,
            int32_t** rp_out, int32_t** ci_out, int64_t* m_out) {
    if (scale < 1 || scale > 30 || n_draws < 0 || a < 0 || b < 0 || c < 0 || a + b + c > 1.0)
        return GG_ERR_ARG;
    const int32_t n = (int32_t)1 << scale;
    const uint64_t key = mix64(seed);
    const uint64_t A = threshold53(a), AB = threshold53(a + b), ABC = threshold53(a + b + c);
    int nt = gg_num_threads();
    if ((int64_t)nt > n_draws / 4096 + 1) nt = (int)(n_draws / 4096 + 1);
    /* Per-thread source histograms: thread t owns draws [lo(t), lo(t+1)), so
     * no counter is shared and edge placement before sorting is fixed. */
    int32_t* cnt = (int32_t*)calloc((size_t)nt * (size_t)n, sizeof(int32_t));
    int64_t* rp = (int64_t*)malloc(sizeof(int64_t) * ((size_t)n + 1));
    if (!cnt || !rp) { free(cnt); free(rp); return GG_ERR_NOMEM; }
#pragma omp parallel num_threads(nt)
    {
        int t = 0;
#ifdef _OPENMP
        t = omp_get_thread_num();
#endif
        int64_t lo = n_draws * t / nt, hi = n_draws * (t + 1) / nt;
        int32_t* my = cnt + (size_t)t * (size_t)n;
        for (int64_t e = lo; e < hi; ++e) {
            int32_t u, v;
            rmat_edge(key, scale, (uint64_t)e, A, AB, ABC, &u, &v);
            if (u != v) my[u]++;
        }
    }
    /* Row starts, then each thread's cursor inside every row. */
    int64_t acc = 0;
    for (int32_t u = 0; u < n; ++u) {
        rp[u] = acc;
        for (int t = 0; t < nt; ++t) {
            int32_t k = cnt[(size_t)t * (size_t)n + u];
            cnt[(size_t)t * (size_t)n + u] = (int32_t)(acc - rp[u]);
            acc += k;
        }
    }
    rp[n] = acc;
    const int64_t raw_m = acc;
    int32_t* raw_ci = (int32_t*)malloc(sizeof(int32_t) * (size_t)(raw_m > 0 ? raw_m : 1));
    if (!raw_ci) { free(cnt); free(rp); return GG_ERR_NOMEM; }
#pragma omp parallel num_threads(nt)
    {
        int t = 0;
#ifdef _OPENMP
        t = omp_get_thread_num();
#endif
        int64_t lo = n_draws * t / nt, hi = n_draws * (t + 1) / nt;
        int32_t* my = cnt + (size_t)t * (size_t)n;
        for (int64_t e = lo; e < hi; ++e) {
            int32_t u, v;
            rmat_edge(key, scale, (uint64_t)e, A, AB, ABC, &u, &v);
            if (u != v) raw_ci[rp[u] + my[u]++] = v;
        }
    }
    free(cnt);
    return finish_csr(n, rp, raw_ci, rp_out, ci_out, m_out);
}

int gg_stencil27(int32_t nx, int32_t ny, int32_t nz, int32_t** rp_out, int32_t** ci_out,
                 int64_t* m_out) {
    if (nx < 1 || ny < 1 || nz < 1) return GG_ERR_ARG;
    const int64_t n64 = (int64_t)nx * ny * nz;
    if (n64 > INT32_MAX || n64 * 26 > INT32_MAX) return GG_ERR_ARG;
    const int32_t n = (int32_t)n64;
    int32_t* rp = (int32_t*)malloc(sizeof(int32_t) * ((size_t)n + 1));
    if (!rp) return GG_ERR_NOMEM;
    /* First pass: neighbour counts (closed form per axis). */
    rp[0] = 0;
    int64_t acc = 0;
    for (int32_t z = 0; z < nz; ++z)
        for (int32_t y = 0; y < ny; ++y)
            for (int32_t x = 0; x < nx; ++x) {
                int64_t cx = 1 + (x > 0) + (x < nx - 1);
                int64_t cy = 1 + (y > 0) + (y < ny - 1);
                int64_t cz = 1 + (z > 0) + (z < nz - 1);
                acc += cx * cy * cz - 1;
                rp[x + (int64_t)nx * (y + (int64_t)ny * z) + 1] = (int32_t)acc;
            }
    int32_t* ci = (int32_t*)malloc(sizeof(int32_t) * (size_t)(acc > 0 ? acc : 1));
    if (!ci) { free(rp); return GG_ERR_NOMEM; }
#pragma omp parallel for schedule(static)
    for (int32_t z = 0; z < nz; ++z)
        for (int32_t y = 0; y < ny; ++y)
            for (int32_t x = 0; x < nx; ++x) {
                int64_t id = x + (int64_t)nx * (y + (int64_t)ny * z);
                int64_t w = rp[id];
                /* dz, dy, dx ascending gives ascending neighbour ids. */
                for (int dz = -1; dz <= 1; ++dz)
                    for (int dy = -1; dy <= 1; ++dy)
                        for (int dx = -1; dx <= 1; ++dx) {
                            if (!dx && !dy && !dz) continue;
                            int32_t X = x + dx, Y = y + dy, Z = z + dz;
                            if (X < 0 || X >= nx || Y < 0 || Y >= ny || Z < 0 || Z >= nz) continue;
                            ci[w++] = (int32_t)(X + (int64_t)nx * (Y + (int64_t)ny * Z));
                        }
            }
    *rp_out = rp;
    *ci_out = ci;
    *m_out = acc;
    return GG_OK;
}

int gg_citation(int32_t n, int32_t n_dangling, double mean_outdeg, uint64_t seed, int32_t** rp_out,
                int32_t** ci_out, int64_t* m_out) {
    if (n < 1 || n_dangling < 0 || n_dangling > n || !(mean_outdeg >= 1.0)) return GG_ERR_ARG;
    const uint64_t key = mix64(seed);
    uint64_t k = 0; /* running draw counter: this generator is sequential */

    /* Dangling papers: first n_dangling entries of a seeded partial
     * Fisher-Yates shuffle of 0..n-1. */
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    uint8_t* dangling = (uint8_t*)calloc((size_t)n, 1);
    int32_t* stamp = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    if (!perm || !dangling || !stamp) { free(perm); free(dangling); free(stamp); return GG_ERR_NOMEM; }
    for (int32_t i = 0; i < n; ++i) { perm[i] = i; stamp[i] = -1; }
    for (int32_t i = 0; i < n_dangling; ++i) {
        int32_t j = i + (int32_t)(draw_unif(key, k++) * (double)(n - i));
        if (j >= n) j = n - 1;
        int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
        dangling[perm[i]] = 1;
    }
    free(perm);

    /* The "bag" holds every paper once (the +1) plus one copy per citation it
     * has received, so a uniform pick from it is proportional to indeg+1. */
    size_t bag_cap = (size_t)n * 16 + 16, bag_len = (size_t)n;
    int32_t* bag = (int32_t*)malloc(sizeof(int32_t) * bag_cap);
    int64_t* rp64 = (int64_t*)malloc(sizeof(int64_t) * ((size_t)n + 1));
    size_t ci_cap = (size_t)n * 16 + 16, m = 0;
    int32_t* ci = (int32_t*)malloc(sizeof(int32_t) * ci_cap);
    if (!bag || !rp64 || !ci) { free(bag); free(rp64); free(ci); free(dangling); free(stamp); return GG_ERR_NOMEM; }
    for (int32_t i = 0; i < n; ++i) bag[i] = i;

    const double p = 1.0 / mean_outdeg;
    const double log_q = log1p(-p);
    rp64[0] = 0;
    for (int32_t u = 0; u < n; ++u) {
        int64_t deg = 0;
        if (!dangling[u] && n > 1) {
            /* Geometric on {1, 2, ...} with success probability p (mean 1/p),
             * by inversion: 1 + floor(log(1 - U) / log(1 - p)). */
            double uu = draw_unif(key, k++);
            double g = (p >= 1.0) ? 0.0 : floor(log1p(-uu) / log_q);
            deg = 1 + (int64_t)(g < (double)(n - 2) ? g : (double)(n - 2));
        }
        if (m + (size_t)deg > ci_cap) {
            ci_cap = (m + (size_t)deg) * 2;
            int32_t* t = (int32_t*)realloc(ci, sizeof(int32_t) * ci_cap);
            if (!t) { free(bag); free(rp64); free(ci); free(dangling); free(stamp); return GG_ERR_NOMEM; }
            ci = t;
        }
        int32_t* row = ci + m;
        stamp[u] = u;
        for (int64_t j = 0; j < deg; ++j) {
            int32_t v = -1;
            for (int tries = 0; tries < 256; ++tries) {
                size_t idx = (size_t)(draw_unif(key, k++) * (double)bag_len);
                if (idx >= bag_len) idx = bag_len - 1;
                int32_t c = bag[idx];
                if (stamp[c] != u) { v = c; break; }
            }
            if (v < 0) { /* deterministic fallback: lowest id not yet taken */
                for (int32_t c = 0; c < n; ++c)
                    if (stamp[c] != u) { v = c; break; }
            }
            stamp[v] = u;
            row[j] = v;
        }
        /* Citations of one paper raise in-degrees only after it is done. */
        if (bag_len + (size_t)deg > bag_cap) {
            bag_cap = (bag_len + (size_t)deg) * 2;
            int32_t* t = (int32_t*)realloc(bag, sizeof(int32_t) * bag_cap);
            if (!t) { free(bag); free(rp64); free(ci); free(dangling); free(stamp); return GG_ERR_NOMEM; }
            bag = t;
        }
        for (int64_t j = 0; j < deg; ++j) bag[bag_len++] = row[j];
        sort_row(row, deg);
        m += (size_t)deg;
        rp64[u + 1] = (int64_t)m;
    }
    free(bag);
    free(dangling);
    free(stamp);
    if (m > INT32_MAX) { free(rp64); free(ci); return GG_ERR_ARG; }
    int32_t* rp = (int32_t*)malloc(sizeof(int32_t) * ((size_t)n + 1));
    if (!rp) { free(rp64); free(ci); return GG_ERR_NOMEM; }
    for (int32_t i = 0; i <= n; ++i) rp[i] = (int32_t)rp64[i];
    free(rp64);
    *rp_out = rp;
    *ci_out = ci;
    *m_out = (int64_t)m;
    return GG_OK;
}


/* Raw R-MAT draws k0 .. k0+count-1 of stream `seed` (the same per-edge draw
 * as gg_rmat, self-loops included): the edges of a seeded insertion batch. */
int gg_rmat_edges(int scale, double a, double b, double c, uint64_t seed, int64_t k0,
                  int64_t count, int32_t* u_out, int32_t* v_out) {
    if (scale < 1 || scale > 30 || k0 < 0 || count < 0 || a < 0 || b < 0 || c < 0 ||
        a + b + c > 1.0)
        return GG_ERR_ARG;
    const uint64_t key = mix64(seed);
    const uint64_t A = threshold53(a), AB = threshold53(a + b), ABC = threshold53(a + b + c);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        rmat_edge(key, scale, (uint64_t)(k0 + i), A, AB, ABC, &u_out[i], &v_out[i]);
    return GG_OK;
}

/* The graph with every vertex v renamed perm[v] (perm a permutation of
 * [0, n)): row perm[u] holds perm[v] for every edge (u, v), sorted. */
int gg_relabel(int32_t n, const int32_t* rp, const int32_t* ci, const int32_t* perm,
               int32_t** rp_out, int32_t** ci_out, int64_t* m_out) {
    if (n < 1) return GG_ERR_ARG;
    int64_t* raw_rp = (int64_t*)malloc(sizeof(int64_t) * ((size_t)n + 1));
    int32_t* inv = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    const int64_t m = rp[n];
    int32_t* raw_ci = (int32_t*)malloc(sizeof(int32_t) * (size_t)(m > 0 ? m : 1));
    if (!raw_rp || !inv || !raw_ci) { free(raw_rp); free(inv); free(raw_ci); return GG_ERR_NOMEM; }
    for (int32_t u = 0; u < n; ++u) {
        if (perm[u] < 0 || perm[u] >= n) { free(raw_rp); free(inv); free(raw_ci); return GG_ERR_ARG; }
        inv[perm[u]] = u;
    }
    int64_t acc = 0;
    for (int32_t p = 0; p < n; ++p) {
        raw_rp[p] = acc;
        acc += rp[inv[p] + 1] - rp[inv[p]];
    }
    raw_rp[n] = acc;
#pragma omp parallel for schedule(dynamic, 1024)
    for (int32_t p = 0; p < n; ++p) {
        const int32_t u = inv[p];
        for (int64_t j = rp[u]; j < rp[u + 1]; ++j) raw_ci[raw_rp[p] + (j - rp[u])] = perm[ci[j]];
    }
    free(inv);
    return finish_csr(n, raw_rp, raw_ci, rp_out, ci_out, m_out);
}

/* The graph after an edge batch: the edges whose indices are listed in
 * del_idx (ascending, each in [0, m)) removed, then the n_ins edges
 * (ins_u[i], ins_v[i]) added; self-loops and edges already present are not
 * added twice.  Rows come out sorted. */
int gg_edit(int32_t n, const int32_t* rp, const int32_t* ci, int64_t n_del, const int64_t* del_idx,
            int64_t n_ins, const int32_t* ins_u, const int32_t* ins_v, int32_t** rp_out,
            int32_t** ci_out, int64_t* m_out) {
    if (n < 1 || n_del < 0 || n_ins < 0) return GG_ERR_ARG;
    const int64_t m = rp[n];
    for (int64_t i = 0; i < n_del; ++i)
        if (del_idx[i] < 0 || del_idx[i] >= m || (i > 0 && del_idx[i] <= del_idx[i - 1]))
            return GG_ERR_ARG;
    for (int64_t i = 0; i < n_ins; ++i)
        if (ins_u[i] < 0 || ins_u[i] >= n || ins_v[i] < 0 || ins_v[i] >= n) return GG_ERR_ARG;
    int64_t* raw_rp = (int64_t*)calloc((size_t)n + 1, sizeof(int64_t));
    int64_t* cur = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
    if (!raw_rp || !cur) { free(raw_rp); free(cur); return GG_ERR_NOMEM; }
    /* kept out-degrees plus inserted ones */
    int64_t d = 0;
    for (int32_t u = 0; u < n; ++u) {
        int64_t keep = rp[u + 1] - rp[u];
        while (d < n_del && del_idx[d] < rp[u + 1]) { --keep; ++d; }
        raw_rp[u + 1] = keep;
    }
    for (int64_t i = 0; i < n_ins; ++i)
        if (ins_u[i] != ins_v[i]) raw_rp[ins_u[i] + 1]++;
    for (int32_t u = 0; u < n; ++u) raw_rp[u + 1] += raw_rp[u];
    const int64_t raw_m = raw_rp[n];
    int32_t* raw_ci = (int32_t*)malloc(sizeof(int32_t) * (size_t)(raw_m > 0 ? raw_m : 1));
    if (!raw_ci) { free(raw_rp); free(cur); return GG_ERR_NOMEM; }
    d = 0;
    for (int32_t u = 0; u < n; ++u) {
        cur[u] = raw_rp[u];
        for (int64_t j = rp[u]; j < rp[u + 1]; ++j) {
            if (d < n_del && del_idx[d] == j) { ++d; continue; }
            raw_ci[cur[u]++] = ci[j];
        }
    }
    for (int64_t i = 0; i < n_ins; ++i)
        if (ins_u[i] != ins_v[i]) raw_ci[cur[ins_u[i]]++] = ins_v[i];
    free(cur);
    return finish_csr(n, raw_rp, raw_ci, rp_out, ci_out, m_out);
}
