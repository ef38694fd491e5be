// pr_plan_create / pr_plan_destroy and plan introspection.
//
// One-time work per graph: inverse out-degrees (the per-vertex ratio
// x[u]/outdeg[u] is then one multiply; Meerkat's PageRank section caches the
// ratio for the same reason, and the "gpu-graph-study" T3 tier precomputes
// 1/deg), and the in-rows split into degree buckets on the device.  The
// buckets are a stable partition of the row ids by bucket number, done with
// the same radix pass as the transpose, so each bucket lists its rows in
// ascending id order.
#include <cstdlib>
#include <cstring>

#include "plan.hpp"
#include "radix.hpp"

namespace pr {

namespace {

struct PlanWs {
    float* inv_out;
    int32_t* rows;
    float* contrib0;
    float* contrib1;
    float* partials;
    RunState* state;
    unsigned long long* stats;  // [2 * kNumBuckets]: rows, edges
    uint32_t* hist;
    uint32_t* scanned;
    uint32_t* error;
    void* scan_ws;
    size_t bytes;
};

PlanWs carve(void* base, int32_t n) {
    PlanWs w{};
    Carver c(base);
    const int64_t T = radix_tiles(n);
    w.inv_out = c.take<float>((size_t)n);
    w.rows = c.take<int32_t>((size_t)n);
    w.contrib0 = c.take<float>((size_t)n);
    w.contrib1 = c.take<float>((size_t)n);
    w.partials = c.take<float>((size_t)3 * kMaxPartials);
    w.state = c.take<RunState>(1);
    w.stats = c.take<unsigned long long>(2 * kNumBuckets);
    w.hist = c.take<uint32_t>((size_t)(kRadixDigits * T));
    w.scanned = c.take<uint32_t>((size_t)(kRadixDigits * T + 1));
    w.error = c.take<uint32_t>(1);
    w.scan_ws = c.base ? c.base + c.used : nullptr;
    c.used += align_up(scan_workspace_bytes(kRadixDigits * T));
    w.bytes = c.used;
    return w;
}

// inv_out[u] = 1/outdeg[u], or 0 when u has no out-edge (0 doubles as the
// dangling flag).  With `validate`, also checks both row-pointer arrays.
__global__ __launch_bounds__(kBlock) void k_inv_out(const int32_t* __restrict__ out_rp,
                                                    const int32_t* __restrict__ in_rp, int32_t n,
                                                    int64_t nnz, int validate,
                                                    float* __restrict__ inv_out,
                                                    uint32_t* __restrict__ err) {
    for (int64_t u = blockIdx.x * (int64_t)kBlock + threadIdx.x; u <= n;
         u += (int64_t)gridDim.x * kBlock) {
        if (u < n) {
            int32_t deg = out_rp[u + 1] - out_rp[u];
            inv_out[u] = deg > 0 ? 1.0f / (float)deg : 0.0f;
        }
        if (validate) {
            bool bad = false;
            if (u == 0 && (out_rp[0] != 0 || in_rp[0] != 0)) bad = true;
            if (u == n && ((int64_t)out_rp[n] != nnz || (int64_t)in_rp[n] != nnz)) bad = true;
            if (u < n && (out_rp[u + 1] < out_rp[u] || in_rp[u + 1] < in_rp[u])) bad = true;
            if (bad) *err = 1u;
        }
    }
}

__global__ __launch_bounds__(kBlock) void k_check_cols(const int32_t* __restrict__ ci, int64_t nnz,
                                                       int32_t n, uint32_t* __restrict__ err) {
    for (int64_t i = blockIdx.x * (int64_t)kBlock + threadIdx.x; i < nnz;
         i += (int64_t)gridDim.x * kBlock)
        if ((uint32_t)ci[i] >= (uint32_t)n) *err = 1u;
}

// Rows and edges per bucket.
__global__ __launch_bounds__(kBlock) void k_bucket_stats(RadixIn in,
                                                         unsigned long long* __restrict__ stats) {
    __shared__ unsigned long long s[2 * kNumBuckets];
    if (threadIdx.x < 2 * kNumBuckets) s[threadIdx.x] = 0;
    __syncthreads();
    for (int64_t v = blockIdx.x * (int64_t)kBlock + threadIdx.x; v < in.count;
         v += (int64_t)gridDim.x * kBlock) {
        int32_t b = radix_key<kFromRowLengths>(in, v);
        int32_t len = in.row_ptr[v + 1] - in.row_ptr[v];
        atomicAdd(&s[b], 1ull);
        atomicAdd(&s[kNumBuckets + b], (unsigned long long)(len > 0 ? len : 0));
    }
    __syncthreads();
    if (threadIdx.x < 2 * kNumBuckets && s[threadIdx.x])
        atomicAdd(&stats[threadIdx.x], s[threadIdx.x]);
}

unsigned grid_for(int64_t items, int64_t cap = 4096) {
    int64_t b = ceil_div(items > 0 ? items : 1, kBlock);
    return (unsigned)(b < cap ? b : cap);
}

// Bucket lower bounds; PR_BUCKET_MIN="0,5,17,65,4097" overrides them (for
// tuning sweeps).  Must start at 0 and increase.
void bucket_bounds(int32_t out[kNumBuckets]) {
    std::memcpy(out, kDefaultBucketMin, sizeof(kDefaultBucketMin));
    const char* env = std::getenv("PR_BUCKET_MIN");
    if (!env) return;
    int32_t tmp[kNumBuckets];
    const char* p = env;
    for (int b = 0; b < kNumBuckets; ++b) {
        char* end = nullptr;
        long v = std::strtol(p, &end, 10);
        if (end == p) return;
        tmp[b] = (int32_t)v;
        p = (*end == ',') ? end + 1 : end;
    }
    if (tmp[0] != 0) return;
    for (int b = 1; b < kNumBuckets; ++b)
        if (tmp[b] < tmp[b - 1]) return;
    std::memcpy(out, tmp, sizeof(tmp));
}

int64_t blocks_cap() {
    const char* env = std::getenv("PR_MAX_BLOCKS_PER_BUCKET");
    if (env) {
        long v = std::strtol(env, nullptr, 10);
        if (v >= 1 && v <= kMaxBlocksPerBucket) return v;
    }
    return kMaxBlocksPerBucket;
}

}  // namespace

}  // namespace pr

using namespace pr;

extern "C" size_t pr_plan_workspace_bytes(int32_t n, int64_t nnz) {
    if (n < 1 || nnz < 0 || nnz > INT32_MAX) return 0;
    return carve(nullptr, n).bytes;
}

extern "C" int pr_plan_create(pr_plan** plan_out, int32_t n, int64_t nnz, const int32_t* out_rp,
                              const int32_t* in_rp, const int32_t* in_ci, void* ws,
                              size_t ws_bytes, uint32_t flags, void* stream_v) {
    if (!plan_out) return fail(PR_ERR_ARG, "plan_out is null");
    *plan_out = nullptr;
    if (n < 1) return fail(PR_ERR_ARG, "n must be >= 1 (got %d)", n);
    if (nnz < 0 || nnz > INT32_MAX)
        return fail(PR_ERR_ARG, "nnz must be in [0, INT32_MAX] (got %lld)", (long long)nnz);
    if (flags & ~PR_VALIDATE) return fail(PR_ERR_ARG, "unknown flags 0x%x", flags);
    if (!out_rp || !in_rp || !ws || (nnz > 0 && !in_ci)) return fail(PR_ERR_ARG, "null pointer argument");
    PlanWs w = carve(ws, n);
    if (ws_bytes < w.bytes || (reinterpret_cast<uintptr_t>(ws) & 255u))
        return fail(PR_ERR_WORKSPACE, "plan workspace needs %zu bytes at 256-byte alignment (got %zu)",
                    w.bytes, ws_bytes);
    hipStream_t stream = as_stream(stream_v);
    const bool validate = flags & PR_VALIDATE;

    PR_TRY(fill_u32(w.error, 0u, 1, stream));
    PR_TRY(fill_u32(reinterpret_cast<uint32_t*>(w.stats), 0u, 4 * kNumBuckets, stream));
    PR_TRY(fill_u32(reinterpret_cast<uint32_t*>(w.state), 0u, sizeof(RunState) / 4, stream));
    k_inv_out<<<grid_for((int64_t)n + 1), kBlock, 0, stream>>>(out_rp, in_rp, n, nnz, validate ? 1 : 0,
                                                               w.inv_out, w.error);
    PR_LAUNCHED("inv_out");
    if (validate) {
        if (nnz > 0) {
            k_check_cols<<<grid_for(nnz), kBlock, 0, stream>>>(in_ci, nnz, n, w.error);
            PR_LAUNCHED("check cols");
        }
        PR_TRY(read_error_word(w.error, stream, "pr_plan_create"));
    }

    // Stable partition of row ids by bucket (one radix pass, keys computed
    // from the in-row lengths).
    RadixIn in{};
    in.count = n;
    in.n = n;
    in.row_ptr = in_rp;
    in.n_buckets = kNumBuckets;
    in.error = w.error;
    int32_t bmin[kNumBuckets];
    bucket_bounds(bmin);
    for (int b = 0; b < kNumBuckets; ++b) in.bucket_min[b] = bmin[b];
    const int64_t T = radix_tiles(n);
    k_radix_hist<kFromRowLengths><<<dim3((unsigned)T), kBlock, 0, stream>>>(in, 0, T, w.hist, nullptr);
    PR_LAUNCHED("bucket histogram");
    PR_TRY(scan_exclusive(w.hist, w.scanned, kRadixDigits * T, w.scan_ws, stream));
    k_radix_scatter<kFromRowLengths, true><<<dim3((unsigned)T), kBlock, 0, stream>>>(
        in, 0, T, w.scanned, nullptr, w.rows);
    PR_LAUNCHED("bucket scatter");
    k_bucket_stats<<<grid_for(n, 1024), kBlock, 0, stream>>>(in, w.stats);
    PR_LAUNCHED("bucket stats");

    unsigned long long stats[2 * kNumBuckets];
    PR_HIP_TRY(hipMemcpyAsync(stats, w.stats, sizeof stats, hipMemcpyDeviceToHost, stream));
    PR_HIP_TRY(hipStreamSynchronize(stream));

    pr_plan* p = static_cast<pr_plan*>(std::calloc(1, sizeof(pr_plan)));
    if (!p) return fail(PR_ERR_ARG, "out of host memory");
    PR_HIP_TRY(hipGetDevice(&p->device));
    p->n = n;
    p->nnz = nnz;
    p->out_rp = out_rp;
    p->in_rp = in_rp;
    p->in_ci = in_ci;
    p->inv_out = w.inv_out;
    p->rows = w.rows;
    p->contrib[0] = w.contrib0;
    p->contrib[1] = w.contrib1;
    p->partials = w.partials;
    p->state = w.state;

    // Launch shape: hub buckets first so the longest rows start earliest.
    const int64_t cap = blocks_cap();
    int64_t row0 = 0;
    int32_t row_begin[kNumBuckets];
    for (int b = 0; b < kNumBuckets; ++b) {
        p->bucket_min[b] = bmin[b];
        p->bucket_rows[b] = (int64_t)stats[b];
        p->bucket_edges[b] = (int64_t)stats[kNumBuckets + b];
        row_begin[b] = (int32_t)row0;
        row0 += (int64_t)stats[b];
    }
    int32_t block = 0;
    for (int b = kNumBuckets - 1; b >= 0; --b) {
        const int64_t rows_per_block = kBlock / kBucketGroup[b];
        int64_t blocks = ceil_div(p->bucket_rows[b], rows_per_block);
        if (blocks > cap) blocks = cap;
        p->launch[b].row_begin = row_begin[b];
        p->launch[b].row_end = row_begin[b] + (int32_t)p->bucket_rows[b];
        p->launch[b].block_begin = block;
        p->launch[b].blocks = (int32_t)blocks;
        block += (int32_t)blocks;
    }
    p->iter_blocks = block > 0 ? block : 1;
    {
        int64_t ib = ceil_div(n, kBlock);
        p->init_blocks = (int32_t)(ib < 1024 ? ib : 1024);
    }

    hipError_t e = hipEventCreate(&p->ev_begin);
    if (e == hipSuccess) e = hipEventCreate(&p->ev_end);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->chunk_ev[0], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->chunk_ev[1], hipEventDisableTiming);
    if (e == hipSuccess)
        e = hipHostMalloc(reinterpret_cast<void**>(&p->host_status), 2 * sizeof(RunStatus),
                          hipHostMallocDefault);
    if (e != hipSuccess) {
        int rc = fail(PR_ERR_HIP, "plan events / pinned status: %s", hipGetErrorString(e));
        pr_plan_destroy(p);
        return rc;
    }
    *plan_out = p;
    return PR_OK;
}

extern "C" int pr_plan_destroy(pr_plan* p) {
    if (!p) return PR_OK;
    if (p->ev_begin) (void)hipEventDestroy(p->ev_begin);
    if (p->ev_end) (void)hipEventDestroy(p->ev_end);
    if (p->chunk_ev[0]) (void)hipEventDestroy(p->chunk_ev[0]);
    if (p->chunk_ev[1]) (void)hipEventDestroy(p->chunk_ev[1]);
    if (p->host_status) (void)hipHostFree(p->host_status);
    std::free(p);
    return PR_OK;
}

extern "C" int pr_plan_num_buckets(void) { return kNumBuckets; }

extern "C" int pr_plan_buckets(const pr_plan* p, int32_t* min_len, int32_t* rows, int64_t* edges) {
    if (!p) return fail(PR_ERR_ARG, "plan is null");
    for (int b = 0; b < kNumBuckets; ++b) {
        if (min_len) min_len[b] = p->bucket_min[b];
        if (rows) rows[b] = (int32_t)p->bucket_rows[b];
        if (edges) edges[b] = p->bucket_edges[b];
    }
    return PR_OK;
}
