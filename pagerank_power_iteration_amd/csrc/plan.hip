// pr_plan_create / pr_plan_destroy and plan introspection.
//
// One-time work per graph, on the device unless noted:
//   * the vertices are renumbered: hub rows first, then by degree bucket of
//     the in-row (longest rows first), and inside a bucket by decreasing
//     out-degree (ties by id).  Each bucket is then one contiguous range of
//     rows, so the per-vertex arrays of the update are read and written in
//     order, and inside each range the sources read most often (contrib[u] is
//     read once per out-edge of u) sit together at its start, where they stay
//     cached;
//   * inverse out-degrees in plan order (the ratio x[u]/outdeg[u] becomes one
//     multiply; Meerkat's PageRank section caches the ratio per vertex and the
//     "gpu-graph-study" T3 tier precomputes 1/deg);
//   * the plan's in-edge CSR: the transpose of the renumbered out-edge CSR,
//     built with the counting-sort transpose of pr_transpose, so every row
//     lists its sources in increasing (plan) id order;
//   * the work items of the iteration kernel: every non-hub bucket cut into
//     row ranges of about equal cost, every hub row one item, or several
//     fixed-size chunks when it is long (built on the host from the hub rows'
//     lengths).
// The caller's x, traces and ids never change: pr_run maps x in and out.
#include <cstdlib>
#include <cstring>
#include <vector>

#include "plan.hpp"
#include "transpose.hpp"

namespace pr {

namespace {

struct PlanWs {  // lives as long as the plan
    float* inv_out;
    int32_t* new_id;
    float* xi;
    float* contrib0;
    float* contrib1;
    int32_t* in_rp;
    int32_t* in_ci;
    WorkItem* items;
    ChunkRow* chunk_rows;
    float* hub_part;
    float* part;
    RunState* state;
    int64_t part_stride;
    int64_t n_items_max, n_slots_max, n_chunk_rows_max;
    size_t bytes;
};

struct PlanScratch {  // needed only while pr_plan_create runs
    int32_t* key;        // [n]
    int32_t* old_of;     // [n]
    uint32_t* deg;       // [n]
    int32_t* perm_rp;    // [n + 1]
    int32_t* perm_ci;    // [nnz]
    unsigned long long* stats;  // [2 * kNumBuckets]: rows, edges per bucket
    RadixWs vsort;       // sort of the n vertex keys (and scans over n)
    TransposeWs tr;
    size_t bytes;
};

PlanWs carve_ws(void* base, int32_t n, int64_t nnz) {
    PlanWs w{};
    Carver c(base);
    w.n_items_max = max_items(n, nnz);
    w.n_slots_max = max_chunk_slots(nnz);
    w.n_chunk_rows_max = max_chunk_rows(nnz);
    w.inv_out = c.take<float>((size_t)n);
    w.new_id = c.take<int32_t>((size_t)n);
    w.xi = c.take<float>((size_t)n);
    w.contrib0 = c.take<float>((size_t)n);
    w.contrib1 = c.take<float>((size_t)n);
    w.in_rp = c.take<int32_t>((size_t)n + 1);
    w.in_ci = c.take<int32_t>((size_t)nnz);
    w.items = c.take<WorkItem>((size_t)w.n_items_max);
    w.chunk_rows = c.take<ChunkRow>((size_t)w.n_chunk_rows_max);
    w.hub_part = c.take<float>((size_t)w.n_slots_max);
    w.part_stride = ceil_div(w.n_items_max, kBatchItems) + kMaxGrid;
    w.part = c.take<float>((size_t)(3 * w.part_stride));
    w.state = c.take<RunState>(1);
    w.bytes = c.used;
    return w;
}

PlanScratch carve_scratch(void* base, int32_t n, int64_t nnz) {
    PlanScratch s{};
    Carver c(base);
    s.key = c.take<int32_t>((size_t)n);
    s.old_of = c.take<int32_t>((size_t)n);
    s.deg = c.take<uint32_t>((size_t)n);
    s.perm_rp = c.take<int32_t>((size_t)n + 1);
    s.perm_ci = c.take<int32_t>((size_t)nnz);
    s.stats = c.take<unsigned long long>(2 * kNumBuckets);
    s.vsort = radix_carve(c, n);
    TransposeWs tw = transpose_carve(c.base ? c.base + c.used : nullptr, n, nnz);
    c.used += align_up(tw.bytes);
    s.tr = tw;
    s.bytes = c.used;
    return s;
}

unsigned grid_for(int64_t items, int64_t cap = 4096) {
    int64_t b = ceil_div(items > 0 ? items : 1, kBlock);
    return (unsigned)(b < cap ? b : cap);
}

#define GRID_STRIDE(i, count)                                                      \
    for (int64_t i = blockIdx.x * (int64_t)kBlock + threadIdx.x; i < (count); \
         i += (int64_t)gridDim.x * kBlock)

struct Bounds {
    int32_t min_len[kNumBuckets];
};

__device__ __forceinline__ int bucket_of(const Bounds& b, uint32_t len) {
    int k = 0;
#pragma unroll
    for (int j = 1; j < kNumBuckets; ++j) k += (len >= (uint32_t)b.min_len[j]) ? 1 : 0;
    return k;
}

// Sort key of each vertex: hub bucket first, then decreasing bucket, then
// decreasing out-degree (saturated at 65535); the stable sort breaks ties by
// id.  Also rows and edges per bucket.
__global__ __launch_bounds__(kBlock) void k_plan_keys(const int32_t* __restrict__ in_rp,
                                                      const int32_t* __restrict__ out_rp, int32_t n,
                                                      Bounds bounds, int32_t* __restrict__ key,
                                                      unsigned long long* __restrict__ stats) {
    __shared__ unsigned long long s[2 * kNumBuckets];
    if (threadIdx.x < 2 * kNumBuckets) s[threadIdx.x] = 0;
    __syncthreads();
    GRID_STRIDE(v, n) {
        const int32_t d_in = in_rp[v + 1] - in_rp[v];
        const uint32_t len = d_in > 0 ? (uint32_t)d_in : 0u;
        const int b = bucket_of(bounds, len);
        int32_t od = out_rp[v + 1] - out_rp[v];
        od = od < 0 ? 0 : (od > 65535 ? 65535 : od);
        key[v] = ((kNumBuckets - 1 - b) << 16) | (65535 - od);
        atomicAdd(&s[b], 1ull);
        atomicAdd(&s[kNumBuckets + b], (unsigned long long)len);
    }
    __syncthreads();
    if (threadIdx.x < 2 * kNumBuckets && s[threadIdx.x])
        atomicAdd(&stats[threadIdx.x], s[threadIdx.x]);
}

// new_id[old_of[p]] = p; deg[p] = out-degree of the vertex placed at p;
// inv_out[p] = 1/deg[p] or 0 (0 doubles as the dangling flag).
__global__ __launch_bounds__(kBlock) void k_order(const int32_t* __restrict__ old_of,
                                                  const int32_t* __restrict__ out_rp, int32_t n,
                                                  int32_t* __restrict__ new_id,
                                                  uint32_t* __restrict__ deg,
                                                  float* __restrict__ inv_out) {
    GRID_STRIDE(p, n) {
        const int32_t u = old_of[p];
        new_id[u] = (int32_t)p;
        int32_t d = out_rp[u + 1] - out_rp[u];
        d = d > 0 ? d : 0;
        deg[p] = (uint32_t)d;
        inv_out[p] = d > 0 ? 1.0f / (float)d : 0.0f;
    }
}

// Out-edge CSR in plan order: row p of the result is row old_of[p] of the
// input with every target renumbered.  Edge-parallel: each workgroup covers
// 4096 positions and finds their rows by binary search.
constexpr int kPermItems = 16;
__global__ __launch_bounds__(kBlock) void k_permute_rows(const int32_t* __restrict__ perm_rp,
                                                         const int32_t* __restrict__ old_of,
                                                         const int32_t* __restrict__ new_id,
                                                         const int32_t* __restrict__ out_rp,
                                                         const int32_t* __restrict__ out_ci,
                                                         int32_t n, int64_t nnz,
                                                         int32_t* __restrict__ perm_ci) {
    __shared__ int32_t s_lo, s_hi;
    const int64_t base = blockIdx.x * (int64_t)(kBlock * kPermItems);
    const int64_t last = (base + kBlock * kPermItems < nnz ? base + kBlock * kPermItems : nnz) - 1;
    if (threadIdx.x == 0) {
        s_lo = owner_row(perm_rp, base, 0, n - 1);
        s_hi = owner_row(perm_rp, last, s_lo, n - 1);
    }
    __syncthreads();
    for (int r = 0; r < kPermItems; ++r) {
        const int64_t p = base + r * kBlock + threadIdx.x;
        if (p > last) break;
        const int32_t j = owner_row(perm_rp, p, s_lo, s_hi);
        int64_t q = (int64_t)out_rp[old_of[j]] + (p - perm_rp[j]);
        q = q < 0 ? 0 : (q >= nnz ? nnz - 1 : q);
        const int32_t t = out_ci[q];
        // out-of-range targets were flagged by the in-degree sort, which
        // clamped them the same way
        perm_ci[p] = new_id[t < 0 ? 0 : (t >= n ? n - 1 : t)];
    }
}

// First p in [lo, hi) with in_rp[p] + kRowCost * p >= target (hi if none).
__device__ __forceinline__ int32_t cost_lower_bound(const int32_t* __restrict__ in_rp, int32_t lo,
                                                    int32_t hi, int64_t target) {
    while (lo < hi) {
        const int32_t mid = lo + (hi - lo) / 2;
        if ((int64_t)in_rp[mid] + kRowCost * (int64_t)mid < target)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

// Items of one non-hub bucket (rows [begin, end)): item k covers the rows
// whose cost prefix lies in [base + k*T, base + (k+1)*T).
__global__ __launch_bounds__(kBlock) void k_bucket_items(const int32_t* __restrict__ in_rp,
                                                         int32_t begin, int32_t end, int32_t kind,
                                                         int32_t n_items, int32_t item0,
                                                         WorkItem* __restrict__ items) {
    GRID_STRIDE(k, n_items) {
        const int64_t base = (int64_t)in_rp[begin] + kRowCost * (int64_t)begin;
        const int32_t lo =
            k == 0 ? begin : cost_lower_bound(in_rp, begin, end, base + k * kItemCost);
        const int32_t hi = (k == n_items - 1)
                               ? end
                               : cost_lower_bound(in_rp, begin, end, base + (k + 1) * kItemCost);
        WorkItem it;
        it.kind = kind;
        it.lo = lo;
        it.hi = hi < lo ? lo : hi;
        it.aux = 0;
        items[item0 + k] = it;
    }
}

// Bucket lower bounds; PR_BUCKET_MIN="0,5,17,65,1025" overrides them (a
// tuning knob).  Must start at 0, not decrease, and keep the hub bound at
// least kMinHubLength.
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
    if (tmp[0] != 0 || tmp[kHubBucket] < kMinHubLength) return;
    for (int b = 1; b < kNumBuckets; ++b)
        if (tmp[b] < tmp[b - 1]) return;
    std::memcpy(out, tmp, sizeof(tmp));
}

int check_sizes(int32_t n, int64_t nnz) {
    if (n < 1) return fail(PR_ERR_ARG, "n must be >= 1 (got %d)", n);
    if (nnz < 0 || nnz > INT32_MAX)
        return fail(PR_ERR_ARG, "nnz must be in [0, INT32_MAX] (got %lld)", (long long)nnz);
    return PR_OK;
}

}  // namespace

}  // namespace pr

using namespace pr;

extern "C" size_t pr_plan_workspace_bytes(int32_t n, int64_t nnz) {
    if (n < 1 || nnz < 0 || nnz > INT32_MAX) return 0;
    return carve_ws(nullptr, n, nnz).bytes;
}

extern "C" size_t pr_plan_scratch_bytes(int32_t n, int64_t nnz) {
    if (n < 1 || nnz < 0 || nnz > INT32_MAX) return 0;
    return carve_scratch(nullptr, n, nnz).bytes;
}

extern "C" int pr_plan_create(pr_plan** plan_out, int32_t n, int64_t nnz, const int32_t* out_rp,
                              const int32_t* out_ci, void* ws, size_t ws_bytes, void* scratch,
                              size_t scratch_bytes, uint32_t flags, void* stream_v) {
    if (!plan_out) return fail(PR_ERR_ARG, "plan_out is null");
    *plan_out = nullptr;
    PR_TRY(check_sizes(n, nnz));
    if (flags & ~PR_VALIDATE) return fail(PR_ERR_ARG, "unknown flags 0x%x", flags);
    if (!out_rp || !ws || !scratch || (nnz > 0 && !out_ci))
        return fail(PR_ERR_ARG, "null pointer argument");
    PlanWs w = carve_ws(ws, n, nnz);
    if (ws_bytes < w.bytes || (reinterpret_cast<uintptr_t>(ws) & 255u))
        return fail(PR_ERR_WORKSPACE, "plan workspace needs %zu bytes at 256-byte alignment (got %zu)",
                    w.bytes, ws_bytes);
    PlanScratch s = carve_scratch(scratch, n, nnz);
    if (scratch_bytes < s.bytes || (reinterpret_cast<uintptr_t>(scratch) & 255u))
        return fail(PR_ERR_WORKSPACE, "plan scratch needs %zu bytes at 256-byte alignment (got %zu)",
                    s.bytes, scratch_bytes);
    int dev = 0, cus = 0;
    PR_HIP_TRY(hipGetDevice(&dev));
    PR_HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    hipStream_t stream = as_stream(stream_v);
    const bool validate = flags & PR_VALIDATE;
    uint32_t* err = s.tr.error;

    PR_TRY(fill_u32(err, 0u, 1, stream));
    PR_TRY(fill_u32(reinterpret_cast<uint32_t*>(s.stats), 0u, 4 * kNumBuckets, stream));
    PR_TRY(fill_u32(reinterpret_cast<uint32_t*>(w.state), 0u, sizeof(RunState) / 4, stream));
    if (validate) {
        PR_TRY(check_out_row_ptr(out_rp, n, nnz, err, stream));
        PR_TRY(read_error_word(err, stream, "pr_plan_create"));
    }

    // 1. Plan order: in-degree buckets, then decreasing out-degree.  The
    //    in-degrees are the row lengths of the transpose, whose row pointers
    //    come from a keys-only sort of the targets (perm_rp holds them until
    //    step 2 needs it).
    PR_TRY(transpose_row_ptr(n, nnz, out_ci, s.perm_rp, s.tr, stream));
    if (validate) PR_TRY(read_error_word(err, stream, "pr_plan_create"));
    Bounds bounds;
    bucket_bounds(bounds.min_len);
    k_plan_keys<<<grid_for(n, 1024), kBlock, 0, stream>>>(s.perm_rp, out_rp, n, bounds, s.key,
                                                          s.stats);
    PR_LAUNCHED("plan keys");
    {
        RadixIn in{};
        in.count = n;
        in.n = n;
        in.keys = s.key;
        in.error = err;
        int32_t* sorted = nullptr;
        PR_TRY(radix_sort<kFromKeys>(in, 19, s.old_of, s.vsort, &sorted, stream));
    }
    k_order<<<grid_for(n), kBlock, 0, stream>>>(s.old_of, out_rp, n, w.new_id, s.deg, w.inv_out);
    PR_LAUNCHED("order");

    // 2. The plan's in-edge CSR: transpose of the out-edge CSR in plan order.
    PR_TRY(scan_exclusive(s.deg, reinterpret_cast<uint32_t*>(s.perm_rp), n, s.vsort.scan_ws,
                          stream));
    if (nnz > 0) {
        const int64_t blocks = ceil_div(nnz, kBlock * kPermItems);
        k_permute_rows<<<dim3((unsigned)blocks), kBlock, 0, stream>>>(
            s.perm_rp, s.old_of, w.new_id, out_rp, out_ci, n, nnz, s.perm_ci);
        PR_LAUNCHED("permute rows");
    }
    PR_TRY(transpose_device(n, nnz, s.perm_rp, s.perm_ci, w.in_rp, w.in_ci, s.tr, stream));

    // 3. Bucket ranges (hub bucket first) and the hub rows' lengths.
    unsigned long long stats[2 * kNumBuckets];
    PR_HIP_TRY(hipMemcpyAsync(stats, s.stats, sizeof stats, hipMemcpyDeviceToHost, stream));
    PR_HIP_TRY(hipStreamSynchronize(stream));
    int32_t row_begin[kNumBuckets + 1];  // indexed by bucket; hub rows start at 0
    {
        int64_t r = 0;
        for (int b = kHubBucket; b >= 0; --b) {
            row_begin[b] = (int32_t)r;
            r += (int64_t)stats[b];
        }
        row_begin[kNumBuckets] = (int32_t)r;  // == n
    }
    const int32_t n_hub = (int32_t)stats[kHubBucket];
    std::vector<int32_t> hub_rp((size_t)n_hub + 1);
    PR_HIP_TRY(hipMemcpyAsync(hub_rp.data(), w.in_rp, sizeof(int32_t) * hub_rp.size(),
                              hipMemcpyDeviceToHost, stream));
    PR_HIP_TRY(hipStreamSynchronize(stream));

    // 4. Work items: hub rows (whole, or chunks with slots), then buckets 3..0.
    std::vector<WorkItem> hub_items;
    std::vector<ChunkRow> chunk_rows;
    int32_t n_slots = 0;
    hub_items.reserve((size_t)n_hub);
    for (int32_t r = 0; r < n_hub; ++r) {
        const int32_t lo = hub_rp[r], hi = hub_rp[r + 1];
        if (hi - lo <= kHubChunk) {
            hub_items.push_back(WorkItem{kHubBucket, lo, hi, r});
            continue;
        }
        ChunkRow cr{r, n_slots, (int32_t)ceil_div(hi - lo, kHubChunk), 0};
        for (int32_t c = 0; c < cr.count; ++c) {
            const int32_t a = lo + c * kHubChunk;
            const int32_t b = (hi - a) < kHubChunk ? hi : a + kHubChunk;
            hub_items.push_back(WorkItem{kKindChunk, a, b, n_slots + c});
        }
        n_slots += cr.count;
        chunk_rows.push_back(cr);
    }
    int32_t items_of[kNumBuckets];
    int64_t total = (int64_t)hub_items.size();
    for (int b = 0; b < kHubBucket; ++b) {
        const int64_t bc = (int64_t)stats[kNumBuckets + b] + kRowCost * (int64_t)stats[b];
        items_of[b] = stats[b] ? (int32_t)ceil_div(bc, kItemCost) : 0;
        total += items_of[b];
    }
    if (total > w.n_items_max || n_slots > w.n_slots_max ||
        (int64_t)chunk_rows.size() > w.n_chunk_rows_max)
        return fail(PR_ERR_ARG, "work items (%lld) exceed the planned bound (%lld)",
                    (long long)total, (long long)w.n_items_max);
    if (!hub_items.empty())
        PR_HIP_TRY(hipMemcpyAsync(w.items, hub_items.data(), sizeof(WorkItem) * hub_items.size(),
                                  hipMemcpyHostToDevice, stream));
    if (!chunk_rows.empty())
        PR_HIP_TRY(hipMemcpyAsync(w.chunk_rows, chunk_rows.data(),
                                  sizeof(ChunkRow) * chunk_rows.size(), hipMemcpyHostToDevice,
                                  stream));
    int32_t item0 = (int32_t)hub_items.size();
    for (int b = kHubBucket - 1; b >= 0; --b) {
        if (items_of[b] > 0) {
            k_bucket_items<<<grid_for(items_of[b]), kBlock, 0, stream>>>(
                w.in_rp, row_begin[b], row_begin[b] + (int32_t)stats[b], b, items_of[b], item0,
                w.items);
            PR_LAUNCHED("bucket items");
        }
        item0 += items_of[b];
    }

    // 5. Launch shape: kIterBlocksPerCU workgroups per CU (each holds the
    //    hot sources in LDS), fewer when there are few item batches.
    int64_t grid = ceil_div(ceil_div(total, kBatchItems), kIterWaves);
    if (grid > (int64_t)cus * kIterBlocksPerCU) grid = (int64_t)cus * kIterBlocksPerCU;
    if (const char* env = std::getenv("PR_GRID"))  // tuning knob: workgroups per launch
        if (std::atoi(env) > 0) grid = std::atoi(env);
    if (grid > kMaxGrid / 2) grid = kMaxGrid / 2;
    if (grid < 1) grid = 1;
    int64_t fix_grid = ceil_div((int64_t)chunk_rows.size(), kFixBlock / kWave);
    if (fix_grid > kMaxGrid - grid) fix_grid = kMaxGrid - grid;

    if (validate) PR_TRY(read_error_word(err, stream, "pr_plan_create"));
    PR_HIP_TRY(hipStreamSynchronize(stream));  // host item arrays must outlive the copies

    pr_plan* p = static_cast<pr_plan*>(std::calloc(1, sizeof(pr_plan)));
    if (!p) return fail(PR_ERR_ARG, "out of host memory");
    p->device = dev;
    p->n = n;
    p->nnz = nnz;
    p->new_id = w.new_id;
    p->inv_out = w.inv_out;
    p->in_rp = w.in_rp;
    p->in_ci = w.in_ci;
    p->xi = w.xi;
    p->contrib[0] = w.contrib0;
    p->contrib[1] = w.contrib1;
    p->items = w.items;
    p->n_items = (int32_t)total;
    p->chunk_rows = w.chunk_rows;
    p->n_chunk_rows = (int32_t)chunk_rows.size();
    p->hub_part = w.hub_part;
    p->part = w.part;
    p->part_stride = w.part_stride;
    p->n_batches = (int32_t)ceil_div(total, kBatchItems);
    p->state = w.state;
    p->grid = (int32_t)grid;
    p->fix_grid = (int32_t)fix_grid;
    {
        const int64_t ig = ceil_div(n, kBlock);
        p->init_grid = (int32_t)(ig < kMaxGrid ? ig : kMaxGrid);
    }
    for (int b = 0; b < kNumBuckets; ++b) {
        p->bucket_min[b] = bounds.min_len[b];
        p->row_begin[b] = row_begin[b];
        p->bucket_edges[b] = (int64_t)stats[kNumBuckets + b];
        p->bucket_items[b] = b < kHubBucket ? items_of[b] : 0;
    }
    p->row_begin[kNumBuckets] = row_begin[kNumBuckets];
    for (const WorkItem& it : hub_items) p->bucket_items[it.kind] += 1;

    hipError_t e = hipEventCreate(&p->ev_begin);
    if (e == hipSuccess) e = hipEventCreate(&p->ev_end);
    for (int i = 0; i < 2 * kTimedLaunches && e == hipSuccess; ++i)
        e = hipEventCreate(&p->kernel_ev[i / kTimedLaunches][i % kTimedLaunches]);
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
    for (int i = 0; i < 2 * kTimedLaunches; ++i)
        if (p->kernel_ev[i / kTimedLaunches][i % kTimedLaunches])
            (void)hipEventDestroy(p->kernel_ev[i / kTimedLaunches][i % kTimedLaunches]);
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
        const int32_t hi = b == 0 ? p->row_begin[kNumBuckets] : p->row_begin[b - 1];
        if (min_len) min_len[b] = p->bucket_min[b];
        if (rows) rows[b] = hi - p->row_begin[b];
        if (edges) edges[b] = p->bucket_edges[b];
    }
    return PR_OK;
}

extern "C" int pr_plan_layout(const pr_plan* p, const int32_t** in_row_ptr,
                              const int32_t** in_col_idx, const int32_t** new_id) {
    if (!p) return fail(PR_ERR_ARG, "plan is null");
    if (in_row_ptr) *in_row_ptr = p->in_rp;
    if (in_col_idx) *in_col_idx = p->in_ci;
    if (new_id) *new_id = p->new_id;
    return PR_OK;
}
