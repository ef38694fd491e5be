// The valued sparse product y = A x of a CSR matrix in double precision.
//
// What it computes ("A Pedagogical Introduction to Porting a Conjugate
// Gradient Solver to CUDA", the sparse product of its CG loop, on the
// flattened row_offsets / cols / vals arrays): y[i] = the sum over row i's
// stored entries j of vals[j] * x[cols[j]].
//
// How rows are scheduled: by length, as the pull iteration schedules its
// in-rows ("gpu-graph-study", PageRank T4: thread, warp or block per vertex
// by degree), re-cut for 64-lane wavefronts and for a value stream:
//   * short rows (at most kShortMax entries) in streamed blocks: a workgroup
//     loads the products of a run of consecutive short rows -- at most kCap
//     entries, read as two contiguous streams -- into LDS, then one lane per
//     row adds its row's products in stored order, starting from zero, as the
//     CPU loop does;
//   * medium rows (up to kMediumMax) one wavefront each, four per workgroup;
//   * long rows in chunks of kChunk entries, one workgroup per chunk, the
//     chunk sums added in order by a second kernel.
// The blocks, row lists and chunks are built once per sparsity pattern on the
// device (flags, two exclusive scans, a scatter) and kept in the plan.
#include <algorithm>
#include <new>

#include "common.hpp"

namespace pr {
namespace {

constexpr int32_t kShortMax = 64;
constexpr int32_t kMediumMax = 1024;
constexpr int32_t kChunk = 4096;
constexpr int32_t kCap = 2048;                   // entries one streamed block holds in LDS
constexpr int32_t kWindow = kCap - kShortMax;    // a block's rows all start in one window
constexpr int32_t kBlockRows = 1024;             // rows one streamed block holds at most
constexpr int kStreamIters = kCap / kBlock;      // 8 entries per lane
constexpr int kRowLoads = 4;                     // entries in flight per lane, medium / chunk
constexpr int kXcds = 8;                         // workgroup b runs on XCD b % 8
static_assert(kCap % kBlock == 0, "a streamed block is whole lane rounds");
static_assert(kChunk % (kBlock * kRowLoads) == 0, "a chunk is whole load rounds");

// A work item.  Chunk items: entries [lo, hi) of row `row`, whose sum goes to
// part[slot].  Wavefront items: mrows[lo .. hi), one row per wavefront.
// Streamed blocks: rows [lo, hi).
struct Item {
    int32_t lo, hi, row, slot;
};

// A long row: its chunk sums are part[first .. first + count).
struct LongRow {
    int32_t row, first, count, pad;
};

__device__ __forceinline__ int row_class(int64_t len) {
    return len <= kShortMax ? 0 : (len <= kMediumMax ? 1 : 2);
}

__device__ __forceinline__ int64_t chunks_of(int64_t len) { return (len + kChunk - 1) / kChunk; }

__device__ __forceinline__ int64_t rp_at(const int32_t* __restrict__ rp, int64_t i) {
    return (int64_t)max(rp[i], 0);  // a malformed (negative) offset reads as 0
}

// Does short row r start a streamed block?  (Row r-1 is known to exist.)
__device__ __forceinline__ bool opens_block(int64_t r, int prev_class, int64_t prev_start,
                                            int64_t start) {
    return prev_class != 0 || r % kBlockRows == 0 || prev_start / kWindow != start / kWindow;
}

// Per row: a = (opens a streamed block) | chunks << 32, b = (medium) | (long) << 32.
__global__ __launch_bounds__(kBlock) void k_spmv_classify(const int32_t* __restrict__ rp, int32_t n,
                                                         uint64_t* __restrict__ a,
                                                         uint64_t* __restrict__ b) {
    for (int64_t r = blockIdx.x * (int64_t)kBlock + threadIdx.x; r < n;
         r += (int64_t)gridDim.x * kBlock) {
        const int64_t s = rp_at(rp, r), e = rp_at(rp, r + 1);
        const int cls = row_class(e - s);
        bool open = false;
        if (cls == 0) {
            if (r == 0) {
                open = true;
            } else {
                const int64_t ps = rp_at(rp, r - 1);
                open = opens_block(r, row_class(s - ps), ps, s);
            }
        }
        const uint64_t chunks = cls == 2 ? (uint64_t)chunks_of(e - s) : 0u;
        a[r] = (open ? 1u : 0u) | chunks << 32;
        b[r] = (cls == 1 ? 1u : 0u) | (uint64_t)(cls == 2 ? 1u : 0u) << 32;
    }
}

struct ScatterArgs {
    const int32_t* rp;
    int32_t n;
    const uint64_t* a_scan;  // exclusive scans of k_spmv_classify's a and b
    const uint64_t* b_scan;
    Item* items;
    int32_t* mrows;
    LongRow* longs;
    int32_t n_medium;
    int32_t medium_base;  // first wavefront item
    int32_t short_base;   // first streamed block
};

__global__ __launch_bounds__(kBlock) void k_spmv_scatter(ScatterArgs g) {
    for (int64_t r = blockIdx.x * (int64_t)kBlock + threadIdx.x; r < g.n;
         r += (int64_t)gridDim.x * kBlock) {
        const int64_t s = rp_at(g.rp, r), e = rp_at(g.rp, r + 1);
        const int cls = row_class(e - s);
        const uint64_t a = g.a_scan[r], b = g.b_scan[r];
        if (cls == 0) {
            bool open = r == 0;
            if (!open) {
                const int64_t ps = rp_at(g.rp, r - 1);
                open = opens_block(r, row_class(s - ps), ps, s);
            }
            // the block this row belongs to: blocks opened before it, plus its own
            const int64_t blk = g.short_base + (int64_t)(uint32_t)a + (open ? 1 : 0) - 1;
            if (open) g.items[blk].lo = (int32_t)r;
            bool close = r + 1 == g.n;
            if (!close) {
                const int64_t ne = rp_at(g.rp, r + 2);
                close = row_class(ne - e) != 0 || opens_block(r + 1, 0, s, e);
            }
            if (close) {
                g.items[blk].hi = (int32_t)(r + 1);
                g.items[blk].row = -1;
                g.items[blk].slot = -1;
            }
        } else if (cls == 1) {
            const int32_t m = (int32_t)(uint32_t)b;
            g.mrows[m] = (int32_t)r;
            if (m % kWaves == 0) {
                Item it;
                it.lo = m;
                it.hi = min(m + kWaves, g.n_medium);
                it.row = -1;
                it.slot = -1;
                g.items[g.medium_base + m / kWaves] = it;
            }
        } else {
            const int32_t first = (int32_t)(a >> 32);
            const int32_t count = (int32_t)chunks_of(e - s);
            LongRow lr;
            lr.row = (int32_t)r;
            lr.first = first;
            lr.count = count;
            lr.pad = 0;
            g.longs[(int32_t)(b >> 32)] = lr;
            for (int32_t k = 0; k < count; ++k) {
                Item it;
                it.lo = (int32_t)(s + (int64_t)k * kChunk);
                it.hi = (int32_t)min(s + (int64_t)(k + 1) * kChunk, e);
                it.row = (int32_t)r;
                it.slot = first + k;
                g.items[first + k] = it;
            }
        }
    }
}

__global__ __launch_bounds__(kBlock) void k_spmv_check_cols(const int32_t* __restrict__ ci,
                                                           int64_t nnz, int32_t n_cols,
                                                           uint32_t* __restrict__ err) {
    for (int64_t j = blockIdx.x * (int64_t)kBlock + threadIdx.x; j < nnz;
         j += (int64_t)gridDim.x * kBlock)
        if ((uint32_t)ci[j] >= (uint32_t)n_cols) *err = 1u;
}

// ------------------------------------------------------------------ product

struct SpmvArgs {
    const int32_t* rp;
    const int32_t* ci;
    const double* vals;
    const double* x;
    double* y;
    const Item* items;
    const int32_t* mrows;
    double* part;
    uint32_t nnz;
    uint32_t col_max;    // n_cols - 1: columns are clamped to it
    int32_t n_chunks;    // items [0, n_chunks)
    int32_t n_wave;      // items [n_chunks, n_chunks + n_wave)
    int32_t long_grid;   // n_chunks + n_wave rounded up to a multiple of kXcds
    int32_t n_short;     // items [n_chunks + n_wave, ... + n_short)
    int32_t per_xcd;     // streamed blocks per XCD: ceil(n_short / kXcds)
};

__device__ __forceinline__ uint32_t clamp_entry(int64_t j, uint32_t nnz) {
    return (uint32_t)min(max(j, (int64_t)0), (int64_t)nnz - 1);
}

__device__ __forceinline__ double gather(const SpmvArgs& a, uint32_t j, double& v) {
    v = a.vals[j];
    return a.x[min((uint32_t)a.ci[j], a.col_max)];
}

// Sum of vals[j] * x[col[j]] over j = first + lane, first + lane + stride, ...
// below end, kRowLoads entries in flight per lane.
template <int kStride>
__device__ __forceinline__ double strided_sum(const SpmvArgs& a, int64_t first, int64_t end,
                                              int lane) {
    double p = 0.0;
    for (int64_t base = first; base < end; base += (int64_t)kStride * kRowLoads) {
        uint32_t j[kRowLoads];
        double v[kRowLoads], xv[kRowLoads];
#pragma unroll
        for (int k = 0; k < kRowLoads; ++k) j[k] = clamp_entry(base + k * kStride + lane, a.nnz);
#pragma unroll
        for (int k = 0; k < kRowLoads; ++k) xv[k] = gather(a, j[k], v[k]);
#pragma unroll
        for (int k = 0; k < kRowLoads; ++k)
            if (base + k * kStride + lane < end) p += v[k] * xv[k];
    }
    return p;
}

__device__ void short_block(const SpmvArgs& a, const Item& it, double* prod) {
    const int t = threadIdx.x;
    const int64_t e0 = rp_at(a.rp, it.lo);
    const int32_t ne = a.nnz == 0 ? 0
                                  : (int32_t)min(max(rp_at(a.rp, it.hi) - e0, (int64_t)0),
                                                 (int64_t)kCap);
    if (ne > 0) {
        uint32_t j[kStreamIters];
        double v[kStreamIters], xv[kStreamIters];
#pragma unroll
        for (int i = 0; i < kStreamIters; ++i)
            j[i] = clamp_entry(e0 + min(i * kBlock + t, ne - 1), a.nnz);
#pragma unroll
        for (int i = 0; i < kStreamIters; ++i) xv[i] = gather(a, j[i], v[i]);
        // Each product is rounded on its own when it is stored: nothing here
        // is fused into the sums below.
#pragma unroll
        for (int i = 0; i < kStreamIters; ++i)
            if (i * kBlock + t < ne) prod[i * kBlock + t] = v[i] * xv[i];
    }
    __syncthreads();
    for (int64_t r = it.lo + t; r < it.hi; r += kBlock) {
        const int32_t s = (int32_t)min(max(rp_at(a.rp, r) - e0, (int64_t)0), (int64_t)ne);
        const int32_t e = (int32_t)min(max(rp_at(a.rp, r + 1) - e0, (int64_t)s), (int64_t)ne);
        // in stored order; the reads of a group of 8 are issued together
        double sum = 0.0;
        int32_t k = s;
        for (; k + 8 <= e; k += 8) {
            double q[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = prod[k + i];
#pragma unroll
            for (int i = 0; i < 8; ++i) sum += q[i];
        }
        for (; k < e; ++k) sum += prod[k];
        a.y[r] = sum;
    }
}

__global__ __launch_bounds__(kBlock) void k_spmv(SpmvArgs a) {
    __shared__ double prod[kCap];
    const int32_t b = blockIdx.x;
    if (b < a.n_chunks) {  // one chunk of a long row, whole workgroup
        const Item it = a.items[b];
        const double p = strided_sum<kBlock>(a, it.lo, it.hi, threadIdx.x);
        const double s = block_sum(p, prod);
        if (threadIdx.x == 0) a.part[it.slot] = s;
        return;
    }
    if (b < a.n_chunks + a.n_wave) {  // up to four medium rows, one per wavefront
        const Item it = a.items[b];
        const int32_t m = it.lo + (int32_t)(threadIdx.x / kWave);
        if (m >= it.hi) return;
        const int32_t row = a.mrows[m];
        const double p = wave_sum(
            strided_sum<kWave>(a, rp_at(a.rp, row), rp_at(a.rp, row + 1), lane_id()));
        if (lane_id() == 0) a.y[row] = p;
        return;
    }
    if (b < a.long_grid) return;
    // Streamed blocks: XCD x takes the contiguous range [x * per_xcd, (x+1) *
    // per_xcd), so neighbouring rows -- which gather neighbouring x -- share an L2.
    const int32_t j = b - a.long_grid;
    const int32_t s = (j % kXcds) * a.per_xcd + j / kXcds;
    if (s >= a.n_short) return;
    short_block(a, a.items[a.n_chunks + a.n_wave + s], prod);
}

__global__ __launch_bounds__(kBlock) void k_spmv_long_rows(const LongRow* __restrict__ longs,
                                                          int32_t n_long,
                                                          const double* __restrict__ part,
                                                          double* __restrict__ y) {
    const int32_t i = blockIdx.x * kBlock + threadIdx.x;
    if (i >= n_long) return;
    const LongRow lr = longs[i];
    double sum = 0.0;
    for (int32_t k = 0; k < lr.count; ++k) sum += part[lr.first + k];
    y[lr.row] = sum;
}

// ------------------------------------------------------------------ sizes

struct Bounds {
    int64_t longs, chunks, medium, wave_items, short_blocks, items;
};

Bounds bounds(int32_t n, int64_t nnz) {
    Bounds B;
    B.longs = nnz / (kMediumMax + 1);
    B.chunks = B.longs + nnz / kChunk;
    B.medium = std::min<int64_t>(n, nnz / (kShortMax + 1));
    B.wave_items = ceil_div(B.medium, kWaves);
    // a streamed block opens at row 0, after a medium or long row, at a
    // multiple of kBlockRows, or where the row starts cross a window
    B.short_blocks = 3 + B.medium + B.longs + n / kBlockRows + nnz / kWindow;
    B.items = B.chunks + B.wave_items + B.short_blocks;
    return B;
}

struct SpmvWs {
    Item* items;
    int32_t* mrows;
    LongRow* longs;
    double* part;
    size_t bytes;
};

SpmvWs carve_ws(void* base, int32_t n, int64_t nnz) {
    const Bounds B = bounds(n, nnz);
    Carver c(base);
    SpmvWs w;
    w.items = c.take<Item>(B.items);
    w.mrows = c.take<int32_t>(B.medium);
    w.longs = c.take<LongRow>(B.longs);
    w.part = c.take<double>(B.chunks);
    w.bytes = c.used;
    return w;
}

struct SpmvScratch {
    uint64_t* a;
    uint64_t* b;
    uint64_t* a_scan;  // [n + 1]
    uint64_t* b_scan;  // [n + 1]
    uint32_t* err;
    void* scan_ws;
    size_t bytes;
};

SpmvScratch carve_scratch(void* base, int32_t n) {
    Carver c(base);
    SpmvScratch s;
    s.a = c.take<uint64_t>(n);
    s.b = c.take<uint64_t>(n);
    s.a_scan = c.take<uint64_t>((size_t)n + 1);
    s.b_scan = c.take<uint64_t>((size_t)n + 1);
    s.err = c.take<uint32_t>(1);
    s.scan_ws = c.take<char>(scan_workspace_bytes(n));
    s.bytes = c.used;
    return s;
}

unsigned rows_grid(int64_t items) {
    const int64_t g = ceil_div(items > 0 ? items : 1, kBlock);
    return (unsigned)(g < 8192 ? g : 8192);
}

int check_sizes(int32_t n_rows, int32_t n_cols, int64_t nnz) {
    if (n_rows < 0 || n_cols < 0) return fail(PR_ERR_ARG, "n_rows and n_cols must be >= 0");
    if (nnz < 0 || nnz > INT32_MAX)
        return fail(PR_ERR_ARG, "nnz must be in [0, INT32_MAX] (got %lld)", (long long)nnz);
    if (nnz > 0 && (n_rows < 1 || n_cols < 1))
        return fail(PR_ERR_ARG, "stored entries need n_rows >= 1 and n_cols >= 1");
    return PR_OK;
}

}  // namespace
}  // namespace pr

struct pr_spmv_plan {
    int device;
    int32_t n_rows, n_cols;
    int64_t nnz;
    const int32_t* rp;
    const int32_t* ci;
    pr::Item* items;
    int32_t* mrows;
    pr::LongRow* longs;
    double* part;
    int32_t n_chunks, n_wave, n_short, n_long, n_medium;
};

using namespace pr;

extern "C" size_t pr_spmv_workspace_bytes(int32_t n_rows, int64_t nnz) {
    if (n_rows < 0 || nnz < 0 || nnz > INT32_MAX) return 0;
    return carve_ws(nullptr, n_rows, nnz).bytes;
}

extern "C" size_t pr_spmv_scratch_bytes(int32_t n_rows, int64_t nnz) {
    if (n_rows < 0 || nnz < 0 || nnz > INT32_MAX) return 0;
    return carve_scratch(nullptr, n_rows).bytes;
}

extern "C" int pr_spmv_plan_create(pr_spmv_plan** plan_out, int32_t n_rows, int32_t n_cols,
                                   int64_t nnz, const int32_t* rp, const int32_t* ci, void* ws,
                                   size_t ws_bytes, void* scratch, size_t scratch_bytes,
                                   uint32_t flags, void* stream_v) {
    if (!plan_out) return fail(PR_ERR_ARG, "plan_out is null");
    *plan_out = nullptr;
    PR_TRY(check_sizes(n_rows, n_cols, nnz));
    if (flags & ~PR_VALIDATE) return fail(PR_ERR_ARG, "unknown flags 0x%x", flags);
    if (!rp || !ws || !scratch || (nnz > 0 && !ci)) return fail(PR_ERR_ARG, "null pointer argument");
    const SpmvWs w = carve_ws(ws, n_rows, nnz);
    if (ws_bytes < w.bytes || (reinterpret_cast<uintptr_t>(ws) & 255u))
        return fail(PR_ERR_WORKSPACE, "product workspace needs %zu bytes at 256-byte alignment (got %zu)",
                    w.bytes, ws_bytes);
    const SpmvScratch s = carve_scratch(scratch, n_rows);
    if (scratch_bytes < s.bytes || (reinterpret_cast<uintptr_t>(scratch) & 255u))
        return fail(PR_ERR_WORKSPACE, "product scratch needs %zu bytes at 256-byte alignment (got %zu)",
                    s.bytes, scratch_bytes);
    int dev = 0;
    PR_HIP_TRY(hipGetDevice(&dev));
    hipStream_t stream = as_stream(stream_v);

    if (flags & PR_VALIDATE) {
        PR_TRY(fill_u32(s.err, 0u, 1, stream));
        PR_TRY(check_out_row_ptr(rp, n_rows, nnz, s.err, stream));
        if (nnz > 0) {
            k_spmv_check_cols<<<rows_grid(nnz), kBlock, 0, stream>>>(ci, nnz, n_cols, s.err);
            PR_LAUNCHED("check columns");
        }
        PR_TRY(read_error_word(s.err, stream, "pr_spmv_plan_create"));
    }

    int32_t n_chunks = 0, n_medium = 0, n_long = 0, n_short = 0;
    if (n_rows > 0) {
        k_spmv_classify<<<rows_grid(n_rows), kBlock, 0, stream>>>(rp, n_rows, s.a, s.b);
        PR_LAUNCHED("classify rows");
        PR_TRY(scan_exclusive(s.a, s.a_scan, n_rows, s.scan_ws, stream));
        PR_TRY(scan_exclusive(s.b, s.b_scan, n_rows, s.scan_ws, stream));
        uint64_t tot[2] = {0, 0};
        PR_HIP_TRY(hipMemcpyAsync(&tot[0], s.a_scan + n_rows, sizeof(uint64_t),
                                  hipMemcpyDeviceToHost, stream));
        PR_HIP_TRY(hipMemcpyAsync(&tot[1], s.b_scan + n_rows, sizeof(uint64_t),
                                  hipMemcpyDeviceToHost, stream));
        PR_HIP_TRY(hipStreamSynchronize(stream));
        n_short = (int32_t)(uint32_t)tot[0];
        n_chunks = (int32_t)(tot[0] >> 32);
        n_medium = (int32_t)(uint32_t)tot[1];
        n_long = (int32_t)(tot[1] >> 32);
        const Bounds B = bounds(n_rows, nnz);
        if (n_short > B.short_blocks || n_chunks > B.chunks || n_medium > B.medium ||
            n_long > B.longs)
            return fail(PR_ERR_GRAPH, "pr_spmv_plan_create: row pointers are not a CSR of %lld entries",
                        (long long)nnz);
        ScatterArgs g;
        g.rp = rp;
        g.n = n_rows;
        g.a_scan = s.a_scan;
        g.b_scan = s.b_scan;
        g.items = w.items;
        g.mrows = w.mrows;
        g.longs = w.longs;
        g.n_medium = n_medium;
        g.medium_base = n_chunks;
        g.short_base = n_chunks + (int32_t)ceil_div(n_medium, kWaves);
        k_spmv_scatter<<<rows_grid(n_rows), kBlock, 0, stream>>>(g);
        PR_LAUNCHED("scatter rows");
        PR_HIP_TRY(hipStreamSynchronize(stream));  // the scratch is free once this returns
    }

    pr_spmv_plan* p = new (std::nothrow) pr_spmv_plan{};
    if (!p) return fail(PR_ERR_ARG, "out of host memory");
    p->device = dev;
    p->n_rows = n_rows;
    p->n_cols = n_cols;
    p->nnz = nnz;
    p->rp = rp;
    p->ci = ci;
    p->items = w.items;
    p->mrows = w.mrows;
    p->longs = w.longs;
    p->part = w.part;
    p->n_chunks = n_chunks;
    p->n_wave = (int32_t)ceil_div(n_medium, kWaves);
    p->n_short = n_short;
    p->n_long = n_long;
    p->n_medium = n_medium;
    *plan_out = p;
    return PR_OK;
}

extern "C" int pr_spmv_plan_destroy(pr_spmv_plan* p) {
    delete p;
    return PR_OK;
}

extern "C" int pr_spmv(const pr_spmv_plan* p, const double* vals, const double* x, double* y,
                       void* stream_v) {
    if (!p) return fail(PR_ERR_ARG, "plan is null");
    if ((p->nnz > 0 && (!vals || !x)) || (p->n_rows > 0 && !y))
        return fail(PR_ERR_ARG, "null pointer argument");
    int dev = -1;
    PR_HIP_TRY(hipGetDevice(&dev));
    if (dev != p->device)
        return fail(PR_ERR_ARG, "plan belongs to device %d but device %d is current", p->device, dev);
    if (p->n_rows == 0) return PR_OK;
    hipStream_t stream = as_stream(stream_v);
    SpmvArgs a;
    a.rp = p->rp;
    a.ci = p->ci;
    a.vals = vals;
    a.x = x;
    a.y = y;
    a.items = p->items;
    a.mrows = p->mrows;
    a.part = p->part;
    a.nnz = (uint32_t)p->nnz;
    a.col_max = p->n_cols > 0 ? (uint32_t)(p->n_cols - 1) : 0u;
    a.n_chunks = p->n_chunks;
    a.n_wave = p->n_wave;
    a.long_grid = (int32_t)ceil_div(p->n_chunks + p->n_wave, kXcds) * kXcds;
    a.n_short = p->n_short;
    a.per_xcd = (int32_t)ceil_div(p->n_short, kXcds);
    const int64_t grid = (int64_t)a.long_grid + (int64_t)a.per_xcd * kXcds;
    if (grid > 0) {
        k_spmv<<<dim3((unsigned)grid), dim3(kBlock), 0, stream>>>(a);
        PR_LAUNCHED("sparse product");
    }
    if (p->n_long > 0) {
        k_spmv_long_rows<<<dim3((unsigned)ceil_div(p->n_long, kBlock)), dim3(kBlock), 0, stream>>>(
            p->longs, p->n_long, p->part, y);
        PR_LAUNCHED("long rows");
    }
    return PR_OK;
}

extern "C" int pr_spmv_plan_items(const pr_spmv_plan* p, int32_t* counts) {
    if (!p || !counts) return fail(PR_ERR_ARG, "null pointer argument");
    counts[0] = p->n_short;
    counts[1] = p->n_medium;
    counts[2] = p->n_long;
    counts[3] = p->n_chunks;
    return PR_OK;
}
