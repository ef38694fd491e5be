// pr_transpose: in-edge CSR from out-edge CSR on the device.
//
// The Day 40 page ("One iteration, three shapes of work") transposes once on
// the host with a counting sort: a histogram of targets, a prefix sum, and a
// scatter.  Here the same steps run on the GPU as a stable LSD radix sort of
// (target, source) pairs by target, 8 bits per pass, each pass a histogram,
// an exclusive scan and a scatter.  Edges enter in source order, so stability
// leaves every in-row sorted by source: the array a sequential counting sort
// produces, bit for bit, independent of scheduling.  in_row_ptr[v] is the
// first position whose sorted target is >= v, read off the boundaries of the
// sorted targets (a per-vertex histogram with atomics would serialize on the
// hub vertices).
#include <atomic>
#include <mutex>

#include "transpose.hpp"

namespace pr {

int vertex_bits(int32_t n) {
    uint32_t hi = (uint32_t)(n - 1);
    int bits = 0;
    while (hi) {
        ++bits;
        hi >>= 1;
    }
    return bits;
}

TransposeWs transpose_carve(void* base, int32_t n, int64_t nnz) {
    (void)n;
    TransposeWs w{};
    Carver c(base);
    w.sort = radix_carve(c, nnz);
    w.tile_row = c.take<int32_t>((size_t)radix_tiles(nnz) + 1);
    w.error = c.take<uint32_t>(1);
    w.bytes = c.used;
    return w;
}

namespace {

// in_rp[v] = first i with keys[i] >= v, for v in [0, n]; keys sorted.  Element
// i writes the vertices in (keys[i-1], keys[i]] (with keys[-1] = -1 and
// keys[m] = n), so every v is written exactly once.  A lane takes kRowsRun
// consecutive elements with two 16-byte loads (keys is 256-byte aligned
// scratch) plus the key before them, so a wavefront keeps 2 KiB of reads in
// flight; the lane holding the end of the array takes its elements one by
// one.
constexpr int kRowsRun = 8;

__global__ __launch_bounds__(kBlock) void k_rows_from_sorted(const int32_t* __restrict__ keys,
                                                             int64_t m, int32_t n,
                                                             int32_t* __restrict__ in_rp) {
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    const int64_t runs = m / kRowsRun + 1;  // the last run holds element m
    for (int64_t c = blockIdx.x * (int64_t)kBlock + threadIdx.x; c < runs;
         c += (int64_t)gridDim.x * kBlock) {
        const int64_t i0 = c * kRowsRun;
        int32_t prev = i0 == 0 ? -1 : keys[i0 - 1];
        if (i0 + kRowsRun <= m) {
            const i32x4 a = *(const i32x4*)(keys + i0);
            const i32x4 b = *(const i32x4*)(keys + i0 + 4);
            const int32_t k[kRowsRun] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int j = 0; j < kRowsRun; ++j) {
                for (int32_t v = prev + 1; v <= k[j]; ++v) in_rp[v] = (int32_t)(i0 + j);
                prev = k[j];
            }
        } else {
            for (int64_t i = i0; i <= m; ++i) {
                const int32_t hi = i == m ? n : keys[i];
                for (int32_t v = prev + 1; v <= hi; ++v) in_rp[v] = (int32_t)i;
                prev = hi;
            }
        }
    }
}

// tile_row[t] = the row that owns edge t * kRadixTile (the first edge of tile
// t), for t < T, and tile_row[T] = n - 1: the first pass's row range of tile
// t is then [tile_row[t], tile_row[t + 1]] (a bound on the owner of its last
// edge).  One lane per tile, each a binary search: the searches run side by
// side here instead of in series at the start of every tile of the pass.
__global__ __launch_bounds__(kBlock) void k_tile_rows(const int32_t* __restrict__ rp, int32_t n,
                                                      int64_t T, int32_t* __restrict__ tile_row) {
    const int64_t t = blockIdx.x * (int64_t)kBlock + threadIdx.x;
    if (t < T) tile_row[t] = owner_row(rp, t * kRadixTile, 0, n - 1);
    if (t == T) tile_row[T] = n - 1;
}

// Checks of an out-edge CSR for PR_VALIDATE: row_ptr[0] == 0, non-decreasing,
// row_ptr[n] == nnz.  (Columns are range-checked by the first sort pass.)
__global__ __launch_bounds__(kBlock) void k_check_row_ptr(const int32_t* __restrict__ rp, int32_t n,
                                                          int64_t nnz, uint32_t* __restrict__ err) {
    for (int64_t i = blockIdx.x * (int64_t)kBlock + threadIdx.x; i <= n;
         i += (int64_t)gridDim.x * kBlock) {
        bool bad = false;
        if (i == 0 && rp[0] != 0) bad = true;
        if (i == n && (int64_t)rp[n] != nnz) bad = true;
        if (i < n && rp[i + 1] < rp[i]) bad = true;
        if (bad) *err = 1u;
    }
}

unsigned grid_for(int64_t items, int64_t cap = 8192) {
    int64_t b = ceil_div(items > 0 ? items : 1, kBlock);
    return (unsigned)(b < cap ? b : cap);
}

}  // namespace

int check_out_row_ptr(const int32_t* rp, int32_t n, int64_t nnz, uint32_t* err, hipStream_t stream) {
    k_check_row_ptr<<<grid_for((int64_t)n + 1), kBlock, 0, stream>>>(rp, n, nnz, err);
    PR_LAUNCHED("check row_ptr");
    return PR_OK;
}

int window_rows(const int32_t* rp, int32_t n, int64_t T, int32_t* win_row, hipStream_t stream) {
    k_tile_rows<<<grid_for(T + 1, INT32_MAX), kBlock, 0, stream>>>(rp, n, T, win_row);
    PR_LAUNCHED("window rows");
    return PR_OK;
}

int transpose_device(int32_t n, int64_t nnz, const int32_t* out_rp, const int32_t* out_ci,
                     int32_t* in_rp, int32_t* in_ci, const TransposeWs& w, hipStream_t stream) {
    if (nnz == 0) return fill_u32(reinterpret_cast<uint32_t*>(in_rp), 0u, (int64_t)n + 1, stream);
    RadixIn in{};
    in.count = nnz;
    in.n = n;
    in.keys = out_ci;
    in.row_ptr = out_rp;
    in.tile_row = w.tile_row;
    in.error = w.error;
    const int64_t T = radix_tiles(nnz);
    k_tile_rows<<<grid_for(T + 1, INT32_MAX), kBlock, 0, stream>>>(out_rp, n, T, w.tile_row);
    PR_LAUNCHED("tile rows");
    int32_t* sorted_keys = nullptr;
    PR_TRY(radix_sort<kFromOutCsr>(in, vertex_bits(n), in_ci, w.sort, &sorted_keys, stream));
    k_rows_from_sorted<<<grid_for(nnz / kRowsRun + 1), kBlock, 0, stream>>>(sorted_keys, nnz, n, in_rp);
    PR_LAUNCHED("row pointers");
    return PR_OK;
}

int transpose_row_ptr(int32_t n, int64_t nnz, const int32_t* out_ci, int32_t* in_rp,
                      const TransposeWs& w, hipStream_t stream) {
    if (nnz == 0) return fill_u32(reinterpret_cast<uint32_t*>(in_rp), 0u, (int64_t)n + 1, stream);
    RadixIn in{};
    in.count = nnz;
    in.n = n;
    in.keys = out_ci;
    in.error = w.error;
    int32_t* sorted_keys = nullptr;
    PR_TRY(radix_sort_keys<kFromTargets>(in, vertex_bits(n), w.sort, &sorted_keys, stream));
    k_rows_from_sorted<<<grid_for(nnz / kRowsRun + 1), kBlock, 0, stream>>>(sorted_keys, nnz, n, in_rp);
    PR_LAUNCHED("row pointers");
    return PR_OK;
}

int read_error_word(const uint32_t* err_dev, hipStream_t stream, const char* what) {
    uint32_t h = 0;
    PR_HIP_TRY(hipMemcpyAsync(&h, err_dev, sizeof h, hipMemcpyDeviceToHost, stream));
    PR_HIP_TRY(hipStreamSynchronize(stream));
    if (h) return fail(PR_ERR_GRAPH, "%s: malformed CSR", what);
    return PR_OK;
}

}  // namespace pr

using namespace pr;

extern "C" size_t pr_transpose_workspace_bytes(int32_t n, int64_t nnz) {
    if (n < 1 || nnz < 0 || nnz > INT32_MAX) return 0;
    return transpose_carve(nullptr, n, nnz).bytes;
}

extern "C" int pr_transpose(int32_t n, int64_t nnz, const int32_t* out_row_ptr,
                            const int32_t* out_col_idx, int32_t* in_row_ptr, int32_t* in_col_idx,
                            void* ws, size_t ws_bytes, uint32_t flags, void* stream_v) {
    if (n < 1) return fail(PR_ERR_ARG, "n must be >= 1 (got %d)", n);
    if (nnz < 0 || nnz > INT32_MAX)
        return fail(PR_ERR_ARG, "nnz must be in [0, INT32_MAX] (got %lld)", (long long)nnz);
    if (flags & ~PR_VALIDATE) return fail(PR_ERR_ARG, "unknown flags 0x%x", flags);
    if (!out_row_ptr || !in_row_ptr || !ws || (nnz > 0 && (!out_col_idx || !in_col_idx)))
        return fail(PR_ERR_ARG, "null pointer argument");
    TransposeWs w = transpose_carve(ws, n, nnz);
    if (ws_bytes < w.bytes || (reinterpret_cast<uintptr_t>(ws) & 255u))
        return fail(PR_ERR_WORKSPACE,
                    "transpose workspace needs %zu bytes at 256-byte alignment (got %zu)", w.bytes,
                    ws_bytes);
    hipStream_t stream = as_stream(stream_v);
    const bool validate = flags & PR_VALIDATE;
    PR_TRY(fill_u32(w.error, 0u, 1, stream));
    if (validate) {
        // A malformed row_ptr makes the owner-row search meaningless: report
        // it before sorting.
        PR_TRY(check_out_row_ptr(out_row_ptr, n, nnz, w.error, stream));
        PR_TRY(read_error_word(w.error, stream, "pr_transpose"));
    }
    PR_TRY(transpose_device(n, nnz, out_row_ptr, out_col_idx, in_row_ptr, in_col_idx, w, stream));
    if (validate) PR_TRY(read_error_word(w.error, stream, "pr_transpose"));
    return PR_OK;
}

// ---------------------------------------------------------------------------
// pr_transpose_noalloc: pr_transpose with its workspace in a device array of
// the library's own, for callers that cannot allocate.
//
// `scratch` is a file-scope device array: every device the library runs on
// holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in, not a device
// address); the device address comes from hipGetSymbolAddress, once per
// device, with that device current, and is kept per device.
namespace {

static __device__ __align__(256) unsigned char scratch[PR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// The current device's copy of `scratch` (its address looked up on the first
// call on that device).
int scratch_on_current_device(void** out) {
    int dev = -1;
    PR_HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PR_ERR_ARG, "device %d is beyond the %d devices the library tracks", dev,
                    kMaxDevices);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            PR_HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
            if (!p) return fail(PR_ERR_HIP, "no device address for the library's scratch array");
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return PR_OK;
}

}  // namespace

extern "C" int pr_transpose_noalloc(int32_t n, int64_t nnz, const int32_t* out_row_ptr,
                                    const int32_t* out_col_idx, int32_t* in_row_ptr,
                                    int32_t* in_col_idx, uint32_t flags, void* stream) {
    if (n < 1) return fail(PR_ERR_ARG, "n must be >= 1 (got %d)", n);
    if (nnz < 0 || nnz > INT32_MAX)
        return fail(PR_ERR_ARG, "nnz must be in [0, INT32_MAX] (got %lld)", (long long)nnz);
    const size_t need = transpose_carve(nullptr, n, nnz).bytes;
    if (need > (size_t)PR_NOALLOC_SCRATCH_BYTES)
        return fail(PR_ERR_WORKSPACE,
                    "pr_transpose_noalloc: n = %d, nnz = %lld need %zu bytes of workspace, more "
                    "than the library's %zu-byte scratch array (use pr_transpose)",
                    n, (long long)nnz, need, (size_t)PR_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    PR_TRY(scratch_on_current_device(&ws));
    return pr_transpose(n, nnz, out_row_ptr, out_col_idx, in_row_ptr, in_col_idx, ws,
                        (size_t)PR_NOALLOC_SCRATCH_BYTES, flags, stream);
}
