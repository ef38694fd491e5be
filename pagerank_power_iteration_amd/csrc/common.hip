// Status strings, the thread-local error message, a fill kernel and the
// device-wide exclusive scan (the "prefix sum" step of the counting-sort
// transpose on the Day 40 page, "One iteration, three shapes of work").
#include <cstdarg>
#include <cstdio>

#include "common.hpp"

namespace pr {

namespace {
thread_local char g_last_error[512] = "";
}

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

// ------------------------------------------------------------------- fill

__global__ __launch_bounds__(kBlock) void k_fill_u32(uint32_t* __restrict__ p, uint32_t value,
                                                     int64_t count) {
    for (int64_t i = blockIdx.x * (int64_t)kBlock + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * kBlock)
        p[i] = value;
}

int fill_u32(uint32_t* p, uint32_t value, int64_t count, hipStream_t stream) {
    if (count <= 0) return PR_OK;
    int64_t blocks = ceil_div(count, kBlock);
    if (blocks > 4096) blocks = 4096;
    k_fill_u32<<<dim3((unsigned)blocks), dim3(kBlock), 0, stream>>>(p, value, count);
    PR_LAUNCHED("fill");
    return PR_OK;
}

// ------------------------------------------------------------------- scan
//
// Tile = 256 lanes x 16 items.  Pass 1 sums each tile; the tile sums are
// scanned recursively; pass 2 rescans each tile with its offset.

constexpr int kScanItems = 16;
constexpr int64_t kScanTile = (int64_t)kBlock * kScanItems;

template <class T>
__global__ __launch_bounds__(kBlock) void k_scan_tile_sums(const T* __restrict__ in, int64_t N,
                                                           T* __restrict__ sums) {
    __shared__ T red[kWaves];
    const int64_t base = blockIdx.x * kScanTile;
    T v[kScanItems];
#pragma unroll
    for (int r = 0; r < kScanItems; ++r) {  // loads first, clamped: they overlap
        const int64_t i = base + r * kBlock + threadIdx.x;
        v[r] = in[i < N ? i : N - 1];
    }
    T s = 0;
#pragma unroll
    for (int r = 0; r < kScanItems; ++r) s += (base + r * kBlock + threadIdx.x < N) ? v[r] : (T)0;
    s = block_sum(s, red);
    if (threadIdx.x == 0) sums[blockIdx.x] = s;
}

template <class T>
__global__ __launch_bounds__(kBlock) void k_scan_tiles(const T* __restrict__ in, int64_t N,
                                                       const T* __restrict__ offsets,
                                                       T* __restrict__ out) {
    __shared__ T tmp[kWaves + 1];
    // A lane's items are contiguous: with both arrays 16-byte aligned (all of
    // the library's scratch is), a full lane moves them as 16-byte vectors.
    constexpr int kVec = kScanItems * (int)sizeof(T) / 16;
    const int64_t base = blockIdx.x * kScanTile + (int64_t)threadIdx.x * kScanItems;
    const bool wide = base + kScanItems <= N &&
                      ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15u) == 0;
    T v[kScanItems];
    T local = 0;
    if (wide) {
        uint4 q[kVec];
#pragma unroll
        for (int j = 0; j < kVec; ++j) q[j] = reinterpret_cast<const uint4*>(in + base)[j];
        __builtin_memcpy(v, q, sizeof v);
    } else {
#pragma unroll
        for (int j = 0; j < kScanItems; ++j) v[j] = base + j < N ? in[base + j] : (T)0;
    }
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) local += v[j];
    T total;
    T run = block_exclusive_scan(local, &total, tmp);
    if (offsets) run += offsets[blockIdx.x];
    T o[kScanItems];
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
        o[j] = run;
        run += v[j];
    }
    if (wide) {
        uint4 q[kVec];
        __builtin_memcpy(q, o, sizeof q);
#pragma unroll
        for (int j = 0; j < kVec; ++j) reinterpret_cast<uint4*>(out + base)[j] = q[j];
    } else {
#pragma unroll
        for (int j = 0; j < kScanItems; ++j)
            if (base + j < N) out[base + j] = o[j];
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == kBlock - 1) out[N] = run;
}

size_t scan_workspace_bytes(int64_t N) {
    int64_t tiles = ceil_div(N > 0 ? N : 1, kScanTile);
    if (tiles <= 1) return 256;
    return align_up(sizeof(uint64_t) * tiles) + align_up(sizeof(uint64_t) * (tiles + 1)) +
           scan_workspace_bytes(tiles);
}

template <class T>
int scan_impl(const T* in, T* out, int64_t N, void* ws, hipStream_t stream) {
    if (N <= 0) {
        k_fill_u32<<<1, kBlock, 0, stream>>>(reinterpret_cast<uint32_t*>(out), 0u,
                                            (int64_t)(sizeof(T) / 4));
        PR_LAUNCHED("scan fill");
        return PR_OK;
    }
    const int64_t tiles = ceil_div(N, kScanTile);
    if (tiles == 1) {
        k_scan_tiles<T><<<1, kBlock, 0, stream>>>(in, N, nullptr, out);
        PR_LAUNCHED("scan");
        return PR_OK;
    }
    // workspace laid out for 8-byte items whatever T is (see scan_workspace_bytes)
    char* base = static_cast<char*>(ws);
    T* sums = reinterpret_cast<T*>(base);
    T* offs = reinterpret_cast<T*>(base + align_up(sizeof(uint64_t) * tiles));
    void* rest = base + align_up(sizeof(uint64_t) * tiles) + align_up(sizeof(uint64_t) * (tiles + 1));
    k_scan_tile_sums<T><<<dim3((unsigned)tiles), kBlock, 0, stream>>>(in, N, sums);
    PR_LAUNCHED("scan sums");
    PR_TRY(scan_impl<T>(sums, offs, tiles, rest, stream));
    k_scan_tiles<T><<<dim3((unsigned)tiles), kBlock, 0, stream>>>(in, N, offs, out);
    PR_LAUNCHED("scan tiles");
    return PR_OK;
}

int scan_exclusive(const uint32_t* in, uint32_t* out, int64_t N, void* ws, hipStream_t stream) {
    return scan_impl<uint32_t>(in, out, N, ws, stream);
}

int scan_exclusive(const uint64_t* in, uint64_t* out, int64_t N, void* ws, hipStream_t stream) {
    return scan_impl<uint64_t>(in, out, N, ws, stream);
}

}  // namespace pr

extern "C" const char* pr_status_string(int status) {
    switch (status) {
        case PR_OK: return "PR_OK";
        case PR_ERR_ARG: return "PR_ERR_ARG: invalid argument";
        case PR_ERR_WORKSPACE: return "PR_ERR_WORKSPACE: workspace too small or misaligned";
        case PR_ERR_GRAPH: return "PR_ERR_GRAPH: malformed CSR";
        case PR_ERR_HIP: return "PR_ERR_HIP: HIP runtime error";
        default: return "unknown pr_status";
    }
}

extern "C" const char* pr_last_error(void) { return pr::g_last_error; }
