// Internal helpers shared by the libpr translation units: status handling,
// workspace carving, and the wavefront/workgroup primitives every kernel uses.
// gfx950 runs 64-lane wavefronts; kernels are launched with 256-lane
// workgroups (4 wavefronts) unless their launch bounds say otherwise.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pr.h"

namespace pr {

constexpr int kBlock = 256;
constexpr int kWave = 64;
constexpr int kWaves = kBlock / kWave;

// ------------------------------------------------------------------ errors

// Record a message for pr_last_error() and return `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

#define PR_HIP_TRY(expr)                                                                   \
    do {                                                                                   \
        hipError_t pr_e_ = (expr);                                                         \
        if (pr_e_ != hipSuccess)                                                           \
            return ::pr::fail(PR_ERR_HIP, "%s: %s (%s:%d)", #expr, hipGetErrorString(pr_e_), \
                              __FILE__, __LINE__);                                         \
    } while (0)

#define PR_LAUNCHED(what) PR_HIP_TRY(hipPeekAtLastError())

#define PR_TRY(expr)              \
    do {                          \
        int pr_s_ = (expr);       \
        if (pr_s_ != PR_OK) return pr_s_; \
    } while (0)

// -------------------------------------------------------------- workspace

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// Hands out 256-byte aligned slices of one caller-provided buffer.  With a
// null base it only measures (used by the *_workspace_bytes queries).
struct Carver {
    char* base;
    size_t used = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <class T>
    T* take(size_t count) {
        size_t off = used;
        used = align_up(used + sizeof(T) * (count > 0 ? count : 1));
        return base ? reinterpret_cast<T*>(base + off) : nullptr;
    }
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ------------------------------------------------------- device primitives

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Count of set bits of `mask` in lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

template <class T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Sum over aligned groups of G lanes (G a power of two <= 64); every lane of
// the group receives the group's total.
template <int G, class T>
__device__ __forceinline__ T group_sum(T v) {
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

template <class T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        T t = __shfl_up(v, off, kWave);
        if (lane >= off) v += t;
    }
    return v;
}

// Workgroup-wide exclusive scan of one value per lane, for workgroups of W
// wavefronts; `scratch` holds at least W + 1 entries of LDS.  Returns the
// exclusive prefix and stores the workgroup total in *total.  Contains
// barriers: call from every lane.
template <class T, int W = kWaves>
__device__ __forceinline__ T block_exclusive_scan(T v, T* total, T* scratch) {
    const int wave = threadIdx.x / kWave;
    T incl = wave_inclusive_scan(v);
    if (lane_id() == kWave - 1) scratch[wave] = incl;
    __syncthreads();
    if constexpr (W > 8) {  // many wavefronts: wavefront 0 scans their totals
        static_assert(W <= kWave, "one lane per wavefront total");
        if (wave == 0) {
            const int l = lane_id();
            const T c = l < W ? scratch[l] : (T)0;
            const T in = wave_inclusive_scan(c);
            if (l < W) scratch[l] = in - c;
            if (l == W - 1) scratch[W] = in;
        }
    } else if (threadIdx.x == 0) {
        T run = 0;
        for (int w = 0; w < W; ++w) {
            T c = scratch[w];
            scratch[w] = run;
            run += c;
        }
        scratch[W] = run;
    }
    __syncthreads();
    T out = scratch[wave] + incl - v;
    *total = scratch[W];
    __syncthreads();
    return out;
}

// Workgroup sum for workgroups of W wavefronts; the result is valid in every
// lane.  `scratch` holds at least W entries of LDS.  Contains barriers.
template <class T, int W = kWaves>
__device__ __forceinline__ T block_sum(T v, T* scratch) {
    v = wave_sum(v);
    if (lane_id() == 0) scratch[threadIdx.x / kWave] = v;
    __syncthreads();
    T r = scratch[0];
#pragma unroll
    for (int w = 1; w < W; ++w) r += scratch[w];
    __syncthreads();
    return r;
}

// ----------------------------------------------------------- host helpers

// Device-wide exclusive scan: out[i] = sum in[0..i) for i in [0, N]; out[N]
// is the total.  uint32 (totals must fit) and uint64 instantiations.
size_t scan_workspace_bytes(int64_t N);
int scan_exclusive(const uint32_t* in, uint32_t* out, int64_t N, void* ws, hipStream_t stream);
int scan_exclusive(const uint64_t* in, uint64_t* out, int64_t N, void* ws, hipStream_t stream);

// Fill `count` 32-bit words with `value` (a kernel, so it is safe under
// stream capture).
int fill_u32(uint32_t* p, uint32_t value, int64_t count, hipStream_t stream);

// Copy a device error word to the host (synchronizing `stream`); PR_ERR_GRAPH
// when it is non-zero.
int read_error_word(const uint32_t* err_dev, hipStream_t stream, const char* what);

// PR_VALIDATE check of an out-edge row-pointer array; sets *err on failure.
int check_out_row_ptr(const int32_t* rp, int32_t n, int64_t nnz, uint32_t* err, hipStream_t stream);

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace pr
