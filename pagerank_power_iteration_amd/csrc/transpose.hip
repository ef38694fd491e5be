// pr_transpose: in-edge CSR from out-edge CSR on the device.
//
// The Day 40 page ("One iteration, three shapes of work") transposes once on
// the host with a counting sort: a histogram of targets, a prefix sum, and a
// scatter.  Here the same three steps run on the GPU: the in-degree
// histogram scanned gives in_row_ptr, and the scatter is a stable LSD radix
// sort of (target, source) pairs by target, 8 bits per pass.  Edges enter in
// source order, so stability leaves every in-row sorted by source: the same
// array a sequential counting sort produces, bit for bit, independent of
// scheduling.
#include "radix.hpp"

namespace pr {

namespace {

int radix_passes(int32_t n) {
    uint32_t hi = (uint32_t)(n - 1);
    int bits = 0;
    while (hi) {
        ++bits;
        hi >>= 1;
    }
    int p = (bits + kRadixBits - 1) / kRadixBits;
    return p < 1 ? 1 : p;
}

struct TransposeWs {
    uint32_t* indeg;    // [n]
    uint32_t* hist;     // [256 * T]
    uint32_t* scanned;  // [256 * T + 1]
    int32_t* key_a;     // [nnz] ping-pong pairs
    int32_t* val_a;
    int32_t* key_b;
    int32_t* val_b;
    uint32_t* error;    // [1]
    void* scan_ws;
    size_t bytes;
};

TransposeWs carve(void* base, int32_t n, int64_t nnz) {
    TransposeWs w{};
    Carver c(base);
    const int64_t T = radix_tiles(nnz);
    const int passes = radix_passes(n);
    w.indeg = c.take<uint32_t>((size_t)n);
    w.hist = c.take<uint32_t>((size_t)(kRadixDigits * T));
    w.scanned = c.take<uint32_t>((size_t)(kRadixDigits * T + 1));
    if (passes > 1) {
        w.key_a = c.take<int32_t>((size_t)nnz);
        w.val_a = c.take<int32_t>((size_t)nnz);
    }
    if (passes > 2) {
        w.key_b = c.take<int32_t>((size_t)nnz);
        w.val_b = c.take<int32_t>((size_t)nnz);
    }
    w.error = c.take<uint32_t>(1);
    int64_t scan_n = kRadixDigits * T > (int64_t)n ? kRadixDigits * T : (int64_t)n;
    size_t sb = scan_workspace_bytes(scan_n);
    w.scan_ws = c.base ? c.base + c.used : nullptr;
    c.used += align_up(sb);
    w.bytes = c.used;
    return w;
}

// Checks of the out-edge CSR for PR_VALIDATE: row_ptr[0] == 0, non-decreasing,
// row_ptr[n] == nnz.  (Column range is checked by the histogram pass.)
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

int check_args(int32_t n, int64_t nnz) {
    if (n < 1) return fail(PR_ERR_ARG, "n must be >= 1 (got %d)", n);
    if (nnz < 0 || nnz > INT32_MAX)
        return fail(PR_ERR_ARG, "nnz must be in [0, INT32_MAX] (got %lld)", (long long)nnz);
    return PR_OK;
}

}  // namespace

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
    return carve(nullptr, n, nnz).bytes;
}

extern "C" int pr_transpose(int32_t n, int64_t nnz, const int32_t* out_row_ptr,
                            const int32_t* out_col_idx, int32_t* in_row_ptr, int32_t* in_col_idx,
                            void* ws, size_t ws_bytes, uint32_t flags, void* stream_v) {
    PR_TRY(check_args(n, nnz));
    if (flags & ~PR_VALIDATE) return fail(PR_ERR_ARG, "unknown flags 0x%x", flags);
    if (!out_row_ptr || !in_row_ptr || !ws || (nnz > 0 && (!out_col_idx || !in_col_idx)))
        return fail(PR_ERR_ARG, "null pointer argument");
    TransposeWs w = carve(ws, n, nnz);
    if (ws_bytes < w.bytes || (reinterpret_cast<uintptr_t>(ws) & 255u))
        return fail(PR_ERR_WORKSPACE, "transpose workspace needs %zu bytes at 256-byte alignment (got %zu)",
                    w.bytes, ws_bytes);
    hipStream_t stream = as_stream(stream_v);
    const bool validate = flags & PR_VALIDATE;

    PR_TRY(fill_u32(w.error, 0u, 1, stream));
    if (validate) {
        int64_t blocks = ceil_div((int64_t)n + 1, kBlock);
        k_check_row_ptr<<<dim3((unsigned)(blocks > 4096 ? 4096 : blocks)), kBlock, 0, stream>>>(
            out_row_ptr, n, nnz, w.error);
        PR_LAUNCHED("check row_ptr");
        // A malformed row_ptr would make the owner-row search meaningless:
        // report it before sorting.
        PR_TRY(read_error_word(w.error, stream, "pr_transpose"));
    }
    PR_TRY(fill_u32(w.indeg, 0u, n, stream));
    if (nnz == 0) {
        // No edges: every in-row is empty.
        return fill_u32(reinterpret_cast<uint32_t*>(in_row_ptr), 0u, (int64_t)n + 1, stream);
    }

    const int64_t T = radix_tiles(nnz);
    const int passes = radix_passes(n);
    RadixIn in{};
    in.count = nnz;
    in.n = n;
    in.error = w.error;

    for (int p = 0; p < passes; ++p) {
        const int shift = p * kRadixBits;
        const bool last = p == passes - 1;
        int32_t* kout = (p % 2 == 0) ? w.key_a : w.key_b;
        int32_t* vout = last ? in_col_idx : ((p % 2 == 0) ? w.val_a : w.val_b);
        if (p == 0) {
            in.keys = out_col_idx;
            in.vals = nullptr;
            in.row_ptr = out_row_ptr;
            k_radix_hist<kFromOutCsr><<<dim3((unsigned)T), kBlock, 0, stream>>>(in, shift, T, w.hist,
                                                                                w.indeg);
            PR_LAUNCHED("transpose histogram");
            // in_row_ptr = exclusive scan of the in-degrees (in_row_ptr[n] = nnz)
            PR_TRY(scan_exclusive(w.indeg, reinterpret_cast<uint32_t*>(in_row_ptr), n, w.scan_ws,
                                  stream));
        } else {
            k_radix_hist<kFromPairs><<<dim3((unsigned)T), kBlock, 0, stream>>>(in, shift, T, w.hist,
                                                                               nullptr);
            PR_LAUNCHED("radix histogram");
        }
        PR_TRY(scan_exclusive(w.hist, w.scanned, kRadixDigits * T, w.scan_ws, stream));
        if (p == 0) {
            if (last)
                k_radix_scatter<kFromOutCsr, true><<<dim3((unsigned)T), kBlock, 0, stream>>>(
                    in, shift, T, w.scanned, nullptr, vout);
            else
                k_radix_scatter<kFromOutCsr, false><<<dim3((unsigned)T), kBlock, 0, stream>>>(
                    in, shift, T, w.scanned, kout, vout);
        } else {
            if (last)
                k_radix_scatter<kFromPairs, true><<<dim3((unsigned)T), kBlock, 0, stream>>>(
                    in, shift, T, w.scanned, nullptr, vout);
            else
                k_radix_scatter<kFromPairs, false><<<dim3((unsigned)T), kBlock, 0, stream>>>(
                    in, shift, T, w.scanned, kout, vout);
        }
        PR_LAUNCHED("radix scatter");
        in.keys = kout;
        in.vals = vout;
    }
    if (validate) PR_TRY(read_error_word(w.error, stream, "pr_transpose"));
    return PR_OK;
}
