// Device transpose shared by pr_transpose and the plan builder.
#pragma once

#include "radix.hpp"

namespace pr {

struct TransposeWs {
    RadixWs sort;
    int32_t* tile_row;  // [radix_tiles(nnz) + 1] the first pass's row range per tile
    uint32_t* error;    // [1]
    size_t bytes;
};

TransposeWs transpose_carve(void* base, int32_t n, int64_t nnz);

// In-edge CSR of the out-edge CSR (n, nnz, out_rp, out_ci): a stable LSD
// sort of (target, source) pairs by target; in_rp from the row boundaries of
// the sorted targets.  Asynchronous on `stream`.  Out-of-range columns are
// clamped and flagged in ws.error.
int transpose_device(int32_t n, int64_t nnz, const int32_t* out_rp, const int32_t* out_ci,
                     int32_t* in_rp, int32_t* in_ci, const TransposeWs& ws, hipStream_t stream);

// Row pointers of the in-edge CSR alone (in_rp[v+1] - in_rp[v] = in-degree
// of v), from a keys-only radix sort of the targets.  Out-of-range targets are
// clamped and flagged in ws.error.  Asynchronous on `stream`.
int transpose_row_ptr(int32_t n, int64_t nnz, const int32_t* out_ci, int32_t* in_rp,
                      const TransposeWs& ws, hipStream_t stream);

// win_row[t] = the row of the CSR row pointers rp[0..n] that owns position
// t * kRadixTile, for t < T, and win_row[T] = n - 1: rows [win_row[t],
// win_row[t + 1]] hold every position of window t.  One binary search per
// window, all side by side.  Asynchronous on `stream`.
int window_rows(const int32_t* rp, int32_t n, int64_t T, int32_t* win_row, hipStream_t stream);

// Bits needed to hold every vertex id in [0, n).
int vertex_bits(int32_t n);

}  // namespace pr
