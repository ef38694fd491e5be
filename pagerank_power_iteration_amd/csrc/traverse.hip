// Breadth-first search and weakly connected components on an out-edge CSR.
//
// What is computed ("gpu-graph-study", sections "Traversal (BFS / WCC)" and
// "Traversal T4 -- degree-bucketed BFS / WCC"):
//   * BFS from one source over the out-edges: level[v] = edges on a shortest
//     directed path source -> v, or -1 when there is none;
//   * WCC, the components of the graph with edge directions ignored:
//     label[v] = the smallest vertex id of v's component (the fixed point of
//     the page's min-label propagation).
//
// Scheduling.  The page splits the vertices by degree into thread, warp and
// block tiers, re-splitting the BFS frontier on the device every level and
// syncing with the host to size each tier's grid.  Here, for 64-lane
// wavefronts and with no split pass and no per-level sizing sync:
//   * a wavefront takes 64 rows (frontier vertices for BFS, every vertex for
//     WCC).  Rows shorter than kHubMin edges are flattened: the wavefront scans
//     their lengths and walks the concatenated edge list 256 edges a round,
//     each lane finding its edge's row by a binary search over the scanned
//     lengths read across lanes, so every lane stays busy whatever the mix of
//     degrees and consecutive lanes read consecutive columns;
//   * longer rows (hubs) are cut into kHubChunk-edge chunks whose descriptors
//     are appended to a list, and a second kernel deals the chunks to
//     workgroups: the page's block tier, without a tail behind one hub.
// Both kernels read their work counts from device memory, so the host
// launches BFS levels in growing batches and reads the next frontier's size
// once per batch.
//
// BFS claims a vertex with a compare-and-swap on its level, as the page's
// kernels do with atomicCAS, and appends the claimed vertices to the next
// frontier with one atomic add per wavefront round.
//
// WCC does not propagate labels round by round (the page's form, whose
// round count grows with the diameter: 2046 levels on its grid).  It hooks
// trees in one pass over the edges: every vertex starts as its own root; for
// an edge (u, v) the roots of u and v are found by following parent links,
// and the larger root is linked under the smaller with a compare-and-swap
// that succeeds only while the larger is still a root, retrying from the new
// roots otherwise.  A parent is always smaller than its child, so every tree's
// root is its smallest vertex; after the pass every edge's ends share a tree,
// so each component is one tree and a final pass that replaces every parent
// by its root gives the smallest id of the component.
#include <algorithm>

#include "common.hpp"

namespace pr {
namespace {

constexpr int32_t kHubMin = 256;   // rows of at least this many edges go to the hub pass
constexpr int32_t kHubChunk = 2048;  // edges per hub chunk: 8 per lane of a workgroup
constexpr int kPerLane = 4;          // edges per lane per round
constexpr int kRowGrid = 2048;       // workgroups of the row and hub kernels (8 per CU)
constexpr int kFirstBatch = 4;       // BFS levels launched before the first frontier check
constexpr int kMaxBatch = 64;
static_assert(kHubChunk % (kBlock * kPerLane) == 0, "a hub chunk is whole rounds");

// One chunk of a hub row: edges [beg, end) of row `row`.
struct HubChunk {
    int32_t row, beg, end, pad;
};

struct TravState {
    uint32_t front[3];     // BFS frontier sizes, by level mod 3
    uint32_t err;          // PR_VALIDATE verdict
    uint32_t chunks[2];    // hub chunks appended, by level mod 2 (WCC: slot 0)
    uint32_t components;   // WCC: roots counted by the final pass
    int32_t depth;         // BFS: deepest level whose frontier was non-empty
    unsigned long long scanned;  // BFS: out-edges of the expanded vertices
    unsigned long long pad[3];
};

struct TravArgs {
    const int32_t* rp;
    const int32_t* ci;
    uint32_t nnz;
    uint32_t col_max;  // n - 1: columns are clamped to it
    int32_t n;
    int32_t level;     // BFS: the level whose frontier this launch expands
    int32_t* out;      // BFS: level[n]; WCC: label[n] (the parent links)
    const int32_t* queue;  // BFS: this level's frontier
    int32_t* next;         // BFS: the next level's frontier
    HubChunk* chunks;
    uint32_t chunk_cap;
    TravState* st;
};

// Edge range of row u, clamped into [0, nnz] so that a malformed row
// pointer cannot send a read outside col_idx.
__device__ __forceinline__ void row_range(const TravArgs& a, int32_t u, int32_t& s, int32_t& len) {
    const int32_t lim = (int32_t)a.nnz;
    const int32_t b = min(max(a.rp[u], 0), lim);
    const int32_t e = min(max(a.rp[u + 1], b), lim);
    s = b;
    len = e - b;
}

// Target of edge e (e is clamped into [0, nnz), columns into [0, n)).  Only
// called when nnz > 0.
__device__ __forceinline__ int32_t column(const TravArgs& a, int32_t e) {
    return (int32_t)min((uint32_t)a.ci[min((uint32_t)e, a.nnz - 1u)], a.col_max);
}

// Append the chunks of hub row u (edges [s, s + len)) to the chunk list of
// `slot`.  One lane per hub.
__device__ __forceinline__ void append_hub(const TravArgs& a, int slot, int32_t u, int32_t s,
                                           int32_t len) {
    const uint32_t c = (uint32_t)((len + kHubChunk - 1) / kHubChunk);
    const uint32_t first = atomicAdd(&a.st->chunks[slot], c);
    for (uint32_t k = 0; k < c; ++k) {
        if (first + k >= a.chunk_cap) break;  // cannot happen for a well-formed CSR
        HubChunk h;
        h.row = u;
        h.beg = s + (int32_t)k * kHubChunk;
        h.end = min(h.beg + kHubChunk, s + len);
        h.pad = 0;
        a.chunks[first + k] = h;
    }
}

// ------------------------------------------------------------------- BFS op

struct BfsOp {
    int32_t* level;
    int32_t next_level;
    int32_t* next;
    uint32_t* next_count;

    __device__ __forceinline__ int32_t prologue(int32_t) const { return 0; }

    // Claim the unvisited targets of up to kPerLane edges per lane and append
    // them to the next frontier.  Called by every lane of the wavefront.
    __device__ __forceinline__ void edges(const int32_t (&v)[kPerLane], const int32_t (&)[kPerLane],
                                          const bool (&ok)[kPerLane]) const {
        int32_t seen[kPerLane];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) seen[k] = ok[k] ? level[v[k]] : 0;
        bool won[kPerLane];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            // a stale read of -1 only costs a failed compare-and-swap
            won[k] = ok[k] && seen[k] == -1 && atomicCAS(&level[v[k]], -1, next_level) == -1;
        }
        uint64_t mask[kPerLane];
        uint32_t count = 0;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            mask[k] = __ballot(won[k]);
            count += (uint32_t)__popcll(mask[k]);
        }
        if (count == 0) return;  // wavefront-uniform
        uint32_t base = 0;
        if (lane_id() == 0) base = atomicAdd(next_count, count);
        base = __shfl(base, 0, kWave);
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            if (won[k]) next[base + lanes_below(mask[k])] = v[k];
            base += (uint32_t)__popcll(mask[k]);
        }
    }
};

// ------------------------------------------------------------------- WCC op

// Root of x's tree.  Each step also points x at its grandparent (path
// halving).  Links only ever point to smaller ids, so the walk ends; a stale
// read returns an older link, which is still an ancestor.
__device__ __forceinline__ int32_t find_root(int32_t* label, int32_t x) {
    while (true) {
        const int32_t p = label[x];
        if (p == x) return x;
        const int32_t g = label[p];
        if (g == p) return p;
        label[x] = g;
        x = g;
    }
}

// Merge the trees holding ru (an ancestor of the edge's source) and v.
__device__ __forceinline__ void hook(int32_t* label, int32_t ru, int32_t v) {
    int32_t rv = find_root(label, v);
    while (ru != rv) {
        const int32_t hi = max(ru, rv), lo = min(ru, rv);
        const int32_t old = atomicCAS(&label[hi], hi, lo);
        if (old == hi) return;
        // hi was linked under old < hi meanwhile: retry from the current roots;
        // the larger of the two strictly decreases, so this ends
        ru = find_root(label, old);
        rv = find_root(label, lo);
    }
}

struct WccOp {
    int32_t* label;

    __device__ __forceinline__ int32_t prologue(int32_t u) const {
        return u >= 0 ? find_root(label, u) : 0;
    }

    __device__ __forceinline__ void edges(const int32_t (&v)[kPerLane],
                                          const int32_t (&root)[kPerLane],
                                          const bool (&ok)[kPerLane]) const {
#pragma unroll
        for (int k = 0; k < kPerLane; ++k)
            if (ok[k]) hook(label, root[k], v[k]);
    }
};

// ------------------------------------------------------------ row walking

// The flattened walk over one wavefront's rows.  Lane l holds row `row` (or
// -1), its first edge `s`, its length `len` (0 for hubs and absent rows) and
// the op's per-row value `aux`.  Every lane of the wavefront calls this.
template <class Op>
__device__ __forceinline__ void walk_rows(const Op& op, const TravArgs& a, int32_t s, int32_t len,
                                          int32_t aux) {
    const int lane = lane_id();
    const int32_t incl = wave_inclusive_scan(len);
    const int32_t excl = incl - len;
    const int32_t total = __shfl(incl, kWave - 1, kWave);
    for (int32_t base = 0; base < total; base += kWave * kPerLane) {
        int32_t e[kPerLane], ax[kPerLane];
        bool ok[kPerLane];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const int32_t j = base + k * kWave + lane;
            // largest lane i with excl_i <= j: the row that edge j of the
            // concatenation belongs to (rows of length 0 are skipped over)
            int i = 0;
#pragma unroll
            for (int step = kWave / 2; step > 0; step >>= 1) {
                const int c = i + step;
                if (__shfl(excl, c, kWave) <= j) i = c;
            }
            // cross-lane reads in converged code only: a lane masked off at a
            // read does not supply its value to the others
            const int32_t first = __shfl(s, i, kWave);
            const int32_t before = __shfl(excl, i, kWave);
            ax[k] = __shfl(aux, i, kWave);
            ok[k] = j < total;
            e[k] = ok[k] ? first + (j - before) : 0;
        }
        int32_t v[kPerLane];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) v[k] = ok[k] ? column(a, e[k]) : 0;
        op.edges(v, ax, ok);
    }
}

// Rows [0, count): row i is rows[i], or i itself when rows is null.  Hub
// rows go to the chunk list of `slot`.  Returns the lane's share of the
// out-edges seen (hubs included).
template <class Op>
__device__ __forceinline__ uint64_t visit_rows(const Op& op, const TravArgs& a,
                                               const int32_t* rows, uint32_t count, int slot) {
    const int wave = threadIdx.x / kWave;
    const int64_t waves = (int64_t)gridDim.x * kWaves;
    uint64_t seen = 0;
    for (int64_t t = (int64_t)blockIdx.x * kWaves + wave; t * kWave < (int64_t)count; t += waves) {
        const int64_t i = t * kWave + lane_id();
        int32_t u = -1, s = 0, len = 0;
        if (i < (int64_t)count) {
            u = rows ? rows[i] : (int32_t)i;
            row_range(a, u, s, len);
            seen += (uint64_t)len;
            if (len >= kHubMin) {
                append_hub(a, slot, u, s, len);
                len = 0;
            }
        }
        const int32_t aux = op.prologue(len > 0 ? u : -1);
        walk_rows(op, a, s, len, aux);
    }
    return seen;
}

// The hub chunks of `slot`, dealt to workgroups round-robin.
template <class Op>
__device__ __forceinline__ void visit_hubs(const Op& op, const TravArgs& a, int slot) {
    const uint32_t count = min(a.st->chunks[slot], a.chunk_cap);
    for (uint32_t t = blockIdx.x; t < count; t += gridDim.x) {
        const HubChunk h = a.chunks[t];
        const int32_t aux = op.prologue(h.row);
        int32_t ax[kPerLane];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) ax[k] = aux;
#pragma unroll
        for (int r = 0; r < kHubChunk / (kBlock * kPerLane); ++r) {
            int32_t v[kPerLane];
            bool ok[kPerLane];
#pragma unroll
            for (int k = 0; k < kPerLane; ++k) {
                const int32_t e = h.beg + (r * kPerLane + k) * kBlock + (int32_t)threadIdx.x;
                ok[k] = e < h.end;
                v[k] = ok[k] ? column(a, e) : 0;
            }
            op.edges(v, ax, ok);
        }
    }
}

// ----------------------------------------------------------------- kernels

__global__ __launch_bounds__(kBlock) void k_bfs_init(int32_t* __restrict__ level, int32_t n,
                                                     int32_t source, int32_t* __restrict__ queue,
                                                     TravState* __restrict__ st) {
    for (int64_t v = blockIdx.x * (int64_t)kBlock + threadIdx.x; v < n;
         v += (int64_t)gridDim.x * kBlock)
        level[v] = v == source ? 0 : -1;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        queue[0] = source;
        st->front[0] = 1;
        st->front[1] = 0;
        st->front[2] = 0;
        st->chunks[0] = 0;
        st->chunks[1] = 0;
        st->depth = 0;
        st->scanned = 0;
    }
}

// Expand the frontier of level a.level: short rows here, hub rows listed for
// k_bfs_hubs.  A launch whose frontier is empty does nothing.
__global__ __launch_bounds__(kBlock) void k_bfs_rows(TravArgs a) {
    const int L = a.level;
    const uint32_t count = min(a.st->front[L % 3], (uint32_t)a.n);
    if (count == 0) return;
    if (blockIdx.x == 0 && threadIdx.x == 0) a.st->depth = L;
    BfsOp op{a.out, L + 1, a.next, &a.st->front[(L + 1) % 3]};
    uint64_t seen = visit_rows(op, a, a.queue, count, L % 2);
    seen = wave_sum(seen);
    if (lane_id() == 0 && seen) atomicAdd(&a.st->scanned, (unsigned long long)seen);
}

// Expand the hub chunks of level a.level, then clear the counters that
// level a.level + 1 appends to (its next frontier count and chunk count)
// after their last reader (level a.level - 1) is done.
__global__ __launch_bounds__(kBlock) void k_bfs_hubs(TravArgs a) {
    const int L = a.level;
    BfsOp op{a.out, L + 1, a.next, &a.st->front[(L + 1) % 3]};
    visit_hubs(op, a, L % 2);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.st->front[(L + 2) % 3] = 0;
        a.st->chunks[(L + 1) % 2] = 0;
    }
}

__global__ __launch_bounds__(kBlock) void k_wcc_init(int32_t* __restrict__ label, int32_t n,
                                                     TravState* __restrict__ st) {
    for (int64_t v = blockIdx.x * (int64_t)kBlock + threadIdx.x; v < n;
         v += (int64_t)gridDim.x * kBlock)
        label[v] = (int32_t)v;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st->chunks[0] = 0;
        st->components = 0;
    }
}

__global__ __launch_bounds__(kBlock) void k_wcc_rows(TravArgs a) {
    WccOp op{a.out};
    visit_rows(op, a, nullptr, (uint32_t)a.n, 0);
}

__global__ __launch_bounds__(kBlock) void k_wcc_hubs(TravArgs a) {
    WccOp op{a.out};
    visit_hubs(op, a, 0);
}

// Replace every link by its root and count the roots.  Concurrent writers
// only ever store roots, so every read is an ancestor.
__global__ __launch_bounds__(kBlock) void k_wcc_compress(int32_t* __restrict__ label, int32_t n,
                                                         TravState* __restrict__ st) {
    __shared__ uint32_t red[kWaves];
    uint32_t roots = 0;
    for (int64_t v = blockIdx.x * (int64_t)kBlock + threadIdx.x; v < n;
         v += (int64_t)gridDim.x * kBlock) {
        int32_t x = label[v];
        while (true) {
            const int32_t p = label[x];
            if (p == x) break;
            x = p;
        }
        label[v] = x;
        roots += x == (int32_t)v ? 1u : 0u;
    }
    roots = block_sum(roots, red);
    if (threadIdx.x == 0 && roots) atomicAdd(&st->components, roots);
}

__global__ __launch_bounds__(kBlock) void k_trav_check_cols(const int32_t* __restrict__ ci,
                                                           int64_t nnz, int32_t n,
                                                           uint32_t* __restrict__ err) {
    for (int64_t j = blockIdx.x * (int64_t)kBlock + threadIdx.x; j < nnz;
         j += (int64_t)gridDim.x * kBlock)
        if ((uint32_t)ci[j] >= (uint32_t)n) *err = 1u;
}

// ------------------------------------------------------------------ host

unsigned vertex_grid(int64_t items) {
    const int64_t g = ceil_div(items > 0 ? items : 1, kBlock);
    return (unsigned)(g < 4096 ? g : 4096);
}

// Hub chunks one pass can list: sum over rows of at least kHubMin edges of
// ceil(len / kHubChunk) <= nnz / kHubChunk + nnz / kHubMin.
uint32_t chunk_capacity(int64_t nnz) {
    return (uint32_t)(nnz / kHubChunk + nnz / kHubMin + 1);
}

struct TravWs {
    TravState* st;
    int32_t* queue[2];
    HubChunk* chunks;
    size_t bytes;
};

TravWs carve(void* base, int32_t n, int64_t nnz, bool queues) {
    Carver c(base);
    TravWs w{};
    w.st = c.take<TravState>(1);
    if (queues) {
        w.queue[0] = c.take<int32_t>(n);
        w.queue[1] = c.take<int32_t>(n);
    }
    w.chunks = c.take<HubChunk>(chunk_capacity(nnz));
    w.bytes = c.used;
    return w;
}

int check_graph(int32_t n, int64_t nnz, const int32_t* rp, const int32_t* ci) {
    if (n < 1) return fail(PR_ERR_ARG, "n must be >= 1 (got %d)", n);
    if (nnz < 0 || nnz > INT32_MAX)
        return fail(PR_ERR_ARG, "nnz must be in [0, INT32_MAX] (got %lld)", (long long)nnz);
    if (!rp || (nnz > 0 && !ci)) return fail(PR_ERR_ARG, "null pointer argument");
    return PR_OK;
}

int check_ws(const TravWs& w, void* ws, size_t ws_bytes, const char* what) {
    if (!ws) return fail(PR_ERR_ARG, "%s: workspace is null", what);
    if (ws_bytes < w.bytes || (reinterpret_cast<uintptr_t>(ws) & 255u))
        return fail(PR_ERR_WORKSPACE, "%s needs %zu workspace bytes at 256-byte alignment (got %zu)",
                    what, w.bytes, ws_bytes);
    return PR_OK;
}

int validate(int32_t n, int64_t nnz, const int32_t* rp, const int32_t* ci, TravState* st,
             hipStream_t stream, const char* what) {
    uint32_t* err = &st->err;
    PR_TRY(fill_u32(err, 0u, 1, stream));
    PR_TRY(check_out_row_ptr(rp, n, nnz, err, stream));
    if (nnz > 0) {
        k_trav_check_cols<<<vertex_grid(nnz), kBlock, 0, stream>>>(ci, nnz, n, err);
        PR_LAUNCHED("check columns");
    }
    return read_error_word(err, stream, what);
}

TravArgs make_args(int32_t n, int64_t nnz, const int32_t* rp, const int32_t* ci, int32_t* out,
                   const TravWs& w) {
    TravArgs a{};
    a.rp = rp;
    a.ci = ci;
    a.nnz = (uint32_t)nnz;
    a.col_max = (uint32_t)(n - 1);
    a.n = n;
    a.out = out;
    a.chunks = w.chunks;
    a.chunk_cap = chunk_capacity(nnz);
    a.st = w.st;
    return a;
}

}  // namespace
}  // namespace pr

using namespace pr;

extern "C" size_t pr_bfs_workspace_bytes(int32_t n, int64_t nnz) {
    if (n < 1 || nnz < 0 || nnz > INT32_MAX) return 0;
    return carve(nullptr, n, nnz, true).bytes;
}

extern "C" size_t pr_wcc_workspace_bytes(int32_t n, int64_t nnz) {
    if (n < 1 || nnz < 0 || nnz > INT32_MAX) return 0;
    return carve(nullptr, n, nnz, false).bytes;
}

extern "C" int pr_bfs(int32_t n, int64_t nnz, const int32_t* rp, const int32_t* ci, int32_t source,
                      int32_t* level, int32_t* depth_host, int64_t* edges_scanned_host, void* ws,
                      size_t ws_bytes, uint32_t flags, void* stream_v) {
    PR_TRY(check_graph(n, nnz, rp, ci));
    if (!level) return fail(PR_ERR_ARG, "level is null");
    if (source < 0 || source >= n)
        return fail(PR_ERR_ARG, "source %d is not a vertex of a %d-vertex graph", source, n);
    if (flags & ~PR_VALIDATE) return fail(PR_ERR_ARG, "unknown flags 0x%x", flags);
    const TravWs w = carve(ws, n, nnz, true);
    PR_TRY(check_ws(w, ws, ws_bytes, "pr_bfs"));
    hipStream_t stream = as_stream(stream_v);
    if (flags & PR_VALIDATE) PR_TRY(validate(n, nnz, rp, ci, w.st, stream, "pr_bfs"));

    k_bfs_init<<<vertex_grid(n), kBlock, 0, stream>>>(level, n, source, w.queue[0], w.st);
    PR_LAUNCHED("bfs init");
    TravArgs a = make_args(n, nnz, rp, ci, level, w);
    TravState h{};
    int32_t L = 0;
    int batch = kFirstBatch;
    // A frontier holds at least one vertex, so at most n levels are non-empty.
    while (L <= n) {
        for (int k = 0; k < batch; ++k, ++L) {
            a.level = L;
            a.queue = w.queue[L % 2];
            a.next = w.queue[(L + 1) % 2];
            k_bfs_rows<<<kRowGrid, kBlock, 0, stream>>>(a);
            PR_LAUNCHED("bfs rows");
            k_bfs_hubs<<<kRowGrid, kBlock, 0, stream>>>(a);
            PR_LAUNCHED("bfs hubs");
        }
        PR_HIP_TRY(hipMemcpyAsync(&h, w.st, sizeof h, hipMemcpyDeviceToHost, stream));
        PR_HIP_TRY(hipStreamSynchronize(stream));
        if (h.front[L % 3] == 0) break;  // the frontier of level L is empty
        batch = std::min(batch * 2, kMaxBatch);
    }
    if (depth_host) *depth_host = h.depth;
    if (edges_scanned_host) *edges_scanned_host = (int64_t)h.scanned;
    return PR_OK;
}

extern "C" int pr_wcc(int32_t n, int64_t nnz, const int32_t* rp, const int32_t* ci, int32_t* label,
                      int32_t* n_components_host, void* ws, size_t ws_bytes, uint32_t flags,
                      void* stream_v) {
    PR_TRY(check_graph(n, nnz, rp, ci));
    if (!label) return fail(PR_ERR_ARG, "label is null");
    if (flags & ~PR_VALIDATE) return fail(PR_ERR_ARG, "unknown flags 0x%x", flags);
    const TravWs w = carve(ws, n, nnz, false);
    PR_TRY(check_ws(w, ws, ws_bytes, "pr_wcc"));
    hipStream_t stream = as_stream(stream_v);
    if (flags & PR_VALIDATE) PR_TRY(validate(n, nnz, rp, ci, w.st, stream, "pr_wcc"));

    k_wcc_init<<<vertex_grid(n), kBlock, 0, stream>>>(label, n, w.st);
    PR_LAUNCHED("wcc init");
    const TravArgs a = make_args(n, nnz, rp, ci, label, w);
    k_wcc_rows<<<kRowGrid, kBlock, 0, stream>>>(a);
    PR_LAUNCHED("wcc rows");
    k_wcc_hubs<<<kRowGrid, kBlock, 0, stream>>>(a);
    PR_LAUNCHED("wcc hubs");
    k_wcc_compress<<<vertex_grid(n), kBlock, 0, stream>>>(label, n, w.st);
    PR_LAUNCHED("wcc compress");
    if (n_components_host) {
        uint32_t c = 0;
        PR_HIP_TRY(hipMemcpyAsync(&c, &w.st->components, sizeof c, hipMemcpyDeviceToHost, stream));
        PR_HIP_TRY(hipStreamSynchronize(stream));
        *n_components_host = (int32_t)c;
    }
    return PR_OK;
}
