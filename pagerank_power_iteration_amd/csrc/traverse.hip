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
// Row scheduling.  The page splits the vertices by degree into thread, warp
// and block tiers, re-splitting the BFS frontier on the device every level
// and syncing with the host to size each tier's grid.  Here, for 64-lane
// wavefronts and with no split pass and no per-level sizing sync:
//   * a wavefront takes 64 rows.  Rows shorter than kHubMin edges are
//     flattened: the wavefront scans their lengths and walks the
//     concatenated edge list 256 edges a round, each lane finding its edge's
//     row by a binary search over the scanned lengths read across lanes, so
//     every lane stays busy whatever the mix of degrees and consecutive lanes
//     read consecutive columns;
//   * longer rows (hubs) are cut into kHubChunk-edge chunks whose descriptors
//     are appended to a list, and a second kernel deals the chunks to
//     workgroups: the page's block tier, without a tail behind one hub.
// Both kernels read their work counts from device memory, so the host
// launches BFS levels in growing batches and reads the frontier's size once
// per batch.  A run of narrow levels (a frontier of at most 2048 vertices and
// 65,536 out-edges) runs instead in one launch of one workgroup, level after
// level, until the frontier grows or empties: on a high-diameter graph the
// two launches per level would be all the time spent.
//
// BFS direction.  A level is expanded top-down (the frontier's out-edges; a
// vertex is claimed with a compare-and-swap on its level, as the page's
// kernels do with atomicCAS) or, when the caller supplies the in-edge CSR and
// the frontier is large, bottom-up: every unvisited vertex looks through its
// in-edges for a parent on the current level and sets its own level, with no
// atomic on the level array.  The choice follows the direction-optimizing
// rule of Beamer, Asanovic and Patterson (SC 2012), which the graph study
// mentions, beside CPU/GPU hybrids, as the known answer where its own tiers
// lose to the CPU: go bottom-up when the
// frontier's out-edges exceed 1/14 of the edges not yet explored, and back
// top-down when the frontier holds fewer than n/24 vertices.  Every kernel of
// a level evaluates the rule from counters the previous level left, so all
// of them agree without a host round trip.
//
// WCC does not propagate labels round by round (the page's form, whose round
// count grows with the diameter: 2046 levels on its grid).  It links trees:
// every vertex starts as its own root; for an edge (u, v) the roots of u and
// v are found by following parent links, and the larger root is linked under
// the smaller with a compare-and-swap that succeeds only while the larger is
// still a root, retrying from the new roots otherwise.  A parent is always
// smaller than its child, so every tree's root is its smallest vertex; once
// every edge's ends share a tree, each component is one tree and pointing
// every vertex at its root gives the smallest id of the component.  The
// order follows Afforest (Sutton, Ben-Nun and Barak, IPDPS 2018): first one
// neighbour per vertex (its first out-edge; with the in-edge CSR, the smaller
// of its first out- and in-neighbour, linked without an atomic because each
// vertex writes only its own link), then its second out-edge, each round
// followed by compression; then the root most of 1024 sampled vertices share
// (the giant component) is found, and the full pass skips every vertex
// already in its tree.  Skipping
// a vertex's out-edges is only safe when its in-edges are seen from the
// other side, so without the in-edge CSR no vertex is skipped.
#include <algorithm>

#include "common.hpp"

namespace pr {
namespace {

constexpr int32_t kHubMin = 256;     // rows of at least this many edges go to the hub pass
constexpr int32_t kHubChunk = 2048;  // edges per hub chunk: 8 per lane of a workgroup
constexpr int kPerLane = 4;          // edges per lane per round
constexpr int kRowGrid = 2048;       // workgroups of the row and hub kernels (8 per CU)
constexpr int kFirstBatch = 8;       // BFS levels launched before the first frontier check
constexpr int kMaxBatch = 64;
constexpr int kTopDown = 0, kBottomUp = 1;
constexpr uint64_t kAlpha = 14, kBeta = 24;  // direction-switch ratios
constexpr int32_t kSampledEdges = 2;         // WCC without in-edges: out-edges linked first
constexpr int kGiantSamples = 1024;          // WCC: vertices sampled for the giant root
constexpr uint32_t kQueueBuf = 512;          // LDS entries per wavefront staging claimed vertices
constexpr int32_t kProbe = 4;                // in-edges a lane checks itself before a bottom-up walk
constexpr int kSmallBlock = 1024;            // lanes of the small-frontier kernel
constexpr int32_t kSmallCap = 2048;          // frontier rows it keeps in LDS
constexpr uint64_t kSmallEdges = 65536;      // frontier out-edges it takes per level
// Graphs of at most kBitVerts vertices run narrow levels with a visited
// bitmap in LDS (128 KB) and a frontier of at most kSmallBitCap rows.
constexpr int32_t kBitVerts = 1 << 20;
constexpr int32_t kSmallBitCap = 1536;
constexpr int kSmallBatch = 4;               // consecutive edges a lane takes
static_assert(kHubChunk % (kBlock * kPerLane) == 0, "a hub chunk is whole rounds");
static_assert(kGiantSamples <= 1024 && kGiantSamples % kWave == 0, "one sample per lane");

// One chunk of a hub row: edges [beg, end) of row `row`.
struct HubChunk {
    int32_t row, beg, end, pad;
};

struct TravState {
    uint32_t front[3];               // BFS frontier sizes, by level mod 3
    uint32_t err;                    // PR_VALIDATE verdict
    uint32_t chunks[2];              // hub chunks appended, by level mod 2 (WCC: by pass)
    uint32_t components;             // WCC: roots counted by the final pass
    int32_t depth;                   // BFS: deepest level whose frontier was non-empty
    unsigned long long mf[3];        // BFS: out-degree sum of a level's frontier, by level mod 3
    unsigned long long explored[2];  // BFS: out-degree sum of the levels below L, by L mod 2
    int32_t mode[2];                 // BFS: direction of level L, by L mod 2
    int32_t giant;                   // WCC: the root the full pass skips (-1: none)
    int32_t small_next;              // BFS: the level a small-frontier run stopped at
};

struct TravArgs {
    const int32_t* rp;     // the CSR a row pass walks (out-edges, or in-edges)
    const int32_t* ci;
    const int32_t* out_rp;  // out-degrees, for the BFS frontier's edge count
    const int32_t* in_rp;   // in-edge CSR, or null
    const int32_t* in_ci;
    uint32_t nnz;
    uint32_t col_max;  // n - 1: columns are clamped to it
    int32_t n;
    int32_t level;     // BFS: the level this launch expands
    int32_t skip;      // WCC: edges skipped at the start of every row
    int32_t* out;      // BFS: level[n]; WCC: label[n] (the parent links)
    const int32_t* queue;  // BFS: this level's frontier
    int32_t* next;         // BFS: the next level's frontier
    HubChunk* chunks;
    uint32_t chunk_cap;
    TravState* st;
};

// Edge range of row u of (rp, nnz), clamped into [0, nnz] so that a
// malformed row pointer cannot send a read outside the column array.
__device__ __forceinline__ void row_range(const int32_t* __restrict__ rp, uint32_t nnz, int32_t u,
                                          int32_t& s, int32_t& len) {
    const int32_t lim = (int32_t)nnz;
    const int32_t b = min(max(rp[u], 0), lim);
    const int32_t e = min(max(rp[u + 1], b), lim);
    s = b;
    len = e - b;
}

// Target of edge e (e is clamped into [0, nnz), columns into [0, n)).  Only
// called when nnz > 0.
__device__ __forceinline__ int32_t column(const TravArgs& a, int32_t e) {
    return (int32_t)min((uint32_t)a.ci[min((uint32_t)e, a.nnz - 1u)], a.col_max);
}

// Append the chunks of the hub rows a wavefront holds (lane l: row u, edges
// [s, s + len), when `hub` is set) to the chunk list of `slot`, with one
// atomic add per wavefront: a counter that every wavefront bumps once per
// row would serialize them.  Every lane calls this.
__device__ __forceinline__ void append_hubs(const TravArgs& a, int slot, bool hub, int32_t u,
                                            int32_t s, int32_t len) {
    const uint32_t c = hub ? (uint32_t)((len + kHubChunk - 1) / kHubChunk) : 0u;
    const uint32_t incl = wave_inclusive_scan(c);
    const uint32_t total = __shfl(incl, kWave - 1, kWave);
    if (total == 0) return;  // wavefront-uniform
    uint32_t base = 0;
    if (lane_id() == 0) base = atomicAdd(&a.st->chunks[slot], total);
    base = __shfl(base, 0, kWave);
    const uint32_t first = base + incl - c;
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

__device__ __forceinline__ uint64_t wave_or(uint64_t v) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v |= __shfl_xor(v, off, kWave);
    return v;
}

// ------------------------------------------------------------ row walking

// The flattened walk over one wavefront's rows of (a.rp, a.ci).  Lane l holds
// its row's first edge `s`, its length `len` (0 for hubs, skipped and absent
// rows) and the op's per-row value `aux`.  Edges of rows for which
// op.active(lane) is false are not loaded.  Every lane of the wavefront calls
// this, and op.edges is called by every lane.
template <class Op>
__device__ __forceinline__ void walk_rows(Op& op, const TravArgs& a, int32_t s, int32_t len,
                                          int32_t aux) {
    const int lane = lane_id();
    const int32_t incl = wave_inclusive_scan(len);
    const int32_t excl = incl - len;
    const int32_t total = __shfl(incl, kWave - 1, kWave);
    for (int32_t base = 0; base < total; base += kWave * kPerLane) {
        int32_t e[kPerLane], ax[kPerLane], own[kPerLane];
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
            own[k] = i;
            ok[k] = j < total && op.active(i);
            e[k] = ok[k] ? first + (j - before) : 0;
        }
        int32_t v[kPerLane];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) v[k] = ok[k] ? column(a, e[k]) : 0;
        op.edges(v, ax, own, ok);
    }
}

// ---------------------------------------------------------------- BFS rule

// Direction of level L, from what the levels before it left in the state:
// the direction of level L-1, the size and out-degree sum of level L's
// frontier, and the out-degree sum of the levels below L.  Every launch of
// a level computes the same value (none of these fields changes during the
// level).
__device__ __forceinline__ int bfs_mode(const TravArgs& a, int L) {
    if (!a.in_rp || L == 0) return kTopDown;
    const TravState* st = a.st;
    const uint64_t nf = st->front[L % 3];
    const uint64_t mf = st->mf[L % 3];
    const uint64_t done = st->explored[L % 2] + mf;
    const uint64_t unexplored = (uint64_t)a.nnz > done ? (uint64_t)a.nnz - done : 0;
    if (st->mode[(L - 1) % 2] == kTopDown) return mf * kAlpha > unexplored ? kBottomUp : kTopDown;
    return nf * kBeta < (uint64_t)a.n ? kTopDown : kBottomUp;
}

__device__ __forceinline__ int32_t out_degree(const int32_t* __restrict__ out_rp, uint32_t nnz,
                                              int32_t v) {
    int32_t s, len;
    row_range(out_rp, nnz, v, s, len);
    return len;
}

// A wavefront's staging of claimed vertices in LDS.  The next frontier's
// counter is bumped once per flush (every 256 or more vertices), not once per
// round: many wavefronts adding to one address serialize.
struct QueueWriter {
    int32_t* buf;     // this wavefront's kQueueBuf entries of LDS
    int32_t* next;    // the next frontier
    uint32_t* count;  // its size
    uint32_t fill;    // entries staged (wavefront-uniform)

    // Stage v for every lane with `take`.  Every lane calls this.
    __device__ __forceinline__ void push(bool take, int32_t v) {
        const uint64_t m = __ballot(take);
        if (take) buf[fill + lanes_below(m)] = v;
        fill += (uint32_t)__popcll(m);
    }

    // Copy the staged entries out once at least `at_least` are staged.  LDS
    // operations of one wavefront complete in order, so the lanes read what
    // the others wrote.  Every lane calls this.
    __device__ __forceinline__ void flush(uint32_t at_least) {
        if (fill == 0 || fill < at_least) return;  // wavefront-uniform
        __builtin_amdgcn_wave_barrier();
        uint32_t base = 0;
        if (lane_id() == 0) base = atomicAdd(count, fill);
        base = __shfl(base, 0, kWave);
        for (uint32_t k = lane_id(); k < fill; k += kWave) next[base + k] = buf[k];
        __builtin_amdgcn_wave_barrier();
        fill = 0;
    }
};

// Top-down: claim the unvisited targets of up to kPerLane edges per lane,
// stage them for the next frontier and add their out-degrees to this lane's
// share of its edge count (`edges`, reduced once per workgroup).
struct TopDownOp {
    int32_t* level;
    const int32_t* out_rp;
    uint32_t nnz;
    int32_t next_level;
    QueueWriter q;
    uint64_t edges_seen;

    __device__ __forceinline__ TopDownOp(const TravArgs& a, int L, int32_t* lds)
        : level(a.out), out_rp(a.out_rp), nnz(a.nnz), next_level(L + 1),
          q{lds, a.next, &a.st->front[(L + 1) % 3], 0u}, edges_seen(0) {}

    __device__ __forceinline__ bool active(int) const { return true; }

    __device__ __forceinline__ void edges(const int32_t (&v)[kPerLane], const int32_t (&)[kPerLane],
                                          const int32_t (&)[kPerLane], const bool (&ok)[kPerLane]) {
        int32_t seen[kPerLane];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) seen[k] = ok[k] ? level[v[k]] : 0;
        bool won[kPerLane];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            // a stale read of -1 only costs a failed compare-and-swap
            won[k] = ok[k] && seen[k] == -1 && atomicCAS(&level[v[k]], -1, next_level) == -1;
        }
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            q.push(won[k], v[k]);
            if (won[k]) edges_seen += (uint64_t)out_degree(out_rp, nnz, v[k]);
        }
        q.flush(kQueueBuf - kWave * kPerLane);
    }

    // Flush what is staged and add the workgroup's edge count.  Every lane of
    // the workgroup calls this.
    __device__ __forceinline__ void finish(unsigned long long* next_edges, uint64_t* red) {
        q.flush(1);
        const uint64_t e = block_sum(edges_seen, red);
        if (threadIdx.x == 0 && e) atomicAdd(next_edges, (unsigned long long)e);
    }
};

// Bottom-up: the wavefront's 64 candidate vertices look through their
// in-edges for a source on the current level; bit l of `found` is set once
// lane l's vertex has one, and its remaining in-edges are not loaded.
struct BottomUpOp {
    const int32_t* level;
    int32_t current;
    uint64_t found;

    __device__ __forceinline__ bool active(int owner) const { return !((found >> owner) & 1u); }

    __device__ __forceinline__ void edges(const int32_t (&w)[kPerLane], const int32_t (&)[kPerLane],
                                          const int32_t (&own)[kPerLane], const bool (&ok)[kPerLane]) {
        int32_t lv[kPerLane];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) lv[k] = ok[k] ? level[w[k]] : -1;
        uint64_t bits = 0;
#pragma unroll
        for (int k = 0; k < kPerLane; ++k)
            if (lv[k] == current) bits |= 1ull << own[k];
        found |= wave_or(bits);
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

    __device__ __forceinline__ bool active(int) const { return true; }

    __device__ __forceinline__ int32_t prologue(int32_t u) const {
        return u >= 0 ? find_root(label, u) : 0;
    }

    __device__ __forceinline__ void edges(const int32_t (&v)[kPerLane],
                                          const int32_t (&root)[kPerLane], const int32_t (&)[kPerLane],
                                          const bool (&ok)[kPerLane]) const {
#pragma unroll
        for (int k = 0; k < kPerLane; ++k)
            if (ok[k]) hook(label, root[k], v[k]);
    }
};

// ----------------------------------------------------------------- kernels

__global__ __launch_bounds__(kBlock) void k_bfs_init(TravArgs a, int32_t source) {
    for (int64_t v = blockIdx.x * (int64_t)kBlock + threadIdx.x; v < a.n;
         v += (int64_t)gridDim.x * kBlock)
        a.out[v] = v == source ? 0 : -1;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        TravState* st = a.st;
        const_cast<int32_t*>(a.queue)[0] = source;
        st->front[0] = 1;
        st->front[1] = 0;
        st->front[2] = 0;
        st->mf[0] = (unsigned long long)out_degree(a.out_rp, a.nnz, source);
        st->mf[1] = 0;
        st->mf[2] = 0;
        st->explored[0] = 0;
        st->explored[1] = 0;
        st->mode[0] = kTopDown;
        st->mode[1] = kTopDown;
        st->chunks[0] = 0;
        st->chunks[1] = 0;
        st->depth = 0;
    }
}

// Level a.level: short rows here (top-down: the frontier's out-rows;
// bottom-up: the unvisited vertices' in-rows), hub rows listed for
// k_bfs_hubs.  A launch whose frontier is empty does nothing.
__global__ __launch_bounds__(kBlock) void k_bfs_rows(TravArgs a) {
    __shared__ int32_t qbuf[kWaves][kQueueBuf];
    __shared__ uint64_t red[kWaves];
    const int L = a.level;
    const uint32_t count = min(a.st->front[L % 3], (uint32_t)a.n);
    if (count == 0) return;  // workgroup-uniform
    const int mode = bfs_mode(a, L);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.st->depth = L;
        a.st->mode[L % 2] = mode;
        a.st->explored[(L + 1) % 2] = a.st->explored[L % 2] + a.st->mf[L % 3];
    }
    const int wave = threadIdx.x / kWave;
    const int64_t waves = (int64_t)gridDim.x * kWaves;
    const int lane = lane_id();
    int32_t* level = a.out;
    if (mode == kTopDown) {
        // after a bottom-up level there is no queue: scan the level array
        const bool scan = L > 0 && a.st->mode[(L - 1) % 2] == kBottomUp;
        const int64_t rows = scan ? (int64_t)a.n : (int64_t)count;
        TopDownOp op(a, L, qbuf[wave]);
        for (int64_t t = (int64_t)blockIdx.x * kWaves + wave; t * kWave < rows; t += waves) {
            const int64_t i = t * kWave + lane;
            int32_t u = -1, s = 0, len = 0;
            if (i < rows) u = scan ? (level[i] == L ? (int32_t)i : -1) : a.queue[i];
            if (u >= 0) row_range(a.rp, a.nnz, u, s, len);
            const bool hub = len >= kHubMin;
            append_hubs(a, L % 2, hub, u, s, len);
            walk_rows(op, a, s, hub ? 0 : len, 0);
        }
        op.finish(&a.st->mf[(L + 1) % 3], red);
    } else {
        TravArgs b = a;  // walk the in-edge CSR
        b.rp = a.in_rp;
        b.ci = a.in_ci;
        uint64_t found_n = 0, found_edges = 0;
        for (int64_t t = (int64_t)blockIdx.x * kWaves + wave; t * kWave < (int64_t)a.n; t += waves) {
            const int64_t i = t * kWave + lane;
            int32_t s = 0, len = 0;
            const bool cand = i < a.n && level[i] == -1;
            if (cand) row_range(b.rp, b.nnz, (int32_t)i, s, len);
            // A parent, when there is one, is nearly always among a row's
            // first few in-edges: each lane first probes its own row's first
            // kProbe in-edges, two at a time; then the rows still without a
            // parent walk the rest of their first kHubMin - 1 in-edges
            // together, and the rest of a long row goes to the hub pass.
            bool hit = false;
            const int32_t probe = min(len, kProbe);
            for (int32_t p = 0; p < probe && !hit; p += 2) {
                const int32_t w0 = column(b, s + p);
                const int32_t w1 = p + 1 < probe ? column(b, s + p + 1) : w0;
                hit = level[w0] == L || level[w1] == L;
            }
            const int32_t head = min(len, kHubMin - 1);
            BottomUpOp op{level, L, 0};
            walk_rows(op, b, s + probe, hit ? 0 : head - probe, 0);
            const bool won = cand && (hit || ((op.found >> lane) & 1u));
            if (won) {
                level[i] = L + 1;
                found_n += 1;
                found_edges += (uint64_t)out_degree(a.out_rp, a.nnz, (int32_t)i);
            }
            const bool rest = cand && !won && len > head;  // (then head > kProbe)
            append_hubs(b, L % 2, rest, (int32_t)i, s + head, len - head);
        }
        const uint64_t fn = block_sum(found_n, red);
        const uint64_t fe = block_sum(found_edges, red);
        if (threadIdx.x == 0 && fn) {
            atomicAdd(&a.st->front[(L + 1) % 3], (uint32_t)fn);
            atomicAdd(&a.st->mf[(L + 1) % 3], (unsigned long long)fe);
        }
    }
}

// The hub chunks of level a.level, then the counters level a.level + 1
// appends to are cleared (their last reader, level a.level - 1, is done).
__global__ __launch_bounds__(kBlock) void k_bfs_hubs(TravArgs a) {
    __shared__ int32_t qbuf[kWaves][kQueueBuf];
    __shared__ uint64_t red[kWaves];
    __shared__ int flag;
    const int L = a.level;
    const uint32_t front = a.st->front[L % 3];
    const uint32_t count = min(a.st->chunks[L % 2], a.chunk_cap);
    if (front > 0 && count > 0) {  // workgroup-uniform
        const int mode = bfs_mode(a, L);
        int32_t* level = a.out;
        if (mode == kTopDown) {
            TopDownOp op(a, L, qbuf[threadIdx.x / kWave]);
            const int32_t none[kPerLane] = {};
            for (uint32_t t = blockIdx.x; t < count; t += gridDim.x) {
                const HubChunk h = a.chunks[t];
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
                    op.edges(v, none, none, ok);
                }
            }
            op.finish(&a.st->mf[(L + 1) % 3], red);
        } else {
            TravArgs b = a;
            b.ci = a.in_ci;
            uint64_t found_n = 0, found_edges = 0;
            for (uint32_t t = blockIdx.x; t < count; t += gridDim.x) {  // workgroup-uniform
                const HubChunk h = a.chunks[t];
                // one read of the row's level decides for the whole workgroup
                // whether another chunk has already found it a parent
                if (threadIdx.x == 0) flag = level[h.row] == -1 ? 0 : 2;
                __syncthreads();
                const int state = flag;
                bool hit = false;
                if (state == 0) {
                    int32_t w[kHubChunk / kBlock];
#pragma unroll
                    for (int r = 0; r < kHubChunk / kBlock; ++r) {
                        const int32_t e = h.beg + r * kBlock + (int32_t)threadIdx.x;
                        w[r] = e < h.end ? column(b, e) : -1;
                    }
#pragma unroll
                    for (int r = 0; r < kHubChunk / kBlock; ++r)
                        if (w[r] >= 0 && level[w[r]] == L) hit = true;
                }
                __syncthreads();  // every lane has read `flag`
                if (hit) flag = 1;
                __syncthreads();
                if (threadIdx.x == 0 && state == 0 && flag == 1 &&
                    atomicCAS(&level[h.row], -1, L + 1) == -1) {
                    found_n += 1;
                    found_edges += (uint64_t)out_degree(a.out_rp, a.nnz, h.row);
                }
                __syncthreads();  // before `flag` is written again
            }
            const uint64_t fn = block_sum(found_n, red);
            const uint64_t fe = block_sum(found_edges, red);
            if (threadIdx.x == 0 && fn) {
                atomicAdd(&a.st->front[(L + 1) % 3], (uint32_t)fn);
                atomicAdd(&a.st->mf[(L + 1) % 3], (unsigned long long)fe);
            }
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.st->front[(L + 2) % 3] = 0;
        a.st->mf[(L + 2) % 3] = 0;
        a.st->chunks[(L + 1) % 2] = 0;
    }
}

// Inclusive prefix sum over a wavefront from DPP row shifts (1, 2, 4, 8
// within each row of 16 lanes) and the two row broadcasts (lane 15 into rows
// 1 and 3, lane 31 into rows 2 and 3): register moves, where a scan from lane
// shuffles takes an LDS round trip per step.  Lanes whose source is outside
// the row, or whose row is masked off, add 0.
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Small frontiers, level after level in one launch of one workgroup (the
// grid-wide kernels pay two launches per level, which is all a search of
// thousands of narrow levels costs).  Entered at level a.level with the
// frontier in a.queue (at most kSmallCap vertices, at most kSmallEdges
// out-edges).  Each level: the frontier's rows that have out-edges sit in
// LDS (first out-edge, and the offset of the row's edges in the
// concatenation of the rows, in any row order); lane t takes the kSmallBatch
// consecutive edges from kSmallBatch * t on (then the next 4096, ...), finds
// the first one's row by binary search and the others' rows among the next
// three (no row is empty), and claims each target.  Claimed vertices go to
// the global queue of their level, and those with out-edges also to LDS
// rows of the next level, whose slots and edge offsets come from one atomic
// add per wavefront on a packed (rows, edges) counter: slot order and offset
// order agree, so the offsets need no scan.  It stops after a level whose
// frontier is empty, or larger than it takes (in rows or out-edges), and
// leaves the state as the grid-wide kernels of the next level expect it
// (counts of that level, the counters it appends to cleared, the queue in
// place), with that level in small_next.
//
// A narrow level is a chain of latencies: LDS for the row search, memory for
// the column, then the claim (LDS or memory) alongside the target's row
// bounds (memory), then the slot counters (LDS).  So a lane issues the loads
// of all its edges together, in straight-line code (a load under a branch is
// waited for where the branch ends), and stores only after its last load (a
// store ahead of a load holds that load's wait until the store completes).
// One barrier per level; the counters of levels L, L + 1 and L + 2 are
// three slots, and level L clears the slot of L + 2.
//
// kBits: the graph has at most kBitVerts vertices, and the workgroup keeps a
// bitmap of the visited vertices in LDS, built from the level array at entry.
// A vertex is then claimed by an LDS atomic OR on its bit and its level is a
// plain store, in place of a compare-and-swap on its level.  The frontier
// then holds at most kSmallBitCap rows.
template <bool kBits>
__global__ __launch_bounds__(kSmallBlock) void k_bfs_small(TravArgs a, int32_t* q0, int32_t* q1) {
    constexpr int32_t kCap = kBits ? kSmallBitCap : kSmallCap;
    __shared__ int32_t fs[2][kCap];   // frontier rows' first out-edges
    __shared__ int32_t pre[2][kCap];  // and their offsets (increasing)
    __shared__ uint32_t seen[kBits ? kBitVerts / 32 : 1];
    __shared__ uint32_t nq[3];             // a level's claims (its queue length)
    __shared__ unsigned long long nre[3];  // its rows << 32 | their out-edges
    __shared__ uint32_t nlong[3];          // non-zero: a row has > kSmallBatch edges
    __shared__ uint32_t sink[kWave];       // targets of unused slots' claims
    TravState* st = a.st;
    int32_t* level = a.out;
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave_u = __builtin_amdgcn_readfirstlane(tid / kWave);
    int L = a.level;
    int cur = 0;
    if (kBits) {
        // bit v of `seen`: level[v] != -1.  A lane builds whole words, from
        // eight 16-byte loads issued together when the level array is
        // 16-byte aligned (word w's levels start at byte 128 w), else and in
        // the last, partial word one level at a time.  Words past the last
        // vertex are never read.
        const int32_t words = (a.n + 31) / 32;
        const bool vec = ((uintptr_t)level & 15u) == 0;
        for (int32_t w = tid; w < words; w += kSmallBlock) {
            const int32_t v0 = w * 32;
            uint32_t bits = 0;
            if (vec && v0 + 32 <= a.n) {
                const int4* p = reinterpret_cast<const int4*>(level + v0);
                int4 q[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) q[k] = p[k];
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    bits |= (uint32_t)(q[k].x != -1) << (4 * k) |
                            (uint32_t)(q[k].y != -1) << (4 * k + 1) |
                            (uint32_t)(q[k].z != -1) << (4 * k + 2) |
                            (uint32_t)(q[k].w != -1) << (4 * k + 3);
            } else {
                for (int k = 0; k < 32 && v0 + k < a.n; ++k)
                    bits |= (uint32_t)(level[v0 + k] != -1) << k;
            }
            seen[w] = bits;
        }
    }
    // out-degree sum of the levels below L, carried in a register: a
    // read-modify-write of the state per level would hold every level's
    // closing barrier for a global load
    uint64_t explored = st->explored[L % 2];
    const uint32_t Fq0 = st->front[L % 3];  // level L's vertices, in its queue
    if (tid == 0) {
        nq[L % 3] = Fq0;
        nre[L % 3] = 0;
        nlong[L % 3] = 0;
        nq[(L + 1) % 3] = 0;
        nre[(L + 1) % 3] = 0;
        nlong[(L + 1) % 3] = 0;
    }
    __syncthreads();
    // the entry frontier's rows with out-edges (Fq0 <= kCap)
    for (uint32_t i = tid; i < Fq0; i += kSmallBlock) {
        int32_t s0, len;
        row_range(a.rp, a.nnz, (L % 2 ? q1 : q0)[i], s0, len);
        if (len > 0) {
            const unsigned long long o = atomicAdd(&nre[L % 3], 1ull << 32 | (uint32_t)len);
            fs[0][o >> 32] = s0;
            pre[0][o >> 32] = (int32_t)(uint32_t)o;
            if (len > kSmallBatch) nlong[L % 3] = 1;
        }
    }
    __syncthreads();
    while (true) {
        // level L: Fq vertices, Fr rows in fs/pre[cur], total out-edges
        const int b = L % 3;
        const uint32_t Fq = nq[b];
        const unsigned long long re = nre[b];
        const uint32_t Fr = (uint32_t)(re >> 32), total = (uint32_t)re;
        if (Fq == 0 || Fr > (uint32_t)kCap || total > kSmallEdges) {
            // an empty level, or one the workgroup does not take: hand it
            // to the grid-wide kernels (uniform: every lane read the same)
            if (tid == 0) {
                st->front[L % 3] = Fq;
                st->mf[L % 3] = total;
                st->front[(L + 1) % 3] = 0;
                st->mf[(L + 1) % 3] = 0;
                st->chunks[L % 2] = 0;
                st->small_next = L;
            }
            return;
        }
        // level L + 2's counters, which level L + 1 fills after the barrier
        // that ends level L (the slot of level L - 1, which every lane read
        // before the barrier that ended it)
        if (tid == 0) {
            nq[(L + 2) % 3] = 0;
            nre[(L + 2) % 3] = 0;
            nlong[(L + 2) % 3] = 0;
        }
        int32_t* next_q = (L + 1) % 2 ? q1 : q0;
        const int nxt = cur ^ 1;
        // direct: no row has more than kSmallBatch edges, so slots are rows
        // (kSmallBatch per row, the unused ones idle) and nothing is
        // searched; else slots are edges, kSmallBatch consecutive ones per
        // lane and pass
        const bool direct = nlong[b] == 0;
        const uint32_t span = direct ? Fr * kSmallBatch : total;
        // binary search steps: powers of two from the largest below Fr
        const int32_t top = Fr > 1 ? 1 << (31 - __builtin_clz(Fr - 1)) : 0;
        for (uint32_t p0 = 0; p0 < span; p0 += (uint32_t)(kSmallBlock * kSmallBatch)) {
            // a wavefront whose first slot is past the end has none (uniform)
            if (p0 + (uint32_t)wave_u * (kWave * kSmallBatch) >= span) continue;
            const uint32_t j0 = p0 + (uint32_t)tid * kSmallBatch;
            bool won[kSmallBatch];
            int32_t v[kSmallBatch], s0[kSmallBatch], len[kSmallBatch];
            uint32_t cnt = 0, esum = 0;
#pragma unroll
            for (int k = 0; k < kSmallBatch; ++k) {
                won[k] = false;
                v[k] = 0;
                s0[k] = 0;
                len[k] = 0;
            }
            if (j0 < span) {
                // offset of row r, with row Fr at `total` (above every edge)
                auto off = [&](int32_t r) -> uint32_t {
                    const uint32_t x = (uint32_t)pre[cur][min(r, (int32_t)Fr - 1)];
                    return r >= (int32_t)Fr ? total : x;
                };
                bool ok[kSmallBatch];
                int32_t e[kSmallBatch];
                if (direct) {
                    // row t < Fr: its first edge and length
                    const int32_t t = (int32_t)(j0 / kSmallBatch);
                    const int32_t sr = fs[cur][t];
                    const uint32_t len0 = off(t + 1) - off(t);
#pragma unroll
                    for (int k = 0; k < kSmallBatch; ++k) {
                        ok[k] = (uint32_t)k < len0;
                        e[k] = ok[k] ? sr + k : 0;
                    }
                } else {
                    int32_t lo = 0;  // the last row whose offset is <= j0
                    for (int32_t step = top; step > 0; step >>= 1)
                        if (off(lo + step) <= j0) lo += step;
                    // rows lo .. lo + 3 hold edges j0 .. j0 + 3 (no row is
                    // empty)
                    uint32_t P[4];
                    int32_t S[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        P[i] = off(lo + i);
                        S[i] = fs[cur][min(lo + i, (int32_t)Fr - 1)];
                    }
#pragma unroll
                    for (int k = 0; k < kSmallBatch; ++k) {
                        const uint32_t j = j0 + (uint32_t)k;
                        int32_t sr = S[0];
                        uint32_t pr = P[0];
#pragma unroll
                        for (int i = 1; i < 4; ++i) {
                            if (P[i] <= j) {
                                sr = S[i];
                                pr = P[i];
                            }
                        }
                        ok[k] = j < total;
                        e[k] = ok[k] ? sr + (int32_t)(j - pr) : 0;
                    }
                }
                // total > 0, so nnz > 0 and column() is defined; unused
                // slots (edge 0) claim nothing
#pragma unroll
                for (int k = 0; k < kSmallBatch; ++k) v[k] = column(a, e[k]);
                int32_t old[kSmallBatch];
#pragma unroll
                for (int k = 0; k < kSmallBatch; ++k) {
                    // an unused slot takes a word of its own lane and
                    // changes nothing
                    if (kBits) {
                        const uint32_t bit = ok[k] ? 1u << (v[k] & 31) : 0u;
                        const uint32_t prev =
                            atomicOr(ok[k] ? &seen[v[k] >> 5] : &sink[lane], bit);
                        won[k] = ok[k] && !(prev & bit);
                    } else {
                        // (no level holds INT32_MIN)
                        old[k] = atomicCAS(&level[ok[k] ? v[k] : min(tid, a.n - 1)],
                                           ok[k] ? -1 : INT32_MIN, L + 1);
                    }
                }
                // kBits: the rows of claimed vertices (the others read row 0's
                // bounds, unused); else every target's, loaded while the
                // compare-and-swap is in flight
#pragma unroll
                for (int k = 0; k < kSmallBatch; ++k)
                    row_range(a.rp, a.nnz, kBits ? (won[k] ? v[k] : 0) : v[k], s0[k], len[k]);
#pragma unroll
                for (int k = 0; k < kSmallBatch; ++k) {
                    if (!kBits) won[k] = ok[k] && old[k] == -1;
                    // claims in the low half, rows with out-edges in the high
                    cnt += won[k] ? (len[k] > 0 ? 0x10001u : 1u) : 0u;
                    esum += won[k] ? (uint32_t)len[k] : 0u;
                    if (won[k] && len[k] > kSmallBatch) nlong[(L + 1) % 3] = 1;
                }
            }
            // one pair of LDS atomics per wavefront; its lanes take slots in
            // lane order (a wavefront's claims stay below 2^16, and the
            // out-edges of claimed vertices below nnz < 2^31)
            const uint32_t cincl = wave_scan_dpp(cnt);
            const uint32_t eincl = wave_scan_dpp(esum);
            const uint32_t wc = (uint32_t)__builtin_amdgcn_readlane((int)cincl, kWave - 1);
            const uint32_t we = (uint32_t)__builtin_amdgcn_readlane((int)eincl, kWave - 1);
            uint32_t bq = 0;
            unsigned long long bre = 0;
            if (lane == kWave - 1 && wc) {
                bq = atomicAdd(&nq[(L + 1) % 3], wc & 0xffffu);
                bre = atomicAdd(&nre[(L + 1) % 3],
                                (unsigned long long)(wc >> 16) << 32 | we);
            }
            const uint32_t cex = cincl - cnt;
            uint32_t pos = (uint32_t)__builtin_amdgcn_readlane((int)bq, kWave - 1) + (cex & 0xffffu);
            uint32_t rpos =
                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bre >> 32), kWave - 1) + (cex >> 16);
            uint32_t epos = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bre, kWave - 1) +
                            (eincl - esum);
#pragma unroll
            for (int k = 0; k < kSmallBatch; ++k) {
                if (!won[k]) continue;
                if (kBits) level[v[k]] = L + 1;
                next_q[pos++] = v[k];  // each vertex is claimed once: pos < n
                if (len[k] > 0) {
                    if (rpos < (uint32_t)kCap) {
                        fs[nxt][rpos] = s0[k];
                        pre[nxt][rpos] = (int32_t)epos;
                    }
                    ++rpos;
                    epos += (uint32_t)len[k];
                }
            }
        }
        __syncthreads();
        explored += total;
        if (tid == 0) {
            st->depth = L;
            st->mode[L % 2] = kTopDown;
            st->explored[(L + 1) % 2] = explored;
        }
        ++L;
        cur = nxt;
    }
}

__global__ __launch_bounds__(kBlock) void k_wcc_init(int32_t* __restrict__ label, int32_t n,
                                                     TravState* __restrict__ st) {
    for (int64_t v = blockIdx.x * (int64_t)kBlock + threadIdx.x; v < n;
         v += (int64_t)gridDim.x * kBlock)
        label[v] = (int32_t)v;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st->chunks[0] = 0;
        st->chunks[1] = 0;
        st->components = 0;
        st->giant = -1;
    }
}

// Point every vertex at the smaller of its first out-neighbour and its first
// in-neighbour when that is below its own id.  Only the vertex's own lane
// writes its link, so no atomic is needed; the links point to smaller ids,
// so they form trees.  (Used with the in-edge CSR: the full pass then walks
// every edge of the vertices outside the giant tree, these included.)
__global__ __launch_bounds__(kBlock) void k_wcc_link_first(TravArgs a) {
    for (int64_t u = blockIdx.x * (int64_t)kBlock + threadIdx.x; u < a.n;
         u += (int64_t)gridDim.x * kBlock) {
        int32_t s, len, is, ilen;
        row_range(a.rp, a.nnz, (int32_t)u, s, len);
        row_range(a.in_rp, a.nnz, (int32_t)u, is, ilen);
        int32_t c = INT32_MAX;
        if (len > 0) c = column(a, s);
        if (ilen > 0) c = min(c, (int32_t)min((uint32_t)a.in_ci[min((uint32_t)is, a.nnz - 1u)], a.col_max));
        if (c < (int32_t)u) a.out[u] = c;
    }
}

// Link every vertex with its r-th out-neighbour (if it has one).
__global__ __launch_bounds__(kBlock) void k_wcc_sample(TravArgs a, int32_t r) {
    for (int64_t u = blockIdx.x * (int64_t)kBlock + threadIdx.x; u < a.n;
         u += (int64_t)gridDim.x * kBlock) {
        int32_t s, len;
        row_range(a.rp, a.nnz, (int32_t)u, s, len);
        if (len > r) hook(a.out, find_root(a.out, (int32_t)u), column(a, s + r));
    }
}

// Point every vertex at its root; with `count`, also count the roots.
// Concurrent writers only ever store roots, so every read is an ancestor.
__global__ __launch_bounds__(kBlock) void k_wcc_compress(int32_t* __restrict__ label, int32_t n,
                                                         TravState* __restrict__ st, int count) {
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
    if (!count) return;
    roots = block_sum(roots, red);
    if (threadIdx.x == 0 && roots) atomicAdd(&st->components, roots);
}

// The root shared by most of kGiantSamples vertices drawn by a fixed
// multiplicative hash (ties: the smaller root).  One workgroup of
// kGiantSamples lanes, one sample each.
__global__ __launch_bounds__(kGiantSamples) void k_wcc_giant(const int32_t* __restrict__ label,
                                                             int32_t n, TravState* __restrict__ st) {
    __shared__ int32_t smp[kGiantSamples];
    __shared__ uint64_t best[kGiantSamples / kWave];
    const int j = threadIdx.x;
    const uint64_t h = (uint64_t)(j + 1) * 0x9E3779B97F4A7C15ull;
    smp[j] = label[(int64_t)((h >> 32) % (uint64_t)n)];
    __syncthreads();
    // key = count << 32 | (INT32_MAX - root): the largest key is the most
    // frequent root, the smaller one on a tie
    const int32_t mine = smp[j];
    uint32_t c = 0;
    for (int i = 0; i < kGiantSamples; ++i) c += smp[i] == mine ? 1u : 0u;
    uint64_t key = (uint64_t)c << 32 | (uint32_t)(INT32_MAX - mine);
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const uint64_t o = __shfl_xor(key, off, kWave);
        key = o > key ? o : key;
    }
    if (lane_id() == 0) best[j / kWave] = key;
    __syncthreads();
    if (j == 0) {
        uint64_t b = best[0];
        for (int w = 1; w < kGiantSamples / kWave; ++w) b = best[w] > b ? best[w] : b;
        st->giant = INT32_MAX - (int32_t)(uint32_t)b;
    }
}

// The full linking pass over the rows of (a.rp, a.ci), from edge a.skip of
// every row, skipping the rows of vertices already in the giant tree.
__global__ __launch_bounds__(kBlock) void k_wcc_rows(TravArgs a, int slot) {
    const int32_t giant = a.st->giant;
    const int wave = threadIdx.x / kWave;
    const int64_t waves = (int64_t)gridDim.x * kWaves;
    WccOp op{a.out};
    for (int64_t t = (int64_t)blockIdx.x * kWaves + wave; t * kWave < (int64_t)a.n; t += waves) {
        const int64_t i = t * kWave + lane_id();
        int32_t s = 0, len = 0, root = 0;
        if (i < a.n && (giant < 0 || a.out[i] != giant)) {
            row_range(a.rp, a.nnz, (int32_t)i, s, len);
            const int32_t k = min(len, a.skip);
            s += k;
            len -= k;
        }
        const bool hub = len >= kHubMin;
        append_hubs(a, slot, hub, (int32_t)i, s, len);
        if (hub) len = 0;
        if (len > 0) root = op.prologue((int32_t)i);
        walk_rows(op, a, s, len, root);
    }
}

__global__ __launch_bounds__(kBlock) void k_wcc_hubs(TravArgs a, int slot) {
    WccOp op{a.out};
    const uint32_t count = min(a.st->chunks[slot], a.chunk_cap);
    const int32_t none[kPerLane] = {};
    for (uint32_t t = blockIdx.x; t < count; t += gridDim.x) {
        const HubChunk h = a.chunks[t];
        const int32_t root = op.prologue(h.row);
        int32_t roots[kPerLane];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) roots[k] = root;
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
            op.edges(v, roots, none, ok);
        }
    }
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

int check_graph(int32_t n, int64_t nnz, const int32_t* rp, const int32_t* ci,
                const int32_t* in_rp, const int32_t* in_ci) {
    if (n < 1) return fail(PR_ERR_ARG, "n must be >= 1 (got %d)", n);
    if (nnz < 0 || nnz > INT32_MAX)
        return fail(PR_ERR_ARG, "nnz must be in [0, INT32_MAX] (got %lld)", (long long)nnz);
    if (!rp || (nnz > 0 && !ci)) return fail(PR_ERR_ARG, "null pointer argument");
    if ((in_ci && !in_rp) || (in_rp && nnz > 0 && !in_ci))
        return fail(PR_ERR_ARG, "in_row_ptr and in_col_idx are given together or not at all");
    return PR_OK;
}

int check_ws(const TravWs& w, void* ws, size_t ws_bytes, const char* what) {
    if (!ws) return fail(PR_ERR_ARG, "%s: workspace is null", what);
    if (ws_bytes < w.bytes || (reinterpret_cast<uintptr_t>(ws) & 255u))
        return fail(PR_ERR_WORKSPACE, "%s needs %zu workspace bytes at 256-byte alignment (got %zu)",
                    what, w.bytes, ws_bytes);
    return PR_OK;
}

// PR_VALIDATE: the out-edge CSR, and the in-edge CSR when given (as a CSR of
// the same size; that it is the transpose is the caller's promise).
int validate(int32_t n, int64_t nnz, const int32_t* rp, const int32_t* ci, const int32_t* in_rp,
             const int32_t* in_ci, TravState* st, hipStream_t stream, const char* what) {
    uint32_t* err = &st->err;
    PR_TRY(fill_u32(err, 0u, 1, stream));
    PR_TRY(check_out_row_ptr(rp, n, nnz, err, stream));
    if (in_rp) PR_TRY(check_out_row_ptr(in_rp, n, nnz, err, stream));
    if (nnz > 0) {
        k_trav_check_cols<<<vertex_grid(nnz), kBlock, 0, stream>>>(ci, nnz, n, err);
        PR_LAUNCHED("check columns");
        if (in_ci) {
            k_trav_check_cols<<<vertex_grid(nnz), kBlock, 0, stream>>>(in_ci, nnz, n, err);
            PR_LAUNCHED("check columns");
        }
    }
    return read_error_word(err, stream, what);
}

TravArgs make_args(int32_t n, int64_t nnz, const int32_t* rp, const int32_t* ci,
                   const int32_t* in_rp, const int32_t* in_ci, int32_t* out, const TravWs& w) {
    TravArgs a{};
    a.rp = rp;
    a.ci = ci;
    a.out_rp = rp;
    a.in_rp = in_rp;
    a.in_ci = in_ci;
    a.nnz = (uint32_t)nnz;
    a.col_max = (uint32_t)(n - 1);
    a.n = n;
    a.out = out;
    a.queue = w.queue[0];
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

extern "C" int pr_bfs(int32_t n, int64_t nnz, const int32_t* rp, const int32_t* ci,
                      const int32_t* in_rp, const int32_t* in_ci, int32_t source, int32_t* level,
                      int32_t* depth_host, int64_t* edges_scanned_host, void* ws, size_t ws_bytes,
                      uint32_t flags, void* stream_v) {
    PR_TRY(check_graph(n, nnz, rp, ci, in_rp, in_ci));
    if (!level) return fail(PR_ERR_ARG, "level is null");
    if (source < 0 || source >= n)
        return fail(PR_ERR_ARG, "source %d is not a vertex of a %d-vertex graph", source, n);
    if (flags & ~PR_VALIDATE) return fail(PR_ERR_ARG, "unknown flags 0x%x", flags);
    const TravWs w = carve(ws, n, nnz, true);
    PR_TRY(check_ws(w, ws, ws_bytes, "pr_bfs"));
    hipStream_t stream = as_stream(stream_v);
    if (flags & PR_VALIDATE)
        PR_TRY(validate(n, nnz, rp, ci, in_rp, in_ci, w.st, stream, "pr_bfs"));

    TravArgs a = make_args(n, nnz, rp, ci, in_rp, in_ci, level, w);
    k_bfs_init<<<vertex_grid(n), kBlock, 0, stream>>>(a, source);
    PR_LAUNCHED("bfs init");
    TravState h{};
    auto read_state = [&]() -> int {
        PR_HIP_TRY(hipMemcpyAsync(&h, w.st, sizeof h, hipMemcpyDeviceToHost, stream));
        PR_HIP_TRY(hipStreamSynchronize(stream));
        return PR_OK;
    };
    PR_TRY(read_state());
    int32_t L = 0;
    int batch = kFirstBatch;
    // A frontier holds at least one vertex, so at most n levels are non-empty.
    while (L <= n && h.front[L % 3] != 0) {
        a.level = L;
        a.queue = w.queue[L % 2];
        a.next = w.queue[(L + 1) % 2];
        if (h.front[L % 3] <= (uint32_t)kSmallCap && h.mf[L % 3] <= kSmallEdges) {
            // narrow levels: one launch runs them until the frontier grows
            if (n <= kBitVerts && h.front[L % 3] <= (uint32_t)kSmallBitCap)
                k_bfs_small<true><<<1, kSmallBlock, 0, stream>>>(a, w.queue[0], w.queue[1]);
            else
                k_bfs_small<false><<<1, kSmallBlock, 0, stream>>>(a, w.queue[0], w.queue[1]);
            PR_LAUNCHED("bfs small levels");
            PR_TRY(read_state());
            L = h.small_next;
            continue;
        }
        for (int k = 0; k < batch; ++k, ++L) {
            a.level = L;
            a.queue = w.queue[L % 2];
            a.next = w.queue[(L + 1) % 2];
            k_bfs_rows<<<kRowGrid, kBlock, 0, stream>>>(a);
            PR_LAUNCHED("bfs rows");
            k_bfs_hubs<<<kRowGrid, kBlock, 0, stream>>>(a);
            PR_LAUNCHED("bfs hubs");
        }
        PR_TRY(read_state());  // then h.front[L % 3]: the frontier of level L
        batch = std::min(batch * 2, kMaxBatch);
    }
    if (depth_host) *depth_host = h.depth;
    // the out-degree sum of every non-empty level, recorded by the level after
    // the deepest one
    if (edges_scanned_host) *edges_scanned_host = (int64_t)h.explored[(h.depth + 1) % 2];
    return PR_OK;
}

extern "C" int pr_wcc(int32_t n, int64_t nnz, const int32_t* rp, const int32_t* ci,
                      const int32_t* in_rp, const int32_t* in_ci, int32_t* label,
                      int32_t* n_components_host, void* ws, size_t ws_bytes, uint32_t flags,
                      void* stream_v) {
    PR_TRY(check_graph(n, nnz, rp, ci, in_rp, in_ci));
    if (!label) return fail(PR_ERR_ARG, "label is null");
    if (flags & ~PR_VALIDATE) return fail(PR_ERR_ARG, "unknown flags 0x%x", flags);
    const TravWs w = carve(ws, n, nnz, false);
    PR_TRY(check_ws(w, ws, ws_bytes, "pr_wcc"));
    hipStream_t stream = as_stream(stream_v);
    if (flags & PR_VALIDATE)
        PR_TRY(validate(n, nnz, rp, ci, in_rp, in_ci, w.st, stream, "pr_wcc"));

    const unsigned vg = vertex_grid(n);
    k_wcc_init<<<vg, kBlock, 0, stream>>>(label, n, w.st);
    PR_LAUNCHED("wcc init");
    TravArgs a = make_args(n, nnz, rp, ci, in_rp, in_ci, label, w);
    if (nnz > 0) {
        // with the in-edge CSR one round already puts nearly every vertex of
        // the giant component in its tree
        const int32_t rounds = in_rp ? 1 : kSampledEdges;
        for (int32_t r = 0; r < rounds; ++r) {
            if (r == 0 && in_rp)
                k_wcc_link_first<<<vg, kBlock, 0, stream>>>(a);
            else
                k_wcc_sample<<<vg, kBlock, 0, stream>>>(a, r);
            PR_LAUNCHED("wcc sample");
            k_wcc_compress<<<vg, kBlock, 0, stream>>>(label, n, w.st, 0);
            PR_LAUNCHED("wcc compress");
        }
        if (in_rp) {
            k_wcc_giant<<<1, kGiantSamples, 0, stream>>>(label, n, w.st);
            PR_LAUNCHED("wcc giant");
        }
        // Without the in-edge CSR every vertex's out-row is walked, and the
        // two sampled out-edges are already linked.  With it only the rows
        // outside the giant tree are walked, each from its first edge (the
        // first sampling round linked one edge per vertex, not necessarily
        // an out-edge).
        a.skip = in_rp ? 0 : kSampledEdges;
        k_wcc_rows<<<kRowGrid, kBlock, 0, stream>>>(a, 0);
        PR_LAUNCHED("wcc rows");
        k_wcc_hubs<<<kRowGrid, kBlock, 0, stream>>>(a, 0);
        PR_LAUNCHED("wcc hubs");
        if (in_rp) {  // the in-edges of the vertices outside the giant tree
            TravArgs b = a;
            b.rp = in_rp;
            b.ci = in_ci;
            b.skip = 0;
            k_wcc_rows<<<kRowGrid, kBlock, 0, stream>>>(b, 1);
            PR_LAUNCHED("wcc in-rows");
            k_wcc_hubs<<<kRowGrid, kBlock, 0, stream>>>(b, 1);
            PR_LAUNCHED("wcc in-hubs");
        }
    }
    // the counting pass adds one value per workgroup to a single counter:
    // keep the workgroups few
    k_wcc_compress<<<std::min(vg, 512u), kBlock, 0, stream>>>(label, n, w.st, 1);
    PR_LAUNCHED("wcc compress");
    if (n_components_host) {
        uint32_t c = 0;
        PR_HIP_TRY(hipMemcpyAsync(&c, &w.st->components, sizeof c, hipMemcpyDeviceToHost, stream));
        PR_HIP_TRY(hipStreamSynchronize(stream));
        *n_components_host = (int32_t)c;
    }
    return PR_OK;
}
