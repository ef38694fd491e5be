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
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <thread>
#include <utility>
#include <vector>

#include "plan.hpp"
#include "transpose.hpp"


namespace pr {

// ------------------------------------------------------- host resources
//
// One pool of PlanHost records per process, each record tied to the device it
// was made on.  Records are created on demand and never freed: there are at
// most as many as plans that were alive at the same time.
namespace {
std::mutex g_pool_mutex;
PlanHost* g_pool = nullptr;
constexpr size_t kStageInitial = 1u << 20;
}  // namespace

int host_stage(PlanHost* h, size_t bytes) {
    if (h->stage_bytes >= bytes) return PR_OK;
    size_t cap = h->stage_bytes ? h->stage_bytes : kStageInitial;
    while (cap < bytes) cap *= 2;
    if (h->stage) PR_HIP_TRY(hipHostFree(h->stage));
    h->stage = nullptr;
    h->stage_bytes = 0;
    // non-coherent: cached on the host side, which reads the read-backs many
    // times (every copy through it is waited for before the host touches it)
    PR_HIP_TRY(hipHostMalloc(reinterpret_cast<void**>(&h->stage), cap, hipHostMallocNonCoherent));
    h->stage_bytes = cap;
    return PR_OK;
}

int host_take(PlanHost** out) {
    *out = nullptr;
    int dev = 0;
    PR_HIP_TRY(hipGetDevice(&dev));
    {
        std::lock_guard<std::mutex> lock(g_pool_mutex);
        for (PlanHost** pp = &g_pool; *pp; pp = &(*pp)->next) {
            if ((*pp)->device == dev) {
                *out = *pp;
                *pp = (*pp)->next;
                (*out)->next = nullptr;
                return PR_OK;
            }
        }
    }
    PlanHost* h = static_cast<PlanHost*>(std::calloc(1, sizeof(PlanHost)));
    if (!h) return fail(PR_ERR_ARG, "out of host memory");
    h->device = dev;
    hipError_t e = hipEventCreate(&h->ev_begin);
    if (e == hipSuccess) e = hipEventCreate(&h->ev_end);
    for (int i = 0; i < 2 * kTimedLaunches && e == hipSuccess; ++i)
        e = hipEventCreate(&h->kernel_ev[i / kTimedLaunches][i % kTimedLaunches]);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&h->chunk_ev[0], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&h->chunk_ev[1], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&h->stage_ev, hipEventDisableTiming);
    if (e == hipSuccess)
        e = hipHostMalloc(reinterpret_cast<void**>(&h->status), 2 * sizeof(RunStatus),
                          hipHostMallocDefault);
    if (e != hipSuccess) {
        const int rc = fail(PR_ERR_HIP, "plan events / pinned status: %s", hipGetErrorString(e));
        if (h->ev_begin) (void)hipEventDestroy(h->ev_begin);
        if (h->ev_end) (void)hipEventDestroy(h->ev_end);
        for (int i = 0; i < 2 * kTimedLaunches; ++i)
            if (h->kernel_ev[i / kTimedLaunches][i % kTimedLaunches])
                (void)hipEventDestroy(h->kernel_ev[i / kTimedLaunches][i % kTimedLaunches]);
        for (int i = 0; i < 2; ++i)
            if (h->chunk_ev[i]) (void)hipEventDestroy(h->chunk_ev[i]);
        if (h->stage_ev) (void)hipEventDestroy(h->stage_ev);
        if (h->status) (void)hipHostFree(h->status);
        std::free(h);
        return rc;
    }
    *out = h;
    return host_stage(h, kStageInitial);
}

void host_give(PlanHost* h) {
    if (!h) return;
    std::lock_guard<std::mutex> lock(g_pool_mutex);
    h->next = g_pool;
    g_pool = h;
}

namespace {

// Work list entries of the in-degree count.
// (chunks hold at least nnz / 256 keys, so 256 buckets make at most 512)
constexpr int kMaxCountChunks = 512;

// Upper bounds of the tiled layout.
inline int64_t max_tiles(int32_t n) { return n / kTileMinRows + kNumBuckets + 1; }
// A tile of e edges and r rows is cut into c <= ceil(e / min_unit_edges(r))
// units, each of at least kMinUnitEdgesFloor edges when c > 1: so at most
// tiles + nnz / kMinUnitEdgesFloor units, at most nnz / kMinUnitEdgesFloor
// cut tiles, and c * r < r * e / min_unit_edges(r) + r <= e / 8 + r partial
// slots per cut tile, nnz / 8 + n over all of them (plus the padding that
// starts each cut tile's slots on a 128-byte line: kSlotAlign - 1 at most).
inline int64_t max_units(int32_t n, int64_t nnz) { return max_tiles(n) + nnz / kMinUnitEdgesFloor + 1; }
inline int64_t max_fixes(int32_t n, int64_t nnz) {
    const int64_t a = max_tiles(n), b = nnz / kMinUnitEdgesFloor + 1;
    return a < b ? a : b;
}
constexpr int64_t kSlotAlign = 16;  // slots of 8 bytes: a 128-byte line
inline int64_t max_partial(int32_t n, int64_t nnz) {
    return nnz / 8 + n + 1 + (kSlotAlign - 1) * max_fixes(n, nnz);
}
// Tile edge slots: every tile padded to whole blocks.
inline int64_t max_edge_slots(int32_t n, int64_t nnz) { return nnz + (int64_t)(kEdgeBlock - 1) * max_tiles(n); }

struct PlanWs {  // lives as long as the plan
    float* inv_out;
    int32_t* new_id;
    float* xi;
    float* contrib0;
    float* contrib1;
    float* part;
    RunState* state;
    int64_t part_stride;
    // bucketed pull
    int32_t* in_rp;
    int32_t* in_ci;
    WorkItem* items;
    ChunkRow* chunk_rows;
    float* hub_part;
    int64_t n_items_max, n_slots_max, n_chunk_rows_max;
    // tiled pull
    int32_t* tsrc;
    uint16_t* tdst;
    int32_t* tblk;
    int32_t* tile_ptr;
    Tile* tiles;
    TileUnit* units;
    TileFix* fixes;
    int32_t* fix_rows;
    int32_t* fix_win;    // [n / kFixBlock + 1] the cut tile holding each 256-row window's first row
    uint32_t* fix_done;  // [n_fixes_max]
    long long* partial;
    int64_t n_tiles_max, n_units_max, n_fixes_max, n_partial_max, n_edge_slots_max;
    size_t bytes;
};

struct PlanScratch {  // needed only while pr_plan_create runs
    int32_t* key;        // [n]
    int32_t* old_of;     // [n]
    uint32_t* deg;       // [n]
    int32_t* perm_rp;    // [n + 1]
    int32_t* perm_ci;    // [nnz]
    int32_t* src_of;     // [nnz] scratch of the tiled layout (sort buffers, chunk costs)
    uint32_t* in_rp_plan;  // [n + 1] tiled: in-degrees in plan order, scanned
    int32_t* order;      // [nnz] tiled: sources sorted by tile
    int32_t* tile_first; // [max_tiles + 1] tiled: first sorted edge of each tile
    int32_t* count_chunks;  // [4 * kMaxCountChunks + 1] in-degree counting work list, its length last
    unsigned long long* stats;  // [2 * kNumBuckets]: rows, edges per bucket
    RadixWs vsort;       // sort of the n vertex keys (and scans over n)
    TransposeWs tr;
    size_t bytes;
};

// The arrays both modes use come first; the rest of the workspace holds one
// mode's arrays (the byte count is the larger of the two).
PlanWs carve_ws(void* base, int32_t n, int64_t nnz, bool tiled) {
    PlanWs w{};
    Carver c(base);
    w.n_items_max = max_items(n, nnz);
    w.n_slots_max = max_chunk_slots(nnz);
    w.n_chunk_rows_max = max_chunk_rows(nnz);
    w.n_tiles_max = max_tiles(n);
    w.n_units_max = max_units(n, nnz);
    w.n_fixes_max = max_fixes(n, nnz);
    w.n_partial_max = max_partial(n, nnz);
    w.n_edge_slots_max = max_edge_slots(n, nnz);
    w.inv_out = c.take<float>((size_t)n);
    w.new_id = c.take<int32_t>((size_t)n);
    w.xi = c.take<float>((size_t)n);
    w.contrib0 = c.take<float>((size_t)n);
    w.contrib1 = c.take<float>((size_t)n);
    const int64_t batches = ceil_div(w.n_items_max, kBatchItems);
    // per-workgroup sums: k_init's workgroups, or a bucketed iteration's
    // batches and k_hubfix workgroups (a tiled iteration adds its sums into
    // RunState::tsum)
    w.part_stride = (tiled ? 0 : batches) + kMaxGrid;
    w.part = c.take<float>((size_t)(3 * w.part_stride));  // [3][stride]
    w.state = c.take<RunState>(1);
    if (!tiled) {
        w.in_rp = c.take<int32_t>((size_t)n + 1);
        w.in_ci = c.take<int32_t>((size_t)nnz);
        w.items = c.take<WorkItem>((size_t)w.n_items_max);
        w.chunk_rows = c.take<ChunkRow>((size_t)w.n_chunk_rows_max);
        w.hub_part = c.take<float>((size_t)w.n_slots_max);
    } else {
        w.tsrc = c.take<int32_t>((size_t)w.n_edge_slots_max);
        w.tdst = c.take<uint16_t>((size_t)w.n_edge_slots_max);
        w.tblk = c.take<int32_t>((size_t)(w.n_edge_slots_max / kEdgeBlock + 1));
        w.tile_ptr = c.take<int32_t>((size_t)w.n_tiles_max + 1);
        w.tiles = c.take<Tile>((size_t)w.n_tiles_max);
        w.units = c.take<TileUnit>((size_t)w.n_units_max);
        w.fixes = c.take<TileFix>((size_t)w.n_fixes_max);
        w.fix_rows = c.take<int32_t>((size_t)w.n_fixes_max + 1);
        w.fix_win = c.take<int32_t>((size_t)ceil_div(n, kFixBlock) + 1);
        w.fix_done = c.take<uint32_t>((size_t)w.n_fixes_max);
        w.partial = c.take<long long>((size_t)w.n_partial_max);
    }
    w.bytes = c.used;
    return w;
}

size_t ws_bytes_needed(int32_t n, int64_t nnz) {
    const size_t a = carve_ws(nullptr, n, nnz, false).bytes;
    const size_t b = carve_ws(nullptr, n, nnz, true).bytes;
    return a > b ? a : b;
}

PlanScratch carve_scratch(void* base, int32_t n, int64_t nnz) {
    PlanScratch s{};
    Carver c(base);
    s.key = c.take<int32_t>((size_t)n);
    s.old_of = c.take<int32_t>((size_t)n);
    s.deg = c.take<uint32_t>((size_t)n);
    s.perm_rp = c.take<int32_t>((size_t)n + 1);
    s.perm_ci = c.take<int32_t>((size_t)nnz);
    s.src_of = c.take<int32_t>((size_t)nnz);
    s.in_rp_plan = c.take<uint32_t>((size_t)n + 1);
    s.order = c.take<int32_t>((size_t)nnz);
    s.tile_first = c.take<int32_t>((size_t)max_tiles(n) + 1);
    s.count_chunks = c.take<int32_t>((size_t)4 * kMaxCountChunks + 1);
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

// ------------------------------------------------------------ in-degrees
//
// Row pointers of the transpose (the in-degrees, scanned) without a full
// sort when vertex ids take 9..23 bits: one radix pass partitions the
// targets by their top 8 bits, so each bucket spans at most kCountMaxSpan
// vertices; a workgroup counts a bucket -- or a chunk of a long one -- in
// LDS counters and stores them (adds them, when the bucket is split); a scan
// of the counts gives the row pointers.  Other widths take the keys-only
// radix sort of the targets.
constexpr int kCountDigitBits = 8;
constexpr int kCountMaxSpan = 1 << 15;  // 128 KB of LDS counters
constexpr int kCountBlock = 1024;
constexpr int kCountGroups = 4;  // 16-byte groups of keys per lane per round
constexpr int64_t kMinCountChunk = 1 << 16;

struct CountChunk {
    int32_t bucket;
    int32_t begin;
    int32_t end;
    int32_t split;  // 1: other chunks count the same bucket
};

// The count's work list, from the partition pass's digit-major histogram
// scan (digit d's keys start at scanned[d * T]; scanned[256 * T] = nnz): the
// keys of bucket d cut into ceil(len / size) chunks of about equal length,
// in bucket order.  One lane per bucket; the list's length goes to
// chunks[4 * kMaxCountChunks].  With size >= nnz / 256 there are at most
// 256 + nnz / size <= kMaxCountChunks chunks.
__global__ __launch_bounds__(kBlock) void k_count_chunks(const uint32_t* __restrict__ scanned,
                                                         int64_t T, int64_t size,
                                                         int32_t* __restrict__ chunks) {
    __shared__ uint32_t scan_tmp[kWaves + 1];
    const int b = threadIdx.x;
    const int64_t lo = scanned[(int64_t)b * T], len = (int64_t)scanned[(int64_t)(b + 1) * T] - lo;
    const int64_t k = len > 0 ? (len + size - 1) / size : 0;
    uint32_t total;
    const uint32_t base = block_exclusive_scan((uint32_t)k, &total, scan_tmp);
    CountChunk* list = reinterpret_cast<CountChunk*>(chunks);
    for (int64_t j = 0; j < k; ++j)
        list[base + j] = CountChunk{b, (int32_t)(lo + len * j / k), (int32_t)(lo + len * (j + 1) / k),
                                    k > 1 ? 1 : 0};
    if (b == 0) chunks[4 * kMaxCountChunks] = (int32_t)total;
}

__global__ __launch_bounds__(kCountBlock) void k_count_buckets(const uint16_t* __restrict__ keys,
                                                               const int32_t* __restrict__ chunks,
                                                               int shift, int32_t n,
                                                               uint32_t* __restrict__ counts) {
    __shared__ uint32_t cnt[kCountMaxSpan];
    if ((int32_t)blockIdx.x >= chunks[4 * kMaxCountChunks]) return;  // the grid covers the bound
    const CountChunk c = reinterpret_cast<const CountChunk*>(chunks)[blockIdx.x];
    const int32_t span = 1 << shift;
    for (int32_t v = threadIdx.x; v < span; v += kCountBlock) cnt[v] = 0u;
    __syncthreads();
    // The chunk's 8-aligned middle in 16-byte groups of 8 keys, kCountGroups
    // groups per lane per round (loads first, clamped: they overlap), so a
    // workgroup keeps 64 KB of reads in flight; the unaligned ends one key
    // per lane.
    const int64_t a0 = ((int64_t)c.begin + 7) & ~(int64_t)7;
    const int64_t a1 = ((int64_t)c.end & ~(int64_t)7) > a0 ? ((int64_t)c.end & ~(int64_t)7) : a0;
    for (int64_t i = c.begin + threadIdx.x; i < c.end && i < a0; i += kCountBlock)
        atomicAdd(&cnt[keys[i] & (span - 1)], 1u);
    for (int64_t i = a1 + threadIdx.x; i < c.end; i += kCountBlock)
        atomicAdd(&cnt[keys[i] & (span - 1)], 1u);
    const uint4* groups = reinterpret_cast<const uint4*>(keys + a0);  // keys: 256-byte aligned
    const int64_t ng = (a1 - a0) / 8;
    for (int64_t g0 = threadIdx.x; g0 < ng; g0 += (int64_t)kCountBlock * kCountGroups) {
        uint4 w[kCountGroups];
#pragma unroll
        for (int j = 0; j < kCountGroups; ++j) {
            const int64_t g = g0 + (int64_t)j * kCountBlock;
            w[j] = groups[g < ng ? g : ng - 1];
        }
#pragma unroll
        for (int j = 0; j < kCountGroups; ++j) {
            if (g0 + (int64_t)j * kCountBlock >= ng) break;
            const uint32_t h[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                atomicAdd(&cnt[(h[q] & 0xFFFFu) & (span - 1)], 1u);
                atomicAdd(&cnt[(h[q] >> 16) & (span - 1)], 1u);
            }
        }
    }
    __syncthreads();
    const int64_t v0 = (int64_t)c.bucket << shift;
    for (int32_t v = threadIdx.x; v < span; v += kCountBlock) {
        if (v0 + v >= n) continue;
        if (!c.split)
            counts[v0 + v] = cnt[v];
        else if (cnt[v])
            atomicAdd(&counts[v0 + v], cnt[v]);
    }
}

// The partition of the targets by their top 8 bits for the count: only the
// number of keys per target matters, so the order inside a digit's range is
// free.  A 512-lane workgroup takes kPartTiles consecutive histogram tiles
// (8192 keys, 16 consecutive keys per lane) and writes each digit's keys of
// both as one run, starting where the scanned histogram puts the first
// tile's: runs twice as long as a stable pass over single tiles writes.
// (1024 lanes over four tiles, with runs twice as long again, hold 64 KB of
// LDS and fit two workgroups per CU instead of four: R-MAT 23's plan was
// 0.1-0.15 ms slower; 256 lanes over one tile in between.)  A lane adds each run of equal
// digits among its keys once (a CSR row lists its targets in increasing
// order, so neighbouring keys share their top bits): first to count, then,
// with the returned offset, to place the run in LDS.  Keys are written as
// their low 16 bits.  Out-of-range targets are clamped and flagged as the
// histogram pass does.
constexpr int kPartBlock = 512;
constexpr int kPartItems = 16;
constexpr int kPartTiles = kPartBlock * kPartItems / kRadixTile;
static_assert(kPartTiles * kRadixTile == kPartBlock * kPartItems, "whole histogram tiles");

__global__ __launch_bounds__(kPartBlock) void k_count_partition(RadixIn in, int shift, int64_t T,
                                                                const uint32_t* __restrict__ scanned,
                                                                uint16_t* __restrict__ out) {
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    __shared__ uint32_t cnt[kRadixDigits];
    __shared__ uint32_t start[kRadixDigits + 1];
    __shared__ uint32_t cursor[kRadixDigits];
    __shared__ uint32_t gstart[kRadixDigits];
    __shared__ int32_t stage[kPartBlock * kPartItems];
    __shared__ uint32_t scan_tmp[kPartBlock / kWave + 1];
    const int tid = threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.x * kPartTiles;
    const int64_t base = t0 * kRadixTile;
    const int count = (int)((in.count - base) < kPartBlock * kPartItems ? (in.count - base)
                                                                         : kPartBlock * kPartItems);
    if (tid < kRadixDigits) {
        cnt[tid] = 0u;
        cursor[tid] = 0u;
        // digit tid's keys of tiles [t0, t0 + kPartTiles) start here
        gstart[tid] = scanned[(int64_t)tid * T + t0];
    }
    const int i0 = tid * kPartItems;
    const int left = count - i0;
    int32_t k[kPartItems];
    if (left >= kPartItems && (reinterpret_cast<uintptr_t>(in.keys) & 15u) == 0) {
#pragma unroll
        for (int q = 0; q < kPartItems / 4; ++q) {
            const i32x4 v = *(const i32x4*)(in.keys + base + i0 + 4 * q);
            k[4 * q] = v.x;
            k[4 * q + 1] = v.y;
            k[4 * q + 2] = v.z;
            k[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int r = 0; r < kPartItems; ++r) k[r] = r < left ? in.keys[base + i0 + r] : 0;
    }
    bool bad = false;
#pragma unroll
    for (int r = 0; r < kPartItems; ++r)
        if (r < left) k[r] = radix_check<kFromTargets>(in, k[r], bad);
    report_bad<kFromTargets>(in, bad);
    // each key's digit (a key past the end gets a digit of its own, so no
    // run reaches it) and the length of the run of equal digits from it on
    uint32_t dg[kPartItems], len[kPartItems];
#pragma unroll
    for (int r = 0; r < kPartItems; ++r)
        dg[r] = r < left ? ((uint32_t)k[r] >> shift) & (kRadixDigits - 1) : kRadixDigits + r;
#pragma unroll
    for (int r = kPartItems - 1; r >= 0; --r)
        len[r] = (r + 1 < kPartItems && dg[r + 1] == dg[r]) ? len[r + 1] + 1 : 1u;
    __syncthreads();  // counters cleared
#pragma unroll
    for (int r = 0; r < kPartItems; ++r)
        if (r < left && (r == 0 || dg[r - 1] != dg[r])) atomicAdd(&cnt[dg[r]], len[r]);
    __syncthreads();
    {  // digit starts inside the workgroup's keys
        uint32_t total;
        const uint32_t c = tid < kRadixDigits ? cnt[tid] : 0u;
        const uint32_t e = block_exclusive_scan<uint32_t, kPartBlock / kWave>(c, &total, scan_tmp);
        if (tid < kRadixDigits) start[tid] = e;
        if (tid == 0) start[kRadixDigits] = total;
    }
    __syncthreads();
    {  // the head of each run takes the run's places at once
        uint32_t pos = 0;
#pragma unroll
        for (int r = 0; r < kPartItems; ++r) {
            if (r < left) {
                const bool head = r == 0 || dg[r - 1] != dg[r];
                pos = head ? start[dg[r]] + atomicAdd(&cursor[dg[r]], len[r]) : pos + 1;
                stage[pos] = k[r];
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < count; i += kPartBlock) {
        const int32_t key = stage[i];
        const uint32_t dg = ((uint32_t)key >> shift) & (kRadixDigits - 1);
        out[(int64_t)gstart[dg] + (i - start[dg])] = (uint16_t)key;
    }
}

// in_rp[0..n] of the transpose of (n, nnz, out_ci).  counts: n words of
// scratch; chunks: 4 * kMaxCountChunks + 1 words; scan_ws: a scan workspace
// for n items.  Out-of-range targets are clamped and flagged in tr.error.
// Asynchronous on `stream`.
int indegree_row_ptr(int32_t n, int64_t nnz, const int32_t* out_ci, int32_t* in_rp,
                     uint32_t* counts, int32_t* chunks, void* scan_ws, const TransposeWs& tr,
                     hipStream_t stream) {
    const int bits = vertex_bits(n);
    if (nnz == 0 || bits <= kCountDigitBits || bits - kCountDigitBits > 15)
        return transpose_row_ptr(n, nnz, out_ci, in_rp, tr, stream);
    const int shift = bits - kCountDigitBits;
    RadixIn in{};
    in.count = nnz;
    in.n = n;
    in.keys = out_ci;
    in.error = tr.error;
    const RadixWs& w = tr.sort;
    const int64_t T = radix_tiles(nnz);
    k_radix_hist<kFromTargets><<<dim3((unsigned)T), kBlock, 0, stream>>>(in, shift, T, w.hist);
    PR_LAUNCHED("radix histogram");
    PR_TRY(scan_exclusive(w.hist, w.scanned, kRadixDigits * T, w.scan_ws, stream));
    // the keys' low 16 bits are enough: a bucket spans at most 2^15 vertices
    k_count_partition<<<dim3((unsigned)ceil_div(T, kPartTiles)), kPartBlock, 0, stream>>>(
        in, shift, T, w.scanned, reinterpret_cast<uint16_t*>(w.key[0]));
    PR_LAUNCHED("count partition");
    // chunks of at least max(nnz / 256, kMinCountChunk) keys, listed on the device
    int64_t size = ceil_div(nnz, kRadixDigits);
    if (size < kMinCountChunk) size = kMinCountChunk;
    k_count_chunks<<<1, kBlock, 0, stream>>>(w.scanned, T, size, chunks);
    PR_LAUNCHED("count chunks");
    PR_TRY(fill_u32(counts, 0u, n, stream));
    k_count_buckets<<<dim3((unsigned)kMaxCountChunks), kCountBlock, 0, stream>>>(
        reinterpret_cast<const uint16_t*>(w.key[0]), chunks, shift, n, counts);
    PR_LAUNCHED("count buckets");
    PR_TRY(scan_exclusive(counts, reinterpret_cast<uint32_t*>(in_rp), n, scan_ws, stream));
    return PR_OK;
}

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
// Also indeg[p]: the in-degree of the vertex placed at p (from in_rp, the
// row pointers of the transpose in input ids).
__global__ __launch_bounds__(kBlock) void k_order(const int32_t* __restrict__ old_of,
                                                  const int32_t* __restrict__ out_rp,
                                                  const int32_t* __restrict__ in_rp, int32_t n,
                                                  int32_t* __restrict__ new_id,
                                                  uint32_t* __restrict__ deg,
                                                  uint32_t* __restrict__ indeg,
                                                  float* __restrict__ inv_out) {
    GRID_STRIDE(p, n) {
        const int32_t u = old_of[p];
        new_id[u] = (int32_t)p;
        int32_t d = out_rp[u + 1] - out_rp[u];
        d = d > 0 ? d : 0;
        deg[p] = (uint32_t)d;
        indeg[p] = (uint32_t)(in_rp[u + 1] - in_rp[u]);
        inv_out[p] = d > 0 ? 1.0f / (float)d : 0.0f;
    }
}

// Out-edge CSR in plan order: row p of the result is row old_of[p] of the
// input with every target renumbered.  Edge-parallel: each workgroup covers
// kBlock * kPermItems positions.  The rows that own them lie in [lo, hi] =
// [win_row[w], win_row[w + 1]] (k_tile_rows over perm_rp, every window's
// search side by side before this kernel).  When there are at most
// kPermRows of them, each row marks its first position in an LDS array and
// keeps the distance from its output start to its input start; a max-scan
// carries the marks forward (owner_max_scan), so a position finds its row
// and its input position with two LDS reads, and a lane's loads of out_ci
// and then of new_id go out together for all its positions.  (A window over
// a long run of empty rows searches perm_rp in global memory instead.)  A tiled plan also gets the
// first pass of the sort by tile here: when `hist` is set, the workgroup's
// histogram of min(tile of the renamed target, 255), stored digit-major as
// the radix histogram of a pass over the same 4096-edge tiles
// (hist[digit * T + workgroup]).
constexpr int kPermItems = 16;
constexpr int kPermRows = kBlock * kPermItems;
static_assert(kPermRows == kRadixTile, "the permutation's windows are the sort's tiles");

__global__ __launch_bounds__(kBlock) void k_permute_rows(const int32_t* __restrict__ perm_rp,
                                                         const int32_t* __restrict__ win_row,
                                                         const int32_t* __restrict__ old_of,
                                                         const int32_t* __restrict__ new_id,
                                                         const int32_t* __restrict__ out_rp,
                                                         const int32_t* __restrict__ out_ci,
                                                         int32_t n, int64_t nnz,
                                                         int32_t* __restrict__ perm_ci,
                                                         TileMap map, uint32_t* __restrict__ hist,
                                                         int64_t T) {
    __shared__ int32_t s_own[kPermRows];      // slot owner_slot(i): local row of position base + i
    __shared__ int32_t s_delta[kPermRows];  // per local row: input start - output start
    __shared__ int32_t s_wave[kWaves];
    const int64_t base = blockIdx.x * (int64_t)kPermRows;
    const int64_t last = (base + kPermRows < nnz ? base + kPermRows : nnz) - 1;
    const int count = (int)(last - base + 1);
    const int32_t lo = min(max(win_row[blockIdx.x], 0), n - 1);
    int32_t hi = min(max(win_row[blockIdx.x + 1], lo), n - 1);
    // rows lo .. hi are staged when they fit, or when the rows past the
    // first kPermRows all start after the window (hi owns the next window's
    // first position, so a window of one-edge rows has one too many); the
    // same in every lane
    bool staged = hi - lo + 1 <= kPermRows;
    if (!staged && perm_rp[lo + kPermRows] > last) {
        hi = lo + kPermRows - 1;
        staged = true;
    }
    if (staged) {
        // position base belongs to row lo (local 0); a later row marks its
        // first position (of rows starting at one position the last wins:
        // the others are empty)
        for (int i = threadIdx.x; i < count; i += kBlock) s_own[owner_slot(i)] = i == 0 ? 0 : -1;
        __syncthreads();
        for (int32_t r = threadIdx.x; r <= hi - lo; r += kBlock) {
            const int32_t d = perm_rp[lo + r];
            s_delta[r] = out_rp[old_of[lo + r]] - d;
            const int64_t pos = (int64_t)d - base;
            if (r > 0 && pos > 0 && pos < count) atomicMax(&s_own[owner_slot((int)pos)], r);
        }
        __syncthreads();
        owner_max_scan(count, s_own, s_wave);
    }
    int32_t q[kPermItems];  // input positions, clamped into [0, nnz): they fit 32 bits
#pragma unroll
    for (int r = 0; r < kPermItems; ++r) {
        int64_t p = base + r * kBlock + threadIdx.x;
        p = p < last ? p : last;
        int64_t qr;
        if (staged) {
            const int32_t a = max(s_own[owner_slot((int)(p - base))], 0);
            qr = p + s_delta[a];
        } else {
            const int32_t j = owner_row(perm_rp, p, lo, hi);
            qr = (int64_t)out_rp[old_of[j]] + (p - perm_rp[j]);
        }
        q[r] = (int32_t)(qr < 0 ? 0 : (qr >= nnz ? nnz - 1 : qr));
    }
    int32_t t[kPermItems];
#pragma unroll
    for (int r = 0; r < kPermItems; ++r) {
        t[r] = __builtin_nontemporal_load(out_ci + q[r]);  // streamed: leave L2 to new_id
        // out-of-range targets were flagged by the in-degree sort, which
        // clamped them the same way
        t[r] = t[r] < 0 ? 0 : (t[r] >= n ? n - 1 : t[r]);
    }
#pragma unroll
    for (int r = 0; r < kPermItems; ++r) t[r] = new_id[t[r]];
#pragma unroll
    for (int r = 0; r < kPermItems; ++r) {
        const int64_t p = base + r * kBlock + threadIdx.x;
        if (p <= last) {
            __builtin_nontemporal_store(t[r], perm_ci + p);
        }
    }
    if (hist) {
        // The targets go through LDS (s_own, and s_delta for the counts, are
        // free once every lane has found its rows), so that the count starts
        // with no per-item registers live: counting from them directly costs
        // occupancy.
        uint32_t* s_hist = reinterpret_cast<uint32_t*>(s_delta);
        __syncthreads();
        s_hist[threadIdx.x] = 0u;
#pragma unroll
        for (int r = 0; r < kPermItems; ++r) s_own[r * kBlock + threadIdx.x] = t[r];
        __syncthreads();
        DigitCounter dc;
        for (int r = 0; r < kPermItems; ++r) {
            const int i = r * kBlock + threadIdx.x;
            if (base + i > last) break;
            const int32_t tile = tile_of(map, s_own[i]);
            dc.add((uint32_t)(tile < kRadixDigits - 1 ? tile : kRadixDigits - 1), s_hist);
        }
        dc.flush(s_hist);
        __syncthreads();
        hist[(int64_t)threadIdx.x * T + blockIdx.x] = s_hist[threadIdx.x];
    }
}

// First plan id of tile t: its segment is the last one whose first tile is
// <= t (an empty segment shares its first tile with the next, which then
// wins); picked with selects, as in tile_locate.
__device__ __forceinline__ int32_t tile_row0(const TileMap& m, int32_t t) {
    int32_t start = m.start[0], tile0 = m.tile0[0], shift = m.shift[0];
#pragma unroll
    for (int j = 1; j < kTileSegments; ++j) {
        const bool in = t >= m.tile0[j];
        start = in ? m.start[j] : start;
        tile0 = in ? m.tile0[j] : tile0;
        shift = in ? m.shift[j] : shift;
    }
    return start + ((t - tile0) << shift);
}

// first[t] = in-edges of the rows before tile t (in_rp: the exclusive scan of
// the in-degrees in plan order), i.e. the first position of tile t in the
// edges sorted by tile; first[tiles] = in_rp[n].
__global__ __launch_bounds__(kBlock) void k_tile_first(const uint32_t* __restrict__ in_rp,
                                                       int32_t n, int32_t tiles, TileMap map,
                                                       int32_t* __restrict__ first) {
    GRID_STRIDE(t, (int64_t)tiles + 1) {
        first[t] = (int32_t)in_rp[t < tiles ? tile_row0(map, (int32_t)t) : n];
    }
}

// The tile edge arrays, one kEdgeBlock-slot block at a time per wavefront.
// Sorted edge f + k of tile t (f = first[t]; target targets[f + k], source
// sources[f + k]) goes to slot slot0[t] + block_slot(k): lane l of the
// wavefront holds edges k0 + 64 i + l (i = 0..3) of the block starting at k0
// and writes its four slots 4 l .. 4 l + 3 with one 16-byte store.  Slots
// past the tile's last edge are padding: the tile's last source and the
// trash row.  A block is narrow when its sources (its first edge and its
// last real one) span less than kNarrowSpan: its slots then hold
// (source - first source) | row << 16 and tblk its first source, otherwise
// the source, with the row in tdst and -1 in tblk.
// The same pass counts, per kSectorChunk slots, the slots whose source's
// 64-byte sector of contributions differs from the previous slot's (in edge
// order; the previous slot of a tile's first is the previous tile's last),
// into sector_counts (zeroed beforehand).
// Each wavefront takes a contiguous range of blocks and finds each block's
// tile by walking forward from the tile of its first block.
// One block's slots (see k_tile_blocks): loads first, then the writes.
struct TileBlockIn {
    int64_t slot;
    int32_t k0, cnt;
    int32_t src[4], row[4];
    int32_t lo, hi, before;
};

__device__ __forceinline__ void tile_block_load(TileBlockIn& in, const int32_t* __restrict__ targets,
                                                const int32_t* __restrict__ sources, int32_t row0,
                                                int32_t f, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int32_t k = in.k0 + i * kWave + lane;
        const bool real = k < in.cnt;
        const int32_t e = f + (real ? k : in.cnt - 1);
        in.src[i] = sources[e];
        in.row[i] = real ? targets[e] - row0 : kTrashRow;  // a tile's edges target its rows
    }
    in.lo = sources[f + in.k0];
    in.hi = sources[f + (in.k0 + kEdgeBlock - 1 < in.cnt ? in.k0 + kEdgeBlock - 1 : in.cnt - 1)];
    // the slot before the block: the previous edge of the tile, or the last
    // edge of the previous non-empty tile
    in.before = in.k0 > 0 ? sources[f + in.k0 - 1] : (f > 0 ? sources[f - 1] : -1);
}

__device__ __forceinline__ void tile_block_store(const TileBlockIn& in, int32_t* __restrict__ tsrc,
                                                 uint16_t* __restrict__ tdst,
                                                 int32_t* __restrict__ tblk,
                                                 int32_t* __restrict__ sector_counts, int lane) {
    const bool narrow = in.hi - in.lo < kNarrowSpan;
    int4 w;
    w.x = narrow ? (in.src[0] - in.lo) | (in.row[0] << 16) : in.src[0];
    w.y = narrow ? (in.src[1] - in.lo) | (in.row[1] << 16) : in.src[1];
    w.z = narrow ? (in.src[2] - in.lo) | (in.row[2] << 16) : in.src[2];
    w.w = narrow ? (in.src[3] - in.lo) | (in.row[3] << 16) : in.src[3];
    *reinterpret_cast<int4*>(tsrc + in.slot + 4 * lane) = w;
    if (!narrow) {
        ushort4 d;
        d.x = (uint16_t)in.row[0];
        d.y = (uint16_t)in.row[1];
        d.z = (uint16_t)in.row[2];
        d.w = (uint16_t)in.row[3];
        *reinterpret_cast<ushort4*>(tdst + in.slot + 4 * lane) = d;
    }
    if (lane == 0) tblk[in.slot / kEdgeBlock] = narrow ? in.lo : -1;
    // sector starts: edge 64 i + l follows edge 64 i + l - 1 (lane l - 1, or
    // lane 63 of round i - 1); edge 0 follows the slot before the block
    int32_t starts = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int32_t up = __shfl_up(in.src[i], 1, kWave);
        const int32_t last_of_round = __shfl(in.src[i > 0 ? i - 1 : 0], kWave - 1, kWave);
        const int32_t prev = lane > 0 ? up : (i > 0 ? last_of_round : in.before);
        starts += (prev < 0 || (in.src[i] >> kSectorShift) != (prev >> kSectorShift)) ? 1 : 0;
    }
    starts = wave_sum(starts);
    if (lane == 0) atomicAdd(&sector_counts[in.slot / kSectorChunk], starts);
}

__global__ __launch_bounds__(kBlock) void k_tile_blocks(const int32_t* __restrict__ targets,
                                                        const int32_t* __restrict__ sources,
                                                        TileMap map, const int32_t* __restrict__ first,
                                                        const int32_t* __restrict__ slot0,
                                                        int32_t tiles, int64_t n_blocks,
                                                        int32_t* __restrict__ tsrc,
                                                        uint16_t* __restrict__ tdst,
                                                        int32_t* __restrict__ tblk,
                                                        int32_t* __restrict__ sector_counts) {
    const int lane = lane_id();
    const int64_t waves = (int64_t)gridDim.x * kWaves;
    const int64_t wave = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
    const int64_t per = (n_blocks + waves - 1) / waves;
    int64_t b = wave * per;
    const int64_t b_end = b + per < n_blocks ? b + per : n_blocks;
    if (b >= b_end) return;
    // last tile whose first slot is at or before this block (it is not empty)
    int32_t t = 0;
    {
        int32_t lo = 0, hi = tiles - 1;
        const int64_t slot = b * kEdgeBlock;
        while (lo < hi) {
            const int32_t mid = (lo + hi + 1) / 2;
            if ((int64_t)slot0[mid] <= slot)
                lo = mid;
            else
                hi = mid - 1;
        }
        t = lo;
    }
    // two blocks per step, all of their loads issued before either is written
    for (; b < b_end; b += 2) {
        TileBlockIn in[2];
        int32_t f[2], row0[2];
        const int nb = b + 1 < b_end ? 2 : 1;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            in[j].slot = (b + (j < nb ? j : 0)) * kEdgeBlock;
            while ((int64_t)slot0[t + 1] <= in[j].slot) ++t;  // skips empty tiles
            in[j].k0 = (int32_t)(in[j].slot - slot0[t]);
            f[j] = first[t];
            in[j].cnt = first[t + 1] - f[j];
            row0[j] = tile_row0(map, t);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) tile_block_load(in[j], targets, sources, row0[j], f[j], lane);
        tile_block_store(in[0], tsrc, tdst, tblk, sector_counts, lane);
        if (nb == 2) tile_block_store(in[1], tsrc, tdst, tblk, sector_counts, lane);
    }
}

// Estimated cost of each kSectorChunk-slot chunk of the tile slots: its slots
// plus kSectorWeight per sector start counted in it (cost[c], c < chunks).
__global__ __launch_bounds__(kBlock) void k_chunk_costs(const int32_t* __restrict__ sectors,
                                                        int64_t slots, int32_t chunks, int64_t weight,
                                                        uint64_t* __restrict__ cost) {
    GRID_STRIDE(c, chunks) {
        const int64_t len = c + 1 < chunks ? (int64_t)kSectorChunk : slots - c * (int64_t)kSectorChunk;
        cost[c] = (uint64_t)(len + weight * (int64_t)sectors[c]);
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

// Bucket lower bounds of a layout (kDefaultTileBucketMin for tiles,
// kDefaultBucketMin for the bucketed pull); PR_BUCKET_MIN="0,5,17,65,1025"
// overrides them (a tuning knob).  Must start at 0, not decrease, and keep
// the hub bound at least kMinHubLength.
void bucket_bounds(bool tiled, int32_t out[kNumBuckets]) {
    std::memcpy(out, tiled ? kDefaultTileBucketMin : kDefaultBucketMin, sizeof(kDefaultBucketMin));
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


// Copies `bytes` of device memory to host array `dst` through the pinned
// stage, synchronizing `stream` (no copy may be using the stage).
int read_back(PlanHost* h, void* dst, const void* src, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return PR_OK;
    PR_TRY(host_stage(h, bytes));
    PR_HIP_TRY(hipMemcpyAsync(h->stage, src, bytes, hipMemcpyDeviceToHost, stream));
    PR_HIP_TRY(hipStreamSynchronize(stream));
    std::memcpy(dst, h->stage, bytes);
    return PR_OK;
}

// What a mode's builder reports back to pr_plan_create.
struct Built {
    int32_t n_items = 0, n_chunk_rows = 0, grid = 1, fix_grid = 0;
    int64_t tile_launch = 1, unit_cost = 0;  // tiled: workgroups per launch, cost per unit
    int32_t items_of[kNumBuckets + 1] = {};
    TileMap map{};
    int32_t n_tiles = 0, n_units = 0, n_fixes = 0, tile_grid = 1;
    int64_t n_slots = 0;
    std::vector<WorkItem> hub_items;   // host arrays copied to the device
    std::vector<ChunkRow> chunk_rows;
    std::vector<Tile> tiles;
    std::vector<TileUnit> units;
    std::vector<TileFix> fixes;
    std::vector<int32_t> fix_rows;
    std::vector<int32_t> fix_win;
    int32_t n_fused = 0;  // cut tiles finished in k_tile: the first n_fused of `fixes`
    // tiled: where the work lists were uploaded
    const Tile* dev_tiles = nullptr;
    const TileUnit* dev_units = nullptr;
    const TileFix* dev_fixes = nullptr;
    const int32_t* dev_fix_rows = nullptr;
    const int32_t* dev_fix_win = nullptr;
};

// Bucketed pull: the plan's in-edge CSR (counting-sort transpose of the
// renumbered out-edge CSR), hub rows whole or in chunks (from the hub rows'
// lengths, read back), and every other bucket cut into row ranges of about
// kItemCost.
int build_bucketed(const PlanWs& w, const PlanScratch& s, int32_t n, int64_t nnz, PlanHost* host,
                   const unsigned long long* stats, const int32_t* row_begin, int cus,
                   hipStream_t stream, Built& bt) {
    PR_TRY(transpose_device(n, nnz, s.perm_rp, s.perm_ci, w.in_rp, w.in_ci, s.tr, stream));
    const int32_t n_hub = (int32_t)stats[kHubBucket];
    std::vector<int32_t> hub_rp((size_t)n_hub + 1);
    PR_TRY(read_back(host, hub_rp.data(), w.in_rp, sizeof(int32_t) * hub_rp.size(), stream));

    std::vector<WorkItem>& hub_items = bt.hub_items;
    std::vector<ChunkRow>& chunk_rows = bt.chunk_rows;
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
    int64_t total = (int64_t)hub_items.size();
    for (int b = 0; b < kHubBucket; ++b) {
        const int64_t bc = (int64_t)stats[kNumBuckets + b] + kRowCost * (int64_t)stats[b];
        bt.items_of[b] = stats[b] ? (int32_t)ceil_div(bc, kItemCost) : 0;
        total += bt.items_of[b];
    }
    for (const WorkItem& it : hub_items) bt.items_of[it.kind] += 1;
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
        if (bt.items_of[b] > 0) {
            k_bucket_items<<<grid_for(bt.items_of[b]), kBlock, 0, stream>>>(
                w.in_rp, row_begin[b], row_begin[b] + (int32_t)stats[b], b, bt.items_of[b], item0,
                w.items);
            PR_LAUNCHED("bucket items");
        }
        item0 += bt.items_of[b];
    }
    bt.n_items = (int32_t)total;
    bt.n_chunk_rows = (int32_t)chunk_rows.size();

    // kIterBlocksPerCU workgroups per CU (each holds the hot sources in LDS),
    // fewer when there are few item batches.
    int64_t grid = ceil_div(ceil_div(total, kBatchItems), kIterWaves);
    if (grid > (int64_t)cus * kIterBlocksPerCU) grid = (int64_t)cus * kIterBlocksPerCU;
    if (const char* env = std::getenv("PR_GRID"))  // tuning knob: workgroups per launch
        if (std::atoi(env) > 0) grid = std::atoi(env);
    if (grid > kMaxGrid / 2) grid = kMaxGrid / 2;
    if (grid < 1) grid = 1;
    int64_t fix_grid = ceil_div((int64_t)chunk_rows.size(), kFixBlock / kWave);
    if (fix_grid > kMaxGrid - grid) fix_grid = kMaxGrid - grid;
    bt.grid = (int32_t)grid;
    bt.fix_grid = (int32_t)fix_grid;
    return PR_OK;
}

int log2_ceil(int64_t x) {
    int k = 0;
    while (((int64_t)1 << k) < x) ++k;
    return k;
}

// Tiled pull, before the permutation: tile sizes per bucket, from the bucket
// sizes (host only).  The permutation counts the edges per tile with the map.
int lay_out_tiles(const PlanWs& w, int64_t nnz, const unsigned long long* stats,
                  const int32_t* row_begin, int32_t n, int cus, Built& bt) {
    // Launch width, and the tuning knobs: edges per tile and estimated cost
    // per unit (each knob, when set, is used as given).
    int64_t grid = cus;
    if (const char* env = std::getenv("PR_GRID"))  // tuning knob: workgroups per launch
        if (std::atoi(env) > 0) grid = std::atoi(env);
    if (grid > kMaxGrid) grid = kMaxGrid;
    if (grid < 1) grid = 1;
    const char* tile_env = std::getenv("PR_TILE_EDGES");
    const char* unit_env = std::getenv("PR_UNIT_COST");
    int64_t target = kTileTargetEdges, unit_cost = kUnitCost;
    if (tile_env && std::atoll(tile_env) > 0) target = std::atoll(tile_env);
    if (unit_env && std::atoll(unit_env) > 0) unit_cost = std::atoll(unit_env);
    const int64_t wg_edges = nnz / grid;
    int64_t max_rows = wg_edges < kWgEdgesMid ? kTileRowsFew
                       : wg_edges < kWgEdgesMany ? kTileRowsMid : kTileMaxRows;
    if (const char* env = std::getenv("PR_TILE_ROWS"))  // tuning knob: rows per tile at most
        if (std::atoll(env) >= kTileMinRows && std::atoll(env) <= kTileMaxRows) max_rows = std::atoll(env);
    int64_t light_rows = kTileRowsLight, light_deg = kLightDeg;
    if (const char* env = std::getenv("PR_LIGHT_ROWS"))  // tuning knob: rows per light tile
        if (std::atoll(env) >= kTileMinRows && std::atoll(env) <= kTileMaxRows) light_rows = std::atoll(env);
    if (const char* env = std::getenv("PR_LIGHT_DEG"))  // tuning knob: in-edges per row of a light segment
        if (std::atoll(env) >= 0) light_deg = std::atoll(env);
    TileMap& map = bt.map;
    auto lay_out = [&](int64_t tgt) -> int32_t {  // the tile map for a target; returns the tiles
        int32_t count = 0;
        for (int seg = 0; seg < kTileSegments; ++seg) {
            const int b = kHubBucket - seg;  // segment 0 = hub bucket
            const int64_t rows = (int64_t)stats[b], edges = (int64_t)stats[kNumBuckets + b];
            int64_t want = edges > 0 ? ceil_div(tgt * rows, edges) : kTileMaxRows;
            if (want > max_rows) want = max_rows;
            if (edges < light_deg * rows && want > light_rows) want = light_rows;
            if (want < kTileMinRows) want = kTileMinRows;
            map.start[seg] = row_begin[b];
            map.tile0[seg] = count;
            map.shift[seg] = log2_ceil(want);
            count += (int32_t)ceil_div(rows, (int64_t)1 << map.shift[seg]);
        }
        return count;
    };
    if (!tile_env) {
        // Smaller graphs get smaller tiles: at most 4 * nnz / grid edges each,
        // and halved further while the tiles are fewer than the workgroups
        // (so that every workgroup has a tile to work on).
        int64_t cap = 4 * nnz / grid;
        if (cap < kMinTileTarget) cap = kMinTileTarget;
        if (target > cap) target = cap;
        while (lay_out(target) < grid && target > kMinTileTarget) target /= 2;
    }
    int32_t tiles = lay_out(target);
    map.start[kTileSegments] = n;
    if (tiles > w.n_tiles_max)
        return fail(PR_ERR_ARG, "tiles (%d) exceed the planned bound (%lld)", tiles,
                    (long long)w.n_tiles_max);
    bt.n_tiles = tiles;
    bt.tile_launch = grid;
    bt.unit_cost = unit_env ? unit_cost : 0;  // 0: chosen from the costs once they are known
    return PR_OK;
}

// Tiled pull, after the permutation (which wrote the first sort pass's
// histogram): the renumbered edges sorted by tile (stable, so each tile
// keeps them in increasing source order), the tile edge arrays, and the
// units (built on the host from the tiles' edge counts, read back).
int build_tiled(const PlanWs& w, const PlanScratch& s, int32_t n, int64_t nnz, PlanHost* host,
                hipStream_t stream, Built& bt) {
    const int64_t grid = bt.tile_launch;
    const bool unit_env = bt.unit_cost > 0;
    int64_t unit_cost = unit_env ? bt.unit_cost : kUnitCost;
    const TileMap& map = bt.map;
    const int32_t tiles = bt.n_tiles;

    // each tile's first edge: the in-edges of the rows before it
    int32_t* first = s.tile_first;
    uint32_t* in_rp_plan = s.in_rp_plan;
    PR_TRY(scan_exclusive(reinterpret_cast<const uint32_t*>(s.key), in_rp_plan, n, s.vsort.scan_ws,
                          stream));
    k_tile_first<<<grid_for((int64_t)tiles + 1, 1024), kBlock, 0, stream>>>(in_rp_plan, n, tiles, map,
                                                                            first);
    PR_LAUNCHED("tile starts");
    // The tile starts go to the host ahead of the sort's full pass: the host
    // waits for that copy alone and queues the work that needs them (the
    // light tiles' sort, the slot layout) while the pass runs.
    const size_t tp_bytes = sizeof(int32_t) * ((size_t)tiles + 1);
    PR_TRY(host_stage(host, tp_bytes));
    PR_HIP_TRY(hipMemcpyAsync(host->stage, first, tp_bytes, hipMemcpyDeviceToHost, stream));
    PR_HIP_TRY(hipEventRecord(host->stage_ev, stream));
    // Edges sorted by tile, stably (so by source inside a tile): keys are the
    // targets, values the sources (into s.order).  One full pass sorts by
    // min(tile, 255), from the histogram the permutation counted, taking each
    // edge's source from the plan-order row pointers (the permutation's row
    // windows are the pass's tiles); the edges of
    // tiles 255 and up (the light tiles, which come last and hold few edges)
    // form one range, [tp[255], nnz), which is then sorted by tile on its own.
    const int32_t* sorted_targets = nullptr;
    constexpr int32_t kCap = kRadixDigits - 1;
    if (nnz > 0) {
        RadixIn in{};
        in.count = nnz;
        in.n = n;
        in.keys = s.perm_ci;
        in.row_ptr = s.perm_rp;
        in.tile_row = s.tr.tile_row;
        in.tiles = map;
        in.tile_cap = kCap;
        in.error = s.tr.error;
        const RadixWs& rw = s.tr.sort;
        const int64_t T = radix_tiles(nnz);
        PR_TRY(scan_exclusive(rw.hist, rw.scanned, kRadixDigits * T, rw.scan_ws, stream));
        k_radix_scatter<kFromTileCsr><<<dim3((unsigned)T), kBlock, 0, stream>>>(
            in, 0, T, rw.scanned, rw.key[0], s.order);
        PR_LAUNCHED("radix scatter");
        sorted_targets = rw.key[0];
    }
    std::vector<int32_t> tp((size_t)tiles + 1);
    PR_HIP_TRY(hipEventSynchronize(host->stage_ev));
    std::memcpy(tp.data(), host->stage, tp_bytes);
    if (nnz > 0) {
        const int64_t lo = tiles > kCap ? tp[(size_t)kCap] : nnz;
        if (lo < nnz) {
            RadixIn rest{};
            rest.count = nnz - lo;
            rest.n = n;
            rest.keys = s.tr.sort.key[0] + lo;
            rest.vals = s.order + lo;
            rest.tiles = map;
            rest.tile_base = kCap;
            rest.error = s.tr.error;
            // scratch: the other ping-pong pair, and the sort's inputs (free now)
            int32_t* const sk[2] = {s.tr.sort.key[1], s.perm_ci};
            int32_t* const sv[2] = {s.tr.sort.val[1], s.src_of};
            PR_TRY(radix_sort_to<kFromTileTargets>(rest, vertex_bits(tiles - kCap), s.tr.sort.key[0] + lo,
                                                   s.order + lo, sk, sv, s.tr.sort, stream));
        }
    }
    std::vector<int32_t> sp((size_t)tiles + 1, 0);
    {
        int64_t q = 0;
        for (int32_t t = 0; t < tiles; ++t) {
            q += ceil_div((int64_t)(tp[(size_t)t + 1] - tp[(size_t)t]), kEdgeBlock) * kEdgeBlock;
            if (q > w.n_edge_slots_max || q > INT32_MAX)
                return fail(PR_ERR_ARG, "tile edge slots exceed the planned bound");
            sp[(size_t)t + 1] = (int32_t)q;
        }
    }
    const int64_t slots = sp[(size_t)tiles];
    bt.n_slots = slots;
    // tile slots and sector starts per chunk of slots (s.perm_ci, scratch of
    // the sort, is free again and takes the counts), then the chunks' cost
    // prefix, scanned on the device into s.src_of (free too) and read back
    // through the pinned stage, which first carries the slot starts up
    const int32_t chunks = (int32_t)ceil_div(slots, kSectorChunk);
    const size_t sp_bytes = align_up(sizeof(int32_t) * sp.size());
    PR_TRY(host_stage(host, sp_bytes + sizeof(uint64_t) * ((size_t)chunks + 1)));
    std::memcpy(host->stage, sp.data(), sizeof(int32_t) * sp.size());
    PR_HIP_TRY(hipMemcpyAsync(w.tile_ptr, host->stage, sizeof(int32_t) * sp.size(),
                              hipMemcpyHostToDevice, stream));
    const int64_t* cp = reinterpret_cast<const int64_t*>(host->stage + sp_bytes);
    if (nnz > 0) {
        int32_t* counts = s.perm_ci;
        // chunks <= nnz / 16 + 1 (a non-empty tile pads at most 255 slots per
        // edge), so both arrays fit the nnz words of s.src_of
        uint64_t* cost = reinterpret_cast<uint64_t*>(s.src_of);
        uint64_t* prefix = cost + chunks + 1;
        PR_TRY(fill_u32(reinterpret_cast<uint32_t*>(counts), 0u, chunks, stream));
        const int64_t n_blocks = slots / kEdgeBlock;
        k_tile_blocks<<<grid_for(n_blocks * kWave, 2048), kBlock, 0, stream>>>(
            sorted_targets, s.order, map, first, w.tile_ptr, tiles, n_blocks, w.tsrc, w.tdst,
            w.tblk, counts);
        PR_LAUNCHED("tile blocks");
        int64_t weight = nnz / grid < kWgEdgesMid ? kSectorWeightFew : kSectorWeight;
        if (const char* env = std::getenv("PR_SECTOR_WEIGHT"))  // tuning knob: cost per sector
            if (std::atoll(env) >= 0) weight = std::atoll(env);
        k_chunk_costs<<<grid_for(chunks, 1024), kBlock, 0, stream>>>(counts, slots, chunks, weight, cost);
        PR_LAUNCHED("chunk costs");
        PR_TRY(scan_exclusive(cost, prefix, chunks, s.tr.sort.scan_ws, stream));
        PR_HIP_TRY(hipMemcpyAsync(host->stage + sp_bytes, prefix,
                                  sizeof(uint64_t) * ((size_t)chunks + 1), hipMemcpyDeviceToHost,
                                  stream));
    } else {
        std::memset(host->stage + sp_bytes, 0, sizeof(uint64_t));
    }
    // The device has nothing else queued until the units are cut, so the host
    // polls for the copy rather than sleep in a synchronize: waking from one
    // took about 150 us after a 2 ms wait here (the device idles meanwhile).
    PR_HIP_TRY(hipEventRecord(host->stage_ev, stream));
    for (;;) {
        const hipError_t q = hipEventQuery(host->stage_ev);
        if (q == hipSuccess) break;
        if (q != hipErrorNotReady) PR_HIP_TRY(q);
        std::this_thread::yield();
    }
    // cost prefix at slot e, linear inside a chunk
    auto cost_at = [&](int64_t e) -> double {
        if (e >= slots) return (double)cp[(size_t)chunks];
        const int64_t c = e / kSectorChunk, r = e - c * kSectorChunk;
        const int64_t len = (c + 1 < chunks ? (int64_t)kSectorChunk : slots - c * kSectorChunk);
        return (double)cp[(size_t)c] + (double)(cp[(size_t)c + 1] - cp[(size_t)c]) * (double)r / (double)len;
    };
    // first block in [lo, hi] whose cost prefix reaches `want` (hi if none).
    // The prefix does not decrease, so the search first narrows [lo, hi] by
    // whole chunks, using the prefix at chunk starts (where cost_at is
    // exactly cp), then steps through the at most kBlocksPerChunk blocks left.
    constexpr int64_t kBlocksPerChunk = kSectorChunk / kEdgeBlock;
    auto block_at = [&](int64_t lo, int64_t hi, double want) -> int64_t {
        int64_t c_lo = ceil_div(lo, kBlocksPerChunk), c_hi = hi / kBlocksPerChunk;
        if (c_lo <= c_hi && (double)cp[(size_t)c_lo] < want) {
            // last chunk start in [c_lo, c_hi] below want
            while (c_lo < c_hi) {
                const int64_t mid = c_lo + (c_hi - c_lo + 1) / 2;
                if ((double)cp[(size_t)mid] < want)
                    c_lo = mid;
                else
                    c_hi = mid - 1;
            }
            lo = c_lo * kBlocksPerChunk;  // cost_at(lo) < want: the answer is later
            // inside chunk c_lo the prefix is linear: jump to one block before
            // where it reaches want, then step
            const double c0 = (double)cp[(size_t)c_lo];
            const double dc = (double)(cp[(size_t)c_lo + 1] - cp[(size_t)c_lo]);
            if (dc > 0.0) {
                const int64_t len = (c_lo + 1 < chunks ? (int64_t)kSectorChunk
                                                       : slots - c_lo * (int64_t)kSectorChunk);
                const int64_t k = (int64_t)((want - c0) * (double)len / (dc * kEdgeBlock)) - 1;
                if (k > 0) lo += k < kBlocksPerChunk ? k : kBlocksPerChunk - 1;
                if (lo > hi) lo = hi;
                while (lo > 0 && lo > c_lo * kBlocksPerChunk && cost_at(lo * kEdgeBlock) >= want) --lo;
            }
        }
        for (; lo < hi; ++lo)
            if (cost_at(lo * kEdgeBlock) >= want) break;
        return lo;
    };

    // The unit cost from the total: when the tiles at kUnitCost would give
    // fewer than two units per workgroup, the cost is (total cost) /
    // (2 * grid), and a tile of few rows may then be cut into units down to
    // min_unit_edges(rows) edges (kMinUnitEdges otherwise): the hubs' tiles
    // of such a graph would else be its longest units.  Otherwise it is
    // kUnitShare * (total cost) / grid.
    bool fine_cuts = false;
    if (!unit_env && tiles > 0) {
        const double total = cost_at(slots) - cost_at(0);
        int64_t units = 0;
        for (int32_t t = 0; t < tiles; ++t) {
            const int64_t e = sp[(size_t)t + 1] - sp[(size_t)t];
            const int64_t c = (int64_t)std::ceil((cost_at(sp[(size_t)t + 1]) - cost_at(sp[(size_t)t])) /
                                                 (double)unit_cost);
            const int64_t cmax = ceil_div(e, kMinUnitEdges);
            units += c < 1 ? 1 : (c > cmax ? cmax : c);
        }
        if (units < 2 * grid) {
            const int64_t t2 = (int64_t)(total / (double)(2 * grid));
            unit_cost = t2 > kMinUnitCost ? t2 : kMinUnitCost;
            fine_cuts = true;
        } else {
            const int64_t t1 = (int64_t)(kUnitShare * total / (double)grid);
            unit_cost = t1 > kMinUnitCost ? t1 : kMinUnitCost;
        }
    }

    // Tiles, units and slots.  A tile is cut at block boundaries into
    // min(ceil(cost / unit_cost), ceil(slots / that minimum)) units of about
    // equal cost; all units are then ordered by decreasing estimated cost.
    bt.tiles.resize((size_t)tiles);
    std::vector<std::pair<int64_t, TileUnit>> list;
    int64_t slot = 0;
    for (int seg = 0; seg < kTileSegments; ++seg) {
        const int32_t end = map.start[seg + 1];
        const int32_t last = seg + 1 < kTileSegments ? map.tile0[seg + 1] : tiles;
        for (int32_t t = map.tile0[seg]; t < last; ++t) {
            const int32_t row0 = map.start[seg] + ((t - map.tile0[seg]) << map.shift[seg]);
            const int32_t rows = (end - row0) < (1 << map.shift[seg]) ? end - row0 : 1 << map.shift[seg];
            bt.tiles[(size_t)t] = Tile{row0, rows};
            const int32_t e0 = sp[(size_t)t], e1 = sp[(size_t)t + 1];
            const double c0 = cost_at(e0), c1 = cost_at(e1);
            const int64_t per_unit = kUnitOverhead + kTileRowWeight * rows;
            int64_t count = (int64_t)std::ceil((c1 - c0) / (double)unit_cost);
            int64_t count_max =
                ceil_div((int64_t)(e1 - e0), fine_cuts ? min_unit_edges(rows) : kMinUnitEdges);
            if (count_max > (e1 - e0) / kEdgeBlock) count_max = (e1 - e0) / kEdgeBlock;
            if (count > count_max) count = count_max;
            const int64_t count_min = ceil_div((int64_t)(e1 - e0), kMaxUnitEdges);
            if (count < count_min) count = count_min;
            if (count <= 1) {
                list.push_back({(int64_t)(c1 - c0) + per_unit, TileUnit{t, e0, e1, -1, row0, rows, -1, 1}});
                continue;
            }
            // No 128-byte line holds slots of two cut tiles, so the unit
            // that finishes a tile reads no line that another tile's finish
            // (maybe on the same XCD, earlier in the launch) has read: what
            // its device-scope loads return never depends on whether an L2
            // kept such a line.
            slot = ceil_div(slot, kSlotAlign) * kSlotAlign;
            if (slot + count * rows > w.n_partial_max)
                return fail(PR_ERR_ARG, "tile slots exceed the planned bound");
            const int32_t fix = (int32_t)bt.fixes.size();
            bt.fixes.push_back(TileFix{row0, rows, (int32_t)slot, (int32_t)count});
            int64_t a = e0;
            for (int64_t j = 0; j < count; ++j) {
                const int64_t b =
                    j + 1 == count ? e1
                                   : kEdgeBlock * block_at(a / kEdgeBlock + 1,
                                                           e1 / kEdgeBlock - (count - 1 - j),
                                                           c0 + (c1 - c0) * (double)(j + 1) / (double)count);
                const TileUnit u{t, (int32_t)a, (int32_t)b, (int32_t)(slot + j * rows), row0, rows, fix,
                                  (int32_t)count};
                list.push_back({(int64_t)(cost_at(b) - cost_at(a)) + per_unit, u});
                a = b;
            }
            slot += count * rows;
        }
    }
    std::stable_sort(list.begin(), list.end(),
                     [](const std::pair<int64_t, TileUnit>& x, const std::pair<int64_t, TileUnit>& y) {
                         return x.first > y.first;
                     });
    bt.units.clear();
    for (const auto& u : list) bt.units.push_back(u.second);
    if ((int64_t)bt.units.size() > w.n_units_max || (int64_t)bt.fixes.size() > w.n_fixes_max)
        return fail(PR_ERR_ARG, "tile units exceed the planned bound");
    bt.n_units = (int32_t)bt.units.size();
    bt.n_fixes = (int32_t)bt.fixes.size();
    // A cut tile is finished inside k_tile, by whichever of its units
    // completes it last, when that finish is short: its last unit adds the
    // other (count - 1) * rows slot entries, at most kFuseSlots.  A longer
    // finish would hold the launch's end back; k_tilefix does those tiles
    // after k_tile.  The tiles finished inside come first in the list (a
    // unit's fix indexes them; -1 for a unit of a tile left to k_tilefix).
    {
        int mode = -1;  // per tile
        if (const char* env = std::getenv("PR_TILE_FUSE"))  // tuning knob: 0 all k_tilefix, 1 all k_tile
            mode = std::atoi(env) != 0 ? 1 : 0;
        int64_t fuse_slots = kFuseSlots;
        if (const char* env = std::getenv("PR_FUSE_SLOTS"))  // tuning knob: the per-tile limit
            if (std::atoll(env) >= 0) fuse_slots = std::atoll(env);
        std::vector<TileFix> inside, outside;
        std::vector<int32_t> remap(bt.fixes.size());
        for (size_t i = 0; i < bt.fixes.size(); ++i) {
            const TileFix& f = bt.fixes[i];
            const bool in = mode < 0 ? (int64_t)(f.count - 1) * f.rows <= fuse_slots : mode == 1;
            remap[i] = in ? (int32_t)inside.size() : -1;
            (in ? inside : outside).push_back(f);
        }
        bt.n_fused = (int32_t)inside.size();
        bt.fixes = inside;
        bt.fixes.insert(bt.fixes.end(), outside.begin(), outside.end());
        for (TileUnit& u : bt.units)
            if (u.fix >= 0) u.fix = remap[(size_t)u.fix];
    }
    bt.fix_rows.assign(1, 0);
    bt.fix_win.clear();
    {
        const int32_t n_out = bt.n_fixes - bt.n_fused;
        for (int32_t i = 0; i < n_out; ++i)
            bt.fix_rows.push_back(bt.fix_rows.back() + bt.fixes[(size_t)(bt.n_fused + i)].rows);
        // for k_tilefix: the last of its cut tiles whose rows start at or
        // before row w * kFixBlock of those tiles' rows, for every window w
        const int32_t total = bt.fix_rows.back();
        int32_t i = 0;
        for (int32_t g0 = 0; g0 < total; g0 += kFixBlock) {
            while (i + 1 < n_out && bt.fix_rows[(size_t)i + 1] <= g0) ++i;
            bt.fix_win.push_back(i);
        }
    }
    if (bt.fix_win.empty()) bt.fix_win.push_back(0);
    // The work lists go up in one copy: packed one after another from the
    // start of their workspace region (which holds each at its largest), from
    // the pinned stage (nothing uses it now: the read-back above was waited
    // for).
    {
        const void* src[5] = {bt.tiles.data(), bt.units.data(), bt.fixes.data(),
                              bt.fix_rows.data(), bt.fix_win.data()};
        const size_t bytes[5] = {sizeof(Tile) * bt.tiles.size(), sizeof(TileUnit) * bt.units.size(),
                                 sizeof(TileFix) * bt.fixes.size(),
                                 sizeof(int32_t) * bt.fix_rows.size(),
                                 sizeof(int32_t) * bt.fix_win.size()};
        size_t off[5], total = 0;
        for (int i = 0; i < 5; ++i) {
            off[i] = total;
            total += align_up(bytes[i]);
        }
        char* region = reinterpret_cast<char*>(w.tiles);
        if (total > (size_t)(reinterpret_cast<char*>(w.fix_done) - region))
            return fail(PR_ERR_ARG, "work lists exceed their workspace region");
        PR_TRY(host_stage(host, total));
        for (int i = 0; i < 5; ++i)
            if (bytes[i]) std::memcpy(host->stage + off[i], src[i], bytes[i]);
        PR_HIP_TRY(hipMemcpyAsync(region, host->stage, total, hipMemcpyHostToDevice, stream));
        bt.dev_tiles = reinterpret_cast<const Tile*>(region + off[0]);
        bt.dev_units = reinterpret_cast<const TileUnit*>(region + off[1]);
        bt.dev_fixes = reinterpret_cast<const TileFix*>(region + off[2]);
        bt.dev_fix_rows = reinterpret_cast<const int32_t*>(region + off[3]);
        bt.dev_fix_win = reinterpret_cast<const int32_t*>(region + off[4]);
    }
    // every cut tile's count of finished units starts at zero (the unit that
    // finishes a tile sets it back to zero)
    if (bt.n_fused > 0) PR_TRY(fill_u32(w.fix_done, 0u, bt.n_fused, stream));
    bt.tile_grid = (int32_t)(grid < bt.n_units ? grid : (bt.n_units > 0 ? bt.n_units : 1));
    return PR_OK;
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
    return ws_bytes_needed(n, nnz);
}

extern "C" size_t pr_plan_scratch_bytes(int32_t n, int64_t nnz) {
    if (n < 1 || nnz < 0 || nnz > INT32_MAX) return 0;
    return carve_scratch(nullptr, n, nnz).bytes;
}

namespace pr {
namespace {
int plan_create(pr_plan** plan_out, int32_t n, int64_t nnz, const int32_t* out_rp,
                const int32_t* out_ci, const PlanWs& w, const PlanScratch& s, uint32_t flags,
                int dev, int cus, PlanHost* host, hipStream_t stream);
}  // namespace
}  // namespace pr

extern "C" int pr_plan_create(pr_plan** plan_out, int32_t n, int64_t nnz, const int32_t* out_rp,
                              const int32_t* out_ci, void* ws, size_t ws_bytes, void* scratch,
                              size_t scratch_bytes, uint32_t flags, void* stream_v) {
    if (!plan_out) return fail(PR_ERR_ARG, "plan_out is null");
    *plan_out = nullptr;
    PR_TRY(check_sizes(n, nnz));
    if (flags & ~(PR_VALIDATE | PR_PLAN_BUCKETED))
        return fail(PR_ERR_ARG, "unknown flags 0x%x", flags);
    if (!out_rp || !ws || !scratch || (nnz > 0 && !out_ci))
        return fail(PR_ERR_ARG, "null pointer argument");
    const bool tiled = !(flags & PR_PLAN_BUCKETED);
    if (tiled && n > kTiledMaxVertices)
        return fail(PR_ERR_ARG, "a tiled plan takes n <= %d (got %d); PR_PLAN_BUCKETED takes more",
                    kTiledMaxVertices, n);
    PlanWs w = carve_ws(ws, n, nnz, tiled);
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
    PlanHost* host = nullptr;
    PR_TRY(host_take(&host));
    const int rc = plan_create(plan_out, n, nnz, out_rp, out_ci, w, s, flags, dev, cus, host, stream);
    if (rc != PR_OK) host_give(host);
    return rc;
}

namespace pr {
namespace {

int plan_create(pr_plan** plan_out, int32_t n, int64_t nnz, const int32_t* out_rp,
                const int32_t* out_ci, const PlanWs& w, const PlanScratch& s, uint32_t flags,
                int dev, int cus, PlanHost* host, hipStream_t stream) {
    const bool tiled = !(flags & PR_PLAN_BUCKETED);
    const bool validate = flags & PR_VALIDATE;
    uint32_t* err = s.tr.error;

    PR_TRY(fill_u32(err, 0u, 1, stream));
    if (validate) {
        PR_TRY(check_out_row_ptr(out_rp, n, nnz, err, stream));
        PR_TRY(read_error_word(err, stream, "pr_plan_create"));
    }

    // 1. Plan order: in-degree buckets, then decreasing out-degree.  The
    //    in-degrees are the row lengths of the transpose, whose row pointers
    //    come from a keys-only sort of the targets (perm_rp holds them until
    //    step 2 needs it).
    PR_TRY(indegree_row_ptr(n, nnz, out_ci, s.perm_rp, s.deg, s.count_chunks, s.vsort.scan_ws, s.tr,
                            stream));
    if (validate) PR_TRY(read_error_word(err, stream, "pr_plan_create"));
    // (cleared once the long in-degree kernels are queued: their launches'
    // host time then overlaps them)
    PR_TRY(fill_u32(reinterpret_cast<uint32_t*>(s.stats), 0u, 4 * kNumBuckets, stream));
    PR_TRY(fill_u32(reinterpret_cast<uint32_t*>(w.state), 0u, sizeof(RunState) / 4, stream));
    Bounds bounds;
    bucket_bounds(tiled, bounds.min_len);
    k_plan_keys<<<grid_for(n, 1024), kBlock, 0, stream>>>(s.perm_rp, out_rp, n, bounds, s.key,
                                                          s.stats);
    PR_LAUNCHED("plan keys");

    // Bucket ranges (hub bucket first), read back: a tiled plan lays out its
    // tiles before the permutation, which counts the edges per tile.  The
    // host waits for the copy alone, after queueing the work that does not
    // need it (the sort by plan key, the order, the permuted row pointers and
    // their windows), so the device runs that work while the host lays out
    // the tiles, with no gaps between its short kernels.
    unsigned long long stats[2 * kNumBuckets];
    PR_HIP_TRY(hipMemcpyAsync(host->stage, s.stats, sizeof stats, hipMemcpyDeviceToHost, stream));
    PR_HIP_TRY(hipEventRecord(host->stage_ev, stream));
    {
        RadixIn in{};
        in.count = n;
        in.n = n;
        in.keys = s.key;
        in.error = err;
        int32_t* sorted = nullptr;
        PR_TRY(radix_sort<kFromKeys>(in, 19, s.old_of, s.vsort, &sorted, stream));
    }
    // (s.key is free again: it holds the in-degrees in plan order from here)
    k_order<<<grid_for(n), kBlock, 0, stream>>>(s.old_of, out_rp, s.perm_rp, n, w.new_id, s.deg,
                                                reinterpret_cast<uint32_t*>(s.key), w.inv_out);
    PR_LAUNCHED("order");
    // row pointers of the out-edge CSR in plan order, and the permutation's
    // windows (the transpose's tile_row scratch is free until a bucketed
    // plan's transpose, after the permutation)
    PR_TRY(scan_exclusive(s.deg, reinterpret_cast<uint32_t*>(s.perm_rp), n, s.vsort.scan_ws,
                          stream));
    const int64_t perm_blocks = ceil_div(nnz, kBlock * kPermItems);
    if (nnz > 0) PR_TRY(window_rows(s.perm_rp, n, perm_blocks, s.tr.tile_row, stream));
    PR_HIP_TRY(hipEventSynchronize(host->stage_ev));
    std::memcpy(stats, host->stage, sizeof stats);
    int32_t row_begin[kNumBuckets + 1];  // indexed by bucket; hub rows start at 0
    {
        int64_t r = 0;
        for (int b = kHubBucket; b >= 0; --b) {
            row_begin[b] = (int32_t)r;
            r += (int64_t)stats[b];
        }
        row_begin[kNumBuckets] = (int32_t)r;  // == n
    }
    Built bt{};
    if (tiled) PR_TRY(lay_out_tiles(w, nnz, stats, row_begin, n, cus, bt));

    // 2. The out-edge CSR in plan order.
    if (nnz > 0) {
        k_permute_rows<<<dim3((unsigned)perm_blocks), kBlock, 0, stream>>>(
            s.perm_rp, s.tr.tile_row, s.old_of, w.new_id, out_rp, out_ci, n, nnz, s.perm_ci,
            bt.map, tiled ? s.tr.sort.hist : nullptr, perm_blocks);
        PR_LAUNCHED("permute rows");
    }

    // 3. The layout's work items.
    if (tiled)
        PR_TRY(build_tiled(w, s, n, nnz, host, stream, bt));
    else
        PR_TRY(build_bucketed(w, s, n, nnz, host, stats, row_begin, cus, stream, bt));
    if (validate) PR_TRY(read_error_word(err, stream, "pr_plan_create"));
    PR_HIP_TRY(hipStreamSynchronize(stream));  // host arrays must outlive the copies

    pr_plan* p = static_cast<pr_plan*>(std::calloc(1, sizeof(pr_plan)));
    if (!p) return fail(PR_ERR_ARG, "out of host memory");
    p->device = dev;
    p->n = n;
    p->nnz = nnz;
    p->new_id = w.new_id;
    p->inv_out = w.inv_out;
    p->tiled = tiled;
    p->in_rp = w.in_rp;
    p->in_ci = w.in_ci;
    p->xi = w.xi;
    p->contrib[0] = w.contrib0;
    p->contrib[1] = w.contrib1;
    p->items = w.items;
    p->n_items = bt.n_items;
    p->chunk_rows = w.chunk_rows;
    p->n_chunk_rows = bt.n_chunk_rows;
    p->hub_part = w.hub_part;
    p->part = w.part;
    p->part_stride = w.part_stride;
    p->n_batches = (int32_t)ceil_div(bt.n_items, kBatchItems);
    p->state = w.state;
    p->grid = bt.grid;
    p->fix_grid = bt.fix_grid;
    p->tile_map = bt.map;
    p->tsrc = w.tsrc;
    p->tdst = w.tdst;
    p->tblk = w.tblk;
    p->tile_ptr = w.tile_ptr;
    p->n_slots = bt.n_slots;
    p->tiles = bt.dev_tiles;
    p->n_tiles = bt.n_tiles;
    p->max_tile_rows = 0;
    for (const Tile& tl : bt.tiles) p->max_tile_rows = tl.rows > p->max_tile_rows ? tl.rows : p->max_tile_rows;
    p->units = bt.dev_units;
    p->n_units = bt.n_units;
    p->fixes = bt.dev_fixes;
    p->n_fused = bt.n_fused;
    p->fix_done = w.fix_done;
    p->fix_rows = bt.dev_fix_rows;
    p->fix_win = bt.dev_fix_win;
    p->n_fixes = bt.n_fixes;
    p->n_fix_rows = bt.fix_rows.empty() ? 0 : bt.fix_rows.back();
    p->partial = w.partial;
    p->tile_grid = bt.tile_grid;
    {
        const int64_t ig = ceil_div(n, kBlock);
        p->init_grid = (int32_t)(ig < kMaxGrid ? ig : kMaxGrid);
    }
    for (int b = 0; b < kNumBuckets; ++b) {
        p->bucket_min[b] = bounds.min_len[b];
        p->row_begin[b] = row_begin[b];
        p->bucket_edges[b] = (int64_t)stats[kNumBuckets + b];
        p->bucket_items[b] = bt.items_of[b];
    }
    p->row_begin[kNumBuckets] = row_begin[kNumBuckets];
    p->bucket_items[kKindChunk] = bt.items_of[kKindChunk];

    p->host = host;
    *plan_out = p;
    return PR_OK;
}

}  // namespace
}  // namespace pr

extern "C" int pr_plan_destroy(pr_plan* p) {
    if (!p) return PR_OK;
    host_give(p->host);
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

extern "C" int pr_plan_tiles(const pr_plan* p, const int32_t** tile_src, const uint16_t** tile_row,
                             const int32_t** tile_block, const int32_t** tile_ptr, int32_t* n_tiles,
                             int32_t* row0, int32_t* rows) {
    if (!p) return fail(PR_ERR_ARG, "plan is null");
    if (!p->tiled) return fail(PR_ERR_ARG, "the plan was built with PR_PLAN_BUCKETED");
    if (tile_src) *tile_src = p->tsrc;
    if (tile_row) *tile_row = p->tdst;
    if (tile_block) *tile_block = p->tblk;
    if (tile_ptr) *tile_ptr = p->tile_ptr;
    if (n_tiles) *n_tiles = p->n_tiles;
    const TileMap& m = p->tile_map;
    for (int seg = 0; seg < kTileSegments; ++seg) {
        const int32_t last = seg + 1 < kTileSegments ? m.tile0[seg + 1] : p->n_tiles;
        for (int32_t t = m.tile0[seg]; t < last; ++t) {
            const int32_t r0 = m.start[seg] + ((t - m.tile0[seg]) << m.shift[seg]);
            const int32_t span = 1 << m.shift[seg];
            if (row0) row0[t] = r0;
            if (rows) rows[t] = (m.start[seg + 1] - r0) < span ? m.start[seg + 1] - r0 : span;
        }
    }
    return PR_OK;
}
