// The iteration plan: the graph renumbered and transposed, its rows split into
// degree buckets and cut into work items, plus the per-run scratch and the
// launch shape of the iteration kernels.
#pragma once

#include "radix.hpp"

namespace pr {

// Degree buckets of the pull product ("gpu-graph-study", PageRank T4: thread /
// warp / block per vertex by degree), re-cut for 64-lane wavefronts.  Bucket
// b holds the in-rows whose length is in [bucket_min[b], bucket_min[b+1]) and
// gives each row kBucketGroup[b] lanes: one lane, a 4- or 16-lane slice of a
// wavefront, a whole wavefront, or a whole 256-lane workgroup (the hubs).
constexpr int kNumBuckets = 5;
constexpr int kHubBucket = kNumBuckets - 1;
constexpr int kBucketGroup[kNumBuckets] = {1, 4, 16, 64, 256};
constexpr int32_t kDefaultBucketMin[kNumBuckets] = {0, 5, 17, 65, 1025};
// The tiled layout uses the buckets only to group rows of similar length into
// tiles; these bounds were the fastest in sweeps on R-MAT scale 23.
constexpr int32_t kDefaultTileBucketMin[kNumBuckets] = {0, 9, 33, 129, 2049};
constexpr int32_t kMinHubLength = 257;  // lower bound for a tuned hub threshold

// Work items.  Wavefronts of the iteration kernel take batches of
// kBatchItems consecutive items from a queue (one atomic increment per
// batch) until the queue is empty:
//   * kind 0..3: a range of rows of one bucket whose cost (edges + kRowCost per
//     row) is about kItemCost;
//   * kind 4: one hub row, whole (at most kHubChunk edges);
//   * kind 5: kHubChunk consecutive edges of a longer hub row; its gathered
//     sum goes to a slot, and a second kernel adds the slots of the row, in
//     order, and applies the update.
// Hub items come first in the list, so the longest work starts first.
constexpr int64_t kItemCost = 2048;
constexpr int64_t kRowCost = 8;
constexpr int32_t kHubChunk = 4096;
constexpr int kKindChunk = 5;
constexpr int kBatchItems = 4;

// The queue is split in kQueues interleaved queues: queue q holds the
// batches q, q + kQueues, ...  A wavefront starts on queue blockIdx %
// kQueues (workgroups are dealt to the XCDs round-robin) and moves on to the
// others once its own is empty.  Each head sits on its own 256-byte line.
constexpr int kQueues = 8;

// The iteration kernel runs kIterBlocksPerCU workgroups of kIterBlock lanes
// per CU; each keeps the contributions of the first kHotSources plan ids --
// the sources with the most out-edges -- in LDS (160 KB per CU on gfx950)
// for the whole launch.
#ifndef PR_ITER_BLOCKS_PER_CU
#define PR_ITER_BLOCKS_PER_CU 1
#endif
constexpr int kIterBlock = 1024;
constexpr int kIterWaves = kIterBlock / kWave;
constexpr int kIterBlocksPerCU = PR_ITER_BLOCKS_PER_CU;
constexpr int32_t kHotSources = (163840 / kIterBlocksPerCU - 1024) / 4;

struct WorkItem {
    int32_t kind;
    int32_t lo;   // kinds 0..3: first row; kinds 4, 5: first edge
    int32_t hi;   // one past the last row / edge
    int32_t aux;  // kind 4: the row; kind 5: the slot
};

// A hub row split into chunks: slots [first, first + count) hold its sums.
struct ChunkRow {
    int32_t row;
    int32_t first;
    int32_t count;
    int32_t pad;
};

// Upper bounds used to size the plan's workspace.
inline int64_t max_hub_rows(int64_t nnz) { return nnz / kMinHubLength + 1; }
// A chunked row has more than kHubChunk edges, so there are at most
// nnz / kHubChunk of them and at most twice that many chunks.
inline int64_t max_chunk_rows(int64_t nnz) { return nnz / kHubChunk + 1; }
inline int64_t max_chunk_slots(int64_t nnz) { return 2 * (nnz / kHubChunk) + 2; }
inline int64_t max_items(int32_t n, int64_t nnz) {
    return ceil_div(nnz + kRowCost * (int64_t)n, kItemCost) + kNumBuckets + max_hub_rows(nnz) +
           max_chunk_slots(nnz);
}
// Workgroups of the iteration kernels (and partial-sum slots).
constexpr int kMaxGrid = 8192;
constexpr int kFixBlock = 256;
// The finalize kernel runs as one workgroup of this many lanes.
constexpr int kFinalBlock = 1024;

// ------------------------------------------------------------ tiled pull
//
// The default iteration.  Rows are cut into tiles: blocks of consecutive plan
// ids inside one degree bucket, 2^k rows each, k chosen per bucket so that a
// tile holds about kTileTargetEdges in-edges (hub tiles are a few hundred
// rows, light tiles kTileMaxRows).  A tile's in-edges are stored grouped by
// tile and, inside a tile, by increasing source, as (source id, row offset in
// the tile) pairs.  A workgroup streams a tile's edges in that order, so
// consecutive lanes read neighbouring contributions (coalesced), and adds
// each one into the row's accumulator in LDS.  Accumulators are 64-bit fixed
// point (contribution * 2^shift, truncated): integer addition is exact and
// order-free, so the sums do not depend on scheduling.  A tile whose
// estimated cost exceeds the unit cost is cut into units of about equal
// cost; each unit writes its accumulators to a slot of `partial`.  When a
// cut tile has at most kFuseSlots slot entries besides one unit's own, the
// unit that finishes it last adds the other slots and applies the update;
// k_tilefix finishes the other cut tiles after k_tile (and is not launched
// when there are none), because one workgroup adding that many entries
// holds the launch's end back.
//
// Cost estimate of a range of tile edges, in edge-equivalents: its edges,
// plus kSectorWeight per distinct 64-byte sector of contributions it gathers
// (sources in increasing order, so a new sector starts where src >> 4
// changes), plus, per unit, kTileRowWeight per row of the tile (clearing and
// reading the accumulators) and kUnitOverhead.  The row and unit weights
// are fitted to per-unit timings of k_tile on gfx950.  The sector weight and
// the unit cost were then re-tuned together by sweeping the whole launch
// (R-MAT 23, original and shuffled ids: weight 6-14, cost 0.7-1.0 M): a
// sector fetched from outside the CU costs about ten edges' worth of
// streaming and adding, and at weight 6 the sparse-source units ran up to 60%
// longer than units of the same estimate, ending the launch late.  Graphs
// with little work per workgroup (R-MAT 18) keep weight 6, their best.
// Units go to the queue in decreasing estimated cost, so the longest start
// first.  A unit costs kUnitShare of one workgroup's share of the total
// (graphs with at least two units per workgroup at kUnitCost; smaller ones
// get half a share, see build_tiled): fewer, longer units cut fewer tiles
// (less partial traffic, fewer accumulator passes) while the longest still
// ends with the rest.  Swept on gfx950 with every workgroup's wavefronts
// sharing a unit's blocks (R-MAT 22, 23, 24; shares 0.6-1.1 of a
// workgroup's): 0.95 was best or within 2% of best on each (R-MAT 23 287 ->
// 274 us, R-MAT 22 158 -> 149 us, R-MAT 24 734 -> 651 us against the fixed
// cost of 900K before).
constexpr int32_t kTileMaxRows = 16384;         // 128 KB of accumulators
constexpr int32_t kTileMinRows = 64;
// Rows per tile at most, by edges per workgroup of the launch: a tile's
// unit clears, reads and updates every row of the tile, so on a graph with
// little work per workgroup the tiles of the light rows (many rows, few
// edges each) would be the longest units.  Measured on gfx950 (R-MAT 18,
// 21, 23, the 27-point stencil): 4096 rows below 2^16 edges per workgroup,
// 8192 below 2^19, else kTileMaxRows.
constexpr int32_t kTileRowsFew = 4096;
constexpr int32_t kTileRowsMid = 8192;
constexpr int64_t kWgEdgesMid = 1 << 16;
constexpr int64_t kWgEdgesMany = 1 << 19;
// Tiles of a light segment (fewer than kLightDeg in-edges per row: one gather
// per edge, no source reuse to lose) hold at most kTileRowsLight rows, so the
// last units of the schedule are short (R-MAT 23: 319 -> 318 us).
constexpr int32_t kTileRowsLight = 8192;
constexpr int64_t kLightDeg = 9;
constexpr int64_t kTileTargetEdges = 1 << 22;  // default; PR_TILE_EDGES overrides
constexpr int64_t kMinTileTarget = 1 << 12;     // smaller graphs' tiles go down to this
constexpr int64_t kUnitCost = 900000;           // sets which graphs are small; PR_UNIT_COST overrides
constexpr double kUnitShare = 0.95;
constexpr int64_t kMinUnitCost = 1 << 15;       // smaller graphs' units go down to this
constexpr int64_t kMinUnitEdges = 1 << 17;     // a unit of a cut tile has at least
constexpr int64_t kMinUnitEdgesFloor = 1 << 12; //   min(kMinUnitEdges, max(this,
constexpr int64_t kUnitEdgesPerRow = 64;        //   this * rows)) edges (min_unit_edges)
constexpr int64_t kMaxUnitEdges = 1 << 26;     // and at most this many
// A cut tile is finished in k_tile when (count - 1) * rows <= kFuseSlots
// (PR_FUSE_SLOTS overrides).  Measured on gfx950 when one rule held for a
// whole plan (iteration time, finish in k_tile against k_tilefix): R-MAT 18,
// largest 896: 22.1 against 25.5 us; R-MAT 21, 184,320: 85.5 against
// 87.0 us; R-MAT 23, 491,520: 311.5 against 304.1 us.  Per tile, R-MAT 23
// finishes all but its most-cut tiles inside: 274.3 -> 270.7 us.  Limits
// from 0 to 2^22: R-MAT 23 271 us from 2^16 to 2^18, 296 us from 2^19 (its
// most-cut tile then finishes inside); R-MAT 21 82-84 us below 2^18, 78 us
// from 2^18.
constexpr int64_t kFuseSlots = 1 << 18;
constexpr int32_t kTiledMaxVertices = 1 << 30; // contribution byte offsets fit 32 bits
constexpr int kSectorShift = 4;                 // 16 fp32 contributions per 64-byte sector
constexpr int64_t kSectorWeight = 10;           // default; PR_SECTOR_WEIGHT overrides
constexpr int64_t kSectorWeightFew = 6;         // below kWgEdgesMid edges per workgroup
constexpr int64_t kTileRowWeight = 1;
constexpr int64_t kUnitOverhead = 27000;

// The fewest edges a unit of a cut tile of `rows` rows may have: a unit
// writes one partial slot per row, so a tile of few rows (the hubs') can be
// cut finely and one of many rows only coarsely.  rows / min_unit_edges(rows)
// is at most max(1 / kUnitEdgesPerRow, kTileMaxRows / kMinUnitEdges) = 1/8.
inline int64_t min_unit_edges(int64_t rows) {
    const int64_t e = kUnitEdgesPerRow * rows;
    return e < kMinUnitEdgesFloor ? kMinUnitEdgesFloor : (e > kMinUnitEdges ? kMinUnitEdges : e);
}
constexpr int32_t kSectorChunk = 4096;          // edges per sector count read back

// Tile edges are stored in blocks of kEdgeBlock: each tile's edges padded to
// a whole number of blocks, and each block transposed so that lane l of a
// wavefront finds edges l, l + 64, l + 128 and l + 192 of the block in one
// 16-byte load of sources and one 8-byte load of row offsets (and lane l of
// the gather for edge l + 64*i reads next to lane l + 1's: still coalesced).
// A padding edge repeats the tile's last source and adds into row
// kTrashRow, an accumulator that is never read.
constexpr int32_t kEdgeBlock = 4 * kWave;
constexpr int32_t kTrashRow = kTileMaxRows;

// Narrow blocks.  Inside a block the sources do not decrease, so the block
// spans [first, last] = its edges 0 and 255.  When last - first < 2^16 the
// block is narrow: tile_block[b] = first, and each slot holds
// (source - first) | row << 16, so one 16-byte load gives a lane four whole
// edges.  Otherwise tile_block[b] = -1 and the slots keep the 32-bit sources,
// with the rows in the 16-bit row array.
constexpr int32_t kNarrowSpan = 1 << 16;

// Storage slot of edge k of a tile, relative to the tile's first slot.
__host__ __device__ inline int64_t block_slot(int64_t k) {
    return (k & ~(int64_t)(kEdgeBlock - 1)) | ((k & (kWave - 1)) << 2) | ((k >> 6) & 3);
}
constexpr int kFxShiftMax = 56;                 // 2^-56 resolution when sum|x| <= 1

static_assert(kTileSegments == kNumBuckets, "one tile segment per degree bucket");

struct Tile {
    int32_t row0;
    int32_t rows;
};

// A unit of k_tile: edges [e0, e1) of one tile (rows [row0, row0 + rows)).
// slot < 0: the unit is the whole tile and applies the update; otherwise the
// tile is cut tile `fix`, cut into `count` units, and the unit's
// accumulators go to partial[slot, slot + rows).
struct TileUnit {
    int32_t tile;
    int32_t e0;
    int32_t e1;
    int32_t slot;
    int32_t row0;
    int32_t rows;
    int32_t fix;    // -1 for a whole tile
    int32_t count;  // 1 for a whole tile
};

// A tile cut into `count` units: unit j's accumulators sit at
// partial[first + j*rows, + rows).  In a plan that finishes cut tiles in
// k_tile, the unit that finishes last adds the others' slots to its own
// accumulators and applies the update; otherwise k_tilefix does, after
// k_tile.
struct TileFix {
    int32_t row0;
    int32_t rows;
    int32_t first;
    int32_t count;
};

constexpr int kSumSlots = 4;  // RunState::tsum lines per iteration

// Device-resident run state.  Written by the finalize and init kernels, read
// by the next launches (kernel boundaries order the accesses); the queue
// heads are incremented atomically by the iteration kernels.
struct RunState {
    double dmass;     // D of the vector the next iteration starts from
    double fx_scale;  // 2^fx_shift: contribution -> fixed point (tiled pull)
    double fx_unit;   // 2^-fx_shift
    int32_t stop;     // 1 once an iteration met the tolerance
    int32_t iters;    // that iteration's number
    int32_t signed_contrib;  // 1 if the start vector had a negative entry
    int32_t fx_shift;
    uint32_t pad[54];
    uint32_t queue[kQueues][64];  // queue heads at [q][0]
    // Tiled pull: iteration t adds its L1 distance, dangling mass and sum of
    // x' into tsum[t % 3][s][0..2] in fixed point (times 2^fx_shift), exact
    // and in any order, workgroup b into line s = b % kSumSlots (one line
    // each: the workgroups finish together, and adds to one address
    // serialize); iteration t + 1 adds the lines up and clears
    // tsum[(t + 2) % 3].
    long long tsum[3][kSumSlots][16];
};

// Launches of the gather kernel that PR_RECORD_EVENTS times one by one.
constexpr int kTimedLaunches = 64;

// Host copy of the fields pr_run polls.
struct RunStatus {
    int32_t stop;
    int32_t iters;
};

// A plan's host-side resources: timing events, the pinned status pair pr_run
// polls, and a pinned staging buffer for the plan builder's read-backs and
// uploads.  They outlive plans: pr_plan_destroy returns them to a pool of the
// device, and the next pr_plan_create takes them from there, so building a
// plan creates no events and allocates no host memory once the pool holds
// enough for it.
struct PlanHost {
    int device;
    hipEvent_t ev_begin, ev_end;
    hipEvent_t kernel_ev[2][kTimedLaunches];  // around k_tile (or k_iterate) launches
    hipEvent_t chunk_ev[2];
    hipEvent_t stage_ev;  // a plan's read-back into `stage` is done
    RunStatus* status;    // pinned, [2]
    char* stage;        // pinned staging buffer of stage_bytes
    size_t stage_bytes;
    PlanHost* next;     // pool link
};

// A PlanHost of the current device (from the pool, or new), and back.
int host_take(PlanHost** out);
void host_give(PlanHost* h);
// Makes h->stage hold at least `bytes` (its contents are not kept).
int host_stage(PlanHost* h, size_t bytes);

}  // namespace pr

struct pr_plan {
    int device;
    int32_t n;
    int64_t nnz;
    bool tiled;            // tiled pull (default) or bucketed pull (PR_PLAN_BUCKETED)
    // plan order: vertex v of the caller sits at p = new_id[v]; rows of bucket
    // b are the plan ids [row_begin[b], row_begin[b+1]), hub rows first
    const int32_t* new_id;
    const float* inv_out;  // 1/outdeg, 0 for a dangling vertex, plan order
    const int32_t* in_rp;  // in-edge CSR in plan order, sources as plan ids
    const int32_t* in_ci;
    float* xi;             // ranks in plan order
    float* contrib[2];     // x[u] * inv_out[u], double-buffered across iterations
    const pr::WorkItem* items;
    int32_t n_items;
    const pr::ChunkRow* chunk_rows;
    int32_t n_chunk_rows;
    float* hub_part;       // chunk sums
    float* part;           // [3][part_stride]: L1, dangling mass and sum of x' per
                           // k_init workgroup, or per item batch and then per
                           // k_hubfix workgroup (a tiled iteration's go to
                           // RunState::tsum)
    int64_t part_stride;
    int32_t n_batches;
    pr::RunState* state;
    int32_t grid;          // workgroups of the iteration kernel
    int32_t fix_grid;      // workgroups of the chunked-row kernel (0: none)
    int32_t init_grid;
    int32_t bucket_min[pr::kNumBuckets];
    int32_t row_begin[pr::kNumBuckets + 1];  // plan ids, hub bucket first
    int64_t bucket_edges[pr::kNumBuckets];
    int32_t bucket_items[pr::kNumBuckets + 1];  // kinds 0..5
    // tiled pull
    pr::TileMap tile_map;
    const int32_t* tsrc;    // [n_slots] source of each tile edge slot (block layout)
    const uint16_t* tdst;   // [n_slots] its row offset in the tile (read for wide blocks)
    const int32_t* tblk;    // [n_slots / kEdgeBlock] narrow block: its first source; wide: -1
    const int32_t* tile_ptr;  // [n_tiles + 1] first slot of each tile (multiples of kEdgeBlock)
    int64_t n_slots;        // tile edge slots, padding included
    const pr::Tile* tiles;
    int32_t n_tiles;
    int32_t max_tile_rows;  // rows of the largest tile (k_tile clears that many accumulators)
    const pr::TileUnit* units;
    int32_t n_units;
    const pr::TileFix* fixes;
    int32_t n_fused;        // cut tiles [0, n_fused) are finished in k_tile, the rest by k_tilefix
    uint32_t* fix_done;     // [n_fused] units of each of those tiles done in this launch (0 between launches)
    const int32_t* fix_rows;  // k_tilefix: [n_fixes - n_fused + 1] rows of its cut tiles before each one
    const int32_t* fix_win;   // k_tilefix: per 256-row window of those rows, the cut tile of its first row
    int32_t n_fixes;
    int32_t n_fix_rows;       // rows of k_tilefix's cut tiles
    long long* partial;
    int32_t tile_grid;
    pr::PlanHost* host;    // events, pinned status and staging (pooled)
    int32_t kernel_timed;  // event pairs around launches the last run recorded
    bool events_recorded;
};
