// The iteration plan: the graph renumbered and transposed, its rows split into
// degree buckets and cut into work items, plus the per-run scratch and the
// launch shape of the iteration kernels.
#pragma once

#include "common.hpp"

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

// Device-resident run state.  Written by the finalize and init kernels, read
// by the next launches (kernel boundaries order the accesses); the queue
// heads are incremented atomically by k_iterate.
struct RunState {
    double dmass;   // D of the vector the next iteration starts from
    int32_t stop;   // 1 once an iteration met the tolerance
    int32_t iters;  // that iteration's number
    uint32_t pad[60];
    uint32_t queue[kQueues][64];  // queue heads at [q][0]
};

// Launches of k_iterate that PR_RECORD_EVENTS times one by one.
constexpr int kTimedLaunches = 64;

// Host copy of the fields pr_run polls.
struct RunStatus {
    int32_t stop;
    int32_t iters;
};

}  // namespace pr

struct pr_plan {
    int device;
    int32_t n;
    int64_t nnz;
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
                           // item batch, then per k_hubfix workgroup
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
    hipEvent_t ev_begin, ev_end;
    hipEvent_t kernel_ev[2][pr::kTimedLaunches];  // around k_iterate launches
    int32_t kernel_timed;                         // pairs the last run recorded
    hipEvent_t chunk_ev[2];
    pr::RunStatus* host_status;  // pinned, [2]
    bool events_recorded;
};
