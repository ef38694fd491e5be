// The iteration plan: inverse out-degrees, in-rows grouped by degree bucket,
// per-run scratch, and the launch shape of the fused iteration kernel.
#pragma once

#include "common.hpp"

namespace pr {

// Degree buckets of the pull product ("gpu-graph-study", PageRank T4:
// thread / warp / block per vertex by degree), re-cut for 64-lane
// wavefronts.  Bucket b holds the in-rows whose length is in
// [bucket_min[b], bucket_min[b+1]) and gives each row kBucketGroup[b] lanes:
// one lane, a 4- or 16-lane slice of a wavefront, a whole wavefront, or a
// whole 256-lane workgroup for the hubs.
constexpr int kNumBuckets = 5;
constexpr int kBucketGroup[kNumBuckets] = {1, 4, 16, 64, 256};
constexpr int32_t kDefaultBucketMin[kNumBuckets] = {0, 5, 17, 65, 4097};

// Upper bound on workgroups per bucket in one iteration launch (rows are
// visited grid-stride beyond it) and on partial-sum slots per launch.
constexpr int kMaxBlocksPerBucket = 2048;
constexpr int kMaxPartials = kNumBuckets * kMaxBlocksPerBucket;

struct BucketLaunch {
    int32_t row_begin;    // first entry of the bucket in plan->rows
    int32_t row_end;
    int32_t block_begin;  // first workgroup of the bucket in the launch
    int32_t blocks;
};

// Device-resident run state: the dangling mass for the next iteration, the
// stop flag, and the arrival counter of the last-workgroup reduction.
struct RunState {
    double dmass;       // D of the vector the next iteration starts from
    int32_t stop;       // 1 once an iteration met the tolerance
    int32_t iters;      // that iteration's number
    uint32_t arrive;    // workgroups finished in the current launch
    uint32_t pad[11];
};

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
    const int32_t* out_rp;
    const int32_t* in_rp;
    const int32_t* in_ci;
    float* inv_out;
    int32_t* rows;
    float* contrib[2];
    float* partials;  // [3][kMaxPartials]
    pr::RunState* state;
    int32_t bucket_min[pr::kNumBuckets];
    int64_t bucket_rows[pr::kNumBuckets];
    int64_t bucket_edges[pr::kNumBuckets];
    pr::BucketLaunch launch[pr::kNumBuckets];
    int32_t iter_blocks;
    int32_t init_blocks;
    hipEvent_t ev_begin, ev_end;
    hipEvent_t chunk_ev[2];
    pr::RunStatus* host_status;  // pinned, [2]
    bool events_recorded;
};
