// pr_run: the power iteration.
//
// One iteration ("100 Days of GPU", Day 40, "One iteration, three shapes of
// work"):  x'[v] = (1-d)/n + d * (sum over in-neighbours u of contrib[u] + D/n)
// with contrib[u] = x[u]/outdeg[u] and D the dangling mass of x.
//
// The page runs five launches per iteration (scale, SpMV, two reduction
// passes, combine).  Here there are two, plus one when the graph has very
// long in-rows:
//   * k_iterate, 1024-lane workgroups, one per CU.  A workgroup first copies
//     the contributions of the hottest sources (the first kHotSources plan
//     ids: the vertices with the most out-edges) into LDS, where about half of
//     all gathers on skewed graphs then land.  Its wavefronts then take
//     batches of work items from a queue: each gathers contrib over the
//     in-rows of an item's degree bucket (lane, 4-lane, 16-lane group or whole
//     wavefront per row), and the lanes that hold a row's sum apply the update
//     on the spot: x'[v], the next iteration's contrib'[v] = x'[v] *
//     inv_out[v], and the running sums of |x'[v] - x[v]|, of the dangling part
//     of x' and of x'.  Each batch writes its three sums once (the page's
//     "one partial per block" write budget), so their total does not depend
//     on which wavefront ran which batch;
//   * k_hubfix, only for rows longer than one chunk: adds each such row's
//     chunk sums, in order, and applies the update;
//   * k_finalize, one workgroup: reduces the per-workgroup sums (in double),
//     appends the L1 distance to the trace, stores D' for the next iteration
//     and raises the stop flag once L1 < tol.
// D never leaves the device (the page's "Keep the dangling mass on the
// device").  No kernel publishes data to another workgroup of the same
// launch, so none needs a device-wide fence; kernel boundaries order every
// store before the loads that depend on it.
//
// Every vector is kept in the plan's vertex order; pr_run maps the caller's
// x in (k_init) and out (k_finish).  contrib is double-buffered across
// iterations (rows read other rows' contrib); x is updated in place (only row
// v's owner touches x[v]).
#include <cstdlib>

#include "plan.hpp"

namespace pr {

namespace {

struct IterArgs {
    const int32_t* __restrict__ in_rp;
    const int32_t* __restrict__ in_ci;
    const float* __restrict__ inv_out;
    const float* __restrict__ contrib_in;
    float* __restrict__ contrib_out;
    float* __restrict__ xi;
    const WorkItem* __restrict__ items;
    float* __restrict__ hub_part;
    float* __restrict__ part;  // [3][stride]: per-batch sums
    int64_t stride;
    RunState* state;
    double d;
    int32_t n;
    int32_t hot_n;  // sources held in LDS: min(n, kHotSources)
    int32_t n_items;
};

struct Acc {
    float l1 = 0.f, dang = 0.f, sum = 0.f;
};

// Damping factor as an unevaluated float pair hi + lo (hi = d rounded to
// float): d*y = hi*y + lo*y keeps the product at the double d to ~1e-15, so
// the rank sum does not drift by (float(d) - d)/(1 - d) ~ 1.6e-7.
struct Damp {
    float hi, lo, base;
};

__device__ __forceinline__ Damp make_damp(double d, int32_t n, double dmass) {
    Damp k;
    k.hi = (float)d;
    k.lo = (float)(d - (double)k.hi);
    k.base = (float)((1.0 - d) / (double)n + d * dmass / (double)n);
    return k;
}

// x'[p] from the gathered sum y, and the lane's running sums.  contrib' is
// written for every row (0 for a dangling one, whose slot is never read) so
// the stores cover whole lines.
__device__ __forceinline__ float apply(float xo, float io, float y, const Damp& k, Acc& acc) {
    const float xn = fmaf(k.lo, y, fmaf(k.hi, y, k.base));
    acc.l1 += fabsf(xn - xo);
    acc.dang += (io == 0.f) ? xn : 0.f;
    acc.sum += xn;
    return xn;
}

__device__ __forceinline__ void update(float* __restrict__ xi, const float* __restrict__ inv_out,
                                       float* __restrict__ contrib_out, int32_t p, float y,
                                       const Damp& k, Acc& acc) {
    const float io = inv_out[p];
    const float xn = apply(xi[p], io, y, k, acc);
    xi[p] = xn;
    contrib_out[p] = xn * io;
}

// One source's contribution: from the LDS copy below hot_n, else from
// global memory.  The plan built every index (in_ci holds plan ids in
// [0, n)), so none is re-checked here.
__device__ __forceinline__ float contrib_of(const IterArgs& a, const float* hot, int32_t u) {
    return u < a.hot_n ? hot[u] : a.contrib_in[u];
}

// col_idx is streamed once per iteration: load it non-temporally, leaving
// the caches to contrib.
__device__ __forceinline__ int32_t col(const IterArgs& a, int32_t k) {
    return __builtin_nontemporal_load(a.in_ci + k);
}

// Rows [lo, hi) of one bucket, run by one wavefront with G lanes per row
// (group g of the wavefront takes rows lo+g, lo+g+64/G, ...), B rows per
// group at a time.  The first U*G edges of all B rows are loaded and gathered
// together, B*U independent gathers per lane, which is what keeps the memory
// system busy at this occupancy; only rows longer than U*G (none, with the
// default bucket bounds, except in bucket 3) take a second, per-row loop.
// Each row's edges are taken by its group's lanes at stride G and summed in a
// fixed order, so the result does not depend on scheduling.
template <int G, int U, int B>
__device__ __forceinline__ void run_rows(const IterArgs& a, const float* hot, int32_t lo,
                                         int32_t hi, const Damp& k, Acc& acc) {
    constexpr int kGroups = kWave / G;
    const int lane = lane_id();
    const int gid = lane / G, gl = lane % G;
    for (int32_t p0 = lo + gid; p0 < hi; p0 += B * kGroups) {
        int32_t s[B], e[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int32_t p = p0 + b * kGroups;
            s[b] = p < hi ? a.in_rp[p] : 0;
            e[b] = p < hi ? a.in_rp[p + 1] : 0;
        }
        int32_t u[B][U];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int j = 0; j < U; ++j) {
                const int32_t q = s[b] + gl + j * G;
                u[b][j] = q < e[b] ? col(a, q) : -1;
            }
        float y[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float c[U];
#pragma unroll
            for (int j = 0; j < U; ++j) c[j] = u[b][j] >= 0 ? contrib_of(a, hot, u[b][j]) : 0.f;
#pragma unroll
            for (int w = 1; w < U; w <<= 1)
#pragma unroll
                for (int j = 0; j + w < U; j += 2 * w) c[j] += c[j + w];
            y[b] = c[0];
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            for (int32_t q = s[b] + gl + U * G; q < e[b]; q += U * G) {  // long rows only
                float c[U];
#pragma unroll
                for (int j = 0; j < U; ++j) {
                    const int32_t r = q + j * G;
                    c[j] = r < e[b] ? contrib_of(a, hot, col(a, r)) : 0.f;
                }
#pragma unroll
                for (int w = 1; w < U; w <<= 1)
#pragma unroll
                    for (int j = 0; j + w < U; j += 2 * w) c[j] += c[j + w];
                y[b] += c[0];
            }
            y[b] = group_sum<G>(y[b]);
            const int32_t p = p0 + b * kGroups;
            if (gl == 0 && p < hi) update(a.xi, a.inv_out, a.contrib_out, p, y[b], k, acc);
        }
    }
}

// Sum of contrib over edges [s, e) by a whole wavefront (a hub row or a
// chunk of one): lane l takes s+l, s+l+64, ..., 16 gathers in flight per
// lane; the lanes are added by a fixed shuffle tree, so every lane gets the
// same, schedule-independent total in y.
__device__ __forceinline__ void run_rows_sum(const IterArgs& a, const float* hot, int32_t s,
                                             int32_t e, int lane, float& y) {
    constexpr int U = 16;
    float acc = 0.f;
    for (int32_t q = s + lane; q < e; q += U * kWave) {
        int32_t u[U];
#pragma unroll
        for (int j = 0; j < U; ++j) u[j] = q + j * kWave < e ? col(a, q + j * kWave) : -1;
        float c[U];
#pragma unroll
        for (int j = 0; j < U; ++j) c[j] = u[j] >= 0 ? contrib_of(a, hot, u[j]) : 0.f;
#pragma unroll
        for (int w = 1; w < U; w <<= 1)
#pragma unroll
            for (int j = 0; j + w < U; j += 2 * w) c[j] += c[j + w];
        acc += c[0];
    }
    y = wave_sum(acc);
}

template <class T, int W>
__device__ __forceinline__ T wide_block_sum(T v, T* scratch) {
    v = wave_sum(v);
    if (lane_id() == 0) scratch[threadIdx.x / kWave] = v;
    __syncthreads();
    T r = scratch[0];
#pragma unroll
    for (int w = 1; w < W; ++w) r += scratch[w];
    __syncthreads();
    return r;
}

// Sums of part[0, count), part[stride + ...) and part[2*stride + ...) in
// double: lane i adds entries i, i + kThreads, ... in that order (eight loads
// in flight), then the workgroup adds the lanes.  The same inputs give the
// same sums in every workgroup.  Contains barriers.
struct Sums3 {
    double l1, dang, sum;
};

constexpr int kPartUnroll = 8;

// One round of the three sums' loads: entries j0 + u * kThreads, u <
// kPartUnroll (0 past count).
struct PartRound {
    float v0[kPartUnroll], v1[kPartUnroll], v2[kPartUnroll];
};

// Every load is unconditional (an entry past count reads the last one, or
// entry 0, and is dropped): a load under a branch is waited for where the
// branch ends, which would make the round's loads one chain of latencies.
// (The part arrays hold at least `stride` entries.)
template <int kThreads, int R>
__device__ __forceinline__ void parts_load_r(const float* __restrict__ part, int64_t stride,
                                             int32_t count, int start, PartRound& p) {
    const int last = count > 0 ? count - 1 : 0;
#pragma unroll
    for (int u = 0; u < kPartUnroll; ++u) {
        if (u < R) {
            const int j = start + (int)threadIdx.x + u * kThreads;
            const int jc = j < last ? j : last;
            p.v0[u] = part[jc];
            p.v1[u] = part[stride + jc];
            p.v2[u] = part[2 * stride + jc];
        } else {
            p.v0[u] = p.v1[u] = p.v2[u] = 0.f;
        }
    }
}

// The first round of the sums holds kPartFirst entries per lane (2048 for
// 1024 lanes: every workload's units fit), the later ones kPartUnroll.
constexpr int kPartFirst = 2;

// Loads entries start + i + u * kThreads (u < R) of the three sums into lane
// i's round, unconditionally: an entry at or past count reads the last one
// (or entry 0) and add_round drops it.  No load sits under a branch (one
// would be waited for where the branch ends), and no value is used here, so
// a caller can issue other loads before the round's first use.  (The part
// arrays hold at least `stride` entries.)
template <int kThreads, int R>
__device__ __forceinline__ void parts_load(const float* __restrict__ part, int64_t stride,
                                           int32_t count, int start, PartRound& p) {
    const int last = count > 0 ? count - 1 : 0;
#pragma unroll
    for (int u = 0; u < kPartUnroll; ++u) {
        if (u < R) {
            const int j = start + (int)threadIdx.x + u * kThreads;
            const int jc = j < last ? j : last;
            p.v0[u] = part[jc];
            p.v1[u] = part[stride + jc];
            p.v2[u] = part[2 * stride + jc];
        } else {
            p.v0[u] = p.v1[u] = p.v2[u] = 0.f;
        }
    }
}

// Adds a round's entries below count to the lane's three sums, in order.
template <int kThreads>
__device__ __forceinline__ void add_round(const PartRound& p, int start, int32_t count, double& r0,
                                          double& r1, double& r2) {
#pragma unroll
    for (int u = 0; u < kPartUnroll; ++u) {
        const bool in = start + (int)threadIdx.x + u * kThreads < count;
        r0 += in ? (double)p.v0[u] : 0.0;
        r1 += in ? (double)p.v1[u] : 0.0;
        r2 += in ? (double)p.v2[u] : 0.0;
    }
}

// The sums, given the first round's loads (parts_load<kThreads, kPartFirst>
// at start 0), so that a caller can issue them before other loads and add
// them later.
template <int kThreads>
__device__ __forceinline__ Sums3 sum_parts_from(const PartRound& first, const float* __restrict__ part,
                                                int64_t stride, int32_t count, double* redd) {
    double r0 = 0.0, r1 = 0.0, r2 = 0.0;
    add_round<kThreads>(first, 0, count, r0, r1, r2);
    for (int start = kPartFirst * kThreads; start < count; start += kPartUnroll * kThreads) {
        PartRound p;
        parts_load<kThreads, kPartUnroll>(part, stride, count, start, p);
        add_round<kThreads>(p, start, count, r0, r1, r2);
    }
    // the three sums of the workgroup at once: one exchange through LDS
    // (`redd` holds 3 * kThreads / kWave doubles), every lane adding the
    // wavefronts' sums in the same order
    constexpr int W = kThreads / kWave;
    r0 = wave_sum(r0);
    r1 = wave_sum(r1);
    r2 = wave_sum(r2);
    if (lane_id() == 0) {
        redd[threadIdx.x / kWave] = r0;
        redd[W + threadIdx.x / kWave] = r1;
        redd[2 * W + threadIdx.x / kWave] = r2;
    }
    __syncthreads();
    Sums3 r{redd[0], redd[W], redd[2 * W]};
#pragma unroll
    for (int w = 1; w < W; ++w) {
        r.l1 += redd[w];
        r.dang += redd[W + w];
        r.sum += redd[2 * W + w];
    }
    __syncthreads();
    return r;
}

template <int kThreads>
__device__ __forceinline__ Sums3 sum_parts(const float* __restrict__ part, int64_t stride,
                                           int32_t count, double* redd) {
    PartRound first;
    parts_load<kThreads, kPartFirst>(part, stride, count, 0, first);
    return sum_parts_from<kThreads>(first, part, stride, count, redd);
}

// Fixed-point shift of the tiled pull: every row sum of every iteration is
// bounded by max(1, sum |x0|) (the update does not grow the L1 norm beyond
// it), so 2^shift times that stays below 2^61.
__device__ __forceinline__ int fx_shift(double sum_abs_x0) {
    int ex = 0;
    (void)frexp(sum_abs_x0 > 1.0 ? sum_abs_x0 : 1.0, &ex);
    const int shift = 61 - ex;
    return shift > kFxShiftMax ? kFxShiftMax : (shift < 0 ? 0 : shift);
}

// An iteration's three sums (L1 distance, dangling mass, sum of x') are
// totals in fixed point, times 2^shift with each workgroup's part rounded:
// integer adds, exact in any order, so the totals do not depend on which
// workgroup adds first.  The shift keeps them below 2^62 (every |x'| sum is
// at most max(1, sum |x0|)).  A workgroup adds its parts up in registers and
// then into its line of RunState::tsum once; a reader adds the lines.
__device__ __forceinline__ long long to_sum(float v, double scale) {
    return (long long)llrint((double)v * scale);
}
__device__ __forceinline__ void add_sums(long long (*ts)[16], const long long (&v)[3]) {
    long long* line = ts[blockIdx.x % kSumSlots];
#pragma unroll
    for (int j = 0; j < 3; ++j)
        if (v[j] != 0) atomicAdd(reinterpret_cast<unsigned long long*>(line + j), (unsigned long long)v[j]);
}
// An iteration's three totals, times 2^-shift (the same in every lane).
__device__ __forceinline__ Sums3 read_sums(const long long (*ts)[16], int shift) {
    long long v[3] = {0, 0, 0};
#pragma unroll
    for (int s = 0; s < kSumSlots; ++s)
#pragma unroll
        for (int j = 0; j < 3; ++j) v[j] += ts[s][j];
    const double un = ldexp(1.0, -shift);
    return Sums3{(double)v[0] * un, (double)v[1] * un, (double)v[2] * un};
}

// A wavefront's next batch: lane 0 increments queue heads, starting with
// queue *q, until one yields a batch that holds items; -1 when every queue is
// empty.  `ticket` is the value the last increment of queue *q returned.
__device__ __forceinline__ int32_t next_batch(RunState* st, int& q, int& tries, int32_t n_batches,
                                              uint32_t ticket) {
    int32_t b = q + kQueues * (int32_t)ticket;
    while (b >= n_batches && ++tries < kQueues) {
        q = (q + 1) % kQueues;
        b = q + kQueues * (int32_t)atomicAdd(&st->queue[q][0], 1u);
    }
    return b < n_batches ? b : -1;
}

// With more than one workgroup per CU, the register budget must leave room
// for all of their wavefronts.
#if PR_ITER_BLOCKS_PER_CU > 1
#define PR_ITER_OCCUPANCY __attribute__((amdgpu_waves_per_eu(4 * PR_ITER_BLOCKS_PER_CU)))
#else
#define PR_ITER_OCCUPANCY
#endif

__global__ __launch_bounds__(kIterBlock) PR_ITER_OCCUPANCY void k_iterate(IterArgs a) {
    __shared__ float hot[kHotSources];
    RunState* st = a.state;
    if (st->stop) return;  // an earlier iteration met the tolerance
    const Damp k = make_damp(a.d, a.n, st->dmass);
    for (int32_t i = threadIdx.x; i < a.hot_n; i += kIterBlock) hot[i] = a.contrib_in[i];
    __syncthreads();

    const int lane = lane_id();
    const int32_t n_batches = (a.n_items + kBatchItems - 1) / kBatchItems;
    int q = blockIdx.x % kQueues, tries = 0;  // lane 0's queue state
    int32_t batch = -1;
    if (lane == 0) batch = next_batch(st, q, tries, n_batches, atomicAdd(&st->queue[q][0], 1u));
    batch = __shfl(batch, 0, kWave);
    while (batch >= 0) {
        Acc acc;
        // ask for the next batch now; the answer is needed only after this one
        uint32_t ticket = 0;
        if (lane == 0 && tries < kQueues) ticket = atomicAdd(&st->queue[q][0], 1u);
        const int32_t i1 = (batch + 1) * kBatchItems < a.n_items ? (batch + 1) * kBatchItems
                                                                 : a.n_items;
        for (int32_t i = batch * kBatchItems; i < i1; ++i) {
            const WorkItem it = a.items[i];
            switch (it.kind) {
                case 0: run_rows<1, 4, 4>(a, hot, it.lo, it.hi, k, acc); break;
                case 1: run_rows<4, 4, 4>(a, hot, it.lo, it.hi, k, acc); break;
                case 2: run_rows<16, 4, 4>(a, hot, it.lo, it.hi, k, acc); break;
                case 3: run_rows<kWave, 8, 2>(a, hot, it.lo, it.hi, k, acc); break;
                case kHubBucket: {
                    float y = 0.f;
                    run_rows_sum(a, hot, it.lo, it.hi, lane, y);
                    if (lane == 0) update(a.xi, a.inv_out, a.contrib_out, it.aux, y, k, acc);
                    break;
                }
                default: {  // kKindChunk
                    float y = 0.f;
                    run_rows_sum(a, hot, it.lo, it.hi, lane, y);
                    if (lane == 0) a.hub_part[it.aux] = y;
                    break;
                }
            }
        }
        // the batch's sums, in a fixed order whichever wavefront ran it
        const float l1 = wave_sum(acc.l1), dg = wave_sum(acc.dang), sm = wave_sum(acc.sum);
        if (lane == 0) {
            a.part[batch] = l1;
            a.part[a.stride + batch] = dg;
            a.part[2 * a.stride + batch] = sm;
            batch = tries < kQueues ? next_batch(st, q, tries, n_batches, ticket) : -1;
        }
        batch = __shfl(batch, 0, kWave);
    }
}

struct FixArgs {
    const float* __restrict__ inv_out;
    float* __restrict__ contrib_out;
    float* __restrict__ xi;
    const ChunkRow* __restrict__ chunk_rows;
    const float* __restrict__ hub_part;
    float* __restrict__ part;  // this kernel's sums go to [part0, part0 + gridDim.x)
    int64_t stride;
    RunState* state;
    double d;
    int32_t n;
    int32_t n_chunk_rows;
    int32_t part0;
};

// Rows longer than one chunk: one wavefront per row adds the row's chunk
// sums (lanes take slots first+lane, first+lane+64, ...; a fixed shuffle tree
// adds the lanes) and applies the update.
__global__ __launch_bounds__(kFixBlock) void k_hubfix(FixArgs f) {
    __shared__ float red[kFixBlock / kWave];
    RunState* st = f.state;
    if (st->stop) return;
    const Damp k = make_damp(f.d, f.n, st->dmass);
    constexpr int kW = kFixBlock / kWave;
    const int lane = lane_id();
    Acc acc;
    for (int32_t r = blockIdx.x * kW + threadIdx.x / kWave; r < f.n_chunk_rows;
         r += gridDim.x * kW) {
        const ChunkRow cr = f.chunk_rows[r];
        float y = 0.f;
        for (int32_t j = lane; j < cr.count; j += kWave) y += f.hub_part[cr.first + j];
        y = wave_sum(y);
        if (lane == 0) update(f.xi, f.inv_out, f.contrib_out, cr.row, y, k, acc);
    }
    const float l1 = wide_block_sum<float, kW>(acc.l1, red);
    const float dg = wide_block_sum<float, kW>(acc.dang, red);
    const float sm = wide_block_sum<float, kW>(acc.sum, red);
    if (threadIdx.x == 0) {
        f.part[f.part0 + blockIdx.x] = l1;
        f.part[f.stride + f.part0 + blockIdx.x] = dg;
        f.part[2 * f.stride + f.part0 + blockIdx.x] = sm;
    }
}

constexpr int kFinalWaves = kFinalBlock / kWave;

// ------------------------------------------------------------ tiled pull

#ifndef PR_TILE_BLOCK
#define PR_TILE_BLOCK 1024
#endif
constexpr int kTileBlock = PR_TILE_BLOCK;
constexpr int kTileWaves = kTileBlock / kWave;
// Edge blocks per wavefront per round: two keep more contribution gathers in
// flight; one wastes fewer loads when units are a few blocks long (a block
// past a unit's end is loaded and dropped).  pr_run picks per plan.
constexpr int kTileQWide = 2;
constexpr int kTileQNarrow = 1;
constexpr int64_t kWideUnitSlots = 4096;  // mean slots per unit from which kTileQWide runs

struct TileArgs {
    const int32_t* __restrict__ tsrc;
    const uint16_t* __restrict__ tdst;
    const int32_t* __restrict__ tblk;
    const TileUnit* __restrict__ units;
    const float* __restrict__ inv_out;
    const float* __restrict__ contrib_in;
    float* __restrict__ contrib_out;
    float* __restrict__ xi;
    long long* __restrict__ partial;
    const TileFix* __restrict__ fixes;
    uint32_t* __restrict__ fix_done;
    const float* __restrict__ part_prev;  // [3][stride]: k_init's sums (read by iteration 1)
    int64_t stride;
    RunState* state;
    float* __restrict__ l1_trace;
    float* __restrict__ sum_trace;
    double d;
    double tol;
    int32_t n;
    int32_t n_units;
    int32_t max_rows;    // rows of the largest tile: the accumulators any unit touches
    int32_t parts_prev;  // sums in part_prev
    int32_t t;           // iteration number, from 1
};

// Fixed point of one contribution: |c| * 2^shift truncated toward zero, with
// c's sign, in two's complement.  |c| * scale is exact in fp32 (scale is a
// power of two and the product stays below 2^61), and so is its split into
// 32-bit halves: hi = trunc(a / 2^32) has at most 24 significant bits, so
// a - hi * 2^32 is exact too.  The result equals truncating the exact product
// in double precision, with single-precision instructions only.
template <bool kSigned>
__device__ __forceinline__ unsigned long long to_fixed(float c, float scale) {
    const float a = (kSigned ? fabsf(c) : c) * scale;
    const uint32_t hi = (uint32_t)(a * 0x1p-32f);
    const uint32_t lo = (uint32_t)fmaf(-(float)hi, 0x1p32f, a);
    const unsigned long long r = ((unsigned long long)hi << 32) | lo;
    return (kSigned && c < 0.f) ? 0ull - r : r;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Element `index` of an array that starts at a uniform address: the byte
// offset is 32-bit (the plan keeps units below kMaxUnitEdges slots and tiled
// plans below kTiledMaxVertices vertices), so the load takes the base in
// scalar registers and one 32-bit offset per lane.
template <class T>
__device__ __forceinline__ T load_at(const T* base, uint32_t index) {
    return *(const T*)((const char*)base + index * (uint32_t)sizeof(T));
}
template <class T>
__device__ __forceinline__ T load_nt_at(const T* base, uint32_t index) {
    return __builtin_nontemporal_load((const T*)((const char*)base + index * (uint32_t)sizeof(T)));
}

// One round of a wavefront: blocks b + j*kTileWaves (j < Q) of the
// unit, each one 16-byte load of four slots per lane (lane l holds edges l,
// l+64, l+128, l+192 of the block) and the block's word of tblk (a scalar
// load: the block index is the same in every lane).  Every load is
// unconditional, so the compiler issues all of a round's loads before
// waiting for any: a block at or past the unit's end reads its last block
// instead, and the caller adds zero for it.  The edge arrays are streamed
// once per iteration: non-temporal.
template <int Q>
struct EdgeRound {
    u32x4 w[Q];
    int32_t first[Q];  // narrow block: its first source; wide: -1
};

// The block a wavefront reads for its block number q (the same in every lane:
// readfirstlane lets the compiler keep it in a scalar register).
__device__ __forceinline__ uint32_t block_of(uint32_t q, uint32_t nblk, uint32_t last) {
    return __builtin_amdgcn_readfirstlane(q < nblk ? q : last);
}

// A read-only word at a wave-uniform address, through the scalar cache (the
// constant address space lets the compiler use a scalar load).
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) {
    return *(const __attribute__((address_space(4))) int32_t*)p;
}

// Blocks b, b + stride, ..., Q of them.
template <int Q>
__device__ __forceinline__ void load_round(const int32_t* ts, const int32_t* tb, uint32_t b,
                                           uint32_t stride, uint32_t nblk, uint32_t last,
                                           EdgeRound<Q>& r) {
    const uint32_t lane = lane_id();
#pragma unroll
    for (int j = 0; j < Q; ++j) {
        const uint32_t bc = block_of(b + (uint32_t)j * stride, nblk, last);
        r.first[j] = load_uniform(tb + bc);
        r.w[j] = load_nt_at((const u32x4*)ts, bc * (kEdgeBlock / 4) + lane);
    }
}

// Adds the contributions of the unit's edge slots [e0, e1) (whole blocks)
// into acc[row offset].  A round of a wavefront is Q blocks: its first round
// is blocks w, w + kTileWaves, ... (wavefront w; `next` holds it, loaded by
// the caller), and each later one the next Q blocks of the unit's counter
// *s_blk (kTileWaves * Q at the start), claimed by lane 0 when the round
// before starts.  Each round loads the following one before gathering its
// own contributions.  Wavefronts of a workgroup progress at different rates
// (the oldest are served first), so with a fixed share each the first
// finished a unit of 10^5 edges at about half its time on R-MAT 23, and the
// unit's last blocks ran on a few wavefronts; the counter keeps them all
// busy to the end.  In one gather instruction lane l reads the source of edge
// l + 64*i of a block: consecutive lanes, neighbouring sources.  A narrow
// block decodes its slots; a wide one (rare) loads its rows here.
template <bool kSigned, int Q>
__device__ __forceinline__ void accumulate(const TileArgs& a, int32_t e0, int32_t e1, float scale,
                                           unsigned long long* acc, uint32_t* s_blk,
                                           EdgeRound<Q>& next) {
    const int32_t* ts = a.tsrc + e0;
    const uint16_t* td = a.tdst + e0;
    const int32_t* tb = a.tblk + e0 / kEdgeBlock;
    const uint32_t nblk = (uint32_t)(e1 - e0) / kEdgeBlock;
    const uint32_t last = nblk > 0 ? nblk - 1 : 0;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    uint32_t b = wave, stride = kTileWaves;  // this round: blocks b + j * stride
    while (b < nblk) {
        const EdgeRound<Q> cur = next;
        uint32_t nb = 0;
        if (lane_id() == 0) nb = atomicAdd(s_blk, (uint32_t)Q);
        nb = __builtin_amdgcn_readlane(nb, 0);
        load_round(ts, tb, nb, 1u, nblk, last, next);
        uint32_t src[Q][4], row[Q][4];
#pragma unroll
        for (int j = 0; j < Q; ++j) {
            if (cur.first[j] >= 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    src[j][i] = (uint32_t)cur.first[j] + (cur.w[j][i] & 0xFFFFu);
                    row[j][i] = cur.w[j][i] >> 16;
                }
            } else {
                const uint32_t bc = block_of(b + (uint32_t)j * stride, nblk, last);
                const u32x2 r2 = load_nt_at((const u32x2*)td, bc * (kEdgeBlock / 4) + lane_id());
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    src[j][i] = cur.w[j][i];
                    row[j][i] = (r2[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                }
            }
        }
        float v[Q][4];
#pragma unroll
        for (int j = 0; j < Q; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[j][i] = load_at(a.contrib_in, src[j][i]);
#pragma unroll
        for (int j = 0; j < Q; ++j) {
            const bool live = b + (uint32_t)j * stride < nblk;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const unsigned long long f = to_fixed<kSigned>(v[j][i], scale);
                atomicAdd(&acc[row[j][i]], live ? f : 0ull);
            }
        }
        b = nb;
        stride = 1;
    }
}

// The first round of a unit's edges.  An empty unit reads block 0 of the
// slot arrays instead (the plan's workspace always holds it; the values go
// unused), so every unit issues the same loads with no branch: a load under
// a branch is waited for where the branch ends, and a path with fewer loads
// in flight makes the waits after the join count too few.
template <int Q>
__device__ __forceinline__ void first_round(const TileArgs& a, const TileUnit& u, EdgeRound<Q>& r) {
    const uint32_t nblk = (uint32_t)(u.e1 - u.e0) / kEdgeBlock;
    const int32_t e0 = nblk > 0 ? u.e0 : 0;
    const uint32_t nb = nblk > 0 ? nblk : 1u;
    load_round(a.tsrc + e0, a.tblk + e0 / kEdgeBlock,
               __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), (uint32_t)kTileWaves, nb, nb - 1, r);
}

// The update of a whole-tile unit's rows: kRowU rows per lane per step, all
// of a step's loads issued before any is used (a lane past the last row
// loads the last row and drops the result).  Each row's accumulator is
// cleared after it is read.
constexpr int kRowU = 4;

__device__ __forceinline__ void update_rows(const TileArgs& a, unsigned long long* acc, int32_t row0,
                                            int32_t rows, double unit, const Damp& k, Acc& sums) {
    for (int32_t r = threadIdx.x; r < rows; r += kRowU * kTileBlock) {
        float xo[kRowU], io[kRowU], y[kRowU];
#pragma unroll
        for (int j = 0; j < kRowU; ++j) {
            const int32_t rj = r + j * kTileBlock;
            const int32_t rc = rj < rows ? rj : rows - 1;
            xo[j] = a.xi[row0 + rc];
            io[j] = a.inv_out[row0 + rc];
            y[j] = (float)((double)(long long)acc[rc] * unit);
        }
#pragma unroll
        for (int j = 0; j < kRowU; ++j) {
            const int32_t rj = r + j * kTileBlock;
            if (rj < rows) {
                acc[rj] = 0ull;
                const float xn = apply(xo[j], io[j], y[j], k, sums);
                a.xi[row0 + rj] = xn;
                a.contrib_out[row0 + rj] = xn * io[j];
            }
        }
    }
}

// A cut tile's units run on workgroups of any XCD, and an XCD's L2 does not
// see another's.  So a unit's slot goes out with device-scope stores, which
// write through to the level every XCD reads, and the unit that finishes the
// tile reads the other slots with device-scope loads.
__device__ __forceinline__ void store_device(long long* p, long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ long long load_device(long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this lane's vector memory operations are done: s_waitcnt with
// vmcnt 0 (bits 3:0 and 15:14) and the other counters at their maximum
// (expcnt 7 in bits 6:4, lgkmcnt 15 in bits 11:8).  A device-scope store is
// done once the level every XCD reads holds it.
__device__ __forceinline__ void wait_vector_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The unit that finishes cut tile fx (its own slot is own_slot, its
// accumulators still in acc) adds the other units' slots into acc: entries
// [first, first + count*rows) minus its own, kFixU per lane with their loads
// issued together, added with LDS atomics (a step may meet a row twice when
// the tile has fewer rows than the workgroup has lanes).  The integer sums
// are exact, so the order of the additions does not matter.
constexpr int kFixU = 8;

__device__ __forceinline__ void gather_slots(const TileArgs& a, unsigned long long* acc,
                                             const TileFix& fx, int32_t own_slot) {
    const uint32_t rows = (uint32_t)fx.rows;
    const uint32_t own = (uint32_t)(own_slot - fx.first);
    const uint32_t total = (uint32_t)(fx.count - 1) * rows;
    long long* base = a.partial + fx.first;
    for (uint32_t e0 = threadIdx.x; e0 < total; e0 += kFixU * kTileBlock) {
        long long v[kFixU];
        uint32_t r[kFixU];
#pragma unroll
        for (int i = 0; i < kFixU; ++i) {
            const uint32_t e = e0 + (uint32_t)(i * kTileBlock);
            const uint32_t ec = e < total ? e : total - 1;
            const uint32_t o = ec < own ? ec : ec + rows;  // skip the own slot
            r[i] = o % rows;
            v[i] = load_device(base + o);
        }
#pragma unroll
        for (int i = 0; i < kFixU; ++i)
            if (e0 + (uint32_t)(i * kTileBlock) < total) atomicAdd(&acc[r[i]], (unsigned long long)v[i]);
    }
}

// One workgroup per CU.  Workgroup b starts with unit b, then takes units
// gridDim.x, gridDim.x + 1, ... from queue 0, one when its current unit's
// edges are done, until they run out.  A whole-tile unit applies the update
// to its rows and writes its three sums; a unit of a cut tile writes its
// accumulators to its slot (and zero sums) and counts itself done on the
// tile; the tile's last unit adds the other slots to its accumulators,
// applies the update and writes the tile's sums to the tile's own entry
// (after the units'), so where they land does not depend on which unit was
// last.  A unit of a cut tile that the plan leaves to k_tilefix (fix -1;
// every cut tile when kFused is false) only writes its slot.
// The accumulators are all zero between units: each unit's epilogue clears
// the rows it read.  The next unit's descriptor and first round of edges are
// loaded before this unit's epilogue, so their latency overlaps it.
template <int Q, bool kFused>
__global__ __launch_bounds__(kTileBlock) void k_tile(TileArgs a) {
    __shared__ unsigned long long acc[kTileMaxRows + 1];  // + the trash row of padding edges
    __shared__ float red[3][kTileWaves];
    __shared__ int32_t s_next;
    __shared__ int32_t s_last;
    __shared__ int32_t s_late;  // a tile's finishing unit's claim, made after the finish
    __shared__ uint32_t s_blk;  // the current unit's next unclaimed edge block
    __shared__ double redd[3 * kTileWaves];
    RunState* st = a.state;
    // An earlier iteration met the tolerance: nothing to do.  The flag is
    // tested after the reduction below, so that its load and the reduction's
    // loads are in flight together (a stopped launch reduces stale sums and
    // drops them).
    const bool stopped = st->stop != 0;
    // Loads in this order: the previous iteration's sums, then the first
    // unit's descriptor and first round of edges (which do not depend on
    // them), so that the sums wait for their own loads only and the unit's
    // are in flight meanwhile.  After iteration 1 the sums are three exact
    // fixed-point totals (RunState::tsum); after k_init (any start vector,
    // whose sums need not fit that scale) every workgroup reduces k_init's
    // per-workgroup sums in the same order.
    // (Every workgroup has a first unit: the launch is at most n_units wide.)
    const bool after_init = a.t == 1;
    PartRound pr0;
    Sums3 ps{0.0, 0.0, 0.0};
    int pshift = 0;
    if (after_init) {
        parts_load<kTileBlock, kPartFirst>(a.part_prev, a.stride, a.parts_prev, 0, pr0);
    } else {
        pshift = st->fx_shift;
        ps = read_sums(st->tsum[(a.t - 1) % 3], pshift);
    }
    int32_t cur = blockIdx.x;
    TileUnit u = a.units[cur];
    EdgeRound<Q> round;
    first_round(a, u, round);
    // The previous iteration's L1 distance (the stop test), its dangling mass
    // D and its sum of x' -- after k_init: sum |x0|, D and the count of
    // negative entries.
    const Sums3 prev =
        after_init ? sum_parts_from<kTileBlock>(pr0, a.part_prev, a.stride, a.parts_prev, redd) : ps;
    if (stopped) return;
    if (a.t > 1 && a.tol > 0.0 && prev.l1 < a.tol) {  // iteration t - 1 met the tolerance
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            a.l1_trace[a.t - 2] = (float)prev.l1;
            if (a.sum_trace) a.sum_trace[a.t - 2] = (float)prev.sum;
            st->stop = 1;
            st->iters = a.t - 1;
        }
        return;
    }
    int shift;
    bool signed_contrib;
    if (a.t == 1) {
        shift = fx_shift(prev.l1);
        signed_contrib = prev.sum > 0.5;
    } else {
        shift = pshift;
        signed_contrib = st->signed_contrib != 0;
    }
    if (blockIdx.x == 0 && threadIdx.x < kSumSlots * 3)  // the next iteration's sums
        st->tsum[(a.t + 1) % 3][threadIdx.x / 3][threadIdx.x % 3] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st->dmass = prev.dang;  // for k_tilefix
        st->queue[(a.t + 1) & 1][0] = 0u;  // the next iteration's queue
        if (a.t == 1) {
            st->fx_shift = shift;
            st->fx_unit = ldexp(1.0, -shift);
            st->signed_contrib = signed_contrib ? 1 : 0;
        } else {
            a.l1_trace[a.t - 2] = (float)prev.l1;
            if (a.sum_trace) a.sum_trace[a.t - 2] = (float)prev.sum;
        }
    }
    const Damp k = make_damp(a.d, a.n, prev.dang);
    const float scale = ldexpf(1.0f, shift);  // a power of two, exact in fp32
    const double unit = ldexp(1.0, -shift);
    const double sum_scale = ldexp(1.0, shift);
    long long wsum[3] = {0, 0, 0};  // this workgroup's sums (lane 0)
    uint32_t* queue = &st->queue[a.t & 1][0];
    for (int32_t r = threadIdx.x; r < a.max_rows; r += kTileBlock) acc[r] = 0ull;  // (not the trash row)
    if (threadIdx.x == 0) s_blk = (uint32_t)(kTileWaves * Q);
    __syncthreads();
    while (cur < a.n_units) {
        if (signed_contrib)
            accumulate<true, Q>(a, u.e0, u.e1, scale, acc, &s_blk, round);
        else
            accumulate<false, Q>(a, u.e0, u.e1, scale, acc, &s_blk, round);
        // A unit of a cut tile finished here sends its slot out (once every
        // wavefront's additions are in) before the claim, so that the stores
        // and the claim are in flight together.
        const bool cut = u.slot >= 0;
        const bool fused = kFused && cut && u.fix >= 0;
        if (fused) {
            __syncthreads();
            for (int32_t r = threadIdx.x; r < u.rows; r += kTileBlock)
                store_device(a.partial + (int64_t)u.slot + r, (long long)acc[r]);
        }
        // claim the next unit only now: a claim made earlier would hold a
        // unit back behind this one while other workgroups run out of work
        // (with no more units than workgroups there is none to claim).  A
        // unit that may complete its tile counts itself done first, and the
        // one that does claims only after finishing the tile (up to 20 us on
        // R-MAT 23, at the end of the launch), so no unit waits behind it.
        auto claim = [&]() -> int32_t {
            return (int32_t)gridDim.x >= a.n_units ? a.n_units
                                                   : (int32_t)(gridDim.x + atomicAdd(queue, 1u));
        };
        if (!fused && threadIdx.x == 0) s_next = claim();
        if (fused) {
            wait_vector_memory();  // this lane's slot stores are done ...
            __syncthreads();       // ... and every lane's, before the count
            if (threadIdx.x == 0) {
                const bool last = atomicAdd(&a.fix_done[u.fix], 1u) + 1u == (uint32_t)u.count;
                s_last = last ? 1 : 0;
                if (!last) s_next = claim();
            }
        }
        __syncthreads();
        // every wavefront is past its last claim: the next unit's counter
        // (the next write of s_blk's readers follows the barrier below)
        if (threadIdx.x == 0) s_blk = (uint32_t)(kTileWaves * Q);
        const bool finisher = fused && s_last;
        int32_t nxt = finisher ? a.n_units : s_next;
        TileUnit un{};
        if (nxt < a.n_units) {
            un = a.units[nxt];
            first_round(a, un, round);
        }
        Acc sums;
        if (!cut) {
            update_rows(a, acc, u.row0, u.rows, unit, k, sums);
        } else if (!fused) {  // k_tilefix finishes the tile
            for (int32_t r = threadIdx.x; r < u.rows; r += kTileBlock) {
                a.partial[(int64_t)u.slot + r] = (long long)acc[r];
                acc[r] = 0ull;
            }
        } else if (s_last) {  // every other unit's slot is out: finish the tile
            const TileFix fx = a.fixes[u.fix];
            gather_slots(a, acc, fx, u.slot);
            if (threadIdx.x == 0)  // no unit of this launch counts on it again
                __hip_atomic_store(&a.fix_done[u.fix], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            update_rows(a, acc, u.row0, u.rows, unit, k, sums);
            if (threadIdx.x == 0) s_late = claim();  // read after the barrier below
        } else {
            for (int32_t r = threadIdx.x; r < u.rows; r += kTileBlock) acc[r] = 0ull;
        }
        const float l1 = wave_sum(sums.l1), dg = wave_sum(sums.dang), sm = wave_sum(sums.sum);
        if (lane_id() == 0) {
            red[0][threadIdx.x / kWave] = l1;
            red[1][threadIdx.x / kWave] = dg;
            red[2][threadIdx.x / kWave] = sm;
        }
        __syncthreads();
        if (threadIdx.x == 0) {  // the next writes of red and s_next follow a barrier
            float t0 = 0.f, t1 = 0.f, t2 = 0.f;
#pragma unroll
            for (int w = 0; w < kTileWaves; ++w) {
                t0 += red[0][w];
                t1 += red[1][w];
                t2 += red[2][w];
            }
            wsum[0] += to_sum(t0, sum_scale);  // (a cut tile's other units: zeros)
            wsum[1] += to_sum(t1, sum_scale);
            wsum[2] += to_sum(t2, sum_scale);
        }
        if (finisher) {  // (s_late is written again only after a later finish's barriers)
            nxt = s_late;
            if (nxt < a.n_units) {
                un = a.units[nxt];
                first_round(a, un, round);
            }
        }
        cur = nxt;
        u = un;
    }
    if (threadIdx.x == 0) add_sums(st->tsum[a.t % 3], wsum);
}

struct TileFixArgs {
    const TileFix* __restrict__ fixes;
    const int32_t* __restrict__ fix_rows;
    const int32_t* __restrict__ fix_win;
    const long long* __restrict__ partial;
    const float* __restrict__ inv_out;
    float* __restrict__ contrib_out;
    float* __restrict__ xi;
    RunState* state;  // the sums go to state->tsum[t % 3]
    double d;
    int32_t n;
    int32_t n_fixes;
    int32_t n_rows;  // rows of all cut tiles
    int32_t t;
};

// Rows of the tiles cut into units, one lane per row (the cut tiles' rows
// numbered one after another; fix_rows[i] is the number of rows before cut
// tile i): the row adds its slots (exact integer sums, so in any order),
// kFixSlots loads at a time, and applies the update.  Lane g of workgroup b takes rows b*256 + g, then
// + gridDim.x*256.  The plan lists the cut tile of every 256-row window's
// first row (fix_win); each lane steps forward from it (a tile has at least
// 64 rows, so a window meets at most five tiles).
constexpr int kFixSlots = 8;

__global__ __launch_bounds__(kFixBlock) void k_tilefix(TileFixArgs f) {
    __shared__ float red[3][kFixBlock / kWave];
    RunState* st = f.state;
    if (st->stop) return;
    const Damp k = make_damp(f.d, f.n, st->dmass);
    const double unit = st->fx_unit;
    Acc sums;
    for (int32_t g0 = blockIdx.x * kFixBlock; g0 < f.n_rows; g0 += gridDim.x * kFixBlock) {
        const int32_t g = g0 + threadIdx.x;
        if (g < f.n_rows) {
            int32_t i = f.fix_win[g0 / kFixBlock];
            while (i + 1 < f.n_fixes && f.fix_rows[i + 1] <= g) ++i;
            const TileFix fx = f.fixes[i];
            const int32_t r = g - f.fix_rows[i];
            const int32_t p = fx.row0 + r;
            // the row's own loads first, then its slots kFixSlots at a time
            // (the last step's extra slots reload the last one and add 0),
            // each step's loads issued together
            const float xo = f.xi[p], io = f.inv_out[p];
            const long long* slot = f.partial + (int64_t)fx.first + r;
            long long y[kFixSlots] = {};
            for (int32_t j = 0; j < fx.count; j += kFixSlots) {
                long long v[kFixSlots];
#pragma unroll
                for (int u = 0; u < kFixSlots; ++u) {
                    const int32_t jj = j + u < fx.count ? j + u : fx.count - 1;
                    v[u] = slot[(int64_t)jj * fx.rows];
                }
#pragma unroll
                for (int u = 0; u < kFixSlots; ++u) y[u] += j + u < fx.count ? v[u] : 0ll;
            }
#pragma unroll
            for (int u = 1; u < kFixSlots; ++u) y[0] += y[u];
            const float xn = apply(xo, io, (float)((double)y[0] * unit), k, sums);
            f.xi[p] = xn;
            f.contrib_out[p] = xn * io;
        }
    }
    const float l1 = wave_sum(sums.l1), dg = wave_sum(sums.dang), sm = wave_sum(sums.sum);
    if (lane_id() == 0) {
        red[0][threadIdx.x / kWave] = l1;
        red[1][threadIdx.x / kWave] = dg;
        red[2][threadIdx.x / kWave] = sm;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float t0 = 0.f, t1 = 0.f, t2 = 0.f;
#pragma unroll
        for (int w = 0; w < kFixBlock / kWave; ++w) {
            t0 += red[0][w];
            t1 += red[1][w];
            t2 += red[2][w];
        }
        const double sc = ldexp(1.0, st->fx_shift);
        const long long v[3] = {to_sum(t0, sc), to_sum(t1, sc), to_sum(t2, sc)};
        add_sums(st->tsum[f.t % 3], v);
    }
}

struct FinArgs {
    const float* __restrict__ part;
    int64_t stride;
    RunState* state;
    float* __restrict__ l1_trace;
    float* __restrict__ sum_trace;
    double tol;
    int32_t parts;  // sums to reduce: part[0, parts)
    int32_t t;      // iteration number; 0 after k_init
    int32_t tiled;  // t >= 1: the sums are RunState::tsum[t % 3], not part
};

// One workgroup of kFinalBlock lanes.  After iteration t: reduce every sum,
// record the trace and the next D, test the tolerance, and reset the work
// queues.  After k_init (t = 0): D, the fixed-point scale and the queues.
__global__ __launch_bounds__(kFinalBlock) void k_finalize(FinArgs f) {
    __shared__ double redd[3 * kFinalWaves];
    RunState* st = f.state;
    if (f.t > 0 && st->stop) return;
    Sums3 r;
    if (f.tiled && f.t > 0) {
        r = read_sums(st->tsum[f.t % 3], st->fx_shift);
    } else {
        r = sum_parts<kFinalBlock>(f.part, f.stride, f.parts, redd);
    }
    if (threadIdx.x < kQueues) st->queue[threadIdx.x][0] = 0u;
    if (threadIdx.x == 0) {
        st->dmass = r.dang;
        if (f.t == 0) {
            st->stop = 0;
            st->iters = 0;
            const int shift = fx_shift(r.l1);
            st->fx_shift = shift;
            st->fx_scale = ldexp(1.0, shift);
            st->fx_unit = ldexp(1.0, -shift);
            // x0 >= 0 keeps every later x and contribution >= 0 (the update
            // only adds non-negative terms), so the tiled pull can skip signs
            st->signed_contrib = r.sum > 0.5 ? 1 : 0;
        } else {
            f.l1_trace[f.t - 1] = (float)r.l1;
            if (f.sum_trace) f.sum_trace[f.t - 1] = (float)r.sum;
            if (f.tol > 0.0 && r.l1 < f.tol) {
                st->stop = 1;
                st->iters = f.t;
            }
        }
    }
}

// Start vector in plan order (the caller's x0, or 1/n), the first contrib,
// and per workgroup: sum of |x0|, dangling mass, and the number of negative
// entries (the third sum's slot; only the sign test of k_finalize reads it).
__global__ __launch_bounds__(kBlock) void k_init(const int32_t* __restrict__ new_id,
                                                 const float* __restrict__ inv_out,
                                                 const float* __restrict__ x,
                                                 float* __restrict__ xi,
                                                 float* __restrict__ contrib, int32_t n,
                                                 int x0_given, float* __restrict__ part,
                                                 int64_t stride, RunState* __restrict__ st) {
    __shared__ float red[kWaves];
    if (blockIdx.x == 0)  // no sums yet
        for (int i = threadIdx.x; i < 3 * kSumSlots * 3; i += kBlock)
            st->tsum[i / (kSumSlots * 3)][(i / 3) % kSumSlots][i % 3] = 0;
    if (blockIdx.x == 0 && threadIdx.x < kQueues) {  // a fresh run: no stop, empty queues
        st->queue[threadIdx.x][0] = 0u;
        if (threadIdx.x == 0) {
            st->stop = 0;
            st->iters = 0;
        }
    }
    const float uniform = (float)(1.0 / (double)n);
    Acc acc;
    for (int64_t v = blockIdx.x * (int64_t)kBlock + threadIdx.x; v < n;
         v += (int64_t)gridDim.x * kBlock) {
        const float xv = x0_given ? x[v] : uniform;
        const int32_t p = new_id[v];
        xi[p] = xv;
        const float io = inv_out[p];
        contrib[p] = xv * io;
        acc.l1 += fabsf(xv);
        acc.dang += (io == 0.f) ? xv : 0.f;
        acc.sum += xv < 0.f ? 1.f : 0.f;
    }
    const float l1 = block_sum(acc.l1, red);
    const float dg = block_sum(acc.dang, red);
    const float sm = block_sum(acc.sum, red);
    if (threadIdx.x == 0) {
        part[blockIdx.x] = l1;
        part[stride + blockIdx.x] = dg;
        part[2 * stride + blockIdx.x] = sm;
    }
}

// The ranks back in the caller's order.
__global__ __launch_bounds__(kBlock) void k_finish(const int32_t* __restrict__ new_id,
                                                   const float* __restrict__ xi,
                                                   float* __restrict__ x, int32_t n) {
    for (int64_t v = blockIdx.x * (int64_t)kBlock + threadIdx.x; v < n;
         v += (int64_t)gridDim.x * kBlock)
        x[v] = xi[new_id[v]];
}

int chunk_size(const pr_plan* p) {
    // Small graphs finish an iteration in microseconds: poll less often.
    if (p->nnz < (1 << 22)) return 16;
    if (p->nnz < (1 << 26)) return 8;
    return 4;
}

}  // namespace

}  // namespace pr

using namespace pr;

extern "C" int pr_run(pr_plan* p, double d, double tol, int32_t max_iter, float* x, float* l1_trace,
                      float* sum_trace, int32_t* iterations, uint32_t flags, void* stream_v) {
    if (!p) return fail(PR_ERR_ARG, "plan is null");
    if (!x || !l1_trace || !iterations) return fail(PR_ERR_ARG, "null pointer argument");
    if (!(d >= 0.0 && d <= 1.0)) return fail(PR_ERR_ARG, "d must be in [0, 1] (got %g)", d);
    if (max_iter < 1) return fail(PR_ERR_ARG, "max_iter must be >= 1 (got %d)", max_iter);
    if (flags & ~(PR_X0_GIVEN | PR_RECORD_EVENTS)) return fail(PR_ERR_ARG, "unknown flags 0x%x", flags);
    if (tol != tol) return fail(PR_ERR_ARG, "tol is NaN");
    int dev = -1;
    PR_HIP_TRY(hipGetDevice(&dev));
    if (dev != p->device)
        return fail(PR_ERR_ARG, "plan belongs to device %d but device %d is current", p->device, dev);
    // k_tile starts every workgroup on unit blockIdx.x without a check: a
    // tiled plan has a unit per tile at least, and launches at most one
    // workgroup per unit
    if (p->tiled && (p->n_units < 1 || p->tile_grid > p->n_units))
        return fail(PR_ERR_ARG, "tiled plan with %d units for %d workgroups", p->n_units, p->tile_grid);
    hipStream_t stream = as_stream(stream_v);

    // Per-workgroup sums: k_init writes its own to part set 0 (sum |x0|, D0,
    // negative entries), reduced by the first k_tile (tiled) or k_finalize
    // (bucketed).  A tiled iteration adds its sums into RunState::tsum, read
    // by the next k_tile: no k_finalize per iteration; a bucketed run uses
    // set 0 and k_finalize after every iteration.
    k_init<<<dim3((unsigned)p->init_grid), kBlock, 0, stream>>>(
        p->new_id, p->inv_out, x, p->xi, p->contrib[0], p->n, (flags & PR_X0_GIVEN) ? 1 : 0,
        p->part, p->part_stride, p->state);
    PR_LAUNCHED("init");

    FinArgs f{};
    f.part = p->part;
    f.stride = p->part_stride;
    f.state = p->state;
    f.l1_trace = l1_trace;
    f.sum_trace = sum_trace;
    f.tol = tol;
    f.parts = p->init_grid;
    f.t = 0;
    if (!p->tiled) {
        k_finalize<<<1, kFinalBlock, 0, stream>>>(f);
        PR_LAUNCHED("init finalize");
    }
    bool wide_rounds = p->n_units > 0 && p->n_slots >= kWideUnitSlots * (int64_t)p->n_units;
    if (const char* env = std::getenv("PR_TILE_Q")) {  // tuning knob: edge blocks per round
        if (std::atoi(env) == 1) wide_rounds = false;
        if (std::atoi(env) == 2) wide_rounds = true;
    }
    int32_t tilefix_grid = (int32_t)((p->n_fix_rows + kFixBlock - 1) / kFixBlock);
    if (tilefix_grid > kMaxGrid) tilefix_grid = kMaxGrid;
    // a bucketed run's sums: per batch, then per k_hubfix workgroup
    const int32_t iter_parts = p->n_batches + p->fix_grid;
    f.parts = iter_parts;

    IterArgs a{};
    a.in_rp = p->in_rp;
    a.in_ci = p->in_ci;
    a.inv_out = p->inv_out;
    a.xi = p->xi;
    a.items = p->items;
    a.n_items = p->n_items;
    a.hub_part = p->hub_part;
    a.part = p->part;
    a.stride = p->part_stride;
    a.state = p->state;
    a.d = d;
    a.n = p->n;
    a.hot_n = p->n < kHotSources ? p->n : kHotSources;

    FixArgs fx{};
    fx.inv_out = p->inv_out;
    fx.xi = p->xi;
    fx.chunk_rows = p->chunk_rows;
    fx.hub_part = p->hub_part;
    fx.part = p->part;
    fx.stride = p->part_stride;
    fx.state = p->state;
    fx.d = d;
    fx.n = p->n;
    fx.n_chunk_rows = p->n_chunk_rows;
    fx.part0 = p->n_batches;

    TileArgs ta{};
    ta.tsrc = p->tsrc;
    ta.tdst = p->tdst;
    ta.tblk = p->tblk;
    ta.units = p->units;
    ta.inv_out = p->inv_out;
    ta.xi = p->xi;
    ta.partial = p->partial;
    ta.fixes = p->fixes;
    ta.fix_done = p->fix_done;
    ta.stride = p->part_stride;
    ta.state = p->state;
    ta.l1_trace = l1_trace;
    ta.sum_trace = sum_trace;
    ta.d = d;
    ta.tol = tol;
    ta.n = p->n;
    ta.n_units = p->n_units;
    ta.max_rows = p->max_tile_rows;

    TileFixArgs tf{};
    tf.fixes = p->fixes + p->n_fused;  // the cut tiles k_tile leaves to it
    tf.fix_rows = p->fix_rows;
    tf.fix_win = p->fix_win;
    tf.n_rows = p->n_fix_rows;
    tf.partial = p->partial;
    tf.inv_out = p->inv_out;
    tf.xi = p->xi;
    tf.state = p->state;
    tf.d = d;
    tf.n = p->n;
    tf.n_fixes = p->n_fixes - p->n_fused;

    const bool record = flags & PR_RECORD_EVENTS;
    p->events_recorded = false;
    p->kernel_timed = 0;
    if (record) PR_HIP_TRY(hipEventRecord(p->host->ev_begin, stream));

    auto launch = [&](int32_t t) -> int {
        a.contrib_in = p->contrib[(t - 1) & 1];
        a.contrib_out = p->contrib[t & 1];
        const bool timed = record && t <= kTimedLaunches;
        if (timed) PR_HIP_TRY(hipEventRecord(p->host->kernel_ev[0][t - 1], stream));
        if (p->tiled) {
            ta.contrib_in = a.contrib_in;
            ta.contrib_out = a.contrib_out;
            ta.part_prev = p->part;  // iteration 1 reduces k_init's sums
            ta.parts_prev = p->init_grid;
            ta.t = t;
            const dim3 grid((unsigned)p->tile_grid);
            if (wide_rounds && p->n_fused > 0)
                k_tile<kTileQWide, true><<<grid, kTileBlock, 0, stream>>>(ta);
            else if (wide_rounds)
                k_tile<kTileQWide, false><<<grid, kTileBlock, 0, stream>>>(ta);
            else if (p->n_fused > 0)
                k_tile<kTileQNarrow, true><<<grid, kTileBlock, 0, stream>>>(ta);
            else
                k_tile<kTileQNarrow, false><<<grid, kTileBlock, 0, stream>>>(ta);
            PR_LAUNCHED("tile");
        } else {
            k_iterate<<<dim3((unsigned)p->grid), kIterBlock, 0, stream>>>(a);
            PR_LAUNCHED("iterate");
        }
        if (timed) {
            PR_HIP_TRY(hipEventRecord(p->host->kernel_ev[1][t - 1], stream));
            p->kernel_timed = t;
        }
        if (p->tiled && tilefix_grid > 0) {
            tf.contrib_out = a.contrib_out;
            tf.t = t;
            k_tilefix<<<dim3((unsigned)tilefix_grid), kFixBlock, 0, stream>>>(tf);
            PR_LAUNCHED("tile rows");
        }
        if (!p->tiled && p->fix_grid > 0) {
            fx.contrib_out = a.contrib_out;
            k_hubfix<<<dim3((unsigned)p->fix_grid), kFixBlock, 0, stream>>>(fx);
            PR_LAUNCHED("hub rows");
        }
        if (!p->tiled) {
            f.t = t;
            k_finalize<<<1, kFinalBlock, 0, stream>>>(f);
            PR_LAUNCHED("finalize");
        }
        return PR_OK;
    };
    // A tiled run reduces its last iteration's sums here (every earlier
    // iteration's were reduced by the next k_tile).
    auto close = [&](int32_t t_last) -> int {
        if (p->tiled) {
            f.t = t_last;
            f.tiled = 1;
            k_finalize<<<1, kFinalBlock, 0, stream>>>(f);
            PR_LAUNCHED("finalize");
        }
        return PR_OK;
    };
    auto finish = [&]() -> int {
        if (record) {
            PR_HIP_TRY(hipEventRecord(p->host->ev_end, stream));
            p->events_recorded = true;
        }
        k_finish<<<dim3((unsigned)p->init_grid), kBlock, 0, stream>>>(p->new_id, p->xi, x, p->n);
        PR_LAUNCHED("finish");
        return PR_OK;
    };

    if (tol <= 0.0) {
        for (int32_t t = 1; t <= max_iter; ++t) PR_TRY(launch(t));
        PR_TRY(close(max_iter));
        PR_TRY(finish());
        *iterations = max_iter;
        return PR_OK;
    }

    // Tolerance mode: chunks of iterations; after enqueuing chunk k, wait for
    // chunk k-1's status copy, so the device always has the next chunk queued.
    const int chunk = chunk_size(p);
    int slot = 0;
    bool have_prev = false, stopped = false;
    int32_t t = 1;
    while (t <= max_iter && !stopped) {
        const int32_t t_end = (max_iter - t + 1) < chunk ? max_iter : t + chunk - 1;
        for (int32_t tt = t; tt <= t_end; ++tt) PR_TRY(launch(tt));
        PR_HIP_TRY(hipMemcpyAsync(&p->host->status[slot], &p->state->stop, sizeof(RunStatus),
                                  hipMemcpyDeviceToHost, stream));
        PR_HIP_TRY(hipEventRecord(p->host->chunk_ev[slot], stream));
        if (have_prev) {
            PR_HIP_TRY(hipEventSynchronize(p->host->chunk_ev[slot ^ 1]));
            if (p->host->status[slot ^ 1].stop) stopped = true;
        }
        have_prev = true;
        slot ^= 1;
        t = t_end + 1;
    }
    PR_TRY(close(t - 1));
    PR_HIP_TRY(hipMemcpyAsync(&p->host->status[slot ^ 1], &p->state->stop, sizeof(RunStatus),
                              hipMemcpyDeviceToHost, stream));
    PR_TRY(finish());
    PR_HIP_TRY(hipStreamSynchronize(stream));
    const RunStatus& last = p->host->status[slot ^ 1];  // copied after every launched iteration
    *iterations = last.stop ? last.iters : max_iter;
    return PR_OK;
}

extern "C" int pr_plan_iteration_ms(pr_plan* p, float* ms) {
    if (!p || !ms) return fail(PR_ERR_ARG, "null pointer argument");
    if (!p->events_recorded) return fail(PR_ERR_ARG, "no pr_run with PR_RECORD_EVENTS on this plan");
    PR_HIP_TRY(hipEventSynchronize(p->host->ev_end));
    PR_HIP_TRY(hipEventElapsedTime(ms, p->host->ev_begin, p->host->ev_end));
    return PR_OK;
}

extern "C" int pr_plan_kernel_ms(pr_plan* p, float* ms, int32_t* launches) {
    if (!p || !ms) return fail(PR_ERR_ARG, "null pointer argument");
    if (!p->events_recorded || p->kernel_timed < 1)
        return fail(PR_ERR_ARG, "no pr_run with PR_RECORD_EVENTS on this plan");
    double total = 0.0;
    for (int i = 0; i < p->kernel_timed; ++i) {
        float one = 0.f;
        PR_HIP_TRY(hipEventSynchronize(p->host->kernel_ev[1][i]));
        PR_HIP_TRY(hipEventElapsedTime(&one, p->host->kernel_ev[0][i], p->host->kernel_ev[1][i]));
        total += one;
    }
    *ms = (float)(total / p->kernel_timed);
    if (launches) *launches = p->kernel_timed;
    return PR_OK;
}
