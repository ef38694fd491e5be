// pr_run: the power iteration.
//
// One iteration ("100 Days of GPU", Day 40, "One iteration, three shapes of
// work"):  x'[v] = (1-d)/n + d * (sum over in-neighbours u of contrib[u] + D/n)
// with contrib[u] = x[u]/outdeg[u] and D the dangling mass of x.
//
// The page runs five launches per iteration (scale, SpMV, two reduction
// passes, combine).  Here there are two:
//   * k_iterate, a persistent grid that takes work items from a queue: it
//     gathers contrib over the in-rows of each item's degree bucket (lane,
//     4-lane, 16-lane, wavefront or workgroup per row), and the lanes that
//     hold a row's sum apply the update on the spot: x'[v], the next
//     iteration's contrib'[v] = x'[v] * inv_out[v], and the three running
//     sums |x'[v] - x[v]|, the dangling part of x' and x'.  Each workgroup
//     writes its three sums once (the page's "gridDim.x + 1" write budget);
//   * k_finalize, one workgroup: it finishes the hub rows that were split in
//     chunks, reduces the per-workgroup sums (in double), appends the L1
//     distance to the trace, stores D' for the next iteration and raises the
//     stop flag once L1 < tol.
// D never leaves the device (the page's "Keep the dangling mass on the
// device").  No kernel publishes data to another workgroup of the same
// launch, so no launch needs a device-wide fence; the kernel boundary orders
// k_iterate's stores before k_finalize's loads.
//
// Every vector is kept in the plan's vertex order; pr_run maps the caller's
// x in (k_init) and out (k_finish).  contrib is double-buffered across
// iterations (rows read other rows' contrib); x is updated in place (only row
// v's owner touches x[v]).
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
    float* __restrict__ wg_part;
    RunState* state;
    double d;
    int32_t n;
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
__device__ __forceinline__ void update(float* __restrict__ xi, const float* __restrict__ inv_out,
                                       float* __restrict__ contrib_out, int32_t p, float y,
                                       const Damp& k, Acc& acc) {
    const float xo = xi[p];
    const float xn = fmaf(k.lo, y, fmaf(k.hi, y, k.base));
    xi[p] = xn;
    const float io = inv_out[p];
    contrib_out[p] = xn * io;
    acc.l1 += fabsf(xn - xo);
    acc.dang += (io == 0.f) ? xn : 0.f;
    acc.sum += xn;
}

// Sum of contrib over the edges [s, e) that lane `gl` of a G-lane group
// takes: s+gl, s+gl+G, ...  U independent loads per step keep U gathers in
// flight per lane.  col_idx is streamed once per iteration, so it is loaded
// non-temporally to leave the caches to contrib.  The plan built every index
// (in_ci holds plan ids in [0, n)), so none is re-checked here.
template <int G, int U>
__device__ __forceinline__ float gather_sum(const IterArgs& a, int32_t s, int32_t e, int gl) {
    float acc[U];
#pragma unroll
    for (int j = 0; j < U; ++j) acc[j] = 0.f;
    for (int32_t k = s + gl; k < e; k += U * G) {
        int32_t u[U];
#pragma unroll
        for (int j = 0; j < U; ++j)
            u[j] = (k + j * G < e) ? __builtin_nontemporal_load(a.in_ci + k + j * G) : -1;
#pragma unroll
        for (int j = 0; j < U; ++j) acc[j] += (u[j] >= 0) ? a.contrib_in[u[j]] : 0.f;
    }
#pragma unroll
    for (int w = 1; w < U; w <<= 1)
#pragma unroll
        for (int j = 0; j + w < U; j += 2 * w) acc[j] += acc[j + w];
    return acc[0];
}

// Rows [lo, hi) of a bucket with G lanes per row (G <= 64): group g of the
// workgroup takes rows lo+g, lo+g+256/G, ...
template <int G, int U>
__device__ __forceinline__ void run_rows(const IterArgs& a, int32_t lo, int32_t hi, const Damp& k,
                                         Acc& acc) {
    constexpr int kGroups = kBlock / G;
    const int gid = threadIdx.x / G, gl = threadIdx.x % G;
    for (int32_t p = lo + gid; p < hi; p += kGroups) {
        const int32_t s = a.in_rp[p], e = a.in_rp[p + 1];
        float y = gather_sum<G, U>(a, s, e, gl);
        y = group_sum<G>(y);
        if (gl == 0) update(a.xi, a.inv_out, a.contrib_out, p, y, k, acc);
    }
}

// Sum over the whole workgroup of edges [s, e) (a hub row or a chunk of one).
__device__ __forceinline__ float hub_sum(const IterArgs& a, int32_t s, int32_t e, float* red) {
    return block_sum(gather_sum<kBlock, 8>(a, s, e, threadIdx.x), red);
}

// The next item for this workgroup: thread 0 increments queue heads, starting
// with queue *q, until one yields an item below n_items; -1 when every queue
// is empty.
__device__ __forceinline__ int32_t next_item(RunState* st, int& q, int& tries, int32_t n_items,
                                             uint32_t ticket) {
    int32_t it = q + kQueues * (int32_t)ticket;
    while (it >= n_items && ++tries < kQueues) {
        q = (q + 1) % kQueues;
        it = q + kQueues * (int32_t)atomicAdd(&st->queue[q][0], 1u);
    }
    return it < n_items ? it : -1;
}

__global__ __launch_bounds__(kBlock) void k_iterate(IterArgs a) {
    __shared__ float red[kWaves];
    __shared__ int32_t s_item;
    RunState* st = a.state;
    if (st->stop) return;  // an earlier iteration met the tolerance
    const Damp k = make_damp(a.d, a.n, st->dmass);

    int q = blockIdx.x % kQueues, tries = 0;  // used by thread 0 only
    if (threadIdx.x == 0) s_item = next_item(st, q, tries, a.n_items, atomicAdd(&st->queue[q][0], 1u));
    __syncthreads();
    int32_t cur = s_item;
    Acc acc;
    while (cur >= 0) {
        // ask for the next item now; its answer is needed only after this one
        uint32_t ticket = 0;
        if (threadIdx.x == 0 && tries < kQueues) ticket = atomicAdd(&st->queue[q][0], 1u);
        const WorkItem it = a.items[cur];
        switch (it.kind) {
            case 0: run_rows<1, 4>(a, it.lo, it.hi, k, acc); break;
            case 1: run_rows<4, 4>(a, it.lo, it.hi, k, acc); break;
            case 2: run_rows<16, 4>(a, it.lo, it.hi, k, acc); break;
            case 3: run_rows<64, 4>(a, it.lo, it.hi, k, acc); break;
            case kHubBucket: {
                const float y = hub_sum(a, it.lo, it.hi, red);
                if (threadIdx.x == 0) update(a.xi, a.inv_out, a.contrib_out, it.aux, y, k, acc);
                break;
            }
            default: {  // kKindChunk
                const float y = hub_sum(a, it.lo, it.hi, red);
                if (threadIdx.x == 0) a.hub_part[it.aux] = y;
                break;
            }
        }
        __syncthreads();  // every lane has read s_item and finished with `red`
        if (threadIdx.x == 0)
            s_item = tries < kQueues ? next_item(st, q, tries, a.n_items, ticket) : -1;
        __syncthreads();
        cur = s_item;
    }
    const float l1 = block_sum(acc.l1, red);
    const float dg = block_sum(acc.dang, red);
    const float sm = block_sum(acc.sum, red);
    if (threadIdx.x == 0) {
        a.wg_part[blockIdx.x] = l1;
        a.wg_part[kMaxGrid + blockIdx.x] = dg;
        a.wg_part[2 * kMaxGrid + blockIdx.x] = sm;
    }
}

constexpr int kFinalWaves = kFinalBlock / kWave;

template <class T>
__device__ __forceinline__ T final_block_sum(T v, T* scratch) {
    v = wave_sum(v);
    if (lane_id() == 0) scratch[threadIdx.x / kWave] = v;
    __syncthreads();
    T r = scratch[0];
#pragma unroll
    for (int w = 1; w < kFinalWaves; ++w) r += scratch[w];
    __syncthreads();
    return r;
}

struct FinArgs {
    const float* __restrict__ inv_out;
    float* __restrict__ contrib_out;
    float* __restrict__ xi;
    const ChunkRow* __restrict__ chunk_rows;
    const float* __restrict__ hub_part;
    const float* __restrict__ wg_part;
    RunState* state;
    float* __restrict__ l1_trace;
    float* __restrict__ sum_trace;
    double d;
    double tol;
    int32_t n;
    int32_t n_chunk_rows;
    int32_t parts;  // per-workgroup sums to reduce
    int32_t t;      // iteration number; 0 after k_init
};

// One workgroup of kFinalBlock lanes.  After iteration t: finish the chunked
// hub rows, reduce every sum, record the trace and the next D, test the
// tolerance, and reset the work queues.  After k_init (t = 0): only D.
__global__ __launch_bounds__(kFinalBlock) void k_finalize(FinArgs f) {
    __shared__ double redd[kFinalWaves];
    RunState* st = f.state;
    if (f.t > 0 && st->stop) return;
    Acc acc;
    if (f.t > 0 && f.n_chunk_rows > 0) {
        const Damp k = make_damp(f.d, f.n, st->dmass);
        const int wave = threadIdx.x / kWave, lane = lane_id();
        for (int32_t r = wave; r < f.n_chunk_rows; r += kFinalWaves) {
            const ChunkRow cr = f.chunk_rows[r];
            float y = 0.f;
            for (int32_t j = lane; j < cr.count; j += kWave) y += f.hub_part[cr.first + j];
            y = wave_sum(y);
            if (lane == 0) update(f.xi, f.inv_out, f.contrib_out, cr.row, y, k, acc);
        }
    }
    double r0 = acc.l1, r1 = acc.dang, r2 = acc.sum;
    for (int j = threadIdx.x; j < f.parts; j += kFinalBlock) {
        r0 += (double)f.wg_part[j];
        r1 += (double)f.wg_part[kMaxGrid + j];
        r2 += (double)f.wg_part[2 * kMaxGrid + j];
    }
    r0 = final_block_sum(r0, redd);
    r1 = final_block_sum(r1, redd);
    r2 = final_block_sum(r2, redd);
    if (threadIdx.x < kQueues) st->queue[threadIdx.x][0] = 0u;
    if (threadIdx.x == 0) {
        st->dmass = r1;
        if (f.t == 0) {
            st->stop = 0;
            st->iters = 0;
        } else {
            f.l1_trace[f.t - 1] = (float)r0;
            if (f.sum_trace) f.sum_trace[f.t - 1] = (float)r2;
            if (f.tol > 0.0 && r0 < f.tol) {
                st->stop = 1;
                st->iters = f.t;
            }
        }
    }
}

// Start vector in plan order (the caller's x0, or 1/n), the first contrib,
// and per-workgroup dangling mass and sum.
__global__ __launch_bounds__(kBlock) void k_init(const int32_t* __restrict__ new_id,
                                                 const float* __restrict__ inv_out,
                                                 const float* __restrict__ x,
                                                 float* __restrict__ xi,
                                                 float* __restrict__ contrib, int32_t n,
                                                 int x0_given, float* __restrict__ wg_part) {
    __shared__ float red[kWaves];
    const float uniform = (float)(1.0 / (double)n);
    Acc acc;
    for (int64_t v = blockIdx.x * (int64_t)kBlock + threadIdx.x; v < n;
         v += (int64_t)gridDim.x * kBlock) {
        const float xv = x0_given ? x[v] : uniform;
        const int32_t p = new_id[v];
        xi[p] = xv;
        const float io = inv_out[p];
        contrib[p] = xv * io;
        acc.dang += (io == 0.f) ? xv : 0.f;
        acc.sum += xv;
    }
    const float dg = block_sum(acc.dang, red);
    const float sm = block_sum(acc.sum, red);
    if (threadIdx.x == 0) {
        wg_part[blockIdx.x] = 0.f;
        wg_part[kMaxGrid + blockIdx.x] = dg;
        wg_part[2 * kMaxGrid + blockIdx.x] = sm;
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

int iterate_blocks_per_cu() {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_iterate, kBlock, 0) != hipSuccess ||
        blocks < 1)
        blocks = 1;
    return blocks;
}

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
    hipStream_t stream = as_stream(stream_v);

    k_init<<<dim3((unsigned)p->init_grid), kBlock, 0, stream>>>(
        p->new_id, p->inv_out, x, p->xi, p->contrib[0], p->n, (flags & PR_X0_GIVEN) ? 1 : 0,
        p->wg_part);
    PR_LAUNCHED("init");

    FinArgs f{};
    f.inv_out = p->inv_out;
    f.xi = p->xi;
    f.chunk_rows = p->chunk_rows;
    f.hub_part = p->hub_part;
    f.wg_part = p->wg_part;
    f.state = p->state;
    f.l1_trace = l1_trace;
    f.sum_trace = sum_trace;
    f.d = d;
    f.tol = tol;
    f.n = p->n;
    f.n_chunk_rows = p->n_chunk_rows;
    f.parts = p->init_grid;
    f.t = 0;
    k_finalize<<<1, kFinalBlock, 0, stream>>>(f);
    PR_LAUNCHED("init finalize");
    f.parts = p->grid;

    IterArgs a{};
    a.in_rp = p->in_rp;
    a.in_ci = p->in_ci;
    a.inv_out = p->inv_out;
    a.xi = p->xi;
    a.items = p->items;
    a.hub_part = p->hub_part;
    a.wg_part = p->wg_part;
    a.state = p->state;
    a.d = d;
    a.n = p->n;
    a.n_items = p->n_items;

    const bool record = flags & PR_RECORD_EVENTS;
    p->events_recorded = false;
    if (record) PR_HIP_TRY(hipEventRecord(p->ev_begin, stream));

    auto launch = [&](int32_t t) -> int {
        a.contrib_in = p->contrib[(t - 1) & 1];
        a.contrib_out = p->contrib[t & 1];
        k_iterate<<<dim3((unsigned)p->grid), kBlock, 0, stream>>>(a);
        PR_LAUNCHED("iterate");
        f.contrib_out = a.contrib_out;
        f.t = t;
        k_finalize<<<1, kFinalBlock, 0, stream>>>(f);
        PR_LAUNCHED("finalize");
        return PR_OK;
    };
    auto finish = [&]() -> int {
        if (record) {
            PR_HIP_TRY(hipEventRecord(p->ev_end, stream));
            p->events_recorded = true;
        }
        k_finish<<<dim3((unsigned)p->init_grid), kBlock, 0, stream>>>(p->new_id, p->xi, x, p->n);
        PR_LAUNCHED("finish");
        return PR_OK;
    };

    if (tol <= 0.0) {
        for (int32_t t = 1; t <= max_iter; ++t) PR_TRY(launch(t));
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
        PR_HIP_TRY(hipMemcpyAsync(&p->host_status[slot], &p->state->stop, sizeof(RunStatus),
                                  hipMemcpyDeviceToHost, stream));
        PR_HIP_TRY(hipEventRecord(p->chunk_ev[slot], stream));
        if (have_prev) {
            PR_HIP_TRY(hipEventSynchronize(p->chunk_ev[slot ^ 1]));
            if (p->host_status[slot ^ 1].stop) stopped = true;
        }
        have_prev = true;
        slot ^= 1;
        t = t_end + 1;
    }
    PR_TRY(finish());
    PR_HIP_TRY(hipStreamSynchronize(stream));
    const RunStatus& last = p->host_status[slot ^ 1];  // copied after every launched iteration
    *iterations = last.stop ? last.iters : max_iter;
    return PR_OK;
}

extern "C" int pr_plan_iteration_ms(pr_plan* p, float* ms) {
    if (!p || !ms) return fail(PR_ERR_ARG, "null pointer argument");
    if (!p->events_recorded) return fail(PR_ERR_ARG, "no pr_run with PR_RECORD_EVENTS on this plan");
    PR_HIP_TRY(hipEventSynchronize(p->ev_end));
    PR_HIP_TRY(hipEventElapsedTime(ms, p->ev_begin, p->ev_end));
    return PR_OK;
}
