// pr_run: the power iteration.
//
// One iteration ("100 Days of GPU", Day 40, "One iteration, three shapes of
// work"):  x'[v] = (1-d)/n + d * (sum over in-neighbours u of contrib[u] + D/n)
// with contrib[u] = x[u]/outdeg[u] and D the dangling mass of x.
//
// The page runs five launches per iteration (scale, SpMV, two reduction
// passes, combine).  Here one launch does all of it:
//   * every workgroup gathers contrib over the in-rows of its degree bucket
//     (lane, 4-lane, 16-lane, wavefront or workgroup per row);
//   * the same lanes apply the combine to their rows, write x'[v] and the
//     next iteration's contrib'[v] = x'[v] * inv_out[v], and accumulate
//     |x'[v] - x[v]|, the dangling part of x' and the sum of x';
//   * each workgroup writes those three partials once; the last workgroup to
//     arrive reduces them (in double), appends the L1 distance to the trace,
//     stores D' for the next launch and raises the stop flag when L1 < tol.
// D therefore never leaves the device (the page's "Keep the dangling mass on
// the device"), and the write budget of the reductions is one slot per
// workgroup plus one (the page's gridDim.x + 1 rule).
//
// contrib is double-buffered across iterations (rows read other rows'
// contrib); x is updated in place (only row v's owner touches x[v]).
#include "plan.hpp"

namespace pr {

namespace {

struct IterArgs {
    const int32_t* __restrict__ in_rp;
    const int32_t* __restrict__ in_ci;
    const int32_t* __restrict__ rows;
    const float* __restrict__ inv_out;
    const float* __restrict__ contrib_in;
    float* __restrict__ contrib_out;
    float* __restrict__ x;
    float* __restrict__ partials;
    RunState* state;
    float* __restrict__ l1_trace;
    float* __restrict__ sum_trace;
    double d;
    double tol;
    int64_t nnz;
    int32_t n;
    int32_t t;  // 1-based iteration number
    int32_t partial_stride;
    BucketLaunch launch[kNumBuckets];
};

struct Acc {
    float l1 = 0.f, dang = 0.f, sum = 0.f;
};

// Clamp a row's edge range to [0, nnz] so a malformed in_row_ptr cannot
// index outside in_col_idx.
__device__ __forceinline__ void row_range(const IterArgs& a, int32_t v, int32_t& s, int32_t& e) {
    int32_t lo = a.in_rp[v], hi = a.in_rp[v + 1];
    const int32_t m = (int32_t)a.nnz;
    lo = lo < 0 ? 0 : (lo > m ? m : lo);
    hi = hi < lo ? lo : (hi > m ? m : hi);
    s = lo;
    e = hi;
}

// Gather of one source's contribution.  The index is clamped to [0, n) so a
// malformed in_col_idx cannot read outside contrib.  col_idx is streamed once
// per iteration, so it is loaded non-temporally to keep L2 for contrib.
__device__ __forceinline__ float gather(const IterArgs& a, int32_t k) {
    uint32_t u = (uint32_t)__builtin_nontemporal_load(a.in_ci + k);
    const uint32_t last = (uint32_t)(a.n - 1);
    u = u < last ? u : last;
    return a.contrib_in[u];
}

// Sum of contrib over edges [s, e) taken by lane `gl` of a G-lane group:
// edges s+gl, s+gl+G, ...  Four independent accumulators keep four gathers
// in flight per lane.
template <int G>
__device__ __forceinline__ float strided_sum(const IterArgs& a, int32_t s, int32_t e, int gl) {
    float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
    int32_t k = s + gl;
    for (; k + 3 * G < e; k += 4 * G) {
        y0 += gather(a, k);
        y1 += gather(a, k + G);
        y2 += gather(a, k + 2 * G);
        y3 += gather(a, k + 3 * G);
    }
    for (; k < e; k += G) y0 += gather(a, k);
    return (y0 + y1) + (y2 + y3);
}

// Damping factor as an unevaluated float pair hi + lo (hi = d rounded to
// float): d*y = hi*y + lo*y keeps the product at the double d to ~1e-15, so
// the rank sum does not drift by (float(d) - d)/(1 - d) ~ 1.6e-7.
struct Damp {
    float hi, lo;
};

// x'[v] from the gathered sum, and the per-lane partials.
__device__ __forceinline__ void combine(const IterArgs& a, int32_t v, float y, float base,
                                        Damp dmp, Acc& acc) {
    const float xo = a.x[v];
    const float xn = fmaf(dmp.lo, y, fmaf(dmp.hi, y, base));
    a.x[v] = xn;
    const float io = a.inv_out[v];
    a.contrib_out[v] = xn * io;
    acc.l1 += fabsf(xn - xo);
    acc.dang += (io == 0.f) ? xn : 0.f;
    acc.sum += xn;
}

template <int G>
__device__ __forceinline__ void run_bucket(const IterArgs& a, const BucketLaunch& L, int lblk,
                                           float base, Damp dmp, Acc& acc) {
    constexpr int kGroups = kBlock / G;
    const int gid = threadIdx.x / G, gl = threadIdx.x % G;
    for (int64_t i = L.row_begin + (int64_t)lblk * kGroups + gid; i < L.row_end;
         i += (int64_t)L.blocks * kGroups) {
        const int32_t v = a.rows[i];
        int32_t s, e;
        row_range(a, v, s, e);
        float y = strided_sum<G>(a, s, e, gl);
        y = group_sum<G>(y);
        if (gl == 0) combine(a, v, y, base, dmp, acc);
    }
}

// Hub rows: the whole workgroup on one row.
__device__ __forceinline__ void run_hubs(const IterArgs& a, const BucketLaunch& L, int lblk,
                                         float base, Damp dmp, Acc& acc, float* red) {
    for (int64_t i = L.row_begin + lblk; i < L.row_end; i += L.blocks) {
        const int32_t v = a.rows[i];
        int32_t s, e;
        row_range(a, v, s, e);
        float y = strided_sum<kBlock>(a, s, e, threadIdx.x);
        y = block_sum(y, red);
        if (threadIdx.x == 0) combine(a, v, y, base, dmp, acc);
    }
}

// Write this workgroup's three partials, and if it is the last to arrive,
// reduce all of them.  Returns true in every lane of the last workgroup,
// with the totals in *tot.
__device__ __forceinline__ bool arrive_and_reduce(float* __restrict__ partials, int stride,
                                                  RunState* st, Acc acc, double tot[3]) {
    __shared__ float redf[kWaves];
    __shared__ double redd[kWaves];
    __shared__ int s_last;
    const float l1 = block_sum(acc.l1, redf);
    const float dg = block_sum(acc.dang, redf);
    const float sm = block_sum(acc.sum, redf);
    if (threadIdx.x == 0) {
        __hip_atomic_store(&partials[blockIdx.x], l1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&partials[stride + blockIdx.x], dg, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&partials[2 * stride + blockIdx.x], sm, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t prev =
            __hip_atomic_fetch_add(&st->arrive, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == gridDim.x - 1) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return false;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    double r0 = 0.0, r1 = 0.0, r2 = 0.0;
    for (int j = threadIdx.x; j < (int)gridDim.x; j += kBlock) {
        r0 += (double)__hip_atomic_load(&partials[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        r1 += (double)__hip_atomic_load(&partials[stride + j], __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
        r2 += (double)__hip_atomic_load(&partials[2 * stride + j], __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    }
    tot[0] = block_sum(r0, redd);
    tot[1] = block_sum(r1, redd);
    tot[2] = block_sum(r2, redd);
    return true;
}

__global__ __launch_bounds__(kBlock) void k_iterate(IterArgs a) {
    __shared__ float red[kWaves];
    RunState* st = a.state;
    if (st->stop) return;  // an earlier iteration met the tolerance
    const double D = st->dmass;
    const float base = (float)((1.0 - a.d) / (double)a.n + a.d * D / (double)a.n);
    Damp dmp;
    dmp.hi = (float)a.d;
    dmp.lo = (float)(a.d - (double)dmp.hi);

    Acc acc;
    const int blk = blockIdx.x;
    if (blk < a.launch[4].block_begin + a.launch[4].blocks)
        run_hubs(a, a.launch[4], blk - a.launch[4].block_begin, base, dmp, acc, red);
    else if (blk < a.launch[3].block_begin + a.launch[3].blocks)
        run_bucket<64>(a, a.launch[3], blk - a.launch[3].block_begin, base, dmp, acc);
    else if (blk < a.launch[2].block_begin + a.launch[2].blocks)
        run_bucket<16>(a, a.launch[2], blk - a.launch[2].block_begin, base, dmp, acc);
    else if (blk < a.launch[1].block_begin + a.launch[1].blocks)
        run_bucket<4>(a, a.launch[1], blk - a.launch[1].block_begin, base, dmp, acc);
    else
        run_bucket<1>(a, a.launch[0], blk - a.launch[0].block_begin, base, dmp, acc);

    double tot[3];
    if (!arrive_and_reduce(a.partials, a.partial_stride, st, acc, tot)) return;
    if (threadIdx.x == 0) {
        const int t = a.t;
        a.l1_trace[t - 1] = (float)tot[0];
        if (a.sum_trace) a.sum_trace[t - 1] = (float)tot[2];
        st->dmass = tot[1];
        if (a.tol > 0.0 && tot[0] < a.tol) {
            st->stop = 1;
            st->iters = t;
        }
        st->arrive = 0u;
    }
}

// Start vector (given, or 1/n), the first contrib, and its dangling mass.
__global__ __launch_bounds__(kBlock) void k_init(const float* __restrict__ inv_out,
                                                 float* __restrict__ x,
                                                 float* __restrict__ contrib, int32_t n,
                                                 int x0_given, float* __restrict__ partials,
                                                 int stride, RunState* st) {
    const float uniform = (float)(1.0 / (double)n);
    Acc acc;
    for (int64_t v = blockIdx.x * (int64_t)kBlock + threadIdx.x; v < n;
         v += (int64_t)gridDim.x * kBlock) {
        float xv = uniform;
        if (x0_given)
            xv = x[v];
        else
            x[v] = xv;
        const float io = inv_out[v];
        contrib[v] = xv * io;
        acc.dang += (io == 0.f) ? xv : 0.f;
        acc.sum += xv;
    }
    double tot[3];
    if (!arrive_and_reduce(partials, stride, st, acc, tot)) return;
    if (threadIdx.x == 0) {
        st->dmass = tot[1];
        st->stop = 0;
        st->iters = 0;
        st->arrive = 0u;
    }
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
    hipStream_t stream = as_stream(stream_v);

    k_init<<<dim3((unsigned)p->init_blocks), kBlock, 0, stream>>>(
        p->inv_out, x, p->contrib[0], p->n, (flags & PR_X0_GIVEN) ? 1 : 0, p->partials,
        kMaxPartials, p->state);
    PR_LAUNCHED("init");

    IterArgs a{};
    a.in_rp = p->in_rp;
    a.in_ci = p->in_ci;
    a.rows = p->rows;
    a.inv_out = p->inv_out;
    a.x = x;
    a.partials = p->partials;
    a.state = p->state;
    a.l1_trace = l1_trace;
    a.sum_trace = sum_trace;
    a.d = d;
    a.tol = tol;
    a.nnz = p->nnz;
    a.n = p->n;
    a.partial_stride = kMaxPartials;
    for (int b = 0; b < kNumBuckets; ++b) a.launch[b] = p->launch[b];

    const bool record = flags & PR_RECORD_EVENTS;
    p->events_recorded = false;
    if (record) PR_HIP_TRY(hipEventRecord(p->ev_begin, stream));

    auto launch = [&](int32_t t) -> int {
        a.t = t;
        a.contrib_in = p->contrib[(t - 1) & 1];
        a.contrib_out = p->contrib[t & 1];
        k_iterate<<<dim3((unsigned)p->iter_blocks), kBlock, 0, stream>>>(a);
        PR_LAUNCHED("iterate");
        return PR_OK;
    };

    if (tol <= 0.0) {
        for (int32_t t = 1; t <= max_iter; ++t) PR_TRY(launch(t));
        if (record) {
            PR_HIP_TRY(hipEventRecord(p->ev_end, stream));
            p->events_recorded = true;
        }
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
    if (record) {
        PR_HIP_TRY(hipEventRecord(p->ev_end, stream));
        p->events_recorded = true;
    }
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
