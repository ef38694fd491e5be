"""Seeded test graphs and GPU/oracle comparison helpers shared by the GPU
parity tests.  Graphs come from graphgen only; expected values come from the
oracle only."""
from __future__ import annotations

import functools

import numpy as np

import graphgen
import oracle

D = 0.85
L1_TOL = 1e-5        # L1(x_gpu - x_oracle)
SUM_TOL = 1e-5       # |sum(x_gpu) - 1|
TRACE_TOL = 2e-5     # per-iteration |L1_gpu - L1_oracle| (triangle inequality on the two vectors)
SPEARMAN_MIN = 0.999  # Day 40, "Validate before timing": rank correlation over the top 100
SUM_GATE_EPS = 4 * float(np.finfo(np.float32).eps)  # Day 40: |sum - 1| <= 4 FLT_EPSILON sqrt(n)


def small_cases():
    """Graphs the oracle finishes in well under a second.  They span several
    4096-element tiles with ragged tails, every bucket, 1..3 radix passes,
    parallel edges, self-loops and the pages' six correctness shapes."""
    return [
        graphgen.tiny(),
        graphgen.single(),
        graphgen.empty(5),
        graphgen.cycle(1000),
        graphgen.chain(8192),
        graphgen.star(10001, inward=True),
        graphgen.star(10001, inward=False),
        graphgen.complete(70),
        graphgen.nodangling(),
        graphgen.dangling(),
        graphgen.random_graph(256, 3000, 11, name="random256"),         # 1 radix pass
        graphgen.random_graph(257, 3001, 12, name="random257"),         # 2 passes
        graphgen.random_graph(4097, 40_961, 13, dedup=False, drop_self=False,
                              name="multigraph4097"),                   # loops + parallel edges
        graphgen.random_graph(70_001, 300_007, 14, name="random70001"),  # 3 passes
        graphgen.stencil27(13, 11, 9),
        graphgen.citation(),
        graphgen.rmat(14),
        graphgen.rmat(16, edge_factor=16),
    ]


@functools.lru_cache(maxsize=None)
def workload(name: str) -> graphgen.Graph:
    return graphgen.workload(name)


def gpu_graph(g):
    import pagerank_power_iteration_amd as prx
    return prx.DeviceGraph.from_csr(g.row_ptr, g.col_idx)


def to_np(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def tie_groups(x: np.ndarray, order: np.ndarray, rel: float = 1e-9) -> np.ndarray:
    """Label of the group of (near-)equal values each position of `order` is
    in: a value joins the current group when it is within `rel` (relative) of
    the group's FIRST value, so a run of values that drift apart step by step
    does not chain into one group."""
    vals = x[order]
    labels = np.zeros(vals.size, dtype=np.int64)
    if vals.size == 0:
        return labels
    head, label = vals[0], 0
    for i in range(1, vals.size):
        v = vals[i]
        if abs(v - head) > rel * max(abs(v), abs(head)):
            label += 1
            head = v
        labels[i] = label
    return labels


def _top_labels(x_ref: np.ndarray, k: int, tie_rel: float):
    """The oracle ranking's first k vertices and the tie-group label of every
    vertex (vertices outside the first k + 1 groups get labels past them)."""
    ref_order = oracle.ranking(x_ref)
    head = ref_order[: min(x_ref.size, 4 * k + 64)]
    labels = np.full(x_ref.size, np.iinfo(np.int64).max, dtype=np.int64)
    labels[head] = tie_groups(x_ref, head, tie_rel)
    return ref_order, labels


FP32_U = 2.0 ** -24  # unit roundoff of the GPU's ranks
LOCAL_ERR = 8 * FP32_U  # relative error one GPU pass adds to a rank (see fp32_rank_bound)


def fp32_rank_bound(g, x_ref: np.ndarray, d: float, iters: int) -> np.ndarray:
    """A priori bound on |x_gpu[v] - x_oracle[v]| after `iters` passes from 1/n.

    One GPU pass rounds each rank with a relative error below 8u (u = 2^-24):
    1/outdeg and x[u]/outdeg (2u), the row sum rounded once from its exact
    fixed-point value (u, plus truncation far below it), the damped update
    (2u), the constant term (u) and the dangling mass it carries (2u).  An
    error e made in one pass reaches the next as d P~ e, where P~ is the
    column-stochastic matrix of the page's update (dangling columns spread
    evenly), so after T passes |e_T| <= sum_k (d P~)^k (8u x_{T-k}).  Every
    iterate from 1/n stays below x*/(1-d) componentwise, giving
    |e_T| <= 8u/(1-d) sum_{k<T} (d P~)^k x*.  x* is taken as the oracle's
    x_T, and each product d P~ y is one oracle pass from y minus its
    constant (1-d)/n, so the bound uses the oracle's own arithmetic."""
    n = x_ref.size
    y = x_ref.astype(np.float64).copy()
    z = y.copy()
    for _ in range(iters - 1):
        y = oracle.pagerank(g.row_ptr, g.col_idx, d=d, max_iter=1, x0=y).x - (1.0 - d) / n
        z += y
        if y.sum() < 1e-14 * z.sum():
            break
    return LOCAL_ERR / (1.0 - d) * z


def assert_same_top(x_gpu: np.ndarray, x_ref: np.ndarray, k: int = 20,
                    tie_rel: float = 1e-9, bound: np.ndarray | None = None) -> int:
    """Top-k of the GPU vector equals the oracle's, position by position.
    Without `bound`, vertices whose oracle values agree to `tie_rel` (exact
    ties from symmetry by default) may appear in any order among themselves.
    With a per-vertex error bound of the GPU ranks (fp32_rank_bound), the
    GPU's vertex a at position i and the oracle's vertex b there may differ
    when their oracle values are within bound[a] + bound[b]: fp32 cannot
    order them.  Returns how many of the k positions hold a different vertex
    than the oracle's (each one excused)."""
    gpu_top = oracle.ranking(x_gpu)[:k]
    if bound is not None:
        ref_top = oracle.ranking(x_ref)[:k]
        gap = np.abs(x_ref[gpu_top] - x_ref[ref_top])
        ok = gap <= bound[gpu_top] + bound[ref_top]
        if not ok.all():
            i = int(np.argmax(~ok))
            raise AssertionError(
                f"top-{k} differs at position {i}: gpu {gpu_top.tolist()} vs oracle "
                f"{ref_top.tolist()}; oracle values there {x_ref[ref_top[i]]!r} / "
                f"{x_ref[gpu_top[i]]!r}, beyond the fp32 bound "
                f"{bound[gpu_top[i]] + bound[ref_top[i]]:.3e}")
        return int((gpu_top != ref_top).sum())
    ref_order, labels = _top_labels(x_ref, k, tie_rel)
    want = labels[ref_order[:k]]
    got = labels[gpu_top]
    if not np.array_equal(want, got):
        i = int(np.argmax(want != got))
        raise AssertionError(
            f"top-{k} differs at position {i}: gpu {gpu_top.tolist()} vs oracle "
            f"{ref_order[:k].tolist()}; oracle values there {x_ref[ref_order[i]]!r} / "
            f"{x_ref[gpu_top[i]]!r}")
    return int((gpu_top != ref_order[:k]).sum())


def spearman_top(x_gpu: np.ndarray, x_ref: np.ndarray, k: int = 100,
                 tie_rel: float = 1e-9, bound: np.ndarray | None = None):
    """Spearman rank correlation between the oracle's and the GPU's values
    over the oracle's top k vertices (Day 40, "Validate before timing").
    Oracle tie groups are compared as wholes: the GPU values of a group are
    replaced by their mean, since the order inside a group is not defined.
    A group is a run of oracle values within tie_rel of its first value, or,
    with a per-vertex error bound of the GPU ranks, within bound[first] +
    bound[v] of it (values fp32 cannot order).  None when either side is
    constant."""
    from scipy import stats
    ref_order = oracle.ranking(x_ref)
    top = ref_order[: min(k, x_ref.size)]
    a = x_ref[top]
    b = np.asarray(x_gpu, dtype=np.float64)[top].copy()
    if bound is None:
        lab = _top_labels(x_ref, k, tie_rel)[1][top]
    else:
        lab = np.zeros(top.size, dtype=np.int64)
        head = 0
        for i in range(1, top.size):
            if abs(a[i] - a[head]) > bound[top[i]] + bound[top[head]]:
                head = i
            lab[i] = lab[i - 1] + (1 if head == i else 0)
    for g in np.unique(lab):
        sel = lab == g
        if sel.sum() > 1:
            a[sel] = a[sel].mean()
            b[sel] = b[sel].mean()
    if np.ptp(a) == 0 or np.ptp(b) == 0:
        return None
    return float(stats.spearmanr(a, b).correlation)


def assert_parity(x_gpu, l1_gpu, sum_gpu, ref, top_k: int = 20, tie_rel: float = 1e-9,
                  bound: np.ndarray | None = None) -> dict:
    """The benchmark spec's bars (L1(x_gpu - x_oracle) <= 1e-5, |sum - 1| <= 1e-5,
    identical top-20), the trace bar (2e-5 per entry), and Day 40's own
    "Validate before timing" gates: Spearman rho >= 0.999 over the oracle's
    top 100 and |sum - 1| <= 4 FLT_EPSILON sqrt(n)."""
    x = np.asarray(x_gpu, dtype=np.float64)
    err = float(np.abs(x - ref.x).sum())
    s = float(x.sum())
    assert err <= L1_TOL, f"L1(x_gpu - x_oracle) = {err:.3e}"
    assert abs(s - 1.0) <= SUM_TOL, f"sum(x_gpu) - 1 = {s - 1:.3e}"
    assert abs(s - 1.0) <= SUM_GATE_EPS * np.sqrt(x.size), \
        f"sum(x_gpu) - 1 = {s - 1:.3e} exceeds 4 FLT_EPSILON sqrt(n)"
    l1 = np.asarray(l1_gpu, dtype=np.float64)
    assert l1.shape == ref.l1_trace.shape
    tr = float(np.abs(l1 - ref.l1_trace).max())
    assert tr <= TRACE_TOL, f"L1 trace differs by {tr:.3e}"
    if sum_gpu is not None:
        st = np.asarray(sum_gpu, dtype=np.float64)
        assert np.abs(st - 1.0).max() <= SUM_TOL, "device sum trace drifted from 1"
    excused = 0
    rho = None
    if x.size > 1:
        excused = assert_same_top(x, ref.x, min(top_k, x.size), tie_rel, bound)
        rho = spearman_top(x, ref.x, 100, tie_rel, bound)
        assert rho is None or rho >= SPEARMAN_MIN, f"Spearman rho over the top 100 = {rho:.6f}"
    return {"l1_err": err, "sum_err": s - 1.0, "trace_err": tr, "tie_excused": excused,
            "spearman_top100": rho}
