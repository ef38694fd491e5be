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
    """Label of the run of (near-)equal values each position of `order` is in."""
    vals = x[order]
    if vals.size == 0:
        return np.zeros(0, dtype=np.int64)
    a, b = vals[1:], vals[:-1]
    same = np.abs(a - b) <= rel * np.maximum(np.abs(a), np.abs(b))
    return np.concatenate([[0], np.cumsum(~same)]).astype(np.int64)


def assert_same_top(x_gpu: np.ndarray, x_ref: np.ndarray, k: int = 20,
                    tie_rel: float = 1e-9) -> None:
    """Top-k of the GPU vector equals the oracle's, position by position;
    vertices whose oracle values agree to `tie_rel` (exact ties from symmetry
    by default) may appear in any order among themselves."""
    ref_order = oracle.ranking(x_ref)
    gpu_top = oracle.ranking(x_gpu)[:k]
    # label every vertex by the oracle tie group it sits in
    labels = np.empty(x_ref.size, dtype=np.int64)
    labels[ref_order] = tie_groups(x_ref, ref_order, tie_rel)
    want = labels[ref_order[:k]]
    got = labels[gpu_top]
    if not np.array_equal(want, got):
        i = int(np.argmax(want != got))
        raise AssertionError(
            f"top-{k} differs at position {i}: gpu {gpu_top.tolist()} vs oracle "
            f"{ref_order[:k].tolist()}; oracle values there {x_ref[ref_order[i]]!r} / "
            f"{x_ref[gpu_top[i]]!r}")


def assert_parity(x_gpu, l1_gpu, sum_gpu, ref, top_k: int = 20, tie_rel: float = 1e-9) -> dict:
    x = np.asarray(x_gpu, dtype=np.float64)
    err = float(np.abs(x - ref.x).sum())
    s = float(x.sum())
    assert err <= L1_TOL, f"L1(x_gpu - x_oracle) = {err:.3e}"
    assert abs(s - 1.0) <= SUM_TOL, f"sum(x_gpu) - 1 = {s - 1:.3e}"
    l1 = np.asarray(l1_gpu, dtype=np.float64)
    assert l1.shape == ref.l1_trace.shape
    tr = float(np.abs(l1 - ref.l1_trace).max())
    assert tr <= TRACE_TOL, f"L1 trace differs by {tr:.3e}"
    if sum_gpu is not None:
        st = np.asarray(sum_gpu, dtype=np.float64)
        assert np.abs(st - 1.0).max() <= SUM_TOL, "device sum trace drifted from 1"
    if x.size > 1:
        assert_same_top(x, ref.x, min(top_k, x.size), tie_rel)
    return {"l1_err": err, "sum_err": s - 1.0, "trace_err": tr}
