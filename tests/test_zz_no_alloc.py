"""pr_transpose_noalloc, the transpose whose workspace is the library's own
device array (for callers that cannot allocate), through the C ABI: its
output equals pr_transpose's bit for bit on consecutive calls of decreasing
size (the array keeps the previous call's contents), at the largest graph
the array takes, and oversized graphs are rejected before any device work."""
import numpy as np
import pytest

import graphgen
import oracle
from tests import _cases

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def prx():
    import pagerank_power_iteration_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def _noalloc(prx, dg, flags=0):
    in_rp = torch.full((dg.n + 1,), -7, dtype=torch.int32, device="cuda")
    in_ci = torch.full((max(dg.nnz, 1),), -7, dtype=torch.int32, device="cuda")[: dg.nnz]
    prx.pr_transpose_noalloc(dg.n, dg.nnz, dg.row_ptr, dg.col_idx, in_rp, in_ci, flags)
    torch.cuda.synchronize()
    return in_rp, in_ci


def _max_nnz(prx, n):
    lo, hi = 0, 1 << 26
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if prx.pr_transpose_workspace_bytes(n, mid) <= prx.PR_NOALLOC_SCRATCH_BYTES:
            lo = mid
        else:
            hi = mid - 1
    return lo


def test_noalloc_matches_pr_transpose_on_consecutive_calls(prx):
    graphs = [graphgen.rmat(17), graphgen.citation(), graphgen.tiny()]
    assert graphs[0].m > graphs[1].m > graphs[2].m
    for g in graphs:
        print(f"[noalloc] {g.name} n={g.n} m={g.m}", flush=True)
        dg = _cases.gpu_graph(g)
        want_rp, want_ci = prx.transpose(dg)
        got_rp, got_ci = _noalloc(prx, dg, prx.PR_VALIDATE)
        assert torch.equal(got_rp, want_rp) and torch.equal(got_ci, want_ci)
        if g.m < 1_000_000:
            ref_rp, ref_ci = oracle.transpose(g.row_ptr, g.col_idx)
            np.testing.assert_array_equal(_cases.to_np(got_rp), ref_rp)
            np.testing.assert_array_equal(_cases.to_np(got_ci), ref_ci)


def test_noalloc_largest_graph_it_takes(prx):
    n = 1 << 20
    m = _max_nnz(prx, n)
    assert m > 4_000_000
    k = np.arange(2 * m, dtype=np.uint64)
    r = (graphgen.splitmix_u64(77, k) % np.uint64(n)).astype(np.int64)
    g = graphgen.from_edges(n, r[:m], r[m:], dedup=False, drop_self=False, name="noalloc_max")
    assert g.m == m
    print(f"[noalloc] largest n={n} m={m}", flush=True)
    dg = _cases.gpu_graph(g)
    got_rp, got_ci = _noalloc(prx, dg)
    want_rp, want_ci = prx.transpose(dg)
    assert torch.equal(got_rp, want_rp) and torch.equal(got_ci, want_ci)
    ref_rp, ref_ci = oracle.transpose(g.row_ptr, g.col_idx)
    np.testing.assert_array_equal(_cases.to_np(got_rp), ref_rp)
    np.testing.assert_array_equal(_cases.to_np(got_ci), ref_ci)
    # then a smaller one on the same array
    small = graphgen.random_graph(70_001, 300_007, 14, name="random70001")
    dsm = _cases.gpu_graph(small)
    got_rp, got_ci = _noalloc(prx, dsm)
    ref_rp, ref_ci = oracle.transpose(small.row_ptr, small.col_idx)
    np.testing.assert_array_equal(_cases.to_np(got_rp), ref_rp)
    np.testing.assert_array_equal(_cases.to_np(got_ci), ref_ci)


def test_noalloc_rejects_what_does_not_fit(prx):
    n = 1 << 20
    m = _max_nnz(prx, n) + 1
    rp = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    ci = torch.zeros(16, dtype=torch.int32, device="cuda")
    out_rp = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    with pytest.raises(prx.PrError) as e:
        prx.pr_transpose_noalloc(n, m, rp, ci, out_rp, ci)
    assert e.value.status == prx.PR_ERR_WORKSPACE
    assert "scratch array" in str(e.value)


def test_noalloc_reports_malformed_input(prx):
    rp = torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda")
    ci = torch.tensor([1, 7], dtype=torch.int32, device="cuda")
    with pytest.raises(prx.PrError) as e:
        prx.pr_transpose_noalloc(2, 2, rp, ci, torch.empty(3, dtype=torch.int32, device="cuda"),
                                 torch.empty(2, dtype=torch.int32, device="cuda"), prx.PR_VALIDATE)
    assert e.value.status == prx.PR_ERR_GRAPH
