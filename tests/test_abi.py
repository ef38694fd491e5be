"""The C ABI on the host side, without a GPU: the library loads, exports every
function include/pr.h declares, and rejects bad arguments before touching the
device."""
import ctypes

import pytest

prx = pytest.importorskip("pagerank_power_iteration_amd")
from pagerank_power_iteration_amd import _lib  # noqa: E402


def test_library_exports_every_header_function():
    names = _lib.header_functions()
    assert len(names) >= 10
    so = prx.lib()
    missing = [n for n in names if not hasattr(so, n)]
    assert not missing, missing
    assert set(names) == set(_lib._SIGNATURES), "binding and header disagree"


def test_workspace_queries():
    assert prx.pr_transpose_workspace_bytes(0, 10) == 0
    assert prx.pr_transpose_workspace_bytes(10, -1) == 0
    assert prx.pr_transpose_workspace_bytes(10, 1 << 31) == 0
    small = prx.pr_transpose_workspace_bytes(1000, 10_000)
    big = prx.pr_transpose_workspace_bytes(1 << 23, 268_435_456)
    assert 0 < small < big
    # ping-pong key/value pairs for three 8-bit passes dominate: 16 bytes per edge
    assert big >= 16 * 268_435_456
    assert prx.pr_plan_workspace_bytes(1 << 23, 268_435_456) >= 4 * 268_435_456 + 24 * (1 << 23)
    assert prx.pr_plan_scratch_bytes(1 << 23, 268_435_456) >= 20 * 268_435_456
    assert prx.pr_plan_workspace_bytes(1, 0) > 0 and prx.pr_plan_scratch_bytes(1, 0) > 0


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert prx.pr_status_string(s)
    assert "unknown" in prx.pr_status_string(-99)


def test_arguments_rejected_before_device_work():
    so = prx.lib()
    assert so.pr_transpose(0, 0, None, None, None, None, None, 0, 0, None) == prx.PR_ERR_ARG
    assert "n must be" in prx.pr_last_error()
    assert so.pr_transpose(5, -3, 1, 1, 1, 1, 1, 0, 0, None) == prx.PR_ERR_ARG
    assert so.pr_transpose(5, 3, 1, 1, 1, 1, 1, 0, 0x80, None) == prx.PR_ERR_ARG
    assert so.pr_transpose(5, 3, None, 1, 1, 1, 1, 0, 0, None) == prx.PR_ERR_ARG
    # workspace too small / misaligned: rejected on the host
    assert so.pr_transpose(5, 3, 256, 256, 256, 256, 256, 8, 0, None) == prx.PR_ERR_WORKSPACE
    assert so.pr_transpose(5, 3, 256, 256, 256, 256, 260, 1 << 30, 0, None) == prx.PR_ERR_WORKSPACE
    h = ctypes.c_void_p()
    assert so.pr_plan_create(None, 5, 3, 1, 1, 1, 1 << 20, 1, 1 << 20, 0, None) == prx.PR_ERR_ARG
    assert so.pr_plan_create(ctypes.byref(h), 0, 3, 1, 1, 1, 1 << 20, 1, 1 << 20, 0, None) == \
        prx.PR_ERR_ARG
    assert so.pr_plan_create(ctypes.byref(h), 5, 3, 256, 256, 256, 1 << 20, 256, 1 << 20, 0x80,
                             None) == prx.PR_ERR_ARG
    assert so.pr_plan_create(ctypes.byref(h), 5, 3, 256, 256, 256, 4, 256, 1 << 20, 0, None) == \
        prx.PR_ERR_WORKSPACE
    assert so.pr_plan_create(ctypes.byref(h), 5, 3, 256, 256, 256, 1 << 20, 256, 4, 0, None) == \
        prx.PR_ERR_WORKSPACE
    assert so.pr_plan_layout(None, None, None, None) == prx.PR_ERR_ARG
    it = ctypes.c_int32()
    assert so.pr_run(None, 0.85, 0.0, 10, 1, 1, None, ctypes.byref(it), 0, None) == prx.PR_ERR_ARG
    assert so.pr_plan_destroy(None) == prx.PR_OK
    ms = ctypes.c_float()
    assert so.pr_plan_iteration_ms(None, ctypes.byref(ms)) == prx.PR_ERR_ARG
    assert so.pr_plan_buckets(None, None, None, None) == prx.PR_ERR_ARG
    assert so.pr_plan_num_buckets() == 5


def test_binding_raises_prerror():
    with pytest.raises(prx.PrError) as e:
        _lib._check(prx.lib().pr_transpose(0, 0, None, None, None, None, None, 0, 0, None))
    assert e.value.status == prx.PR_ERR_ARG


def test_traversal_workspace_queries_and_argument_checks():
    so = prx.lib()
    assert prx.pr_bfs_workspace_bytes(0, 10) == 0
    assert prx.pr_wcc_workspace_bytes(10, -1) == 0
    assert prx.pr_bfs_workspace_bytes(10, 1 << 31) == 0
    n, m = 1 << 23, 268_435_456
    # two int32 frontier queues for BFS; hub chunk descriptors for both
    assert prx.pr_bfs_workspace_bytes(n, m) >= 8 * n + prx.pr_wcc_workspace_bytes(n, m) - 256
    assert 0 < prx.pr_wcc_workspace_bytes(n, m) < 4 * m
    ws = prx.pr_bfs_workspace_bytes(100, 1000)
    # n < 1, bad source, unknown flags, null level, short / misaligned workspace:
    # all rejected on the host, before any device work
    assert so.pr_bfs(0, 0, 256, 256, None, None, 0, 256, None, None, 256, ws, 0, None) == prx.PR_ERR_ARG
    assert so.pr_bfs(100, 1000, 256, 256, None, None, 100, 256, None, None, 256, ws, 0, None) == prx.PR_ERR_ARG
    assert "source" in prx.pr_last_error()
    assert so.pr_bfs(100, 1000, 256, 256, None, None, -1, 256, None, None, 256, ws, 0, None) == prx.PR_ERR_ARG
    assert so.pr_bfs(100, 1000, 256, 256, None, None, 0, 256, None, None, 256, ws, 0x10, None) == prx.PR_ERR_ARG
    assert so.pr_bfs(100, 1000, 256, 256, None, None, 0, None, None, None, 256, ws, 0, None) == prx.PR_ERR_ARG
    assert so.pr_bfs(100, 1000, 256, 256, None, None, 0, 256, None, None, 256, ws - 1, 0, None) == \
        prx.PR_ERR_WORKSPACE
    assert so.pr_bfs(100, 1000, 256, 256, None, None, 0, 256, None, None, 260, ws, 0, None) == \
        prx.PR_ERR_WORKSPACE
    ws = prx.pr_wcc_workspace_bytes(100, 1000)
    assert so.pr_wcc(100, -1, 256, 256, None, None, 256, None, 256, ws, 0, None) == prx.PR_ERR_ARG
    assert so.pr_wcc(100, 1000, 256, None, None, None, 256, None, 256, ws, 0, None) == prx.PR_ERR_ARG
    assert so.pr_wcc(100, 1000, 256, 256, None, None, 256, None, 256, ws - 1, 0, None) == prx.PR_ERR_WORKSPACE
    assert so.pr_wcc(100, 1000, 256, 256, None, None, 256, None, 256, ws, 0x4, None) == prx.PR_ERR_ARG
    # an in-edge CSR needs both arrays
    assert so.pr_wcc(100, 1000, 256, 256, 256, None, 256, None, 256, ws, 0, None) == prx.PR_ERR_ARG
    assert so.pr_bfs(100, 1000, 256, 256, None, 256, 0, 256, None, None, 256,
                     prx.pr_bfs_workspace_bytes(100, 1000), 0, None) == prx.PR_ERR_ARG
