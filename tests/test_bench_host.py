"""Host logic of the benchmark script (no GPU): its byte models, the gate on
the committed counter summary, and the one-GPU rule."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_day40_byte_model_reproduces_the_pages_rate():
    # "100 Days of GPU", Day 40, "Results": the citation graph has 28,042
    # nodes and 314,010 edges, and the page's own kernels ran 50 iterations
    # in 1.7963 ms, which it reports as 95.7 GB/s effective.
    b = bench.day40_hand_bytes(28_042, 314_010)
    assert b == 3_437_470
    assert round(b * 50 / 1.7963e-3 / 1e9, 1) == 95.7


def test_min_bytes_is_the_sum_of_the_arrays_a_pull_iteration_touches():
    # each array at its own size, 4-byte elements: row_ptr (n + 1), the
    # column array (m), one gathered contribution per edge (m), x read (n),
    # x' written (n), inverse out-degrees (n), contributions written (n)
    for n, m in [(0, 0), (1, 0), (3, 3), (28_042, 311_579), (8_388_608, 258_667_197)]:
        arrays = {"row_ptr": n + 1, "col_idx": m, "gather": m, "x": n, "x_new": n,
                  "inv_out": n, "contrib_new": n}
        assert bench.min_bytes_per_iteration(n, m) == 4 * sum(arrays.values())
    # the headline graph's figure quoted beside the roofline
    assert bench.min_bytes_per_iteration(8_388_608, 258_667_197) == 2_237_109_740


def test_counter_traffic_is_used_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    path = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(path))
    assert bench.traffic_from_counters(0) == (None, None)  # no file
    path.write_text("{not json")
    assert bench.traffic_from_counters(0) == (None, None)
    path.write_text(json.dumps({"kernel_source_hash": "0" * 16, "hbm_bytes_per_launch": 123}))
    assert bench.traffic_from_counters(0) == (None, "0" * 16)  # other sources: not used
    h = bench.kernel_source_hash()
    path.write_text(json.dumps({"kernel_source_hash": h, "hbm_bytes_per_launch": 123}))
    assert bench.traffic_from_counters(0) == (123, h)


def test_kernel_source_hash_covers_the_kernel_and_its_layout():
    for rel in bench.KERNEL_SOURCES:
        assert os.path.isfile(os.path.join(ROOT, rel)), rel
    assert any(rel.endswith("run.hip") for rel in bench.KERNEL_SOURCES)
    assert any(rel.endswith("plan.hip") for rel in bench.KERNEL_SOURCES)
    assert len(bench.kernel_source_hash()) == 16


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused_with_a_message(argv, env):
    e = dict(os.environ)
    e.update(env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, timeout=120, env=e)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
