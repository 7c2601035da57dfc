"""Host logic of bench.py, without a GPU: the algorithmic byte counts
against the per-configuration totals of the workloads (real rows only,
metadata once per kernel), the buffer-set rule, the graph-size rule, the
traffic summary's source check, the one-GPU rule, and a short CPU-oracle
baseline leg."""

import importlib.util
import os
import subprocess
import sys

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test",
                                                  os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,total,dispatch,combine", [
    # whole-step bytes: layout + dispatch + combine, H = 7168, K = 8
    ("decode", 34.90e6, 16.52e6, 18.36e6),
    ("skewed", 1.117e9, 528.7e6, 587.6e6),
    ("fp8", 889.1e6, 301.2e6, 587.6e6),
    ("large", 4.466e9, 2.115e9, 2.350e9),
])
def test_algorithmic_bytes(bench, name, total, dispatch, combine):
    w = workloads.WORKLOADS[name]
    b = bench.algorithmic_bytes(w.bs, w.hidden, w.experts, w.topk, True, fp8=w.fp8)
    assert sum(b.values()) == pytest.approx(total, rel=5e-4)
    assert b["dispatch"] == pytest.approx(dispatch, rel=5e-4)
    assert b["combine"] == pytest.approx(combine, rel=5e-4)


def test_algorithmic_bytes_by_hand(bench):
    """One token, two experts, H = 128: every term written out."""
    b = bench.algorithmic_bytes(1, 128, 4, 2, shared=True)
    assert b["layout"] == 8 + 8 + 16 + 20
    assert b["dispatch"] == 256 + 2 * 256 + 16 + 20          # x once, 2 copies, ids + ranks
    assert b["combine"] == 2 * 256 + 256 + 256 + 24 + 20     # 2 rows, shared, out, metadata
    no_shared = bench.algorithmic_bytes(1, 128, 4, 2, shared=False)
    assert b["combine"] - no_shared["combine"] == 256
    e4m3 = bench.algorithmic_bytes(1, 128, 4, 2, fp8=True)
    assert e4m3["dispatch"] == 256 + 2 * (128 + 4) + 16 + 20  # codes + one fp32 scale per copy


@pytest.mark.parametrize("name", ["decode", "skewed", "fp8", "large"])
def test_buffer_sets_rule(bench, name):
    """Enough sets that the other sets' token rows between two uses of one
    set's rows are at least twice the Infinity Cache (unless the memory cap
    binds, as at decode size), and at most 64 sets within the memory cap."""
    w = workloads.WORKLOADS[name]
    import oracle
    cap = oracle.capacity(w.bs, w.topk, w.experts, w.align)
    step = sum(bench.algorithmic_bytes(w.bs, w.hidden, w.experts, w.topk, True,
                                       fp8=w.fp8).values())
    sets = bench.buffer_sets(w, cap, step, False)
    x_bytes = 2 * w.bs * w.hidden
    per_set = x_bytes * 3 + cap * w.hidden * (1 if w.fp8 else 2) + cap * w.hidden * 2
    assert 1 <= sets <= 64 and sets * per_set <= bench.SET_MEMORY_CAP
    if name != "decode":
        assert (sets - 1) * x_bytes >= 2 * bench.MALL_BYTES
        assert sets * step >= 2 << 30
    else:
        assert sets == bench.SET_MEMORY_CAP // per_set or sets == 64


def test_traffic_needs_the_current_kernel_source(bench, tmp_path, monkeypatch):
    """The committed counter summary is used only while the combine's
    sources hash to the value it records."""
    src = tmp_path / "k.hip"
    src.write_text("// kernel\n")
    summary = tmp_path / "traffic.txt"
    summary.write_text(f"source_hash: {bench.source_hash([str(src)])}\n"
                       "traffic_bytes_per_launch: 123456\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(summary))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    assert bench.read_traffic("skewed") == 123456.0
    assert bench.read_traffic("decode") is None          # recorded for the skewed line only
    src.write_text("// kernel, changed\n")
    assert bench.read_traffic("skewed") is None


@pytest.mark.parametrize("steps,per_graph", [(20, 20), (100, 20), (40, 20), (10, 10), (7, 7),
                                            (13, 13), (23, 1), (21, 7), (30, 15), (1, 1)])
def test_graph_size_divides_the_timed_steps(bench, steps, per_graph):
    """The timed region replays whole graphs of at most GRAPH_STEPS steps."""
    got = bench.steps_per_graph(steps)
    assert got == per_graph
    assert steps % got == 0 and got <= bench.GRAPH_STEPS


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("flags", [["--fused", "--separate"], ["--ep", "8", "--replicas", "4"],
                                   ["--ep", "8", "--fused"], ["--prepared"]])
def test_conflicting_options_are_refused(flags):
    """Refused before anything touches a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *flags],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, r.stderr


@pytest.mark.parametrize("threads", [1, 2])
def test_cpu_baseline_leg(bench, threads):
    w = workloads.WORKLOADS["tiny"]
    res = bench.cpu_baseline(w, 0.05, threads)
    assert res["kind"] == "oracle" and res["unit"] == "GB/s" and res["cores"] == threads
    assert res["value"] > 0 and res["tokens_per_s"] > 0
    assert "passes" in res["sample"]
