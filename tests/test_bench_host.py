"""Host logic of bench.py (CPU): the one-GPU contract, the per-kernel algorithmic work and
the rule that counter traffic is reported only for the sources it was measured on."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, env=dict(os.environ, WORLD_SIZE="1"))
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_kernel_work_adds_up_to_the_layer(name):
    w = WORKLOADS[name]
    counts = np.ones(w.E + w.S, dtype=np.int64)
    f1, b1 = bench.kernel_work(w, "linear1", counts)
    f2, b2 = bench.kernel_work(w, "linear2", counts)
    fr, _ = bench.kernel_work(w, "route", counts)
    experts, router = bench.flops_of(w)
    # linear1 (gate and up) is twice linear2; together they are the experts' work
    assert f1 == 2 * f2 and f1 + f2 == experts and fr == router
    # every touched group's weights are read at least once by the two GEMMs
    assert b1 + b2 >= (w.E + w.S) * bench.weight_bytes_per_group(w)
    # untouched groups cost no weight bytes
    none = np.zeros_like(counts)
    assert bench.kernel_work(w, "linear1", none)[1] < b1


def _fake_tree(tmp_path, files):
    csrc = tmp_path / "mixture_experts_layer_dispatch_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name, body in files.items():
        (csrc / name).write_bytes(body)
    (tmp_path / "profiles").mkdir()
    return csrc


def test_traffic_only_for_the_measured_sources(tmp_path, monkeypatch):
    csrc = _fake_tree(tmp_path, {"ffn.hip": b"launchers v1", "gemm_bf16_dev.hpp": b"tile v1",
                                 "common.hpp": b"helpers", "dispatch_dev.hpp": b"dispatch", "route.hip": b"r1"})
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    w = WORKLOADS["mixtral_bf16"]
    h = bench.sources_hash("linear1", "bf16")
    (tmp_path / "profiles" / "traffic.txt").write_text(
        "# header\n"
        f"workload={w.name} T={w.T} kernel=linear1 fetch_kib=100.0 write_kib=10.0 fetch_scale=2.0 "
        f"write_scale=1.0 dispatches=8 sources={h}\n")
    assert bench.traffic_of(w, "linear1") == (100.0 * 2.0 + 10.0) * 1024.0
    assert bench.traffic_of(w, "linear2") is None  # not measured
    (csrc / "route.hip").write_bytes(b"r2")  # a file the GEMM is not built from
    assert bench.traffic_of(w, "linear1") == (100.0 * 2.0 + 10.0) * 1024.0
    (csrc / "gemm_bf16_dev.hpp").write_bytes(b"tile v2")  # the GEMM changed since the counters
    assert bench.sources_hash("linear1", "bf16") != h
    assert bench.traffic_of(w, "linear1") is None


def test_traffic_of_a_sweep_entry_is_keyed_by_its_label(tmp_path, monkeypatch):
    """The capacity / EP / dense-GEMM entries run the layer's kernels on other shapes: their
    counters sit under the entry's label and never stand in for the layer's."""
    _fake_tree(tmp_path, {"ffn.hip": b"l", "ffn_fp8.hip": b"f", "gemm_fp8_dev.hpp": b"t", "common.hpp": b"c",
                          "dispatch_dev.hpp": b"d"})
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    w = WORKLOADS["dsv3_fp8fp4"].with_T(8192)
    h = bench.sources_hash("linear1", w.mode)
    (tmp_path / "profiles" / "traffic.txt").write_text(
        f"workload=dsv3_fp8fp4+ep T=8192 kernel=linear1 fetch_kib=50.0 write_kib=5.0 fetch_scale=2.0 "
        f"write_scale=1.0 dispatches=5 sources={h}\n")
    assert bench.traffic_of(w, "linear1", "dsv3_fp8fp4+ep") == (50.0 * 2.0 + 5.0) * 1024.0
    assert bench.traffic_of(w, "linear1") is None  # the layer itself was not measured
    assert bench.parse(["--entry", "ep"]).entry == "ep"


def test_load_statistics():
    w = WORKLOADS["dsv3_fp8fp4"].with_T(64)
    even = np.full(w.G, 2, dtype=np.int64)
    st = bench.load_stats(w, even)
    assert st["max_over_mean"] == 1.0 and st["gini"] == 0.0 and st["experts_touched"] == w.E
    one = np.zeros(w.G, dtype=np.int64)
    one[5] = 512
    st = bench.load_stats(w, one)
    # all load on one of E experts: max / mean = E, Gini = 1 - 1/E
    assert st["max_over_mean"] == w.E and abs(st["gini"] - (1 - 1 / w.E)) < 1e-12
