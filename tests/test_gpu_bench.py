"""GPU: bench.py prints one JSON line of the agreed shape, for the 3pCF line (C1, small) and the
parity 4pCF line (C4), with the roofline object of each line's dominant kernel."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
        "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}


def run_bench(*args) -> dict:
    print("bench", args, flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


@pytest.mark.gpu
def test_bench_3pcf_line(gpu_available):
    out = run_bench("--config", "C1", "--steps", "2", "--warmup", "1", "--no-cpu-baseline")
    assert KEYS <= set(out)
    assert out["n_gpus"] == 1 and out["steps"] == 2 and out["value"] > 0
    assert out["config"]["workload"].startswith("C1") and out["config"]["triangles"] > 0
    rf = out["roofline"]
    assert rf["bound"] == "hbm" and rf["kernel"] == "k_triplet" and rf["peak"] == 8000.0
    assert 0 < rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert "frac_traffic" in rf
    assert "valu" in out  # (a stored VALU count, or None when no run matches this workload)
    # one merge-walk per forward edge
    assert out["config"]["merge_walks"] == out["config"]["edges"]
    assert out["modes"] is None  # resident workload: no mode comparison


@pytest.mark.gpu
def test_bench_tiled_line_reports_every_mode(gpu_available):
    # the tiled form of the line on a small workload: host-streamed windows, with the resident and
    # re-emitted-window modes timed beside it and counting the same triangles
    out = run_bench("--config", "C1", "--tile-bytes", "40000", "--csr-mode", "host", "--steps",
                    "1", "--warmup", "1", "--mode-steps", "1", "--no-cpu-baseline")
    cfg = out["config"]
    assert cfg["csr_mode"] == "host" and cfg["windows"] > 1 and cfg["tiles"] >= 1
    assert set(out["modes"]) == {"host", "resident", "rebuild"}
    assert out["modes"]["resident"]["vs_resident"] == pytest.approx(1.0)
    assert all(m["kernel_ms"] > 0 for m in out["modes"].values())


@pytest.mark.gpu
def test_bench_4pcf_line(gpu_available):
    out = run_bench("--config", "C4", "--steps", "1", "--warmup", "1", "--no-cpu-baseline")
    assert KEYS <= set(out)
    assert out["unit"] == "tetrahedra/s" and out["value"] > 0
    assert out["config"]["tetrahedra"] > 0
    rf = out["roofline"]
    assert rf["bound"] == "alu" and rf["kernel"] == "k_clique4" and rf["peak"] == pytest.approx(614.4)
    assert rf["kernel_ms"] > 0 and rf["kernel_tetrahedra_per_s"] > 0


def test_bench_refuses_several_gpus():
    # runs without a GPU: the count is checked before anything touches the device
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr
