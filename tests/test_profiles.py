"""CPU: the committed counter runs that bench.py replays (HBM traffic and VALU instructions of
k_triplet, VALU instructions of k_clique4) are keyed to the kernels' machine code as built, so the
bench line reports them; and bench.py reads them back by workload, fingerprint and launch mode."""
from __future__ import annotations

import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "graph_triangle_counting_amd")


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def stored(path):
    rows = []
    with open(path) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            rows.append(line.split())
    return rows


@pytest.mark.parametrize("name,kernel", [("k_triplet_traffic.txt", "k_triplet"),
                                         ("k_triplet_valu.txt", "k_triplet"),
                                         ("k_clique4_valu.txt", "k_clique4")])
def test_stored_counter_runs_match_the_built_kernels(name, kernel):
    fp_file = os.path.join(PKG, f"{kernel}.fingerprint")
    if not os.path.exists(fp_file):
        pytest.skip("no build")
    fp = open(fp_file).read().strip()
    rows = stored(os.path.join(ROOT, "profiles", name))
    assert rows, name
    for row in rows:
        assert row[1] == fp, f"{name}: {row[0]} was measured on {row[1]}, the build is {fp}"
        assert float(row[-1]) > 0


def test_bench_reads_the_stored_runs_by_key_and_mode():
    bench = load_bench()
    if bench.kernel_fingerprint() is None:
        pytest.skip("no build")
    for key, fp, mode, value in stored(bench.TRAFFIC_FILE):
        assert bench.measured_traffic(key, int(mode)) == pytest.approx(float(value))
        assert bench.measured_traffic(key, int(mode) ^ 4) is None  # another kernel variant
    for key, fp, mode, value in stored(bench.TRIPLET_VALU_FILE):
        assert bench.measured_traffic(key, int(mode), bench.TRIPLET_VALU_FILE) == \
            pytest.approx(float(value))
    assert bench.measured_traffic("no-such-workload", 3) is None
