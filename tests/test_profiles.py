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


def test_triplet_kernels_declare_no_static_lds():
    # the sorted-histogram hit reads its rank tables at absolute LDS addresses 0 and 1024: every
    # k_triplet instantiation must keep its LDS in the dynamic block, which then starts at 0
    import re
    import subprocess
    from graph_triangle_counting_amd import _build
    if not os.path.exists(_build.HIPCC):
        pytest.skip("no hipcc")
    src = os.path.join(_build.CSRC, "triplet.hip")
    r = subprocess.run([_build.HIPCC, *_build.FLAGS, "--cuda-device-only", "-S", src, "-o", "-"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    kernels = re.findall(r"\.amdhsa_kernel (_ZN3gtc9k_triplet\w+)", r.stdout)
    sizes = re.findall(r"\.amdhsa_group_segment_fixed_size (\d+)", r.stdout)
    assert kernels and len(sizes) >= len(kernels)
    blocks = r.stdout.split(".amdhsa_kernel ")[1:]
    for b in blocks:
        name = b.split()[0]
        if "k_triplet" in name:
            m = re.search(r"\.amdhsa_group_segment_fixed_size (\d+)", b)
            assert m and int(m.group(1)) == 0, name
