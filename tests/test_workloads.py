"""Input generators: deterministic, in range, right sizes, and the stated bin-edge rule."""
import math

import numpy as np

import workloads
from workloads import GRID, CONFIGS, linear_edges_sq


def test_configs_have_calibrated_radii():
    for k, c in CONFIGS.items():
        assert c.r > 0, k
        e = c.edges_sq()
        assert e[0] == 0 and e[-1] == c.r * c.r and np.all(np.diff(e) > 0) and e.size == c.nbins + 1


def test_edge_rule_is_exact_ceiling():
    r, nb = 115150, 10
    e = linear_edges_sq(r, nb)
    for b in range(nb + 1):
        # smallest integer d2 with sqrt(d2) >= b r / nb
        t = b * r
        want = (t * t + nb * nb - 1) // (nb * nb)
        assert e[b] == want
        assert math.isqrt(int(e[b])) * nb >= t or e[b] * nb * nb >= t * t
        assert (e[b] - 1) * nb * nb < t * t or b == 0


def test_generators_deterministic_and_in_range():
    for key in ("C1", "C2", "C4"):
        c = CONFIGS[key]
        a, wa = c.generate(20_000)
        b, wb = c.generate(20_000)
        np.testing.assert_array_equal(a, b)
        assert a.dtype == np.int32 and a.shape == (20_000, 3)
        assert a.min() >= 0 and a.max() < GRID
        if c.weighted:
            np.testing.assert_array_equal(wa, wb)
            assert wa.min() >= 0.5 and wa.max() < 1.5
        assert workloads.coords_sha256(a) == workloads.coords_sha256(b)


def test_mixed_generator_halves():
    c = CONFIGS["C5"]
    xyz, _ = c.generate(40_000)
    assert xyz.shape == (40_000, 3) and xyz.min() >= 0 and xyz.max() < GRID


def test_crop_keeps_density():
    c = CONFIGS["C1"]
    xyz, _ = c.generate()
    sub, _ = c.crop(xyz, None, 0.5)
    assert abs(sub.shape[0] / xyz.shape[0] - 0.125) < 0.02
