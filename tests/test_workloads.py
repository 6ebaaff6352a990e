"""The seeded input generators: sizes, determinism and validity of the recipes."""
import math

import numpy as np
import pytest

import workloads
from workloads import generators as g


@pytest.mark.parametrize("name,n,G", [("c1_16_8", 410, 16), ("c2_64_64", 26214, 64), ("c3_128_128", 209715, 128)])
def test_uniform_configs(name, n, G):
    a = workloads.make(name)
    b = workloads.make(name)
    assert a.n == n
    np.testing.assert_array_equal(a.coords, b.coords)
    np.testing.assert_array_equal(a.feats, b.feats)
    assert a.coords.dtype == np.int32 and a.feats.dtype == np.float16
    assert (a.coords[:, 1:] >= 0).all() and (a.coords[:, 1:] < G).all()
    lin = (a.coords[:, 1].astype(np.int64) * G + a.coords[:, 2]) * G + a.coords[:, 3]
    assert np.all(np.diff(lin) > 0)  # unique, raster order
    for L in a.layers:
        assert L.W.dtype == np.float16 and L.W.shape == (27 if L.ksize == 3 else 1, L.cin, L.cout)
        std = float(L.W.astype(np.float64).std())
        assert abs(std - 1 / math.sqrt(27 * L.cin)) < 0.1 / math.sqrt(27 * L.cin)


def test_real_sph_harm_matches_scipy():
    from scipy.special import sph_harm_y
    rng = np.random.default_rng(0)
    th = rng.uniform(0, math.pi, 200)
    ph = rng.uniform(0, 2 * math.pi, 200)
    for l in range(1, 4):
        for m in range(-l, l + 1):
            y = sph_harm_y(l, abs(m), th, ph)
            if m > 0:
                ref = math.sqrt(2) * (-1) ** m * y.real
            elif m < 0:
                ref = math.sqrt(2) * (-1) ** m * y.imag
            else:
                ref = y.real
            np.testing.assert_allclose(g.real_sph_harm(l, m, th, ph), ref, atol=1e-12)


def test_small_shell_is_two_voxels_thick():
    c = g.shell_coords(64, 20.0, 3.0, seed=7)
    assert len(np.unique(c, axis=0)) == len(c)
    occ = np.zeros((64, 64, 64), dtype=bool)
    occ[c[:, 1], c[:, 2], c[:, 3]] = True
    ctr = 31.5
    r = np.sqrt(((c[:, 1:] - ctr) ** 2).sum(axis=1))
    assert r.min() > 20 - 3 - 1 - 2 * math.sqrt(3) - 1e-9 and r.max() <= 20 + 3 + 1
    assert 4 * math.pi * 20 ** 2 * 1.2 < len(c) < 4 * math.pi * 20 ** 2 * 4


@pytest.mark.slow
def test_shell_configs_sizes():
    c4 = workloads.make("c4_256_shell")
    assert c4.batch == 2 and 300_000 < (c4.coords[:, 0] == 0).sum() < 420_000
    assert 300_000 < (c4.coords[:, 0] == 1).sum() < 420_000
