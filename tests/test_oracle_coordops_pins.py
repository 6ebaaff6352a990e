"""Pins of the downsample / subdivide oracle.

* hand cases: the parent of a site, the max over two children, the 8
  children of a site;
* brute force: the parent set is the set of halved sites, each site's parent
  contains it, each parent row is the maximum of its children and equals one
  of them in every channel;
* subdivide followed by downsample gives back the input exactly (all 8
  children share the parent's features, so the maximum is that row);
* mutation checks: a planted mistake fails these pins.
"""
import numpy as np
import pytest

import workloads
from oracle import oracle as O


def test_hand_cases():
    coords = np.array([[0, 3, 5, 7], [0, 2, 4, 6], [1, 0, 0, 1]], dtype=np.int32)
    feats = np.array([[1.0, -2.0], [3.0, -5.0], [7.0, 7.0]], dtype=np.float16)
    pc, inv, pf, pg = O.downsample(coords, feats, (8, 8, 8))
    np.testing.assert_array_equal(pc, [[0, 1, 2, 3], [1, 0, 0, 0]])
    np.testing.assert_array_equal(inv, [0, 0, 1])
    np.testing.assert_array_equal(pf, np.array([[3.0, -2.0], [7.0, 7.0]], dtype=np.float16))
    assert pg == (4, 4, 4)
    cc, cf, cg = O.subdivide(coords[:1], feats[:1], (8, 8, 8))
    np.testing.assert_array_equal(cc[0], [0, 6, 10, 14])
    np.testing.assert_array_equal(cc[7], [0, 7, 11, 15])
    np.testing.assert_array_equal(cc[4], [0, 7, 10, 14])   # c = 4: dx = 1
    np.testing.assert_array_equal(cc[1], [0, 6, 10, 15])   # c = 1: dz = 1
    assert cg == (16, 16, 16) and np.all(cf == feats[0])


def test_odd_grid_parent_extent():
    pc, _, _, pg = O.downsample(np.array([[0, 4, 0, 2]], dtype=np.int32), None, (5, 3, 3))
    assert pg == (3, 2, 2)
    np.testing.assert_array_equal(pc, [[0, 2, 0, 1]])


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_brute_force_properties(seed):
    wl = workloads.random_small(seed, G=9, occ=0.2, cin=5, cout=1, batch=2)
    pc, inv, pf, _ = O.downsample(wl.coords, wl.feats, wl.grid)
    half = wl.coords.copy()
    half[:, 1:] //= 2
    assert {tuple(r) for r in half} == {tuple(r) for r in pc}
    assert len(pc) == len({tuple(r) for r in pc})
    assert all(tuple(pc[i]) <= tuple(pc[i + 1]) for i in range(len(pc) - 1))
    np.testing.assert_array_equal(pc[inv], half)
    for p in range(len(pc)):
        kids = wl.feats[inv == p].astype(np.float64)
        np.testing.assert_array_equal(pf[p].astype(np.float64), kids.max(0))


@pytest.mark.parametrize("seed", [4, 5])
def test_subdivide_then_downsample_is_identity(seed):
    wl = workloads.random_small(seed, G=7, occ=0.3, cin=3, cout=1, batch=2)
    order = np.lexsort(wl.coords.T[::-1])
    coords, feats = wl.coords[order], wl.feats[order]
    cc, cf, cg = O.subdivide(coords, feats, wl.grid)
    pc, inv, pf, pg = O.downsample(cc, cf, cg)
    np.testing.assert_array_equal(pc, coords)
    np.testing.assert_array_equal(pf, feats)
    np.testing.assert_array_equal(inv, np.repeat(np.arange(len(coords)), 8))
    assert pg == tuple(wl.grid)


def test_mutation_mean_instead_of_max_fails():
    coords = np.array([[0, 0, 0, 0], [0, 1, 1, 1]], dtype=np.int32)
    feats = np.array([[1.0], [3.0]], dtype=np.float16)
    _, _, pf, _ = O.downsample(coords, feats, (4, 4, 4))
    assert pf[0, 0] == 3.0 and pf[0, 0] != feats.astype(np.float64).mean()


def test_mutation_round_instead_of_floor_fails():
    # (3, 5, 7) // 2 = (1, 2, 3); rounding would give (2, 2, 4)
    pc, _, _, _ = O.downsample(np.array([[0, 3, 5, 7]], dtype=np.int32), None, (8, 8, 8))
    assert tuple(pc[0]) == (0, 1, 2, 3)


def test_range_errors_and_repeated_sites():
    with pytest.raises(O.OracleInputError):
        O.downsample(np.array([[0, 8, 0, 0]], dtype=np.int32), None, (8, 8, 8))
    with pytest.raises(O.OracleInputError):
        O.downsample(np.array([[2, 0, 0, 0]], dtype=np.int32), None, (8, 8, 8), batch=2)
    # a repeated site is one more child of its parent
    c = np.array([[0, 1, 1, 1], [0, 1, 1, 1]], dtype=np.int32)
    f = np.array([[1.0], [2.0]], dtype=np.float16)
    pc, inv, pf, _ = O.downsample(c, f, (4, 4, 4))
    np.testing.assert_array_equal(pc, [[0, 0, 0, 0]])
    np.testing.assert_array_equal(inv, [0, 0])
    assert pf[0, 0] == 2.0


@pytest.mark.parametrize("seed", [6, 7])
def test_vectorised_downsample_matches_loop(seed):
    wl = workloads.random_small(seed, G=10, occ=0.3, cin=8, cout=1, batch=3)
    a = O.downsample(wl.coords, wl.feats, wl.grid)
    b = O.downsample_np(wl.coords, wl.feats, wl.grid)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(x, y)
    assert a[3] == b[3]
