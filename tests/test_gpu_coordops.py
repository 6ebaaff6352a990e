"""GPU parity of x2 downsample (max) and subdivide through the C ABI against
the CPU oracle: integer coordinates, inverse indices and fp16 maxima are
compared bit for bit."""
import numpy as np
import pytest
import torch

import workloads
from oracle import oracle as O

gpu = pytest.mark.gpu


def _sc():
    import submanifold_sparse_convolution_hash_amd as sc
    sc.load_library()
    return sc


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _to(dev, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _check_down(sc, dev, coords, feats, grid, batch, ref_fn):
    pc, inv, pf, pg = sc.downsample(_to(dev, coords), None if feats is None else _to(dev, feats),
                                    grid, batch)
    rpc, rinv, rpf, rpg = ref_fn(coords, feats, grid)
    np.testing.assert_array_equal(pc.cpu().numpy(), rpc)
    np.testing.assert_array_equal(inv.cpu().numpy(), rinv)
    assert pg == rpg
    if feats is not None:
        np.testing.assert_array_equal(pf.cpu().numpy().view(np.uint16), rpf.view(np.uint16))


@gpu
@pytest.mark.parametrize("seed,G,occ,batch,c", [(1, 9, 0.2, 2, 16), (2, 17, 0.5, 1, 8), (3, 5, 1.0, 3, 64),
                                                 (4, 33, 0.05, 2, 32)])
def test_downsample_small(dev, seed, G, occ, batch, c):
    sc = _sc()
    wl = workloads.random_small(seed, G=G, occ=occ, cin=c, cout=1, batch=batch)
    print(f"[coordops] downsample small seed={seed} N={wl.n}", flush=True)
    _check_down(sc, dev, wl.coords, wl.feats, wl.grid, batch, O.downsample)


def _clustered_sites(rng, batch, grid, parents):
    """Distinct sites in the 2x2x2 blocks of `parents` random parent sites (1 to 8
    children each), plus the grid's two extreme corners."""
    pg = [(g + 1) // 2 for g in grid]
    pb = rng.integers(0, batch, parents)
    px = [rng.integers(0, pg[a], parents) for a in range(3)]
    rows = [[0, 0, 0, 0], [batch - 1, grid[0] - 1, grid[1] - 1, grid[2] - 1]]
    for i in range(parents):
        for c in rng.choice(8, size=int(rng.integers(1, 9)), replace=False):
            s = [int(pb[i])] + [2 * int(px[a][i]) + ((int(c) >> (2 - a)) & 1) for a in range(3)]
            if all(s[1 + a] < grid[a] for a in range(3)):
                rows.append(s)
    return np.unique(np.array(rows, dtype=np.int32), axis=0)


@gpu
@pytest.mark.parametrize("batch,grid", [(1, (4096, 4096, 2048)), (3, (4096, 4096, 4095)),
                                        (2, (2, 1 << 20, 1 << 20))])
def test_downsample_wide_keys(dev, batch, grid):
    # parent-key spans of exactly 2^32 (largest key 2^32 - 1, 32-bit sort keys)
    # and beyond 2^32 (64-bit sort keys), odd extents included
    sc = _sc()
    rng = np.random.default_rng(sum(grid) + batch)
    coords = _clustered_sites(rng, batch, grid, 3000)
    coords = coords[rng.permutation(len(coords))]
    feats = rng.standard_normal((len(coords), 16)).astype(np.float16)
    print(f"[coordops] downsample wide keys batch={batch} grid={grid} N={len(coords)}", flush=True)
    _check_down(sc, dev, coords, feats, grid, batch, O.downsample)


@gpu
@pytest.mark.parametrize("name", ["c2_64_64", "c3_128_128", "c5_512_chain"])
def test_downsample_configs(dev, name):
    sc = _sc()
    wl = workloads.make(name)
    print(f"[coordops] downsample {name} N={wl.n}", flush=True)
    # shuffled rows: the parents and maxima must not depend on the input order
    perm = np.random.default_rng(5).permutation(wl.n)
    _check_down(sc, dev, wl.coords[perm], wl.feats[perm], wl.grid, wl.batch, O.downsample_np)


@gpu
def test_subdivide_small_and_roundtrip(dev):
    sc = _sc()
    wl = workloads.random_small(11, G=9, occ=0.3, cin=24, cout=1, batch=2)
    cc, cf, cg = sc.subdivide(_to(dev, wl.coords), _to(dev, wl.feats), wl.grid)
    rcc, rcf, rcg = O.subdivide(wl.coords, wl.feats, wl.grid)
    np.testing.assert_array_equal(cc.cpu().numpy(), rcc)
    np.testing.assert_array_equal(cf.cpu().numpy().view(np.uint16), rcf.view(np.uint16))
    assert cg == rcg
    cc2, _, _ = sc.subdivide(_to(dev, wl.coords), None, wl.grid)
    np.testing.assert_array_equal(cc2.cpu().numpy(), rcc)


@gpu
@pytest.mark.parametrize("name", ["c2_64_64", "c5_512_chain"])
def test_subdivide_configs_roundtrip(dev, name):
    """Full size: children of sampled sites against the oracle, and
    downsampling the children gives back the sorted input exactly."""
    sc = _sc()
    wl = workloads.make(name)
    print(f"[coordops] subdivide {name} N={wl.n}", flush=True)
    C = 16
    feats = wl.feats[:, :C].copy()
    cd = _to(dev, wl.coords)
    cc, cf, cg = sc.subdivide(cd, _to(dev, feats), wl.grid)
    rows = np.random.default_rng(3).choice(wl.n, 500, replace=False)
    rcc, rcf, _ = O.subdivide(wl.coords[rows], feats[rows], wl.grid)
    idx = (8 * rows[:, None] + np.arange(8)[None, :]).reshape(-1)
    np.testing.assert_array_equal(cc.cpu().numpy()[idx], rcc)
    np.testing.assert_array_equal(cf.cpu().numpy()[idx].view(np.uint16), rcf.view(np.uint16))
    pc, inv, pf, pg = sc.downsample(cc, cf, cg, wl.batch)
    order = np.lexsort(wl.coords.T[::-1])
    np.testing.assert_array_equal(pc.cpu().numpy(), wl.coords[order])
    np.testing.assert_array_equal(pf.cpu().numpy().view(np.uint16), feats[order].view(np.uint16))
    assert pg == tuple(wl.grid)


@gpu
def test_coordops_edges(dev):
    sc = _sc()
    # empty
    e = torch.zeros((0, 4), dtype=torch.int32, device=dev)
    pc, inv, pf, pg = sc.downsample(e, torch.zeros((0, 8), dtype=torch.float16, device=dev), (4, 4, 4), 1)
    assert pc.shape == (0, 4) and inv.shape == (0,) and pf.shape == (0, 8) and pg == (2, 2, 2)
    cc, cf, cg = sc.subdivide(e, None, (4, 4, 4))
    assert cc.shape == (0, 4)
    # out of range and a bad channel count are errors
    bad = _to(dev, np.array([[0, 4, 0, 0]], dtype=np.int32))
    with pytest.raises(sc.SubmconvError) as ex:
        sc.downsample(bad, None, (4, 4, 4), 1)
    assert ex.value.status == -2
    ok = _to(dev, np.array([[0, 1, 0, 0]], dtype=np.int32))
    with pytest.raises(sc.SubmconvError) as ex:
        sc.downsample(ok, torch.zeros((1, 12), dtype=torch.float16, device=dev), (4, 4, 4), 1)
    assert ex.value.status == -4
    # a repeated site is one more child of its parent
    rep = np.array([[0, 1, 1, 1], [0, 1, 1, 1], [0, 3, 3, 3]], dtype=np.int32)
    f = np.array([[1.0] * 8, [2.0] * 8, [-1.0] * 8], dtype=np.float16)
    _check_down(sc, dev, rep, f, (4, 4, 4), 1, O.downsample)
