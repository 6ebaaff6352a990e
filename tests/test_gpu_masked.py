"""GPU parity of the masked implicit-GEMM forward through the C ABI against
the CPU oracle (same tolerance as the forward: fp32 accumulation, one fp16
rounding), and its agreement with the compacted forward."""
import numpy as np
import pytest
import torch

import workloads
from oracle import cpu as oc

gpu = pytest.mark.gpu
ATOL, RTOL = 1e-3, 1e-2


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
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _assert_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    bad = np.abs(got - ref) > ATOL + RTOL * np.abs(ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first {idx.tolist()}")


@gpu
@pytest.mark.parametrize("name,layer,nrows", [("c2_64_64", 0, None), ("c3_128_128", 0, 3000),
                                               ("c3_occ1", 0, None), ("c3_occ30", 0, 3000),
                                               ("c4_256_shell", 0, 1500), ("c5_512_chain", 0, 2000),
                                               ("c5_512_chain", 1, 2000)])
def test_masked_forward(dev, name, layer, nrows):
    sc = _sc()
    wl = workloads.make(name)
    L = wl.layers[layer]
    print(f"[masked] {name} layer {layer} {L.cin}->{L.cout} N={wl.n}", flush=True)
    feats = wl.feats if layer == 0 else np.random.default_rng(9).standard_normal((wl.n, L.cin)).astype(np.float16)
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    plan = sc.masked_plan(km)
    assert plan.row_taps >= km.active_pairs(3)
    fd, Wd, bd = _to(dev, feats), _to(dev, L.W), _to(dev, L.bias)
    out = sc.forward_masked(plan, fd, Wd, bd).cpu().numpy()
    rows = None if nrows is None else np.random.default_rng(2).choice(wl.n, nrows, replace=False)
    kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    ref = oc.submconv_rows(kmap, feats, L.W, L.bias, rows)
    _assert_close(out if rows is None else out[rows], ref, f"masked {name}")
    # the compacted forward gives the same values up to the addition order
    comp = sc.forward(km, fd, Wd, bd).cpu().numpy()
    _assert_close(out, comp.astype(np.float64), f"masked vs compacted {name}")
    # bitwise reproducible
    assert np.array_equal(out, sc.forward_masked(plan, fd, Wd, bd).cpu().numpy())
    plan.free()
    km.free()


@gpu
def test_masked_shapes_and_errors(dev):
    sc = _sc()
    for cin, cout in [(32, 32), (64, 96), (128, 64), (256, 128)]:
        wl = workloads.random_small(500 + cin + cout, G=12, occ=0.3, cin=cin, cout=cout, batch=2)
        L = wl.layers[0]
        km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
        plan = sc.masked_plan(km)
        out = sc.forward_masked(plan, _to(dev, wl.feats), _to(dev, L.W), _to(dev, L.bias)).cpu().numpy()
        kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
        _assert_close(out, oc.submconv_rows(kmap, wl.feats, L.W, L.bias), f"masked {cin}->{cout}")
        plan.free()
        km.free()
    wl = workloads.random_small(7, G=8, occ=0.3, cin=40, cout=32)
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    plan = sc.masked_plan(km)
    with pytest.raises(sc.SubmconvError) as ex:
        sc.forward_masked(plan, _to(dev, wl.feats), _to(dev, wl.layers[0].W))
    assert ex.value.status == -4
    plan.free()
    km.free()


@gpu
@pytest.mark.parametrize("cin,cout", [(64, 64), (128, 128)])
def test_masked_dense_map_with_isolated_tiles(dev, cin, cout):
    """The masked variant on a dense block with tiles of isolated sites (mask:
    the centre only) between its rows: sampled rows of both kinds."""
    sc = _sc()
    rng = np.random.default_rng(cin + 5 * cout)
    G, side, iso0, n_iso = 128, 32, 24, 16
    dense = np.argwhere(np.ones((side, side, side), dtype=bool)).astype(np.int32)
    iso = (np.argwhere(np.ones((20, 20, 20), dtype=bool)) * 2 + 70).astype(np.int32)[:n_iso * 256]
    xyz = np.concatenate([dense[:iso0 * 256], iso, dense[iso0 * 256:]])
    coords = np.ascontiguousarray(np.concatenate([np.zeros((len(xyz), 1), np.int32), xyz], axis=1))
    n = len(coords)
    feats = rng.standard_normal((n, cin)).astype(np.float16)
    W = (rng.standard_normal((27, cin, cout)) / np.sqrt(27 * cin)).astype(np.float16)
    bias = (rng.standard_normal(cout) * 0.1).astype(np.float32)
    km = sc.build_map(_to(dev, coords), (G, G, G), 1)
    plan = sc.masked_plan(km)
    out = sc.forward_masked(plan, _to(dev, feats), _to(dev, W), _to(dev, bias)).float().cpu().numpy()
    rows = np.concatenate([np.arange(iso0 * 256 - 300, (iso0 + n_iso) * 256 + 300, 7),
                           rng.choice(n, 1500, replace=False)])
    kmap = oc.kernel_map(coords, (G, G, G), 1, 3)
    np.testing.assert_array_equal(km.export().cpu().numpy(), kmap)
    ref = oc.submconv_rows(kmap, feats, W, bias, rows)
    _assert_close(out[rows], ref, "masked, isolated tiles")
    km.free()
