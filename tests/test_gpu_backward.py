"""GPU parity of the backward (input and weight gradients) through the C ABI
against the CPU oracle.

Input gradient: fp16 output from fp32 accumulation, like the forward, so the
forward's tolerance |gpu - oracle| <= 1e-3 + 1e-2 |oracle| applies.

Weight gradient: fp32 output, each element a sum over the m pairs of one tap
(up to ~10^6 on the shell workloads) of exact fp16 x fp16 products, added in
fp32. With terms of random sign the running sums stay near sqrt(j) times a
term's size, so the rounding error of the whole sum has a standard deviation
of about 0.6 u S (u = 2^-24, S = sum |feats[j] grad_out[i]| over the summed
terms, computed by the oracle on absolute values); the GPU adds in blocks (the
MFMA accumulator per run of pairs, then a fixed-order sum of the runs'
partials), which only lowers it. The bound per element is |gpu - oracle| <=
1e-3 + 1e-5 |oracle| + 4 u S, several times that standard deviation; one
dropped, doubled or misplaced pair moves an element by about S / m on
average (0.6 S / m for a typical pair), which exceeds 4 u S for every m
below ~150,000 and stays near it above, and a dropped group of 32 pairs or
a tile moves it far beyond the bound at any m.
"""
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


def _say(msg):
    print(msg, flush=True)


def _to(dev, a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _assert_close(got, ref, what, atol=ATOL, rtol=RTOL, extra=None):
    got = np.asarray(got, dtype=np.float64)
    tol = atol + rtol * np.abs(ref)
    if extra is not None:
        tol = tol + extra
    bad = np.abs(got - ref) > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside tolerance; "
                             f"first {idx.tolist()} got {got[tuple(idx.T)]} ref {ref[tuple(idx.T)]}")


def _grad_out(wl, cout, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((wl.n, cout)).astype(np.float16)


U = 2.0 ** -24


def _check_weight_grad(got, kmap, feats, g, what, taps=None):
    """Element-wise against the oracle; ``taps`` restricts the check to those
    taps (the oracle then computes only their columns of the map)."""
    if taps is not None:
        km = np.full_like(kmap, -1)
        km[:, taps] = kmap[:, taps]
        kmap = km
    ref = oc.backward_weight(kmap, feats, g)
    scale = oc.backward_weight(kmap, np.abs(feats.astype(np.float64)), np.abs(g.astype(np.float64)))
    if taps is not None:
        got, ref, scale = got[taps], ref[taps], scale[taps]
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    _say(f"[{what}] max |err| = {err.max():.3g}, max |err| / (u S) = {(err / (U * scale + 1e-300)).max():.3g}")
    _assert_close(got, ref, what, atol=1e-3, rtol=1e-5, extra=4 * U * scale)


def _layer_case(sc, dev, wl, L, seed, morton=False, rows=None):
    coords = _to(dev, wl.coords)
    km = sc.build_map(coords, wl.grid, wl.batch, morton=morton)
    g = _grad_out(wl, L.cout, seed)
    gd = _to(dev, g)
    Wd = _to(dev, L.W)
    dx = sc.backward_input(km, gd, Wd).cpu().numpy()
    ref = oc.backward_input_rows(wl.coords, wl.grid, wl.batch, L.ksize, g, L.W, rows)
    _assert_close(dx if rows is None else dx[rows], ref, f"{wl.name} input grad")
    return km, g, gd


@gpu
@pytest.mark.parametrize("morton", [False, True])
@pytest.mark.parametrize("name", ["c1_16_8", "c2_64_64"])
def test_backward_uniform_full(dev, name, morton):
    sc = _sc()
    wl = workloads.make(name)
    for li, L in enumerate(wl.layers):
        _say(f"[backward] {name} layer {li} ksize={L.ksize} {L.cin}->{L.cout} morton={morton}")
        km, g, gd = _layer_case(sc, dev, wl, L, 50 + li, morton)
        dw = sc.backward_weight(km, _to(dev, wl.feats), gd, L.ksize).cpu().numpy()
        kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, L.ksize)
        _check_weight_grad(dw, kmap, wl.feats, g, f"{name} weight grad")
        km.free()


@gpu
@pytest.mark.parametrize("morton", [False, True])
def test_backward_c3_sampled_and_weight_grad(dev, morton):
    sc = _sc()
    wl = workloads.make("c3_128_128")
    L = wl.layers[0]
    rows = np.random.default_rng(7).choice(wl.n, 3000, replace=False)
    _say(f"[backward] c3 N={wl.n} morton={morton}")
    km, g, gd = _layer_case(sc, dev, wl, L, 60, morton=morton, rows=rows)
    dw = sc.backward_weight(km, _to(dev, wl.feats), gd, 3).cpu().numpy()
    kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    _check_weight_grad(dw, kmap, wl.feats, g, "c3 weight grad")
    # bitwise reproducible run to run
    dw2 = sc.backward_weight(km, _to(dev, wl.feats), gd, 3).cpu().numpy()
    np.testing.assert_array_equal(dw, dw2)
    km.free()


@gpu
@pytest.mark.slow
def test_backward_shell_c5_first_layer(dev):
    """Full size, the C5 shell's 64 -> 32 layer (1.5M rows, ~31M pairs): input
    gradient on sampled rows, weight gradient element by element against the
    oracle on the oracle's own map, which the GPU's must equal."""
    sc = _sc()
    wl = workloads.make("c5_512_chain")
    L = wl.layers[0]
    rows = np.random.default_rng(8).choice(wl.n, 2000, replace=False)
    _say(f"[backward] c5 layer 0 N={wl.n} {L.cin}->{L.cout}")
    km, g, gd = _layer_case(sc, dev, wl, L, 61, rows=rows)
    dw = sc.backward_weight(km, _to(dev, wl.feats), gd, 3).cpu().numpy()
    kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    np.testing.assert_array_equal(km.export().cpu().numpy(), kmap)
    _check_weight_grad(dw, kmap, wl.feats, g, "c5 weight grad")
    km.free()


@gpu
@pytest.mark.slow
def test_backward_shell_c4(dev):
    """Full size, the C4 shells (batch 2, 256 -> 256 channels, ~750k rows,
    ~15.6M pairs; 64-row groups and two 128-channel passes): input gradient
    on sampled rows; weight gradient element by element on the centre and
    three off-centre taps (the oracle's cost grows with every tap checked)."""
    sc = _sc()
    wl = workloads.make("c4_256_shell")
    L = wl.layers[0]
    rows = np.concatenate([np.random.default_rng(10).choice(wl.n, 1500, replace=False), [0, wl.n - 1]])
    _say(f"[backward] c4 N={wl.n} {L.cin}->{L.cout}")
    km, g, gd = _layer_case(sc, dev, wl, L, 62, rows=rows)
    dw = sc.backward_weight(km, _to(dev, wl.feats), gd, 3).cpu().numpy()
    kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    np.testing.assert_array_equal(km.export().cpu().numpy(), kmap)
    _check_weight_grad(dw, kmap, wl.feats, g, "c4 weight grad", taps=[0, 4, 13, 22])
    km.free()


SHAPES = [(8, 8), (16, 24), (40, 48), (32, 16), (32, 32), (64, 32), (64, 64), (128, 64),
          (128, 128), (96, 160), (256, 256), (32, 128), (128, 256)]


@gpu
@pytest.mark.parametrize("ksize", [3, 1])
@pytest.mark.parametrize("cin,cout", SHAPES)
def test_backward_shapes(dev, cin, cout, ksize):
    sc = _sc()
    wl = workloads.random_small(400 + cin + cout, G=14, occ=0.25, cin=cin, cout=cout, batch=2,
                                ksize=ksize, bias=False)
    L = wl.layers[0]
    _say(f"[backward] shape {cin}->{cout} ksize={ksize} N={wl.n}")
    km, g, gd = _layer_case(sc, dev, wl, L, 70)
    dw = sc.backward_weight(km, _to(dev, wl.feats), gd, ksize).cpu().numpy()
    kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, ksize)
    _check_weight_grad(dw, kmap, wl.feats, g, f"{cin}->{cout} weight grad")
    km.free()


@gpu
def test_backward_empty_and_single_site(dev):
    sc = _sc()
    # empty: zero gradients, no error
    coords = torch.zeros((0, 4), dtype=torch.int32, device=dev)
    km = sc.build_map(coords, (4, 4, 4), 1)
    dw = sc.backward_weight(km, torch.zeros((0, 16), dtype=torch.float16, device=dev),
                            torch.zeros((0, 8), dtype=torch.float16, device=dev), 3)
    assert dw.shape == (27, 16, 8) and float(dw.abs().max()) == 0.0
    km.free()
    # one site: dX = dY W[13]^T, dW[13] = X^T dY, the other taps zero
    c = np.array([[0, 1, 2, 3]], dtype=np.int32)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 32)).astype(np.float16)
    gy = rng.standard_normal((1, 32)).astype(np.float16)
    W = (rng.standard_normal((27, 32, 32)) * 0.1).astype(np.float16)
    km = sc.build_map(_to(dev, c), (5, 5, 5), 1)
    dx = sc.backward_input(km, _to(dev, gy), _to(dev, W)).cpu().numpy()
    _assert_close(dx, gy.astype(np.float64) @ W[13].astype(np.float64).T, "single-site input grad")
    dw = sc.backward_weight(km, _to(dev, x), _to(dev, gy), 3).cpu().numpy()
    exp = np.zeros((27, 32, 32))
    exp[13] = x.astype(np.float64).T @ gy.astype(np.float64)
    _assert_close(dw, exp, "single-site weight grad", atol=1e-5, rtol=1e-5)
    km.free()


@gpu
def test_autograd_function(dev):
    sc = _sc()
    wl = workloads.make("c2_64_64")
    L = wl.layers[0]
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    x = _to(dev, wl.feats).requires_grad_(True)
    W = _to(dev, L.W).requires_grad_(True)
    b = _to(dev, L.bias).requires_grad_(True)
    y = sc.SubMConv3dFunction.apply(x, W, b, km)
    g = _grad_out(wl, L.cout, 80)
    y.backward(_to(dev, g))
    rows = np.arange(0, wl.n, 7)
    _assert_close(x.grad.cpu().numpy()[rows],
                  oc.backward_input_rows(wl.coords, wl.grid, wl.batch, 3, g, L.W, rows), "autograd dX")
    kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    ref_w = oc.backward_weight(kmap, wl.feats, g)
    # the weight gradient is rounded to the weight's dtype (fp16) here
    _assert_close(W.grad.float().cpu().numpy(), ref_w, "autograd dW", atol=1e-2, rtol=2e-3)
    _assert_close(b.grad.cpu().numpy(), g.astype(np.float64).sum(0), "autograd db", atol=1e-2, rtol=1e-4)
    km.free()


@gpu
@pytest.mark.parametrize("n,cout", [(0, 8), (1, 16), (1000, 64), (209715, 128)])
def test_backward_bias(dev, n, cout):
    sc = _sc()
    g = np.random.default_rng(n + cout).standard_normal((n, cout)).astype(np.float16)
    got = sc.backward_bias(_to(dev, g)).cpu().numpy()
    ref = g.astype(np.float64).sum(0)
    # fp32 sums of n fp16 values: bound from sqrt(n) u sum |g|
    scale = np.abs(g.astype(np.float64)).sum(0)
    _assert_close(got, ref, "bias grad", atol=1e-5, rtol=1e-5, extra=1e-6 * scale)
    np.testing.assert_array_equal(got, sc.backward_bias(_to(dev, g)).cpu().numpy())


@gpu
@pytest.mark.parametrize("cin,cout", [(64, 64), (128, 128)])
def test_backward_dense_map_with_isolated_tiles(dev, cin, cout):
    """Input and weight gradients on a dense map (64-row groups) with 16 tiles
    of isolated sites between dense ones: units and positions with no
    off-centre entries inside the walks and windows."""
    sc = _sc()
    rng = np.random.default_rng(cin * 3 + cout)
    G, side, iso0, n_iso = 128, 32, 24, 16
    dense = np.argwhere(np.ones((side, side, side), dtype=bool)).astype(np.int32)
    iso = (np.argwhere(np.ones((20, 20, 20), dtype=bool)) * 2 + 70).astype(np.int32)[:n_iso * 256]
    xyz = np.concatenate([dense[:iso0 * 256], iso, dense[iso0 * 256:]])
    coords = np.ascontiguousarray(np.concatenate([np.zeros((len(xyz), 1), np.int32), xyz], axis=1))
    n = len(coords)
    _say(f"[backward isolated tiles] {cin}->{cout} N={n}")
    feats = rng.standard_normal((n, cin)).astype(np.float16)
    g = rng.standard_normal((n, cout)).astype(np.float16)
    W = (rng.standard_normal((27, cin, cout)) / np.sqrt(27 * cin)).astype(np.float16)
    km = sc.build_map(_to(dev, coords), (G, G, G), 1)
    gd = _to(dev, g)
    dx = sc.backward_input(km, gd, _to(dev, W)).cpu().numpy()
    rows = np.arange(0, n, 3)
    ref = oc.backward_input_rows(coords, (G, G, G), 1, 3, g, W, rows)
    _assert_close(dx[rows], ref, "input grad")
    dw = sc.backward_weight(km, _to(dev, feats), gd, 3).cpu().numpy()
    kmap = oc.kernel_map(coords, (G, G, G), 1, 3)
    np.testing.assert_array_equal(km.export().cpu().numpy(), kmap)
    _check_weight_grad(dw, kmap, feats, g, "weight grad")
    km.free()
