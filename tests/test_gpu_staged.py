"""GPU parity of the staged forwards (dense maps) against the CPU oracle,
through the C ABI.

On a dense map the build also makes the staged plan (units of up to 128 rows
whose distinct neighbour rows fit in LDS), and forwards of 32 -> 32, 64 -> 32
and 32 -> 64 channels (k_fwd_staged) and of 128 -> 256 and 256 -> 256
channels (k_fwd_staged_wide, the rows staged in 64-channel slices) take it.
The tolerance is the forward's: |gpu - oracle| <= 1e-3 + 1e-2 |oracle| per
element. A row's result is summed in the same order whatever unit it falls
in, so maps in raster and Morton order give the same bits.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import cpu as oc
from oracle import oracle as op

from test_gpu_parity import (_assert_close, _bf16_tensor, _bf16_values, _say, _sc, _to, dev,  # noqa: F401
                             gpu)

STAGED_SHAPES = [(32, 32), (64, 32), (32, 64), (128, 256), (256, 256)]


def _dense_cube(G, batch=1):
    c = np.stack(np.meshgrid(np.arange(G), np.arange(G), np.arange(G), indexing="ij"), -1).reshape(-1, 3)
    parts = [np.concatenate([np.full((c.shape[0], 1), b, np.int32), c.astype(np.int32)], 1)
             for b in range(batch)]
    return np.concatenate(parts, 0)


def _layer(rng, cin, cout, bias=True):
    W = (rng.standard_normal((27, cin, cout)) / np.sqrt(27 * cin)).astype(np.float16)
    b = (rng.standard_normal(cout) * 0.1).astype(np.float32) if bias else None
    return W, b


@gpu
def test_kernel_choice_reports_the_staged_forward(dev):
    sc = _sc()
    # 20 neighbours per row: dense; 3.5: sparse
    assert sc.forward_kernel(1000, 20000, 64, 32) == 2
    assert sc.forward_kernel(1000, 20000, 32, 64) == 2
    assert sc.forward_kernel(1000, 20000, 32, 32) == 2
    assert sc.forward_kernel(1000, 20000, 64, 64) == 1
    assert sc.forward_kernel(1000, 20000, 128, 32) == 1
    assert sc.forward_kernel(1000, 3500, 64, 32) == 1
    assert sc.forward_kernel(1000, 20000, 64, 32, ksize=1) == 1
    assert sc.forward_kernel(1000, 20000, 256, 256) == 2
    assert sc.forward_kernel(1000, 20000, 128, 256) == 2
    assert sc.forward_kernel(1000, 20000, 256, 128) == 1
    assert sc.forward_kernel(1000, 20000, 128, 128) == 1
    assert sc.forward_kernel(1000, 3500, 256, 256) == 1


@gpu
@pytest.mark.slow
@pytest.mark.parametrize("morton", [False, True])
def test_c5_layers_staged(dev, morton):
    # the 512^3 shell: both 3x3x3 layers and the first layer's input gradient
    # against the oracle on sampled rows, against the compacted-list kernel
    # on every row, and raster against Morton order bit for bit
    sc = _sc()
    wl = workloads.make("c5_512_chain")
    coords = _to(dev, wl.coords)
    _say(f"[staged c5] N={wl.n} morton={morton}")
    km = sc.build_map(coords, wl.grid, wl.batch, morton=morton)
    kp = sc.build_map(coords, wl.grid, wl.batch, morton=morton, staged=False)
    ko = sc.build_map(coords, wl.grid, wl.batch, morton=not morton)
    # dense: the plan is built by default; every row staged at least once
    units, srows = km.staged()
    assert units >= -(-wl.n // 128) and srows >= wl.n, (units, srows)
    kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    rows = np.random.default_rng(11).choice(wl.n, 3000, replace=False)
    rows_t = torch.from_numpy(rows).to(dev)
    x = _to(dev, wl.feats)
    for li, L in enumerate(wl.layers[:2]):
        _say(f"[staged c5] layer {li} {L.cin}->{L.cout}")
        W = _to(dev, L.W)
        y = sc.forward(km, x, W)
        ref = oc.submconv_rows(kmap, x.cpu().numpy(), L.W, None, rows)
        _assert_close(y[rows_t].float().cpu().numpy(), ref, f"staged c5 layer {li}")
        yp = sc.forward(kp, x, W)
        _assert_close(y.float().cpu().numpy(), yp.float().cpu().numpy().astype(np.float64),
                      f"staged vs compacted, layer {li}")
        assert torch.equal(y, sc.forward(ko, x, W)), "raster and Morton order differ"
        assert torch.equal(y, sc.forward(km, x, W)), "not reproducible"
        x = y
    L = wl.layers[0]
    g = torch.from_numpy(workloads.normal_f16(np.random.default_rng(12), (wl.n, L.cout))).to(dev)
    _say("[staged c5] input gradient 32->64")
    dx = sc.backward_input(km, g, _to(dev, L.W))
    ref = oc.backward_input_rows(wl.coords, wl.grid, wl.batch, 3, g.cpu().numpy(), L.W, rows)
    _assert_close(dx[rows_t].float().cpu().numpy(), ref, "staged c5 input gradient")
    for k in (km, kp, ko):
        k.free()


@gpu
@pytest.mark.slow
def test_c4_layer_staged_wide(dev):
    # the 256^3 shells (two items, 256 -> 256): the forward against the oracle
    # on sampled rows and against the compacted-list kernel on every row,
    # raster against Morton order bit for bit; the input gradient (also
    # 256 -> 256, so staged too) on sampled rows
    sc = _sc()
    wl = workloads.make("c4_256_shell")
    L = wl.layers[0]
    coords = _to(dev, wl.coords)
    _say(f"[staged c4] N={wl.n} {L.cin}->{L.cout}")
    km = sc.build_map(coords, wl.grid, wl.batch)
    kp = sc.build_map(coords, wl.grid, wl.batch, staged=False)
    ko = sc.build_map(coords, wl.grid, wl.batch, morton=True)
    units, srows = km.staged()
    assert units >= -(-wl.n // 128) and srows >= wl.n, (units, srows)
    assert sc.forward_kernel(wl.n, km.active_pairs(3), L.cin, L.cout) == 2
    kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    rows = np.concatenate([np.random.default_rng(21).choice(wl.n, 1500, replace=False), [0, wl.n - 1]])
    rows_t = torch.from_numpy(rows).to(dev)
    x, W = _to(dev, wl.feats), _to(dev, L.W)
    b = _to(dev, (np.random.default_rng(22).standard_normal(L.cout) * 0.1).astype(np.float32))
    y = sc.forward(km, x, W, b)
    ref = oc.submconv_rows(kmap, wl.feats, L.W, b.cpu().numpy(), rows)
    _assert_close(y[rows_t].float().cpu().numpy(), ref, "staged c4 forward")
    yp = sc.forward(kp, x, W, b)
    _assert_close(y.float().cpu().numpy(), yp.float().cpu().numpy().astype(np.float64),
                  "staged vs compacted, c4")
    assert torch.equal(y, sc.forward(ko, x, W, b)), "raster and Morton order differ"
    assert torch.equal(y, sc.forward(km, x, W, b)), "not reproducible"
    g = torch.from_numpy(workloads.normal_f16(np.random.default_rng(23), (wl.n, L.cout))).to(dev)
    _say("[staged c4] input gradient")
    dx = sc.backward_input(km, g, W)
    ref = oc.backward_input_rows(wl.coords, wl.grid, wl.batch, 3, g.cpu().numpy(), L.W, rows)
    _assert_close(dx[rows_t].float().cpu().numpy(), ref, "staged c4 input gradient")
    for k in (km, kp, ko):
        k.free()


@gpu
@pytest.mark.parametrize("cin,cout", STAGED_SHAPES)
@pytest.mark.parametrize("morton", [False, True])
def test_dense_cube_splits_units(dev, cin, cout, morton):
    # a fully occupied 24^3 cube in raster order: a 128-row tile touches
    # ~3 x 7 x 24 rows, more than a unit stages, so tiles split into halves
    # (and quarters); every row against the oracle
    sc = _sc()
    coords = _dense_cube(24)
    rng = np.random.default_rng(cin * 7 + cout)
    W, b = _layer(rng, cin, cout)
    feats = workloads.normal_f16(rng, (coords.shape[0], cin))
    _say(f"[staged cube] {cin}->{cout} morton={morton}")
    km = sc.build_map(_to(dev, coords), (24, 24, 24), 1, morton=morton)
    out = sc.forward(km, _to(dev, feats), _to(dev, W), _to(dev, b)).float().cpu().numpy()
    kmap = oc.kernel_map(coords, (24, 24, 24), 1, 3)
    _assert_close(out, oc.submconv_rows(kmap, feats, W, b), f"staged cube {cin}->{cout}")
    km.free()


@gpu
@pytest.mark.parametrize("n", [1, 2, 3, 31, 127, 128, 129, 257, 1001])
@pytest.mark.parametrize("cin,cout", STAGED_SHAPES)
def test_forced_staged_ragged(dev, n, cin, cout):
    # the plan forced on small sparse maps: row counts around the unit size,
    # odd counts (the table's padded stride), isolated sites (only the centre)
    sc = _sc()
    rng = np.random.default_rng(n * 13 + cin + cout)
    G = 12
    flat = rng.choice(G ** 3, n, replace=False)
    coords = np.stack([np.zeros(n, np.int64), flat // (G * G), (flat // G) % G, flat % G], 1).astype(np.int32)
    W, b = _layer(rng, cin, cout, bias=bool(n % 2))
    feats = workloads.normal_f16(rng, (n, cin))
    km = sc.build_map(_to(dev, coords), (G, G, G), 1, staged=True)
    out = sc.forward(km, _to(dev, feats), _to(dev, W), _to(dev, b)).float().cpu().numpy()
    kmap = oc.kernel_map(coords, (G, G, G), 1, 3)
    _assert_close(out, oc.submconv_rows(kmap, feats, W, b), f"forced staged n={n} {cin}->{cout}")
    kp = sc.build_map(_to(dev, coords), (G, G, G), 1, staged=False)
    units, srows = km.staged()
    assert 1 <= units <= -(-n // 16) and n <= srows <= 27 * n, (units, srows)
    assert kp.staged() == (0, 0)
    outp = sc.forward(kp, _to(dev, feats), _to(dev, W), _to(dev, b)).float().cpu().numpy()
    _assert_close(out, outp.astype(np.float64), "staged vs compacted")
    km.free()
    kp.free()


@gpu
@pytest.mark.parametrize("cin,cout", STAGED_SHAPES)
def test_staged_bf16_and_input_grad(dev, cin, cout):
    # bf16 features and weights on a dense two-item map; the forward and the
    # input gradient (cout -> cin channels: staged when that shape is)
    sc = _sc()
    wl = workloads.random_small(500 + cin + cout, G=14, occ=0.9, cin=cin, cout=cout, batch=2, ksize=3)
    rng = np.random.default_rng(cin + 3 * cout)
    fb = workloads.normal_bf16_bits(rng, (wl.n, cin))
    Wb = workloads.normal_bf16_bits(rng, wl.layers[0].W.shape, std=1.0 / np.sqrt(27 * cin))
    gb = workloads.normal_bf16_bits(rng, (wl.n, cout))
    _say(f"[staged bf16] {cin}->{cout} N={wl.n}")
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    F, Wd, G = (op.bf16_bits_to_float64(v) for v in (fb, Wb, gb))
    out = sc.forward(km, _bf16_tensor(dev, fb), _bf16_tensor(dev, Wb), _to(dev, wl.layers[0].bias))
    _assert_close(_bf16_values(out), oc.submconv_rows(kmap, F, Wd, wl.layers[0].bias), "bf16 forward")
    dx = sc.backward_input(km, _bf16_tensor(dev, gb), _bf16_tensor(dev, Wb))
    _assert_close(_bf16_values(dx), oc.backward_input_rows(wl.coords, wl.grid, wl.batch, 3, G, Wd),
                  "bf16 input gradient")
    km.free()


# ----------------------------------------------------------------------------
# weight gradient on the staged plan (k_bwd_weight_staged)
# ----------------------------------------------------------------------------

WGRAD_SHAPES = [(32, 32), (64, 32), (32, 64)]


def _wgrad(sc, dev, km, feats, g, cin, cout):
    return sc.backward_weight(km, _to(dev, feats), _to(dev, g), 3).cpu().numpy()


@gpu
@pytest.mark.parametrize("n", [1, 2, 3, 31, 127, 128, 129, 257, 1001])
@pytest.mark.parametrize("cin,cout", WGRAD_SHAPES)
def test_staged_weight_grad_ragged(dev, n, cin, cout):
    # the plan forced on small sparse maps: units of every size, workgroups
    # with no unit (their partials are zero), odd row counts
    from test_gpu_backward import _check_weight_grad
    sc = _sc()
    rng = np.random.default_rng(n * 31 + cin + 2 * cout)
    G = 12
    flat = rng.choice(G ** 3, n, replace=False)
    coords = np.stack([np.zeros(n, np.int64), flat // (G * G), (flat // G) % G, flat % G], 1).astype(np.int32)
    feats = workloads.normal_f16(rng, (n, cin))
    g = workloads.normal_f16(rng, (n, cout))
    km = sc.build_map(_to(dev, coords), (G, G, G), 1, staged=True)
    kp = sc.build_map(_to(dev, coords), (G, G, G), 1, staged=False)
    dw = _wgrad(sc, dev, km, feats, g, cin, cout)
    kmap = oc.kernel_map(coords, (G, G, G), 1, 3)
    _check_weight_grad(dw, kmap, feats, g, f"staged weight grad n={n} {cin}->{cout}")
    dwp = _wgrad(sc, dev, kp, feats, g, cin, cout)
    _check_weight_grad(dwp, kmap, feats, g, f"pairwise weight grad n={n} {cin}->{cout}")
    km.free()
    kp.free()


@gpu
@pytest.mark.parametrize("cin,cout", WGRAD_SHAPES)
@pytest.mark.parametrize("morton", [False, True])
def test_staged_weight_grad_dense_cube(dev, cin, cout, morton):
    # a fully occupied 24^3 cube (units split into halves and quarters), every
    # element against the oracle; the same call twice gives the same bits
    from test_gpu_backward import _check_weight_grad
    sc = _sc()
    coords = _dense_cube(24)
    rng = np.random.default_rng(cin * 5 + cout + morton)
    feats = workloads.normal_f16(rng, (coords.shape[0], cin))
    g = workloads.normal_f16(rng, (coords.shape[0], cout))
    _say(f"[staged wgrad cube] {cin}->{cout} morton={morton}")
    km = sc.build_map(_to(dev, coords), (24, 24, 24), 1, morton=morton)
    assert km.staged()[0] > 0
    dw = _wgrad(sc, dev, km, feats, g, cin, cout)
    _check_weight_grad(dw, oc.kernel_map(coords, (24, 24, 24), 1, 3), feats, g,
                       f"staged weight grad cube {cin}->{cout}")
    assert np.array_equal(dw, _wgrad(sc, dev, km, feats, g, cin, cout)), "not reproducible"
    km.free()


@gpu
@pytest.mark.slow
def test_c5_second_layer_weight_grad(dev):
    # the 512^3 shell's 32 -> 32 layer: every element of the centre tap and
    # of two off-centre taps against the oracle (the first layer's weight
    # gradient, 64 -> 32, is checked in full in the backward tests)
    from test_gpu_backward import _check_weight_grad
    sc = _sc()
    wl = workloads.make("c5_512_chain")
    L = wl.layers[1]
    rng = np.random.default_rng(71)
    x = workloads.normal_f16(rng, (wl.n, L.cin))
    g = workloads.normal_f16(rng, (wl.n, L.cout))
    _say(f"[staged wgrad c5] N={wl.n} {L.cin}->{L.cout}")
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    assert km.staged()[0] > 0
    dw = _wgrad(sc, dev, km, x, g, L.cin, L.cout)
    kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    _check_weight_grad(dw, kmap, x, g, "staged weight grad c5 32->32", taps=[0, 13, 22])
    km.free()
