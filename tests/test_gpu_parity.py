"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Kernel map: bit for bit (caller row order, -1 sentinel), active pairs equal.
Features: |gpu - oracle| <= 1e-3 + 1e-2 |oracle| per element, the tolerance
fixed for this operation (fp16 inputs, fp32 accumulation, one fp16 rounding:
the rounding alone is 2^-11 relative, well inside it).
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from oracle import cpu as oc
from oracle import oracle as op

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


def _assert_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside tolerance; "
                             f"first {idx.tolist()} got {got[tuple(idx.T)]} ref {ref[tuple(idx.T)]}")


def _run_map(sc, dev, wl, morton):
    coords = _to(dev, wl.coords)
    km = sc.build_map(coords, wl.grid, wl.batch, morton=morton)
    return km


def _check_map(km, wl, ref_map=None):
    if ref_map is None:
        ref_map = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    got = km.export().cpu().numpy()
    np.testing.assert_array_equal(got, ref_map)
    assert km.active_pairs(3) == int((ref_map >= 0).sum())
    assert km.active_pairs(1) == wl.n
    order = km.order().cpu().numpy()
    np.testing.assert_array_equal(np.sort(order), np.arange(wl.n))
    return ref_map


# ----------------------------------------------------------------------------
# the named configurations
# ----------------------------------------------------------------------------


@gpu
@pytest.mark.parametrize("morton", [False, True])
@pytest.mark.parametrize("name", ["c1_16_8", "c2_64_64", "c3_128_128"])
def test_uniform_configs_full(dev, name, morton):
    sc = _sc()
    wl = workloads.make(name)
    _say(f"[{name} morton={morton}] N={wl.n}")
    km = _run_map(sc, dev, wl, morton)
    ref_map = _check_map(km, wl)
    feats = _to(dev, wl.feats)
    for li, L in enumerate(wl.layers):
        _say(f"[{name}] layer {li} ksize={L.ksize} {L.cin}->{L.cout}")
        out = sc.forward(km, feats, _to(dev, L.W), _to(dev, L.bias)).float().cpu().numpy()
        km_l = ref_map if L.ksize == 3 else np.arange(wl.n, dtype=np.int32)[:, None]
        ref = oc.submconv_rows(km_l, wl.feats, L.W, L.bias)
        _assert_close(out, ref, f"{name} layer {li}")


@gpu
@pytest.mark.slow
def test_c4_shell_256(dev):
    sc = _sc()
    wl = workloads.make("c4_256_shell")
    _say(f"[c4] N={wl.n}")
    km = _run_map(sc, dev, wl, False)
    ref_map = _check_map(km, wl)
    L = wl.layers[0]
    out = sc.forward(km, _to(dev, wl.feats), _to(dev, L.W), None)
    rows = np.random.default_rng(0).choice(wl.n, 1500, replace=False)
    rows = np.concatenate([rows, [0, wl.n - 1]])
    got = out[torch.from_numpy(rows).to(dev)].float().cpu().numpy()
    ref = oc.submconv_rows(ref_map, wl.feats, L.W, None, rows)
    _assert_close(got, ref, "c4 sampled rows")


@gpu
@pytest.mark.slow
def test_c5_chain_512(dev):
    sc = _sc()
    wl = workloads.make("c5_512_chain")
    _say(f"[c5] N={wl.n}")
    km = _run_map(sc, dev, wl, True)
    ref_map = _check_map(km, wl)
    x = _to(dev, wl.feats)
    rows = np.random.default_rng(1).choice(wl.n, 3000, replace=False)
    rows_t = torch.from_numpy(rows).to(dev)
    for li, L in enumerate(wl.layers):
        _say(f"[c5] layer {li} ksize={L.ksize} {L.cin}->{L.cout}")
        x_np = x.cpu().numpy()  # the oracle consumes the GPU's fp16 input of this layer
        y = sc.forward(km, x, _to(dev, L.W), None)
        km_l = ref_map if L.ksize == 3 else np.arange(wl.n, dtype=np.int32)[:, None]
        ref = oc.submconv_rows(km_l, x_np, L.W, None, rows)
        _assert_close(y[rows_t].float().cpu().numpy(), ref, f"c5 layer {li}")
        x = y


# ----------------------------------------------------------------------------
# shapes, ragged tiles and edge cases
# ----------------------------------------------------------------------------

SHAPES = [(8, 8), (16, 24), (40, 48), (32, 16), (32, 32), (64, 32), (64, 64), (128, 64),
          (128, 128), (256, 256), (32, 128), (128, 256)]


@gpu
@pytest.mark.parametrize("cin,cout", SHAPES)
@pytest.mark.parametrize("ksize", [3, 1])
def test_shapes_small(dev, cin, cout, ksize):
    sc = _sc()
    wl = workloads.random_small(1000 + cin + cout, G=14, occ=0.25, cin=cin, cout=cout, batch=2,
                                ksize=ksize, bias=True)
    _say(f"[shape {cin}->{cout} k{ksize}] N={wl.n}")
    L = wl.layers[0]
    km = _run_map(sc, dev, wl, False)
    out = sc.forward(km, _to(dev, wl.feats), _to(dev, L.W), _to(dev, L.bias)).float().cpu().numpy()
    kref = op.kernel_map(wl.coords, wl.grid, ksize, wl.batch)
    ref = oc.submconv_rows(kref, wl.feats, L.W, L.bias)
    _assert_close(out, ref, f"{cin}->{cout} k{ksize}")


@gpu
@pytest.mark.parametrize("cin,cout,ksize,morton", [(64, 256, 3, False), (128, 64, 3, True),
                                                   (32, 32, 3, False), (128, 128, 1, False)])
def test_persistent_walk_many_units(dev, cin, cout, ksize, morton):
    # ~60k rows: 235 row tiles, several units per workgroup of the persistent
    # forward (two column tiles at Cout = 256, several workgroups per CU at
    # 32 and 64 columns), every output row against the oracle
    sc = _sc()
    wl = workloads.uniform_workload(64, 60000, [(ksize, cin, cout)], seed=900 + cin + cout,
                                    bias_kind="normal", name="walk")
    L = wl.layers[0]
    _say(f"[walk {cin}->{cout} k{ksize} morton={morton}] N={wl.n}")
    km = _run_map(sc, dev, wl, morton)
    out = sc.forward(km, _to(dev, wl.feats), _to(dev, L.W), _to(dev, L.bias)).float().cpu().numpy()
    kref = oc.kernel_map(wl.coords, wl.grid, wl.batch, ksize)
    ref = oc.submconv_rows(kref, wl.feats, L.W, L.bias)
    _assert_close(out, ref, f"walk {cin}->{cout} k{ksize}")
    km.free()


@gpu
@pytest.mark.parametrize("n", [1, 2, 15, 16, 17, 63, 64, 65, 255, 256, 257, 511, 513, 1000])
def test_ragged_row_counts(dev, n):
    sc = _sc()
    rng = np.random.default_rng(n)
    G = 12
    coords = workloads.uniform_coords(G, n, rng)
    feats = workloads.normal_f16(rng, (n, 128))
    W = workloads.normal_f16(rng, (27, 128, 128), std=0.05)
    bias = rng.standard_normal(128).astype(np.float32)
    _say(f"[ragged n={n}]")
    km = sc.build_map(_to(dev, coords), (G, G, G), 1)
    ref_map = oc.kernel_map(coords, (G, G, G), 1, 3)
    np.testing.assert_array_equal(km.export().cpu().numpy(), ref_map)
    out = sc.forward(km, _to(dev, feats), _to(dev, W), _to(dev, bias)).float().cpu().numpy()
    ref = oc.submconv_rows(ref_map, feats, W, bias)
    _assert_close(out, ref, f"ragged {n}")


@gpu
def test_empty_input(dev):
    sc = _sc()
    coords = torch.zeros((0, 4), dtype=torch.int32, device=dev)
    km = sc.build_map(coords, (8, 8, 8), 1)
    assert km.num_rows == 0 and km.active_pairs() == 0
    assert km.export().shape == (0, 27)
    out = sc.forward(km, torch.zeros((0, 32), dtype=torch.float16, device=dev),
                     torch.zeros((27, 32, 32), dtype=torch.float16, device=dev))
    assert out.shape == (0, 32)


@gpu
def test_dense_block_full_occupancy(dev):
    """100 % occupancy: every interior site has all 27 neighbours."""
    sc = _sc()
    G = 9
    lin = np.arange(G ** 3)
    coords = np.stack([np.zeros_like(lin), lin // (G * G), (lin // G) % G, lin % G], 1).astype(np.int32)
    rng = np.random.default_rng(5)
    feats = workloads.normal_f16(rng, (len(lin), 64))
    W = workloads.normal_f16(rng, (27, 64, 64), std=0.03)
    km = sc.build_map(_to(dev, coords), (G, G, G), 1)
    ref_map = oc.kernel_map(coords, (G, G, G), 1, 3)
    np.testing.assert_array_equal(km.export().cpu().numpy(), ref_map)
    out = sc.forward(km, _to(dev, feats), _to(dev, W)).float().cpu().numpy()
    _assert_close(out, oc.submconv_rows(ref_map, feats, W, None), "dense block")


@gpu
def test_golden_hand_case_on_gpu(dev):
    """The hand-derived four-site case, padded to Cin = Cout = 8 with zeros."""
    sc = _sc()
    coords = np.array([[0, 1, 1, 1], [0, 2, 1, 1], [0, 1, 2, 1], [0, 2, 2, 2]], dtype=np.int32)
    feats = np.zeros((4, 8), dtype=np.float16)
    feats[:, 0] = [1, 2, 3, 5]
    W = np.zeros((27, 8, 8), dtype=np.float16)
    W[:, 0, 0] = np.arange(1, 28)
    bias = np.zeros(8, dtype=np.float32)
    bias[0] = 0.5
    km = sc.build_map(_to(dev, coords), (4, 4, 4), 1)
    out = sc.forward(km, _to(dev, feats), _to(dev, W), _to(dev, bias)).float().cpu().numpy()
    np.testing.assert_array_equal(out[:, 0], [246.5, 147.5, 213.5, 103.5])
    np.testing.assert_array_equal(out[:, 1:], 0)


# ----------------------------------------------------------------------------
# properties: determinism, order independence, batch independence
# ----------------------------------------------------------------------------


@gpu
def test_bitwise_determinism_and_morton_order(dev):
    sc = _sc()
    wl = workloads.make("c2_64_64")
    L = wl.layers[0]
    feats, W = _to(dev, wl.feats), _to(dev, L.W)
    km0 = _run_map(sc, dev, wl, False)
    km1 = _run_map(sc, dev, wl, True)
    a = sc.forward(km0, feats, W)
    b = sc.forward(km0, feats, W)
    c = sc.forward(km1, feats, W)
    c2 = sc.forward(km1, feats, W)
    # run to run: bit for bit (fixed accumulation order, no atomics)
    assert torch.equal(a, b)
    assert torch.equal(c, c2)
    # the processing order changes which rows share a tile, not the order in
    # which a row's terms are added (the centre first, then the other taps in
    # a fixed order): the same map and the same outputs bit for bit
    assert torch.equal(km0.export(), km1.export())
    assert torch.equal(a, c)
    ref = oc.submconv_rows(oc.kernel_map(wl.coords, wl.grid, wl.batch, 3), wl.feats, L.W, None)
    _assert_close(a.float().cpu().numpy(), ref, "raster order")
    assert not torch.equal(km1.order().cpu(), torch.arange(wl.n, dtype=torch.int32))


@gpu
def test_shuffled_rows_permute_outputs(dev):
    sc = _sc()
    wl = workloads.random_small(77, G=16, occ=0.2, cin=64, cout=64)
    L = wl.layers[0]
    perm = np.random.default_rng(3).permutation(wl.n)
    km = sc.build_map(_to(dev, wl.coords), wl.grid, 1)
    kp = sc.build_map(_to(dev, wl.coords[perm]), wl.grid, 1)
    a = sc.forward(km, _to(dev, wl.feats), _to(dev, L.W), _to(dev, L.bias))
    b = sc.forward(kp, _to(dev, wl.feats[perm]), _to(dev, L.W), _to(dev, L.bias))
    assert torch.equal(a[torch.from_numpy(perm).to(dev)], b)


@gpu
def test_batch_items_are_independent(dev):
    sc = _sc()
    wl = workloads.random_small(78, G=12, occ=0.3, cin=32, cout=32)
    two = np.concatenate([wl.coords, wl.coords])
    two[wl.n:, 0] = 1
    L = wl.layers[0]
    km = sc.build_map(_to(dev, two), wl.grid, 2)
    kmap = km.export().cpu().numpy()
    # no neighbour crosses the batch items
    assert (kmap[:wl.n][kmap[:wl.n] >= 0] < wl.n).all() and (kmap[wl.n:][kmap[wl.n:] >= 0] >= wl.n).all()
    out = sc.forward(km, _to(dev, np.concatenate([wl.feats, wl.feats])), _to(dev, L.W), _to(dev, L.bias))
    # the two items sit in different tiles; each row's terms are still added
    # in the same order, so the items' outputs are equal bit for bit, and
    # both equal the single-item result to tolerance
    assert torch.equal(out[:wl.n], out[wl.n:])
    ref = oc.submconv_rows(op.kernel_map(wl.coords, wl.grid), wl.feats, L.W, L.bias)
    _assert_close(out[:wl.n].float().cpu().numpy(), ref, "item 0")


@gpu
def test_prepared_weights_and_module(dev):
    sc = _sc()
    wl = workloads.random_small(79, G=12, occ=0.3, cin=64, cout=128)
    L = wl.layers[0]
    km = sc.build_map(_to(dev, wl.coords), wl.grid, 1)
    feats = _to(dev, wl.feats)
    ref = sc.forward(km, feats, _to(dev, L.W), _to(dev, L.bias))
    wp = sc.prepare_weights(_to(dev, L.W))
    again = sc.forward(km, feats, bias=_to(dev, L.bias), prepared=wp)
    assert torch.equal(ref, again)
    # new values into the same handle
    W2 = _to(dev, (L.W * 0.5).astype(np.float16))
    wp.set(W2)
    assert torch.equal(sc.forward(km, feats, bias=_to(dev, L.bias), prepared=wp),
                       sc.forward(km, feats, W2, _to(dev, L.bias)))
    wp.free()
    mod = sc.SubMConv3d(64, 128, 3, bias=True, device=dev)
    with torch.no_grad():
        mod.weight.copy_(_to(dev, L.W))
        mod.bias.copy_(_to(dev, L.bias))
    assert torch.equal(mod(km, feats), ref)


# ----------------------------------------------------------------------------
# errors (forced from the host with bad inputs; every kernel exits normally)
# ----------------------------------------------------------------------------


@gpu
def test_errors(dev):
    sc = _sc()
    dup = np.array([[0, 1, 1, 1], [0, 2, 2, 2], [0, 1, 1, 1]], dtype=np.int32)
    with pytest.raises(sc.SubmconvError) as e:
        sc.build_map(_to(dev, dup), (4, 4, 4), 1)
    assert e.value.status == -3
    oob = np.array([[0, 1, 1, 1], [0, 4, 0, 0]], dtype=np.int32)
    with pytest.raises(sc.SubmconvError) as e:
        sc.build_map(_to(dev, oob), (4, 4, 4), 1)
    assert e.value.status == -2
    neg = np.array([[0, 1, -1, 1]], dtype=np.int32)
    with pytest.raises(sc.SubmconvError) as e:
        sc.build_map(_to(dev, neg), (4, 4, 4), 1)
    assert e.value.status == -2
    bad_b = np.array([[1, 1, 1, 1]], dtype=np.int32)
    with pytest.raises(sc.SubmconvError) as e:
        sc.build_map(_to(dev, bad_b), (4, 4, 4), 1)
    assert e.value.status == -2
    ok = np.array([[0, 1, 1, 1], [0, 1, 1, 2]], dtype=np.int32)
    km = sc.build_map(_to(dev, ok), (4, 4, 4), 1)
    with pytest.raises(sc.SubmconvError) as e:
        sc.forward(km, torch.zeros((2, 12), dtype=torch.float16, device=dev),
                   torch.zeros((27, 12, 16), dtype=torch.float16, device=dev))
    assert e.value.status == -4
    # prepared weights carry their use: input-gradient weights are refused by
    # the forward, forward weights by the input gradient (checked in the
    # library, through the C ABI)
    lib = sc.load_library()
    W16 = torch.zeros((27, 16, 16), dtype=torch.float16, device=dev)
    wg = sc.Weights(W16, input_grad=True)
    wf = sc.Weights(W16)
    f16 = torch.zeros((2, 16), dtype=torch.float16, device=dev)
    o16 = torch.zeros((2, 16), dtype=torch.float16, device=dev)
    st = sc._stream(dev)
    assert lib.submconv_forward_prepared(km.handle, sc._ptr(f16), wg.handle, None, sc._ptr(o16),
                                         st) == -1
    assert lib.submconv_backward_input_prepared(km.handle, sc._ptr(f16), wf.handle, sc._ptr(o16),
                                                st) == -1
    assert lib.submconv_forward_prepared(km.handle, sc._ptr(f16), wf.handle, None, sc._ptr(o16),
                                         st) == 0
    # a misaligned bias is refused before launch
    b = torch.zeros(20, dtype=torch.float32, device=dev)
    assert lib.submconv_forward(km.handle, sc._ptr(f16), sc._ptr(W16), ctypes.c_void_p(b.data_ptr() + 4),
                                sc._ptr(o16), 16, 16, 3, st) == -1
    # the binding checks shapes and dtypes of out and bias
    with pytest.raises(ValueError):
        sc.forward(km, f16, W16, torch.zeros(15, dtype=torch.float32, device=dev))
    with pytest.raises(TypeError):
        sc.forward(km, f16, W16, torch.zeros(16, dtype=torch.float16, device=dev))
    with pytest.raises(ValueError):
        sc.forward(km, f16, W16, out=torch.zeros((2, 8), dtype=torch.float16, device=dev))
    torch.cuda.synchronize(dev)
    wg.free()
    wf.free()


def _blob_sites(rng, grid, batch, corners, side=10, occ=0.35):
    """Sites of occupancy ``occ`` in blocks of up to side^3 cells at the given
    corners (one per batch item and corner), with their batch column."""
    dims = [min(side, g) for g in grid]
    out = []
    for b in range(batch):
        for c in corners:
            lo = np.array([min(max(c[a], 0), grid[a] - dims[a]) for a in range(3)])
            cells = np.argwhere(rng.random(dims) < occ) + lo
            out.append(np.concatenate([np.full((len(cells), 1), b), cells], axis=1))
    return np.ascontiguousarray(np.concatenate(out).astype(np.int32))


@gpu
@pytest.mark.parametrize("grid,batch", [
    ((2048, 2048, 1024), 1),  # batch x volume = 2^32: one-word slots, top key 2^32 - 1
    ((2048, 2048, 1024), 2),  # 2^33: keys and rows in two arrays
    ((4096, 4096, 4096), 1),  # 2^36
    ((100, 3000, 7), 3),      # odd extents, a z extent below the blocks
])
def test_map_key_widths(dev, grid, batch):
    """The hash table's two slot layouts (packed keys below 2^32, or wider)
    give the oracle's map bit for bit, including the largest key; duplicates
    are found in both."""
    sc = _sc()
    rng = np.random.default_rng(sum(grid) + batch)
    far = tuple(g - 1 for g in grid)
    coords = _blob_sites(rng, grid, batch, [(0, 0, 0), far, (grid[0] // 2, grid[1] // 3, grid[2] // 5)])
    top = np.array([[batch - 1, *far]], dtype=np.int32)
    if not (coords == top).all(axis=1).any():
        coords = np.concatenate([coords, top])
    coords = coords[rng.permutation(len(coords))]
    _say(f"[map_key_widths] grid {grid} batch {batch}: {len(coords)} sites")
    ref = oc.kernel_map(coords, grid, batch, 3)
    for morton in (False, True):
        km = sc.build_map(_to(dev, coords), grid, batch, morton=morton)
        np.testing.assert_array_equal(km.export().cpu().numpy(), ref)
        assert km.active_pairs(3) == int((ref >= 0).sum())
        km.free()
    # a small forward on the same map
    cin = cout = 32
    feats = rng.standard_normal((len(coords), cin)).astype(np.float16)
    W = (rng.standard_normal((27, cin, cout)) / np.sqrt(27 * cin)).astype(np.float16)
    km = sc.build_map(_to(dev, coords), grid, batch)
    out = sc.forward(km, _to(dev, feats), _to(dev, W), None)
    _assert_close(out.float().cpu().numpy(), oc.submconv_rows(ref, feats, W, None), "forward")
    km.free()
    dup = np.concatenate([coords, coords[len(coords) // 2:len(coords) // 2 + 1]])
    with pytest.raises(sc.SubmconvError) as e:
        sc.build_map(_to(dev, dup), grid, batch)
    assert e.value.status == -3


@gpu
@pytest.mark.parametrize("cin,cout,side,iso0,n_iso,checked", [
    (64, 64, 75, 64, 64, 128),
    (128, 128, 75, 64, 64, 128),
    (256, 256, 46, 16, 16, 64),  # two 128-channel passes per unit
])
def test_dense_map_with_isolated_tiles(dev, cin, cout, side, iso0, n_iso, checked):
    """A dense map (64-row groups) whose row order puts n_iso tiles of
    isolated sites (no neighbour: only the centre's steps) after iso0 dense
    tiles, in a map large enough that the workgroups walk several units: every
    unit's lookahead must reach past such a short unit into the next one. The
    first `checked` rows of each tile of the first XCD's run are compared with
    the oracle."""
    sc = _sc()
    rng = np.random.default_rng(cin + cout)
    G = 160
    dense = np.argwhere(np.ones((side, side, side), dtype=bool)).astype(np.int32)  # raster order
    iso = (np.argwhere(np.ones((26, 26, 26), dtype=bool)) * 2 + 100).astype(np.int32)[:n_iso * 256]
    xyz = np.concatenate([dense[:iso0 * 256], iso, dense[iso0 * 256:]])
    coords = np.ascontiguousarray(np.concatenate([np.zeros((len(xyz), 1), np.int32), xyz], axis=1))
    n = len(coords)
    n_tiles = (n + 255) // 256
    per_xcd = (n_tiles + 7) // 8
    _say(f"[isolated tiles] {cin}->{cout} N={n} tiles={n_tiles}")
    feats = rng.standard_normal((n, cin)).astype(np.float16)
    W = (rng.standard_normal((27, cin, cout)) / np.sqrt(27 * cin)).astype(np.float16)
    km = sc.build_map(_to(dev, coords), (G, G, G), 1)
    assert km.tile_rows == 256  # dense: no wider tiles
    out = sc.forward(km, _to(dev, feats), _to(dev, W), None).float().cpu().numpy()
    # the reference uses the oracle's own map, which the GPU's must equal
    kmap = oc.kernel_map(coords, (G, G, G), 1, 3)
    np.testing.assert_array_equal(km.export().cpu().numpy(), kmap)
    # the isolated rows see only themselves
    assert (kmap[iso0 * 256:(iso0 + n_iso) * 256] >= 0).sum() == n_iso * 256
    rows = (np.arange(per_xcd)[:, None] * 256 + np.arange(checked)[None, :]).reshape(-1)
    rows = rows[rows < n]
    ref = oc.submconv_rows(kmap, feats, W, None, rows)
    _assert_close(out[rows], ref, "rows after short units")
    km.free()

@gpu
def test_builds_reuse_the_kept_scratch(dev):
    """Builds of alternating sizes and builders in one process: each reuses
    (or regrows) the device's kept scratch, left holding the previous build's
    table, keys and counts, and still gives the oracle's map."""
    sc = _sc()
    wls = [workloads.random_small(400 + i, G=g, occ=o, cin=8, cout=8)
           for i, (g, o) in enumerate([(48, 0.3), (10, 0.5), (64, 0.1), (6, 0.9), (48, 0.3)])]
    for i, w in enumerate(wls):
        ref = oc.kernel_map(w.coords, w.grid, w.batch, 3)
        for morton, sk in [(False, False), (True, False), (False, True), (True, True)]:
            km = sc.build_map(_to(dev, w.coords), w.grid, w.batch, morton=morton, sorted_keys=sk)
            np.testing.assert_array_equal(km.export().cpu().numpy(), ref,
                                          err_msg=f"build {i} morton={morton} sorted={sk}")
            assert km.active_pairs(3) == int((ref >= 0).sum())
            km.free()


@gpu
def test_builds_from_two_threads(dev):
    """Builds from two host threads on their own streams (they share the
    device's kept scratch, one at a time), of different sizes, in both
    orders: every map is the oracle's."""
    import threading
    sc = _sc()
    wls = [workloads.random_small(300 + i, G=g, occ=0.2, cin=32, cout=32) for i, g in enumerate((40, 14))]
    refs = [oc.kernel_map(w.coords, w.grid, w.batch, 3) for w in wls]
    coords = [_to(dev, w.coords) for w in wls]
    torch.cuda.synchronize()
    got = {}
    errs = []

    def work(i, reps):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for r in range(reps):
                    km = sc.build_map(coords[i], wls[i].grid, wls[i].batch, morton=bool(r & 1))
                    got[(i, r)] = km.export().cpu().numpy()
                    km.free()
        except Exception as e:  # reported below
            errs.append(repr(e))

    ts = [threading.Thread(target=work, args=(i, 6)) for i in (0, 1)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errs, errs
    for (i, r), k in got.items():
        np.testing.assert_array_equal(k, refs[i], err_msg=f"item {i} build {r}")
    assert len(got) == 12


# ----------------------------------------------------------------------------
# the sorted-key map builder: the same map, lists and results as the hash
# ----------------------------------------------------------------------------


@gpu
@pytest.mark.parametrize("morton", [False, True])
@pytest.mark.parametrize("name", ["c1_16_8", "c2_64_64", "c3_128_128", "c4_256_shell", "c5_512_chain"])
def test_sorted_key_builder_same_map(dev, name, morton):
    sc = _sc()
    wl = workloads.make(name)
    _say(f"[sorted keys] {name} morton={morton} N={wl.n}")
    coords = _to(dev, wl.coords)
    km_h = sc.build_map(coords, wl.grid, wl.batch, morton=morton)
    km_s = sc.build_map(coords, wl.grid, wl.batch, morton=morton, sorted_keys=True)
    a, b = km_h.export(), km_s.export()
    assert torch.equal(a, b)
    if name in ("c1_16_8", "c2_64_64"):
        np.testing.assert_array_equal(b.cpu().numpy(), oc.kernel_map(wl.coords, wl.grid, wl.batch, 3))
    assert km_h.active_pairs(3) == km_s.active_pairs(3)
    L = wl.layers[0]
    feats = _to(dev, wl.feats)
    Wd = _to(dev, L.W)
    bias = _to(dev, L.bias)
    # identical per-tile lists, so bitwise identical outputs
    assert torch.equal(sc.forward(km_h, feats, Wd, bias), sc.forward(km_s, feats, Wd, bias))
    km_h.free()
    km_s.free()


@gpu
def test_sorted_key_builder_errors(dev):
    sc = _sc()
    dup = _to(dev, np.array([[0, 1, 1, 1], [0, 2, 2, 2], [0, 1, 1, 1]], dtype=np.int32))
    with pytest.raises(sc.SubmconvError) as ex:
        sc.build_map(dup, (4, 4, 4), 1, sorted_keys=True)
    assert ex.value.status == -3
    out = _to(dev, np.array([[0, 1, 1, 4]], dtype=np.int32))
    with pytest.raises(sc.SubmconvError) as ex:
        sc.build_map(out, (4, 4, 4), 1, sorted_keys=True)
    assert ex.value.status == -2


# ----------------------------------------------------------------------------
# bf16: features, weights and output in bfloat16, fp32 accumulation. The
# output rounding is 2^-9 relative, inside the same tolerance.
# ----------------------------------------------------------------------------


def _bf16_case(wl_seed, n_rows_G, occ, cin, cout, ksize, batch=1):
    wl = workloads.random_small(wl_seed, G=n_rows_G, occ=occ, cin=cin, cout=cout, batch=batch,
                                ksize=ksize)
    rng = np.random.default_rng(wl_seed + 77)
    fb = workloads.normal_bf16_bits(rng, (wl.n, cin))
    Wb = workloads.normal_bf16_bits(rng, wl.layers[0].W.shape, std=1.0 / np.sqrt(27 * cin))
    return wl, fb, Wb


def _bf16_tensor(dev, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _bf16_values(t):
    return op.bf16_bits_to_float64(t.view(torch.int16).cpu().numpy().view(np.uint16))


@gpu
@pytest.mark.parametrize("ksize", [3, 1])
@pytest.mark.parametrize("cin,cout", [(8, 8), (32, 32), (64, 32), (64, 64), (128, 128), (256, 256), (40, 48)])
def test_bf16_forward_shapes(dev, cin, cout, ksize):
    sc = _sc()
    wl, fb, Wb = _bf16_case(900 + cin + cout, 14, 0.25, cin, cout, ksize, batch=2)
    _say(f"[bf16] forward {cin}->{cout} ksize={ksize} N={wl.n}")
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    bias = _to(dev, wl.layers[0].bias)
    out = sc.forward(km, _bf16_tensor(dev, fb), _bf16_tensor(dev, Wb), bias)
    assert out.dtype == torch.bfloat16
    kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, ksize)
    ref = oc.submconv_rows(kmap, op.bf16_bits_to_float64(fb), op.bf16_bits_to_float64(Wb),
                           wl.layers[0].bias)
    _assert_close(_bf16_values(out), ref, f"bf16 {cin}->{cout}")
    km.free()


@gpu
def test_bf16_c3_sampled_and_input_grad(dev):
    sc = _sc()
    wl = workloads.make("c3_128_128")
    L = wl.layers[0]
    rng = np.random.default_rng(31)
    fb = workloads.normal_bf16_bits(rng, (wl.n, L.cin))
    Wb = workloads.normal_bf16_bits(rng, L.W.shape, std=1.0 / np.sqrt(27 * L.cin))
    _say(f"[bf16] c3 N={wl.n}")
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    out = sc.forward(km, _bf16_tensor(dev, fb), _bf16_tensor(dev, Wb))
    rows = np.random.default_rng(4).choice(wl.n, 3000, replace=False)
    kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    F, Wd = op.bf16_bits_to_float64(fb), op.bf16_bits_to_float64(Wb)
    _assert_close(_bf16_values(out)[rows], oc.submconv_rows(kmap, F, Wd, None, rows), "bf16 c3")
    dx = sc.backward_input(km, _bf16_tensor(dev, fb), _bf16_tensor(dev, Wb))
    _assert_close(_bf16_values(dx)[rows],
                  oc.backward_input_rows(wl.coords, wl.grid, wl.batch, 3, F, Wd, rows), "bf16 c3 input grad")
    km.free()


@gpu
@pytest.mark.parametrize("cin,cout,dtype", [(32, 32, "fp16"), (64, 32, "bf16"), (32, 128, "fp16"),
                                            (64, 64, "bf16"), (128, 128, "fp16"), (128, 128, "bf16"),
                                            (256, 128, "bf16"), (256, 256, "fp16")])
def test_dense_maps_64row_groups(dev, cin, cout, dtype):
    # 95 % occupancy: ~240 entries per position and tile, so the forward takes
    # 64-row groups (Cin <= 64, or 128-channel passes with 128 columns);
    # every row against the oracle. The maps are built without the staged
    # plan, which 32- and 64-channel forwards on dense maps take otherwise.
    sc = _sc()
    seed = 700 + cin + cout
    _say(f"[dense {cin}->{cout} {dtype}]")
    if dtype == "fp16":
        wl = workloads.random_small(seed, G=14, occ=0.95, cin=cin, cout=cout, batch=2, ksize=3,
                                    bias=True)
        L = wl.layers[0]
        km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch, staged=False)
        out = sc.forward(km, _to(dev, wl.feats), _to(dev, L.W), _to(dev, L.bias)).float().cpu().numpy()
        kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
        ref = oc.submconv_rows(kmap, wl.feats, L.W, L.bias)
    else:
        wl, fb, Wb = _bf16_case(seed, 14, 0.95, cin, cout, 3, batch=2)
        km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch, staged=False)
        out = _bf16_values(sc.forward(km, _bf16_tensor(dev, fb), _bf16_tensor(dev, Wb),
                                      _to(dev, wl.layers[0].bias)))
        kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
        ref = oc.submconv_rows(kmap, op.bf16_bits_to_float64(fb), op.bf16_bits_to_float64(Wb),
                               wl.layers[0].bias)
    _assert_close(out, ref, f"dense {cin}->{cout} {dtype}")
    km.free()


@gpu
@pytest.mark.parametrize("cin,cout,dtype,morton,bias", [(128, 128, "fp16", False, False),
                                                       (128, 128, "bf16", True, True),
                                                       (256, 128, "fp16", False, True),
                                                       (64, 32, "fp16", True, False),
                                                       (32, 64, "bf16", False, False)])
def test_tiles_288_same_results(dev, cin, cout, dtype, morton, bias):
    # ~60k rows at 10 %: lists of 288-row tiles (209 tiles, a ragged last one)
    # give bit-identical forward and input-gradient outputs to 256-row tiles
    # (each row's products are summed in the same order); the weight gradient
    # against the oracle; every forward row against the oracle
    sc = _sc()
    seed = 950 + cin + cout
    wl = workloads.uniform_workload(85, 60000, [(3, cin, cout)], seed=seed,
                                    bias_kind="normal" if bias else None, name="t288")
    L = wl.layers[0]
    _say(f"[tiles 288 {cin}->{cout} {dtype} morton={morton} bias={bias}] N={wl.n}")
    coords = _to(dev, wl.coords)
    km256 = sc.build_map(coords, wl.grid, wl.batch, morton=morton, tile_rows=256)
    km288 = sc.build_map(coords, wl.grid, wl.batch, morton=morton, tile_rows=288)
    assert (km256.tile_rows, km288.tile_rows) == (256, 288)
    assert km256.active_pairs() == km288.active_pairs()
    assert torch.equal(km256.export(), km288.export())
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    feats = _to(dev, wl.feats).to(tdt)
    W = _to(dev, L.W).to(tdt)
    b = _to(dev, L.bias) if bias else None
    o256 = sc.forward(km256, feats, W, b)
    o288 = sc.forward(km288, feats, W, b)
    assert torch.equal(o256, o288), "forward differs between tile sizes"
    g = torch.from_numpy(np.random.default_rng(seed).standard_normal((wl.n, cout)).astype(np.float16))
    g = g.to(dev).to(tdt)
    gi256 = sc.backward_input(km256, g, W)
    gi288 = sc.backward_input(km288, g, W)
    assert torch.equal(gi256, gi288), "input gradient differs between tile sizes"
    if dtype == "fp16":
        feats64 = wl.feats.astype(np.float64)
        W64 = L.W.astype(np.float64)
    else:
        feats64 = feats.float().cpu().numpy().astype(np.float64)
        W64 = W.float().cpu().numpy().astype(np.float64)
    kref = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    ref = oc.submconv_rows(kref, feats64, W64, L.bias if bias else None)
    _assert_close(o288.float().cpu().numpy(), ref, f"t288 {cin}->{cout}")
    if dtype == "fp16":
        dw = sc.backward_weight(km288, feats, g, 3).cpu().numpy()
        dref = oc.backward_weight(kref, wl.feats, g.cpu().numpy())
        tol = 1e-3 + 1e-2 * np.abs(dref)
        assert (np.abs(dw - dref) <= tol).all(), "weight gradient (288-row tiles)"
    km256.free()
    km288.free()


@gpu
@pytest.mark.parametrize("n_tiles", [1, 9, 263])
def test_wide_tile_walk_sizes(dev, n_tiles):
    """288-row tiles walked in the balanced order the map build writes, with
    tile counts that leave XCDs empty (1), uneven (9) and one workgroup with
    fewer tiles than the rest (263): the 128 -> 128 forward (one workgroup
    per CU) equals the 256-row tiles' bit for bit and the oracle on every
    row."""
    sc = _sc()
    n = 288 * n_tiles - 7
    G = max(16, int(round((n / 0.1) ** (1 / 3))))
    wl = workloads.uniform_workload(G, n, [(3, 128, 128)], seed=1300 + n_tiles, bias_kind=None,
                                    name="walk")
    L = wl.layers[0]
    _say(f"[wide walk] n_tiles={n_tiles} N={wl.n} G={G}")
    coords = _to(dev, wl.coords)
    km256 = sc.build_map(coords, wl.grid, wl.batch, tile_rows=256)
    km288 = sc.build_map(coords, wl.grid, wl.batch, tile_rows=288)
    assert km288.tile_rows == 288
    feats = _to(dev, wl.feats)
    W = _to(dev, L.W)
    o288 = sc.forward(km288, feats, W)
    assert torch.equal(sc.forward(km256, feats, W), o288)
    ref = oc.submconv_rows(oc.kernel_map(wl.coords, wl.grid, wl.batch, 3), wl.feats, L.W, None)
    _assert_close(o288.float().cpu().numpy(), ref, f"wide walk {n_tiles} tiles")
    km256.free()
    km288.free()


@gpu
def test_c3_map_takes_wider_tiles(dev):
    # 128^3 at 10 %: under one 32-entry group per off-centre position and
    # 256-row tile, and tiles of up to 288 rows fill three rounds of 256 CUs
    # where 820 tiles of 256 rows need four: the builder takes the fewest
    # rows that do, ceil(209715 / 768) = 274; the outputs equal those of
    # 256-row tiles bit for bit
    sc = _sc()
    wl = workloads.make("c3_128_128")
    L = wl.layers[0]
    coords = _to(dev, wl.coords)
    km = sc.build_map(coords, wl.grid, wl.batch)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    _say(f"[c3 tiles] CUs={cus} tile_rows={km.tile_rows}")
    if cus == 256:
        assert km.tile_rows == 274
    k256 = sc.build_map(coords, wl.grid, wl.batch, tile_rows=256)
    feats, W = _to(dev, wl.feats), _to(dev, L.W)
    assert torch.equal(sc.forward(km, feats, W), sc.forward(k256, feats, W))
    k256.free()
    # and a dense map keeps 256-row tiles
    wd = workloads.random_small(17, G=14, occ=0.95, cin=8, cout=8, batch=2, ksize=3)
    kd = sc.build_map(_to(dev, wd.coords), wd.grid, wd.batch)
    assert kd.tile_rows == 256
    km.free()
    kd.free()


@gpu
def test_two_streams_share_a_map(dev):
    # one immutable map serves forwards on two side streams at once; each
    # stream's outputs equal the same forward run alone
    sc = _sc()
    wl = workloads.uniform_workload(48, 11000, [(3, 64, 64)], seed=1201, bias_kind="normal", name="st")
    L = wl.layers[0]
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    rng = np.random.default_rng(1202)
    fa = _to(dev, rng.standard_normal((wl.n, 64)).astype(np.float16))
    fb = _to(dev, rng.standard_normal((wl.n, 64)).astype(np.float16))
    W, b = _to(dev, L.W), _to(dev, L.bias)
    wp = sc.prepare_weights(W)
    ra = sc.forward(km, fa, prepared=wp, bias=b)
    rb = sc.forward(km, fb, prepared=wp, bias=b)
    oa = torch.empty_like(ra)
    ob = torch.empty_like(rb)
    s1, s2 = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    s1.wait_stream(torch.cuda.current_stream(dev))
    s2.wait_stream(torch.cuda.current_stream(dev))
    for _ in range(4):
        with torch.cuda.stream(s1):
            sc.forward(km, fa, prepared=wp, bias=b, out=oa)
        with torch.cuda.stream(s2):
            sc.forward(km, fb, prepared=wp, bias=b, out=ob)
    torch.cuda.current_stream(dev).wait_stream(s1)
    torch.cuda.current_stream(dev).wait_stream(s2)
    torch.cuda.synchronize(dev)
    assert torch.equal(oa, ra) and torch.equal(ob, rb)
    km.free()


@gpu
def test_forward_in_a_captured_graph(dev):
    # the forward (prepared weights, caller's output) launches kernels only:
    # it can be captured in a HIP graph; every replay, with new features
    # copied in eagerly between replays, equals the eager forward
    sc = _sc()
    wl = workloads.uniform_workload(48, 11000, [(3, 128, 128)], seed=1203, bias_kind=None, name="gr")
    L = wl.layers[0]
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    feats = _to(dev, wl.feats).clone()
    wp = sc.prepare_weights(_to(dev, L.W))
    out = torch.empty((wl.n, 128), dtype=torch.float16, device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for _ in range(2):
            sc.forward(km, feats, prepared=wp, out=out)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sc.forward(km, feats, prepared=wp, out=out)
    rng = np.random.default_rng(1204)
    for rep in range(3):
        feats.copy_(_to(dev, rng.standard_normal((wl.n, 128)).astype(np.float16)))
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        ref = sc.forward(km, feats, prepared=wp)
        torch.cuda.synchronize(dev)
        assert torch.equal(out, ref), f"replay {rep}"
    km.free()


# ----------------------------------------------------------------------------
# the MFMA kernel's 32-bit buffer offsets: largest features below 2 GiB, and
# an explicit error above (no silent change of kernel)
# ----------------------------------------------------------------------------


@gpu
@pytest.mark.slow
def test_features_at_the_2gib_limit(dev):
    """256 input channels on 4,194,303 rows: features of 2 GiB - 512 bytes,
    the largest the MFMA gather-GEMM addresses (row offsets up to bit 30),
    checked on sampled rows against the oracle on the oracle's own map. One
    row more reaches 2 GiB: the forward, the input gradient and the weight
    gradient return SUBMCONV_ERR_UNSUPPORTED_SHAPE before launching anything
    (tiny placeholder buffers, since nothing is read)."""
    sc = _sc()
    lib = sc.load_library()
    G, cin, cout = 256, 256, 128
    n_ok = (2 ** 31 - 64) // (cin * 2)
    assert n_ok * cin * 2 <= 2 ** 31 - 64 < (n_ok + 1) * cin * 2
    rng = np.random.default_rng(2024)
    lin = np.sort(rng.choice(G ** 3, n_ok + 1, replace=False))
    xyz = np.stack([lin // (G * G), (lin // G) % G, lin % G], axis=1).astype(np.int32)
    coords = np.ascontiguousarray(np.concatenate([np.zeros((n_ok + 1, 1), np.int32), xyz], axis=1))
    _say(f"[2 GiB] N={n_ok} Cin={cin}: {n_ok * cin * 2} feature bytes")
    # above: one more row
    km_big = sc.build_map(_to(dev, coords), (G, G, G), 1)
    with pytest.raises(sc.SubmconvError) as e:
        sc.forward_kernel(km_big.num_rows, km_big.active_pairs(3), cin, cout, 3)
    assert e.value.status == -4
    tiny = torch.zeros(64, dtype=torch.float16, device=dev)
    tw = torch.zeros(27 * cin * cout, dtype=torch.float16, device=dev)
    st = sc._stream(dev)
    assert lib.submconv_forward(km_big.handle, sc._ptr(tiny), sc._ptr(tw), None, sc._ptr(tiny),
                                cin, cout, 3, st) == -4
    assert lib.submconv_backward_input(km_big.handle, sc._ptr(tiny), sc._ptr(tw), sc._ptr(tiny),
                                       cout, cin, 3, st) == -4
    assert lib.submconv_backward_weight(km_big.handle, sc._ptr(tiny), sc._ptr(tiny), sc._ptr(tw),
                                        sc._ptr(tiny), cin, cout, 3, st) == -4
    torch.cuda.synchronize(dev)
    km_big.free()
    # just below: the largest features the kernel takes
    coords = np.ascontiguousarray(coords[:n_ok])
    km = sc.build_map(_to(dev, coords), (G, G, G), 1)
    g = torch.Generator(device=dev)
    g.manual_seed(2025)
    feats = torch.randn((n_ok, cin), generator=g, device=dev, dtype=torch.float32).to(torch.float16)
    W = (rng.standard_normal((27, cin, cout)) / np.sqrt(27 * cin)).astype(np.float16)
    out = sc.forward(km, feats, _to(dev, W))
    kmap = oc.kernel_map(coords, (G, G, G), 1, 3)
    rows = np.concatenate([rng.choice(n_ok, 1500, replace=False), [0, n_ok - 1]])
    # the oracle on the sampled rows and their neighbours only: a compact map
    sub = kmap[rows]
    need = np.unique(sub[sub >= 0])
    f_sub = feats[torch.from_numpy(need.astype(np.int64)).to(dev)].cpu().numpy()
    sub_c = np.where(sub >= 0, np.searchsorted(need, np.maximum(sub, 0)), -1).astype(np.int32)
    ref = oc.submconv_rows(sub_c, f_sub, W, None)
    got = out[torch.from_numpy(rows).to(dev)].float().cpu().numpy()
    _assert_close(got, ref, "2 GiB features, sampled rows")
    np.testing.assert_array_equal(km.export()[torch.from_numpy(rows).to(dev)].cpu().numpy(), sub)
    km.free()


@gpu
def test_two_streams_raw_weights(dev):
    """Forwards on weights as the caller holds them on two side streams at
    once, each with its own W: every output equals the same forward run
    alone (each stream stages W in its own buffer, or, once three streams
    own one, in the shared buffer ordered by an event)."""
    sc = _sc()
    wl = workloads.uniform_workload(48, 11000, [(3, 64, 64)], seed=1211, bias_kind="normal", name="rw")
    L = wl.layers[0]
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    rng = np.random.default_rng(1212)
    fa = _to(dev, rng.standard_normal((wl.n, 64)).astype(np.float16))
    fb = _to(dev, rng.standard_normal((wl.n, 64)).astype(np.float16))
    Wa = _to(dev, L.W)
    Wb = _to(dev, (rng.standard_normal(L.W.shape) / 40).astype(np.float16))
    b = _to(dev, L.bias)
    ra = sc.forward(km, fa, Wa, b)
    rb = sc.forward(km, fb, Wb, b)
    torch.cuda.synchronize(dev)
    oa = torch.empty_like(ra)
    ob = torch.empty_like(rb)
    s1, s2 = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    s1.wait_stream(torch.cuda.current_stream(dev))
    s2.wait_stream(torch.cuda.current_stream(dev))
    for _ in range(6):
        with torch.cuda.stream(s1):
            sc.forward(km, fa, Wa, b, out=oa)
        with torch.cuda.stream(s2):
            sc.forward(km, fb, Wb, b, out=ob)
    torch.cuda.current_stream(dev).wait_stream(s1)
    torch.cuda.current_stream(dev).wait_stream(s2)
    torch.cuda.synchronize(dev)
    assert torch.equal(oa, ra) and torch.equal(ob, rb)
    ref = oc.submconv_rows(oc.kernel_map(wl.coords, wl.grid, wl.batch, 3), fb.cpu().numpy(),
                           Wb.cpu().numpy(), L.bias)
    _assert_close(ob.float().cpu().numpy(), ref, "stream b")
    km.free()


@gpu
def test_many_streams_raw_weights(dev):
    """Six side streams forwarding on their own W at once: at most three
    streams of a device own a staging buffer, so at least three of these
    share the fourth, ordered by its event. Every output equals the same
    forward run alone, and one matches the oracle."""
    sc = _sc()
    wl = workloads.uniform_workload(40, 7000, [(3, 128, 128)], seed=1215, bias_kind="normal", name="ms")
    L = wl.layers[0]
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    rng = np.random.default_rng(1216)
    b = _to(dev, L.bias)
    fs, ws, refs = [], [], []
    for i in range(6):
        fs.append(_to(dev, rng.standard_normal((wl.n, 128)).astype(np.float16)))
        ws.append(_to(dev, (rng.standard_normal(L.W.shape) / 60).astype(np.float16)))
        refs.append(sc.forward(km, fs[i], ws[i], b))
    torch.cuda.synchronize(dev)
    outs = [torch.empty_like(r) for r in refs]
    streams = [torch.cuda.Stream(device=dev) for _ in range(6)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream(dev))
    for _ in range(4):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                sc.forward(km, fs[i], ws[i], b, out=outs[i])
    for s in streams:
        torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize(dev)
    for i in range(6):
        assert torch.equal(outs[i], refs[i]), f"stream {i}"
    ref = oc.submconv_rows(oc.kernel_map(wl.coords, wl.grid, wl.batch, 3), fs[5].cpu().numpy(),
                           ws[5].cpu().numpy(), L.bias)
    _assert_close(outs[5].float().cpu().numpy(), ref, "stream 5")
    km.free()


@gpu
def test_many_streams_forward_and_input_grad(dev):
    """Five side streams, each alternating a forward and an input gradient
    on its own W (the input gradient stages the flipped, transposed W in the
    same buffers), fp16 and bf16 mixed: every output equals the same call
    run alone."""
    sc = _sc()
    wl = workloads.uniform_workload(36, 5000, [(3, 64, 64)], seed=1217, bias_kind=None, name="mi")
    L = wl.layers[0]
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    rng = np.random.default_rng(1218)
    args, refs = [], []
    for i in range(5):
        dt = torch.bfloat16 if i % 2 else torch.float16
        f = _to(dev, rng.standard_normal((wl.n, 64)).astype(np.float16)).to(dt)
        g = _to(dev, rng.standard_normal((wl.n, 64)).astype(np.float16)).to(dt)
        W = _to(dev, (rng.standard_normal(L.W.shape) / 40).astype(np.float16)).to(dt)
        args.append((f, g, W))
        refs.append((sc.forward(km, f, W), sc.backward_input(km, g, W)))
    torch.cuda.synchronize(dev)
    outs = [(torch.empty_like(a), torch.empty_like(b)) for a, b in refs]
    streams = [torch.cuda.Stream(device=dev) for _ in range(5)]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream(dev))
    for _ in range(3):
        for i, st in enumerate(streams):
            f, g, W = args[i]
            with torch.cuda.stream(st):
                sc.forward(km, f, W, out=outs[i][0])
                sc.backward_input(km, g, W, out=outs[i][1])
    for st in streams:
        torch.cuda.current_stream(dev).wait_stream(st)
    torch.cuda.synchronize(dev)
    for i in range(5):
        assert torch.equal(outs[i][0], refs[i][0]), f"forward, stream {i}"
        assert torch.equal(outs[i][1], refs[i][1]), f"input gradient, stream {i}"
    km.free()


@gpu
def test_raw_weights_forward_in_a_captured_graph(dev):
    """submconv_forward on W inside a captured graph (the weight
    rearrangement and the gather-GEMM are both captured): every replay, with
    new features and new weights copied in eagerly between replays, equals
    the eager forward."""
    sc = _sc()
    wl = workloads.uniform_workload(48, 11000, [(3, 128, 128)], seed=1213, bias_kind=None, name="gw")
    L = wl.layers[0]
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    feats = _to(dev, wl.feats).clone()
    W = _to(dev, L.W).clone()
    out = torch.empty((wl.n, 128), dtype=torch.float16, device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for _ in range(2):
            sc.forward(km, feats, W, out=out)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sc.forward(km, feats, W, out=out)
    rng = np.random.default_rng(1214)
    for rep in range(3):
        feats.copy_(_to(dev, rng.standard_normal((wl.n, 128)).astype(np.float16)))
        W.copy_(_to(dev, (rng.standard_normal(L.W.shape) / 60).astype(np.float16)))
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        ref = sc.forward(km, feats, W)
        torch.cuda.synchronize(dev)
        assert torch.equal(out, ref), f"replay {rep}"
    km.free()


@gpu
def test_release_scratch_then_build(dev):
    """The kept build scratch can be released between builds; the next build
    allocates it again and gives the oracle's map."""
    sc = _sc()
    wl = workloads.random_small(91, G=20, occ=0.2, cin=32, cout=32, batch=2)
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    sc.release_scratch(dev)
    sc.release_scratch(dev)  # nothing kept: a no-op
    km2 = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    ref = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    np.testing.assert_array_equal(km.export().cpu().numpy(), ref)
    np.testing.assert_array_equal(km2.export().cpu().numpy(), ref)
    km.free()
    km2.free()
