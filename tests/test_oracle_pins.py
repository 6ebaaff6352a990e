"""Pins of the CPU oracle against facts that do not come from the oracle itself.

* hand-derived cases (tests/golden/hand_cases.json, derivations inside);
* the textbook special case: on a tiny dense grid, submanifold convolution at
  the active sites equals a dense 3D cross-correlation with zero padding
  (``torch.nn.functional.conv3d``) of the zero-filled grid;
* the 1x1x1 kernel is a plain matrix product;
* invariants of the kernel map (centre tap, symmetry, pair count by brute
  force over all site pairs) and of the convolution (linearity, permutation
  covariance, translation invariance, batch independence);
* mutation checks: an oracle with a planted mistake (flipped offset sign,
  transposed weights, dropped tap) fails these pins.
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import cpu as C
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _golden_weights(case):
    K = 27 if case["ksize"] == 3 else 1
    if "W_explicit" in case:
        return np.array(case["W_explicit"], dtype=np.float16)
    cout = len(case["expected_out"][0])
    W = np.zeros((K, 1, cout), dtype=np.float16)
    for k in range(K):
        W[k, 0, 0] = k + 1
        if cout == 2:
            W[k, 0, 1] = 100 if k == 13 else 0
    return W


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("impl", ["python", "c"])
def test_golden_hand_cases(case, impl):
    coords = np.array(case["coords"], dtype=np.int32)
    feats = np.array(case["feats"], dtype=np.float16)
    W = _golden_weights(case)
    bias = None if case["bias"] is None else np.array(case["bias"], dtype=np.float32)
    K = W.shape[0]
    if impl == "python":
        km = O.kernel_map(coords, case["grid"], case["ksize"], case["batch"])
        out = O.submconv(coords, feats, W, bias, case["grid"], case["ksize"], case["batch"], kmap=km)
    else:
        km = C.kernel_map(coords, case["grid"], case["batch"], case["ksize"])
        out = C.submconv_rows(km, feats, W, bias)
    expected_km = np.full((len(coords), K), -1, dtype=np.int32)
    for i, hits in case["expected_kmap_hits"].items():
        for k, j in hits.items():
            expected_km[int(i), int(k)] = j
    np.testing.assert_array_equal(km, expected_km)
    np.testing.assert_array_equal(out, np.array(case["expected_out"], dtype=np.float64))


def test_single_voxel_row():
    coords = np.array([[0, 5, 6, 7]], dtype=np.int32)
    km = O.kernel_map(coords, (10, 10, 10))
    assert km.tolist() == [[-1] * 13 + [0] + [-1] * 13]
    rng = np.random.default_rng(0)
    F = rng.standard_normal((1, 5)).astype(np.float16)
    W = rng.standard_normal((27, 5, 3)).astype(np.float16)
    b = rng.standard_normal(3).astype(np.float32)
    out = O.submconv(coords, F, W, b, (10, 10, 10))
    # centre tap alone: F W[13] + b, each entry a 5-term sum
    exp = np.array([[sum(float(F[0, c]) * float(W[13, c, o]) for c in range(5)) + float(b[o])
                     for o in range(3)]])
    np.testing.assert_allclose(out, exp, rtol=0, atol=1e-12)


# taps for the six unit offsets, from k = 9(dx+1) + 3(dy+1) + (dz+1)
UNIT_TAPS = {0: (22, 4), 1: (16, 10), 2: (14, 12)}


@pytest.mark.parametrize("axis", [0, 1, 2])
@pytest.mark.parametrize("impl", ["python", "c"])
def test_two_voxels_axis_and_sign(axis, impl):
    A = [0, 2, 2, 2]
    B = list(A)
    B[1 + axis] += 1
    coords = np.array([A, B], dtype=np.int32)
    kp, km_ = UNIT_TAPS[axis]
    if impl == "python":
        kmap = O.kernel_map(coords, (5, 5, 5))
    else:
        kmap = C.kernel_map(coords, (5, 5, 5), 1)
    exp = np.full((2, 27), -1, dtype=np.int32)
    exp[0, 13], exp[1, 13] = 0, 1
    exp[0, kp] = 1   # A's neighbour at +e_axis is B
    exp[1, km_] = 0  # B's neighbour at -e_axis is A
    np.testing.assert_array_equal(kmap, exp)
    # sign: only the +e tap carries weight 1. Cross-correlation reads
    # feats[c + d]: O[A] = F[B] = 2, O[B] = 0 (convolution would give 0 and 1).
    F = np.array([[1.0], [2.0]], dtype=np.float16)
    W = np.zeros((27, 1, 1), dtype=np.float16)
    W[kp, 0, 0] = 1.0
    if impl == "python":
        out = O.submconv(coords, F, W, None, (5, 5, 5), kmap=kmap)
    else:
        out = C.submconv_rows(kmap, F, W, None)
    np.testing.assert_array_equal(out, [[2.0], [0.0]])


def test_one_by_one_is_linear():
    rng = np.random.default_rng(11)
    wl = workloads.random_small(11, G=6, occ=0.5, cin=7, cout=5, ksize=1)
    L = wl.layers[0]
    out = O.submconv(wl.coords, wl.feats, L.W, L.bias, wl.grid, ksize=1)
    exp = wl.feats.astype(np.float64) @ L.W[0].astype(np.float64) + L.bias.astype(np.float64)
    np.testing.assert_allclose(out, exp, rtol=1e-12, atol=1e-12)
    del rng


def _dense_conv3d(coords, feats, W, bias, grid, batch):
    """Zero-filled dense grid, torch conv3d (cross-correlation, padding 1), read at sites."""
    cin, cout = W.shape[1], W.shape[2]
    dense = torch.zeros((batch, cin) + tuple(grid), dtype=torch.float64)
    c = torch.as_tensor(coords.astype(np.int64))
    dense[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]] = torch.as_tensor(feats.astype(np.float64))
    Wd = torch.as_tensor(W.astype(np.float64)).reshape(3, 3, 3, cin, cout).permute(4, 3, 0, 1, 2).contiguous()
    y = torch.nn.functional.conv3d(dense, Wd, padding=1)
    out = y[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]].numpy()
    if bias is not None:
        out = out + bias.astype(np.float64)[None, :]
    return out


DENSE_CASES = [(5, 1.0 / 125, 1), (8, 0.05, 1), (8, 0.3, 2), (12, 0.3, 1), (6, 1.0, 1), (7, 1.0, 2)]


@pytest.mark.parametrize("G,occ,batch", DENSE_CASES)
def test_matches_dense_conv3d_on_tiny_grids(G, occ, batch):
    wl = workloads.random_small(100 + G, G=G, occ=occ, cin=3, cout=4, batch=batch)
    L = wl.layers[0]
    out = O.submconv(wl.coords, wl.feats, L.W, L.bias, wl.grid, batch=batch)
    ref = _dense_conv3d(wl.coords, wl.feats, L.W, L.bias, wl.grid, batch)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-10)


def _brute_adjacent_pairs(coords):
    """Unordered pairs of distinct sites in the same batch item at Chebyshev distance 1."""
    c = coords.astype(np.int64)
    cnt = 0
    for i in range(len(c)):
        for j in range(i + 1, len(c)):
            if c[i, 0] == c[j, 0] and np.max(np.abs(c[i, 1:] - c[j, 1:])) == 1:
                cnt += 1
    return cnt


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_map_invariants(seed):
    wl = workloads.random_small(200 + seed, G=7, occ=0.25, batch=2)
    km = O.kernel_map(wl.coords, wl.grid, batch=2)
    n = wl.n
    np.testing.assert_array_equal(km[:, 13], np.arange(n))
    for i in range(n):
        for k in range(27):
            j = km[i, k]
            if j >= 0:
                assert km[j, 26 - k] == i
                d = wl.coords[j, 1:] - wl.coords[i, 1:]
                assert tuple(int(v) for v in d) == O.OFFSETS_3[k]
                assert wl.coords[j, 0] == wl.coords[i, 0]
    assert O.active_pairs(km) == n + 2 * _brute_adjacent_pairs(wl.coords)


def test_conv_invariants():
    wl = workloads.random_small(300, G=6, occ=0.4, cin=3, cout=2, batch=1)
    L = wl.layers[0]
    grid = wl.grid
    base = O.submconv(wl.coords, wl.feats, L.W, None, grid)
    # linearity in the features (values exactly representable in fp16)
    F2 = (wl.feats.astype(np.float32) * 2).astype(np.float16)
    np.testing.assert_allclose(O.submconv(wl.coords, F2, L.W, None, grid), 2 * base, rtol=1e-12, atol=1e-12)
    # permutation covariance
    perm = np.random.default_rng(1).permutation(wl.n)
    outp = O.submconv(wl.coords[perm], wl.feats[perm], L.W, None, grid)
    np.testing.assert_allclose(outp, base[perm], rtol=1e-12, atol=1e-12)
    # translation invariance inside a larger grid
    shifted = wl.coords.copy()
    shifted[:, 1:] += np.array([3, 1, 2], dtype=np.int32)
    outs = O.submconv(shifted, wl.feats, L.W, None, (10, 10, 10))
    np.testing.assert_allclose(outs, base, rtol=1e-12, atol=1e-12)
    # batch independence: the same set twice, as two batch items
    two = np.concatenate([wl.coords, wl.coords], axis=0)
    two[wl.n:, 0] = 1
    out2 = O.submconv(two, np.concatenate([wl.feats, wl.feats]), L.W, None, grid, batch=2)
    np.testing.assert_array_equal(out2[:wl.n], out2[wl.n:])
    np.testing.assert_allclose(out2[:wl.n], base, rtol=1e-12, atol=1e-12)


def test_corners_have_no_outside_neighbours():
    G = 4
    corners = [(x, y, z) for x in (0, G - 1) for y in (0, G - 1) for z in (0, G - 1)]
    coords = np.array([[0, *c] for c in corners], dtype=np.int32)
    full = np.array([[0, x, y, z] for x in range(G) for y in range(G) for z in range(G)], dtype=np.int32)
    km = O.kernel_map(full, (G, G, G))
    idx = {tuple(r[1:]): i for i, r in enumerate(full)}
    for c in corners:
        i = idx[c]
        hits = int(np.count_nonzero(km[i] >= 0))
        assert hits == 8  # a corner of a full grid has 2x2x2 sites around it, itself included
    km_c = O.kernel_map(coords, (G, G, G))
    assert int(np.count_nonzero(km_c >= 0)) == len(corners)  # corners of a 4^3 grid are not adjacent


def test_errors():
    with pytest.raises(O.OracleInputError):
        O.kernel_map(np.array([[0, 1, 1, 1], [0, 1, 1, 1]], dtype=np.int32), (4, 4, 4))
    with pytest.raises(O.OracleInputError):
        O.kernel_map(np.array([[0, 4, 1, 1]], dtype=np.int32), (4, 4, 4))
    with pytest.raises(O.OracleInputError):
        O.kernel_map(np.array([[2, 1, 1, 1]], dtype=np.int32), (4, 4, 4), batch=2)
    with pytest.raises(C.OracleCError):
        C.kernel_map(np.array([[0, 1, 1, 1], [0, 1, 1, 1]], dtype=np.int32), (4, 4, 4), 1)
    with pytest.raises(C.OracleCError):
        C.kernel_map(np.array([[0, -1, 1, 1]], dtype=np.int32), (4, 4, 4), 1)


@pytest.mark.parametrize("seed", list(range(20)))
def test_c_twin_matches_python_oracle_small(seed):
    rng = np.random.default_rng(seed)
    G = int(rng.integers(3, 9))
    batch = int(rng.integers(1, 3))
    ksize = 3 if seed % 5 else 1
    wl = workloads.random_small(500 + seed, G=G, occ=float(rng.uniform(0.05, 1.0)),
                                cin=int(rng.integers(1, 9)), cout=int(rng.integers(1, 9)),
                                batch=batch, ksize=ksize, bias=bool(seed % 2))
    L = wl.layers[0]
    kp = O.kernel_map(wl.coords, wl.grid, ksize, batch)
    kc = C.kernel_map(wl.coords, wl.grid, batch, ksize)
    np.testing.assert_array_equal(kp, kc)
    op = O.submconv(wl.coords, wl.feats, L.W, L.bias, wl.grid, ksize, batch, kmap=kp)
    oc = C.submconv_rows(kc, wl.feats, L.W, L.bias)
    np.testing.assert_allclose(oc, op, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("name", ["c1_16_8", "c2_64_64"])
def test_c_twin_matches_python_oracle_configs(name):
    wl = workloads.make(name)
    kp = O.kernel_map(wl.coords, wl.grid, 3, wl.batch)
    kc = C.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    np.testing.assert_array_equal(kp, kc)
    for L in wl.layers:
        if L.ksize == 3:
            km_p, km_c = kp, kc
        else:
            km_p = O.kernel_map(wl.coords, wl.grid, 1, wl.batch)
            km_c = C.kernel_map(wl.coords, wl.grid, wl.batch, 1)
        rows = np.arange(0, wl.n, max(1, wl.n // 500))
        op = O.submconv_rows(km_p, wl.feats, L.W, L.bias, rows)
        oc = C.submconv_rows(km_c, wl.feats, L.W, L.bias, rows)
        np.testing.assert_allclose(oc, op, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# planted mistakes: the pins above must reject a wrong oracle
# ----------------------------------------------------------------------------


def _dense_pin_passes(oracle_fn):
    wl = workloads.random_small(42, G=6, occ=0.4, cin=3, cout=4)
    L = wl.layers[0]
    out = oracle_fn(wl, L)
    ref = _dense_conv3d(wl.coords, wl.feats, L.W, L.bias, wl.grid, 1)
    return np.allclose(out, ref, rtol=1e-10, atol=1e-10)


def test_mutation_flipped_offsets_fail_dense_pin(monkeypatch):
    assert _dense_pin_passes(lambda wl, L: O.submconv(wl.coords, wl.feats, L.W, L.bias, wl.grid))
    flipped = tuple((-dx, -dy, -dz) for (dx, dy, dz) in O.OFFSETS_3)
    monkeypatch.setattr(O, "OFFSETS_3", flipped)
    assert not _dense_pin_passes(lambda wl, L: O.submconv(wl.coords, wl.feats, L.W, L.bias, wl.grid))


def test_mutation_transposed_weights_fail_dense_pin():
    def wrong(wl, L):
        Wt = np.ascontiguousarray(L.W[:, :3, :3].transpose(0, 2, 1))
        W = L.W.copy()
        W[:, :3, :3] = Wt
        return O.submconv(wl.coords, wl.feats, W, L.bias, wl.grid)
    assert not _dense_pin_passes(wrong)


def test_mutation_dropped_tap_fails_dense_pin():
    def wrong(wl, L):
        km = O.kernel_map(wl.coords, wl.grid)
        km[:, 5] = -1
        return O.submconv(wl.coords, wl.feats, L.W, L.bias, wl.grid, kmap=km)
    assert not _dense_pin_passes(wrong)


def test_bf16_decoding_pins():
    # bfloat16 patterns with known values (the top half of the binary32 pattern)
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x4049, 0x7F7F, 0x0001], dtype=np.uint16)
    exp = [1.0, -2.0, 1.0078125, 0.0, -0.0, 3.140625, 3.3895313892515355e38, 9.183549615799121e-41]
    np.testing.assert_array_equal(O.bf16_bits_to_float64(bits), np.array(exp))
    # the generator's rounding: nearest, ties to even, against exact values
    x = np.array([1.0, 1.00390625, 1.01171875, -3.0, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    r = O.bf16_bits_to_float64(workloads.f32_to_bf16_bits(x))
    np.testing.assert_array_equal(r, [1.0, 1.0, 1.015625, -3.0, 1.0078125])
