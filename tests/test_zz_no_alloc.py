"""submconv_backward_weight_noalloc against submconv_backward_weight (the
entry point with a caller's workspace) and the oracle, through the C ABI.

Two calls in a row, the second on a smaller input, share the library's fixed
per-device workspace; a 256 -> 256 layer on a map whose usual work split
needs more partials than that workspace holds takes the longer-run split.
Tolerance: the weight gradient's bound from the parity tests (per element
1e-3 + 1e-5 |ref| + 4 u S, S the sum of the absolute terms, u = 2^-24).
The device's free memory is the same before and after the calls: the entry
point allocates nothing.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import cpu as oc

gpu = pytest.mark.gpu
U = 2.0 ** -24


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


def _close(got, ref, scale, what):
    tol = 1e-3 + 1e-5 * np.abs(ref) + 4 * U * scale
    bad = np.abs(np.asarray(got, np.float64) - ref) > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} elements outside tolerance"


def _case(sc, dev, wl, seed):
    L = wl.layers[0]
    km = sc.build_map(_to(dev, wl.coords), wl.grid, wl.batch)
    g = np.random.default_rng(seed).standard_normal((wl.n, L.cout)).astype(np.float16)
    return km, L, _to(dev, wl.feats), _to(dev, g), g


def _noalloc(sc, km, f, g, out, cin, cout):
    lib = sc.load_library()
    return lib.submconv_backward_weight_noalloc(km.handle, sc._ptr(f), sc._ptr(g), sc._ptr(out),
                                                cin, cout, 3, sc._stream(f.device))


@gpu
def test_noalloc_two_calls_second_smaller(dev):
    sc = _sc()
    big = workloads.make("c3_128_128")
    small = workloads.make("c2_64_64")
    cases = [_case(sc, dev, big, 90), _case(sc, dev, small, 91)]
    outs = [torch.empty((27, L.cin, L.cout), dtype=torch.float32, device=dev) for _, L, _, _, _ in cases]
    # a first call loads the kernels and looks up the workspace's address
    km, L, f, gd, _ = cases[1]
    assert _noalloc(sc, km, f, gd, outs[1], L.cin, L.cout) == 0
    torch.cuda.synchronize(dev)
    free0 = torch.cuda.mem_get_info(dev)[0]
    for (km, L, f, gd, _), out in zip(cases, outs):
        print(f"[noalloc] {L.cin}->{L.cout} N={km.num_rows}", flush=True)
        assert _noalloc(sc, km, f, gd, out, L.cin, L.cout) == 0
    torch.cuda.synchronize(dev)
    assert torch.cuda.mem_get_info(dev)[0] == free0
    for (km, L, f, gd, g), out, wl in zip(cases, outs, [big, small]):
        ref_ws = sc.backward_weight(km, f, gd, 3).cpu().numpy()
        kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
        ref = oc.backward_weight(kmap, wl.feats, g)
        scale = oc.backward_weight(kmap, np.abs(wl.feats.astype(np.float64)), np.abs(g.astype(np.float64)))
        got = out.cpu().numpy()
        _close(got, ref_ws.astype(np.float64), scale, f"noalloc vs workspace entry {L.cin}->{L.cout}")
        _close(got, ref, scale, f"noalloc vs oracle {L.cin}->{L.cout}")
        km.free()


@gpu
def test_noalloc_split_that_does_not_fit(dev):
    sc = _sc()
    wl = workloads.uniform_workload(40, 19200, [(3, 256, 256)], seed=1301, bias_kind=None, name="na")
    km, L, f, gd, g = _case(sc, dev, wl, 92)
    lib = sc.load_library()
    need = int(lib.submconv_backward_weight_workspace_bytes(km.handle, 256, 256, 3))
    assert need > 32 << 20  # the allocating entry point's split needs more partials
    out = torch.empty((27, 256, 256), dtype=torch.float32, device=dev)
    assert _noalloc(sc, km, f, gd, out, 256, 256) == 0
    kmap = oc.kernel_map(wl.coords, wl.grid, wl.batch, 3)
    taps = [4, 13, 22]
    km_t = np.full_like(kmap, -1)
    km_t[:, taps] = kmap[:, taps]
    ref = oc.backward_weight(km_t, wl.feats, g)[taps]
    scale = oc.backward_weight(km_t, np.abs(wl.feats.astype(np.float64)), np.abs(g.astype(np.float64)))[taps]
    _close(out.cpu().numpy()[taps], ref, scale, "noalloc 256->256, longer runs")
    km.free()


@gpu
@pytest.mark.parametrize("cin,cout", [(32, 32), (64, 32)])
def test_noalloc_on_a_staged_map(dev, cin, cout):
    # a dense map (a fully occupied 20^3 cube) has a staged plan: at 32 -> 32
    # the staged kernel's partials fit the static workspace and the call takes
    # it, as the allocating entry point does (the same bits); at 64 -> 32 they
    # do not, and the call keeps the pair-by-pair kernel (the oracle's bound)
    sc = _sc()
    G = 20
    c = np.stack(np.meshgrid(np.arange(G), np.arange(G), np.arange(G), indexing="ij"), -1).reshape(-1, 3)
    coords = np.concatenate([np.zeros((c.shape[0], 1), np.int32), c.astype(np.int32)], 1)
    rng = np.random.default_rng(cin + cout)
    feats = rng.standard_normal((coords.shape[0], cin)).astype(np.float16)
    g = rng.standard_normal((coords.shape[0], cout)).astype(np.float16)
    km = sc.build_map(_to(dev, coords), (G, G, G), 1)
    assert km.staged()[0] > 0
    f, gd = _to(dev, feats), _to(dev, g)
    out = torch.empty((27, cin, cout), dtype=torch.float32, device=dev)
    print(f"[noalloc staged map] {cin}->{cout} N={coords.shape[0]}", flush=True)
    assert _noalloc(sc, km, f, gd, out, cin, cout) == 0
    ref_ws = sc.backward_weight(km, f, gd, 3)
    kmap = oc.kernel_map(coords, (G, G, G), 1, 3)
    ref = oc.backward_weight(kmap, feats, g)
    scale = oc.backward_weight(kmap, np.abs(feats.astype(np.float64)), np.abs(g.astype(np.float64)))
    _close(out.cpu().numpy(), ref, scale, f"noalloc on a staged map {cin}->{cout}")
    if (cin, cout) == (32, 32):
        assert torch.equal(out, ref_ws), "the same kernel and partials: the same bits"
    else:
        _close(out.cpu().numpy(), ref_ws.cpu().numpy().astype(np.float64), scale,
               "noalloc vs workspace entry on a staged map")
    km.free()
