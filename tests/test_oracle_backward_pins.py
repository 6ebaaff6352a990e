"""Pins of the backward oracle (input and weight gradients) against facts that
do not come from the oracle itself.

* the adjoint identities of a linear map: for any X, dY and a direction E of
  the weights, <dY, conv(X; W)> = <dX(dY), X> and <dY, conv(X; E)> =
  <dW(X, dY), E> (the forward oracle is pinned separately);
* torch autograd through the dense 3D cross-correlation with zero padding of
  the zero-filled grid, read back at the sites (the textbook special case);
* a single site: dX = dY @ W[13]^T and dW[13] = X^T dY, every other tap zero;
* the C twin against the Python oracle;
* mutation checks: a planted mistake (transposed weights, the c-d lookup
  mirrored, a dropped tap) fails the pins.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import cpu as C
from oracle import oracle as O


def _case(seed, G=7, occ=0.3, cin=3, cout=4, batch=1):
    wl = workloads.random_small(seed, G=G, occ=occ, cin=cin, cout=cout, batch=batch)
    rng = np.random.default_rng(seed + 1000)
    dy = rng.standard_normal((wl.n, cout))
    return wl, wl.layers[0], dy


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_adjoint_identity_input(seed):
    wl, L, dy = _case(seed)
    y = O.submconv(wl.coords, wl.feats, L.W, None, wl.grid)
    dx = O.submconv_backward_input(wl.coords, dy, L.W, wl.grid)
    lhs = float(np.sum(dy * y))
    rhs = float(np.sum(dx * wl.feats.astype(np.float64)))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


@pytest.mark.parametrize("seed", [4, 5])
def test_adjoint_identity_weight(seed):
    wl, L, dy = _case(seed)
    E = np.random.default_rng(seed + 7).standard_normal(L.W.shape)
    y = O.submconv(wl.coords, wl.feats, E, None, wl.grid)
    dw = O.submconv_backward_weight(wl.coords, wl.feats, dy, wl.grid)
    lhs = float(np.sum(dy * y))
    rhs = float(np.sum(dw * E))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def _dense_grads(coords, feats, W, dy, grid, batch):
    cin, cout = W.shape[1], W.shape[2]
    c = torch.as_tensor(coords.astype(np.int64))
    x = torch.as_tensor(feats.astype(np.float64)).requires_grad_(True)
    Wt = torch.as_tensor(W.astype(np.float64)).requires_grad_(True)
    dense = torch.zeros((batch, cin) + tuple(grid), dtype=torch.float64)
    dense[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]] = x
    Wd = Wt.reshape(3, 3, 3, cin, cout).permute(4, 3, 0, 1, 2)
    y = torch.nn.functional.conv3d(dense, Wd, padding=1)
    out = y[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]]
    out.backward(torch.as_tensor(dy))
    return x.grad.numpy(), Wt.grad.numpy()


@pytest.mark.parametrize("G,occ,batch", [(5, 0.2, 1), (6, 1.0, 1), (7, 0.3, 2)])
def test_matches_dense_autograd(G, occ, batch):
    wl, L, dy = _case(200 + G, G=G, occ=occ, batch=batch)
    dx_ref, dw_ref = _dense_grads(wl.coords, wl.feats, L.W, dy, wl.grid, batch)
    dx = O.submconv_backward_input(wl.coords, dy, L.W, wl.grid, batch=batch)
    dw = O.submconv_backward_weight(wl.coords, wl.feats, dy, wl.grid, batch=batch)
    np.testing.assert_allclose(dx, dx_ref, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dw, dw_ref, rtol=1e-10, atol=1e-10)


def test_single_site():
    coords = np.array([[0, 2, 3, 1]], dtype=np.int32)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 3))
    W = rng.standard_normal((27, 3, 2))
    dy = rng.standard_normal((1, 2))
    dx = O.submconv_backward_input(coords, dy, W, (5, 5, 5))
    dw = O.submconv_backward_weight(coords, x, dy, (5, 5, 5))
    np.testing.assert_allclose(dx, dy @ W[13].T, rtol=1e-14)
    exp = np.zeros_like(W)
    exp[13] = x.T @ dy
    np.testing.assert_allclose(dw, exp, rtol=1e-14)


@pytest.mark.parametrize("ksize", [3, 1])
@pytest.mark.parametrize("seed", [11, 12])
def test_c_twin_backward_matches_python(seed, ksize):
    wl, L, dy = _case(seed, G=8, occ=0.25, cin=5, cout=6, batch=2)
    W = L.W if ksize == 3 else L.W[13:14]
    kmap = O.kernel_map(wl.coords, wl.grid, ksize)
    dx = O.submconv_backward_input(wl.coords, dy, W, wl.grid, ksize)
    dw = O.submconv_backward_weight(wl.coords, wl.feats, dy, wl.grid, ksize)
    dx_c = C.backward_input_rows(wl.coords, wl.grid, wl.batch, ksize, dy, W)
    dw_c = C.backward_weight(kmap, wl.feats, dy)
    np.testing.assert_allclose(dx_c, dx, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw_c, dw, rtol=1e-12, atol=1e-12)
    rows = np.array([0, wl.n - 1, wl.n // 2])
    np.testing.assert_allclose(C.backward_input_rows(wl.coords, wl.grid, wl.batch, ksize, dy, W, rows),
                               dx[rows], rtol=1e-12, atol=1e-12)


def _pins_pass(bwd_input, bwd_weight):
    wl, L, dy = _case(300, G=6, occ=0.5)
    dx_ref, dw_ref = _dense_grads(wl.coords, wl.feats, L.W, dy, wl.grid, 1)
    ok_x = np.allclose(bwd_input(wl, L, dy), dx_ref, rtol=1e-8, atol=1e-8)
    ok_w = np.allclose(bwd_weight(wl, L, dy), dw_ref, rtol=1e-8, atol=1e-8)
    return ok_x and ok_w


def test_pins_accept_the_oracle():
    assert _pins_pass(lambda wl, L, dy: O.submconv_backward_input(wl.coords, dy, L.W, wl.grid),
                      lambda wl, L, dy: O.submconv_backward_weight(wl.coords, wl.feats, dy, wl.grid))


def test_mutation_untransposed_weights_fail():
    # gradient sent back through W[k] without the transpose: only defined for
    # square channels, so compare through a square case
    wl, L, dy = _case(301, G=6, occ=0.5, cin=4, cout=4)
    dx_ref, _ = _dense_grads(wl.coords, wl.feats, L.W, dy, wl.grid, 1)
    wrong = O.submconv_backward_input(wl.coords, dy, np.transpose(L.W, (0, 2, 1)), wl.grid)
    assert not np.allclose(wrong, dx_ref, rtol=1e-6, atol=1e-6)


def test_mutation_mirrored_lookup_fails():
    # the input gradient computed as a forward with W[k]^T at the same tap
    # (gathering c+d instead of scattering): the kernel flip is missing
    def wrong_x(wl, L, dy):
        Wt = np.transpose(L.W, (0, 2, 1))
        return O.submconv(wl.coords, dy, Wt, None, wl.grid)
    assert not _pins_pass(wrong_x, lambda wl, L, dy: O.submconv_backward_weight(wl.coords, wl.feats, dy, wl.grid))


def test_mutation_dropped_tap_fails():
    def wrong_w(wl, L, dy):
        dw = O.submconv_backward_weight(wl.coords, wl.feats, dy, wl.grid)
        dw[4] = 0.0
        return dw
    assert not _pins_pass(lambda wl, L, dy: O.submconv_backward_input(wl.coords, dy, L.W, wl.grid), wrong_w)
