"""Plain CPU oracle for submanifold sparse 3D convolution (SubMConv3d).

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this module. It shares no code with the
GPU library: no lookup structure, no kernel, no table and no helper.

What it computes, written from the definition:

* Submanifold convolution with stride 1 and no padding argument produces an
  output only at the input sites (trellis_sparse_mlx README, "Why this is a
  package", the stride=1 / padding=None dispatch to SubMConv3d).
* The kernel is 3x3x3 or 1x1x1 (same README, "What's in it" table, SubMConv3d
  row); a sparse tensor is coordinates ``[N,4]`` plus features ``[N,C]``
  (same table, SparseTensor row).
* Each output row accumulates, over the kernel offsets, the gathered input
  feature row times that offset's weight matrix (same README, "Performance":
  it describes the unfused form as one gather and one product per offset,
  and its fused ``[N, K^3*Cin] x [K^3*Cin, Cout]`` matmul computes the same
  sum).
* The gather reads ``feats[c + d]``, cross-correlation (same README,
  "Correctness", the unverified c+d assumption; this oracle takes c+d).
* It is a deliberately naive dict lookup with a per-voxel loop, sharing no
  indexing code with the fast path (same README, "Correctness").

Readings where the pages are silent (each listed in the design notes):

* tap index ``k = 9*(dx+1) + 3*(dy+1) + (dz+1)``, dx slowest; centre k = 13;
  for a 1x1x1 kernel the single tap is offset (0,0,0) at k = 0;
* coordinate columns are (batch, x, y, z); offsets never change the batch;
* a neighbour outside ``[0, G)`` on any axis is absent (zero padding);
* the missing-neighbour sentinel in the kernel map is -1;
* the bias, when given, is added once per output row;
* everything is accumulated in fp64 from the exactly up-cast inputs.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np

# (dx, dy, dz) for k = 0..26, dx slowest, dz fastest.
OFFSETS_3 = tuple((dx, dy, dz) for dx in (-1, 0, 1) for dy in (-1, 0, 1) for dz in (-1, 0, 1))
OFFSETS_1 = ((0, 0, 0),)
CENTER_TAP_3 = 13
SENTINEL = -1


class OracleInputError(ValueError):
    """Raised for coordinates outside the grid or batch, or duplicated sites."""


def offsets(ksize: int) -> Tuple[Tuple[int, int, int], ...]:
    if ksize == 3:
        return OFFSETS_3
    if ksize == 1:
        return OFFSETS_1
    raise OracleInputError(f"ksize must be 1 or 3, got {ksize}")


def site_index(coords: np.ndarray, grid: Sequence[int], batch: Optional[int] = None) -> Dict[tuple, int]:
    """Dictionary from the site tuple (b, x, y, z) to its row.

    Validates that every site lies in ``[0, batch) x [0, G0) x [0, G1) x [0, G2)``
    and that no site occurs twice.
    """
    coords = np.asarray(coords)
    index: Dict[tuple, int] = {}
    for i in range(coords.shape[0]):
        b, x, y, z = (int(v) for v in coords[i])
        if b < 0 or (batch is not None and b >= batch):
            raise OracleInputError(f"row {i}: batch index {b} out of range")
        if not (0 <= x < grid[0] and 0 <= y < grid[1] and 0 <= z < grid[2]):
            raise OracleInputError(f"row {i}: site {(x, y, z)} outside the grid {tuple(grid)}")
        key = (b, x, y, z)
        if key in index:
            raise OracleInputError(f"row {i}: duplicate site {key} (first at row {index[key]})")
        index[key] = i
    return index


def kernel_map(coords: np.ndarray, grid: Sequence[int], ksize: int = 3,
               batch: Optional[int] = None) -> np.ndarray:
    """``kmap[i, k]`` = row of the site ``coords[i] + d_k`` in the same batch
    item, or -1 if there is no such site (int32 ``[N, K]``)."""
    coords = np.asarray(coords)
    index = site_index(coords, grid, batch)
    offs = offsets(ksize)
    n = coords.shape[0]
    kmap = np.full((n, len(offs)), SENTINEL, dtype=np.int32)
    for i in range(n):
        b, x, y, z = (int(v) for v in coords[i])
        for k, (dx, dy, dz) in enumerate(offs):
            nx, ny, nz = x + dx, y + dy, z + dz
            if not (0 <= nx < grid[0] and 0 <= ny < grid[1] and 0 <= nz < grid[2]):
                continue
            j = index.get((b, nx, ny, nz))
            if j is not None:
                kmap[i, k] = j
    return kmap


def active_pairs(kmap: np.ndarray) -> int:
    """Number of (row, tap) pairs with a neighbour, the centre tap included."""
    return int(np.count_nonzero(np.asarray(kmap) != SENTINEL))


def submconv(coords: np.ndarray, feats: np.ndarray, W: np.ndarray, bias: Optional[np.ndarray],
             grid: Sequence[int], ksize: int = 3, batch: Optional[int] = None,
             kmap: Optional[np.ndarray] = None) -> np.ndarray:
    """fp64 output ``[N, Cout]``: ``out[i] = bias + sum_k feats[kmap[i,k]] @ W[k]``
    over the taps whose neighbour exists."""
    feats = np.asarray(feats)
    W = np.asarray(W)
    n = feats.shape[0]
    K = 27 if ksize == 3 else 1
    if W.ndim != 3 or W.shape[0] != K or W.shape[1] != feats.shape[1]:
        raise OracleInputError(f"weights of shape {W.shape} do not fit K={K}, Cin={feats.shape[1]}")
    if kmap is None:
        kmap = kernel_map(coords, grid, ksize, batch)
    F = feats.astype(np.float64)
    Wd = W.astype(np.float64)
    cout = W.shape[2]
    out = np.zeros((n, cout), dtype=np.float64)
    if bias is not None:
        out += np.asarray(bias, dtype=np.float64)[None, :]
    for i in range(n):
        for k in range(K):
            j = int(kmap[i, k])
            if j != SENTINEL:
                out[i] += F[j] @ Wd[k]
    return out


def submconv_rows(kmap: np.ndarray, feats: np.ndarray, W: np.ndarray, bias: Optional[np.ndarray],
                  rows: Sequence[int]) -> np.ndarray:
    """Same sum as :func:`submconv` for selected output rows only, given a map."""
    F = np.asarray(feats)
    Wd = np.asarray(W).astype(np.float64)
    out = np.zeros((len(rows), Wd.shape[2]), dtype=np.float64)
    if bias is not None:
        out += np.asarray(bias, dtype=np.float64)[None, :]
    for r, i in enumerate(rows):
        for k in range(Wd.shape[0]):
            j = int(kmap[i, k])
            if j != SENTINEL:
                out[r] += F[j].astype(np.float64) @ Wd[k]
    return out


# ---------------------------------------------------------------------------
# Backward of the same operation (gradients of a scalar loss L with
# dL/dout = grad_out): the adjoint of the forward sum, written as scatters.
# The issue #1 thread ("Fixed" list) names forward, input-gradient and
# weight-gradient kernels; the sums below are what the chain rule makes of
# the forward definition above.
# ---------------------------------------------------------------------------


def submconv_backward_input(coords: np.ndarray, grad_out: np.ndarray, W: np.ndarray,
                            grid: Sequence[int], ksize: int = 3, batch: Optional[int] = None,
                            kmap: Optional[np.ndarray] = None) -> np.ndarray:
    """fp64 ``[N, Cin]``: every forward term ``feats[j] @ W[k]`` added to
    ``out[i]`` (with ``j = kmap[i,k]``) sends ``grad_out[i] @ W[k]^T`` back
    to row ``j``."""
    G = np.asarray(grad_out).astype(np.float64)
    Wd = np.asarray(W).astype(np.float64)
    if kmap is None:
        kmap = kernel_map(coords, grid, ksize, batch)
    n = G.shape[0]
    dx = np.zeros((n, Wd.shape[1]), dtype=np.float64)
    for i in range(n):
        for k in range(Wd.shape[0]):
            j = int(kmap[i, k])
            if j != SENTINEL:
                dx[j] += Wd[k] @ G[i]
    return dx


def submconv_backward_weight(coords: np.ndarray, feats: np.ndarray, grad_out: np.ndarray,
                             grid: Sequence[int], ksize: int = 3, batch: Optional[int] = None,
                             kmap: Optional[np.ndarray] = None) -> np.ndarray:
    """fp64 ``[K, Cin, Cout]``: every forward term ``feats[j] @ W[k]`` in
    ``out[i]`` contributes the outer product ``feats[j]^T grad_out[i]`` to
    the gradient of ``W[k]``."""
    F = np.asarray(feats).astype(np.float64)
    G = np.asarray(grad_out).astype(np.float64)
    if kmap is None:
        kmap = kernel_map(coords, grid, ksize, batch)
    K = kmap.shape[1]
    dw = np.zeros((K, F.shape[1], G.shape[1]), dtype=np.float64)
    for i in range(G.shape[0]):
        for k in range(K):
            j = int(kmap[i, k])
            if j != SENTINEL:
                dw[k] += np.outer(F[j], G[i])
    return dw


# ---------------------------------------------------------------------------
# The coordinate operations beside SubMConv3d in the same sparse stack
# (trellis_sparse_mlx README, "What's in it" table, subdivide / downsample
# row: x2 coordinate expansion, and x2 max-pooling -- the upstream reduce is
# "amax" whatever its docstring says).
# ---------------------------------------------------------------------------

# child offsets of subdivide, c = 4*dx + 2*dy + dz (dx slowest)
SUBDIVIDE_OFFSETS = tuple((dx, dy, dz) for dx in (0, 1) for dy in (0, 1) for dz in (0, 1))


def downsample(coords: np.ndarray, feats: Optional[np.ndarray], grid: Sequence[int],
               batch: Optional[int] = None):
    """x2 max-pool of a sparse tensor.

    Every site (b, x, y, z) belongs to the parent (b, x//2, y//2, z//2). The
    parents are the distinct such tuples in ascending lexicographic order of
    (b, x, y, z) (the order a sorting unique gives); a parent's feature row is
    the channel-wise maximum over its sites. Returns (parent coords [M,4]
    int32, inverse [N] int32 = parent row of each site, parent features
    [M,C] in the input dtype or None, parent grid).
    """
    coords = np.asarray(coords)
    for i in range(coords.shape[0]):  # range only: repeated sites are allowed here
        b, x, y, z = (int(v) for v in coords[i])
        if b < 0 or (batch is not None and b >= batch):
            raise OracleInputError(f"row {i}: batch index {b} out of range")
        if not (0 <= x < grid[0] and 0 <= y < grid[1] and 0 <= z < grid[2]):
            raise OracleInputError(f"row {i}: site {(x, y, z)} outside the grid {tuple(grid)}")
    parents = {}
    for i in range(coords.shape[0]):
        b, x, y, z = (int(v) for v in coords[i])
        parents.setdefault((b, x // 2, y // 2, z // 2), []).append(i)
    keys = sorted(parents)
    pc = np.array(keys, dtype=np.int32).reshape(-1, 4)
    inv = np.empty(coords.shape[0], dtype=np.int32)
    for p, key in enumerate(keys):
        for i in parents[key]:
            inv[i] = p
    pf = None
    if feats is not None:
        feats = np.asarray(feats)
        pf = np.empty((len(keys), feats.shape[1]), dtype=feats.dtype)
        for p, key in enumerate(keys):
            rows = parents[key]
            m = feats[rows[0]].copy()
            for i in rows[1:]:
                m = np.maximum(m, feats[i])
            pf[p] = m
    pgrid = tuple((int(g) + 1) // 2 for g in grid)
    return pc, inv, pf, pgrid


def subdivide(coords: np.ndarray, feats: Optional[np.ndarray], grid: Sequence[int]):
    """x2 coordinate expansion: site i becomes the 8 sites
    (b, 2x+dx, 2y+dy, 2z+dz) at rows 8*i + c, c = 4*dx + 2*dy + dz, each with
    site i's feature row. Returns (child coords [8N,4] int32, child features
    [8N,C] or None, child grid)."""
    coords = np.asarray(coords)
    n = coords.shape[0]
    cc = np.empty((8 * n, 4), dtype=np.int32)
    for i in range(n):
        b, x, y, z = (int(v) for v in coords[i])
        for c, (dx, dy, dz) in enumerate(SUBDIVIDE_OFFSETS):
            cc[8 * i + c] = (b, 2 * x + dx, 2 * y + dy, 2 * z + dz)
    cf = None
    if feats is not None:
        feats = np.asarray(feats)
        cf = np.repeat(feats, 8, axis=0)
    return cc, cf, tuple(2 * int(g) for g in grid)


def downsample_np(coords: np.ndarray, feats: Optional[np.ndarray], grid: Sequence[int]):
    """The same result as :func:`downsample` through numpy's sorting unique
    and an unbuffered maximum scatter, for sizes the loop version cannot
    finish in seconds (pinned to it on small cases)."""
    coords = np.asarray(coords)
    half = coords.astype(np.int64).copy()
    half[:, 1:] //= 2
    pc, inv = np.unique(half, axis=0, return_inverse=True)
    inv = inv.reshape(-1)
    pf = None
    if feats is not None:
        feats = np.asarray(feats)
        pf = np.full((pc.shape[0], feats.shape[1]), -np.inf, dtype=np.float64)
        np.maximum.at(pf, inv, feats.astype(np.float64))
        pf = pf.astype(feats.dtype)
    return pc.astype(np.int32), inv.astype(np.int32), pf, tuple((int(g) + 1) // 2 for g in grid)


def bf16_bits_to_float64(bits: np.ndarray) -> np.ndarray:
    """Exact values of bfloat16 numbers given as their 16-bit patterns: a
    bfloat16 is the top half of an IEEE binary32, so the pattern shifted left
    by 16 bits is that binary32, which fp64 holds exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)
