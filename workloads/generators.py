"""Seeded synthetic inputs for submanifold sparse 3D convolution.

This module only draws inputs: voxel coordinate sets, fp16 features, fp16
weights and fp32 biases. It holds none of the convolution's arithmetic (no
neighbour lookup, no kernel map, no products), so the GPU path and the CPU
oracle can both consume it without sharing any of the method.

Workloads (stand-ins for the pages' synthetic grids and for the surface-
concentrated voxel sets of the TRELLIS-lineage VAE decoders, whose real voxel
sets are not available):

* ``uniform``: ``round(occ * G^3)`` distinct voxels drawn uniformly without
  replacement from a ``G^3`` grid, emitted in raster order (x slowest, z
  fastest), batch 0. The 128^3 / 10 % case is the workload of the
  "Performance" table of the trellis_sparse_mlx README (209,715 voxels).
* ``shell``: the 2-voxel-thick boundary of a blob whose radius is a sphere
  radius perturbed by a random combination of real spherical harmonics of
  degree 1..3; per batch item its own seed.

Draw order within one configuration is fixed: coordinates, then features,
then each layer's weights and bias in layer order.
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

# ----------------------------------------------------------------------------
# coordinate sets
# ----------------------------------------------------------------------------


def uniform_coords(G: int, n: int, rng: np.random.Generator, batch_index: int = 0) -> np.ndarray:
    """``n`` distinct voxels of a ``G^3`` grid, uniform without replacement.

    Returns int32 ``[n, 4]`` rows ``(b, x, y, z)`` sorted in raster order.
    """
    if n > G ** 3:
        raise ValueError("more voxels than grid cells")
    lin = np.sort(rng.choice(G ** 3, size=n, replace=False)).astype(np.int64)
    out = np.empty((n, 4), dtype=np.int32)
    out[:, 0] = batch_index
    out[:, 1] = lin // (G * G)
    out[:, 2] = (lin // G) % G
    out[:, 3] = lin % G
    return out


# Real spherical harmonics of degree 1..3 as polynomials in the unit vector
# (x, y, z) = (sin t cos p, sin t sin p, cos t); orthonormal on the sphere,
# without the Condon-Shortley phase. Index: (l, m) -> f(x, y, z).
_PI = math.pi
_REAL_SH = {
    (1, -1): lambda x, y, z: math.sqrt(3 / (4 * _PI)) * y,
    (1, 0): lambda x, y, z: math.sqrt(3 / (4 * _PI)) * z,
    (1, 1): lambda x, y, z: math.sqrt(3 / (4 * _PI)) * x,
    (2, -2): lambda x, y, z: 0.5 * math.sqrt(15 / _PI) * x * y,
    (2, -1): lambda x, y, z: 0.5 * math.sqrt(15 / _PI) * y * z,
    (2, 0): lambda x, y, z: 0.25 * math.sqrt(5 / _PI) * (3 * z * z - 1),
    (2, 1): lambda x, y, z: 0.5 * math.sqrt(15 / _PI) * x * z,
    (2, 2): lambda x, y, z: 0.25 * math.sqrt(15 / _PI) * (x * x - y * y),
    (3, -3): lambda x, y, z: 0.25 * math.sqrt(35 / (2 * _PI)) * y * (3 * x * x - y * y),
    (3, -2): lambda x, y, z: 0.5 * math.sqrt(105 / _PI) * x * y * z,
    (3, -1): lambda x, y, z: 0.25 * math.sqrt(21 / (2 * _PI)) * y * (5 * z * z - 1),
    (3, 0): lambda x, y, z: 0.25 * math.sqrt(7 / _PI) * (5 * z ** 3 - 3 * z),
    (3, 1): lambda x, y, z: 0.25 * math.sqrt(21 / (2 * _PI)) * x * (5 * z * z - 1),
    (3, 2): lambda x, y, z: 0.25 * math.sqrt(105 / _PI) * (x * x - y * y) * z,
    (3, 3): lambda x, y, z: 0.25 * math.sqrt(35 / (2 * _PI)) * x * (x * x - 3 * y * y),
}


def real_sph_harm(l: int, m: int, theta: np.ndarray, phi: np.ndarray) -> np.ndarray:
    """Real spherical harmonic Y_lm (l <= 3) at polar angle theta, azimuth phi."""
    st = np.sin(theta)
    return _REAL_SH[(l, m)](st * np.cos(phi), st * np.sin(phi), np.cos(theta))


def _blob_radius_fn(R0: float, amp: float, rng: np.random.Generator, lmax: int = 3):
    """Radius function of the unit direction: R0 + amp * delta / max|delta|.

    ``delta`` is a sum of real spherical harmonics of degree 1..lmax with
    N(0,1) coefficients; ``max|delta|`` is taken on a 721 x 1441 polar/azimuth
    grid, so the perturbation is bounded by ``amp`` up to that sampling.
    """
    coeffs = [(l, m, float(rng.standard_normal())) for l in range(1, lmax + 1) for m in range(-l, l + 1)]

    def delta_xyz(x, y, z):
        acc = np.zeros(np.broadcast(x, y, z).shape, dtype=np.float64)
        for l, m, a in coeffs:
            acc += a * _REAL_SH[(l, m)](x, y, z)
        return acc

    th = np.linspace(0.0, math.pi, 721)
    ph = np.linspace(0.0, 2.0 * math.pi, 1441)
    TH, PH = np.meshgrid(th, ph, indexing="ij")
    st = np.sin(TH)
    dmax = float(np.abs(delta_xyz(st * np.cos(PH), st * np.sin(PH), np.cos(TH))).max())

    def radius(ux, uy, uz):
        return R0 + amp * delta_xyz(ux, uy, uz) / dmax

    return radius


def shell_coords(G: int, R0: float, amp: float, seed: int, batch_index: int = 0,
                 thickness: int = 2) -> np.ndarray:
    """Voxels of a perturbed solid sphere that lie within Chebyshev distance
    ``thickness`` of a voxel outside it (its ``thickness``-voxel boundary).

    The solid is ``S = {v : |v - c| <= R(theta, phi)}`` with ``c = (G-1)/2``
    per axis; the shell is ``S`` minus its erosion by a ``(2t+1)^3`` cube.
    Returns int32 ``[n, 4]`` rows ``(b, x, y, z)`` in raster order.
    """
    from scipy.ndimage import minimum_filter

    rng = np.random.default_rng(seed)
    radius = _blob_radius_fn(R0, amp, rng)
    ctr = (G - 1) / 2.0
    rmin, rmax = R0 - amp - 1.0, R0 + amp + 1.0
    if rmax + thickness + 1 >= ctr:
        raise ValueError("blob does not fit in the grid")
    solid = np.zeros((G, G, G), dtype=np.uint8)
    ax = np.arange(G, dtype=np.float64) - ctr
    Y, Z = np.meshgrid(ax, ax, indexing="ij")
    for xi in range(G):
        px = ax[xi]
        r2 = px * px + Y * Y + Z * Z
        if px * px > rmax * rmax:
            continue
        r = np.sqrt(r2)
        inside = r <= rmin
        band = (~inside) & (r <= rmax)
        if band.any():
            rb = r[band]
            inside_band = rb <= radius(px / rb, Y[band] / rb, Z[band] / rb)
            tmp = np.zeros_like(inside)
            tmp[band] = inside_band
            inside |= tmp
        solid[xi] = inside
    size = 2 * thickness + 1
    eroded = minimum_filter(solid, size=size, mode="constant", cval=0)
    shell = (solid == 1) & (eroded == 0)
    idx = np.argwhere(shell)  # raster (C) order
    out = np.empty((idx.shape[0], 4), dtype=np.int32)
    out[:, 0] = batch_index
    out[:, 1:] = idx.astype(np.int32)
    return out


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------


def normal_f16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) samples rounded to fp16 (``std`` is a standard deviation)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x.astype(np.float16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to bfloat16 (nearest, ties to even), returned as
    16-bit patterns (numpy has no bfloat16 type). Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def normal_bf16_bits(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) samples rounded to bfloat16, as 16-bit patterns."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


@dataclass
class Layer:
    ksize: int                     # 3 (27 taps) or 1 (1 tap)
    cin: int
    cout: int
    W: np.ndarray                  # fp16 [K, cin, cout]
    bias: Optional[np.ndarray]     # fp32 [cout] or None


@dataclass
class Workload:
    name: str
    grid: Tuple[int, int, int]
    batch: int
    coords: np.ndarray             # int32 [N, 4] (b, x, y, z)
    feats: np.ndarray              # fp16 [N, cin of the first layer]
    layers: List[Layer] = field(default_factory=list)
    seed: int = 0
    recipe: str = ""

    @property
    def n(self) -> int:
        return int(self.coords.shape[0])


def _layer(rng, ksize, cin, cout, bias_kind):
    K = 27 if ksize == 3 else 1
    W = normal_f16(rng, (K, cin, cout), std=1.0 / math.sqrt(27 * cin))
    if bias_kind == "zeros":
        b = np.zeros(cout, dtype=np.float32)
    elif bias_kind == "normal":
        b = (rng.standard_normal(cout) * 0.1).astype(np.float32)
    else:
        b = None
    return Layer(ksize, cin, cout, W, b)


def uniform_workload(G: int, n: int, channels: List[Tuple[int, int, int]], seed: int,
                     bias_kind: Optional[str], name: str = "uniform") -> Workload:
    """Uniform occupancy workload; ``channels`` lists (ksize, cin, cout) per layer."""
    rng = np.random.default_rng(seed)
    coords = uniform_coords(G, n, rng)
    feats = normal_f16(rng, (n, channels[0][1]))
    layers = [_layer(rng, k, ci, co, bias_kind) for (k, ci, co) in channels]
    return Workload(name, (G, G, G), 1, coords, feats, layers, seed,
                    f"uniform G={G} N={n} seed={seed}")


@functools.lru_cache(maxsize=8)
def _shell_cached(G, R0, amp, seed, batch_index):
    return shell_coords(G, R0, amp, seed, batch_index)


def shell_workload(G: int, R0: float, amp: float, coord_seeds: List[int],
                   channels: List[Tuple[int, int, int]], seed: int, name: str = "shell") -> Workload:
    """Shell workload with one blob per batch item (item b uses coord_seeds[b])."""
    parts = [_shell_cached(G, R0, amp, s, b) for b, s in enumerate(coord_seeds)]
    coords = np.concatenate(parts, axis=0)
    rng = np.random.default_rng(seed)
    feats = normal_f16(rng, (coords.shape[0], channels[0][1]))
    layers = [_layer(rng, k, ci, co, None) for (k, ci, co) in channels]
    return Workload(name, (G, G, G), len(coord_seeds), coords, feats, layers, seed,
                    f"shell G={G} R0={R0} amp={amp} coord_seeds={coord_seeds} seed={seed}")


# ----------------------------------------------------------------------------
# the five named configurations
# ----------------------------------------------------------------------------

CONFIG_NAMES = ("c1_16_8", "c2_64_64", "c3_128_128", "c4_256_shell", "c5_512_chain")


def make(name: str) -> Workload:
    """Build one of the named configurations (seeded, deterministic)."""
    if name == "c1_16_8":
        return uniform_workload(16, 410, [(3, 8, 8)], seed=1, bias_kind="zeros", name=name)
    if name == "c2_64_64":
        return uniform_workload(64, 26214, [(3, 64, 64), (1, 64, 64)], seed=2,
                                bias_kind="normal", name=name)
    if name == "c3_128_128":
        return uniform_workload(128, 209715, [(3, 128, 128)], seed=3, bias_kind=None, name=name)
    # the 128^3 / C=128 layer at 1 % and 30 % occupancy (the masked-GEMM
    # comparison's other occupancies)
    if name == "c3_occ1":
        return uniform_workload(128, round(0.01 * 128 ** 3), [(3, 128, 128)], seed=31, bias_kind=None,
                                name=name)
    if name == "c3_occ30":
        return uniform_workload(128, round(0.30 * 128 ** 3), [(3, 128, 128)], seed=33, bias_kind=None,
                                name=name)
    if name == "c4_256_shell":
        return shell_workload(256, 100.0, 15.0, [40, 41], [(3, 256, 256)], seed=4, name=name)
    if name == "c5_512_chain":
        return shell_workload(512, 200.0, 15.0, [5], [(3, 64, 32), (3, 32, 32), (1, 32, 32)],
                              seed=5, name=name)
    raise KeyError(name)


def random_small(seed: int, G: int = 8, occ: float = 0.3, cin: int = 4, cout: int = 3,
                 batch: int = 1, ksize: int = 3, bias: bool = True) -> Workload:
    """A tiny random case for brute-force checks (possibly several batch items)."""
    rng = np.random.default_rng(seed)
    parts = []
    for b in range(batch):
        n = max(1, int(round(occ * G ** 3)))
        parts.append(uniform_coords(G, n, rng, batch_index=b))
    coords = np.concatenate(parts, axis=0)
    feats = normal_f16(rng, (coords.shape[0], cin))
    layers = [_layer(rng, ksize, cin, cout, "normal" if bias else None)]
    return Workload(f"small{seed}", (G, G, G), batch, coords, feats, layers, seed,
                    f"small G={G} occ={occ} batch={batch} seed={seed}")
