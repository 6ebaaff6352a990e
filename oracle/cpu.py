"""ctypes wrapper of the C twin of the oracle (``liboracle_cpu.so``).

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see ``oracle.py``). The C twin follows
the same definition as ``oracle.py``; the tests pin it to the Python oracle.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_cpu.so")
_lib = None


class OracleCError(RuntimeError):
    pass


def load(build_if_missing: bool = True):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        if not build_if_missing:
            raise OracleCError(f"{_LIB_PATH} is not built")
        from .build_oracle import build
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    lib.oracle_kernel_map.argtypes = [P, ctypes.c_int64, P, ctypes.c_int32, ctypes.c_int32, P]
    lib.oracle_kernel_map.restype = ctypes.c_int
    lib.oracle_submconv_rows.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P, P, P,
                                         ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int64, P]
    lib.oracle_submconv_rows.restype = ctypes.c_int
    lib.oracle_backward_input_rows.argtypes = [P, ctypes.c_int64, P, ctypes.c_int32, ctypes.c_int32,
                                               P, P, ctypes.c_int32, ctypes.c_int32, P,
                                               ctypes.c_int64, P]
    lib.oracle_backward_input_rows.restype = ctypes.c_int
    lib.oracle_backward_weight.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P, P, ctypes.c_int32,
                                           ctypes.c_int32, P]
    lib.oracle_backward_weight.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def kernel_map(coords: np.ndarray, grid: Sequence[int], batch: int, ksize: int = 3) -> np.ndarray:
    lib = load()
    c = np.ascontiguousarray(coords, dtype=np.int32)
    g = np.ascontiguousarray(grid, dtype=np.int32)
    n = c.shape[0]
    K = 27 if ksize == 3 else 1
    kmap = np.empty((n, K), dtype=np.int32)
    rc = lib.oracle_kernel_map(_ptr(c), n, _ptr(g), int(batch), int(ksize), _ptr(kmap))
    if rc != 0:
        raise OracleCError({-2: "site outside the grid or batch", -3: "duplicate site"}.get(rc, f"error {rc}"))
    return kmap


def submconv_rows(kmap: np.ndarray, feats: np.ndarray, W: np.ndarray, bias: Optional[np.ndarray],
                  rows: Optional[np.ndarray] = None) -> np.ndarray:
    """fp64 outputs for ``rows`` (all rows if None) from fp16/fp32 inputs."""
    lib = load()
    km = np.ascontiguousarray(kmap, dtype=np.int32)
    F = np.ascontiguousarray(feats, dtype=np.float64)
    Wd = np.ascontiguousarray(W, dtype=np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64)
    n, K = km.shape
    cin, cout = Wd.shape[1], Wd.shape[2]
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = n if r is None else r.shape[0]
    out = np.empty((nrows, cout), dtype=np.float64)
    rc = lib.oracle_submconv_rows(_ptr(km), n, K, _ptr(F), _ptr(Wd), _ptr(b), cin, cout,
                                  _ptr(r), nrows, _ptr(out))
    if rc != 0:
        raise OracleCError(f"error {rc}")
    return out


def backward_input_rows(coords: np.ndarray, grid: Sequence[int], batch: int, ksize: int,
                        grad_out: np.ndarray, W: np.ndarray,
                        rows: Optional[np.ndarray] = None) -> np.ndarray:
    """fp64 input gradient for ``rows`` (all rows if None), found through the
    sites at ``coords[j] - d_k``."""
    lib = load()
    c = np.ascontiguousarray(coords, dtype=np.int32)
    g = np.ascontiguousarray(grid, dtype=np.int32)
    G = np.ascontiguousarray(grad_out, dtype=np.float64)
    Wd = np.ascontiguousarray(W, dtype=np.float64)
    n = c.shape[0]
    cin, cout = Wd.shape[1], Wd.shape[2]
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = n if r is None else r.shape[0]
    out = np.empty((nrows, cin), dtype=np.float64)
    rc = lib.oracle_backward_input_rows(_ptr(c), n, _ptr(g), int(batch), int(ksize), _ptr(G),
                                        _ptr(Wd), cin, cout, _ptr(r), nrows, _ptr(out))
    if rc != 0:
        raise OracleCError(f"error {rc}")
    return out


def backward_weight(kmap: np.ndarray, feats: np.ndarray, grad_out: np.ndarray) -> np.ndarray:
    """fp64 ``[K, Cin, Cout]`` weight gradient."""
    lib = load()
    km = np.ascontiguousarray(kmap, dtype=np.int32)
    F = np.ascontiguousarray(feats, dtype=np.float64)
    G = np.ascontiguousarray(grad_out, dtype=np.float64)
    n, K = km.shape
    out = np.empty((K, F.shape[1], G.shape[1]), dtype=np.float64)
    rc = lib.oracle_backward_weight(_ptr(km), n, K, _ptr(F), _ptr(G), F.shape[1], G.shape[1], _ptr(out))
    if rc != 0:
        raise OracleCError(f"error {rc}")
    return out


def num_threads() -> int:
    return int(load().oracle_num_threads())
