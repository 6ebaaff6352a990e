"""Submanifold sparse 3D convolution (SubMConv3d) on AMD Instinct MI355X.

Thin Python binding of ``libsubmconv.so`` (C ABI in ``include/submconv.h``).
It only marshals arguments: tensors are passed as device pointers together
with PyTorch's current HIP stream; every step runs in the library's kernels.
The library must be built (``python -m submanifold_sparse_convolution_hash_amd.build``
or ``__graft_entry__.build()``); nothing here falls back to another
implementation when it is missing.

Operation (trellis_sparse_mlx README, "What's in it", "Performance",
"Correctness"): for sites ``coords[N,4] = (b,x,y,z)`` and features
``feats[N,Cin]``, ``out[i] = bias + sum_k feats[j_k(i)] @ W[k]`` where
``j_k(i)`` is the site at ``coords[i] + d_k`` (same batch item), absent
neighbours contributing zero; ``k = 9(dx+1)+3(dy+1)+(dz+1)`` for 3x3x3 and
``k = 0`` for 1x1x1.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

__all__ = [
    "SubmconvError", "KernelMap", "build_map", "Weights", "prepare_weights", "forward",
    "forward_kernel", "backward_input",
    "backward_weight", "backward_bias", "SubMConv3dFunction", "SubMConv3d", "library_path", "load_library",
    "abi_version", "release_scratch", "FLAG_MORTON", "downsample", "subdivide", "MaskedPlan", "masked_plan",
    "forward_masked",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsubmconv.so")
FLAG_MORTON = 1
FLAG_SORTED_KEYS = 2
FLAG_TILES_256 = 4
FLAG_TILES_288 = 8
FLAG_STAGED = 16
FLAG_NO_STAGED = 32
PREP_INPUT_GRAD = 1
_lib = None


class SubmconvError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Loads ``libsubmconv.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built: run `python -m submanifold_sparse_convolution_hash_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, U32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    sig = {
        "submconv_build_map": ([P, I64, I32, P, U32, P, P], ctypes.c_int),
        "submconv_release_scratch": ([], ctypes.c_int),
        "submconv_map_num_rows": ([P], I64),
        "submconv_map_tile_rows": ([P], I32),
        "submconv_map_active_pairs": ([P, I32], I64),
        "submconv_map_staged": ([P, P], I32),
        "submconv_map_export": ([P, P, P], ctypes.c_int),
        "submconv_map_order": ([P, P, P], ctypes.c_int),
        "submconv_map_free": ([P], ctypes.c_int),
        "submconv_weights_create": ([I32, I32, I32, I32, U32, P], ctypes.c_int),
        "submconv_weights_set": ([P, P, P], ctypes.c_int),
        "submconv_weights_free": ([P], ctypes.c_int),
        "submconv_forward_prepared": ([P, P, P, P, P, P], ctypes.c_int),
        "submconv_forward_kernel": ([I64, I64, I32, I32, I32], ctypes.c_int),
        "submconv_backward_input": ([P, P, P, P, I32, I32, I32, P], ctypes.c_int),
        "submconv_backward_input_prepared": ([P, P, P, P, P], ctypes.c_int),
        "submconv_backward_weight_workspace_bytes": ([P, I32, I32, I32], I64),
        "submconv_backward_weight": ([P, P, P, P, P, I32, I32, I32, P], ctypes.c_int),
        "submconv_backward_weight_noalloc": ([P, P, P, P, I32, I32, I32, P], ctypes.c_int),
        "submconv_backward_bias": ([P, I64, I32, P, P], ctypes.c_int),
        "submconv_downsample_plan": ([P, I64, I32, P, P, P], ctypes.c_int),
        "submconv_downsample_rows": ([P], I64),
        "submconv_downsample_grid": ([P, P], ctypes.c_int),
        "submconv_downsample_coords": ([P, P, P, P], ctypes.c_int),
        "submconv_downsample_max": ([P, P, I32, P, P], ctypes.c_int),
        "submconv_downsample_free": ([P], ctypes.c_int),
        "submconv_subdivide": ([P, I64, P, I32, P, P, P], ctypes.c_int),
        "submconv_masked_plan": ([P, P, P], ctypes.c_int),
        "submconv_masked_row_taps": ([P], I64),
        "submconv_forward_masked": ([P, P, P, P, P, P], ctypes.c_int),
        "submconv_masked_free": ([P], ctypes.c_int),
        "submconv_forward": ([P, P, P, P, P, I32, I32, I32, P], ctypes.c_int),
        "submconv_forward_dtype": ([P, P, P, P, P, I32, I32, I32, I32, P], ctypes.c_int),
        "submconv_backward_input_dtype": ([P, P, P, P, I32, I32, I32, I32, P], ctypes.c_int),
        "submconv_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "submconv_last_error": ([], ctypes.c_char_p),
        "submconv_abi_version": ([], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def abi_version() -> int:
    return int(load_library().submconv_abi_version())


def release_scratch(device: Optional[torch.device] = None) -> None:
    """Frees the map-build scratch the library keeps on ``device`` (default:
    the current device) for its next build."""
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        _check(load_library().submconv_release_scratch())


def _check(status: int) -> None:
    if status != 0:
        lib = load_library()
        msg = lib.submconv_last_error().decode() or lib.submconv_status_string(status).decode()
        raise SubmconvError(int(status), msg)


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[ctypes.c_void_p]:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_DTYPES = {torch.float16: 0, torch.bfloat16: 1}


def _require(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    allowed = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in allowed:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in allowed)}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class KernelMap:
    """Handle of a built neighbour map (library-owned device memory)."""

    def __init__(self, handle: ctypes.c_void_p, device: torch.device, grid, batch: int, flags: int):
        self._h = handle
        self.device = device
        self.grid = tuple(int(g) for g in grid)
        self.batch = int(batch)
        self.flags = int(flags)
        lib = load_library()
        self.num_rows = int(lib.submconv_map_num_rows(self._h))
        self.tile_rows = int(lib.submconv_map_tile_rows(self._h))

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise SubmconvError(-1, "map already freed")
        return self._h

    def active_pairs(self, ksize: int = 3) -> int:
        v = int(load_library().submconv_map_active_pairs(self.handle, ksize))
        if v < 0:
            _check(v)
        return v

    def staged(self) -> Tuple[int, int]:
        """(units, staged rows) of the map's staged plan; (0, 0) without one."""
        v = (ctypes.c_int64 * 2)()
        _check(load_library().submconv_map_staged(self.handle, v))
        return int(v[0]), int(v[1])

    def export(self) -> torch.Tensor:
        """[N,27] int32 neighbour rows in the caller's order, -1 for none."""
        out = torch.empty((self.num_rows, 27), dtype=torch.int32, device=self.device)
        _check(load_library().submconv_map_export(self.handle, _ptr(out), _stream(self.device)))
        return out

    def order(self) -> torch.Tensor:
        """[N] int32 processing order (caller row processed t-th)."""
        out = torch.empty((self.num_rows,), dtype=torch.int32, device=self.device)
        _check(load_library().submconv_map_order(self.handle, _ptr(out), _stream(self.device)))
        return out

    def free(self) -> None:
        if self._h is not None and _lib is not None:
            _check(_lib.submconv_map_free(self._h))
        self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def build_map(coords: torch.Tensor, grid: Sequence[int], batch: Optional[int] = None,
              morton: bool = False, sorted_keys: bool = False,
              tile_rows: Optional[int] = None, staged: Optional[bool] = None) -> KernelMap:
    """Hashes the sites ``coords`` ([N,4] int32 (b,x,y,z), device) and builds
    their 3x3x3 neighbour map. Waits for the stream (validation).
    ``sorted_keys`` finds neighbours by binary search in the sorted site keys
    instead of the hash table (same map). ``tile_rows`` (256 or 288) forces
    the tile size of the lists the forward streams (default: the library's
    choice; the results are the same). ``staged`` True builds the staged plan
    of dense maps on any map, False on none (default: on dense maps)."""
    if tile_rows not in (None, 256, 288):
        raise ValueError("tile_rows must be None, 256 or 288")
    _require(coords, "coords", torch.int32, 2)
    if coords.shape[1] != 4:
        raise ValueError("coords must be [N,4]")
    if batch is None:
        batch = int(coords[:, 0].max().item()) + 1 if coords.shape[0] else 1
    lib = load_library()
    g = (ctypes.c_int32 * 3)(*[int(v) for v in grid])
    h = ctypes.c_void_p()
    flags = (FLAG_MORTON if morton else 0) | (FLAG_SORTED_KEYS if sorted_keys else 0)
    flags |= {None: 0, 256: FLAG_TILES_256, 288: FLAG_TILES_288}[tile_rows]
    flags |= {None: 0, True: FLAG_STAGED, False: FLAG_NO_STAGED}[staged]
    with torch.cuda.device(coords.device):
        _check(lib.submconv_build_map(_ptr(coords), coords.shape[0], int(batch), g, flags,
                                      _stream(coords.device), ctypes.byref(h)))
    return KernelMap(h, coords.device, grid, batch, flags)


class Weights:
    """Prepared weights of one layer (``submconv_weights_t``): the library's
    device copy of ``W`` ([K,Cin,Cout], K = 27 or 1, fp16 or bf16) in the MFMA
    kernels' order, for the forward, or with ``input_grad`` for the input
    gradient. The handle records the shape, dtype and use, and the library
    checks them at every call. ``set`` re-prepares new values of ``W``."""

    def __init__(self, W: torch.Tensor, input_grad: bool = False):
        _require(W, "W", tuple(_DTYPES), 3)
        K, cin, cout = (int(v) for v in W.shape)
        if K not in (27, 1):
            raise ValueError("W must be [27,Cin,Cout] or [1,Cin,Cout]")
        self.ksize = 3 if K == 27 else 1
        self.cin, self.cout = cin, cout
        self.dtype = W.dtype
        self.device = W.device
        self.input_grad = bool(input_grad)
        self._h = None
        h = ctypes.c_void_p()
        with torch.cuda.device(W.device):
            _check(load_library().submconv_weights_create(
                self.ksize, cin, cout, _DTYPES[W.dtype], PREP_INPUT_GRAD if input_grad else 0,
                ctypes.byref(h)))
        self._h = h
        self.set(W)

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise SubmconvError(-1, "weights already freed")
        return self._h

    def set(self, W: torch.Tensor) -> None:
        _require(W, "W", self.dtype, 3)
        if tuple(W.shape) != (27 if self.ksize == 3 else 1, self.cin, self.cout):
            raise ValueError(f"W is {tuple(W.shape)}, the handle's layer "
                             f"[{27 if self.ksize == 3 else 1},{self.cin},{self.cout}]")
        if W.device != self.device:
            raise ValueError(f"W is on {W.device}, the handle on {self.device}")
        with torch.cuda.device(W.device):
            _check(load_library().submconv_weights_set(self.handle, _ptr(W), _stream(W.device)))

    def free(self) -> None:
        if self._h is not None and _lib is not None:
            _check(_lib.submconv_weights_free(self._h))
        self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def prepare_weights(W: torch.Tensor, input_grad: bool = False) -> Weights:
    """Prepares ``W`` ([K,Cin,Cout], fp16 or bf16) for :func:`forward` (or,
    with ``input_grad``, for :func:`backward_input`)."""
    return Weights(W, input_grad)


def forward_kernel(n: int, active_pairs: int, cin: int, cout: int, ksize: int = 3) -> int:
    """The kernel a forward of this shape takes on a map built with default
    flags (host only): 2 the staged MFMA kernel (dense maps, 32 -> 32,
    64 -> 32, 32 -> 64, 128 -> 256 or 256 -> 256 channels), 1 the MFMA kernel
    on the per-tile lists,
    0 VALU; raises :class:`SubmconvError` for a shape the library rejects
    (e.g. MFMA features of 2 GiB or more)."""
    v = int(load_library().submconv_forward_kernel(int(n), int(active_pairs), int(cin), int(cout),
                                                    int(ksize)))
    if v < 0:
        _check(v)
    return v


def _check_bias(bias, cout):
    if bias is not None:
        _require(bias, "bias", torch.float32, 1)
        if bias.shape[0] != cout:
            raise ValueError(f"bias must be [Cout] = [{cout}], got {tuple(bias.shape)}")


def _out_tensor(out, rows, cols, dtype, device):
    if out is None:
        return torch.empty((rows, cols), dtype=dtype, device=device)
    _require(out, "out", dtype, 2)
    if tuple(out.shape) != (rows, cols):
        raise ValueError(f"out must be [{rows},{cols}], got {tuple(out.shape)}")
    return out


def forward(kmap: KernelMap, feats: torch.Tensor, W: Optional[torch.Tensor] = None,
            bias: Optional[torch.Tensor] = None, *, prepared: Optional[Weights] = None,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One SubMConv3d layer: ``out[N,Cout]`` in the caller's row order, in
    the features' dtype (fp16 or bf16; fp32 accumulation).

    Pass either ``W`` ([K,Cin,Cout], the features' dtype: ``submconv_forward``,
    which rearranges it on the fly) or ``prepared`` (a :class:`Weights`:
    ``submconv_forward_prepared``)."""
    _require(feats, "feats", tuple(_DTYPES), 2)
    if feats.shape[0] != kmap.num_rows:
        raise ValueError(f"feats has {feats.shape[0]} rows, the map {kmap.num_rows}")
    cin = feats.shape[1]
    lib = load_library()
    if prepared is not None:
        if W is not None:
            raise ValueError("pass W or prepared, not both")
        if prepared.input_grad:
            raise ValueError("these weights are prepared for the input gradient")
        if prepared.dtype != feats.dtype or prepared.cin != cin:
            raise ValueError(f"weights are {prepared.dtype} with Cin = {prepared.cin}, feats "
                             f"{feats.dtype} with Cin = {cin}")
        cout = prepared.cout
        _check_bias(bias, cout)
        out = _out_tensor(out, feats.shape[0], cout, feats.dtype, feats.device)
        with torch.cuda.device(feats.device):
            _check(lib.submconv_forward_prepared(kmap.handle, _ptr(feats), prepared.handle,
                                                 _ptr(bias), _ptr(out), _stream(feats.device)))
        return out
    if W is None:
        raise ValueError("pass W or prepared")
    _require(W, "W", feats.dtype, 3)
    if W.shape[0] not in (27, 1) or W.shape[1] != cin:
        raise ValueError(f"W is {tuple(W.shape)} but feats has Cin = {cin}")
    ksize = 3 if W.shape[0] == 27 else 1
    cout = W.shape[2]
    _check_bias(bias, cout)
    out = _out_tensor(out, feats.shape[0], cout, feats.dtype, feats.device)
    with torch.cuda.device(feats.device):
        _check(lib.submconv_forward_dtype(kmap.handle, _ptr(feats), _ptr(W), _ptr(bias), _ptr(out),
                                          cin, cout, ksize, _DTYPES[feats.dtype],
                                          _stream(feats.device)))
    return out


def backward_input(kmap: KernelMap, grad_out: torch.Tensor, W: Optional[torch.Tensor] = None, *,
                   prepared: Optional[Weights] = None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Input gradient ``[N,Cin]`` (fp16 or bf16) of a layer with weights ``W``
    ([K,Cin,Cout]) for the output gradient ``grad_out`` ([N,Cout]). Pass ``W``
    or ``prepared`` (``Weights(W, input_grad=True)``)."""
    _require(grad_out, "grad_out", tuple(_DTYPES), 2)
    if grad_out.shape[0] != kmap.num_rows:
        raise ValueError(f"grad_out has {grad_out.shape[0]} rows, the map {kmap.num_rows}")
    cout = grad_out.shape[1]
    lib = load_library()
    if prepared is not None:
        if W is not None:
            raise ValueError("pass W or prepared, not both")
        if not prepared.input_grad:
            raise ValueError("these weights are prepared for the forward, not the input gradient")
        if prepared.dtype != grad_out.dtype or prepared.cout != cout:
            raise ValueError(f"weights are {prepared.dtype} with Cout = {prepared.cout}, grad_out "
                             f"{grad_out.dtype} with Cout = {cout}")
        out = _out_tensor(out, grad_out.shape[0], prepared.cin, grad_out.dtype, grad_out.device)
        with torch.cuda.device(grad_out.device):
            _check(lib.submconv_backward_input_prepared(kmap.handle, _ptr(grad_out),
                                                        prepared.handle, _ptr(out),
                                                        _stream(grad_out.device)))
        return out
    if W is None:
        raise ValueError("pass W or prepared")
    _require(W, "W", grad_out.dtype, 3)
    if W.shape[0] not in (27, 1) or W.shape[2] != cout:
        raise ValueError(f"W is {tuple(W.shape)} but grad_out has Cout = {cout}")
    ksize = 3 if W.shape[0] == 27 else 1
    cin = W.shape[1]
    out = _out_tensor(out, grad_out.shape[0], cin, grad_out.dtype, grad_out.device)
    with torch.cuda.device(grad_out.device):
        _check(lib.submconv_backward_input_dtype(
            kmap.handle, _ptr(grad_out), _ptr(W), _ptr(out), cin, cout, ksize,
            _DTYPES[grad_out.dtype], _stream(grad_out.device)))
    return out


def backward_weight(kmap: KernelMap, feats: torch.Tensor, grad_out: torch.Tensor,
                    ksize: int = 3, out: Optional[torch.Tensor] = None,
                    no_alloc: bool = False) -> torch.Tensor:
    """Weight gradient ``[K,Cin,Cout]`` fp32 from the layer input ``feats``
    ([N,Cin] fp16) and the output gradient ``grad_out`` ([N,Cout] fp16).
    ``no_alloc`` takes ``submconv_backward_weight_noalloc`` (the library's
    fixed per-device workspace instead of a workspace tensor)."""
    _require(feats, "feats", torch.float16, 2)
    _require(grad_out, "grad_out", torch.float16, 2)
    n, cin = feats.shape
    cout = grad_out.shape[1]
    if n != kmap.num_rows or grad_out.shape[0] != n:
        raise ValueError("feats and grad_out must have the map's rows")
    K = 27 if ksize == 3 else 1
    lib = load_library()
    if no_alloc:
        if out is None:
            out = torch.empty((K, cin, cout), dtype=torch.float32, device=feats.device)
        else:
            _require(out, "out", torch.float32, 3)
            if tuple(out.shape) != (K, cin, cout):
                raise ValueError("out must be [K,Cin,Cout]")
        with torch.cuda.device(feats.device):
            _check(lib.submconv_backward_weight_noalloc(kmap.handle, _ptr(feats), _ptr(grad_out),
                                                        _ptr(out), cin, cout, int(ksize),
                                                        _stream(feats.device)))
        return out
    ws = int(lib.submconv_backward_weight_workspace_bytes(kmap.handle, cin, cout, int(ksize)))
    if ws < 0:
        _check(ws)
    work = torch.empty((max(ws, 1),), dtype=torch.uint8, device=feats.device)
    if out is None:
        out = torch.empty((K, cin, cout), dtype=torch.float32, device=feats.device)
    else:
        _require(out, "out", torch.float32, 3)
        if tuple(out.shape) != (K, cin, cout):
            raise ValueError("out must be [K,Cin,Cout]")
    with torch.cuda.device(feats.device):
        _check(lib.submconv_backward_weight(kmap.handle, _ptr(feats), _ptr(grad_out), _ptr(out),
                                            _ptr(work), cin, cout, int(ksize), _stream(feats.device)))
    return out


def backward_bias(grad_out: torch.Tensor) -> torch.Tensor:
    """Bias gradient ``[Cout]`` fp32: the column sums of ``grad_out`` ([N,Cout] fp16)."""
    _require(grad_out, "grad_out", torch.float16, 2)
    out = torch.empty((grad_out.shape[1],), dtype=torch.float32, device=grad_out.device)
    with torch.cuda.device(grad_out.device):
        _check(load_library().submconv_backward_bias(_ptr(grad_out), grad_out.shape[0],
                                                     grad_out.shape[1], _ptr(out),
                                                     _stream(grad_out.device)))
    return out


class MaskedPlan:
    """Handle of a masked implicit-GEMM plan built on a map (rows sorted by
    neighbour mask, per-block tap lists); free it before the map."""

    def __init__(self, handle, kmap: KernelMap):
        self._h = handle
        self.kmap = kmap
        self.row_taps = int(load_library().submconv_masked_row_taps(handle))

    @property
    def handle(self):
        if self._h is None:
            raise SubmconvError(-1, "plan already freed")
        return self._h

    def free(self) -> None:
        if self._h is not None and _lib is not None:
            _check(_lib.submconv_masked_free(self._h))
        self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def masked_plan(kmap: KernelMap) -> MaskedPlan:
    """Builds the masked implicit-GEMM plan of a map (waits for the stream)."""
    h = ctypes.c_void_p()
    with torch.cuda.device(kmap.device):
        _check(load_library().submconv_masked_plan(kmap.handle, _stream(kmap.device), ctypes.byref(h)))
    return MaskedPlan(h, kmap)


def forward_masked(plan: MaskedPlan, feats: torch.Tensor, W: Optional[torch.Tensor] = None,
                   bias: Optional[torch.Tensor] = None, *, prepared: Optional[Weights] = None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The 3x3x3 forward by the masked implicit GEMM (fp16); same result as
    :func:`forward` up to the order of the fp32 additions. Pass ``W``
    ([27,Cin,Cout] fp16, prepared here) or ``prepared``."""
    _require(feats, "feats", torch.float16, 2)
    if feats.shape[0] != plan.kmap.num_rows:
        raise ValueError(f"feats has {feats.shape[0]} rows, the map {plan.kmap.num_rows}")
    if prepared is None:
        if W is None:
            raise ValueError("pass W or prepared")
        prepared = Weights(W)
    if prepared.input_grad or prepared.ksize != 3 or prepared.dtype != torch.float16:
        raise ValueError("masked forward: fp16 3x3x3 weights prepared for the forward")
    if prepared.cin != feats.shape[1]:
        raise ValueError(f"weights have Cin = {prepared.cin}, feats {feats.shape[1]}")
    _check_bias(bias, prepared.cout)
    out = _out_tensor(out, feats.shape[0], prepared.cout, torch.float16, feats.device)
    with torch.cuda.device(feats.device):
        _check(load_library().submconv_forward_masked(plan.handle, _ptr(feats), prepared.handle,
                                                      _ptr(bias), _ptr(out),
                                                      _stream(feats.device)))
    return out


def downsample(coords: torch.Tensor, feats: Optional[torch.Tensor], grid: Sequence[int],
               batch: Optional[int] = None):
    """x2 max-pool: returns ``(pcoords [M,4] int32, inverse [N] int32, pfeats
    [M,C] fp16 or None, pgrid)``; parents in ascending (b,x,y,z) order, each
    parent's features the channel-wise max over its sites."""
    _require(coords, "coords", torch.int32, 2)
    if batch is None:
        batch = int(coords[:, 0].max().item()) + 1 if coords.shape[0] else 1
    lib = load_library()
    g = (ctypes.c_int32 * 3)(*[int(v) for v in grid])
    h = ctypes.c_void_p()
    st = _stream(coords.device)
    with torch.cuda.device(coords.device):
        _check(lib.submconv_downsample_plan(_ptr(coords), coords.shape[0], int(batch), g, st,
                                            ctypes.byref(h)))
        try:
            m = int(lib.submconv_downsample_rows(h))
            pg = (ctypes.c_int32 * 3)()
            _check(lib.submconv_downsample_grid(h, pg))
            pcoords = torch.empty((m, 4), dtype=torch.int32, device=coords.device)
            inverse = torch.empty((coords.shape[0],), dtype=torch.int32, device=coords.device)
            _check(lib.submconv_downsample_coords(h, _ptr(pcoords), _ptr(inverse), st))
            pfeats = None
            if feats is not None:
                _require(feats, "feats", torch.float16, 2)
                pfeats = torch.empty((m, feats.shape[1]), dtype=torch.float16, device=coords.device)
                _check(lib.submconv_downsample_max(h, _ptr(feats), feats.shape[1], _ptr(pfeats), st))
        finally:
            lib.submconv_downsample_free(h)
    return pcoords, inverse, pfeats, tuple(int(v) for v in pg)


def subdivide(coords: torch.Tensor, feats: Optional[torch.Tensor], grid: Sequence[int]):
    """x2 expansion: returns ``(ccoords [8N,4] int32, cfeats [8N,C] fp16 or
    None, cgrid)``, children of site i at rows 8i + 4dx + 2dy + dz."""
    _require(coords, "coords", torch.int32, 2)
    n = coords.shape[0]
    cc = torch.empty((8 * n, 4), dtype=torch.int32, device=coords.device)
    cf = None
    cdim = 0
    if feats is not None:
        _require(feats, "feats", tuple(_DTYPES), 2)  # a copy: any 16-bit type
        cdim = feats.shape[1]
        cf = torch.empty((8 * n, cdim), dtype=feats.dtype, device=coords.device)
    with torch.cuda.device(coords.device):
        _check(load_library().submconv_subdivide(_ptr(coords), n, _ptr(feats), cdim, _ptr(cc),
                                                 _ptr(cf), _stream(coords.device)))
    return cc, cf, tuple(2 * int(v) for v in grid)


class SubMConv3dFunction(torch.autograd.Function):
    """Autograd over the library's kernels (fp16): forward, input gradient
    (the forward with the flipped, transposed kernel on the same map) and
    weight gradient. The weight gradient is computed in fp32 and returned in the
    weight's dtype; the bias gradient is the fp32 column sum of grad_out."""

    @staticmethod
    def forward(ctx, feats, weight, bias, kmap):
        ctx.kmap = kmap
        ctx.save_for_backward(feats, weight)
        ctx.has_bias = bias is not None
        return forward(kmap, feats, weight, bias)

    @staticmethod
    def backward(ctx, grad_out):
        feats, weight = ctx.saved_tensors
        kmap = ctx.kmap
        g = grad_out.contiguous().to(torch.float16)
        ksize = 3 if weight.shape[0] == 27 else 1
        gx = backward_input(kmap, g, weight) if ctx.needs_input_grad[0] else None
        gw = (backward_weight(kmap, feats, g, ksize).to(weight.dtype)
              if ctx.needs_input_grad[1] else None)
        gb = backward_bias(g) if ctx.has_bias and ctx.needs_input_grad[2] else None
        return gx, gw, gb, None


class SubMConv3d(torch.nn.Module):
    """Inference module: weight [K,Cin,Cout] fp16 (K = 27 or 1), optional fp32
    bias; caches the prepared weights until the weight tensor changes."""

    def __init__(self, cin: int, cout: int, ksize: int = 3, bias: bool = True,
                 device=None, dtype=torch.float16):
        super().__init__()
        K = 27 if ksize == 3 else 1
        self.ksize = ksize
        self.weight = torch.nn.Parameter(torch.empty((K, cin, cout), device=device, dtype=dtype),
                                         requires_grad=False)
        self.bias = (torch.nn.Parameter(torch.zeros(cout, device=device, dtype=torch.float32),
                                        requires_grad=False) if bias else None)
        self._cache = None
        self._cache_key = None

    def prepared(self) -> Weights:
        key = (self.weight.data_ptr(), self.weight._version)
        if self._cache is None or self._cache_key != key:
            if self._cache is None or self._cache.device != self.weight.device:
                self._cache = Weights(self.weight.data)
            else:
                self._cache.set(self.weight.data)
            self._cache_key = key
        return self._cache

    def forward(self, kmap: KernelMap, feats: torch.Tensor) -> torch.Tensor:
        return forward(kmap, feats, bias=self.bias, prepared=self.prepared())
