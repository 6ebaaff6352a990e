"""The C-ABI library loads and exports every symbol that include/submconv.h
declares. Only host-side entry points (no device work) are called here."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "submconv.h")
LIB = os.path.join(ROOT, "submanifold_sparse_convolution_hash_amd", "libsubmconv.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(submconv_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from submanifold_sparse_convolution_hash_amd import build
        build.build()
    return ctypes.CDLL(LIB)


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["submconv_build_map", "submconv_forward", "submconv_map_export", "submconv_map_free",
              "submconv_weights_create", "submconv_weights_set", "submconv_forward_prepared",
              "submconv_forward_kernel", "submconv_map_active_pairs"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    for name in _declared():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_host_only_entry_points(lib):
    lib.submconv_abi_version.restype = ctypes.c_int
    assert lib.submconv_abi_version() == 2
    lib.submconv_status_string.restype = ctypes.c_char_p
    lib.submconv_status_string.argtypes = [ctypes.c_int]
    assert lib.submconv_status_string(0) == b"ok"
    assert lib.submconv_status_string(-3) == b"duplicate coordinate"
    # weights handles: shape, dtype and flag errors before any device call
    wc = lib.submconv_weights_create
    wc.restype = ctypes.c_int
    wc.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_uint32, ctypes.c_void_p]
    h = ctypes.c_void_p()
    assert wc(3, 12, 16, 0, 0, ctypes.byref(h)) == -4   # Cin not a multiple of 8
    assert wc(2, 16, 16, 0, 0, ctypes.byref(h)) == -1   # bad ksize
    assert wc(3, 16, 16, 2, 0, ctypes.byref(h)) == -1   # bad dtype
    assert wc(3, 16, 16, 0, 2, ctypes.byref(h)) == -1   # unknown flag
    assert wc(3, 16, 16, 0, 0, None) == -1              # no handle pointer
    lib.submconv_weights_free.restype = ctypes.c_int
    assert lib.submconv_weights_free(None) == 0
    # argument errors are reported before any device work
    lib.submconv_build_map.restype = ctypes.c_int
    lib.submconv_build_map.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    h = ctypes.c_void_p()
    g = (ctypes.c_int32 * 3)(4, 4, 4)
    assert lib.submconv_build_map(None, 10, 1, g, 0, None, ctypes.byref(h)) == -1  # coords NULL
    assert lib.submconv_build_map(None, -1, 1, g, 0, None, ctypes.byref(h)) == -1  # n < 0
    g0 = (ctypes.c_int32 * 3)(0, 4, 4)
    assert lib.submconv_build_map(None, 0, 1, g0, 0, None, ctypes.byref(h)) == -1  # grid[0] < 1
    assert lib.submconv_build_map(None, 0, 1, g, 4 | 8, None, ctypes.byref(h)) == -1  # two tile sizes
    assert lib.submconv_build_map(None, 0, 1, g, 16 | 32, None, ctypes.byref(h)) == -1  # staged and not
    assert lib.submconv_build_map(None, 0, 1, g, 64, None, ctypes.byref(h)) == -1  # unknown flag
    lib.submconv_forward.restype = ctypes.c_int
    assert lib.submconv_forward(None, None, None, None, None, 8, 8, 3, None) == -1  # map NULL
    lib.submconv_map_free.restype = ctypes.c_int
    assert lib.submconv_map_free(None) == 0


def test_forward_kernel_choice_and_buffer_limit(lib):
    """Which kernel a forward takes, decided on the host: the MFMA gather-GEMM
    for its channel counts while features and lists stay below 2 GiB (its
    32-bit buffer offsets), an explicit SUBMCONV_ERR_UNSUPPORTED_SHAPE above,
    the VALU kernel for other channel counts (64-bit addressing, no limit);
    on dense maps (12 or more neighbours per row) the staged kernels for
    32 -> 32, 64 -> 32, 32 -> 64, 128 -> 256 and 256 -> 256 channels."""
    f = lib.submconv_forward_kernel
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    assert f(209715, 744981, 128, 128, 3) == 1
    assert f(1495574, 31_200_000, 64, 32, 3) == 2   # dense: the staged kernel
    assert f(1495574, 31_200_000, 64, 64, 3) == 1   # (not for 64 -> 64)
    assert f(1495574, 5_000_000, 64, 32, 3) == 1    # under 12 neighbours per row
    assert f(1495574, 31_200_000, 64, 32, 1) == 1   # a 1x1x1 layer
    assert f(744643, 15_556_763, 256, 256, 3) == 2  # the 256^3 shells
    assert f(744643, 15_556_763, 128, 256, 3) == 2
    assert f(744643, 15_556_763, 256, 128, 3) == 1
    assert f(744643, 15_556_763, 128, 128, 3) == 1
    assert f(1000, 4000, 256, 256, 1) == 1
    assert f(1000, 4000, 96, 96, 3) == 0        # no MFMA tile for 96 channels
    assert f(1000, 4000, 256, 64, 3) == 0       # Cin 256 needs Cout a multiple of 128
    limit = 2 ** 31 - 64
    n_ok = limit // (256 * 2)                   # the last row count below the limit
    assert f(n_ok, 10, 256, 256, 3) == 1
    assert f(n_ok + 1, 10, 256, 256, 3) == -4
    assert f(n_ok + 1, 10, 96, 96, 3) == 0      # the VALU kernel has no such limit
    p_ok = limit // 8 - 1                       # (pairs + 1) * 8 at the limit
    assert f(1000, p_ok, 128, 128, 3) == 1
    assert f(1000, p_ok + 1, 128, 128, 3) == -4
    assert f(1000, p_ok + 1, 128, 128, 1) == 1  # a 1x1x1 layer reads no lists
    assert f(1000, 10, 12, 16, 3) == -4         # shape errors as the forward
    assert f(1000, 10, 16, 16, 2) == -1
    assert f(-1, 10, 16, 16, 3) == -1


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import submanifold_sparse_convolution_hash_amd as sc
    monkeypatch.setattr(sc, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(sc, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        sc.load_library()
