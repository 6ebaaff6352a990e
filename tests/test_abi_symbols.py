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
              "submconv_prepare_weights", "submconv_map_active_pairs"]:
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
    assert lib.submconv_abi_version() == 1
    lib.submconv_status_string.restype = ctypes.c_char_p
    lib.submconv_status_string.argtypes = [ctypes.c_int]
    assert lib.submconv_status_string(0) == b"ok"
    assert lib.submconv_status_string(-3) == b"duplicate coordinate"
    f = lib.submconv_prepared_weights_elems
    f.restype = ctypes.c_int64
    f.argtypes = [ctypes.c_int32] * 3
    assert f(3, 128, 128) == 27 * 128 * 128
    assert f(1, 32, 32) == 32 * 32
    assert f(3, 12, 16) == -4   # Cin not a multiple of 8
    assert f(2, 16, 16) == -1   # bad ksize
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
    assert lib.submconv_build_map(None, 0, 1, g, 16, None, ctypes.byref(h)) == -1  # unknown flag
    lib.submconv_forward.restype = ctypes.c_int
    assert lib.submconv_forward(None, None, None, None, None, 8, 8, 3, None) == -1  # map NULL
    lib.submconv_map_free.restype = ctypes.c_int
    assert lib.submconv_map_free(None) == 0


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import submanifold_sparse_convolution_hash_amd as sc
    monkeypatch.setattr(sc, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(sc, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        sc.load_library()
