"""The C-ABI library: loads, exports every declared symbol, rejects bad
arguments on the host before touching the device. No GPU needed."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tr_sparseconv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tr_sparseconv_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    from submanifold_sparse_conv_amd import _lib
    return _lib.lib()


def test_header_and_binding_agree(L):
    from submanifold_sparse_conv_amd import _lib
    decl = declared_functions()
    assert len(decl) >= 14
    bound = sorted(name for name, _, _ in _lib.SIGNATURES)
    assert bound == decl


def test_library_exports_every_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_one_hip_runtime_in_process(L):
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) <= 1, paths


def test_version(L):
    import submanifold_sparse_conv_amd as sc
    assert sc.version() >= (0, 1)


def test_workspace_sizes(L):
    assert L.tr_sparseconv_hash_workspace_bytes(-1) == 0
    assert L.tr_sparseconv_hash_workspace_bytes(0) > 0
    a = L.tr_sparseconv_hash_workspace_bytes(1000)
    b = L.tr_sparseconv_hash_workspace_bytes(100000)
    # table of >= 2N 16-byte slots plus sort buffers
    assert b >= 100000 * (2 * 16 + 24) and b > a
    assert L.tr_sparseconv_hash_workspace_bytes((1 << 30) + 1) == 0
    assert L.tr_sparseconv_kmap_workspace_bytes(1000) >= 4000
    assert L.tr_sparseconv_forward_workspace_bytes(64, 32, 1) >= 27 * 64 * 32 * 2
    assert L.tr_sparseconv_forward_workspace_bytes(0, 32, 1) == 0


def test_grid_workspace_sizes(L):
    G = L.tr_sparseconv_hash_grid_workspace_bytes
    for g, batch in ((1, 1), (17, 1), (8, 0), (8, 65537)):
        assert G(1000, g, batch) == 0                     # grid outside [2, 16] x [1, 65536]
    assert G(-1, 8, 1) == 0 and G((1 << 30) + 1, 8, 1) == 0
    # bitmap build: the bitmap (2^(3g) bits per object) plus per-voxel and per-word arrays;
    # 256^3 x 1: 2 MB of bitmap and 1 MB of word prefixes at least
    n = 393720
    dense = G(n, 8, 1)
    assert dense >= n * 12 + (1 << 21) + (1 << 20)
    assert G(n, 8, 2) > dense                            # twice the bitmap
    # beyond 32 MB of bitmap the build is the radix one, with its workspace
    assert G(n, 10, 1) == L.tr_sparseconv_hash_workspace_bytes(n)
    assert G(n, 16, 65536) == L.tr_sparseconv_hash_workspace_bytes(n)
    assert G(0, 8, 1) == L.tr_sparseconv_hash_workspace_bytes(0)  # empty: the radix path


def test_host_argument_errors(L):
    from submanifold_sparse_conv_amd import _lib
    P = ctypes.c_void_p
    out = ctypes.c_void_p()
    fake = P(0x10000)  # never dereferenced: every call below fails its host checks first
    assert L.tr_sparseconv_build_hash(fake, 10, fake, 1 << 20, None, None) == _lib.ERR_INVALID_ARG
    assert L.tr_sparseconv_build_hash(fake, -1, fake, 1 << 20, None, ctypes.byref(out)) == _lib.ERR_INVALID_ARG
    assert out.value is None
    assert L.tr_sparseconv_build_hash(None, 10, fake, 1 << 20, None, ctypes.byref(out)) == _lib.ERR_INVALID_ARG
    assert L.tr_sparseconv_build_hash(fake, 10, None, 1 << 20, None, ctypes.byref(out)) == _lib.ERR_INVALID_ARG
    assert L.tr_sparseconv_build_hash(fake, 10, P(0x10010), 1 << 20, None,
                                      ctypes.byref(out)) == _lib.ERR_INVALID_ARG  # misaligned
    assert L.tr_sparseconv_build_hash(fake, 10, fake, 64, None, ctypes.byref(out)) == _lib.ERR_WORKSPACE
    assert b"workspace" in L.tr_sparseconv_last_error()
    bg = L.tr_sparseconv_build_hash_grid
    assert bg(fake, 10, 8, 1, fake, 1 << 20, None, None) == _lib.ERR_INVALID_ARG
    assert bg(fake, 10, 1, 1, fake, 1 << 20, None, ctypes.byref(out)) == _lib.ERR_INVALID_ARG
    assert bg(fake, 10, 8, 0, fake, 1 << 20, None, ctypes.byref(out)) == _lib.ERR_INVALID_ARG
    assert bg(fake, -1, 8, 1, fake, 1 << 20, None, ctypes.byref(out)) == _lib.ERR_INVALID_ARG
    assert bg(None, 10, 8, 1, fake, 1 << 20, None, ctypes.byref(out)) == _lib.ERR_INVALID_ARG
    assert bg(fake, 10, 8, 1, P(0x10010), 1 << 30, None, ctypes.byref(out)) == _lib.ERR_INVALID_ARG
    assert bg(fake, 10, 8, 1, fake, 64, None, ctypes.byref(out)) == _lib.ERR_WORKSPACE
    assert bg(fake, 10, 12, 1, fake, 64, None, ctypes.byref(out)) == _lib.ERR_WORKSPACE  # radix fallback
    assert out.value is None
    assert L.tr_sparseconv_status(None, None) == _lib.ERR_INVALID_ARG
    assert L.tr_sparseconv_hash_size(None) == -1
    assert L.tr_sparseconv_build_kernel_map(None, fake, fake, 1 << 20, None,
                                            ctypes.byref(out)) == _lib.ERR_INVALID_ARG
    assert L.tr_sparseconv_forward(None, fake, fake, fake, 8, 8, 0, None, 0, None) == _lib.ERR_INVALID_ARG
    assert L.tr_sparseconv_hash_lookup(None, fake, 1, fake, None) == _lib.ERR_INVALID_ARG
    L.tr_sparseconv_hash_destroy(None)
    L.tr_sparseconv_kmap_destroy(None)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    from submanifold_sparse_conv_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        _lib.lib()
