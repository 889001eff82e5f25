"""CPU oracle for the submanifold sparse 3D convolution (ctypes wrapper).

TEST INFRASTRUCTURE. Only the tests, the package entry's smoke check and the
benchmark's CPU-baseline leg may import this module. The HIP library never
loads it, and it loads nothing of the HIP library.

The arithmetic lives in `oracle.cpp` (plain C++17, std::unordered_map lookup,
fp64 direct summation); its header cites the passages it follows. This file
only compiles it, marshals numpy arrays and widens inputs exactly to float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "_oracle.so")

OK = 0
ERR_INVALID = -1
ERR_COORD_RANGE = -2
ERR_DUPLICATE = -3

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (-O2, OpenMP; no hand SIMD, no blocking)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", "-std=c++17", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oc_build.argtypes = [P, I64, ctypes.POINTER(P)]
        lib.oc_build.restype = ctypes.c_int
        lib.oc_free.argtypes = [P]
        lib.oc_free.restype = None
        lib.oc_lookup.argtypes = [P, P, I64, P]
        lib.oc_lookup.restype = ctypes.c_int
        lib.oc_kernel_map.argtypes = [P, P]
        lib.oc_kernel_map.restype = ctypes.c_int
        lib.oc_forward.argtypes = [P, I64, P, I64, P, P, ctypes.c_int, ctypes.c_int, P]
        lib.oc_forward.restype = ctypes.c_int
        lib.oc_epilogue.argtypes = [P, I64, ctypes.c_int, P, P, ctypes.c_int]
        lib.oc_epilogue.restype = ctypes.c_int
        lib.oc_backward_data.argtypes = [P, I64, P, I64, P, P, ctypes.c_int, ctypes.c_int, P]
        lib.oc_backward_data.restype = ctypes.c_int
        lib.oc_backward_weights.argtypes = [P, I64, P, P, ctypes.c_int, ctypes.c_int, P, I64, P]
        lib.oc_backward_weights.restype = ctypes.c_int
        lib.oc_downsample.argtypes = [P, I64, P, P, P]
        lib.oc_downsample.restype = ctypes.c_int
        lib.oc_subdivide.argtypes = [P, I64, P, P, P, P]
        lib.oc_subdivide.restype = ctypes.c_int
        lib.oc_regroup.argtypes = [P, I64, I64, ctypes.c_int, ctypes.c_int, P, P]
        lib.oc_regroup.restype = ctypes.c_int
        lib.oc_num_threads.argtypes = []
        lib.oc_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: oracle status {code}")
        self.code = code


class Table:
    """The coordinate -> row map (std::unordered_map), built in caller order."""

    def __init__(self, coords: np.ndarray):
        lib = _load()
        self.coords = np.ascontiguousarray(coords, dtype=np.int32).reshape(-1, 4)
        self.n = int(self.coords.shape[0])
        h = ctypes.c_void_p()
        st = lib.oc_build(_ptr(self.coords), self.n, ctypes.byref(h))
        if st != OK:
            raise OracleError(st, "build")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.oc_free(h)
            self._h = None

    def lookup(self, q: np.ndarray) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.int32).reshape(-1, 4)
        idx = np.empty(q.shape[0], dtype=np.int32)
        st = _load().oc_lookup(self._h, _ptr(q), q.shape[0], _ptr(idx))
        if st != OK:
            raise OracleError(st, "lookup")
        return idx

    def kernel_map(self) -> np.ndarray:
        nbr = np.empty((self.n, 27), dtype=np.int32)
        st = _load().oc_kernel_map(self._h, _ptr(nbr))
        if st != OK:
            raise OracleError(st, "kernel_map")
        return nbr


def build_status(coords: np.ndarray) -> int:
    """Status of building the map for `coords` (0, ERR_COORD_RANGE, ERR_DUPLICATE)."""
    try:
        Table(coords)
    except OracleError as e:
        return e.code
    return OK


def kernel_map(coords: np.ndarray) -> np.ndarray:
    """int32 [N, 27] neighbour rows (-1 where absent), caller row order."""
    return Table(coords).kernel_map()


def widen(a: np.ndarray) -> np.ndarray:
    """Exact widening to float64 (float32 values, or bf16 values held in float32)."""
    return np.ascontiguousarray(a, dtype=np.float64)


def forward(nbr: np.ndarray, x: np.ndarray, w: np.ndarray, rows=None) -> np.ndarray:
    """fp64 y[r, :] for r in `rows` (default all rows): sum over taps k with
    nbr[r, k] >= 0 and input channels of W[k, ci, :] * x[nbr[r, k], ci]."""
    nbr = np.ascontiguousarray(nbr, dtype=np.int32)
    n = int(nbr.shape[0])
    wd = widen(w)
    if wd.ndim != 3:
        raise ValueError(f"weights must be [27, C_in, C_out], got {wd.shape}")
    c_in = int(wd.shape[1])
    xd = widen(x).reshape(n, c_in)
    if wd.shape[0] != 27:
        raise ValueError(f"weights must have 27 taps, got {wd.shape}")
    c_out = int(wd.shape[2])
    if rows is None:
        y = np.empty((n, c_out), dtype=np.float64)
        st = _load().oc_forward(_ptr(nbr), n, None, 0, _ptr(xd), _ptr(wd), c_in, c_out, _ptr(y))
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        y = np.empty((r.shape[0], c_out), dtype=np.float64)
        st = _load().oc_forward(_ptr(nbr), n, _ptr(r), r.shape[0], _ptr(xd), _ptr(wd),
                                c_in, c_out, _ptr(y))
    if st != OK:
        raise OracleError(st, "forward")
    return y


def backward_data(nbr: np.ndarray, dy: np.ndarray, w: np.ndarray, rows=None) -> np.ndarray:
    """dx[rows] (fp64) of L = sum <y, dy> for y = forward(nbr, x, w)."""
    nbr = np.ascontiguousarray(nbr, dtype=np.int32)
    n = nbr.shape[0]
    wd = widen(w)
    c_in, c_out = wd.shape[1], wd.shape[2]
    dyd = widen(dy).reshape(n, c_out)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    m = n if r is None else len(r)
    dx = np.empty((m, c_in), dtype=np.float64)
    st = _load().oc_backward_data(_ptr(nbr), n, None if r is None else _ptr(r), 0 if r is None else len(r),
                                  _ptr(dyd), _ptr(wd), c_in, c_out, _ptr(dx))
    if st != OK:
        raise OracleError(st, "backward_data")
    return dx


def backward_weights(nbr: np.ndarray, x: np.ndarray, dy: np.ndarray, sel=None) -> np.ndarray:
    """dw (fp64): [27, c_in, c_out], or [len(sel), c_out] for sel = [(k, ci), ...]."""
    nbr = np.ascontiguousarray(nbr, dtype=np.int32)
    n = nbr.shape[0]
    xd = widen(x).reshape(n, -1)
    dyd = widen(dy).reshape(n, -1)
    c_in, c_out = xd.shape[1], dyd.shape[1]
    s = None if sel is None else np.ascontiguousarray(sel, dtype=np.int32).reshape(-1, 2)
    m = 27 * c_in if s is None else len(s)
    dw = np.empty((m, c_out), dtype=np.float64)
    st = _load().oc_backward_weights(_ptr(nbr), n, _ptr(xd), _ptr(dyd), c_in, c_out,
                                     None if s is None else _ptr(s), 0 if s is None else len(s), _ptr(dw))
    if st != OK:
        raise OracleError(st, "backward_weights")
    return dw.reshape(27, c_in, c_out) if s is None else dw


def downsample(coords: np.ndarray):
    """(coarse coords [m, 4], children [m, 8]) of the parent level."""
    c = np.ascontiguousarray(coords, dtype=np.int32).reshape(-1, 4)
    n = len(c)
    coarse = np.empty((n, 4), dtype=np.int32)
    children = np.empty((n, 8), dtype=np.int32)
    m = ctypes.c_int64(0)
    st = _load().oc_downsample(_ptr(c), n, _ptr(coarse), _ptr(children), ctypes.byref(m))
    if st != OK:
        raise OracleError(st, "downsample")
    return coarse[:m.value].copy(), children[:m.value].copy()


def subdivide(coords: np.ndarray, keep=None):
    """(fine coords [f, 4], children [n, 8]); keep: uint8 [n] child bitmasks or None (all)."""
    c = np.ascontiguousarray(coords, dtype=np.int32).reshape(-1, 4)
    n = len(c)
    k = None if keep is None else np.ascontiguousarray(keep, dtype=np.uint8).reshape(n)
    fine = np.empty((8 * n, 4), dtype=np.int32)
    children = np.empty((n, 8), dtype=np.int32)
    f = ctypes.c_int64(0)
    st = _load().oc_subdivide(_ptr(c), n, None if k is None else _ptr(k), _ptr(fine), _ptr(children),
                              ctypes.byref(f))
    if st != OK:
        raise OracleError(st, "subdivide")
    return fine[:f.value].copy(), children


def channel2spatial(children: np.ndarray, x_coarse: np.ndarray, n_fine: int) -> np.ndarray:
    """x_fine [n_fine, C] (fp64) from x_coarse [n_coarse, 8 C]."""
    ch = np.ascontiguousarray(children, dtype=np.int32).reshape(-1, 8)
    xc = widen(x_coarse).reshape(len(ch), -1)
    c_fine = xc.shape[1] // 8
    xf = np.zeros((n_fine, c_fine), dtype=np.float64)
    st = _load().oc_regroup(_ptr(ch), len(ch), n_fine, c_fine, 1, _ptr(xc), _ptr(xf))
    if st != OK:
        raise OracleError(st, "channel2spatial")
    return xf


def spatial2channel(children: np.ndarray, x_fine: np.ndarray) -> np.ndarray:
    """x_coarse [n_coarse, 8 C] (fp64) from x_fine [n_fine, C]."""
    ch = np.ascontiguousarray(children, dtype=np.int32).reshape(-1, 8)
    xf = widen(x_fine)
    c_fine = xf.shape[1]
    xc = np.empty((len(ch), 8 * c_fine), dtype=np.float64)
    st = _load().oc_regroup(_ptr(ch), len(ch), len(xf), c_fine, 0, _ptr(xc), _ptr(xf))
    if st != OK:
        raise OracleError(st, "spatial2channel")
    return xc


ACTS = {"none": 0, "relu": 1, "silu": 2}


def epilogue(y: np.ndarray, bias=None, residual=None, act: str = "none") -> np.ndarray:
    """act(y + bias) + residual in fp64 (y: [m, c_out]; residual rows match y's rows)."""
    yd = np.array(y, dtype=np.float64, copy=True, order="C")
    m, c_out = yd.shape
    b = None if bias is None else widen(bias).reshape(c_out)
    r = None if residual is None else widen(residual).reshape(m, c_out)
    st = _load().oc_epilogue(_ptr(yd), m, c_out, None if b is None else _ptr(b),
                             None if r is None else _ptr(r), ACTS[act])
    if st != OK:
        raise OracleError(st, "epilogue")
    return yd


def conv(coords: np.ndarray, x: np.ndarray, w: np.ndarray, rows=None):
    """Kernel map and forward in one call: returns (nbr, y)."""
    nbr = kernel_map(coords)
    return nbr, forward(nbr, x, w, rows)


def num_threads() -> int:
    return int(_load().oc_num_threads())
