"""Submanifold sparse 3D convolution on MI355X (gfx950): Python binding.

Thin marshalling over the C ABI in include/tr_sparseconv.h (same names without
the `tr_sparseconv_` prefix). Every step of the computation runs in the HIP
library; torch only provides device memory and the current stream.

    h = build_hash(coords)          # int32 [N, 4] (b, x, y, z) on the GPU
    m = build_kernel_map(h)         # m.nbr: int32 [N, 27]
    y = forward(m, x, w)            # x [N, C_in], w [27, C_in, C_out] -> [N, C_out]
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import TrSparseConvError, check  # noqa: F401

__all__ = ["build_hash", "build_kernel_map", "forward", "pack_weights", "forward_packed", "forward_fused",
           "pack_weights_dgrad", "backward_data", "backward_weights", "downsample", "subdivide",
           "channel2spatial", "spatial2channel",
           "status", "hash_lookup", "hash_sorted_rows", "HashTable", "KernelMap", "PackedWeights",
           "TrSparseConvError", "version", "forward_workspace_bytes", "Workspace", "forward_noalloc"]

_DTYPES = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16, torch.float16: _lib.F16}
_ACTS = {"none": _lib.ACT_NONE, "relu": _lib.ACT_RELU, "silu": _lib.ACT_SILU}


def version() -> tuple[int, int]:
    v = _lib.lib().tr_sparseconv_version()
    return v >> 16, v & 0xFFFF


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() else None)


class Workspace:
    """Device bytes starting at a 256-byte boundary. Reusable across builds
    (pass it as `workspace=`) when it is large enough."""

    def __init__(self, nbytes: int, device):
        self.nbytes = int(nbytes)
        self.buf = torch.empty(max(self.nbytes, 1) + 256, dtype=torch.uint8, device=device)
        self.ptr = ctypes.c_void_p(self.buf.data_ptr() + (-self.buf.data_ptr()) % 256)


def _workspace(nbytes: int, device, given: "Workspace | None" = None) -> Workspace:
    if given is not None:
        if given.nbytes < nbytes:
            raise ValueError(f"workspace of {given.nbytes} bytes, {nbytes} needed")
        return given
    return Workspace(nbytes, device)


def _require(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class HashTable:
    """Coordinate hash (tr_sparseconv_build_hash, or tr_sparseconv_build_hash_grid
    when the grid is given: spatial components < 2^grid_log2, object index <
    batch). Keeps its workspace alive."""

    def __init__(self, coords: torch.Tensor, check_status: bool = True,
                 workspace: Workspace | None = None, grid_log2: int | None = None, batch: int = 1):
        _require(coords, "coords", torch.int32, 2)
        if coords.shape[1] != 4:
            raise ValueError(f"coords must be [N, 4], got {tuple(coords.shape)}")
        L = _lib.lib()
        self.device = coords.device
        self.n = int(coords.shape[0])
        h = ctypes.c_void_p()
        if grid_log2 is None:
            self._ws = _workspace(L.tr_sparseconv_hash_workspace_bytes(self.n), self.device, workspace)
            with torch.cuda.device(self.device):
                check(L.tr_sparseconv_build_hash(_ptr(coords), self.n, self._ws.ptr, self._ws.nbytes,
                                                 _stream(self.device), ctypes.byref(h)))
        else:
            need = L.tr_sparseconv_hash_grid_workspace_bytes(self.n, int(grid_log2), int(batch))
            if need == 0:
                raise ValueError(f"grid_log2 = {grid_log2} must be in [2, 16] and batch = {batch} in [1, 65536]")
            self._ws = _workspace(need, self.device, workspace)
            with torch.cuda.device(self.device):
                check(L.tr_sparseconv_build_hash_grid(_ptr(coords), self.n, int(grid_log2), int(batch), self._ws.ptr,
                                                      self._ws.nbytes, _stream(self.device), ctypes.byref(h)))
        self._h = h
        self._destroy = L.tr_sparseconv_hash_destroy
        if check_status:
            self.check_status()

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    def status(self) -> int:
        with torch.cuda.device(self.device):
            return _lib.lib().tr_sparseconv_status(self._h, _stream(self.device))

    def check_status(self) -> None:
        check(self.status())

    def lookup(self, q: torch.Tensor) -> torch.Tensor:
        _require(q, "queries", torch.int32, 2)
        idx = torch.empty(q.shape[0], dtype=torch.int32, device=self.device)
        with torch.cuda.device(self.device):
            check(_lib.lib().tr_sparseconv_hash_lookup(self._h, _ptr(q), int(q.shape[0]), _ptr(idx),
                                                       _stream(self.device)))
        return idx

    def sorted_rows(self) -> torch.Tensor:
        perm = torch.empty(self.n, dtype=torch.int32, device=self.device)
        with torch.cuda.device(self.device):
            check(_lib.lib().tr_sparseconv_hash_sorted_rows(self._h, _ptr(perm), _stream(self.device)))
        return perm

    def __del__(self):
        # the bound C function is held by the instance: module globals may
        # already be gone when this runs at interpreter exit
        h, destroy = getattr(self, "_h", None), getattr(self, "_destroy", None)
        if h is not None and destroy is not None:
            destroy(h)
            self._h = None


class KernelMap:
    """Neighbour table (tr_sparseconv_build_kernel_map); `nbr` is int32 [N, 27]."""

    def __init__(self, h: HashTable, nbr: torch.Tensor | None = None,
                 workspace: Workspace | None = None):
        L = _lib.lib()
        self.hash = h                      # its workspace holds the Morton order
        self.device = h.device
        self.n = h.n
        if nbr is None:
            nbr = torch.empty((self.n, 27), dtype=torch.int32, device=self.device)
        else:
            _require(nbr, "nbr", torch.int32, 2)
            if tuple(nbr.shape) != (self.n, 27):
                raise ValueError(f"nbr must be [{self.n}, 27]")
        self.nbr = nbr
        self._ws = _workspace(L.tr_sparseconv_kmap_workspace_bytes(self.n), self.device, workspace)
        m = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            check(L.tr_sparseconv_build_kernel_map(h.handle, _ptr(self.nbr), self._ws.ptr,
                                                   self._ws.nbytes, _stream(self.device),
                                                   ctypes.byref(m)))
        self._m = m
        self._destroy = L.tr_sparseconv_kmap_destroy

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._m

    def __del__(self):
        m, destroy = getattr(self, "_m", None), getattr(self, "_destroy", None)
        if m is not None and destroy is not None:
            destroy(m)
            self._m = None


def build_hash(coords: torch.Tensor, check_status: bool = True,
               workspace: Workspace | None = None, grid_log2: int | None = None, batch: int = 1) -> HashTable:
    """grid_log2 (with batch): the grid the coordinates lie in, when the caller
    knows it (the resolution of a level); the hash is the same, built from an
    occupancy bitmap when that fits (tr_sparseconv_build_hash_grid)."""
    return HashTable(coords, check_status=check_status, workspace=workspace, grid_log2=grid_log2, batch=batch)


def build_kernel_map(h: HashTable, nbr: torch.Tensor | None = None,
                     workspace: Workspace | None = None) -> KernelMap:
    return KernelMap(h, nbr=nbr, workspace=workspace)


class PackedWeights:
    """Weights re-laid out for the gather-GEMM (tr_sparseconv_pack_weights), or,
    with dgrad=True, for the data gradient (tr_sparseconv_pack_weights_dgrad)."""

    def __init__(self, w: torch.Tensor, dgrad: bool = False):
        if w.dtype not in _DTYPES:
            raise ValueError(f"unsupported dtype {w.dtype}")
        _require(w, "w", w.dtype, 3)
        if w.shape[0] != 27:
            raise ValueError(f"w must be [27, C_in, C_out], got {tuple(w.shape)}")
        self.dtype = w.dtype
        self.dgrad = dgrad
        self.c_in, self.c_out = int(w.shape[1]), int(w.shape[2])
        dt = _DTYPES[w.dtype]
        L = _lib.lib()
        self._ws = Workspace(L.tr_sparseconv_packed_weights_bytes(self.c_in, self.c_out, dt), w.device)
        fn = L.tr_sparseconv_pack_weights_dgrad if dgrad else L.tr_sparseconv_pack_weights
        with torch.cuda.device(w.device):
            check(fn(_ptr(w), self.c_in, self.c_out, dt, self._ws.ptr, self._ws.nbytes, _stream(w.device)))


def pack_weights(w: torch.Tensor) -> PackedWeights:
    return PackedWeights(w)


def pack_weights_dgrad(w: torch.Tensor) -> PackedWeights:
    """w [27, C_in, C_out] packed for backward_data (taps mirrored)."""
    return PackedWeights(w, dgrad=True)


def _check_x(m, x, c_in, dtype):
    if x.dtype != dtype:
        raise ValueError(f"x is {x.dtype}, weights are {dtype}")
    _require(x, "x", dtype, 2)
    if int(x.shape[0]) != m.n or int(x.shape[1]) != c_in:
        raise ValueError(f"x must be [{m.n}, {c_in}], got {tuple(x.shape)}")


def _out(out, n, c_out, x):
    if out is None:
        return torch.empty((n, c_out), dtype=x.dtype, device=x.device)
    _require(out, "out", x.dtype, 2)
    if tuple(out.shape) != (n, c_out):
        raise ValueError(f"out must be [{n}, {c_out}]")
    return out


def forward_packed(m: KernelMap, x: torch.Tensor, wp: PackedWeights,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """forward() with weights packed once by pack_weights()."""
    _check_x(m, x, wp.c_in, wp.dtype)
    out = _out(out, m.n, wp.c_out, x)
    with torch.cuda.device(x.device):
        check(_lib.lib().tr_sparseconv_forward_packed(m.handle, _ptr(x), wp._ws.ptr, _ptr(out),
                                                      wp.c_in, wp.c_out, _DTYPES[wp.dtype],
                                                      _stream(x.device)))
    return out


def forward_fused(m: KernelMap, x: torch.Tensor, wp: PackedWeights, bias: torch.Tensor | None = None,
                  act: str = "none", residual: torch.Tensor | None = None,
                  out_dtype: torch.dtype | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """act(conv(x, w) + bias) + residual in one pass (tr_sparseconv_forward_fused).

    x may be fp32 with half weights (mixed precision); the output is the weights'
    type or fp32 (out_dtype, default: x's type). bias is fp32 [C_out]; residual
    has the output's type and shape and may be `out` itself."""
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {x.dtype}")
    _require(x, "x", x.dtype, 2)
    if int(x.shape[0]) != m.n or int(x.shape[1]) != wp.c_in:
        raise ValueError(f"x must be [{m.n}, {wp.c_in}], got {tuple(x.shape)}")
    if act not in _ACTS:
        raise ValueError(f"act must be one of {sorted(_ACTS)}")
    out_dtype = out_dtype or (out.dtype if out is not None else x.dtype)
    if out_dtype not in _DTYPES:
        raise ValueError(f"unsupported output dtype {out_dtype}")
    if out is None:
        out = torch.empty((m.n, wp.c_out), dtype=out_dtype, device=x.device)
    _require(out, "out", out_dtype, 2)
    if tuple(out.shape) != (m.n, wp.c_out):
        raise ValueError(f"out must be [{m.n}, {wp.c_out}]")
    if bias is not None:
        _require(bias, "bias", torch.float32, 1)
        if int(bias.shape[0]) != wp.c_out:
            raise ValueError(f"bias must be [{wp.c_out}]")
    if residual is not None:
        _require(residual, "residual", out_dtype, 2)
        if tuple(residual.shape) != (m.n, wp.c_out):
            raise ValueError(f"residual must be [{m.n}, {wp.c_out}]")
    with torch.cuda.device(x.device):
        check(_lib.lib().tr_sparseconv_forward_fused(
            m.handle, _ptr(x), _DTYPES[x.dtype], wp._ws.ptr, _DTYPES[wp.dtype], _ptr(bias), _ACTS[act],
            _ptr(residual), _ptr(out), _DTYPES[out_dtype], wp.c_in, wp.c_out, _stream(x.device)))
    return out


def backward_data(m: KernelMap, dy: torch.Tensor, wpd: PackedWeights, out_dtype: torch.dtype | None = None,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """dx [N, C_in] of L = sum <y, dy> (tr_sparseconv_backward_data); wpd from pack_weights_dgrad."""
    if not wpd.dgrad:
        raise ValueError("backward_data needs weights from pack_weights_dgrad")
    if dy.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dy.dtype}")
    _require(dy, "dy", dy.dtype, 2)
    if tuple(dy.shape) != (m.n, wpd.c_out):
        raise ValueError(f"dy must be [{m.n}, {wpd.c_out}], got {tuple(dy.shape)}")
    out_dtype = out_dtype or (out.dtype if out is not None else dy.dtype)
    if out_dtype not in _DTYPES:
        raise ValueError(f"unsupported output dtype {out_dtype}")
    if out is None:
        out = torch.empty((m.n, wpd.c_in), dtype=out_dtype, device=dy.device)
    _require(out, "out", out_dtype, 2)
    if tuple(out.shape) != (m.n, wpd.c_in):
        raise ValueError(f"out must be [{m.n}, {wpd.c_in}]")
    with torch.cuda.device(dy.device):
        check(_lib.lib().tr_sparseconv_backward_data(
            m.handle, _ptr(dy), _DTYPES[dy.dtype], wpd._ws.ptr, _DTYPES[wpd.dtype], _ptr(out), _DTYPES[out_dtype],
            wpd.c_in, wpd.c_out, _stream(dy.device)))
    return out


def backward_weights(m: KernelMap, x: torch.Tensor, dy: torch.Tensor, out: torch.Tensor | None = None,
                     workspace: Workspace | None = None) -> torch.Tensor:
    """dw [27, C_in, C_out] (fp32) of L = sum <y, dy> (tr_sparseconv_backward_weights)."""
    if x.dtype not in _DTYPES or dy.dtype != x.dtype:
        raise ValueError(f"x and dy must share a supported dtype, got {x.dtype}, {dy.dtype}")
    _require(x, "x", x.dtype, 2)
    _require(dy, "dy", x.dtype, 2)
    if int(x.shape[0]) != m.n or int(dy.shape[0]) != m.n:
        raise ValueError(f"x and dy must have {m.n} rows")
    c_in, c_out = int(x.shape[1]), int(dy.shape[1])
    if out is None:
        out = torch.empty((27, c_in, c_out), dtype=torch.float32, device=x.device)
    _require(out, "out", torch.float32, 3)
    if tuple(out.shape) != (27, c_in, c_out):
        raise ValueError(f"out must be [27, {c_in}, {c_out}]")
    dt = _DTYPES[x.dtype]
    L = _lib.lib()
    ws = _workspace(L.tr_sparseconv_backward_weights_workspace_bytes(m.n, c_in, c_out, dt), x.device, workspace)
    with torch.cuda.device(x.device):
        check(L.tr_sparseconv_backward_weights(m.handle, _ptr(x), _ptr(dy), _ptr(out), c_in, c_out, dt, ws.ptr,
                                               ws.nbytes, _stream(x.device)))
    return out


def downsample(h: HashTable, workspace: Workspace | None = None):
    """Parent level of the voxel set of `h`: (coarse coords int32 [M, 4] in
    (b, Z-order) order, children int32 [M, 8] = row of child o or -1)."""
    L = _lib.lib()
    coarse = torch.empty((max(h.n, 1), 4), dtype=torch.int32, device=h.device)
    children = torch.empty((max(h.n, 1), 8), dtype=torch.int32, device=h.device)
    ws = _workspace(L.tr_sparseconv_level_workspace_bytes(h.n), h.device, workspace)
    m = ctypes.c_int64(0)
    with torch.cuda.device(h.device):
        check(L.tr_sparseconv_downsample(h.handle, _ptr(coarse), _ptr(children), h.n, ws.ptr, ws.nbytes,
                                         _stream(h.device), ctypes.byref(m)))
    return coarse[:m.value], children[:m.value]


def subdivide(coords: torch.Tensor, keep: torch.Tensor | None = None, workspace: Workspace | None = None):
    """Finer level: child o of row i exists where bit o of keep[i] (uint8 [N])
    is set (all eight if keep is None). Returns (fine coords int32 [F, 4] in
    (row, octant) order, children int32 [N, 8] = fine row of child o or -1)."""
    _require(coords, "coords", torch.int32, 2)
    n = int(coords.shape[0])
    if keep is not None:
        _require(keep, "keep", torch.uint8, 1)
        if int(keep.shape[0]) != n:
            raise ValueError(f"keep must be [{n}]")
    L = _lib.lib()
    cap = 8 * n
    fine = torch.empty((max(cap, 1), 4), dtype=torch.int32, device=coords.device)
    children = torch.empty((max(n, 1), 8), dtype=torch.int32, device=coords.device)
    ws = _workspace(L.tr_sparseconv_level_workspace_bytes(n), coords.device, workspace)
    f = ctypes.c_int64(0)
    with torch.cuda.device(coords.device):
        check(L.tr_sparseconv_subdivide(_ptr(coords), n, _ptr(keep), _ptr(fine), _ptr(children), cap, ws.ptr,
                                        ws.nbytes, _stream(coords.device), ctypes.byref(f)))
    return fine[:f.value], children[:n]


def _require_children(children: torch.Tensor) -> None:
    _require(children, "children", torch.int32, 2)
    if int(children.shape[1]) != 8:
        raise ValueError(f"children must be [M, 8], got {tuple(children.shape)}")


def channel2spatial(children: torch.Tensor, x_coarse: torch.Tensor, n_fine: int,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """x_fine [n_fine, C] from x_coarse [M, 8C]: channel c * 8 + o of parent q
    goes to channel c of its child o (children [M, 8])."""
    _require_children(children)
    _require(x_coarse, "x_coarse", x_coarse.dtype, 2)
    if x_coarse.dtype not in _DTYPES or x_coarse.shape[1] % 8:
        raise ValueError("x_coarse must be [M, 8C] of a supported dtype")
    if int(x_coarse.shape[0]) != int(children.shape[0]):
        raise ValueError(f"x_coarse has {int(x_coarse.shape[0])} rows, children {int(children.shape[0])}")
    c_fine = int(x_coarse.shape[1]) // 8
    n_fine = int(n_fine)
    if n_fine < 0:
        raise ValueError(f"n_fine = {n_fine}")
    if out is None:
        out = torch.empty((n_fine, c_fine), dtype=x_coarse.dtype, device=x_coarse.device)
    _require(out, "out", x_coarse.dtype, 2)
    if tuple(out.shape) != (n_fine, c_fine):
        raise ValueError(f"out must be [{n_fine}, {c_fine}], got {tuple(out.shape)}")
    with torch.cuda.device(x_coarse.device):
        check(_lib.lib().tr_sparseconv_channel2spatial(_ptr(children), int(children.shape[0]), _ptr(x_coarse),
                                                       _ptr(out), c_fine, _DTYPES[x_coarse.dtype],
                                                       _stream(x_coarse.device)))
    return out


def spatial2channel(children: torch.Tensor, x_fine: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """x_coarse [M, 8C] from x_fine [F, C]; absent children give zeros."""
    _require_children(children)
    if x_fine.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {x_fine.dtype}")
    _require(x_fine, "x_fine", x_fine.dtype, 2)
    c_fine = int(x_fine.shape[1])
    n_coarse = int(children.shape[0])
    if out is None:
        out = torch.empty((n_coarse, 8 * c_fine), dtype=x_fine.dtype, device=x_fine.device)
    _require(out, "out", x_fine.dtype, 2)
    if tuple(out.shape) != (n_coarse, 8 * c_fine):
        raise ValueError(f"out must be [{n_coarse}, {8 * c_fine}], got {tuple(out.shape)}")
    with torch.cuda.device(x_fine.device):
        check(_lib.lib().tr_sparseconv_spatial2channel(_ptr(children), int(children.shape[0]), _ptr(x_fine),
                                                       _ptr(out), c_fine, _DTYPES[x_fine.dtype],
                                                       _stream(x_fine.device)))
    return out


def status(h: HashTable) -> int:
    return h.status()


def hash_lookup(h: HashTable, q: torch.Tensor) -> torch.Tensor:
    return h.lookup(q)


def hash_sorted_rows(h: HashTable) -> torch.Tensor:
    return h.sorted_rows()


def forward_workspace_bytes(c_in: int, c_out: int, dtype: torch.dtype) -> int:
    return int(_lib.lib().tr_sparseconv_forward_workspace_bytes(c_in, c_out, _DTYPES[dtype]))


def forward(m: KernelMap, x: torch.Tensor, w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """y[N, C_out] = submanifold 3x3x3 convolution of x[N, C_in] with w[27, C_in, C_out]."""
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {x.dtype}")
    _require(x, "x", x.dtype, 2)
    _require(w, "w", x.dtype, 3)
    n, c_in = int(x.shape[0]), int(x.shape[1])
    if n != m.n:
        raise ValueError(f"x has {n} rows, kernel map has {m.n}")
    if w.shape[0] != 27 or w.shape[1] != c_in:
        raise ValueError(f"w must be [27, {c_in}, C_out], got {tuple(w.shape)}")
    c_out = int(w.shape[2])
    if out is None:
        out = torch.empty((n, c_out), dtype=x.dtype, device=x.device)
    else:
        _require(out, "out", x.dtype, 2)
        if tuple(out.shape) != (n, c_out):
            raise ValueError(f"out must be [{n}, {c_out}]")
    dt = _DTYPES[x.dtype]
    # A fresh packing buffer per call, from torch's stream-ordered allocator:
    # calls on other streams (same map, other weights) never share it, and it
    # returns to the pool of this stream only, behind the launch that reads it.
    ws = Workspace(_lib.lib().tr_sparseconv_forward_workspace_bytes(c_in, c_out, dt), x.device)
    with torch.cuda.device(x.device):
        check(_lib.lib().tr_sparseconv_forward(m.handle, _ptr(x), _ptr(w), _ptr(out), c_in, c_out, dt,
                                               ws.ptr, ws.nbytes, _stream(x.device)))
    return out


def forward_noalloc(m: KernelMap, x: torch.Tensor, w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """forward() without a workspace (tr_sparseconv_forward_noalloc): the packed
    weights go to the library's per-GPU scratch array, so the call allocates no
    device memory of its own (pass `out` to allocate nothing at all). Calls that
    overlap in time on one GPU race on that array."""
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {x.dtype}")
    _require(x, "x", x.dtype, 2)
    _require(w, "w", x.dtype, 3)
    n, c_in = int(x.shape[0]), int(x.shape[1])
    if n != m.n:
        raise ValueError(f"x has {n} rows, kernel map has {m.n}")
    if w.shape[0] != 27 or w.shape[1] != c_in:
        raise ValueError(f"w must be [27, {c_in}, C_out], got {tuple(w.shape)}")
    c_out = int(w.shape[2])
    out = _out(out, n, c_out, x)
    with torch.cuda.device(x.device):
        check(_lib.lib().tr_sparseconv_forward_noalloc(m.handle, _ptr(x), _ptr(w), _ptr(out), c_in, c_out,
                                                       _DTYPES[x.dtype], _stream(x.device)))
    return out
