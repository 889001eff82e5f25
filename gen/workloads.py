"""Seeded synthetic workloads for the submanifold sparse 3D convolution.

This module only makes inputs: which voxels are active (coordinates), the
feature rows and the weights. It holds none of the convolution's arithmetic
(no neighbour search, no hashing, no products or sums), so both the HIP path
and the CPU oracle can take their inputs from it without sharing any of the
method.

Conventions followed (cited from the pages):
  * coordinates are int32 rows (b, x, y, z) -- "Running TRELLIS.2 on Apple
    Silicon" startup packet (page 5), section 5, fixture table, row B;
  * features are [N, C] rows (same table, rows C and D);
  * weights are tap-major [27, C_in, C_out] -- same page, section 5 (on-disk
    sparse conv layout and the per-offset gather-GEMM contract) and section 8.

The occupancy shapes stand in for the decoders' surface-voxel sets the pages
measure on (a 64^3 occupancy grid from the structure decoder; 1.9M-5.5M
surface voxels at the higher resolutions -- "Porting TRELLIS.2 From Python to
Rust and Metal", sections II and III; trellis2mlx README, result tables). No
public dataset is involved; every array is drawn from numpy's PCG64 with the
seed recorded on the returned object.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# ----------------------------------------------------------------------------
# Config table. `seed` is the config's base seed; correctness runs add 100 and
# 200 to it. Geometry and values come from separate SeedSequence children.
# ----------------------------------------------------------------------------
CONFIGS = {
    "T": dict(D=16, B=1, c_in=8, c_out=8, dtype="f32", seed=1,
              desc="16^3, 1 object, sphere shell radius 6 thickness 1, C 8->8 fp32"),
    "S": dict(D=64, B=1, c_in=64, c_out=64, dtype="bf16", seed=2,
              desc="64^3, 1 object, union of 3 ellipsoid shells (thickness 2), C 64->64 bf16"),
    "W": dict(D=64, B=4, c_in=1024, c_out=1024, dtype="bf16", seed=3,
              desc="64^3 x 4 objects, ellipsoid-shell unions, C 1024->1024 bf16"),
    "L": dict(D=256, B=1, c_in=128, c_out=128, dtype="bf16", seed=4,
              desc="256^3, 1 object, thickened fBm level set (thickness 2), C 128->128 bf16"),
    "X": dict(D=512, B=2, c_in=64, c_out=32, dtype="bf16", seed=5,
              desc="512^3 x 2 objects, Gaussian blobs + holed thin sheets, C 64->32 bf16"),
}
CONFIG_ORDER = ["T", "S", "W", "L", "X"]

# Base period of the 256^3 fBm field. Chosen once by `select_fbm_period` with
# the config's geometry seed: among FBM_CANDIDATES, the one whose active count
# falls in 350k-450k, nearest 400k (48..128 all give more than 450k voxels with
# this field, so the list reaches up to 256). Frozen here so that generating the
# workload needs one field evaluation, not seven.
FBM_PERIOD_L = 192
FBM_CANDIDATES = (48, 64, 96, 128, 160, 192, 256)


@dataclasses.dataclass
class Workload:
    name: str
    D: int
    B: int
    c_in: int
    c_out: int
    dtype: str            # "f32", "bf16", "f16", "mixed-bf16" or "mixed-f16"
    seed: int
    order: str            # "raster" or "shuffled"
    coords: np.ndarray    # int32 [N, 4] (b, x, y, z)
    x: np.ndarray | None = None   # float32 [N, c_in], representable in dtype's feature type
    w: np.ndarray | None = None   # float32 [27, c_in, c_out], representable in dtype's weight type

    @property
    def n(self) -> int:
        return int(self.coords.shape[0])

    def x_bits(self) -> np.ndarray:
        """bf16 bit patterns (uint16) of x; only for dtype == 'bf16'."""
        return f32_to_bf16_bits(self.x)

    def w_bits(self) -> np.ndarray:
        return f32_to_bf16_bits(self.w)


# ----------------------------------------------------------------------------
# bf16 encoding of generated values (round to nearest, ties to even).
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the
    16-bit patterns. Inputs here are finite Gaussian draws (no NaN/Inf)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


# ----------------------------------------------------------------------------
# Geometry helpers
# ----------------------------------------------------------------------------
def _grid_axis(D: int) -> np.ndarray:
    return np.arange(D, dtype=np.float64)


def _random_rotation(rng: np.random.Generator) -> np.ndarray:
    """Uniform random rotation from a normalised Gaussian quaternion."""
    q = rng.standard_normal(4)
    q /= np.linalg.norm(q)
    w, x, y, z = q
    return np.array([
        [1 - 2 * (y * y + z * z), 2 * (x * y - z * w), 2 * (x * z + y * w)],
        [2 * (x * y + z * w), 1 - 2 * (x * x + z * z), 2 * (y * z - x * w)],
        [2 * (x * z - y * w), 2 * (y * z + x * w), 1 - 2 * (x * x + y * y)],
    ])


def sphere_shell(rng: np.random.Generator, D: int = 16, radius: float = 6.0,
                 thickness: float = 1.0) -> np.ndarray:
    """Occupancy (bool [D,D,D]) of an integer sphere shell: voxel p is active
    when radius - t/2 <= |p - c| < radius + t/2, c = grid centre jittered by
    U(-1/2, 1/2) per axis."""
    c = (D - 1) / 2.0 + rng.uniform(-0.5, 0.5, 3)
    a = _grid_axis(D)
    d2 = ((a[:, None, None] - c[0]) ** 2 + (a[None, :, None] - c[1]) ** 2
          + (a[None, None, :] - c[2]) ** 2)
    d = np.sqrt(d2)
    return (d >= radius - thickness / 2) & (d < radius + thickness / 2)


def ellipsoid_shells(rng: np.random.Generator, D: int = 64, count: int = 3) -> np.ndarray:
    """Union of `count` random ellipsoid shells of thickness about 2.

    Each ellipsoid: centre U(22,42)^3 (scaled to D/64), semi-axes U(10,22)^3,
    uniform random rotation R. With s(p) = |diag(1/a) R^T (p - c)| the voxel
    is active when |s - 1| < |grad s|, i.e. its first-order distance to the
    surface s = 1 is below one voxel on either side."""
    sc = D / 64.0
    a0 = _grid_axis(D)
    P = np.stack(np.meshgrid(a0, a0, a0, indexing="ij"), axis=-1).reshape(-1, 3)
    occ = np.zeros(P.shape[0], dtype=bool)
    for _ in range(count):
        c = rng.uniform(22 * sc, 42 * sc, 3)
        semi = rng.uniform(10 * sc, 22 * sc, 3)
        R = _random_rotation(rng)
        u = ((P - c) @ R) / semi          # u = diag(1/a) R^T (p - c)
        s = np.sqrt((u * u).sum(axis=1))
        g = np.sqrt(((u / semi) ** 2).sum(axis=1))   # |grad s| * s
        occ |= np.abs(s - 1.0) * s < g
    return occ.reshape(D, D, D)


def ellipsoid_object(rng: np.random.Generator, D: int, n_lo: int, n_hi: int,
                     max_tries: int = 200) -> np.ndarray:
    """Redraw ellipsoid-shell unions until the active count is in [n_lo, n_hi]."""
    for _ in range(max_tries):
        occ = ellipsoid_shells(rng, D)
        if n_lo <= int(occ.sum()) <= n_hi:
            return occ
    raise RuntimeError("ellipsoid_object: no draw landed in the requested size range")


def _quintic(f: np.ndarray) -> np.ndarray:
    return f * f * f * (f * (f * 6.0 - 15.0) + 10.0)


def _interp_matrix(D: int, period: float, n_lat: int) -> np.ndarray:
    """[D, n_lat] weights of quintic-smoothed linear interpolation between
    lattice points spaced `period` voxels apart."""
    t = np.arange(D, dtype=np.float64) / period
    i0 = np.floor(t).astype(np.int64)
    f = _quintic(t - i0)
    M = np.zeros((D, n_lat))
    M[np.arange(D), i0] = 1.0 - f
    M[np.arange(D), i0 + 1] = f
    return M


def fbm_field(rng: np.random.Generator, D: int, period0: float, octaves: int = 4,
              gain: float = 0.5, lacunarity: float = 2.0) -> np.ndarray:
    """Fractal sum of value noise: lattice values U(-1,1), quintic-smoothed
    trilinear interpolation (separable), `octaves` octaves."""
    F = np.zeros((D, D, D))
    amp, period = 1.0, float(period0)
    for _ in range(octaves):
        n_lat = int(math.ceil((D - 1) / period)) + 2
        lat = rng.uniform(-1.0, 1.0, (n_lat, n_lat, n_lat))
        M = _interp_matrix(D, period, n_lat)
        t = np.tensordot(M, lat, axes=([1], [0]))          # [D, n, n]
        t = np.tensordot(t, M, axes=([2], [1]))            # [D, n, D]
        t = np.einsum("bj,ajc->abc", M, t, optimize=True)  # [D, D, D]
        F += amp * t
        amp *= gain
        period /= lacunarity
    return F


def fbm_shell(rng: np.random.Generator, D: int, period0: float) -> np.ndarray:
    """Thickened level set F = 0 of an fBm field: |F| < |grad F| (central
    differences), i.e. within about one voxel of the surface on either side."""
    F = fbm_field(rng, D, period0)
    gx, gy, gz = np.gradient(F)
    return np.abs(F) < np.sqrt(gx * gx + gy * gy + gz * gz)


def select_fbm_period(seed: int, D: int = 256, lo: int = 350_000, hi: int = 450_000,
                      target: int = 400_000) -> tuple[int, dict]:
    """The selection rule behind FBM_PERIOD_L: evaluate every candidate base
    period with the same geometry stream; keep the in-range one nearest target."""
    counts = {}
    for p0 in FBM_CANDIDATES:
        counts[p0] = int(fbm_shell(_children(seed)[0], D, p0).sum())
    ok = [p for p in FBM_CANDIDATES if lo <= counts[p] <= hi]
    if not ok:
        raise RuntimeError(f"no fBm base period lands in [{lo},{hi}]: {counts}")
    return min(ok, key=lambda p: abs(counts[p] - target)), counts


def _disc_sheet(rng: np.random.Generator, D: int) -> np.ndarray:
    """Voxels of a thin planar disc: random unit normal n, centre U(40,472)^3
    (scaled to D/512), radius U(24,96); p is in the sheet when |n.(p-c)| < 1/2
    and its in-plane distance to c is below the radius. 20 % of the sheet's
    voxels are then removed at random (holes). Returns int64 [K,3]."""
    sc = D / 512.0
    n = rng.standard_normal(3)
    n /= np.linalg.norm(n)
    c = rng.uniform(40 * sc, 472 * sc, 3)
    r = rng.uniform(24 * sc, 96 * sc)
    ax = int(np.argmax(np.abs(n)))            # solve along the dominant axis
    o1, o2 = [a for a in range(3) if a != ax]
    span = int(math.ceil(r)) + 1
    u = np.arange(int(math.floor(c[o1])) - span, int(math.floor(c[o1])) + span + 2)
    v = np.arange(int(math.floor(c[o2])) - span, int(math.floor(c[o2])) + span + 2)
    U, V = np.meshgrid(u, v, indexing="ij")
    U = U.ravel().astype(np.float64)
    V = V.ravel().astype(np.float64)
    # n.(p-c) = n_ax (w - c_ax) + rest; |.| < 1/2  =>  w in an open interval
    rest = n[o1] * (U - c[o1]) + n[o2] * (V - c[o2])
    w_mid = c[ax] - rest / n[ax]
    half = 0.5 / abs(n[ax])                    # <= sqrt(3)/2 < 1: at most 2 integers
    pts = []
    for dw in (-1, 0, 1):
        W = np.floor(w_mid) + dw
        ok = np.abs(W - w_mid) < half
        P = np.empty((int(ok.sum()), 3))
        P[:, ax] = W[ok]
        P[:, o1] = U[ok]
        P[:, o2] = V[ok]
        pts.append(P)
    P = np.concatenate(pts)
    d = P - c
    along = d @ n
    radial = np.sqrt(np.maximum((d * d).sum(axis=1) - along * along, 0.0))
    P = P[(np.abs(along) < 0.5) & (radial < r)]
    keep = rng.random(P.shape[0]) >= 0.2
    return P[keep].astype(np.int64)


def clustered_object(rng: np.random.Generator, D: int = 512, n_blobs: int = 48,
                     n_sheets: int = 16) -> np.ndarray:
    """Gaussian blobs (dense cores, ragged halos) plus holed thin sheets.

    Blob: centre U(40,472)^3 (scaled to D/512), sigma U(4,12), 5k-25k points
    p = round(c + sigma * N(0, I)). Sheets: `_disc_sheet`. Union, clipped to
    the grid, deduplicated. Returns int64 [K,3] sorted in raster order."""
    sc = D / 512.0
    parts = []
    for _ in range(n_blobs):
        c = rng.uniform(40 * sc, 472 * sc, 3)
        sigma = rng.uniform(4 * sc, 12 * sc)
        k = int(rng.integers(5000, 25001))
        parts.append(np.rint(c + sigma * rng.standard_normal((k, 3))).astype(np.int64))
    for _ in range(n_sheets):
        parts.append(_disc_sheet(rng, D))
    P = np.concatenate(parts)
    P = P[((P >= 0) & (P < D)).all(axis=1)]
    lin = np.unique((P[:, 0] * D + P[:, 1]) * D + P[:, 2])
    return np.stack([lin // (D * D), (lin // D) % D, lin % D], axis=1)


# ----------------------------------------------------------------------------
# Workload assembly
# ----------------------------------------------------------------------------
def _children(seed: int):
    """Independent generators: [geometry, values, ordering]."""
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(3)]


def _occ_to_coords(occ: np.ndarray, b: int) -> np.ndarray:
    xyz = np.argwhere(occ)                     # raster (x, y, z) order
    out = np.empty((xyz.shape[0], 4), dtype=np.int32)
    out[:, 0] = b
    out[:, 1:] = xyz
    return out


def make_coords(name: str, seed: int | None = None) -> np.ndarray:
    """Active voxel coordinates int32 [N,4] (b,x,y,z) of config `name`, in
    raster order (b, then x, y, z lexicographic)."""
    cfg = CONFIGS[name]
    seed = cfg["seed"] if seed is None else seed
    g = _children(seed)[0]
    D, B = cfg["D"], cfg["B"]
    if name == "T":
        return _occ_to_coords(sphere_shell(g, D), 0)
    if name == "S":
        return _occ_to_coords(ellipsoid_object(g, D, 15_000, 25_000), 0)
    if name == "W":
        subs = [np.random.Generator(np.random.PCG64(s))
                for s in np.random.SeedSequence(seed).spawn(4)[3].spawn(B)]
        return np.concatenate([_occ_to_coords(ellipsoid_object(subs[b], D, 15_000, 30_000), b)
                               for b in range(B)])
    if name == "L":
        return _occ_to_coords(fbm_shell(g, D, FBM_PERIOD_L), 0)
    if name == "X":
        subs = [np.random.Generator(np.random.PCG64(s))
                for s in np.random.SeedSequence(seed).spawn(4)[3].spawn(B)]
        out = []
        for b in range(B):
            xyz = clustered_object(subs[b], D)
            c = np.empty((xyz.shape[0], 4), dtype=np.int32)
            c[:, 0] = b
            c[:, 1:] = xyz
            out.append(c)
        return np.concatenate(out)
    raise KeyError(name)


def round_to_f16(a: np.ndarray) -> np.ndarray:
    """Nearest-even rounding to IEEE half precision (numpy's own conversion),
    returned as float32."""
    return np.asarray(a, dtype=np.float32).astype(np.float16).astype(np.float32)


# dtype -> (rounding of x, rounding of w). "mixed-bf16" / "mixed-f16": fp32
# features with half-precision weights.
_ROUNDINGS = {
    "f32": (None, None),
    "bf16": (round_to_bf16, round_to_bf16),
    "f16": (round_to_f16, round_to_f16),
    "mixed-bf16": (None, round_to_bf16),
    "mixed-f16": (None, round_to_f16),
}


def make_values(n: int, c_in: int, c_out: int, dtype: str, rng: np.random.Generator):
    """Features N(0,1) [n, c_in]; weights N(0, 1/(27 c_in)) [27, c_in, c_out];
    each rounded (nearest-even) to the type `dtype` gives it. float32 arrays."""
    if dtype not in _ROUNDINGS:
        raise ValueError(dtype)
    x = rng.standard_normal((n, c_in), dtype=np.float32)
    w = rng.standard_normal((27, c_in, c_out), dtype=np.float32)
    w *= np.float32(1.0 / math.sqrt(27.0 * c_in))
    rx, rw = _ROUNDINGS[dtype]
    if rx is not None:
        x = rx(x)
    if rw is not None:
        w = rw(w)
    return x, w


def make_epilogue(n: int, c_out: int, out_dtype: str, rng: np.random.Generator):
    """Bias N(0, 1/4) [c_out] (float32) and residual N(0, 1) [n, c_out], the
    residual rounded to out_dtype ('f32', 'bf16' or 'f16')."""
    bias = (rng.standard_normal(c_out, dtype=np.float32) * np.float32(0.5)).astype(np.float32)
    res = rng.standard_normal((n, c_out), dtype=np.float32)
    rx = _ROUNDINGS[out_dtype][0]
    return bias, (res if rx is None else rx(res))


def make(name: str, seed_offset: int = 0, order: str = "raster",
         with_values: bool = True, dtype: str | None = None) -> Workload:
    """Config `name` with seed = base seed + seed_offset. order='shuffled'
    applies a seeded random row permutation to the coordinates (values are
    drawn after ordering, row i of x belongs to row i of coords)."""
    cfg = CONFIGS[name]
    seed = cfg["seed"] + seed_offset
    coords = make_coords(name, seed)
    _, vg, og = _children(seed)
    if order == "shuffled":
        coords = coords[og.permutation(coords.shape[0])]
    elif order != "raster":
        raise ValueError(order)
    dt = dtype or cfg["dtype"]
    wl = Workload(name=name, D=cfg["D"], B=cfg["B"], c_in=cfg["c_in"], c_out=cfg["c_out"],
                  dtype=dt, seed=seed, order=order, coords=np.ascontiguousarray(coords))
    if with_values:
        wl.x, wl.w = make_values(wl.n, wl.c_in, wl.c_out, dt, vg)
    return wl


def custom(coords: np.ndarray, c_in: int, c_out: int, dtype: str, seed: int) -> Workload:
    """Values for caller-supplied coordinates (edge-case tests)."""
    coords = np.ascontiguousarray(coords, dtype=np.int32).reshape(-1, 4)
    _, vg, _ = _children(seed)
    wl = Workload(name="custom", D=0, B=0, c_in=c_in, c_out=c_out, dtype=dtype, seed=seed,
                  order="given", coords=coords)
    wl.x, wl.w = make_values(wl.n, c_in, c_out, dtype, vg)
    return wl


def full_cube(n: int, b: int = 0, origin=(0, 0, 0)) -> np.ndarray:
    """All voxels of an n^3 cube (raster order)."""
    r = np.arange(n)
    X, Y, Z = np.meshgrid(r, r, r, indexing="ij")
    c = np.stack([np.full(n ** 3, b), X.ravel() + origin[0], Y.ravel() + origin[1],
                  Z.ravel() + origin[2]], axis=1)
    return c.astype(np.int32)


def random_sparse(rng: np.random.Generator, n: int, D: int, B: int = 1) -> np.ndarray:
    """n distinct uniformly random voxels in B objects of a D^3 grid."""
    lin = rng.choice(B * D ** 3, size=n, replace=False)
    c = np.stack([lin // D ** 3, (lin // D ** 2) % D, (lin // D) % D, lin % D], axis=1)
    return c.astype(np.int32)
