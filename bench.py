#!/usr/bin/env python3
"""Benchmark of the submanifold sparse 3D convolution hot path on one MI355X.

One step = the whole path over one synthetic voxel set: build_hash (Morton
order + open-addressing table of 4x4x4 blocks, given the workload's grid;
`hash_without_grid_ms` times the build without it), build_kernel_map (27
neighbours per voxel),
pack_weights and the gather-GEMM (forward_packed). Inputs are resident in HBM
before the timed region. Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--config L] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP32_VECTOR_TFLOPS = 157.3  # MI355X fp32 vector (256 CUs, 2.4 GHz)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_mfma.json")
# the gather-GEMM kernel and the headers it includes: counters taken on other sources are stale
GEMM_SOURCES = [os.path.join(ROOT, "submanifold_sparse_conv_amd", "csrc", f)
                for f in ("gemm_mfma.hip", "common.h", "launch.h", "halo_plan.h")]

WORKLOAD_NAMES = {
    "T": "16^3 sphere shell (radius 6, thickness 1), C 8->8 fp32",
    "S": "64^3 union of 3 ellipsoid shells (thickness 2), C 64->64 bf16",
    "W": "64^3 x 4 objects, ellipsoid shells, C 1024->1024 bf16",
    "L": "256^3 thickened fBm level set (thickness 2), C 128->128 bf16",
    "X": "512^3 x 2 objects, Gaussian blobs + holed sheets, C 64->32 bf16",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # The GPU needs on the order of 0.1 s of sustained load to reach its steady
    # clocks: 50 warm-up steps, then 200 timed steps (about 0.15 s) by default.
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--config", default="L", choices=list(WORKLOAD_NAMES))
    p.add_argument("--also", default="T,S,W,X",
                   help="other configs measured the same way (path phases + steady forward), comma list ('' = none)")
    p.add_argument("--no-ceilings", action="store_true", help="skip the measured MFMA / copy ceilings")
    p.add_argument("--no-wide-keys", action="store_true", help="skip the hash build over keys with > 33 varying bits")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-variants", action="store_true",
                   help="skip the fused-epilogue / fp16 / mixed-precision / backward timings")
    p.add_argument("--no-chain", action="store_true", help="skip the decoder-level layer chain")
    p.add_argument("--chain-blocks", type=int, default=4)
    p.add_argument("--chain-channels", type=int, default=64)
    p.add_argument("--cpu-seconds", type=float, default=8.0, help="target wall time of the oracle forward sample")
    p.add_argument("--gemm-reps", type=int, default=50)
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


def copy_probe(mib):
    """A plain device-to-device copy of known size, the reference that scales
    the HBM byte counters (FETCH_SIZE / WRITE_SIZE) of the profiled kernels."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "reps": 5}))


def sha_of(paths):
    """SHA-256 of the files' bytes, concatenated in the order given."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def to_device(wl, torch):
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    c = torch.from_numpy(wl.coords).cuda()
    x = torch.from_numpy(wl.x).cuda().to(dt)
    w = torch.from_numpy(wl.w).cuda().to(dt)
    return c, x, w


class TimingEvent:
    """A HIP event created with hipEventDisableSystemFence, recorded on torch's
    current stream (the stream the library launches on). A default event
    (torch.cuda.Event) makes its record a system-scope release with a cache
    write-back: measured between the path's kernels, about 3.5 us of GPU time
    per record, against about 1.5 us for this one."""
    _hip = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._c = ctypes
        self.e = ctypes.c_void_p()
        st = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.e), ctypes.c_uint(self.FLAGS))
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self):
        import torch
        st = TimingEvent._hip.hipEventRecord(self.e, self._c.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_time(self, end) -> float:
        ms = self._c.c_float()
        st = TimingEvent._hip.hipEventElapsedTime(self._c.byref(ms), self.e, end.e)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def __del__(self):
        if TimingEvent._hip is not None and self.e:
            TimingEvent._hip.hipEventDestroy(self.e)


def grid_of(wl):
    """(log2 of the grid side, object count) of a workload: the grid its
    coordinates lie in, which the hash build is given."""
    g = max(int(wl.D - 1).bit_length(), 2)
    return g, max(int(wl.B), 1)


class Path:
    """Pre-allocated buffers and one step of the hot path. The hash is built
    with the workload's grid (build_hash(grid_log2=..., batch=...)), as a
    decoder level knows its resolution."""

    def __init__(self, sc, torch, coords, x, w, grid):
        self.sc, self.torch = sc, torch
        self.coords, self.x, self.w = coords, x, w
        self.grid = grid
        n = int(coords.shape[0])
        L = sc._lib.lib()
        self.hws = sc.Workspace(L.tr_sparseconv_hash_grid_workspace_bytes(n, grid[0], grid[1]), coords.device)
        self.kws = sc.Workspace(L.tr_sparseconv_kmap_workspace_bytes(n), coords.device)
        self.nbr = torch.empty((n, 27), dtype=torch.int32, device=coords.device)
        self.y = torch.empty((n, int(w.shape[2])), dtype=x.dtype, device=x.device)
        self.h = self.m = self.wp = None

    def step(self, ev=None, gemm_ev=None):
        """ev: five events around the four phases; gemm_ev: two events around
        the gather-GEMM only."""
        sc = self.sc
        if ev is not None:
            ev[0].record()
        self.h = sc.build_hash(self.coords, check_status=False, workspace=self.hws, grid_log2=self.grid[0],
                               batch=self.grid[1])
        if ev is not None:
            ev[1].record()
        self.m = sc.build_kernel_map(self.h, nbr=self.nbr, workspace=self.kws)
        if ev is not None:
            ev[2].record()
        self.wp = sc.pack_weights(self.w)
        if ev is not None:
            ev[3].record()
        if gemm_ev is not None:
            gemm_ev[0].record()
        sc.forward_packed(self.m, self.x, self.wp, out=self.y)
        if gemm_ev is not None:
            gemm_ev[1].record()
        if ev is not None:
            ev[4].record()


def pairs_of(nbr_t):
    return int((nbr_t >= 0).sum().item())


def measure_forward_only(sc, torch, path, reps):
    """Back-to-back gather-GEMM launches between two events (steady state,
    after 2 x reps untimed launches)."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2 * reps):
        sc.forward_packed(path.m, path.x, path.wp, out=path.y)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        sc.forward_packed(path.m, path.x, path.wp, out=path.y)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def time_reps(torch, fn, reps):
    """Mean ms of `fn` launched back to back between two events (after reps
    untimed calls)."""
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def variants(sc, torch, wl, path, M, reps):
    """The other precision paths, the fused epilogue and the backward, on the
    same kernel map: steady-state ms and effective TFLOP/s (2 C_in C_out M
    useful flops per call)."""
    n, ci, co = wl.n, wl.c_in, wl.c_out
    flops = 2.0 * ci * co * M
    g = torch.Generator(device="cuda").manual_seed(7)
    bias = torch.randn(co, device="cuda", generator=g) * 0.5
    res = torch.randn((n, co), device="cuda", generator=g).bfloat16()
    dy = torch.randn((n, co), device="cuda", generator=g).bfloat16()
    x16, w16 = path.x.half(), path.w.half()
    wp16 = sc.pack_weights(w16)
    xf = torch.randn((n, ci), device="cuda", generator=g)
    wpd = sc.pack_weights_dgrad(path.w)
    y_f32 = torch.empty((n, co), device="cuda")
    dx = torch.empty((n, ci), device="cuda", dtype=torch.bfloat16)
    dw = torch.empty((27, ci, co), device="cuda")
    y16 = torch.empty((n, co), device="cuda", dtype=torch.float16)
    wsw = sc.Workspace(sc._lib.lib().tr_sparseconv_backward_weights_workspace_bytes(n, ci, co, sc._lib.BF16),
                       "cuda")
    cases = {
        "forward_bf16_bias_silu_residual": lambda: sc.forward_fused(path.m, path.x, path.wp, bias=bias, act="silu",
                                                                    residual=res, out=path.y),
        "forward_f16": lambda: sc.forward_packed(path.m, x16, wp16, out=y16),
        "forward_f32x_bf16w_f32y": lambda: sc.forward_fused(path.m, xf, path.wp, out=y_f32),
        "backward_data_bf16": lambda: sc.backward_data(path.m, dy, wpd, out=dx),
        "backward_weights_bf16": lambda: sc.backward_weights(path.m, path.x, dy, out=dw, workspace=wsw),
    }
    out = {}
    for name, fn in cases.items():
        ms = time_reps(torch, fn, reps)
        out[name] = {"ms": ms, "effective_tflops": flops / (ms * 1e-3) / 1e12}
    return out


def layer_chain(sc, torch, wl, blocks, ch, reps=5):
    """A decoder level: the coarse voxel set subdivided with every child kept
    (Channel2Spatial step: 8x the voxels at twice the resolution), then one
    hash + kernel map and `blocks` residual blocks of two fp16 convolutions,
    h = silu(conv(x) + b1), x = conv(h) + b2 + x, epilogues fused. Times the
    whole level (subdivide + regroup + map + convs) and its parts."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cuda").manual_seed(11)
    coarse = torch.from_numpy(wl.coords).to(dev)
    xc = (torch.randn((wl.n, 8 * ch), device=dev, generator=g)).half()
    ws = [sc.pack_weights((torch.randn((27, ch, ch), device=dev, generator=g) / (27 * ch) ** 0.5).half())
          for _ in range(2 * blocks)]
    bs = [torch.randn(ch, device=dev, generator=g) * 0.1 for _ in range(2 * blocks)]

    fg, fb = grid_of(wl)[0] + 1, grid_of(wl)[1]  # the fine level: twice the side

    def level():
        fine, children = sc.subdivide(coarse)
        x = sc.channel2spatial(children, xc, int(fine.shape[0]))
        h = sc.build_hash(fine, check_status=False, grid_log2=fg, batch=fb)
        m = sc.build_kernel_map(h)
        t = torch.empty_like(x)
        for b in range(blocks):
            sc.forward_fused(m, x, ws[2 * b], bias=bs[2 * b], act="silu", out=t)
            sc.forward_fused(m, t, ws[2 * b + 1], bias=bs[2 * b + 1], residual=x, out=x)
        return fine, children, m, x

    fine, children, m, x = level()
    torch.cuda.synchronize()
    nf = int(fine.shape[0])
    M = pairs_of(m.nbr)
    t_level = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        level()
        torch.cuda.synchronize()
        t_level.append((time.perf_counter() - t0) * 1e3)
    t_map = time_reps(torch, lambda: sc.build_kernel_map(sc.build_hash(fine, check_status=False, grid_log2=fg,
                                                                        batch=fb)), reps)
    t = torch.empty_like(x)
    t_conv = time_reps(torch, lambda: sc.forward_fused(m, x, ws[0], bias=bs[0], act="silu", out=t), 4 * reps)
    flops = 2.0 * ch * ch * M
    # The level moves on their own (subdivide and downsample include the read-back
    # of the produced row count), against their algorithmic bytes.
    nc = wl.n
    hf = sc.build_hash(fine, check_status=False)
    xf2, xc2 = torch.empty_like(x), torch.empty_like(xc)
    moves = {
        "subdivide": (lambda: sc.subdivide(coarse), nc * 16 + nf * 16 + nc * 32),
        "channel2spatial": (lambda: sc.channel2spatial(children, xc, nf, out=xf2),
                            nc * 8 * ch * 2 + nc * 32 + nf * ch * 2),
        "downsample": (lambda: sc.downsample(hf), nf * 12 + nc * 48),
        "spatial2channel": (lambda: sc.spatial2channel(children, x, out=xc2),
                            nf * ch * 2 + nc * 32 + nc * 8 * ch * 2),
    }
    levels = {}
    for name, (fn, nbytes) in moves.items():
        ms = time_reps(torch, fn, reps)
        gbs = nbytes / (ms * 1e-3) / 1e9
        levels[name] = {"ms": ms, "algorithmic_bytes": nbytes, "gbs": gbs, "frac_hbm": gbs / PEAK_HBM_GBS}
    return {"workload": f"256^3 fBm shell subdivided (all children kept) -> {nf} voxels at 512^3, "
                        f"{blocks} residual blocks of two 3x3x3 convs, C {ch}->{ch} fp16",
            "n_voxels": nf, "pairs_M": M, "convs": 2 * blocks,
            "ms_level": float(np.median(t_level)),
            "ms_hash_and_map": t_map, "ms_per_conv": t_conv,
            "map_share_of_level": t_map / float(np.median(t_level)),
            "conv_effective_tflops": flops / (t_conv * 1e-3) / 1e12,
            "voxel_layers_per_s": nf * 2 * blocks / (float(np.median(t_level)) * 1e-3),
            "level_moves": levels}


def cpu_baseline(wl, target_s):
    """The oracle (plain C++, unordered_map + fp64 direct sum) on the host
    cores: full map build and kernel map, fp64 forward on a timed random
    sample of rows, scaled to all rows."""
    import oracle
    t0 = time.perf_counter()
    table = oracle.Table(wl.coords)
    t1 = time.perf_counter()
    nbr = table.kernel_map()
    t2 = time.perf_counter()
    rng = np.random.default_rng(12345)
    probe = rng.choice(wl.n, size=min(wl.n, 2000), replace=False)
    tp = time.perf_counter()
    oracle.forward(nbr, wl.x, wl.w, rows=probe)
    rate = len(probe) / max(time.perf_counter() - tp, 1e-9)
    k = int(min(wl.n, max(2000, rate * target_s)))
    rows = rng.choice(wl.n, size=k, replace=False)
    t3 = time.perf_counter()
    oracle.forward(nbr, wl.x, wl.w, rows=rows)
    t4 = time.perf_counter()
    t_fwd_all = (t4 - t3) * wl.n / k
    total = (t1 - t0) + (t2 - t1) + t_fwd_all
    return {
        "value": wl.n / total,
        "unit": "voxels/s",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": (f"full unordered_map build ({t1 - t0:.2f} s, serial) and kernel map "
                   f"({t2 - t1:.2f} s) over all {wl.n} voxels; fp64 forward over {k} random rows "
                   f"({t4 - t3:.2f} s) scaled to all rows ({t_fwd_all:.2f} s)"),
    }


def wide_keys(sc, torch, wl, reps=5):
    """build_hash over keys with many varying bits: the voxels of the workload
    spread over 64 object ids whose values span 16 bits (b = (row % 64) *
    1021), so 16 + 24 = 40 key bits vary and the sort needs four radix passes
    (bits beyond four 11-bit digits, 44, would go to a single-workgroup pass)."""
    c = wl.coords.copy()
    c[:, 0] = (np.arange(wl.n) % 64) * 1021
    vary = np.bitwise_or.reduce(c, axis=0) ^ np.bitwise_and.reduce(c, axis=0)
    nbits = int(sum(bin(int(v)).count("1") for v in vary))
    cd = torch.from_numpy(c).cuda()
    ws = sc.Workspace(sc._lib.lib().tr_sparseconv_hash_workspace_bytes(wl.n), cd.device)
    sc.build_hash(cd, workspace=ws)  # checks the status once
    ms = time_reps(torch, lambda: sc.build_hash(cd, check_status=False, workspace=ws), reps)
    return {"n_voxels": wl.n, "varying_key_bits": nbits, "radix_passes": min(4, (nbits + 10) // 11),
            "bits_in_single_workgroup_pass": max(0, nbits - 44),
            "ms_build_hash": ms}


def block_count(coords):
    """Occupied 4x4x4 blocks of a voxel set (per object)."""
    c = coords.astype(np.int64)
    return int(np.unique(((c[:, 0] * 16384 + (c[:, 1] >> 2)) * 16384 + (c[:, 2] >> 2)) * 16384
                         + (c[:, 3] >> 2)).size)


def hash_map_bytes(n, nblocks):
    """Algorithmic bytes of the topology passes under two conventions.

    "block table" (what this library moves): hash = coordinates read (16 B) +
    sorted key and row written (12 B) per voxel + one 32-byte slot per occupied
    4x4x4 block; map = sorted key and row read, the row order read once more,
    nbr (108 B), mask and the tile order (row + mask) written per voxel, the
    block table read once.
    "per-voxel table" (a table of P = pow2 >= 2N slots of 12 B, as a one-slot-
    per-voxel hash would move): hash = 16 + 12 B per voxel + 12 B per slot; map
    = 12 B per voxel read + the table read + nbr (108 B) and mask (4 B) written.
    """
    P = 1
    while P < 2 * max(n, 1):
        P *= 2
    blk = {"hash": 16 * n + 12 * n + 32 * nblocks,
           "map": 12 * n + 4 * n + 32 * nblocks + 108 * n + 4 * n + 8 * n}
    vox = {"hash": 16 * n + 12 * n + 12 * P, "map": 12 * n + 12 * P + 108 * n + 4 * n}
    return blk, vox


def hash_without_grid(sc, torch, coords, reps=50):
    """build_hash over the same voxels without the grid (the radix-sorted
    build), ms back to back."""
    L = sc._lib.lib()
    ws = sc.Workspace(L.tr_sparseconv_hash_workspace_bytes(int(coords.shape[0])), coords.device)
    return time_reps(torch, lambda: sc.build_hash(coords, check_status=False, workspace=ws), reps)


def config_record(name, wl, M, phases, t_fwd_steady, t_hash_no_grid=None):
    """One config's path phases (ms), steady forward, effective TFLOP/s and
    fraction of the peak of its arithmetic, and the topology passes' GB/s."""
    t_hash, t_map, t_pack, t_gemm = (float(v) for v in phases)
    flops = 2.0 * wl.c_in * wl.c_out * M
    tf = flops / (t_fwd_steady * 1e-3) / 1e12
    half = wl.dtype == "bf16"
    blk, vox = hash_map_bytes(wl.n, block_count(wl.coords))
    t_hm = (t_hash + t_map) * 1e-3

    def gbs(b):
        return {"bytes": b["hash"] + b["map"], "gbs": (b["hash"] + b["map"]) / t_hm / 1e9,
                "frac": (b["hash"] + b["map"]) / t_hm / 1e9 / PEAK_HBM_GBS,
                "hash_gbs": b["hash"] / (t_hash * 1e-3) / 1e9, "map_gbs": b["map"] / (t_map * 1e-3) / 1e9}
    return {"workload": WORKLOAD_NAMES[name], "n_voxels": wl.n, "pairs_M": M, "c_in": wl.c_in,
            "c_out": wl.c_out, "dtype": "bf16" if half else "f32",
            "grid": {"log2_side": grid_of(wl)[0], "objects": grid_of(wl)[1]},
            "ms": {"build_hash": t_hash, "build_kernel_map": t_map, "pack_weights": t_pack,
                   "gather_gemm_in_path": t_gemm, "forward_steady": t_fwd_steady,
                   "build_hash_without_grid": t_hash_no_grid},
            "voxels_per_s_path": wl.n / ((t_hash + t_map + t_pack + t_gemm) * 1e-3),
            "voxels_per_s_forward": wl.n / (t_fwd_steady * 1e-3),
            "effective_tflops": tf,
            "peak_tflops": PEAK_BF16_TFLOPS if half else PEAK_FP32_VECTOR_TFLOPS,
            "frac_peak": tf / (PEAK_BF16_TFLOPS if half else PEAK_FP32_VECTOR_TFLOPS),
            "hash_map_hbm": {"block_table": gbs(blk), "per_voxel_table": gbs(vox)}}


def measure_ceilings(sc, torch):
    """The chip's measured ceilings beside the published peaks: a loop of
    independent bf16 32x32x16 matrix multiply-accumulates, and a 1 GiB
    device-to-device streaming copy (best of five launches each)."""
    import ctypes
    L = sc._lib.lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    grid, iters = 4096, 2000
    buf = torch.empty(grid * 256, device="cuda")
    flops = L.tr_sparseconv_ceiling_mfma_flops(grid, iters)

    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            ts.append(s.elapsed_time(e))
        return min(ts)
    ms_m = best(lambda: sc.check(L.tr_sparseconv_ceiling_mfma(ctypes.c_void_p(buf.data_ptr()), grid, iters, st)))
    nbytes = 1 << 30
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    ms_c = best(lambda: sc.check(L.tr_sparseconv_ceiling_copy(ctypes.c_void_p(a.data_ptr()),
                                                               ctypes.c_void_p(b.data_ptr()), nbytes, 1024, st)))
    mfma = flops / (ms_m * 1e-3) / 1e12
    copy = 2 * nbytes / (ms_c * 1e-3) / 1e9
    return {"mfma_bf16_tflops": {"measured": mfma, "spec": PEAK_BF16_TFLOPS, "frac_of_spec": mfma / PEAK_BF16_TFLOPS,
                                 "probe": f"{grid} x 4 waves x {iters} x 4 v_mfma_f32_32x32x16_bf16"},
            "hbm_gbs": {"measured": copy, "spec": PEAK_HBM_GBS, "frac_of_spec": copy / PEAK_HBM_GBS,
                        "probe": "1 GiB device copy, 16-byte accesses, bytes read + written"}}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def note(msg):
    """One progress line per finished phase, on stderr (the JSON line stays alone on stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def traffic_entry():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current gather-GEMM source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != sha_of(GEMM_SOURCES):
        return None
    return t.get("bytes_per_launch")


def main():
    args = parse()
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the path is built "
              "and measured for a single GPU; sharding it across GPUs is not built.", file=sys.stderr)
        sys.exit(2)
    import torch
    import submanifold_sparse_conv_amd as sc
    from gen import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = W.make(args.config)
    coords, x, w = to_device(wl, torch)
    path = Path(sc, torch, coords, x, w, grid_of(wl))
    for _ in range(args.warmup):
        path.step()
    torch.cuda.synchronize()
    note(f"{args.warmup} warm-up steps done")
    M = pairs_of(path.nbr)
    assert bool((path.nbr[:, 13] == torch.arange(wl.n, device=dev, dtype=torch.int32)).all())

    # The timed region: K whole steps, with two events per step around the
    # gather-GEMM only (its live per-launch duration for the roofline).
    gev = [[TimingEvent() for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        path.step(gemm_ev=gev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    t_gemm = float(np.mean([gev[i][0].elapsed_time(gev[i][1]) for i in range(args.steps)]))
    assert bool(torch.isfinite(path.y.float()).all())
    note(f"{args.steps} timed steps: {ms_step:.4f} ms per step")
    # The split of a step into its phases, from a separate run of the same steps
    # with events between the phases (outside the timed region: each event
    # record still adds a little GPU time).
    n_split = min(args.steps, 100)
    evs = [[TimingEvent() for _ in range(5)] for _ in range(n_split)]
    for i in range(n_split):
        path.step(evs[i])
    torch.cuda.synchronize()
    ph = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(4)] for i in range(n_split)])
    t_hash, t_map, t_pack, _ = ph.mean(axis=0)

    flops = 2.0 * wl.c_in * wl.c_out * M
    gemm_tflops = flops / (t_gemm * 1e-3) / 1e12
    # --gemm-reps 0 skips the back-to-back forward launches (profiling runs, where
    # the per-kernel average must cover the timed steps' launches only)
    t_gemm_ss = measure_forward_only(sc, torch, path, args.gemm_reps) if args.gemm_reps > 0 else t_gemm

    # the committed counters were taken on the 256^3 config's launch
    traffic = traffic_entry() if args.config == "L" else None
    main_cfg = config_record(args.config, wl, M, (t_hash, t_map, t_pack, t_gemm), t_gemm_ss,
                             hash_without_grid(sc, torch, coords))
    if wl.dtype == "bf16":
        roof = {"kernel": "fwd_halo (gather-GEMM over LDS-staged halo rows)", "bound": "mfma", "achieved": gemm_tflops,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": gemm_tflops / PEAK_BF16_TFLOPS,
                "traffic": traffic}
    else:  # fp32 features and weights: the plain FMA kernel
        roof = {"kernel": "fwd_simple (fp32 FMA)", "bound": "alu", "achieved": gemm_tflops,
                "peak": PEAK_FP32_VECTOR_TFLOPS, "unit": "TFLOP/s",
                "frac": gemm_tflops / PEAK_FP32_VECTOR_TFLOPS, "traffic": None}

    out = {
        "metric": "sparse-conv voxels/s (whole path: hash + kernel map + gather-GEMM)",
        "value": wl.n / (ms_step * 1e-3),
        "unit": "voxels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.config], "n_voxels": wl.n, "pairs_M": M,
                   "c_in": wl.c_in, "c_out": wl.c_out, "grid": wl.D, "batch": wl.B, "seed": wl.seed},
        "phases_ms": {"build_hash": t_hash, "build_kernel_map": t_map, "pack_weights": t_pack,
                      "gather_gemm": t_gemm},
        "timing": "ms_per_step: host clock over the timed steps (synchronised on both sides); "
                  "gather_gemm: events around each launch in those steps; the other phases: "
                  "events between phases in a separate run of the same steps",
        "forward": {"voxels_per_s_steady": wl.n / (t_gemm_ss * 1e-3), "ms_steady": t_gemm_ss,
                    "effective_tflops": flops / (t_gemm_ss * 1e-3) / 1e12,
                    "frac_bf16_peak": flops / (t_gemm_ss * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "hash_without_grid_ms": main_cfg["ms"]["build_hash_without_grid"],
        "hash_map_hbm": main_cfg["hash_map_hbm"],
        "roofline": roof,
    }
    configs = {args.config: main_cfg}
    for name in [a for a in args.also.split(",") if a and a != args.config]:
        wl2 = W.make(name)
        c2, x2, w2 = to_device(wl2, torch)
        p2 = Path(sc, torch, c2, x2, w2, grid_of(wl2))
        for _ in range(3):
            p2.step()
        torch.cuda.synchronize()
        M2 = pairs_of(p2.nbr)
        reps = 20
        ev = [[TimingEvent() for _ in range(5)] for _ in range(reps)]
        for i in range(reps):
            p2.step(ev[i])
        torch.cuda.synchronize()
        ph2 = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(4)] for i in range(reps)])
        tss = measure_forward_only(sc, torch, p2, args.gemm_reps) if args.gemm_reps > 0 else float(
            np.median(ph2[:, 3]))
        configs[name] = config_record(name, wl2, M2, tuple(np.median(ph2, axis=0)), tss,
                                      hash_without_grid(sc, torch, c2))
        del p2, c2, x2, w2
        note(f"config {name} measured")
    out["configs"] = configs
    if not args.no_ceilings:
        out["ceilings"] = measure_ceilings(sc, torch)
        if wl.dtype == "bf16":
            mp = out["ceilings"]["mfma_bf16_tflops"]["measured"]
            out["roofline"]["measured_peak"] = mp
            out["roofline"]["frac_of_measured_peak"] = gemm_tflops / mp
        note("ceilings measured")
    if args.config == "L" and not args.no_wide_keys:
        out["hash_wide_keys"] = wide_keys(sc, torch, wl)
        note("wide-key hash measured")
    if not args.no_variants and wl.dtype == "bf16":
        out["variants"] = variants(sc, torch, wl, path, M, max(5, args.gemm_reps // 2))
        note("variants measured")
    if not args.no_chain and args.config == "L":
        out["chain"] = layer_chain(sc, torch, wl, args.chain_blocks, args.chain_channels)
        note("layer chain measured")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        note("cpu baseline measured")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
