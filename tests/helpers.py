"""Shared helpers of the test suite (no test functions here)."""
from __future__ import annotations

import sys

import numpy as np

# Tolerances of the feature comparison: max relative error, with the
# denominator floored at 1e-2 * rms(y) so that outputs that cancel to about
# zero do not turn fp32 accumulation noise into an unbounded ratio.
# fp16 outputs: one rounding to 11 significant bits (relative error <= 2^-11,
# about 4.9e-4) plus fp32 accumulation noise, with a 4x margin.
TOL = {"bf16": 2e-2, "f16": 2e-3, "f32": 1e-4}


def tol_f32(k_products: int) -> float:
    """fp32 outputs: 1e-4 holds for the 27 * 8 = 216 products per output of the
    fp32 workload; fp32 accumulation error grows like the square root of the
    number of products summed (a random walk of roundings), so longer sums get
    1e-4 * sqrt(K / 216)."""
    return 1e-4 * max(1.0, (k_products / 216.0) ** 0.5)


def max_rel(got: np.ndarray, ref: np.ndarray, rms: float | None = None) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    if rms is None:
        rms = float(np.sqrt(np.mean(ref * ref)))
    floor = max(1e-2 * rms, 1e-300)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), floor)))


def say(*a) -> None:
    """Print and flush, so the case is named before a GPU step starts."""
    print(*a, flush=True)
    sys.stdout.flush()


def morton_keys_numpy(coords: np.ndarray) -> np.ndarray:
    """Z-order keys written independently of the library: bit i of x, y, z goes
    to bit 3i+2, 3i+1, 3i of the low 48 bits; b above them."""
    c = coords.astype(np.uint64)
    key = c[:, 0] << np.uint64(48)
    for i in range(16):
        bit = np.uint64(i)
        key |= ((c[:, 1] >> bit) & np.uint64(1)) << np.uint64(3 * i + 2)
        key |= ((c[:, 2] >> bit) & np.uint64(1)) << np.uint64(3 * i + 1)
        key |= ((c[:, 3] >> bit) & np.uint64(1)) << np.uint64(3 * i)
    return key


def sample_rows(n: int, k: int, seed: int) -> np.ndarray:
    """First rows, last rows (ragged tail) and a random sample."""
    rng = np.random.default_rng(seed)
    head = np.arange(min(n, 64))
    tail = np.arange(max(0, n - 300), n)
    rnd = rng.choice(n, size=min(n, k), replace=False) if n else np.zeros(0, np.int64)
    return np.unique(np.concatenate([head, tail, rnd])).astype(np.int64)
