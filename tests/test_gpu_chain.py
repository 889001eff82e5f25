"""A whole decoder level end to end, against the oracle's composition of the
same steps.

The level: subdivide the coarse voxels (all children, or a seeded subset),
move the coarse features to the children (Channel2Spatial), build the hash and
kernel map of the fine set once, then residual blocks of two fused fp16
convolutions, h = silu(conv(x) + b1), x = conv(h) + b2 + x. The library runs it
exactly as the benchmark's decoder level does. The oracle runs the same steps
in fp64 and rounds every stored intermediate to fp16, as the level stores them,
so the two differ only where an fp32 and an fp64 sum round to different fp16
values (one unit). A unit flipped in one layer reaches the next as an absolute
error on the scale of the features, not of the element it lands on, so each
element is compared against max(|ref|, rms(ref)): elements near zero carry the
propagated error of their neighbours. Per fp16 rounding on the path (one per
convolution) the tolerance is the single-output bound tests.helpers.TOL["f16"];
an fp32-accumulating numpy model of the same level stays at 2.3e-3 (2 blocks)
and 1.0e-3 (1 block) against those 8e-3 and 4e-3.
"""
import numpy as np
import pytest
import torch

import oracle
from gen import workloads as W
from tests.helpers import TOL, say

pytestmark = pytest.mark.gpu

sc = pytest.importorskip("submanifold_sparse_conv_amd")
DEV = "cuda:0"


def rel_to_scale(got, ref):
    """max |got - ref| / max(|ref|, rms(ref)) over all elements."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), rms)))


def level_params(n_coarse, ch, blocks, seed):
    rng = np.random.default_rng(seed)
    xc = W.round_to_f16(rng.standard_normal((n_coarse, 8 * ch)).astype(np.float32))
    ws = [W.round_to_f16((rng.standard_normal((27, ch, ch)) / np.sqrt(27 * ch)).astype(np.float32))
          for _ in range(2 * blocks)]
    bs = [(rng.standard_normal(ch) * 0.1).astype(np.float32) for _ in range(2 * blocks)]
    return xc, ws, bs


def oracle_level(coarse, keep, xc, ws, bs):
    fine, children = oracle.subdivide(coarse, keep)
    x = W.round_to_f16(oracle.channel2spatial(children, xc, len(fine)))
    nbr = oracle.kernel_map(fine)
    for b in range(len(ws) // 2):
        h = W.round_to_f16(oracle.epilogue(oracle.forward(nbr, x, ws[2 * b]), bias=bs[2 * b], act="silu"))
        x = W.round_to_f16(oracle.epilogue(oracle.forward(nbr, h, ws[2 * b + 1]), bias=bs[2 * b + 1],
                                           residual=x))
    return fine, children, x


def library_level(coarse, keep, xc, ws, bs):
    fine, children = sc.subdivide(coarse, keep)
    x = sc.channel2spatial(children, xc, int(fine.shape[0]))
    m = sc.build_kernel_map(sc.build_hash(fine))
    t = torch.empty_like(x)
    for b in range(len(ws) // 2):
        sc.forward_fused(m, x, ws[2 * b], bias=bs[2 * b], act="silu", out=t)
        sc.forward_fused(m, t, ws[2 * b + 1], bias=bs[2 * b + 1], residual=x, out=x)
    return fine, children, x


@pytest.mark.parametrize("coarse_src,ch,blocks,pruned", [("S", 32, 2, False), ("S", 64, 1, True),
                                                         ("grid", 16, 2, True)])
def test_decoder_level_end_to_end(coarse_src, ch, blocks, pruned):
    rng = np.random.default_rng(40 + ch)
    if coarse_src == "S":
        coarse = W.make("S", with_values=False).coords
    else:
        lin = rng.choice(2 * 20 ** 3, size=3000, replace=False)
        coarse = np.stack([lin // 8000, (lin // 400) % 20, (lin // 20) % 20, lin % 20], 1).astype(np.int32)
    n = len(coarse)
    keep = rng.integers(1, 256, size=n).astype(np.uint8) if pruned else None
    xc, ws, bs = level_params(n, ch, blocks, seed=50 + ch)
    say(f"[chain] coarse={coarse_src} n={n} ch={ch} blocks={blocks} pruned={pruned}")
    fine_o, children_o, y_o = oracle_level(coarse, keep, xc, ws, bs)

    d = torch.device(DEV)
    fine, children, y = library_level(
        torch.from_numpy(coarse).to(d), None if keep is None else torch.from_numpy(keep).to(d),
        torch.from_numpy(xc).to(d).half(),
        [sc.pack_weights(torch.from_numpy(w).to(d).half()) for w in ws],
        [torch.from_numpy(b).to(d) for b in bs])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(fine.cpu().numpy(), fine_o)
    np.testing.assert_array_equal(children.cpu().numpy(), children_o)
    err = rel_to_scale(y.float().cpu().numpy(), y_o)
    tol = 2 * blocks * TOL["f16"]
    say(f"    fine={len(fine_o)} err={err:.3e} (tol {tol:.1e})")
    assert err <= tol
    # The comparison is sharp enough to see a dropped block: the level's output
    # without its last block is far outside the tolerance.
    assert rel_to_scale(oracle_level(coarse, keep, xc, ws[:-2], bs[:-2])[2], y_o) > 10 * tol
