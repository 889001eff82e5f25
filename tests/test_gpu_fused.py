"""Fused epilogue and mixed precision of the gather-GEMM, against the oracle.

y = round_y(act(conv(x, w) + bias) + residual), with half or fp32 features,
bf16 or fp16 weights and half or fp32 outputs. The oracle computes the same
expression in fp64 from the exactly widened inputs (oracle.forward, then
oracle.epilogue). Tolerances are those of the output type (tests.helpers.TOL).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from gen import workloads as W
from tests.helpers import TOL, max_rel, sample_rows, say, tol_f32

pytestmark = pytest.mark.gpu

sc = pytest.importorskip("submanifold_sparse_conv_amd")
DEV = "cuda:0"
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@functools.lru_cache(maxsize=None)
def grid(n, D, B, seed):
    rng = np.random.default_rng(seed)
    c = W.random_sparse(rng, n, D=D, B=B)
    return c[rng.permutation(len(c))]


SPLIT_TERMS = {("f32", "bf16"): 3, ("f32", "f16"): 2, ("f32", "f32"): 1, ("bf16", "bf16"): 1,
               ("f16", "f16"): 1}


def run_case(coords, c_in, c_out, w_t, x_t, y_t, act, use_bias, use_res, seed, rows=None,
             in_place=False):
    gen = w_t if x_t == w_t else "mixed-" + w_t
    wl = W.custom(coords, c_in, c_out, gen, seed)
    bias, res = W.make_epilogue(wl.n, c_out, y_t, np.random.default_rng(seed + 7))
    say(f"[fused] n={wl.n} c={c_in}->{c_out} w={w_t} x={x_t} y={y_t} act={act} "
        f"bias={use_bias} res={use_res} in_place={in_place} seed={seed}")
    x = torch.from_numpy(wl.x).to(DEV).to(TD[x_t])
    w = torch.from_numpy(wl.w).to(DEV).to(TD[w_t])
    b = torch.from_numpy(bias).to(DEV) if use_bias else None
    r = torch.from_numpy(res).to(DEV).to(TD[y_t]) if use_res else None
    h = sc.build_hash(torch.from_numpy(wl.coords).to(DEV))
    m = sc.build_kernel_map(h)
    wp = sc.pack_weights(w)
    if in_place:
        y = sc.forward_fused(m, x, wp, bias=b, act=act, residual=r, out=r)
        assert y.data_ptr() == r.data_ptr()
    else:
        y = sc.forward_fused(m, x, wp, bias=b, act=act, residual=r, out_dtype=TD[y_t])
    torch.cuda.synchronize()
    assert y.dtype == TD[y_t]
    nbr = m.nbr.cpu().numpy()
    np.testing.assert_array_equal(nbr, oracle.kernel_map(wl.coords))
    if rows is None:
        rows = np.arange(wl.n)
    ref = oracle.epilogue(oracle.forward(nbr, wl.x, wl.w, rows=rows),
                          bias=bias if use_bias else None,
                          residual=res[rows] if use_res else None, act=act)
    got = y.float().cpu().numpy()[rows]
    err = max_rel(got, ref)
    # fp32 features are carried as 3 bf16 / 2 fp16 terms: that many products each
    tol = tol_f32(27 * c_in * SPLIT_TERMS[(x_t, w_t)]) if y_t == "f32" else TOL[y_t]
    say(f"    max_rel={err:.3e} (tol {tol:.2e})")
    assert err <= tol
    return err


EPILOGUES = [("none", False, False), ("relu", True, False), ("silu", True, True), ("none", False, True)]
TYPES = [(w, x, y) for w in ("bf16", "f16") for x in (w, "f32") for y in (w, "f32")]
SHAPES = [(64, 64), (32, 96), (16, 8), (128, 136), (64, 24),  # one shape per output-tile width
          (64, 32), (128, 128)]  # the halo kernel's 32- and 128-column items


@pytest.mark.parametrize("w_t,x_t,y_t", TYPES)
@pytest.mark.parametrize("act,use_bias,use_res", EPILOGUES)
@pytest.mark.parametrize("c_in,c_out", SHAPES)
def test_fused_small(w_t, x_t, y_t, act, use_bias, use_res, c_in, c_out):
    # 1500 random voxels in 2 x 14^3: several 128/256-row tiles and a ragged tail
    run_case(grid(1500, 14, 2, 3), c_in, c_out, w_t, x_t, y_t, act, use_bias, use_res, seed=11)


@pytest.mark.parametrize("w_t,y_t", [("bf16", "bf16"), ("f16", "f16"), ("f16", "f32")])
def test_fused_in_place_residual(w_t, y_t):
    run_case(grid(3000, 20, 1, 4), 64, 64, w_t, w_t, y_t, "silu", True, True, seed=12, in_place=True)


def test_fused_f32_weights():
    # the fp32 path carries the same epilogue
    run_case(grid(700, 12, 1, 5), 8, 24, "f32", "f32", "f32", "silu", True, True, seed=13)
    run_case(grid(700, 12, 1, 5), 3, 5, "f32", "f32", "f32", "relu", True, False, seed=14)


def test_mixed_input_keeps_fp32_precision():
    # fp32 features with bf16 weights and an fp32 output agree with the fp64
    # oracle to fp32 accuracy; rounding the features to bf16 first does not.
    coords = grid(4000, 24, 1, 6)
    err = run_case(coords, 64, 64, "bf16", "f32", "f32", "none", False, False, seed=15)
    wl = W.custom(coords, 64, 64, "mixed-bf16", 15)
    nbr = oracle.kernel_map(wl.coords)
    early = oracle.forward(nbr, W.round_to_bf16(wl.x), wl.w)
    assert max_rel(early, oracle.forward(nbr, wl.x, wl.w)) > 10 * tol_f32(27 * 64 * 3) > 10 * err


@pytest.mark.parametrize("name,w_t,x_t,y_t", [("L", "bf16", "bf16", "bf16"), ("L", "f16", "f16", "f16"),
                                              ("S", "bf16", "f32", "bf16"), ("X", "f16", "f32", "f32")])
def test_fused_config_sizes(name, w_t, x_t, y_t):
    wl = W.make(name, with_values=False)
    rows = sample_rows(wl.n, 3000, wl.seed) if wl.n > 20000 else None
    run_case(wl.coords, wl.c_in, wl.c_out, w_t, x_t, y_t, "silu", True, True, seed=wl.seed + 300,
             rows=rows)


def test_fused_decoder_level():
    # The layer chain's shape: the 256^3 set subdivided with every child kept
    # (3,149,760 voxels at 512^3), C 64->64 fp16, bias + SiLU + residual.
    base = W.make("L", with_values=False).coords.astype(np.int64)
    octs = np.array([[0, o >> 2, (o >> 1) & 1, o & 1] for o in range(8)], np.int64)
    coords = (base[:, None, :] * np.array([1, 2, 2, 2]) + octs[None]).reshape(-1, 4).astype(np.int32)
    rows = sample_rows(len(coords), 3000, 21)
    run_case(coords, 64, 64, "f16", "f16", "f16", "silu", True, True, seed=21, rows=rows)


def test_fp16_identity_bitexact():
    rng = np.random.default_rng(8)
    coords = grid(2000, 16, 1, 7)
    x = torch.from_numpy(W.round_to_f16(rng.standard_normal((len(coords), 64)).astype(np.float32)))
    w = torch.zeros((27, 64, 64), dtype=torch.float16)
    w[13] = torch.eye(64, dtype=torch.float16)
    m = sc.build_kernel_map(sc.build_hash(torch.from_numpy(coords).to(DEV)))
    xd = x.to(DEV).half()
    y = sc.forward(m, xd, w.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), x.half())
    # fp32 features through the split path. bf16 weights: three 8-bit terms
    # hold all 24 significant bits, so the identity is exact. fp16 weights: the
    # remainder after the first term is below 2^(E-11) for 2^E <= |x|, so the
    # second term's rounding leaves at most 2^(E-23) <= 2^-23 |x| (2^-25
    # absolute where that term falls below the fp16 normal range).
    xf = torch.from_numpy(rng.standard_normal((len(coords), 64)).astype(np.float32)).to(DEV)
    for wt in (torch.bfloat16, torch.float16):
        wi = torch.zeros((27, 64, 64), dtype=wt)
        wi[13] = torch.eye(64, dtype=wt)
        y = sc.forward_fused(m, xf, sc.pack_weights(wi.to(DEV)), out_dtype=torch.float32)
        torch.cuda.synchronize()
        if wt == torch.bfloat16:
            assert torch.equal(y, xf)
        else:
            bound = xf.abs() * 2.0 ** -23 + 2.0 ** -25
            assert bool(((y - xf).abs() <= bound).all())


def test_fused_errors():
    coords = torch.from_numpy(grid(300, 10, 1, 9)).to(DEV)
    m = sc.build_kernel_map(sc.build_hash(coords))
    n = int(coords.shape[0])
    wp = sc.pack_weights(torch.zeros((27, 16, 16), dtype=torch.bfloat16, device=DEV))
    x16 = torch.zeros((n, 16), dtype=torch.float16, device=DEV)
    with pytest.raises(sc.TrSparseConvError) as e:
        sc.forward_fused(m, x16, wp)            # fp16 features with bf16 weights
    assert e.value.code == sc._lib.ERR_UNSUPPORTED
    xb = torch.zeros((n, 16), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sc.TrSparseConvError) as e:
        sc.forward_fused(m, xb, wp, out_dtype=torch.float16)
    assert e.value.code == sc._lib.ERR_UNSUPPORTED
    y = torch.empty((n, 16), dtype=torch.bfloat16, device=DEV)
    L = sc._lib.lib()
    st = L.tr_sparseconv_forward_fused(m.handle, sc._ptr(xb), sc._lib.BF16, wp._ws.ptr, sc._lib.BF16, None, 7,
                                      None, sc._ptr(y), sc._lib.BF16, 16, 16, None)
    assert st == sc._lib.ERR_INVALID_ARG
    st = L.tr_sparseconv_forward_fused(m.handle, sc._ptr(xb), sc._lib.BF16, wp._ws.ptr, sc._lib.BF16, None, 0,
                                      None, sc._ptr(xb), sc._lib.BF16, 16, 16, None)
    assert st == sc._lib.ERR_INVALID_ARG     # y is x
    with pytest.raises(ValueError):
        sc.forward_fused(m, xb, wp, act="gelu")
