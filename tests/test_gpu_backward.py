"""Backward of the convolution on the GPU against the oracle's fp64 gradients.

Data gradient (tr_sparseconv_backward_data) element by element with the output
type's tolerance; weight gradient (tr_sparseconv_backward_weights, fp32 out)
with the fp32 tolerance for sums over K voxel pairs (tests.helpers.tol_f32).
At the workload sizes: every row of dx (sampled rows and the ragged tail at the
1024-wide config) and sampled (tap, channel) rows of dw, each computed one by
one by the oracle. The oracle is always given its own kernel map, which the
GPU's map must equal bit for bit.
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
ROUND = {"f32": lambda a: a, "bf16": W.round_to_bf16, "f16": W.round_to_f16}


@functools.lru_cache(maxsize=None)
def grid(n, D, B, seed):
    rng = np.random.default_rng(seed)
    c = W.random_sparse(rng, n, D=D, B=B)
    return c[rng.permutation(len(c))]


def setup(coords, c_in, c_out, w_t, dy_t, seed):
    gen = w_t if dy_t == w_t else "mixed-" + w_t
    wl = W.custom(coords, c_in, c_out, gen, seed)
    rng = np.random.default_rng(seed + 1)
    dy = ROUND[dy_t](rng.standard_normal((wl.n, c_out), dtype=np.float32))
    m = sc.build_kernel_map(sc.build_hash(torch.from_numpy(wl.coords).to(DEV)))
    # the expected gradients use the oracle's own kernel map, and the GPU's map
    # must equal it bit for bit
    nbr = oracle.kernel_map(wl.coords)
    np.testing.assert_array_equal(m.nbr.cpu().numpy(), nbr)
    return wl, dy, m, nbr


def sel_sample(c_in, k_count, seed):
    rng = np.random.default_rng(seed)
    ks = np.concatenate([[0, 13, 26], rng.integers(0, 27, k_count)])
    cis = np.concatenate([[0, c_in - 1, c_in // 2], rng.integers(0, c_in, k_count)])
    return np.stack([ks, cis], 1).astype(np.int32)


def check_dgrad(wl, dy, m, nbr, w_t, dy_t, dx_t, rows=None):
    w = torch.from_numpy(wl.w).to(DEV).to(TD[w_t])
    dx = sc.backward_data(m, torch.from_numpy(dy).to(DEV).to(TD[dy_t]), sc.pack_weights_dgrad(w),
                          out_dtype=TD[dx_t])
    torch.cuda.synchronize()
    rows = np.arange(wl.n) if rows is None else rows
    ref = oracle.backward_data(nbr, dy, wl.w, rows=rows)
    got = dx.float().cpu().numpy()[rows]
    terms = 27 * wl.c_out * (3 if (dy_t, w_t) == ("f32", "bf16") else 2 if dy_t != w_t else 1)
    tol = tol_f32(terms) if dx_t == "f32" else TOL[dx_t]
    err = max_rel(got, ref)
    say(f"    dgrad max_rel={err:.3e} (tol {tol:.2e})")
    assert err <= tol


def check_wgrad(wl, dy, m, nbr, t, sel=None):
    x = torch.from_numpy(wl.x).to(DEV).to(TD[t])
    dw = sc.backward_weights(m, x, torch.from_numpy(dy).to(DEV).to(TD[t]))
    torch.cuda.synchronize()
    if sel is None:
        ref = oracle.backward_weights(nbr, wl.x, dy).reshape(-1, wl.c_out)
        got = dw.cpu().numpy().reshape(-1, wl.c_out)
    else:
        ref = oracle.backward_weights(nbr, wl.x, dy, sel=sel)
        got = dw.cpu().numpy()[sel[:, 0], sel[:, 1]]
    k_pairs = int((nbr >= 0).sum(0).max()) if wl.n else 1
    tol = tol_f32(k_pairs) if t != "f32" else tol_f32(wl.n)
    err = max_rel(got, ref)
    say(f"    wgrad max_rel={err:.3e} (tol {tol:.2e}, up to {k_pairs} pairs per tap)")
    assert err <= tol
    return dw


DG_TYPES = [("f32", "f32", "f32"), ("bf16", "bf16", "bf16"), ("f16", "f16", "f16"), ("bf16", "f32", "f32"),
            ("f16", "f16", "f32"), ("f16", "f32", "f16")]
SHAPES = [(64, 64), (32, 96), (16, 8), (136, 128)]


@pytest.mark.parametrize("w_t,dy_t,dx_t", DG_TYPES)
@pytest.mark.parametrize("c_in,c_out", SHAPES)
def test_dgrad_small(w_t, dy_t, dx_t, c_in, c_out):
    say(f"[dgrad] c={c_in}->{c_out} w={w_t} dy={dy_t} dx={dx_t}")
    wl, dy, m, nbr = setup(grid(1500, 14, 2, 3), c_in, c_out, w_t, dy_t, 21)
    check_dgrad(wl, dy, m, nbr, w_t, dy_t, dx_t)


@pytest.mark.parametrize("t", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("c_in,c_out", SHAPES)
def test_wgrad_small(t, c_in, c_out):
    say(f"[wgrad] c={c_in}->{c_out} {t}")
    wl, dy, m, nbr = setup(grid(1500, 14, 2, 3), c_in, c_out, t, t, 22)
    check_wgrad(wl, dy, m, nbr, t)


@pytest.mark.parametrize("n,D", [(20000, 40), (70000, 64)])
def test_wgrad_many_splits(n, D):
    # enough voxels for several position ranges and rounds of 1024 per workgroup
    say(f"[wgrad-splits] n~{n} D={D}")
    wl, dy, m, nbr = setup(grid(n, D, 1, 4), 64, 128, "bf16", "bf16", 23)
    check_wgrad(wl, dy, m, nbr, "bf16")


@pytest.mark.parametrize("name,t", [("T", "f32"), ("S", "bf16"), ("L", "bf16"), ("L", "f16"), ("X", "bf16"),
                                         ("W", "bf16")])
def test_backward_config_sizes(name, t):
    wl0 = W.make(name, with_values=False)
    say(f"[backward] config={name} n={wl0.n} c={wl0.c_in}->{wl0.c_out} {t}")
    wl, dy, m, nbr = setup(wl0.coords, wl0.c_in, wl0.c_out, t, t, wl0.seed + 400)
    # every row of dx, except at the 1024-wide config (sampled rows and the tail)
    rows = sample_rows(wl.n, 1500, wl.seed) if wl.c_in >= 1024 else None
    check_dgrad(wl, dy, m, nbr, t, t, t, rows=rows)
    sel = sel_sample(wl.c_in, 13 if wl.c_in >= 1024 else 29, wl.seed) if wl.n > 20000 else None
    check_wgrad(wl, dy, m, nbr, t, sel=sel)


def test_backward_deterministic_and_adjoint():
    wl, dy, m, _ = setup(grid(30000, 48, 1, 5), 64, 64, "bf16", "bf16", 24)
    x = torch.from_numpy(wl.x).to(DEV).bfloat16()
    g = torch.from_numpy(dy).to(DEV).bfloat16()
    w = torch.from_numpy(wl.w).to(DEV).bfloat16()
    a = sc.backward_weights(m, x, g)
    b = sc.backward_weights(m, x, g)
    d1 = sc.backward_data(m, g, sc.pack_weights_dgrad(w), out_dtype=torch.float32)
    d2 = sc.backward_data(m, g, sc.pack_weights_dgrad(w), out_dtype=torch.float32)
    y = sc.forward_fused(m, x, sc.pack_weights(w), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(d1, d2)
    # <conv(x), dy> = <x, dx> = <w, dw>, each summed in float64 on the host
    s_y = float((y.double() * g.double()).sum())
    s_x = float((x.double() * d1.double()).sum())
    s_w = float((w.double() * a.double()).sum())
    assert abs(s_y - s_x) <= 1e-5 * abs(s_y) and abs(s_y - s_w) <= 1e-5 * abs(s_y)


def test_backward_edge_cases():
    # one voxel: only the centre tap; dw[13] = x^T dy, all other taps zero
    for t in ("bf16", "f32"):
        wl, dy, m, nbr = setup(np.array([[0, 5, 6, 7]], np.int32), 16, 24, t, t, 25)
        dw = check_wgrad(wl, dy, m, nbr, t)
        assert float(dw[:13].abs().max()) == 0.0 and float(dw[14:].abs().max()) == 0.0
        check_dgrad(wl, dy, m, nbr, t, t, t)
    # no voxels: dw all zero, dx empty
    m = sc.build_kernel_map(sc.build_hash(torch.zeros((0, 4), dtype=torch.int32, device=DEV)))
    e = torch.zeros((0, 16), dtype=torch.bfloat16, device=DEV)
    dw = sc.backward_weights(m, e, torch.zeros((0, 8), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert dw.shape == (27, 16, 8) and float(dw.abs().max()) == 0.0
    w = torch.zeros((27, 16, 8), dtype=torch.bfloat16, device=DEV)
    dx = sc.backward_data(m, torch.zeros((0, 8), dtype=torch.bfloat16, device=DEV), sc.pack_weights_dgrad(w))
    assert dx.shape == (0, 16)


def test_backward_errors():
    coords = torch.from_numpy(grid(300, 10, 1, 9)).to(DEV)
    m = sc.build_kernel_map(sc.build_hash(coords))
    n = int(coords.shape[0])
    w = torch.zeros((27, 16, 16), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        sc.backward_data(m, torch.zeros((n, 16), dtype=torch.bfloat16, device=DEV), sc.pack_weights(w))
    with pytest.raises(sc.TrSparseConvError) as e:
        sc.backward_data(m, torch.zeros((n, 16), dtype=torch.float16, device=DEV), sc.pack_weights_dgrad(w))
    assert e.value.code == sc._lib.ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        sc.backward_weights(m, torch.zeros((n, 16), dtype=torch.bfloat16, device=DEV),
                            torch.zeros((n, 16), dtype=torch.float16, device=DEV))
    L = sc._lib.lib()
    x = torch.zeros((n, 16), dtype=torch.bfloat16, device=DEV)
    dw = torch.zeros((27, 16, 16), dtype=torch.float32, device=DEV)
    need = L.tr_sparseconv_backward_weights_workspace_bytes(n, 16, 16, sc._lib.BF16)
    assert need >= 256
    ws = sc.Workspace(need, DEV)
    st = L.tr_sparseconv_backward_weights(m.handle, sc._ptr(x), sc._ptr(x), sc._ptr(dw), 16, 16, sc._lib.BF16,
                                          ws.ptr, need - 1, None)
    assert st == sc._lib.ERR_WORKSPACE
    st = L.tr_sparseconv_backward_weights(m.handle, sc._ptr(x), sc._ptr(x), sc._ptr(dw), 12, 16, sc._lib.BF16,
                                          ws.ptr, need, None)
    assert st == sc._lib.ERR_UNSUPPORTED
