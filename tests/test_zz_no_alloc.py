"""The no-allocation forward (tr_sparseconv_forward_noalloc) through the C ABI
against tr_sparseconv_forward on the same inputs: the same bits, on two calls
in a row whose second input is smaller (the scratch array keeps the first
call's packed weights, which the second call must fully replace); the size
limit is enforced before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

from gen import workloads as W
from tests.helpers import say

pytestmark = pytest.mark.gpu

sc = pytest.importorskip("submanifold_sparse_conv_amd")
DEV = "cuda:0"
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def call_both(coords, c_in, c_out, dtype, seed):
    wl = W.custom(coords, c_in, c_out, "bf16" if dtype == "f16" else dtype, seed)
    dt = TD[dtype]
    x = torch.from_numpy(wl.x).to(DEV).to(dt)
    w = torch.from_numpy(wl.w).to(DEV).to(dt)
    m = sc.build_kernel_map(sc.build_hash(torch.from_numpy(wl.coords).to(DEV)))
    L = sc._lib.lib()
    st = sc._stream(torch.device(DEV))
    code = {"f32": sc._lib.F32, "bf16": sc._lib.BF16, "f16": sc._lib.F16}[dtype]
    y_ref = torch.empty((wl.n, c_out), dtype=dt, device=DEV)
    ws = sc.Workspace(L.tr_sparseconv_forward_workspace_bytes(c_in, c_out, code), DEV)
    sc.check(L.tr_sparseconv_forward(m.handle, sc._ptr(x), sc._ptr(w), sc._ptr(y_ref), c_in, c_out, code,
                                     ws.ptr, ws.nbytes, st))
    y = torch.full((wl.n, c_out), float("nan"), dtype=dt, device=DEV)
    sc.check(L.tr_sparseconv_forward_noalloc(m.handle, sc._ptr(x), sc._ptr(w), sc._ptr(y), c_in, c_out, code, st))
    torch.cuda.synchronize()
    view = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(y.view(view), y_ref.view(view))
    return wl.n


@pytest.mark.parametrize("dtype,c1,c2", [("bf16", (64, 64), (32, 16)), ("f16", (64, 64), (32, 16)),
                                         ("f32", (8, 8), (3, 5)),
                                         ("bf16", (128, 128), (64, 32))])  # both halo shapes
def test_noalloc_matches_forward_twice(dtype, c1, c2):
    rng = np.random.default_rng(91)
    big = W.make("S", with_values=False).coords
    small = W.random_sparse(rng, 700, D=12, B=1)
    say(f"[noalloc] {dtype}: n={len(big)} c={c1} then n={len(small)} c={c2}")
    call_both(big, c1[0], c1[1], dtype, 5)
    call_both(small, c2[0], c2[1], dtype, 6)


def test_noalloc_wide_and_binding():
    # the largest shapes in range (a row-gather shape and a halo shape, whose
    # packing holds a second, fragment-ordered copy), through the Python binding
    rng = np.random.default_rng(92)
    coords = W.random_sparse(rng, 3000, D=16, B=1)
    say(f"[noalloc] 392 x 392 and 256 x 256 bf16, n={len(coords)}")
    call_both(coords, 392, 392, "bf16", 7)
    call_both(coords, 256, 256, "bf16", 9)
    wl = W.custom(coords, 64, 32, "bf16", 8)
    x = torch.from_numpy(wl.x).to(DEV).bfloat16()
    w = torch.from_numpy(wl.w).to(DEV).bfloat16()
    m = sc.build_kernel_map(sc.build_hash(torch.from_numpy(wl.coords).to(DEV)))
    a = sc.forward_noalloc(m, x, w)
    b = sc.forward(m, x, w)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_noalloc_limit():
    coords = torch.tensor([[0, 1, 2, 3], [0, 1, 2, 4]], dtype=torch.int32, device=DEV)
    m = sc.build_kernel_map(sc.build_hash(coords))
    L = sc._lib.lib()
    x = torch.zeros((2, 512), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((27, 512, 512), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros((2, 512), dtype=torch.bfloat16, device=DEV)
    st = L.tr_sparseconv_forward_noalloc(m.handle, sc._ptr(x), sc._ptr(w), sc._ptr(y), 512, 512, sc._lib.BF16,
                                         sc._stream(torch.device(DEV)))
    assert st == sc._lib.ERR_WORKSPACE
    assert b"scratch" in L.tr_sparseconv_last_error()
