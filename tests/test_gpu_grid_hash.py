"""The hash built for voxels in a known grid (tr_sparseconv_build_hash_grid),
against the oracle and against the grid-less build, on the GPU.

The result must be the grid-less hash exactly: the same Morton order (compared
with Z-order keys written independently in numpy), the same kernel map and the
same lookups (both compared with the oracle bit for bit), for the occupancy-
bitmap build and for the radix fallback of grids whose bitmap is too large.
Coordinates outside the given grid and duplicates are reported as errors.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from gen import workloads as W
from tests.helpers import morton_keys_numpy, say

pytestmark = pytest.mark.gpu

sc = pytest.importorskip("submanifold_sparse_conv_amd")
DEV = "cuda:0"


@functools.lru_cache(maxsize=None)
def workload(name, off=0, order="raster"):
    return W.make(name, seed_offset=off, order=order, with_values=False)


def grid_of(wl):
    g = int(wl.D - 1).bit_length()
    assert 1 << g >= wl.D
    return max(g, 2), max(wl.B, 1)


CASES = ([(n, 0, "raster") for n in W.CONFIG_ORDER] + [(n, 100, "shuffled") for n in W.CONFIG_ORDER])


@pytest.mark.parametrize("name,off,order", CASES)
def test_grid_hash_matches(name, off, order):
    wl = workload(name, off, order)
    g, b = grid_of(wl)
    say(f"[grid hash] config={name} seed={wl.seed} order={order} n={wl.n} grid=2^{g} batch={b}")
    c = torch.from_numpy(wl.coords).to(DEV)
    h = sc.build_hash(c, grid_log2=g, batch=b)
    perm = h.sorted_rows().cpu().numpy()
    np.testing.assert_array_equal(perm, np.argsort(morton_keys_numpy(wl.coords), kind="stable"))
    np.testing.assert_array_equal(perm, sc.build_hash(c).sorted_rows().cpu().numpy())
    m = sc.build_kernel_map(h)
    np.testing.assert_array_equal(m.nbr.cpu().numpy(), oracle.kernel_map(wl.coords))
    rng = np.random.default_rng(wl.seed)
    q = np.concatenate([
        wl.coords,
        np.stack([rng.integers(0, b + 1, 50000), rng.integers(-1, wl.D + 2, 50000),
                  rng.integers(-1, wl.D + 2, 50000), rng.integers(-1, wl.D + 2, 50000)], 1),
    ]).astype(np.int32)
    got = h.lookup(torch.from_numpy(q).to(DEV)).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.Table(wl.coords).lookup(q))


@pytest.mark.parametrize("g,batch,n", [(2, 1, 40), (3, 3, 700), (5, 7, 20000), (9, 2, 3000),
                                       (10, 1, 50000), (12, 1, 5000), (16, 2, 3000)])
def test_grid_hash_shapes(g, batch, n):
    # Grids from 4^3 to 65536^3, odd object counts, sparse and dense fills; the
    # last two grids exceed the bitmap limit and take the radix build.
    rng = np.random.default_rng(g * 100 + batch)
    side = 1 << g
    cells = batch * side ** 3
    n = min(n, cells)
    if cells <= 4 * n:
        lin = rng.permutation(cells)[:n]
    else:
        lin = np.unique(rng.integers(0, cells, size=2 * n))[:n]
        rng.shuffle(lin)
    coords = np.stack([lin // side ** 3, (lin // side ** 2) % side, (lin // side) % side, lin % side], 1)
    coords = np.ascontiguousarray(coords.astype(np.int32))
    say(f"[grid shapes] grid=2^{g} batch={batch} n={len(coords)}")
    c = torch.from_numpy(coords).to(DEV)
    h = sc.build_hash(c, grid_log2=g, batch=batch)
    perm = h.sorted_rows().cpu().numpy()
    np.testing.assert_array_equal(perm, np.argsort(morton_keys_numpy(coords), kind="stable"))
    m = sc.build_kernel_map(h)
    np.testing.assert_array_equal(m.nbr.cpu().numpy(), oracle.kernel_map(coords))


def test_grid_hash_reuse_workspace():
    # The bitmap and the table are cleared by the build itself: a second build
    # into the same workspace, of a different set in the same grid, is exact.
    a = workload("S", 0, "raster")
    b = workload("S", 300, "shuffled")
    g, batch = grid_of(a)
    L = sc._lib.lib()
    n = max(a.n, b.n)
    ws = sc.Workspace(L.tr_sparseconv_hash_grid_workspace_bytes(n, g, batch), torch.device(DEV))
    for wl in (a, b, a):
        say(f"[grid reuse] n={wl.n}")
        h = sc.build_hash(torch.from_numpy(wl.coords).to(DEV), grid_log2=g, batch=batch, workspace=ws)
        np.testing.assert_array_equal(sc.build_kernel_map(h).nbr.cpu().numpy(), oracle.kernel_map(wl.coords))


def test_grid_hash_errors():
    say("[grid errors]")
    ok = [[0, 1, 2, 3], [0, 7, 7, 7], [1, 0, 0, 0]]
    for bad in ([0, 8, 0, 0], [0, 0, -1, 0], [0, 0, 0, 8], [2, 0, 0, 0], [-1, 0, 0, 0]):
        c = torch.tensor(ok + [bad], dtype=torch.int32, device=DEV)
        with pytest.raises(sc.TrSparseConvError) as e:
            sc.build_hash(c, grid_log2=3, batch=2)
        assert e.value.code == sc._lib.ERR_COORD_RANGE
    c = torch.tensor(ok + [[0, 7, 7, 7]], dtype=torch.int32, device=DEV)
    with pytest.raises(sc.TrSparseConvError) as e:
        sc.build_hash(c, grid_log2=3, batch=2)
    assert e.value.code == sc._lib.ERR_DUPLICATE
    # the same grid on the radix fallback (bitmap too large) reports the same
    c = torch.tensor(ok + [[0, 1 << 15, 0, 0]], dtype=torch.int32, device=DEV)
    with pytest.raises(sc.TrSparseConvError) as e:
        sc.build_hash(c, grid_log2=15, batch=2)
    assert e.value.code == sc._lib.ERR_COORD_RANGE
    for g, batch in ((1, 1), (17, 1), (3, 0), (3, 65537)):
        with pytest.raises(ValueError):
            sc.build_hash(torch.tensor(ok, dtype=torch.int32, device=DEV), grid_log2=g, batch=batch)
    empty = sc.build_hash(torch.zeros((0, 4), dtype=torch.int32, device=DEV), grid_log2=4)
    assert sc.build_kernel_map(empty).nbr.shape == (0, 27)
