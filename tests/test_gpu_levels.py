"""Resolution levels on the GPU against the oracle: parent level (downsample),
subdivision, Channel2Spatial / Spatial2Channel. Index and coordinate outputs
and the moved features are compared bit for bit."""
import functools

import numpy as np
import pytest
import torch

import oracle
from gen import workloads as W
from tests.helpers import say

pytestmark = pytest.mark.gpu

sc = pytest.importorskip("submanifold_sparse_conv_amd")
DEV = "cuda:0"
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
ROUND = {"f32": lambda a: a, "bf16": W.round_to_bf16, "f16": W.round_to_f16}


@functools.lru_cache(maxsize=None)
def workload_coords(name, off, order):
    return W.make(name, seed_offset=off, order=order, with_values=False).coords


@pytest.mark.parametrize("name,off,order", [("T", 0, "raster"), ("S", 100, "shuffled"), ("L", 0, "raster"),
                                            ("X", 100, "shuffled"), ("W", 0, "raster")])
def test_downsample_bitexact(name, off, order):
    coords = workload_coords(name, off, order)
    say(f"[downsample] config={name} order={order} n={len(coords)}")
    h = sc.build_hash(torch.from_numpy(coords).to(DEV))
    coarse, children = sc.downsample(h)
    ref_c, ref_ch = oracle.downsample(coords)
    np.testing.assert_array_equal(coarse.cpu().numpy(), ref_c)
    np.testing.assert_array_equal(children.cpu().numpy(), ref_ch)


def keep_masks(n, seed, density):
    rng = np.random.default_rng(seed)
    bits = rng.random((n, 8)) < density
    return (bits * (1 << np.arange(8))).sum(1).astype(np.uint8)


@pytest.mark.parametrize("name,density", [("T", 1.0), ("S", 0.5), ("S", 0.05), ("X", 0.3)])
def test_subdivide_bitexact(name, density):
    coords = workload_coords(name, 0, "raster")
    keep = None if density == 1.0 else keep_masks(len(coords), 7, density)
    say(f"[subdivide] config={name} n={len(coords)} density={density}")
    fine, children = sc.subdivide(torch.from_numpy(coords).to(DEV),
                                  None if keep is None else torch.from_numpy(keep).to(DEV))
    ref_f, ref_ch = oracle.subdivide(coords, keep)
    np.testing.assert_array_equal(fine.cpu().numpy(), ref_f)
    np.testing.assert_array_equal(children.cpu().numpy(), ref_ch)


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("c_fine", [8, 64, 1024, 1032])
def test_regroup_bitexact(dt, c_fine):
    # Parent rows of 8 * c_fine elements: up to 16 KiB they move through the LDS
    # tile (1024 half / 512 float channels: one row per tile); longer rows take
    # the register path.
    if dt == "f32":
        c_fine = {8: 4, 64: 64, 1024: 512, 1032: 516}[c_fine]
    rng = np.random.default_rng(3)
    coords = W.random_sparse(rng, 5000, D=30, B=2)
    keep = keep_masks(len(coords), 8, 0.4)
    say(f"[regroup] {dt} c_fine={c_fine} n={len(coords)}")
    cd = torch.from_numpy(coords).to(DEV)
    fine, children = sc.subdivide(cd, torch.from_numpy(keep).to(DEV))
    xc = ROUND[dt](rng.standard_normal((len(coords), 8 * c_fine)).astype(np.float32))
    xf = sc.channel2spatial(children, torch.from_numpy(xc).to(DEV).to(TD[dt]), int(fine.shape[0]))
    ch = children.cpu().numpy()
    np.testing.assert_array_equal(xf.float().cpu().numpy(), oracle.channel2spatial(ch, xc, int(fine.shape[0])))
    back = sc.spatial2channel(children, xf)
    np.testing.assert_array_equal(back.float().cpu().numpy(), oracle.spatial2channel(ch, xf.float().cpu().numpy()))


def test_level_round_trip_and_fine_map():
    # coarse -> subdivide -> hash + kernel map at the fine level -> downsample
    coords = workload_coords("S", 0, "raster")
    keep = keep_masks(len(coords), 9, 0.5)
    keep[keep == 0] = 1
    cd = torch.from_numpy(coords).to(DEV)
    fine, children = sc.subdivide(cd, torch.from_numpy(keep).to(DEV))
    say(f"[levels] coarse n={len(coords)} fine n={int(fine.shape[0])}")
    h = sc.build_hash(fine)
    m = sc.build_kernel_map(h)
    np.testing.assert_array_equal(m.nbr.cpu().numpy(), oracle.kernel_map(fine.cpu().numpy()))
    coarse, ch2 = sc.downsample(h)
    c_np, ch_np = coarse.cpu().numpy(), ch2.cpu().numpy()
    row = {tuple(r): i for i, r in enumerate(coords.tolist())}
    idx = np.array([row[tuple(r)] for r in c_np.tolist()])
    assert len(idx) == len(coords)
    np.testing.assert_array_equal(ch_np, children.cpu().numpy()[idx])


def test_level_edge_cases():
    empty = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    fine, children = sc.subdivide(empty)
    assert fine.shape == (0, 4) and children.shape == (0, 8)
    coarse, ch = sc.downsample(sc.build_hash(empty))
    assert coarse.shape == (0, 4)
    one = torch.tensor([[3, 32767, 0, 5]], dtype=torch.int32, device=DEV)
    fine, children = sc.subdivide(one, torch.tensor([0b10000001], dtype=torch.uint8, device=DEV))
    assert fine.cpu().tolist() == [[3, 65534, 0, 10], [3, 65535, 1, 11]]
    assert children.cpu().tolist() == [[0, -1, -1, -1, -1, -1, -1, 1]]
    with pytest.raises(sc.TrSparseConvError) as e:
        sc.subdivide(torch.tensor([[0, 32768, 0, 0]], dtype=torch.int32, device=DEV))
    assert e.value.code == sc._lib.ERR_COORD_RANGE
    top = torch.tensor([[65535, 65535, 65535, 65535], [65535, 65534, 65535, 65534]], dtype=torch.int32,
                       device=DEV)
    coarse, ch = sc.downsample(sc.build_hash(top))
    assert coarse.cpu().tolist() == [[65535, 32767, 32767, 32767]]
    assert ch.cpu().tolist() == [[-1, -1, 1, -1, -1, -1, -1, 0]]   # octants 4*0 + 2*1 + 0 and 7


def test_regroup_shape_errors():
    # mis-sized operands are refused on the host, before anything is launched
    children = torch.full((5, 8), -1, dtype=torch.int32, device=DEV)
    xc = torch.zeros((5, 64), dtype=torch.bfloat16, device=DEV)
    bad = [
        lambda: sc.channel2spatial(children[:, :7].contiguous(), xc, 3),       # children not [M, 8]
        lambda: sc.channel2spatial(children, xc[:4], 3),                      # x_coarse rows != M
        lambda: sc.channel2spatial(children, xc[:, :60].contiguous(), 3),     # 8C not a multiple of 8
        lambda: sc.channel2spatial(children, xc, 3,
                                   out=torch.zeros((2, 8), dtype=torch.bfloat16, device=DEV)),  # rows
        lambda: sc.channel2spatial(children, xc, 3,
                                   out=torch.zeros((3, 16), dtype=torch.bfloat16, device=DEV)),  # channels
        lambda: sc.channel2spatial(children, xc, -1),
        lambda: sc.spatial2channel(children[:, :4].contiguous(), torch.zeros((3, 8), dtype=torch.bfloat16,
                                                                              device=DEV)),
        lambda: sc.spatial2channel(children, torch.zeros((3, 8), dtype=torch.bfloat16, device=DEV),
                                   out=torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)),  # rows
        lambda: sc.spatial2channel(children, torch.zeros((3, 8), dtype=torch.bfloat16, device=DEV),
                                   out=torch.zeros((5, 32), dtype=torch.bfloat16, device=DEV)),  # channels
    ]
    for i, f in enumerate(bad):
        with pytest.raises(ValueError):
            f()
