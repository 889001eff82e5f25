"""Parity of the HIP path with the CPU oracle, through the C ABI, on the GPU.

Kernel maps and hash lookups are compared bit for bit. Features are compared
element by element (every row, except at the 1024-wide config: sampled rows
plus the ragged tail) with the max relative error of helpers.max_rel against
2e-2 (bf16) and 1e-4 (fp32).
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from gen import workloads as W
from tests.helpers import TOL, max_rel, morton_keys_numpy, sample_rows, say

pytestmark = pytest.mark.gpu

sc = pytest.importorskip("submanifold_sparse_conv_amd")
DEV = "cuda:0"
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@functools.lru_cache(maxsize=None)
def workload(name, off=0, order="raster"):
    return W.make(name, seed_offset=off, order=order)


@functools.lru_cache(maxsize=None)
def oracle_map(name, off=0, order="raster"):
    return oracle.kernel_map(workload(name, off, order).coords)


def to_dev(wl):
    dt = TORCH_DT[wl.dtype]
    c = torch.from_numpy(wl.coords).to(DEV)
    x = torch.from_numpy(wl.x).to(DEV).to(dt)   # exact: values are representable
    w = torch.from_numpy(wl.w).to(DEV).to(dt)
    return c, x, w


def run_all(coords, x, w):
    h = sc.build_hash(coords)
    m = sc.build_kernel_map(h)
    y = sc.forward(m, x, w)
    torch.cuda.synchronize()
    return h, m, y


MAP_CASES = ([(n, 0, "raster") for n in W.CONFIG_ORDER]
             + [(n, 100, "shuffled") for n in W.CONFIG_ORDER]
             + [("T", 200, "shuffled"), ("S", 200, "raster")])


@pytest.mark.parametrize("name,off,order", MAP_CASES)
def test_kernel_map_bitexact(name, off, order):
    wl = workload(name, off, order)
    say(f"[kmap] config={name} seed={wl.seed} order={order} n={wl.n}")
    h = sc.build_hash(torch.from_numpy(wl.coords).to(DEV))
    m = sc.build_kernel_map(h)
    nbr = m.nbr.cpu().numpy()
    np.testing.assert_array_equal(nbr, oracle_map(name, off, order))


@pytest.mark.parametrize("name,off,order", [(n, 100, "shuffled") for n in W.CONFIG_ORDER])
def test_hash_lookup_bitexact(name, off, order):
    wl = workload(name, off, order)
    say(f"[lookup] config={name} seed={wl.seed} n={wl.n}")
    h = sc.build_hash(torch.from_numpy(wl.coords).to(DEV))
    rng = np.random.default_rng(wl.seed)
    q = np.concatenate([
        wl.coords,
        np.stack([rng.integers(0, wl.B + 1, 100000), rng.integers(-1, wl.D + 2, 100000),
                  rng.integers(-1, wl.D + 2, 100000), rng.integers(-1, wl.D + 2, 100000)], 1),
    ]).astype(np.int32)
    got = h.lookup(torch.from_numpy(q).to(DEV)).cpu().numpy()
    ref = oracle.Table(wl.coords).lookup(q)
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(got[:wl.n], np.arange(wl.n))


@pytest.mark.parametrize("name,off,order", [("S", 100, "shuffled"), ("X", 0, "raster"),
                                            ("W", 100, "shuffled")])
def test_morton_order_bitexact(name, off, order):
    wl = workload(name, off, order)
    say(f"[morton] config={name} seed={wl.seed} n={wl.n}")
    h = sc.build_hash(torch.from_numpy(wl.coords).to(DEV))
    perm = h.sorted_rows().cpu().numpy()
    np.testing.assert_array_equal(perm, np.argsort(morton_keys_numpy(wl.coords), kind="stable"))


FWD_CASES = ([(n, 0, "raster") for n in W.CONFIG_ORDER]
             + [(n, 100, "shuffled") for n in W.CONFIG_ORDER]
             + [("S", 200, "raster"), ("L", 200, "shuffled")])


@pytest.mark.parametrize("name,off,order", FWD_CASES)
def test_forward_parity(name, off, order):
    wl = workload(name, off, order)
    say(f"[forward] config={name} seed={wl.seed} order={order} n={wl.n} "
        f"c={wl.c_in}->{wl.c_out} {wl.dtype}")
    c, x, w = to_dev(wl)
    _, m, y = run_all(c, x, w)
    nbr = oracle_map(name, off, order)
    np.testing.assert_array_equal(m.nbr.cpu().numpy(), nbr)
    # every row, except at the 1024-wide config (the oracle's fp64 sums there
    # take minutes): first rows, the ragged tail and a random sample
    rows = sample_rows(wl.n, 1500, wl.seed) if wl.c_in >= 1024 else np.arange(wl.n)
    ref = oracle.forward(nbr, wl.x, wl.w, rows=rows)
    got = y.float().cpu().numpy()[rows]
    err = max_rel(got, ref)
    say(f"    max_rel={err:.3e} (unfloored max abs {np.abs(got - ref).max():.3e}, "
        f"normwise {np.abs(got - ref).max() / np.abs(ref).max():.3e})")
    assert err <= TOL[wl.dtype]


SMALL_SHAPES = [(8, 8, "f32"), (3, 5, "f32"), (8, 8, "bf16"), (16, 8, "bf16"), (64, 64, "bf16"),
                (32, 96, "bf16"), (128, 128, "bf16"), (64, 32, "bf16"), (256, 64, "bf16"),
                (136, 64, "bf16"), (72, 128, "bf16"),  # a last 64-channel chunk of 8 or 8 of 72
                (256, 128, "bf16"), (512, 256, "bf16"), (264, 136, "bf16"),  # the wide-layer tiles
                (192, 384, "bf16"), (320, 64, "bf16"), (64, 256, "bf16")]  # more halo-kernel shapes


@pytest.mark.parametrize("n", [1, 63, 64, 65, 257, 1000, 4097])
@pytest.mark.parametrize("c_in,c_out,dtype", SMALL_SHAPES)
def test_forward_small_all_rows(n, c_in, c_out, dtype):
    rng = np.random.default_rng(n * 1000 + c_in + c_out)
    coords = W.random_sparse(rng, n, D=14 if n > 500 else 7, B=2)
    coords = coords[rng.permutation(n)]
    wl = W.custom(coords, c_in, c_out, dtype, seed=n + c_in)
    say(f"[small] n={n} c={c_in}->{c_out} {dtype}")
    c, x, w = to_dev(wl)
    _, m, y = run_all(c, x, w)
    nbr, ref = oracle.conv(coords, wl.x, wl.w)
    np.testing.assert_array_equal(m.nbr.cpu().numpy(), nbr)
    assert max_rel(y.float().cpu().numpy(), ref) <= TOL[dtype]


@pytest.mark.parametrize("n", [65, 4097])
def test_forward_wide_all_rows(n):
    # the 1024-wide layer's tile shape on every row, partial last tile included
    rng = np.random.default_rng(n + 1024)
    coords = W.random_sparse(rng, n, D=14 if n > 500 else 7, B=2)
    coords = coords[rng.permutation(n)]
    wl = W.custom(coords, 1024, 1024, "bf16", seed=n + 7)
    say(f"[wide] n={n} c=1024->1024 bf16")
    c, x, w = to_dev(wl)
    _, m, y = run_all(c, x, w)
    nbr, ref = oracle.conv(coords, wl.x, wl.w)
    np.testing.assert_array_equal(m.nbr.cpu().numpy(), nbr)
    err = max_rel(y.float().cpu().numpy(), ref)
    say(f"    max_rel={err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("c_in,c_out", [(64, 64), (72, 48)])
def test_forward_large_64wide_all_rows(c_in, c_out):
    # 64-wide layers over more than 65,536 voxels take the LDS-staged gather
    # path; every row against the oracle, with a ragged last tile
    rng = np.random.default_rng(c_in * 31 + c_out)
    coords = W.random_sparse(rng, 70001, D=48, B=1)
    coords = coords[rng.permutation(len(coords))]
    wl = W.custom(coords, c_in, c_out, "bf16", seed=c_in + 5)
    say(f"[large 64-wide] n={wl.n} c={c_in}->{c_out} bf16")
    c, x, w = to_dev(wl)
    _, m, y = run_all(c, x, w)
    nbr, ref = oracle.conv(coords, wl.x, wl.w)
    np.testing.assert_array_equal(m.nbr.cpu().numpy(), nbr)
    err = max_rel(y.float().cpu().numpy(), ref)
    say(f"    max_rel={err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("c_in,c_out,tiles", [(128, 128, 532), (256, 256, 532), (64, 128, 532), (64, 64, 532),
                                               (128, 32, 532), (128, 128, 600), (256, 256, 600), (64, 128, 600)])
def test_forward_split_last_round(c_in, c_out, tiles):
    # tiles of 256 voxels over surface shells. On a 256-CU device (512
    # workgroup slots of the tile kernel), at 532 tiles the last round holds 20
    # items (40 at 256 output channels), each run as eight K-split 32-row parts
    # (of 128, 64 or 32 columns); at 600 tiles it holds 88 (176) 128-column
    # items, too many for their parts to fit at once, so they run whole.
    # Sampled rows (about 1 in 17) against the oracle, the last round's tiles
    # included
    n = tiles * 256 - 37
    rng = np.random.default_rng(c_in * 7 + c_out)
    occ = W.ellipsoid_object(rng, 192, n, 10 * n)
    coords = np.argwhere(occ).astype(np.int32)
    coords = coords[rng.permutation(len(coords))[:n]]
    coords = np.concatenate([np.zeros((n, 1), np.int32), coords], axis=1)
    wl = W.custom(coords, c_in, c_out, "bf16", seed=c_in + c_out)
    say(f"[split last round] n={wl.n} tiles={tiles} c={c_in}->{c_out} bf16")
    c, x, w = to_dev(wl)
    _, m, y = run_all(c, x, w)
    nbr = oracle.kernel_map(coords)
    rows = sample_rows(wl.n, 8000, seed=c_in + c_out)
    np.testing.assert_array_equal(m.nbr.cpu().numpy()[rows], nbr[rows])
    ref = oracle.forward(nbr, wl.x, wl.w, rows=rows)
    err = max_rel(y.float().cpu().numpy()[rows], ref)
    say(f"    max_rel={err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("c", [8, 64, 128])
def test_identity_kernel_bitexact(dtype, c):
    wl = workload("S", 100, "shuffled")
    say(f"[identity] c={c} {dtype}")
    dt = TORCH_DT[dtype]
    xv, _ = W.make_values(wl.n, c, c, dtype, np.random.default_rng(c))
    x = torch.from_numpy(xv).to(DEV).to(dt)
    w = torch.zeros((27, c, c), dtype=dt, device=DEV)
    w[13] = torch.eye(c, dtype=dt, device=DEV)
    _, _, y = run_all(torch.from_numpy(wl.coords).to(DEV), x, w)
    assert torch.equal(y.view(torch.int16) if dtype == "bf16" else y.view(torch.int32),
                       x.view(torch.int16) if dtype == "bf16" else x.view(torch.int32))


@pytest.mark.parametrize("name", ["S", "L"])
def test_deterministic_bits(name):
    wl = workload(name, 100, "shuffled")
    say(f"[determinism] config={name}")
    c, x, w = to_dev(wl)
    _, m1, y1 = run_all(c, x, w)
    _, m2, y2 = run_all(c, x, w)
    assert torch.equal(m1.nbr, m2.nbr)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_shared_map_on_two_streams():
    # A kernel map is read-only once built: forwards on two streams over one map
    # (different weights, running concurrently) give the bits of sequential runs.
    wl = workload("S", 300, "shuffled")
    say(f"[streams] config=S n={wl.n}")
    c, x, w = to_dev(wl)
    m = sc.build_kernel_map(sc.build_hash(c))
    w2 = (w.float() * -0.5).to(w.dtype)
    wp1, wp2 = sc.pack_weights(w), sc.pack_weights(w2)
    torch.cuda.synchronize()
    ref1 = sc.forward_packed(m, x, wp1)
    ref2 = sc.forward_packed(m, x, wp2)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            a = sc.forward_packed(m, x, wp1)
        with torch.cuda.stream(s2):
            b = sc.forward_packed(m, x, wp2)
        outs.append((a, b))
    torch.cuda.synchronize()
    for a, b in outs:
        assert torch.equal(a.view(torch.int16), ref1.view(torch.int16))
        assert torch.equal(b.view(torch.int16), ref2.view(torch.int16))


def test_forward_on_two_streams():
    # forward() packs its weights on the calling stream: two streams over one
    # map with different weights, in flight together, give the bits of
    # sequential runs (no packing buffer is shared between the calls).
    wl = workload("S", 300, "shuffled")
    say(f"[streams] forward() config=S n={wl.n}")
    c, x, w = to_dev(wl)
    m = sc.build_kernel_map(sc.build_hash(c))
    w2 = (w.float() * -0.5).to(w.dtype)
    ref1 = sc.forward(m, x, w)
    ref2 = sc.forward(m, x, w2)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        with torch.cuda.stream(s1):
            a = sc.forward(m, x, w)
        with torch.cuda.stream(s2):
            b = sc.forward(m, x, w2)
        outs.append((a, b))
    torch.cuda.synchronize()
    for a, b in outs:
        assert torch.equal(a.view(torch.int16), ref1.view(torch.int16))
        assert torch.equal(b.view(torch.int16), ref2.view(torch.int16))


def test_translation_invariance():
    wl = workload("S", 200, "raster")
    say("[translation] config=S")
    c, x, w = to_dev(wl)
    _, m1, y1 = run_all(c, x, w)
    shift = torch.tensor([0, 1000, 37, 60000], dtype=torch.int32, device=DEV)
    _, m2, y2 = run_all(c + shift, x, w)
    assert torch.equal(m1.nbr, m2.nbr)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_empty_and_single():
    say("[edge] empty and single voxel")
    c = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    x = torch.zeros((0, 16), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((27, 16, 8), dtype=torch.bfloat16, device=DEV)
    h, m, y = run_all(c, x, w)
    assert m.nbr.shape == (0, 27) and y.shape == (0, 8)
    wl = W.custom(np.array([[3, 9, 9, 9]], np.int32), 16, 8, "bf16", seed=4)
    cc, xx, ww = to_dev(wl)
    _, m, y = run_all(cc, xx, ww)
    assert m.nbr.cpu().numpy().tolist() == [[-1] * 13 + [0] + [-1] * 13]
    ref = oracle.conv(wl.coords, wl.x, wl.w)[1]
    assert max_rel(y.float().cpu().numpy(), ref) <= TOL["bf16"]


def test_coordinate_extremes():
    say("[edge] coordinates at 0 and 65535, the all-ones key")
    top = 65535
    pts = [[top, top, top, top], [top, top - 1, top, top], [top, top, top - 1, top - 1],
           [0, 0, 0, 0], [0, 1, 1, 1], [0, 0, 0, 1], [top, 0, top, 0], [1, top, top, top]]
    coords = np.array(pts, np.int32)
    wl = W.custom(coords, 8, 8, "f32", seed=1)
    c, x, w = to_dev(wl)
    h, m, y = run_all(c, x, w)
    nbr, ref = oracle.conv(coords, wl.x, wl.w)
    np.testing.assert_array_equal(m.nbr.cpu().numpy(), nbr)
    assert max_rel(y.cpu().numpy(), ref) <= TOL["f32"]
    np.testing.assert_array_equal(h.lookup(c).cpu().numpy(), np.arange(len(pts)))


def _colliding_blocks(count, log2_cap, rng):
    """`count` distinct 4x4x4 block coordinates (batch 0) whose block keys
    (Z-order key >> 6) share one home slot of a 2^log2_cap-slot table under the
    table's multiplicative hash (top bits of key * 0x9E3779B97F4A7C15 mod 2^64),
    plus one more such block to leave absent."""
    shift = np.uint64(64 - log2_cap)
    chosen, target = [], None
    while len(chosen) < count + 1:
        bc = rng.integers(0, 1 << 14, size=(8192, 3)).astype(np.int64)
        c4 = np.column_stack([np.zeros(len(bc), np.int64), bc * 4])
        bkey = morton_keys_numpy(c4) >> np.uint64(6)
        home = (bkey * np.uint64(0x9E3779B97F4A7C15)) >> shift
        if target is None:
            target = home[0]
        for j in np.nonzero(home == target)[0]:
            if len(chosen) <= count and not any((bc[j] == c).all() for c in chosen):
                chosen.append(bc[j])
    return np.array(chosen[:count]), chosen[count]


def test_colliding_blocks():
    # 64 occupied blocks (table capacity 128) whose keys all hash to one home
    # slot: probe runs up to 64 slots long, for the kernel map, for lookups of
    # present voxels and for an absent block on the same home slot.
    say("[edge] 64 blocks on one home slot of a 128-slot table")
    rng = np.random.default_rng(77)
    blocks, absent = _colliding_blocks(64, 7, rng)
    pts = []
    for bc in blocks:
        cells = rng.choice(64, size=int(rng.integers(1, 6)), replace=False)
        for cell in cells:  # in-block (x, y, z) from the cell's bits; corners reach neighbours
            lx, ly, lz = (cell >> 2 & 1) | (cell >> 5 & 1) << 1, (cell >> 1 & 1) | (cell >> 4 & 1) << 1, \
                (cell & 1) | (cell >> 3 & 1) << 1
            pts.append([0, 4 * bc[0] + lx, 4 * bc[1] + ly, 4 * bc[2] + lz])
    coords = np.array(pts, np.int32)
    wl = W.custom(coords, 8, 8, "f32", seed=3)
    c, x, w = to_dev(wl)
    h, m, y = run_all(c, x, w)
    assert sc.status(h) == 0
    nbr, ref = oracle.conv(coords, wl.x, wl.w)
    np.testing.assert_array_equal(m.nbr.cpu().numpy(), nbr)
    assert max_rel(y.cpu().numpy(), ref) <= TOL["f32"]
    q = np.concatenate([coords, [[0, 4 * absent[0] + a, 4 * absent[1] + b, 4 * absent[2] + d]
                                 for a in range(4) for b in range(4) for d in range(4)]]).astype(np.int32)
    got = h.lookup(torch.from_numpy(q).to(DEV)).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.Table(coords).lookup(q))
    np.testing.assert_array_equal(got[:len(coords)], np.arange(len(coords)))


@pytest.mark.parametrize("n", [2_400_000, 3_200_000, 7_000_000])
def test_large_sorts(n):
    # Radix tiles of 16 and 32 keys per thread, and more tiles than one pass of
    # the column scan covers (n > 768 tiles of 8192 keys): the Morton order
    # bit-exact, and sampled kernel-map rows against the oracle's table.
    rng = np.random.default_rng(n)
    idx = rng.choice(2 * 256 ** 3, size=n, replace=False)
    b, r = np.divmod(idx, 256 ** 3)
    x, r = np.divmod(r, 256 * 256)
    y, z = np.divmod(r, 256)
    coords = np.stack([b, x, y, z], 1).astype(np.int32)
    say(f"[large sort] n={n} in 2 x 256^3")
    h = sc.build_hash(torch.from_numpy(coords).to(DEV))
    perm = h.sorted_rows().cpu().numpy()
    np.testing.assert_array_equal(perm, np.argsort(morton_keys_numpy(coords), kind="stable"))
    m = sc.build_kernel_map(h)
    rows = sample_rows(n, 20000, seed=n)
    got = m.nbr[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    offs = np.array([[0, k // 9 - 1, (k // 3) % 3 - 1, k % 3 - 1] for k in range(27)], np.int32)
    q = (coords[rows][:, None, :] + offs[None]).reshape(-1, 4).astype(np.int32)
    ref = oracle.Table(coords).lookup(q).reshape(len(rows), 27)
    np.testing.assert_array_equal(got, ref)


def test_wide_keys_morton_order():
    # 40 varying key bits (object ids spread over 16 bits): the last 7 go
    # through the single-workgroup rest pass of the sort
    wl = workload("L")
    c = wl.coords.copy()
    c[:, 0] = (np.arange(wl.n) % 64) * 1021
    c = c[np.random.default_rng(5).permutation(wl.n)]
    say(f"[wide keys] n={wl.n}")
    h = sc.build_hash(torch.from_numpy(c).to(DEV))
    perm = h.sorted_rows().cpu().numpy()
    np.testing.assert_array_equal(perm, np.argsort(morton_keys_numpy(c), kind="stable"))
    m = sc.build_kernel_map(h)
    rows = sample_rows(wl.n, 20000, seed=9)
    np.testing.assert_array_equal(m.nbr.cpu().numpy()[rows], oracle.kernel_map(c)[rows])


def test_errors():
    say("[edge] error codes")
    dup = torch.tensor([[0, 1, 2, 3], [0, 5, 5, 5], [0, 1, 2, 3]], dtype=torch.int32, device=DEV)
    with pytest.raises(sc.TrSparseConvError) as e:
        sc.build_hash(dup)
    assert e.value.code == -3
    dup_top = torch.tensor([[65535] * 4, [65535] * 4], dtype=torch.int32, device=DEV)
    with pytest.raises(sc.TrSparseConvError) as e:
        sc.build_hash(dup_top)
    assert e.value.code == -3
    for bad in ([0, -1, 2, 3], [0, 1, 65536, 3], [70000, 1, 2, 3]):
        c = torch.tensor([[0, 0, 0, 0], bad], dtype=torch.int32, device=DEV)
        with pytest.raises(sc.TrSparseConvError) as e:
            sc.build_hash(c)
        assert e.value.code == -2
    c = torch.tensor([[0, 0, 0, 0]], dtype=torch.int32, device=DEV)
    m = sc.build_kernel_map(sc.build_hash(c))
    with pytest.raises(sc.TrSparseConvError) as e:
        sc.forward(m, torch.zeros((1, 12), dtype=torch.bfloat16, device=DEV),
                   torch.zeros((27, 12, 8), dtype=torch.bfloat16, device=DEV))
    assert e.value.code == -6
    x8 = torch.zeros((1, 8), dtype=torch.bfloat16, device=DEV)
    wp8 = sc.pack_weights(torch.zeros((27, 8, 8), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(sc.TrSparseConvError) as e:  # in place: other rows would read x while y is written
        sc.forward_packed(m, x8, wp8, out=x8)
    assert e.value.code == -1


@pytest.mark.parametrize("name", ["S", "X"])
def test_forward_packed_matches_forward(name):
    wl = workload(name, 100, "shuffled")
    say(f"[packed] config={name}")
    c, x, w = to_dev(wl)
    h, m, y = run_all(c, x, w)
    wp = sc.pack_weights(w)
    y2 = sc.forward_packed(m, x, wp)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_forward_packed_f32():
    wl = workload("T", 100, "shuffled")
    say("[packed] config=T f32")
    c, x, w = to_dev(wl)
    h, m, y = run_all(c, x, w)
    y2 = sc.forward_packed(m, x, sc.pack_weights(w))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
