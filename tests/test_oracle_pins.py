"""Pins for the CPU oracle, checked against things other than itself.

Each test compares the oracle with an independent fact: a hand-worked example,
a library routine (torch's dense conv3d in float64), a dense brute force, a
closed form, or an invariant the definition implies. They run without a GPU.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from gen import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tap_offsets():
    # d_k for k = 9*Kd + 3*Kh + Kw, component = K - 1 (written from the tap
    # numbering, independently of the oracle's own helper).
    return np.array([(a - 1, b - 1, c - 1) for a in range(3) for b in range(3) for c in range(3)])


# --------------------------------------------------------------------------
# hand-worked example
# --------------------------------------------------------------------------
def load_hand_example():
    rows, nb = [], {}
    section = None
    with open(os.path.join(GOLDEN, "hand_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line in ("coords_features_y", "neighbours"):
                section = line
                continue
            parts = line.split()
            if section == "coords_features_y":
                rows.append([int(v) for v in parts])
            else:
                nb[int(parts[0])] = {int(p.split(":")[0]): int(p.split(":")[1]) for p in parts[1:]}
    a = np.array(rows, dtype=np.int64)
    return a[:, :4].astype(np.int32), a[:, 4].astype(np.float64), a[:, 5].astype(np.float64), nb


def test_hand_example_map_and_values():
    coords, feat, y_exp, nb = load_hand_example()
    nbr = oracle.kernel_map(coords)
    expected = np.full((len(coords), 27), -1, dtype=np.int32)
    for i, d in nb.items():
        for k, j in d.items():
            expected[i, k] = j
    np.testing.assert_array_equal(nbr, expected)
    w = (np.arange(27, dtype=np.float64) + 1.0).reshape(27, 1, 1)
    y = oracle.forward(nbr, feat.reshape(-1, 1), w)
    np.testing.assert_array_equal(y[:, 0], y_exp)


# --------------------------------------------------------------------------
# kernel map against brute force and a dense look-up table
# --------------------------------------------------------------------------
def brute_force_map(coords):
    c = coords.astype(np.int64)
    n = len(c)
    nbr = np.full((n, 27), -1, dtype=np.int32)
    d = c[None, :, 1:] - c[:, None, 1:]                   # [i, j, 3]: p_j - p_i
    same_b = c[None, :, 0] == c[:, None, 0]
    close = same_b & (np.abs(d) <= 1).all(axis=2)
    ii, jj = np.nonzero(close)
    dd = d[ii, jj]
    k = 9 * (dd[:, 0] + 1) + 3 * (dd[:, 1] + 1) + (dd[:, 2] + 1)
    nbr[ii, k] = jj
    return nbr


def lut_map(coords, D, B):
    lut = np.full((B, D, D, D), -1, dtype=np.int32)
    c = coords.astype(np.int64)
    lut[c[:, 0], c[:, 1], c[:, 2], c[:, 3]] = np.arange(len(c), dtype=np.int32)
    nbr = np.full((len(c), 27), -1, dtype=np.int32)
    for k, (dx, dy, dz) in enumerate(tap_offsets()):
        q = c[:, 1:] + np.array([dx, dy, dz])
        ok = ((q >= 0) & (q < D)).all(axis=1)
        nbr[ok, k] = lut[c[ok, 0], q[ok, 0], q[ok, 1], q[ok, 2]]
    return nbr


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_map_brute_force_random(seed):
    rng = np.random.default_rng(seed)
    coords = W.random_sparse(rng, 1500, D=12, B=2)
    coords = coords[rng.permutation(len(coords))]
    np.testing.assert_array_equal(oracle.kernel_map(coords), brute_force_map(coords))


def test_map_brute_force_tiny_config():
    wl = W.make("T", with_values=False)
    np.testing.assert_array_equal(oracle.kernel_map(wl.coords), brute_force_map(wl.coords))
    wl = W.make("T", seed_offset=100, order="shuffled", with_values=False)
    np.testing.assert_array_equal(oracle.kernel_map(wl.coords), brute_force_map(wl.coords))


@pytest.mark.parametrize("name", ["S", "W", "L", "X"])
def test_map_lut_configs(name):
    wl = W.make(name, with_values=False)
    nbr = oracle.kernel_map(wl.coords)
    np.testing.assert_array_equal(nbr, lut_map(wl.coords, wl.D, wl.B))


def test_map_invariants():
    wl = W.make("S", seed_offset=100, order="shuffled", with_values=False)
    nbr = oracle.kernel_map(wl.coords)
    n = wl.n
    np.testing.assert_array_equal(nbr[:, 13], np.arange(n))
    # mirror symmetry: nbr[i][k] = j  <=>  nbr[j][26-k] = i
    ii, kk = np.nonzero(nbr >= 0)
    jj = nbr[ii, kk]
    np.testing.assert_array_equal(nbr[jj, 26 - kk], ii)
    # per-offset counts: |A intersect (A - d_k)| with Python sets
    A = set(map(tuple, wl.coords.tolist()))
    for k, (dx, dy, dz) in enumerate(tap_offsets()):
        expect = sum((b, x + dx, y + dy, z + dz) in A for (b, x, y, z) in A)
        assert int((nbr[:, k] >= 0).sum()) == expect


@pytest.mark.parametrize("n", [1, 2, 3, 5, 7])
def test_map_full_cube_closed_form(n):
    coords = W.full_cube(n, origin=(3, 4, 5))
    nbr = oracle.kernel_map(coords)
    assert int((nbr >= 0).sum()) == (3 * n - 2) ** 3
    deg = (nbr >= 0).sum(axis=1)
    # interior 27, face 18, edge 12, corner 8 (n >= 2)
    if n >= 2:
        counts = {27: (n - 2) ** 3, 18: 6 * (n - 2) ** 2, 12: 12 * (n - 2), 8: 8}
        got = {int(v): int((deg == v).sum()) for v in np.unique(deg)}
        assert got == {k: v for k, v in counts.items() if v}


def test_lookup_against_dict():
    rng = np.random.default_rng(7)
    coords = W.random_sparse(rng, 3000, D=40, B=3)
    t = oracle.Table(coords)
    d = {tuple(r): i for i, r in enumerate(coords.tolist())}
    np.testing.assert_array_equal(t.lookup(coords), np.arange(len(coords)))
    q = rng.integers(-2, 42, size=(20000, 4)).astype(np.int32)
    q[:, 0] = rng.integers(0, 4, size=20000)
    exp = np.array([d.get(tuple(r), -1) for r in q.tolist()], dtype=np.int32)
    np.testing.assert_array_equal(t.lookup(q), exp)


def test_errors_and_empty():
    assert oracle.build_status(np.array([[0, 1, 2, 3], [0, 1, 2, 3]], np.int32)) == oracle.ERR_DUPLICATE
    assert oracle.build_status(np.array([[0, -1, 2, 3]], np.int32)) == oracle.ERR_COORD_RANGE
    assert oracle.build_status(np.array([[0, 1, 65536, 3]], np.int32)) == oracle.ERR_COORD_RANGE
    assert oracle.build_status(np.array([[65535, 65535, 65535, 65535]], np.int32)) == oracle.OK
    nbr = oracle.kernel_map(np.zeros((0, 4), np.int32))
    assert nbr.shape == (0, 27)
    y = oracle.forward(nbr, np.zeros((0, 4)), np.zeros((27, 4, 3)))
    assert y.shape == (0, 3)
    # neighbours at the top of the coordinate range do not wrap around
    c = np.array([[0, 65535, 65535, 65535], [0, 0, 0, 0], [0, 65534, 65535, 65535]], np.int32)
    nbr = oracle.kernel_map(c)
    assert (nbr[0] >= 0).sum() == 2 and nbr[0, 4] == 2
    assert (nbr[1] >= 0).sum() == 1


# --------------------------------------------------------------------------
# feature sum against dense 3x3x3 convolution (zero padding 1)
# --------------------------------------------------------------------------
def dense_inputs(coords, x, B, D):
    dense = np.zeros((B, x.shape[1], D, D, D))
    c = coords.astype(np.int64)
    dense[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]] = x
    return dense


def torch_dense_conv(coords, x, w, B, D):
    dense = torch.from_numpy(dense_inputs(coords, x, B, D))
    # Wt[co, ci, a, b, c] = W[9a + 3b + c, ci, co]; spatial dims (D, H, W) = (x, y, z)
    wt = torch.from_numpy(np.ascontiguousarray(w.reshape(3, 3, 3, w.shape[1], w.shape[2])
                                               .transpose(4, 3, 0, 1, 2)))
    out = torch.nn.functional.conv3d(dense, wt, padding=1).numpy()
    c = coords.astype(np.int64)
    return out[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]]


def naive_dense_conv(coords, x, w, B, D):
    """Dense zero-padded 3x3x3 cross-correlation, looping over the 27 shifts of
    a padded grid (no hashing, no neighbour lists)."""
    dense = dense_inputs(coords, x, B, D)
    pad = np.zeros((B, x.shape[1], D + 2, D + 2, D + 2))
    pad[:, :, 1:-1, 1:-1, 1:-1] = dense
    out = np.zeros((B, w.shape[2], D, D, D))
    for a in range(3):
        for b in range(3):
            for cc in range(3):
                sh = pad[:, :, a:a + D, b:b + D, cc:cc + D]            # in[p + (a-1, b-1, c-1)]
                out += np.einsum("icxyz,io->ocxyz", sh.transpose(1, 0, 2, 3, 4),
                                 w[9 * a + 3 * b + cc]).transpose(1, 0, 2, 3, 4)
    c = coords.astype(np.int64)
    return out[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]]


def rel_err(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


@pytest.mark.parametrize("seed", [0, 1])
def test_forward_vs_dense_conv(seed):
    rng = np.random.default_rng(100 + seed)
    D, B, ci, co = 9, 2, 3, 5
    coords = W.random_sparse(rng, 300, D=D, B=B)
    coords = coords[rng.permutation(len(coords))]
    x = rng.standard_normal((len(coords), ci))
    w = rng.standard_normal((27, ci, co))
    y = oracle.conv(coords, x, w)[1]
    assert rel_err(y, torch_dense_conv(coords, x, w, B, D)) < 1e-12
    assert rel_err(y, naive_dense_conv(coords, x, w, B, D)) < 1e-12


def test_forward_vs_dense_conv_tiny_config():
    wl = W.make("T")
    y = oracle.conv(wl.coords, wl.x, wl.w)[1]
    ref = torch_dense_conv(wl.coords, wl.x.astype(np.float64), wl.w.astype(np.float64), 1, wl.D)
    assert rel_err(y, ref) < 1e-12


@pytest.mark.parametrize("k", [0, 4, 13, 22, 26])
def test_single_tap(k):
    rng = np.random.default_rng(k)
    D, ci, co = 8, 4, 3
    coords = W.random_sparse(rng, 200, D=D)
    x = rng.standard_normal((len(coords), ci))
    w = np.zeros((27, ci, co))
    w[k] = rng.standard_normal((ci, co))
    nbr, y = oracle.conv(coords, x, w)
    j = nbr[:, k]
    exp = np.where((j >= 0)[:, None], x[np.maximum(j, 0)] @ w[k], 0.0)
    np.testing.assert_allclose(y, exp, rtol=1e-13, atol=1e-13)
    assert rel_err(y, torch_dense_conv(coords, x, w, 1, D)) < 1e-12


# --------------------------------------------------------------------------
# exact special cases and invariances
# --------------------------------------------------------------------------
def test_identity_kernel_exact():
    wl = W.make("S", seed_offset=100, order="shuffled")
    x = wl.x.astype(np.float64)
    w = np.zeros((27, wl.c_in, wl.c_in))
    w[13] = np.eye(wl.c_in)
    y = oracle.conv(wl.coords, x, w)[1]
    np.testing.assert_array_equal(y, x)


def test_isolated_voxel():
    rng = np.random.default_rng(3)
    coords = np.array([[0, 10, 10, 10], [0, 20, 20, 20], [1, 10, 10, 11]], np.int32)
    x = rng.standard_normal((3, 6))
    w = rng.standard_normal((27, 6, 4))
    y = oracle.conv(coords, x, w)[1]
    for i in range(3):
        exp = [sum(x[i, c] * w[13, c, o] for c in range(6)) for o in range(4)]
        np.testing.assert_allclose(y[i], exp, rtol=1e-14, atol=1e-14)


def test_translation_invariance_exact():
    wl = W.make("T", seed_offset=200, order="shuffled")
    nbr, y = oracle.conv(wl.coords, wl.x, wl.w)
    shifted = wl.coords + np.array([0, 1000, 3, 777], np.int32)
    nbr2, y2 = oracle.conv(shifted, wl.x, wl.w)
    np.testing.assert_array_equal(nbr2, nbr)
    np.testing.assert_array_equal(y2, y)


def test_permutation_exact():
    wl = W.make("T", seed_offset=100)
    nbr, y = oracle.conv(wl.coords, wl.x, wl.w)
    pi = np.random.default_rng(5).permutation(wl.n)
    inv = np.argsort(pi)
    nbr2, y2 = oracle.conv(wl.coords[pi], wl.x[pi], wl.w)
    np.testing.assert_array_equal(y2, y[pi])
    exp = np.where(nbr[pi] >= 0, inv[np.maximum(nbr[pi], 0)], -1)
    np.testing.assert_array_equal(nbr2, exp)


def test_batch_isolation_exact():
    rng = np.random.default_rng(11)
    a = W.random_sparse(rng, 400, D=10)
    b = a.copy()
    b[:, 0] = 1                                   # same places, second object
    c = W.random_sparse(rng, 300, D=10)
    c[:, 0] = 2
    coords = np.concatenate([a, b, c])
    x = rng.standard_normal((len(coords), 3))
    w = rng.standard_normal((27, 3, 2))
    nbr, y = oracle.conv(coords, x, w)
    off = 0
    for part in (a, b, c):
        n = len(part)
        nb_p, y_p = oracle.conv(part, x[off:off + n], w)
        np.testing.assert_array_equal(y[off:off + n], y_p)
        np.testing.assert_array_equal(nbr[off:off + n], np.where(nb_p >= 0, nb_p + off, -1))
        off += n


def test_linearity():
    wl = W.make("T")
    rng = np.random.default_rng(9)
    x1 = rng.standard_normal((wl.n, wl.c_in))
    x2 = rng.standard_normal((wl.n, wl.c_in))
    w = wl.w.astype(np.float64)
    nbr = oracle.kernel_map(wl.coords)
    lhs = oracle.forward(nbr, 0.75 * x1 - 2.5 * x2, w)
    rhs = 0.75 * oracle.forward(nbr, x1, w) - 2.5 * oracle.forward(nbr, x2, w)
    assert rel_err(lhs, rhs) < 1e-12


def test_rows_subset_matches_full():
    wl = W.make("S", seed_offset=100)
    nbr = oracle.kernel_map(wl.coords)
    rows = np.random.default_rng(1).choice(wl.n, 500, replace=False)
    full = oracle.forward(nbr, wl.x, wl.w)
    np.testing.assert_array_equal(oracle.forward(nbr, wl.x, wl.w, rows=rows), full[rows])


# --------------------------------------------------------------------------
# fused epilogue: act(conv + bias) + residual
# --------------------------------------------------------------------------
def test_epilogue_values():
    y = np.array([[-2.0, -0.5, 0.0, 0.5, 3.0]])
    bias = np.array([1.0, 0.0, -1.0, 0.25, -3.0])
    res = np.array([[10.0, 20.0, 30.0, 40.0, 50.0]])
    np.testing.assert_array_equal(oracle.epilogue(y), y)
    np.testing.assert_array_equal(oracle.epilogue(y, bias=bias), y + bias)
    np.testing.assert_array_equal(oracle.epilogue(y, act="relu"), [[0.0, 0.0, 0.0, 0.5, 3.0]])
    np.testing.assert_array_equal(oracle.epilogue(y, bias=bias, act="relu", residual=res),
                                  [[10.0, 20.0, 30.0, 40.75, 50.0]])
    # SiLU(v) = v * sigmoid(v): torch's silu in float64 is an independent routine
    v = y + bias
    ref = torch.nn.functional.silu(torch.from_numpy(v)).numpy() + res
    np.testing.assert_allclose(oracle.epilogue(y, bias=bias, act="silu", residual=res), ref,
                               rtol=1e-15, atol=1e-15)
    assert oracle.epilogue(np.array([[0.0]]), act="silu")[0, 0] == 0.0


def test_epilogue_resblock_matches_dense_torch():
    # x + conv2(silu(conv1(x) + b1)) + ... on a tiny grid, against torch's dense conv3d
    rng = np.random.default_rng(21)
    D, c = 7, 4
    coords = W.random_sparse(rng, 150, D=D)
    x = rng.standard_normal((len(coords), c))
    w1, w2 = rng.standard_normal((27, c, c)), rng.standard_normal((27, c, c))
    b1 = rng.standard_normal(c)
    nbr = oracle.kernel_map(coords)
    h = oracle.epilogue(oracle.forward(nbr, x, w1), bias=b1, act="silu")
    out = oracle.epilogue(oracle.forward(nbr, h, w2), residual=x)
    h_ref = torch.nn.functional.silu(torch.from_numpy(torch_dense_conv(coords, x, w1, 1, D) + b1)).numpy()
    out_ref = torch_dense_conv(coords, h_ref, w2, 1, D) + x
    assert rel_err(out, out_ref) < 1e-12


# --------------------------------------------------------------------------
# backward: data and weight gradients of L = sum_i <y[i], dy[i]>
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1])
def test_backward_vs_dense_autograd(seed):
    # torch autograd through a dense float64 conv3d, read at the active sites
    rng = np.random.default_rng(300 + seed)
    D, B, ci, co = 8, 2, 3, 4
    coords = W.random_sparse(rng, 250, D=D, B=B)
    coords = coords[rng.permutation(len(coords))]
    x = rng.standard_normal((len(coords), ci))
    w = rng.standard_normal((27, ci, co))
    dy = rng.standard_normal((len(coords), co))
    c = torch.from_numpy(coords.astype(np.int64))
    dense = torch.from_numpy(dense_inputs(coords, x, B, D)).requires_grad_(True)
    wt = torch.from_numpy(np.ascontiguousarray(w.reshape(3, 3, 3, ci, co).transpose(4, 3, 0, 1, 2)))
    wt.requires_grad_(True)
    out = torch.nn.functional.conv3d(dense, wt, padding=1)
    y = out[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]]
    (y * torch.from_numpy(dy)).sum().backward()
    dx_ref = dense.grad[c[:, 0], :, c[:, 1], c[:, 2], c[:, 3]].numpy()
    dw_ref = wt.grad.numpy().transpose(2, 3, 4, 1, 0).reshape(27, ci, co)
    nbr = oracle.kernel_map(coords)
    assert rel_err(oracle.backward_data(nbr, dy, w), dx_ref) < 1e-12
    assert rel_err(oracle.backward_weights(nbr, x, dy), dw_ref) < 1e-12


def test_backward_adjoint_identities():
    # <conv(x), dy> = <x, dx(dy)> = <w, dw(x, dy)>: the three are the same sum
    wl = W.make("T", seed_offset=50, order="shuffled")
    rng = np.random.default_rng(5)
    dy = rng.standard_normal((wl.n, wl.c_out))
    nbr = oracle.kernel_map(wl.coords)
    a = float((oracle.forward(nbr, wl.x, wl.w) * dy).sum())
    b = float((wl.x.astype(np.float64) * oracle.backward_data(nbr, dy, wl.w)).sum())
    c = float((wl.w.astype(np.float64) * oracle.backward_weights(nbr, wl.x, dy)).sum())
    assert abs(a - b) <= 1e-10 * abs(a) and abs(a - c) <= 1e-10 * abs(a)


def test_backward_subsets_and_single_tap():
    rng = np.random.default_rng(9)
    coords = W.random_sparse(rng, 400, D=10, B=1)
    x = rng.standard_normal((len(coords), 4))
    dy = rng.standard_normal((len(coords), 6))
    w = rng.standard_normal((27, 4, 6))
    nbr = oracle.kernel_map(coords)
    full = oracle.backward_data(nbr, dy, w)
    rows = np.array([5, 0, len(coords) - 1, 17])
    np.testing.assert_array_equal(oracle.backward_data(nbr, dy, w, rows=rows), full[rows])
    dw = oracle.backward_weights(nbr, x, dy)
    sel = np.array([[0, 0], [13, 3], [26, 1], [4, 2]])
    np.testing.assert_array_equal(oracle.backward_weights(nbr, x, dy, sel=sel), dw[sel[:, 0], sel[:, 1]])
    # centre tap: every voxel is its own neighbour, so dw[13] = x^T dy exactly up to rounding
    assert rel_err(dw[13], x.T @ dy) < 1e-12
    # a single non-zero tap k: dx[j] = w[k] dy[i] for the i whose tap k reads j
    k = 5
    wk = np.zeros_like(w)
    wk[k] = w[k]
    ii = np.nonzero(nbr[:, k] >= 0)[0]
    exp = np.zeros((len(coords), 4))
    exp[nbr[ii, k]] = dy[ii] @ w[k].T
    assert rel_err(oracle.backward_data(nbr, dy, wk), exp) < 1e-12


# --------------------------------------------------------------------------
# resolution levels: parents, children, Channel2Spatial regrouping
# --------------------------------------------------------------------------
def test_downsample_brute_force():
    from tests.helpers import morton_keys_numpy
    rng = np.random.default_rng(31)
    coords = W.random_sparse(rng, 700, D=13, B=2)
    coords = coords[rng.permutation(len(coords))]
    coarse, children = oracle.downsample(coords)
    par = {(b, x // 2, y // 2, z // 2) for b, x, y, z in coords.tolist()}
    assert set(map(tuple, coarse.tolist())) == par and len(coarse) == len(par)
    keys = morton_keys_numpy(coarse)
    assert (np.diff(keys.astype(np.float64)) > 0).all()          # strictly in (b, Z-order)
    row = {tuple(r): i for i, r in enumerate(coords.tolist())}
    for q, (b, x, y, z) in enumerate(coarse.tolist()):
        for o in range(8):
            dx, dy, dz = o >> 2, (o >> 1) & 1, o & 1
            assert children[q, o] == row.get((b, 2 * x + dx, 2 * y + dy, 2 * z + dz), -1)
    ch = children[children >= 0]
    np.testing.assert_array_equal(np.sort(ch), np.arange(len(coords)))


def test_subdivide_definition_and_round_trip():
    rng = np.random.default_rng(32)
    coords = W.random_sparse(rng, 300, D=20, B=2)
    keep = rng.integers(0, 256, len(coords)).astype(np.uint8)
    keep[:5] = 0
    fine, children = oracle.subdivide(coords, keep)
    assert len(fine) == int(sum(bin(int(k)).count("1") for k in keep))
    f = 0
    for i, (b, x, y, z) in enumerate(coords.tolist()):
        for o in range(8):
            if (keep[i] >> o) & 1:
                assert fine[f].tolist() == [b, 2 * x + (o >> 2), 2 * y + ((o >> 1) & 1), 2 * z + (o & 1)]
                assert children[i, o] == f
                f += 1
            else:
                assert children[i, o] == -1
    # coarsening the subdivided set gives back the parents that kept a child
    coarse, ch2 = oracle.downsample(fine)
    kept = {tuple(c) for c, k in zip(coords.tolist(), keep) if k}
    assert set(map(tuple, coarse.tolist())) == kept
    back = {tuple(c): i for i, c in enumerate(coords.tolist())}
    for q, c in enumerate(coarse.tolist()):
        np.testing.assert_array_equal(ch2[q], children[back[tuple(c)]])
    all_fine, _ = oracle.subdivide(coords)
    assert len(all_fine) == 8 * len(coords)
    with pytest.raises(oracle.OracleError):
        oracle.subdivide(np.array([[0, 32768, 0, 0]], np.int32))


def test_channel2spatial_is_a_dense_pixel_shuffle():
    # dense 3D pixel shuffle by reshape/permute: channel c*8 + (4dx + 2dy + dz)
    # of coarse cell p goes to channel c of fine cell 2p + (dx, dy, dz)
    rng = np.random.default_rng(33)
    D, B, C = 6, 2, 3
    coords = W.random_sparse(rng, 120, D=D, B=B)
    keep = rng.integers(1, 256, len(coords)).astype(np.uint8)
    fine, children = oracle.subdivide(coords, keep)
    xc = rng.standard_normal((len(coords), 8 * C))
    dense = torch.from_numpy(dense_inputs(coords, xc, B, D))          # [B, 8C, D, D, D]
    fine_dense = (dense.reshape(B, C, 2, 2, 2, D, D, D).permute(0, 1, 5, 2, 6, 3, 7, 4)
                  .reshape(B, C, 2 * D, 2 * D, 2 * D).numpy())
    f = fine.astype(np.int64)
    expect = fine_dense[f[:, 0], :, f[:, 1], f[:, 2], f[:, 3]]
    got = oracle.channel2spatial(children, xc, len(fine))
    np.testing.assert_array_equal(got, expect)
    # Spatial2Channel is its inverse on kept children and puts zeros elsewhere
    back = oracle.spatial2channel(children, got)
    mask = np.repeat((children >= 0)[:, None, :], C, axis=1).reshape(len(coords), 8 * C)
    np.testing.assert_array_equal(back, np.where(mask, xc, 0.0))
