"""Synthetic workload generator: sizes, determinism, bf16 encoding, structure."""
import numpy as np
import pytest
import torch

import oracle
from gen import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        np.array([1.0, -0.0, 1e-40, 3.0e38, 1.00390625, 1.01171875], np.float32)])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(W.f32_to_bf16_bits(a), ref)
    back = W.bf16_bits_to_f32(ref)
    np.testing.assert_array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                                  .float().numpy())


def test_deterministic():
    a = W.make("S", seed_offset=100, order="shuffled")
    b = W.make("S", seed_offset=100, order="shuffled")
    np.testing.assert_array_equal(a.coords, b.coords)
    np.testing.assert_array_equal(a.x, b.x)
    np.testing.assert_array_equal(a.w, b.w)
    c = W.make("S", seed_offset=200)
    assert c.n != a.n or not np.array_equal(c.coords, a.coords)


def test_sizes_and_ranges():
    t = W.make("T", with_values=False)
    assert 400 <= t.n <= 500
    s = W.make("S", with_values=False)
    assert 15_000 <= s.n <= 25_000
    w = W.make("W", with_values=False)
    per = np.bincount(w.coords[:, 0])
    assert len(per) == 4 and (per >= 15_000).all() and (per <= 30_000).all()
    assert len(set(per.tolist())) == 4
    l = W.make("L", with_values=False)
    assert 350_000 <= l.n <= 450_000
    x = W.make("X", with_values=False)
    assert 1_200_000 <= x.n <= 1_800_000
    for wl in (t, s, w, l, x):
        c = wl.coords
        assert c.dtype == np.int32 and c.shape[1] == 4
        assert (c[:, 1:] >= 0).all() and (c[:, 1:] < wl.D).all()
        assert (c[:, 0] >= 0).all() and (c[:, 0] < wl.B).all()
        lin = ((c[:, 0].astype(np.int64) * wl.D + c[:, 1]) * wl.D + c[:, 2]) * wl.D + c[:, 3]
        assert (np.diff(lin) > 0).all()          # raster order, no duplicates


def test_value_distributions():
    wl = W.make("S")
    assert wl.x.dtype == np.float32 and wl.x.shape == (wl.n, 64)
    np.testing.assert_array_equal(W.round_to_bf16(wl.x), wl.x)
    np.testing.assert_array_equal(W.round_to_bf16(wl.w), wl.w)
    assert abs(wl.x.std() - 1.0) < 0.02
    assert abs(wl.w.std() * np.sqrt(27 * 64) - 1.0) < 0.02
    t = W.make("T")
    assert not np.array_equal(W.round_to_bf16(t.x), t.x)   # fp32 config keeps fp32 values


def test_fbm_period_selection_rule():
    p, counts = W.select_fbm_period(W.CONFIGS["L"]["seed"])
    assert p == W.FBM_PERIOD_L, counts


def test_clustered_config_has_sparse_neighbourhoods():
    wl = W.make("X", with_values=False)
    deg = (oracle.kernel_map(wl.coords) >= 0).sum(axis=1) - 1     # excluding self
    frac = float((deg < 6).mean())
    assert frac >= 0.25, frac


@pytest.mark.parametrize("name", ["S", "L"])
def test_shell_thickness(name):
    # thickness-2 shells: most voxels see 10-26 neighbours (r = M/N well above 9)
    wl = W.make(name, with_values=False)
    r = (oracle.kernel_map(wl.coords) >= 0).sum() / wl.n
    assert 12 <= r <= 22, r
