"""Pins of the oracle's dynamic tile shapes (Prism speed-ablation page, section
on Prism: per 8x8x8 region the most varying axis gets the short extent, the
tile stays at 64 tokens).

Planted fields whose per-axis variation is known in closed form fix both the
statistic and the rule; an independent numpy computation of the statistic
checks the general case.
"""
import numpy as np
from synthetic import bf16_bits_to_f32, to_bf16_bits


def _field(grid, fn, B=1, H=2, D=4, n_prefix=0):
    T, Hg, W = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(W), indexing="ij")
    val = fn(t, h, w).astype(np.float32).reshape(-1)
    x = np.broadcast_to(val[None, :, None, None], (B, T * Hg * W, H, D)).astype(np.float32)
    if n_prefix:
        x = np.concatenate([np.full((B, n_prefix, H, D), 50.0, np.float32), x], axis=1)
    return to_bf16_bits(x)


def _numpy_stats(q_raster, n_prefix, grid):
    T, Hg, W = grid
    B, _, H, D = q_raster.shape
    x = bf16_bits_to_f32(q_raster[:, n_prefix:]).astype(np.float64).reshape(B, T, Hg, W, H, D)
    RT, RH, RW = T // 8, Hg // 8, W // 8
    out = np.empty((B, RT * RH * RW, 3))
    for b in range(B):
        for r in range(RT * RH * RW):
            rt, rh, rw = r // (RH * RW), (r // RW) % RH, r % RW
            blk = x[b, rt * 8:rt * 8 + 8, rh * 8:rh * 8 + 8, rw * 8:rw * 8 + 8]
            for ax in range(3):
                out[b, r, ax] = np.abs(np.diff(blk, axis=ax)).mean()
    return out


def test_stats_match_numpy(orc):
    rng = np.random.default_rng(21)
    grid = (8, 16, 24)
    q = to_bf16_bits(rng.standard_normal((2, 64 + 8 * 16 * 24, 3, 8)).astype(np.float32))
    st = orc.shape_stats(q, 64, grid)
    np.testing.assert_allclose(st, _numpy_stats(q, 64, grid), rtol=1e-13, atol=0)


def test_pure_t_ramp(orc):
    grid = (16, 16, 16)
    q = _field(grid, lambda t, h, w: 0.25 * t, n_prefix=64)
    st = orc.shape_stats(q, 64, grid)
    np.testing.assert_array_equal(st[..., 0], 0.25)
    np.testing.assert_array_equal(st[..., 1:], 0.0)
    shape, near = orc.shape_choose(st, grid, 0.10)
    assert np.all(shape == 1)          # 2x4x8: short on t; h before w on the tie
    assert orc.shape_extent(1) == (2, 4, 8)


def test_pure_h_ramp(orc):
    # a1 = h; t and w tie and t ranks first: a2 = t, a3 = w
    # -> extent 2 on h, 4 on t, 8 on w = 4x2x8 (id 4)
    grid = (8, 16, 16)
    st = orc.shape_stats(_field(grid, lambda t, h, w: 0.5 * h), 0, grid)
    shape, _ = orc.shape_choose(st, grid, 0.10)
    assert np.all(shape == 4)
    assert orc.shape_extent(4) == (4, 2, 8)


def test_t_and_h_vary_w_calm_pairs_into_2x2x16(orc):
    grid = (8, 8, 32)   # 4 regions along w -> two pairs
    st = orc.shape_stats(_field(grid, lambda t, h, w: 0.5 * t + 0.25 * h), 0, grid)
    np.testing.assert_allclose(st[0, :, 0], 0.5)
    np.testing.assert_allclose(st[0, :, 1], 0.25)
    np.testing.assert_allclose(st[0, :, 2], 0.0)
    shape, _ = orc.shape_choose(st, grid, 0.10)
    assert np.all(shape == 7)
    perm = orc.perm_dynamic(shape, grid)
    assert np.array_equal(np.sort(perm[0]), np.arange(8 * 8 * 32))


def test_h_and_w_vary_t_calm_pairs_into_16x2x2(orc):
    grid = (16, 8, 8)
    st = orc.shape_stats(_field(grid, lambda t, h, w: 0.25 * h + 0.5 * w), 0, grid)
    shape, _ = orc.shape_choose(st, grid, 0.10)
    assert np.all(shape == 8)


def test_unpaired_long_request_falls_back_to_box(orc):
    grid = (8, 8, 24)   # 3 regions along w: the third has no partner
    st = orc.shape_stats(_field(grid, lambda t, h, w: 0.5 * t + 0.25 * h), 0, grid)
    shape, _ = orc.shape_choose(st, grid, 0.10)
    np.testing.assert_array_equal(shape[0], [7, 7, 1])


def test_pair_needs_both_regions(orc):
    # region 0 varies in t and h (asks 2x2x16); region 1 varies in t only (box 2x4x8)
    grid = (8, 8, 16)
    st = np.array([[[0.5, 0.25, 0.0], [0.5, 0.0, 0.0]]])
    shape, _ = orc.shape_choose(st, grid, 0.10)
    np.testing.assert_array_equal(shape[0], [1, 1])


def test_tau_infinite_gives_default_everywhere(orc):
    rng = np.random.default_rng(22)
    st = rng.random((2, 2 * 3 * 4, 3))
    shape, _ = orc.shape_choose(st, (16, 24, 32), np.inf)
    assert np.all(shape == 0)


def test_isotropic_threshold_and_near_flags(orc):
    grid = (8, 8, 8)
    st = np.array([[[1.09, 1.0, 1.0]], [[1.11, 1.0, 1.0]], [[1.0, 1.0, 1.0]]])
    shape, near = orc.shape_choose(st, grid, 0.10)
    assert shape[0, 0] == 0 and shape[1, 0] == 1 and shape[2, 0] == 0
    assert near[0, 0] == 1  # h and w tie exactly
    assert near[2, 0] == 1
    # t and h vary, w calm: asks for 2x2x16, but a lone region has no partner
    st2 = np.array([[[3.0, 2.0, 1.0]]])
    shape2, near2 = orc.shape_choose(st2, grid, 0.10)
    assert shape2[0, 0] == 1 and near2[0, 0] == 0
