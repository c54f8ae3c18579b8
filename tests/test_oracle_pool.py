"""Pins of the oracle's tile pooling (mean of the 64 tokens of a video tile,
Prism speed-ablation page, section on Prism's block selection)."""
import numpy as np

from synthetic import bf16_bits_to_f32, to_bf16_bits


def test_pool_equals_numpy_mean(orc):
    rng = np.random.default_rng(11)
    B, H, nvt, D, npf = 2, 3, 5, 32, 128
    x = to_bf16_bits(rng.standard_normal((B, H, npf + nvt * 64, D)).astype(np.float32) * 3)
    out = orc.pool(x, npf)
    vid = bf16_bits_to_f32(x[:, :, npf:]).astype(np.float64).reshape(B, H, nvt, 64, D)
    expect = vid.mean(axis=3).astype(np.float32)
    assert out.shape == (B, H, nvt, D)
    np.testing.assert_array_equal(out, expect)


def test_pool_constant_and_ramp_tiles(orc):
    D = 4
    x = np.zeros((1, 1, 128, D), np.float32)
    x[0, 0, :64] = 1.5                     # constant tile
    x[0, 0, 64:] = np.arange(64, dtype=np.float32)[:, None] * 0.25  # ramp 0 .. 15.75
    out = orc.pool(to_bf16_bits(x), 0)
    np.testing.assert_array_equal(out[0, 0, 0], np.full(D, 1.5, np.float32))
    np.testing.assert_array_equal(out[0, 0, 1], np.full(D, 63 * 0.25 / 2, np.float32))


def test_pool_rounds_once_from_exact_sum(orc):
    # one 2^24 and 63 ones: a float running sum would lose every 1; the exact
    # mean 2^18 + 63/64 rounds (to even) to 2^18 + 1 in float.
    x = np.ones((1, 1, 64, 1), np.float32)
    x[0, 0, 0, 0] = 2.0 ** 24
    out = orc.pool(to_bf16_bits(x), 0)
    assert out[0, 0, 0, 0] == np.float32(2.0 ** 18 + 1.0)


def test_pool_ignores_prefix(orc):
    rng = np.random.default_rng(12)
    vid = to_bf16_bits(rng.standard_normal((1, 2, 3 * 64, 8)).astype(np.float32))
    pre = to_bf16_bits(np.full((1, 2, 64, 8), 1000.0, np.float32))
    a = orc.pool(vid, 0)
    b = orc.pool(np.concatenate([pre, vid], axis=2), 64)
    np.testing.assert_array_equal(a, b)
