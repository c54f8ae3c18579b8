"""The seeded input generator: reproducible bytes, bf16 rounding to nearest even."""
import numpy as np
import torch

import synthetic as S


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0, -0.0, 65504.0], np.float32)])
    ours = S.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_slices_are_reproducible_and_independent_of_threads():
    wl = S.Workload("t", 2, 3, 16, (4, 8, 8), 2, seed=9, n_prefix=64)
    a = S.tensor(wl, "k", threads=1)
    b = S.tensor(wl, "k", threads=4)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a[1, :, 2], S.slice_bh(wl, "k", 1, 2))
    assert not np.array_equal(S.tensor(wl, "q"), a)


def test_offsets_recipe_statistics():
    wl = S.Workload("t", 1, 1, 64, (8, 16, 16), 8, seed=0)
    x = S.bf16_bits_to_f32(S.slice_bh(wl, "q", 0, 0)).astype(np.float64)
    # per-tile offsets N(0, 0.25) plus N(0,1) noise: total variance about 1.25
    assert abs(x.var() - 1.25) < 0.1


def test_field_recipe_is_deterministic():
    wl = S.WORKLOADS["prism720p_dynamic"]
    small = S.Workload("f", 1, 1, 8, (8, 8, 16), 2, seed=3, recipe="field", dynamic=True)
    np.testing.assert_array_equal(S.slice_bh(small, "q", 0, 0), S.slice_bh(small, "q", 0, 0))
    assert wl.keep_tiles == 480


def test_workload_flops():
    wl = S.WORKLOADS["prism720p"]
    assert abs(wl.effective_flops() / 1e12 - 92.77) < 0.01
    assert abs(S.WORKLOADS["prefix"].effective_flops() / 1e12 - 33.69) < 0.01
