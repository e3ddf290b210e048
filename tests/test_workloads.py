"""The seeded input generator: determinism and exact regeneration of subsets."""

import numpy as np

from workloads import bf16_to_f32, decode_inputs, stats_inputs, to_bf16


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e-3], np.float32)
    h = to_bf16(x)
    back = bf16_to_f32(h)
    assert back[0] == 1.0 and back[1] == 1.0          # tie -> even
    assert back[2] == np.float32(1.0078125)           # above the tie -> up
    assert back[3] == -2.5
    assert abs(back[4] - 3.0e-3) <= 3.0e-3 * 2 ** -8


def test_decode_subset_regenerates_exactly():
    cfg = dict(seed=5, B=6, gamma=3, V=300, r=16, d=8, dtype="bf16", draft_std=3.0,
               noise_std=1.0, w_std=0.02, mode="mixed", policy="random", zipf=1.1)
    full = decode_inputs(cfg)
    sub = decode_inputs(cfg, requests=[4, 1])
    for key in ["backbone", "target", "anchor", "hidden", "mode", "temperature", "top_k", "top_p",
                "position"]:
        assert np.array_equal(sub[key], full[key][[4, 1]]), key
    assert np.array_equal(sub["w1"], full["w1"]) and np.array_equal(sub["embed"], full["embed"])
    assert list(full["mode"]) == [1, 0, 1, 0, 1, 0]
    assert np.array_equal(bf16_to_f32(full["backbone"]), bf16_to_f32(full["target"][:, :3]) * 0
                          + bf16_to_f32(full["backbone"]))


def test_stats_subset_and_mask():
    cfg = dict(seed=9, N=5, gamma=2, V=64, dtype="f32", draft_std=3.0, noise_std=1.0)
    full = stats_inputs(cfg, mask_every=2)
    sub = stats_inputs(cfg, blocks=[3], mask_every=2)
    assert np.array_equal(sub["draft"][0], full["draft"][3])
    assert list(full["block_mask"]) == [1, 0, 1, 0, 1]
    assert sub["block_mask"][0] == 0
