"""Pins of the oracle's training-side acceptance statistics (CPU only).

Pages: "DSpark Speculative Decoding (Draft Training) Design", sections
"Training objective" (position weights exp(-k/gamma); 0.1 CE + 0.9 L1 +
1.0 BCE), "Acceptance and confidence" (raw L1, accept_rate =
clamp(1 - 0.5 L1, 0, 1), tau = sum cumprod + 1) and "Loss return contract"
(unnormalised numerator, token count and [sum, count] report pairs, normalised
once after reduction).

Pins: the pages' own fixed points (tests/golden/accept_stats_fixed_points.txt);
L1 == 2 (1 - sum_v min(P, T)) (an independent formula, scipy softmax); CE and
BCE against torch's cross_entropy and binary_cross_entropy_with_logits in
binary64; a uniform draft gives CE = ln V; c = 0 gives BCE = ln 2 for any
label; closed-form numerator of a one-position block; the masked-block and
two-shard reduction contract.
"""

from __future__ import annotations

import os

import numpy as np
import pytest
import torch
from scipy.special import softmax

from tests._cases import stats_case
from workloads import bf16_to_f32, stats_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden", "accept_stats_fixed_points.txt")


def golden():
    rows = {}
    for line in open(GOLD):
        if line.strip() and not line.startswith("#"):
            name, l1, a, tau = line.split()
            rows[name] = (float(l1), float(a), float(tau))
    return rows


def test_page_fixed_points(oracle):
    g = golden()
    V, gamma = 64, 7
    rng = np.random.default_rng(0)
    d = np.full((1, gamma, V), -np.inf, np.float32)
    t = np.full((1, gamma, V), -np.inf, np.float32)
    d[..., :32] = rng.normal(0, 1, (1, gamma, 32))
    t[..., 32:] = rng.normal(0, 1, (1, gamma, 32))
    o = oracle.accept_stats(stats_case(d, t))
    l1, a, tau = g["disjoint"]
    # exact in real arithmetic; binary64 sums of the normalised rows round
    assert np.allclose(o["l1"], l1, rtol=0, atol=1e-14)
    assert np.allclose(o["accept_rate"], a, rtol=0, atol=1e-14)
    assert o["tau"][0] == pytest.approx(tau, abs=1e-14)
    same = rng.normal(0, 2, (1, gamma, V)).astype(np.float32)
    o = oracle.accept_stats(stats_case(same, same))
    l1, a, tau = g["identical"]
    assert np.all(o["l1"] == l1) and np.all(o["accept_rate"] == a) and o["tau"][0] == tau


def test_l1_equals_two_minus_twice_overlap(oracle):
    rng = np.random.default_rng(1)
    d = rng.normal(0, 3, (3, 4, 500)).astype(np.float32)
    t = (d + rng.normal(0, 1, d.shape)).astype(np.float32)
    o = oracle.accept_stats(stats_case(d, t))
    P = softmax(d.astype(np.float64), axis=-1)
    T = softmax(t.astype(np.float64), axis=-1)
    overlap = np.minimum(P, T).sum(-1)
    assert np.allclose(o["l1"], 2.0 * (1.0 - overlap), rtol=1e-12, atol=1e-14)
    assert np.allclose(o["accept_rate"], overlap, rtol=1e-12)
    cum = np.cumprod(overlap, axis=1)
    assert np.allclose(o["tau"], 1.0 + cum.sum(1), rtol=1e-12)


def test_ce_and_bce_match_torch(oracle):
    rng = np.random.default_rng(2)
    N, g, V = 4, 3, 300
    d = rng.normal(0, 2, (N, g, V)).astype(np.float32)
    t = (d + rng.normal(0, 1, d.shape)).astype(np.float32)
    teacher = rng.integers(0, V, (N, g)).astype(np.int32)
    c = rng.normal(0, 1, (N, g)).astype(np.float32)
    o = oracle.accept_stats(stats_case(d, t, teacher, c))
    ce = torch.nn.functional.cross_entropy(torch.from_numpy(d.astype(np.float64)).reshape(-1, V),
                                           torch.from_numpy(teacher.astype(np.int64)).reshape(-1),
                                           reduction="none").reshape(N, g).numpy()
    assert np.allclose(o["ce"], ce, rtol=1e-12)
    bce = torch.nn.functional.binary_cross_entropy_with_logits(
        torch.from_numpy(c.astype(np.float64)), torch.from_numpy(o["accept_rate"]),
        reduction="none").numpy()
    assert np.allclose(o["bce"], bce, rtol=1e-12)


def test_uniform_draft_and_zero_confidence(oracle):
    V = 1000
    d = np.zeros((2, 2, V), np.float32)
    t = np.random.default_rng(3).normal(0, 1, (2, 2, V)).astype(np.float32)
    o = oracle.accept_stats(stats_case(d, t, teacher=np.full((2, 2), 17)))
    assert np.allclose(o["ce"], np.log(V), rtol=1e-14)
    assert np.allclose(o["bce"], np.log(2.0), rtol=1e-14)


def test_numerator_closed_form_one_position(oracle):
    V = 50
    d = np.zeros((1, 1, V), np.float32)
    o = oracle.accept_stats(stats_case(d, d, teacher=np.array([[3]])))
    # identical rows: L1 = 0, a = 1; uniform draft: CE = ln V; c = 0: BCE = ln 2
    want = np.exp(-1.0) * (0.1 * np.log(V) + 0.9 * 0.0 + 1.0 * np.log(2.0))
    assert o["sums"][0] == pytest.approx(want, rel=1e-14)
    assert o["sums"][1] == 1.0


def test_mask_and_two_shard_reduction(oracle):
    inp = stats_inputs(dict(seed=7, N=6, gamma=3, V=700, dtype="bf16", draft_std=3.0,
                            noise_std=1.0), mask_every=3)
    full = oracle.accept_stats(inp)
    assert full["sums"][1] == 3 * 4 and full["sums"][7] == 4  # blocks 2 and 5 masked
    parts = []
    for lo, hi in [(0, 2), (2, 6)]:
        sub = dict(inp, draft=inp["draft"][lo:hi], target=inp["target"][lo:hi],
                   teacher=inp["teacher"][lo:hi], conf_logits=inp["conf_logits"][lo:hi],
                   block_mask=inp["block_mask"][lo:hi], N=hi - lo)
        parts.append(oracle.accept_stats(sub)["sums"])
    assert np.allclose(parts[0] + parts[1], full["sums"], rtol=1e-13)
    # masked blocks still get their per-position outputs
    assert np.all(full["l1"][2] > 0)
    # a masked block adds nothing
    unmasked = oracle.accept_stats(dict(inp, block_mask=None))
    assert unmasked["sums"][1] == 3 * 6
    # bf16 inputs are read exactly: the same values given as fp32 agree
    f32 = dict(inp, draft=bf16_to_f32(inp["draft"]), target=bf16_to_f32(inp["target"]), dtype="f32")
    assert np.array_equal(oracle.accept_stats(f32)["l1"], full["l1"])
