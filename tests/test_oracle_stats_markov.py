"""Pins of the oracle's statistics of the teacher-forced Markov draft (CPU).

Pages: "DSpark Speculative Decoding (Draft Training) Design",
"Semi-autoregressive draft" (the Markov head adds a low-rank,
token-conditioned bias to the parallel logits; at training time it is
teacher-forced with the previous block tokens) and "Training objective".
Reading: the draft row of position k is backbone + W1[x_{k-1}] W2^T with
x_0 the block's anchor and x_{k-1} the teacher token of position k-1.

Pins:
- zero Markov factors: exactly the statistics of the backbone rows;
- the Markov oracle itself (pinned on its own), run at temperature 1 with
  every drawn token forced to the teacher token, produces z rows whose
  statistics (binary64 rows, no rounding) equal these bit for bit;
- a rank-one factor pair: bias = u[x] w[v], built with numpy outer products.
"""

from __future__ import annotations

import numpy as np

from tests._cases import decode_case
from workloads import bf16_to_f32, stats_markov_inputs, to_bf16

CFG = dict(seed=31, N=5, gamma=4, V=700, dtype="f32", draft_std=2.0, noise_std=0.7)


def small(r=32, **kw):
    return stats_markov_inputs(dict(CFG, **kw), r=r, w_std=0.2)


def test_zero_factors_equal_backbone_statistics(oracle):
    inp = small()
    inp["w1"] = np.zeros_like(inp["w1"])
    a = oracle.accept_stats_markov(inp)
    b = oracle.accept_stats(dict(inp, draft=inp["backbone"]))
    for key in ["l1", "accept_rate", "ce", "bce", "tau", "sums"]:
        assert np.array_equal(a[key], b[key]), key


def test_equals_forced_markov_chain(oracle):
    inp = small(mask_every=3)
    N, g, V, r = inp["N"], inp["gamma"], inp["V"], inp["r"]
    # the Markov oracle on the same backbone, sampled at T = 1 without
    # truncation (z = y), every proposal forced to the teacher token
    dc = decode_case(inp["backbone"], np.zeros((N, g + 1, V), np.float32), r=r, d=8,
                     anchor=inp["anchor"], w1=bf16_to_f32(inp["w1"]), w2=bf16_to_f32(inp["w2"]),
                     mode=1, temperature=1.0)
    mk = oracle.markov_sample(dc, forced_tokens=inp["teacher"])
    assert np.array_equal(mk["draft_tokens"], inp["teacher"])
    via_chain = oracle.accept_stats_f64_draft(mk["q_z"], inp)
    direct = oracle.accept_stats_markov(inp)
    for key in ["l1", "accept_rate", "ce", "bce", "tau", "sums"]:
        assert np.array_equal(via_chain[key], direct[key]), key


def test_rank_one_closed_form(oracle):
    inp = small(r=16)
    V, r = inp["V"], inp["r"]
    rng = np.random.default_rng(2)
    u = to_bf16(rng.normal(0, 1, V).astype(np.float32))
    w = to_bf16(rng.normal(0, 1, V).astype(np.float32))
    w1 = np.zeros((V, r), np.uint16)
    w2 = np.zeros((V, r), np.uint16)
    w1[:, 3], w2[:, 3] = u, w
    inp["w1"], inp["w2"] = w1, w2
    N, g = inp["N"], inp["gamma"]
    x = np.concatenate([inp["anchor"][:, None], inp["teacher"][:, :-1]], axis=1)
    draft = inp["backbone"].astype(np.float64) + \
        bf16_to_f32(u)[x][..., None].astype(np.float64) * bf16_to_f32(w)[None, None, :].astype(np.float64)
    ref = oracle.accept_stats_f64_draft(draft, inp)
    got = oracle.accept_stats_markov(inp)
    for key in ["l1", "accept_rate", "ce", "bce", "tau", "sums"]:
        assert np.allclose(got[key], ref[key], rtol=1e-13, atol=1e-13), key
