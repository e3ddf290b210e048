"""Pins of the oracle's Markov draft sampler and confidence head (CPU only).

Pages: "[2/3] feat(dsv4): implement exact DSpark speculative decoding",
"Checkpoint-faithful DSpark architecture" (the Markov head is sampled left to
right, the first proposal conditioning on the anchor; q and the confidence
scores are kept) and "DSpark Speculative Decoding (Draft Training) Design",
"Semi-autoregressive draft" (rank-r additive logit bias; confidence head
sigmoid(w . [h_k ; embed(x_{k-1})])).

Pins:
* zero Markov weights: q_k is the textbook softmax of the backbone row / T
  (scipy), and the chain no longer depends on the anchor;
* chain construction: a bias of +100 on token (x + 1) forces x_k = x_0 + k,
  which fixes the anchor conditioning and the left-to-right order;
* rank one: the bias is the outer product a_x b_v (greedy argmax checked);
* conditional law: with a moderate chain bias, x_2 given x_1 follows the
  softmax of backbone row 1 plus the bias of x_1 (chi-square);
* confidence head: w = 0 gives 1/2, w = e_i picks sigmoid(h[i]) or
  sigmoid(E[x_{k-1}][i]) (the [h ; E] order and the anchor at k = 1).
"""

from __future__ import annotations

import numpy as np
import pytest
from scipy.special import expit, logsumexp

from tests._cases import chisq_pvalue, decode_case, softmax64
from workloads import bf16_to_f32, decode_inputs, to_bf16


def test_zero_bias_gives_plain_softmax(oracle):
    rng = np.random.default_rng(1)
    B, g, V = 3, 4, 700
    bb = rng.normal(0, 2, (B, g, V)).astype(np.float32)
    inp = decode_case(bb, r=16, anchor=[5, 9, 600], temperature=[1.0, 0.5, 1.3])
    out = oracle.markov_sample(inp)
    T = inp["temperature"].astype(np.float64)
    for b in range(B):
        for k in range(g):
            z = bb[b, k].astype(np.float64) / T[b]
            assert np.array_equal(out["q_z"][b, k], z)
            assert out["q_lse"][b, k] == pytest.approx(logsumexp(z), rel=1e-14)
            x = out["draft_tokens"][b, k]
            assert out["q_tok"][b, k] == pytest.approx(np.exp(z[x] - logsumexp(z)), rel=1e-12)
    inp2 = decode_case(bb, r=16, anchor=[1, 2, 3], temperature=[1.0, 0.5, 1.3])
    assert np.array_equal(oracle.markov_sample(inp2)["draft_tokens"], out["draft_tokens"])


@pytest.mark.parametrize("mode", [0, 1])
def test_chain_forces_left_to_right_order(oracle, mode):
    V, r, g = 16, 16, 5
    w1 = np.eye(V, r, dtype=np.float32)
    w2 = 100.0 * np.roll(np.eye(V, r, dtype=np.float32), 1, axis=0)  # row v = e_{v-1}
    bb = np.random.default_rng(2).normal(0, 1, (3, g, V)).astype(np.float32)
    inp = decode_case(bb, r=r, w1=w1, w2=w2, anchor=[0, 7, 13], mode=mode)
    out = oracle.markov_sample(inp)
    for b, a in enumerate([0, 7, 13]):
        assert list(out["draft_tokens"][b]) == [(a + k) % V for k in range(1, g + 1)]


def test_chain_across_chunks(oracle):
    V, r, g = 600, 16, 5
    w1 = np.zeros((V, r), np.float32)
    w1[np.arange(V), np.arange(V) % r] = 1.0
    w2 = np.zeros((V, r), np.float32)
    w2[1:17] = 100.0 * np.eye(16, r, dtype=np.float32)  # token v in 1..16 <- code v-1
    inp = decode_case(np.zeros((1, g, V), np.float32), r=r, w1=w1, w2=w2, anchor=590, mode=1)
    out = oracle.markov_sample(inp)
    # 590 % 16 = 14 -> 15 -> 16 -> (16 % 16 = 0) 1 -> 2 -> 3
    assert list(out["draft_tokens"][0]) == [15, 16, 1, 2, 3]


def test_rank_one_bias_greedy(oracle):
    rng = np.random.default_rng(3)
    V, r, g = 300, 16, 3
    a = to_bf16(rng.normal(0, 1, V).astype(np.float32))
    bvec = to_bf16(rng.normal(0, 1, V).astype(np.float32))
    w1 = np.zeros((V, r), np.float32)
    w1[:, 0] = bf16_to_f32(a)
    w2 = np.zeros((V, r), np.float32)
    w2[:, 0] = bf16_to_f32(bvec)
    bb = rng.normal(0, 1, (1, g, V)).astype(np.float32)
    inp = decode_case(bb, r=r, w1=w1, w2=w2, anchor=17, mode=0)
    out = oracle.markov_sample(inp)
    x = 17
    for k in range(g):
        y = bb[0, k].astype(np.float64) + np.float64(bf16_to_f32(a)[x]) * bf16_to_f32(bvec).astype(np.float64)
        x = int(np.argmax(y))
        assert out["draft_tokens"][0, k] == x


def test_conditional_law_of_second_proposal(oracle):
    V, r, g, n = 8, 16, 2, 24000
    rng = np.random.default_rng(4)
    row0 = rng.normal(0, 1, V)
    row1 = rng.normal(0, 1, V)
    bb = np.broadcast_to(np.stack([row0, row1])[None].astype(np.float32), (n, g, V))
    w1 = np.eye(V, r, dtype=np.float32)
    w2 = 1.5 * np.roll(np.eye(V, r, dtype=np.float32), 1, axis=0)
    inp = decode_case(np.ascontiguousarray(bb), r=r, w1=w1, w2=w2, anchor=3, mode=1)
    out = oracle.markov_sample(inp, want_q=False)
    x1, x2 = out["draft_tokens"][:, 0], out["draft_tokens"][:, 1]
    bias0 = np.zeros(V)
    bias0[4] = 1.5  # anchor 3 -> +1.5 on token 4
    assert chisq_pvalue(x1, softmax64(row0 + bias0)) > 1e-4
    for x in np.unique(x1)[np.bincount(x1)[np.unique(x1)] > 2000]:
        bias = np.zeros(V)
        bias[(x + 1) % V] = 1.5
        assert chisq_pvalue(x2[x1 == x], softmax64(row1 + bias)) > 1e-4


def test_confidence_head(oracle):
    rng = np.random.default_rng(5)
    B, g, V, d = 2, 3, 40, 8
    hidden = rng.normal(0, 1, (B, g, d)).astype(np.float32)
    embed = rng.normal(0, 1, (V, d)).astype(np.float32)
    bb = rng.normal(0, 1, (B, g, V)).astype(np.float32)
    base = dict(r=16, d=d, hidden=hidden, embed=embed, anchor=[4, 31], mode=0)
    out = oracle.markov_sample(decode_case(bb, **base))
    assert np.all(out["confidence"] == 0.5)
    h16, e16 = bf16_to_f32(to_bf16(hidden)), bf16_to_f32(to_bf16(embed))
    for i in [0, 5]:
        w = np.zeros(2 * d, np.float32)
        w[i] = 1.0
        o = oracle.markov_sample(decode_case(bb, conf_w=w, **base))
        assert np.allclose(o["confidence"], expit(h16[:, :, i].astype(np.float64)), rtol=1e-15)
        w = np.zeros(2 * d, np.float32)
        w[d + i] = 1.0
        o = oracle.markov_sample(decode_case(bb, conf_w=w, **base))
        prev = np.concatenate([np.array([[4], [31]]), o["draft_tokens"][:, :-1]], axis=1)
        assert np.allclose(o["confidence"], expit(e16[prev, i].astype(np.float64)), rtol=1e-15)


def test_tiny_workload_runs_and_is_deterministic(oracle):
    inp = decode_inputs("tiny")
    a = oracle.markov_sample(inp)
    b = oracle.markov_sample(inp)
    assert np.array_equal(a["draft_tokens"], b["draft_tokens"])
    assert np.all((a["draft_tokens"] >= 0) & (a["draft_tokens"] < inp["V"]))
    assert np.all((a["confidence"] > 0) & (a["confidence"] < 1))
    # forced tokens replace the draw and the chain follows them
    forced = np.full((inp["B"], inp["gamma"]), -1, np.int32)
    forced[:, 1] = 7
    c = oracle.markov_sample(inp, forced_tokens=forced)
    assert np.all(c["draft_tokens"][:, 1] == 7)
    assert np.array_equal(c["draft_tokens"][:, 0], a["draft_tokens"][:, 0])
