"""Pins of the oracle's exact verify (CPU only).

Pages: "[2/3] feat(dsv4): implement exact DSpark speculative decoding",
"Exact decoding semantics": greedy accepts the contiguous prefix equal to the
target argmax and emits the target token at the first disagreement, never
accepting a later accidental match ("Greedy"); sampled accepts x with
probability min(1, p(x)/q(x)), resamples the first rejection from normalised
max(p - q, 0), and draws a bonus token from the next-position target
distribution on full survival, so that the output is distributed exactly as
target-only sampling ("Probabilistic").  "DeepSeek V4 DSpark NPU Serving Dev
Notes", "Speculative decoding (K=7)": 1..8 tokens per step at K = 7.

Pins: hand-built greedy cases; p == q accepts everything; disjoint supports
reject at once and emit a p-distributed token; a one-hot q accepts with
probability p(x) and otherwise emits p without x; chi-square that the first,
second and bonus emitted tokens follow the target rows in agreeing,
disagreeing and nearly disjoint regimes; the acceptance frequency at the first
proposal equals sum_v min(p_v, q_v), which the acceptance statistics give as
1 - L1/2 (links the verify to the training-side statistics).
"""

from __future__ import annotations

import numpy as np
import pytest

from tests._cases import binom_pvalue, chisq_pvalue, decode_case, softmax64, stats_case


def onehot_rows(tokens, V, hi=10.0):
    rows = np.zeros((len(tokens), V), np.float32)
    rows[np.arange(len(tokens)), tokens] = hi
    return rows


# ---------------------------------------------------------------- greedy ----
def greedy_case(oracle, draft, targets, V=32, n_draft=None):
    g = len(draft)
    tgt = onehot_rows(targets, V)[None]
    inp = decode_case(None, tgt, B=1, gamma=g, V=V, mode=0)
    return oracle.verify(inp, np.array([draft], np.int32),
                         n_draft=None if n_draft is None else np.array([n_draft], np.int32))


def test_greedy_all_match_emits_bonus(oracle):
    o = greedy_case(oracle, [3, 4, 5, 6, 7], [3, 4, 5, 6, 7, 9])
    assert o["accept_len"][0] == 5
    assert list(o["out_tokens"][0]) == [3, 4, 5, 6, 7, 9]


def test_greedy_first_mismatch(oracle):
    o = greedy_case(oracle, [3, 4, 5, 6, 7], [3, 4, 11, 6, 7, 9])
    assert o["accept_len"][0] == 2
    assert list(o["out_tokens"][0]) == [3, 4, 11, -1, -1, -1]


def test_greedy_never_accepts_after_a_mismatch(oracle):
    # x_1 mismatches, x_2..x_5 all match their rows: still only the target token
    o = greedy_case(oracle, [3, 4, 5, 6, 7], [20, 4, 5, 6, 7, 9])
    assert o["accept_len"][0] == 0
    assert list(o["out_tokens"][0]) == [20, -1, -1, -1, -1, -1]


def test_greedy_k7_emits_one_to_eight_tokens(oracle):
    draft = [1, 2, 3, 4, 5, 6, 7]
    for n in range(8):
        targets = draft[:n] + [30] + [0] * (7 - n) if n < 7 else draft + [30]
        o = greedy_case(oracle, draft, targets)
        assert o["accept_len"][0] == n
        emitted = [t for t in o["out_tokens"][0] if t >= 0]
        assert len(emitted) == n + 1 and emitted[-1] == 30


def test_greedy_ties_take_lowest_index(oracle):
    tgt = np.zeros((1, 2, 8), np.float32)
    tgt[0, 0, [2, 5]] = 3.0
    tgt[0, 1, [6, 1]] = 3.0
    inp = decode_case(None, tgt, B=1, gamma=1, V=8, mode=0)
    o = oracle.verify(inp, np.array([[2]], np.int32))
    assert list(o["out_tokens"][0]) == [2, 1]


def test_greedy_n_draft_moves_bonus_row(oracle):
    o = greedy_case(oracle, [3, 4, 5, 6, 7], [3, 4, 9, 6, 7, 9], n_draft=2)
    assert o["accept_len"][0] == 2 and list(o["out_tokens"][0]) == [3, 4, 9, -1, -1, -1]
    o = greedy_case(oracle, [3, 4, 5, 6, 7], [3, 4, 9, 6, 7, 9], n_draft=0)
    assert o["accept_len"][0] == 0 and list(o["out_tokens"][0]) == [3, -1, -1, -1, -1, -1]


# --------------------------------------------------------------- sampled ----
def q_from_rows(oracle, rows, T=1.0):
    """Stored-format q (z, lse, thr) of draft rows [B,g,V] under temperature T."""
    B, g, V = rows.shape
    qz = np.zeros((B, g, V), np.float32)
    lse = np.zeros((B, g), np.float32)
    thr = np.full((B, g), -np.inf, np.float32)
    for b in range(B):
        for k in range(g):
            _, z, l, t, _ = oracle.policy_row(rows[b, k], T, 0, 1.0)
            qz[b, k], lse[b, k], thr[b, k] = z, l, t
    return qz, lse, thr


def sampled_run(oracle, p_rows, q_rows, n, seed=0, rng_seed=0):
    """n independent requests verifying x_k ~ q_k against fixed target rows."""
    g1, V = p_rows.shape
    g = g1 - 1
    rng = np.random.default_rng(rng_seed)
    qd = [softmax64(q_rows[k]) for k in range(g)]
    draft = np.stack([rng.choice(V, size=n, p=qd[k]) for k in range(g)], axis=1).astype(np.int32)
    tgt = np.broadcast_to(p_rows[None].astype(np.float32), (n, g1, V))
    inp = decode_case(None, np.ascontiguousarray(tgt), B=n, gamma=g, V=V, mode=1, seed=seed)
    qz1, lse1, thr1 = q_from_rows(oracle, q_rows[None])
    qz = np.broadcast_to(qz1, (n, g, V))
    lse = np.broadcast_to(lse1, (n, g))
    thr = np.broadcast_to(thr1, (n, g))
    q_tok = np.stack([qd[k][draft[:, k]] for k in range(g)], axis=1)
    return oracle.verify(inp, draft, qz, lse, thr, q_tok), draft


def test_identical_p_q_accepts_everything(oracle):
    rng = np.random.default_rng(10)
    rows = rng.normal(0, 1, (4, 12))
    o, draft = sampled_run(oracle, rows, rows[:3], 3000)
    assert np.all(o["accept_len"] == 3)
    assert np.array_equal(o["out_tokens"][:, :3], draft)
    assert chisq_pvalue(o["out_tokens"][:, 3], softmax64(rows[3])) > 1e-4  # bonus ~ p_gamma


def test_disjoint_supports_reject_and_emit_p(oracle):
    V = 10
    p_rows = np.full((3, V), -np.inf)
    p_rows[:, :5] = np.random.default_rng(11).normal(0, 1, (3, 5))
    q_rows = np.full((2, V), -np.inf)
    q_rows[:, 5:] = 0.0
    o, _ = sampled_run(oracle, p_rows, q_rows, 4000)
    assert np.all(o["accept_len"] == 0)
    assert chisq_pvalue(o["out_tokens"][:, 0], softmax64(p_rows[0])) > 1e-4


def test_one_hot_q_accept_probability_and_residual(oracle):
    V, x = 9, 4
    p_rows = np.random.default_rng(12).normal(0, 1, (2, V))
    q_rows = np.full((1, V), -np.inf)
    q_rows[0, x] = 0.0
    n = 20000
    o, _ = sampled_run(oracle, p_rows, q_rows, n)
    p0 = softmax64(p_rows[0])
    acc = o["accept_len"] == 1
    assert binom_pvalue(acc.sum(), n, p0[x]) > 1e-4
    resid = p0.copy()
    resid[x] = 0.0
    assert chisq_pvalue(o["out_tokens"][~acc, 0], resid / resid.sum()) > 1e-4


@pytest.mark.parametrize("regime", ["agreeing", "disagreeing", "nearly_disjoint"])
def test_emitted_tokens_follow_target(oracle, regime):
    V, g, n = 12, 2, 30000
    rng = np.random.default_rng({"agreeing": 20, "disagreeing": 21, "nearly_disjoint": 22}[regime])
    p_rows = rng.normal(0, 1.5, (g + 1, V))
    if regime == "agreeing":
        q_rows = p_rows[:g] + rng.normal(0, 0.3, (g, V))
    elif regime == "disagreeing":
        q_rows = rng.normal(0, 1.5, (g, V))
    else:
        q_rows = -p_rows[:g] * 4.0
    o, _ = sampled_run(oracle, p_rows, q_rows, n, seed=3)
    out, al = o["out_tokens"], o["accept_len"]
    assert chisq_pvalue(out[:, 0], softmax64(p_rows[0])) > 1e-4
    two = al >= 1
    assert chisq_pvalue(out[two, 1], softmax64(p_rows[1])) > 1e-4
    full = al == g
    if full.sum() > 200:
        assert chisq_pvalue(out[full, g], softmax64(p_rows[g])) > 1e-4
    # acceptance of x_1 happens with probability sum_v min(p, q) = 1 - L1/2
    st = oracle.accept_stats(stats_case(q_rows[None, :1].astype(np.float32),
                                        p_rows[None, :1].astype(np.float32)))
    pa = st["accept_rate"][0, 0]
    p0, q1 = softmax64(p_rows[0].astype(np.float32)), softmax64(q_rows[0].astype(np.float32))
    assert pa == pytest.approx(np.minimum(p0, q1).sum(), rel=1e-9)
    assert binom_pvalue((al >= 1).sum(), n, pa) > 1e-4


def test_sampled_with_top_k_policy_emits_only_kept_tokens(oracle):
    V, n = 30, 3000
    rng = np.random.default_rng(30)
    p_rows = rng.normal(0, 2, (2, V))
    q_rows = rng.normal(0, 2, (1, V))
    tgt = np.broadcast_to(p_rows[None].astype(np.float32), (n, 2, V))
    inp = decode_case(None, np.ascontiguousarray(tgt), B=n, gamma=1, V=V, mode=1, top_k=3,
                      temperature=0.8)
    kq, zq, lq, tq, _ = oracle.policy_row(q_rows[0].astype(np.float32), 0.8, 3, 1.0)
    qd = np.where(kq, np.exp(zq - lq), 0.0)
    draft = rng.choice(V, size=(n, 1), p=qd / qd.sum()).astype(np.int32)
    o = oracle.verify(inp, draft, np.broadcast_to(zq.astype(np.float32), (n, 1, V)),
                      np.full((n, 1), lq, np.float32), np.full((n, 1), tq, np.float32),
                      qd[draft].astype(np.float32))
    kp, zp, lp, _, _ = oracle.policy_row(p_rows[0].astype(np.float32), 0.8, 3, 1.0)
    p0 = np.where(kp, np.exp(zp - lp), 0.0)
    assert chisq_pvalue(o["out_tokens"][:, 0], p0) > 1e-4


def test_bad_temperature_falls_back_to_greedy(oracle):
    tgt = onehot_rows([3, 4, 5], 16)[None]
    inp = decode_case(None, tgt, B=1, gamma=2, V=16, mode=1, temperature=0.0)
    o = oracle.verify(inp, np.array([[3, 9]], np.int32))
    assert o["accept_len"][0] == 1 and list(o["out_tokens"][0]) == [3, 4, -1]
    assert o["flags"][0, 0] & oracle.F_BAD_POLICY


def test_nonfinite_and_empty_rows_are_flagged(oracle):
    tgt = np.zeros((1, 3, 8), np.float32)
    tgt[0, 1, 2] = np.nan
    tgt[0, 2, :] = -np.inf
    inp = decode_case(None, tgt, B=1, gamma=2, V=8, mode=0)
    o = oracle.verify(inp, np.array([[5, 6]], np.int32))
    assert o["flags"][0, 1] & oracle.F_NONFINITE
    assert o["flags"][0, 2] & oracle.F_EMPTY


def test_zero_residual_falls_back_to_p(oracle):
    # q equal to p but q_tok claiming q(x) = 1: rejections happen, max(p - q, 0)
    # has no mass, and the emitted token is drawn from p with the flag set
    V, n = 6, 6000
    rows = np.random.default_rng(40).normal(0, 1, (2, V))
    tgt = np.broadcast_to(rows[None].astype(np.float32), (n, 2, V))
    inp = decode_case(None, np.ascontiguousarray(tgt), B=n, gamma=1, V=V, mode=1)
    qz, lse, thr = q_from_rows(oracle, rows[None, :1])
    draft = np.random.default_rng(41).choice(V, size=(n, 1), p=softmax64(rows[0])).astype(np.int32)
    o = oracle.verify(inp, draft, np.broadcast_to(qz, (n, 1, V)), np.broadcast_to(lse, (n, 1)),
                      np.broadcast_to(thr, (n, 1)), np.ones((n, 1), np.float32))
    rej = o["accept_len"] == 0
    assert rej.sum() > 1000
    assert np.all(o["flags"][rej, 0] & oracle.F_RESID_ZERO)
    assert chisq_pvalue(o["out_tokens"][rej, 0], softmax64(rows[0])) > 1e-4
