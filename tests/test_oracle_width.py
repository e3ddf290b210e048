"""Pins of the oracle's confidence-scheduled draft width (CPU only).

Pages: "[2/3] feat(dsv4): implement exact DSpark speculative decoding"
(scope notes and the author's reply: a hardware-measured choice over 0..5
proposals, declining or shortening speculation when the measured D + V(k)
cost does not pay) and "DSpark Speculative Decoding (Draft Training) Design",
"Overview" (the confidence head predicts per-position acceptance so that the
server can schedule its verify budget).  The reading: verifying the first w
proposals emits E(w) = 1 + sum_{k<=w} prod_{j<=k} c_j tokens in expectation,
and the width maximising E(w) / (D + V(w)) is chosen (ties: the smaller w).

Pins, none of which re-evaluates the oracle's own loop:
- the geometric closed form (1 - p^(w+1)) / (1 - p) of E(w) for a constant
  confidence p, and the resulting choice over a linear cost table;
- a Monte Carlo simulation of the acceptance chain the reading describes
  (accept proposal j with probability c_j until the first rejection, plus the
  target's own token) reproduces E(w) within its sampling error;
- E(gamma) equals the tau the acceptance statistics report when the
  confidences are the statistics' own accept rates;
- degenerate tables: c = 0 (every width emits one token: the cheapest width
  wins), c = 1 with a flat cost (the widest wins), exact ties (the smaller
  width), ineligible costs (zero, negative, NaN, inf: skipped; none eligible:
  width 0), NaN / out-of-range confidences (clamped to [0, 1]).
"""

from __future__ import annotations

import numpy as np
import pytest

from tests._cases import stats_case
from workloads import width_inputs


def _ratio_choice(E, cost):
    """Argmax of E[w] / (D + V(w)) with the smaller w on ties, from a given E."""
    den = float(cost[0]) + cost[1:].astype(np.float64)
    r = np.where((den > 0) & np.isfinite(den), E / np.where(den > 0, den, 1.0), -np.inf)
    return int(np.flatnonzero(r == r.max())[0])


@pytest.mark.parametrize("p", [0.0, 0.25, 0.6, 0.9, 0.97])
def test_geometric_closed_form(oracle, p):
    g = 7
    conf = np.full((1, g), p, np.float32)
    pf = float(np.float32(p))
    w = np.arange(g + 1)
    E = (1 - pf ** (w + 1)) / (1 - pf) if pf != 1.0 else w + 1.0
    for D, v0, v1 in [(1.0, 3.0, 0.45), (0.5, 2.0, 0.05), (4.0, 1.0, 2.0)]:
        cost = np.array([D] + [v0 + v1 * (k + 1) for k in range(g + 1)], np.float32)
        n, e = oracle.select_width(conf, cost)
        assert n[0] == _ratio_choice(E, cost)
        assert e[0] == pytest.approx(E[n[0]], rel=1e-12)


def test_expected_tokens_by_simulation(oracle):
    rng = np.random.default_rng(7)
    g = 5
    conf = rng.uniform(0.2, 0.95, (1, g)).astype(np.float32)
    c = conf[0].astype(np.float64)
    trials = 200_000
    u = rng.random((trials, g))
    acc = np.cumprod(u < c, axis=1)  # 1 while every earlier proposal was accepted
    for w in range(g + 1):
        # flat cost: the oracle then picks gamma; E(w) is read back by
        # restricting the table so that only widths 0..w are eligible
        cost = np.array([1.0] + [1.0 if k <= w else np.nan for k in range(g + 1)], np.float32)
        n, e = oracle.select_width(conf, cost)
        assert n[0] == w
        tokens = 1.0 + acc[:, :w].sum(axis=1)
        se = tokens.std() / np.sqrt(trials)
        assert abs(e[0] - tokens.mean()) < 5 * se + 1e-12


def test_matches_stats_tau(oracle):
    # confidences set to the accept rates that the statistics compute from a
    # pair of blocks: E(gamma) must be their tau
    rng = np.random.default_rng(3)
    g, V = 5, 96
    d = rng.normal(0, 1.5, (2, g, V)).astype(np.float32)
    t = (d + rng.normal(0, 0.7, (2, g, V))).astype(np.float32)
    st = oracle.accept_stats(stats_case(d, t))
    a = st["accept_rate"].astype(np.float32)
    cost = np.array([1.0] + [1.0] * (g + 1), np.float32)  # flat: the widest wins
    n, e = oracle.select_width(a, cost)
    assert np.all(n == g)
    # the statistics run on the binary64 rates, the width on their float32 copy
    assert np.allclose(e, st["tau"], rtol=1e-6, atol=0)


def test_degenerate_tables(oracle):
    g = 5
    inc = np.array([1.0] + [2.0 + k for k in range(g + 1)], np.float32)
    # nothing is accepted: one token whatever the width, so the cheapest wins
    n, e = oracle.select_width(np.zeros((3, g), np.float32), inc)
    assert np.all(n == 0) and np.all(e == 1.0)
    dec = inc[::-1].copy()
    dec[0] = 1.0
    dec[1:] = np.arange(g + 1, 0, -1)
    n, _ = oracle.select_width(np.zeros((1, g), np.float32), dec)
    assert n[0] == g
    # everything is accepted and verification costs the same at every width
    flat = np.full(g + 2, 2.0, np.float32)
    n, e = oracle.select_width(np.ones((2, g), np.float32), flat)
    assert np.all(n == g) and np.all(e == g + 1)


def test_exact_tie_goes_to_smaller_width(oracle):
    g = 3
    # c = 1: E(w) = 1 + w; D + V(w) = 1 + w for w = 1, 2 gives the ratio 1
    # at both (exactly representable), lower elsewhere
    cost = np.array([0.5, 2.0, 1.5, 2.5, 8.0], np.float32)
    n, e = oracle.select_width(np.ones((1, g), np.float32), cost)
    assert n[0] == 1 and e[0] == 2.0


def test_ineligible_costs_and_bad_confidences(oracle):
    g = 4
    conf = np.array([[0.9, 0.9, 0.9, 0.9]], np.float32)
    cost = np.array([1.0, 3.0, 3.2, 3.4, 3.6, 3.8], np.float32)
    base, _ = oracle.select_width(conf, cost)
    assert base[0] == g
    for bad in [0.0, -1.0, np.nan, np.inf]:
        c2 = cost.copy()
        c2[1 + g] = bad if bad != 0.0 else -1.0  # D + V(g) = 0 for -1.0
        n, _ = oracle.select_width(conf, c2)
        assert n[0] == g - 1
    none = np.array([1.0, -1.0, np.nan, -5.0, np.inf, -2.0], np.float32)
    n, e = oracle.select_width(conf, none)
    assert n[0] == 0 and e[0] == 1.0
    # NaN and negative confidences count as 0, values above 1 as 1
    odd = np.array([[np.nan, 0.9, 0.9, 0.9], [-0.5, 0.9, 0.9, 0.9], [1.5, 1.0, 1.0, 1.0]],
                   np.float32)
    flat = np.full(g + 2, 1.0, np.float32)
    n, e = oracle.select_width(odd, flat)
    assert np.all(e[:2] == 1.0) and n[2] == g and e[2] == g + 1


def test_seeded_inputs_spread(oracle):
    inp = width_inputs()
    n, e = oracle.select_width(inp["confidence"], inp["cost"])
    assert len(np.unique(n)) >= 3  # the synthetic batch exercises several widths
    assert np.all(e >= 1.0) and np.all(e <= inp["gamma"] + 1)
