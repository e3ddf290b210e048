"""Pins of the oracle's sampling policy (temperature, top-k, top-p) on the CPU.

The pages ("[2/3] feat(dsv4): implement exact DSpark speculative decoding",
section "Exact decoding semantics", "Probabilistic") apply the request's
temperature, top-k and top-p to both p and q before the accept test; the order
and tie handling are the reading stated in the oracle (temperature, then top-k
keeping ties with the k-th value, then top-p on the renormalised top-k set).

Pinned by brute force on tiny vocabularies with a formulation different from
the oracle's sort-and-walk:
* top-k keeps v iff fewer than k values are strictly larger;
* top-p is found by enumerating every subset: the smallest subset size m whose
  best subset reaches mass top_p, and the cut value is the largest possible
  minimum probability of such a subset; every token at or above it is kept;
* the log-normaliser is scipy's logsumexp over the kept set.
Special cases reduce to the identity (top_k >= V, top_p >= 1) or to the argmax
set (top_k = 1, top_p -> 0).
"""

from __future__ import annotations

import itertools

import numpy as np
import pytest
from scipy.special import logsumexp


def brute_kept(l, T, top_k, top_p):
    V = len(l)
    z = np.asarray(l, np.float64) / T
    keep = np.isfinite(z)
    if 0 < top_k < V:
        keep &= np.array([(z > z[v]).sum() < top_k for v in range(V)])
    if top_p < 1.0:
        idx = [v for v in range(V) if keep[v]]
        pi = np.exp(z[idx] - logsumexp(z[idx]))
        best = None
        for m in range(1, len(idx) + 1):
            cands = [min(pi[list(S)]) for S in itertools.combinations(range(len(idx)), m)
                     if pi[list(S)].sum() >= top_p]
            if cands:
                best = max(cands)
                break
        if best is None:  # mass never reaches top_p by rounding: keep everything
            best = pi.min()
        # tokens whose probability is at least the cut value; compare on z so
        # that equal logits are never split by rounding
        cut_z = min(z[idx[i]] for i in range(len(idx)) if pi[i] >= best)
        keep &= z >= cut_z
    return keep


def check(oracle, l, T, k, p):
    kept, z, lse, thr, _ = oracle.policy_row(l, T, k, p)
    want = brute_kept(l, T, k, p)
    assert np.array_equal(kept.astype(bool), want), (l, T, k, p)
    zz = np.asarray(l, np.float64) / T
    assert lse == pytest.approx(logsumexp(zz[want]), rel=1e-14, abs=1e-14)
    if (0 < k < len(l)) or p < 1.0:
        assert thr == zz[want].min()
    else:
        assert thr == -np.inf


def test_policy_brute_force_random(oracle):
    rng = np.random.default_rng(0)
    for trial in range(400):
        V = int(rng.integers(1, 9))
        l = rng.normal(0, 2, V)
        if trial % 3 == 0:  # ties
            l = np.round(l)
        T = float(rng.choice([0.3, 1.0, 1.7]))
        k = int(rng.choice([0, 1, 2, 3, V, V + 3]))
        p = float(rng.choice([1.0, 0.95, 0.8, 0.5, 0.2, 1e-9]))
        check(oracle, l, T, k, p)


def test_policy_identity_and_argmax_cases(oracle):
    l = np.array([0.5, 3.0, -1.0, 3.0, 2.0])
    kept, _, _, thr, _ = oracle.policy_row(l, 1.0, 0, 1.0)
    assert kept.all() and thr == -np.inf
    kept, *_ = oracle.policy_row(l, 1.0, 5, 1.0)
    assert kept.all()
    kept, *_ = oracle.policy_row(l, 1.0, 1, 1.0)         # argmax set, ties kept
    assert list(np.nonzero(kept)[0]) == [1, 3]
    kept, *_ = oracle.policy_row(l, 0.7, 0, 1e-12)       # top-p -> 0: argmax set
    assert list(np.nonzero(kept)[0]) == [1, 3]
    kept, *_ = oracle.policy_row(l, 1.0, 0, 0.0)
    assert list(np.nonzero(kept)[0]) == [1, 3]


def test_policy_excludes_masked_tokens(oracle):
    l = np.array([-np.inf, 1.0, -np.inf, 0.0])
    kept, z, lse, _, _ = oracle.policy_row(l, 2.0, 0, 1.0)
    assert list(kept) == [0, 1, 0, 1]
    assert lse == pytest.approx(np.log(np.exp(0.5) + 1.0), rel=1e-15)


def test_policy_top_p_boundary_near_flag(oracle):
    # masses 0.5 / 0.3 / 0.2: with top_p = 0.5 the mass above the second token
    # sits on the cut
    kept, _, _, _, near = oracle.policy_row(np.log([0.5, 0.3, 0.2]), 1.0, 0, 0.5)
    assert near
    kept, _, _, _, near = oracle.policy_row(np.array([2.0, 0.0, -1.0]), 1.0, 0, 0.5)
    assert not near and list(kept) == [1, 0, 0]


def test_policy_top_k_near_flag_only_for_computed_rows(oracle):
    l = np.array([1.0, 1.0 - 1e-9, -3.0])
    assert oracle.policy_row(l, 1.0, 1, 1.0, exact_order=False)[4]
    assert not oracle.policy_row(l, 1.0, 1, 1.0, exact_order=True)[4]
