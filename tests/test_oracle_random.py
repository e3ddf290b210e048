"""Pins of the oracle's random-number layer (CPU only).

* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
  as 1, 2, 3", SC'11): the oracle's words equal those of ROCm's rocRAND
  implementation of the same generator, run on the host, on counters that
  exercise every counter and key word.
* Uniform and Gumbel maps: a Kolmogorov-Smirnov test of the oracle's Gumbel
  noise against scipy's standard Gumbel law, and of the accept uniform
  against U[0,1).
* Three-level Gumbel-max (chunk of 256 tokens by its log-mass, then a 16-token
  sub-chunk inside it by its log-mass, then the token inside that): chi-square
  of its draws against softmax of the log-weights, at small vocabularies and
  at one spanning 101 chunks with a ragged tail, including top-k / top-p kept
  sets (from the oracle's own policy, itself pinned by brute force) whose
  members straddle chunk and sub-chunk boundaries; chunk-level frequencies
  against the chunk masses; and the special cases where a level has a single
  candidate, so that the draw reduces to a textbook per-token Gumbel-max
  (argmax of log-weight plus standard Gumbel noise) written out here with
  numpy from the pinned noise stream.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from tests._cases import chisq_pvalue, softmax64

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference")
    exe = str(tmp_path_factory.mktemp("rocrand") / "ref")
    subprocess.run([hipcc, "-O1", os.path.join(HERE, "rocrand_philox_ref.cpp"), "-o", exe],
                   check=True, capture_output=True, cwd=str(tmp_path_factory.getbasetemp()))
    return exe


def test_philox_matches_rocrand(oracle, rocrand_ref):
    rng = np.random.default_rng(7)
    cases = [(0, (0, 0, 0, 0)), (0, (1, 0, 0, 0)), (0, (0, 1, 0, 0)), (0, (0, 0, 1, 0)),
             (0, (0, 0, 0, 1)), (0xFFFFFFFFFFFFFFFF, (0xFFFFFFFF,) * 4),
             (0x0123456789ABCDEF, (5, 0x80000000, 17, 2))]
    for _ in range(200):
        seed = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        cases.append((seed, tuple(int(x) for x in rng.integers(0, 2**32, 4))))
    text = "".join("%x %x %x %x %x\n" % (s, *c) for s, c in cases)
    res = subprocess.run([rocrand_ref], input=text, capture_output=True, text=True, check=True)
    lines = res.stdout.strip().splitlines()
    assert len(lines) == len(cases)
    for (seed, ctr), line in zip(cases, lines):
        want = [int(w, 16) for w in line.split()]
        got = oracle.philox4x32_10(np.array(ctr, np.uint32),
                                   np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32))
        assert list(got) == want, (hex(seed), ctr)


def test_philox_word_layout(oracle):
    """Word i of the stream keyed (seed, position, request, tag) is output word
    i % 4 of counter (i // 4, position, request, tag)."""
    seed = 0xDEADBEEF12345678
    for i, pos, req, tag in [(0, 100, 3, 0), (5, 7, 0, 2), (1023, -1, 9, 4), (77, 2**31 - 1, 2**32 - 1, 1)]:
        block = oracle.philox4x32_10(np.array([i >> 2, pos & 0xFFFFFFFF, req, tag], np.uint32),
                                     np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32))
        assert oracle.philox_word(seed, i, pos, req, tag) == int(block[i & 3])


def test_gumbel_law(oracle):
    g = np.array([oracle.gumbel(3, i, 11, 5, 0) for i in range(40000)])
    assert np.all(np.isfinite(g))
    assert stats.kstest(g, stats.gumbel_r.cdf).pvalue > 1e-3
    # tags and positions give different streams
    g2 = np.array([oracle.gumbel(3, i, 11, 5, 2) for i in range(2000)])
    assert not np.allclose(g[:2000], g2)


def test_accept_uniform_law(oracle):
    u = np.array([oracle.accept_uniform(1, p, r) for p in range(200) for r in range(100)])
    assert u.min() >= 0.0 and u.max() < 1.0
    assert stats.kstest(u, stats.uniform.cdf).pvalue > 1e-3


@pytest.mark.parametrize("V", [600, 256, 5])
def test_three_level_gumbel_max_is_softmax(oracle, V):
    rng = np.random.default_rng(V)
    lw = rng.normal(0.0, 1.5, V)
    if V > 10:
        lw[rng.choice(V, V // 5, replace=False)] = -np.inf  # excluded tokens
        lw[:3] += 4.0                                         # a few heavy tokens
    p = softmax64(lw)
    n = 30000
    draws = [oracle.sample_three_level(lw, 9, req, 40)[0] for req in range(n)]
    assert chisq_pvalue(draws, p) > 1e-4


def _binned(draws, bins, nbins):
    """Map each draw through `bins` (token -> bin) and count."""
    return np.bincount(bins[np.asarray(draws)], minlength=nbins)


def _wide_row(rng, V):
    """Log-weights over V tokens: a low background, plus about 180 heavy tokens
    placed on both sides of chunk (256) and sub-chunk (16) boundaries."""
    lw = rng.normal(-3.0, 0.5, V)
    heavy = []
    for c in rng.choice(V // 256, 60, replace=False):
        heavy += [c * 256 - 1, c * 256] if c > 0 else [0, 1]
    for j in rng.choice(np.arange(1, V // 16), 30, replace=False):
        heavy += [j * 16 - 1, j * 16]
    heavy = np.array(sorted(set(heavy)))
    lw[heavy] = rng.normal(3.0, 0.7, heavy.size)
    lw[rng.choice(V, V // 10, replace=False)] = -np.inf  # excluded tokens
    return lw, heavy


def test_three_level_wide_vocabulary(oracle):
    """V = 25800: 101 chunks, the last one ragged (200 tokens)."""
    V = 25800
    rng = np.random.default_rng(11)
    lw, heavy = _wide_row(rng, V)
    p = softmax64(lw)
    kept = heavy[np.isfinite(lw[heavy])]
    bins = np.full(V, kept.size, np.int64)
    bins[kept] = np.arange(kept.size)
    probs = np.append(p[kept], 1.0 - p[kept].sum())
    n = 12000
    draws = [oracle.sample_three_level(lw, 5, req, 77)[0] for req in range(n)]
    counts = _binned(draws, bins, kept.size + 1)
    assert stats.chisquare(counts, probs * n).pvalue > 1e-4
    # chunk level: the chosen chunk follows the chunk masses
    chunk_p = np.bincount(np.arange(V) // 256, weights=p)
    cc = np.bincount(np.asarray(draws) // 256, minlength=chunk_p.size)
    assert np.all(chunk_p * n >= 5)
    assert stats.chisquare(cc, chunk_p * n).pvalue > 1e-4


@pytest.mark.parametrize("top_k,top_p", [(40, 1.0), (0, 0.6), (90, 0.8)])
def test_three_level_truncated_across_boundaries(oracle, top_k, top_p):
    """Kept sets from the policy (top-k, top-p, both) whose tokens sit on both
    sides of chunk and sub-chunk boundaries of a 101-chunk vocabulary."""
    V = 25800
    rng = np.random.default_rng(100 + top_k)
    lw, _ = _wide_row(rng, V)
    lw[~np.isfinite(lw)] = -30.0  # the policy row is finite; truncation excludes
    kept, z, lse, thr, near = oracle.policy_row(lw, 1.0, top_k, top_p)
    assert not near
    kept = np.flatnonzero(kept)
    assert 20 < kept.size < 200
    assert len(set(kept // 256)) > 15  # the kept set spans many chunks
    assert np.any(np.diff(kept // 256) != 0) and np.any(kept % 256 == 0)
    row = np.full(V, -np.inf)
    row[kept] = z[kept]
    p = softmax64(row)
    n = 12000
    draws = np.array([oracle.sample_three_level(row, 3, req, 900 + top_k)[0] for req in range(n)])
    assert np.all(np.isin(draws, kept))
    counts = np.array([(draws == v).sum() for v in kept])
    assert stats.chisquare(counts, p[kept] * n).pvalue > 1e-4


def test_three_level_reduces_to_token_gumbel_max(oracle):
    """V <= 16: one chunk and one sub-chunk, so the draw is the per-token
    Gumbel-max argmax_v (lw_v + g(v, token tag)) with ties to the lowest index."""
    rng = np.random.default_rng(3)
    for req in range(300):
        V = int(rng.integers(1, 17))
        lw = rng.normal(0.0, 2.0, V)
        lw[rng.random(V) < 0.2] = -np.inf
        g = np.array([oracle.gumbel(21, v, 55, req, oracle.TAG_TARGET_TOKEN) for v in range(V)])
        score = np.where(np.isfinite(lw), lw + g, -np.inf)
        want = int(np.argmax(score)) if np.isfinite(score).any() else -1
        got = oracle.sample_three_level(lw, 21, req, 55, oracle.TAG_TARGET_CHUNK,
                                        oracle.TAG_TARGET_SUB, oracle.TAG_TARGET_TOKEN)[0]
        assert got == want


def test_three_level_levels_with_one_candidate(oracle):
    """With exactly one token per chunk the draw is a Gumbel-max over chunks
    (chunk noise); with one token per sub-chunk inside a single chunk it is a
    Gumbel-max over sub-chunks (sub-chunk noise, global sub-chunk index)."""
    rng = np.random.default_rng(4)
    V = 256 * 9 + 40
    for req in range(100):
        # one token per chunk, at a random offset inside its chunk
        lw = np.full(V, -np.inf)
        toks = np.array([c * 256 + int(rng.integers(0, min(256, V - c * 256))) for c in range(10)])
        lw[toks] = rng.normal(0.0, 1.0, toks.size)
        g = np.array([oracle.gumbel(8, c, 9, req, oracle.TAG_DRAFT_CHUNK) for c in range(10)])
        want = toks[int(np.argmax(lw[toks] + g))]
        assert oracle.sample_three_level(lw, 8, req, 9)[0] == want
        # one token per sub-chunk, all in chunk 3
        lw = np.full(V, -np.inf)
        subs = np.arange(3 * 16, 4 * 16)
        toks = subs * 16 + rng.integers(0, 16, subs.size)
        lw[toks] = rng.normal(0.0, 1.0, toks.size)
        g = np.array([oracle.gumbel(8, int(j), 9, req, oracle.TAG_DRAFT_SUB) for j in subs])
        want = toks[int(np.argmax(lw[toks] + g))]
        assert oracle.sample_three_level(lw, 8, req, 9)[0] == want


def test_three_level_empty_and_single(oracle):
    lw = np.full(300, -np.inf)
    assert oracle.sample_three_level(lw, 0, 0, 0)[0] == -1
    lw[277] = 0.0
    assert all(oracle.sample_three_level(lw, 0, r, 0)[0] == 277 for r in range(20))
