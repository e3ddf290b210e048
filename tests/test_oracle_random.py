"""Pins of the oracle's random-number layer (CPU only).

* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
  as 1, 2, 3", SC'11): the oracle's words equal those of ROCm's rocRAND
  implementation of the same generator, run on the host, on counters that
  exercise every counter and key word.
* Uniform and Gumbel maps: a Kolmogorov-Smirnov test of the oracle's Gumbel
  noise against scipy's standard Gumbel law, and of the accept uniform
  against U[0,1).
* Two-level Gumbel-max (chunk by chunk log-mass, then token inside the chunk):
  chi-square of its draws against softmax of the log-weights, with a ragged
  last chunk and excluded (-inf) tokens.
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
def test_two_level_gumbel_max_is_softmax(oracle, V):
    rng = np.random.default_rng(V)
    lw = rng.normal(0.0, 1.5, V)
    if V > 10:
        lw[rng.choice(V, V // 5, replace=False)] = -np.inf  # excluded tokens
        lw[:3] += 4.0                                         # a few heavy tokens
    p = softmax64(lw)
    n = 30000
    draws = [oracle.sample_two_level(lw, 9, req, 40)[0] for req in range(n)]
    assert chisq_pvalue(draws, p) > 1e-4


def test_two_level_empty_and_single(oracle):
    lw = np.full(300, -np.inf)
    assert oracle.sample_two_level(lw, 0, 0, 0)[0] == -1
    lw[277] = 0.0
    assert all(oracle.sample_two_level(lw, 0, r, 0)[0] == 277 for r in range(20))
