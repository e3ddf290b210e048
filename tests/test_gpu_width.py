"""GPU parity of the confidence-scheduled draft width against the CPU oracle
(needs an MI355X).

Inputs come from the seeded generator (workloads.width_inputs), from
hand-written edge tables, or from the oracle (the decode chain's confidences,
proposals and q); nothing the GPU computes is fed back to the oracle.

Bars: n_draft bit-exact (both sides take the decision in binary64 with the
same operation order and rounding); expected bit-exact (both round the same
binary64 E to float32).  Through dspark_verify, the usual verify bar.
"""

from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import dspark_draft_sampling_amd as ds  # noqa: E402
from oracle import oracle as O  # noqa: E402
from tests import _gpu as G  # noqa: E402
from workloads import decode_inputs, width_inputs  # noqa: E402


def run(conf, cost):
    out = ds.dspark_select_width(G.f32(conf), G.f32(cost))
    torch.cuda.synchronize()
    return out["n_draft"].cpu().numpy(), out["expected"].cpu().numpy()


def check(conf, cost):
    n, e = run(conf, cost)
    rn, re = O.select_width(conf, cost)
    assert np.array_equal(n, rn)
    assert np.array_equal(e, re.astype(np.float32))
    return n


def test_seeded_batch():
    inp = width_inputs()
    n = check(inp["confidence"], inp["cost"])
    assert len(np.unique(n)) >= 3


@pytest.mark.parametrize("B,gamma", [(1, 1), (255, 5), (257, 7), (4099, 16), (100003, 5)])
def test_shapes_and_ragged_grids(B, gamma):
    inp = width_inputs(B=B, gamma=gamma)
    check(inp["confidence"], inp["cost"])


def test_random_tables_near_ties():
    # many requests whose ratios differ by a few ulps: cost steps of one ulp
    # around a common value, confidences on a coarse grid
    rng = np.random.default_rng(5)
    g = 6
    conf = (rng.integers(0, 9, (20000, g)) / 8).astype(np.float32)
    for t in range(8):
        base = np.float32(rng.uniform(1, 4))
        cost = np.nextafter(np.full(g + 2, base, np.float32), np.float32(np.inf)) * \
            (1 + np.arange(g + 2, dtype=np.float32) * np.float32(rng.uniform(0, 0.3)))
        cost[0] = np.float32(rng.uniform(0, 2))
        check(conf, cost.astype(np.float32))


def test_edge_values():
    g = 5
    conf = np.array([[np.nan, 0.9, 0.9, 0.9, 0.9],
                     [-0.5, 0.9, 0.9, 0.9, 0.9],
                     [1.5, 1.0, 1.0, 1.0, 1.0],
                     [0.0, 0.0, 0.0, 0.0, 0.0],
                     [1e-40, 0.5, 0.5, 0.5, 0.5],  # subnormal float32
                     [0.999999, 0.999999, 0.999999, 0.999999, 0.999999],
                     [np.inf, -np.inf, 0.5, np.nan, 1.0]], np.float32)
    tables = [
        np.array([1.0, 3.0, 3.2, 3.4, 3.6, 3.8, 4.0], np.float32),
        np.array([1.0, 3.0, 3.2, np.nan, 3.6, -9.0, np.inf], np.float32),
        np.array([1.0, -1.0, np.nan, -5.0, np.inf, -2.0, -1.0], np.float32),  # none eligible
        np.array([0.0, 0.0, 1.0, 2.0, 3.0, 4.0, 5.0], np.float32),  # w = 0 costs nothing
        np.array([np.nan, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0], np.float32),  # D itself NaN
        np.full(7, 2.0, np.float32),
        np.array([0.5, 2.0, 1.5, 2.5, 3.5, 8.0, 9.0], np.float32),  # exact tie at w = 1, 2
    ]
    for cost in tables:
        check(conf, cost)


def test_empty_batch():
    out = ds.dspark_select_width(torch.empty((0, 5), dtype=torch.float32, device=G.DEV),
                                 G.f32(np.ones(7, np.float32)))
    torch.cuda.synchronize()
    assert out["n_draft"].numel() == 0


def test_width_feeds_verify():
    # oracle chain: Markov -> width -> verify(n_draft); the GPU takes the same
    # oracle confidences, proposals and q, and its own n_draft
    inp = decode_inputs("tiny", B=48)
    mk = O.markov_sample(inp)
    conf = mk["confidence"].astype(np.float32)
    cost = np.array([1.0, 3.0, 3.3, 3.6, 3.9, 4.2, 4.5], np.float32)
    rn, _ = O.select_width(conf, cost)
    gn, _ = run(conf, cost)
    assert np.array_equal(gn, rn)
    q = G.q_of(mk)
    ref = O.verify(inp, mk["draft_tokens"], n_draft=rn, **q)
    got = G.verify(inp, mk["draft_tokens"], q, n_draft=gn)
    flagged = (ref["flags"] & O.F_NEAR).any(1)
    ok = ~flagged
    assert np.array_equal(got["accept_len"][ok], ref["accept_len"][ok])
    assert np.array_equal(got["out_tokens"][ok], ref["out_tokens"][ok])
    assert np.all(got["accept_len"] <= gn)
