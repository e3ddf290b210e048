"""GPU parity of the statistics of the teacher-forced Markov draft against
the CPU oracle (needs an MI355X).

Inputs come from the seeded generator (workloads.stats_markov_inputs) or
from hand-built arrays; nothing the GPU computes is fed back to the oracle.

Bar: per-position outputs and the sums within 1e-4 relative (atol 1e-6), as
for the plain statistics: the bias is an fp32-accumulated bf16 MFMA product
(rank r, relative error ~1e-6) added to the backbone, and the statistics run
in fp32.  At the full 2048 x 7 configuration the oracle checks sampled
blocks; tau and the sums are checked against the call's own per-position
outputs on every block.
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
from workloads import STATS_CONFIG, stats_markov_inputs  # noqa: E402

RTOL = 1e-4
KEYS = ["l1", "accept_rate", "ce", "bce"]


def run(inp):
    bm = inp.get("block_mask")
    out = ds.dspark_accept_stats_markov(
        G.logits(inp["backbone"], inp["dtype"]), G.logits(inp["target"], inp["dtype"]),
        G.i32(inp["anchor"]), G.bf(inp["w1"]), G.bf(inp["w2"]), G.i32(inp["teacher"]),
        G.f32(inp["conf_logits"]),
        None if bm is None else torch.from_numpy(np.ascontiguousarray(bm, np.uint8)).to(G.DEV))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def check(inp):
    got = run(inp)
    ref = O.accept_stats_markov(inp)
    for key in KEYS + ["tau"]:
        assert np.allclose(got[key], ref[key], rtol=RTOL, atol=1e-6), key
    assert np.allclose(got["sums"], ref["sums"], rtol=RTOL, atol=1e-6)


@pytest.mark.parametrize("dtype,r", [("f32", 16), ("bf16", 32), ("bf16", 256)])
def test_small(dtype, r):
    inp = stats_markov_inputs(dict(seed=41, N=3, gamma=5, V=1024, dtype=dtype, draft_std=2.0,
                                   noise_std=0.6), r=r, w_std=0.1, mask_every=3)
    check(inp)


@pytest.mark.parametrize("dtype,r,V", [("bf16", 256, 1000), ("f32", 256, 1024), ("f32", 256, 1000),
                                       ("bf16", 96, 1536)])
def test_aligned_shapes_several_tiles(dtype, r, V):
    # 147 rows: two full 64-row tiles and a ragged third; rank 256 takes the
    # compile-time rank path, V = 1000 the per-element token mask, rank 96 a
    # padded k range
    inp = stats_markov_inputs(dict(seed=V + r, N=21, gamma=7, V=V, dtype=dtype, draft_std=2.0,
                                   noise_std=0.8), r=r, w_std=0.05, mask_every=4)
    check(inp)


@pytest.mark.parametrize("V,gamma", [(999, 3), (1000, 1), (513, 4), (40, 7), (1024, ds.DSPARK_MAX_GAMMA)])
def test_ragged(V, gamma):
    inp = stats_markov_inputs(dict(seed=V, N=9, gamma=gamma, V=V, dtype="bf16", draft_std=2.0,
                                   noise_std=0.8), r=48, w_std=0.1)
    check(inp)


def test_zero_factors_match_plain_statistics():
    inp = stats_markov_inputs(dict(seed=5, N=20, gamma=7, V=4096, dtype="bf16", draft_std=3.0,
                                   noise_std=1.0), r=64)
    inp["w1"] = np.zeros_like(inp["w1"])
    got = run(inp)
    plain = G.stats(dict(inp, draft=inp["backbone"]))
    for key in KEYS + ["tau", "sums"]:
        assert np.allclose(got[key], plain[key], rtol=1e-5, atol=1e-6), key


def test_full_config_sampled():
    # the training configuration of the benchmark (2048 blocks x gamma 7, V =
    # 129280, rank 256), the oracle on sampled blocks
    inp = stats_markov_inputs(mask_every=5)
    got = run(inp)
    for blocks in ([0, 1], [1023, 2047]):
        sub = stats_markov_inputs(blocks=blocks, mask_every=5)
        sub["block_mask"] = inp["block_mask"][blocks]
        ref = O.accept_stats_markov(sub)
        for key in KEYS + ["tau"]:
            assert np.allclose(got[key][blocks], ref[key], rtol=RTOL, atol=1e-6), key
    # tau and the sums from the call's own per-position values (binary64)
    N, g = STATS_CONFIG["N"], STATS_CONFIG["gamma"]
    a = got["accept_rate"].astype(np.float64)
    tau = 1 + np.cumprod(a, axis=1).sum(1)
    assert np.allclose(got["tau"], tau, rtol=1e-5)
    m = inp["block_mask"].astype(bool)
    wk = np.exp(-np.arange(1, g + 1) / g)
    num = (wk * (0.1 * got["ce"] + 0.9 * got["l1"] + 1.0 * got["bce"]))[m].sum()
    assert got["sums"][0] == pytest.approx(num, rel=1e-5)
    assert got["sums"][1] == m.sum() * g
