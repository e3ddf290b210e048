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
from workloads import STATS_CONFIG, bf16_to_f32, stats_markov_inputs, to_bf16  # noqa: E402

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


def test_near_rows_full_vocab():
    """L1 relative to itself (1e-4) at V=129280 for row pairs from equal to
    disjoint (the rows of the plain statistics' test), the Markov bias zero
    (W1 = 0) so that the draft rows are the backbone's bf16 values; and with
    a small bias (W1, W2 ~ N(0, 0.02^2), rank 16) against the oracle's own
    Markov rows, where each draft logit backbone + bias is itself rounded to
    fp32 once (|delta| <= 2^-24 |d|), which may move L1 by up to
    2^-23 sum_v P_v |d_v| on top of the 1e-4 relative bar."""
    from tests.test_gpu_parity import _near_rows
    si = _near_rows(2, 7, 129280, 77)
    rng = np.random.default_rng(3)
    V, r = si["V"], 16
    w = lambda: np.asarray(to_bf16(rng.normal(0, 0.02, (V, r)).astype(np.float32)))
    for w1 in (np.zeros((V, r), np.uint16), w()):
        inp = dict(backbone=si["draft"], target=si["target"], anchor=np.arange(si["N"], dtype=np.int32),
                   w1=w1, w2=w(), r=r, teacher=si["teacher"], conf_logits=si["conf_logits"],
                   block_mask=None, N=si["N"], gamma=si["gamma"], V=V, dtype="bf16")
        got = run(inp)
        ref = O.accept_stats_markov(inp)
        l1r, l1g = ref["l1"], got["l1"].astype(np.float64)
        bound = RTOL * l1r + 1e-9
        if w1.any():
            bb = bf16_to_f32(si["draft"]).astype(np.float64)
            fin = np.isfinite(bb)
            e = np.where(fin, np.exp(bb - np.max(np.where(fin, bb, -np.inf), -1, keepdims=True)), 0.0)
            P = e / e.sum(-1, keepdims=True)
            bound = bound + 2.0 ** -23 * (P * np.where(fin, np.abs(bb), 0.0)).sum(-1)
        bad = np.abs(l1g - l1r) > bound
        assert not bad.any(), (bool(w1.any()), np.argwhere(bad), l1g[bad], l1r[bad])
        for key in ["accept_rate", "bce", "tau"]:
            assert np.allclose(got[key], ref[key], rtol=RTOL, atol=1e-6), key


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
