"""Pins of the oracle's gradient of the acceptance-statistics loss (CPU only).

Pages: "DSpark Speculative Decoding (Draft Training) Design", "Training
objective" (the draft is trained by 0.1 CE + 0.9 raw L1, position weights
exp(-k/gamma); the BCE term trains the confidence head against the
acceptance label; the target distribution is detached) and "Memory contract
for the full-vocabulary terms" (the row chunks are recomputed in the
backward).  Reading: the label is held fixed in the BCE; the subgradient of
|x| at 0 is 0.

Pins, none of which re-evaluates the oracle's gradient formula:
- central finite differences, in binary64, of the forward oracle's loss
  numerator (oracle_accept_stats) with respect to every draft logit
  (w_conf = 0, since the label is held fixed) and every confidence logit;
- torch autograd in float64 of the same loss written with torch's own
  log_softmax / cross_entropy / abs / BCE-with-logits, the label detached;
- invariants: each gradient row sums to 0 (the loss ignores a constant added
  to a draft row); disjoint supports (the pages' L1 = 2 fixed point) and
  identical rows leave no L1 gradient; masked blocks get none; the scale is
  linear.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from tests._cases import stats_case


def grid_case(seed, N=2, g=3, V=9, with_conf=True):
    """Logits on a 2^-8 grid (so +-2^-10 steps are exact in float32) whose
    target differs from the draft by at least 0.3 per token (no kink of |P-T|
    near the evaluation point)."""
    rng = np.random.default_rng(seed)
    d = np.round(rng.normal(0, 1.0, (N, g, V)) * 256) / 256
    off = rng.choice([-1, 1], (N, g, V)) * (0.3 + rng.uniform(0, 0.7, (N, g, V)))
    t = np.round((d + off) * 256) / 256
    teacher = rng.integers(0, V, (N, g))
    conf = np.round(rng.normal(0, 1.0, (N, g)) * 256) / 256 if with_conf else None
    return stats_case(d.astype(np.float32), t.astype(np.float32), teacher=teacher, conf_logits=conf)


def numerator(oracle, inp, **w):
    return oracle.accept_stats(inp, **w)["sums"][0]


@pytest.mark.parametrize("seed", [0, 1])
def test_finite_differences_draft(oracle, seed):
    inp = grid_case(seed)
    w = dict(w_ce=0.1, w_l1=0.9, w_conf=0.0)
    g = oracle.accept_stats_backward(inp, **w)["grad_draft"]
    h = 2.0 ** -10
    fd = np.zeros_like(g)
    base = inp["draft"].copy()
    for idx in np.ndindex(*base.shape):
        plus, minus = base.copy(), base.copy()
        plus[idx] += h
        minus[idx] -= h
        fp = numerator(oracle, dict(inp, draft=plus), **w)
        fm = numerator(oracle, dict(inp, draft=minus), **w)
        fd[idx] = (fp - fm) / (2 * h)
    # central differences: O(h^2) truncation on O(1) curvature
    assert np.allclose(g, fd, rtol=0, atol=2e-6)
    # the weights are exp(-k/gamma): a dropped weight would fail above, and so
    # would a per-row scale error; the BCE must not leak into the draft
    g2 = oracle.accept_stats_backward(inp, w_ce=0.1, w_l1=0.9, w_conf=5.0)["grad_draft"]
    assert np.array_equal(g, g2)


def test_finite_differences_conf(oracle):
    inp = grid_case(3)
    w = dict(w_ce=0.1, w_l1=0.9, w_conf=1.0)
    gc = oracle.accept_stats_backward(inp, **w)["grad_conf"]
    h = 2.0 ** -10
    base = inp["conf_logits"].copy()
    fd = np.zeros_like(gc)
    for idx in np.ndindex(*base.shape):
        plus, minus = base.copy(), base.copy()
        plus[idx] += h
        minus[idx] -= h
        fd[idx] = (numerator(oracle, dict(inp, conf_logits=plus), **w) -
                   numerator(oracle, dict(inp, conf_logits=minus), **w)) / (2 * h)
    assert np.allclose(gc, fd, rtol=0, atol=1e-7)


def torch_loss(d, t, teacher, c, mask, w_ce, w_l1, w_conf):
    N, g, V = d.shape
    lp = torch.log_softmax(d, -1)
    P = lp.exp()
    T = torch.softmax(t, -1)
    ce = torch.nn.functional.cross_entropy(d.reshape(-1, V), teacher.reshape(-1),
                                           reduction="none").reshape(N, g)
    l1 = (P - T).abs().sum(-1)
    a = (1 - 0.5 * l1).clamp(0, 1).detach()
    bce = torch.nn.functional.binary_cross_entropy_with_logits(c, a, reduction="none")
    wk = torch.exp(-torch.arange(1, g + 1, dtype=torch.float64) / g)
    per = wk * (w_ce * ce + w_l1 * l1 + w_conf * bce)
    return (mask[:, None] * per).sum()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_torch_autograd(oracle, dtype):
    rng = np.random.default_rng(11)
    N, g, V = 3, 4, 300
    d = rng.normal(0, 2.0, (N, g, V)).astype(np.float32)
    t = (d + rng.normal(0, 1.0, (N, g, V))).astype(np.float32)
    d[0, 1, :50] = -np.inf  # excluded tokens of the draft
    teacher = rng.integers(50, V, (N, g))
    conf = rng.normal(0, 1.5, (N, g)).astype(np.float32)
    mask = np.array([1, 0, 1], np.uint8)
    inp = stats_case(d, t, teacher=teacher, conf_logits=conf, block_mask=mask, dtype=dtype)
    w = dict(w_ce=0.1, w_l1=0.9, w_conf=1.0)
    o = oracle.accept_stats_backward(inp, scale=0.25, **w)
    from workloads import bf16_to_f32
    dv = bf16_to_f32(inp["draft"]) if dtype == "bf16" else inp["draft"]
    tv = bf16_to_f32(inp["target"]) if dtype == "bf16" else inp["target"]
    D = torch.tensor(dv, dtype=torch.float64, requires_grad=True)
    C = torch.tensor(conf, dtype=torch.float64, requires_grad=True)
    loss = 0.25 * torch_loss(D, torch.tensor(tv, dtype=torch.float64), torch.tensor(teacher),
                             C, torch.tensor(mask, dtype=torch.float64), **w)
    loss.backward()
    gd = D.grad.numpy()
    gd = np.where(np.isfinite(dv), gd, 0.0)  # autograd leaves 0 (or nan) at -inf inputs
    assert np.allclose(o["grad_draft"], gd, rtol=1e-9, atol=1e-13)
    assert np.allclose(o["grad_conf"], C.grad.numpy(), rtol=1e-9, atol=1e-13)


def test_rows_sum_to_zero(oracle):
    rng = np.random.default_rng(4)
    d = rng.normal(0, 3.0, (4, 5, 777)).astype(np.float32)
    t = (d + rng.normal(0, 1.0, d.shape)).astype(np.float32)
    inp = stats_case(d, t, teacher=rng.integers(0, 777, (4, 5)), dtype="bf16")
    g = oracle.accept_stats_backward(inp)["grad_draft"]
    assert np.abs(g.sum(-1)).max() < 1e-12


def test_disjoint_and_identical_rows(oracle):
    rng = np.random.default_rng(6)
    g_, V = 3, 40
    d = np.full((1, g_, V), -np.inf, np.float32)
    t = np.full((1, g_, V), -np.inf, np.float32)
    d[..., :20] = rng.normal(0, 1, (1, g_, 20))
    t[..., 20:] = rng.normal(0, 1, (1, g_, 20))
    o = oracle.accept_stats_backward(stats_case(d, t), w_ce=0.0, w_l1=1.0, w_conf=0.0)
    # L1 == 2 whatever the draft logits: no gradient
    assert np.abs(o["grad_draft"]).max() < 1e-15
    same = rng.normal(0, 2, (1, g_, V)).astype(np.float32)
    o = oracle.accept_stats_backward(stats_case(same, same), w_ce=0.0, w_l1=1.0, w_conf=0.0)
    assert np.all(o["grad_draft"] == 0.0)


def test_mask_and_scale(oracle):
    inp = grid_case(9, N=3, V=33)
    inp["block_mask"] = np.array([1, 0, 1], np.uint8)
    o1 = oracle.accept_stats_backward(inp, scale=1.0)
    o3 = oracle.accept_stats_backward(inp, scale=3.0)
    assert np.all(o1["grad_draft"][1] == 0) and np.all(o1["grad_conf"][1] == 0)
    assert np.allclose(o3["grad_draft"], 3.0 * o1["grad_draft"], rtol=1e-15, atol=0)
    assert np.allclose(o3["grad_conf"], 3.0 * o1["grad_conf"], rtol=1e-15, atol=0)
