"""GPU parity of the acceptance-statistics gradient against the CPU oracle
(needs an MI355X).

Inputs come from the seeded generator (workloads.stats_inputs) or from
hand-built rows; nothing the GPU computes is fed back to the oracle.

Bar, per element, from the arithmetic: the kernels form P_v and T_v in fp32
(relative error ~1e-6) and S = sum sign(P-T) P in fp32, so an element may
differ from the binary64 oracle by 1e-5 of the size of its terms,
alpha (w_ce + w_l1) P_v (plus alpha w_ce at the teacher), plus one bf16 ulp
for bf16 outputs.  Where the oracle's P_v and T_v agree to 1e-5 the fp32
sign of P_v - T_v may differ, and the element may differ by 2 alpha w_l1 P_v.
The confidence-logit gradient within 1e-4 relative.  Every gradient row must
also sum to 0 (the loss ignores a constant added to a draft row) within the
same bound summed over the row.
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
from tests._cases import stats_case  # noqa: E402
from workloads import bf16_to_f32, stats_inputs  # noqa: E402

W = dict(w_ce=0.1, w_l1=0.9, w_conf=1.0)


def softmax_rows(x):
    """Row softmax in binary64; an empty row (all -inf) gives zeros."""
    x = np.asarray(x, np.float64)
    fin = np.isfinite(x)
    m = np.max(np.where(fin, x, -np.inf), axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(fin, np.exp(np.where(fin, x, 0.0) - m), 0.0)
    s = e.sum(-1, keepdims=True)
    return e / np.where(s > 0, s, 1.0)


def run(inp, scale=None, **w):
    sc = None if scale is None else torch.tensor([scale], dtype=torch.float32, device=G.DEV)
    out = ds.dspark_accept_stats_backward(
        G.logits(inp["draft"], inp["dtype"]), G.logits(inp["target"], inp["dtype"]),
        G.i32(inp["teacher"]), G.f32(inp["conf_logits"]),
        None if inp.get("block_mask") is None else
        torch.from_numpy(np.ascontiguousarray(inp["block_mask"], np.uint8)).to(G.DEV),
        grad_scale=sc, **w)
    torch.cuda.synchronize()
    g = out["grad_draft"]
    g = g.float().cpu().numpy() if g.dtype == torch.bfloat16 else g.cpu().numpy()
    return g, out["grad_conf"].cpu().numpy()


def tolerance(inp, ref_grad, scale, w, near_rel=1e-5):
    """Per-element bound of the module docstring (near_rel: the relative
    gap |P - T| / max(P, T) below which the sign of P - T may differ)."""
    N, g, V = inp["N"], inp["gamma"], inp["V"]
    to32 = bf16_to_f32 if inp["dtype"] == "bf16" else (lambda x: x)
    P = softmax_rows(to32(inp["draft"]))
    T = softmax_rows(to32(inp["target"]))
    m = np.ones(N) if inp.get("block_mask") is None else (np.asarray(inp["block_mask"]) != 0) * 1.0
    alpha = scale * m[:, None] * np.exp(-np.arange(1, g + 1) / g)[None, :]
    onehot = np.zeros((N, g, V))
    np.put_along_axis(onehot, np.clip(inp["teacher"], 0, V - 1)[..., None].astype(np.int64), 1.0, -1)
    size = alpha[..., None] * ((w["w_ce"] + w["w_l1"]) * P + w["w_ce"] * onehot)
    tol = 1e-5 * size + 1e-12
    if inp["dtype"] == "bf16":
        tol = tol + 2.0 ** -8 * np.abs(ref_grad)
    near = np.abs(P - T) <= near_rel * np.maximum(P, T)
    return np.where(near, tol + 2 * alpha[..., None] * w["w_l1"] * P, tol)


def check(inp, scale=1.0, w=W, near_rel=1e-5, got=None):
    """Compare every element of the gradient with the oracle."""
    got, gotc = run(inp, scale=scale, **w) if got is None else got
    ref = O.accept_stats_backward(inp, scale=scale, **w)
    tol = tolerance(inp, ref["grad_draft"], scale, w, near_rel)
    err = np.abs(got - ref["grad_draft"])
    bad = err > tol
    assert not bad.any(), (np.argwhere(bad)[:5], err[bad][:5], tol[bad][:5])
    assert np.allclose(gotc, ref["grad_conf"], rtol=1e-4, atol=1e-6 * max(scale, 1.0))
    # rows sum to zero
    row_tol = tol.sum(-1) + 1e-6 * np.abs(got).max(-1)
    assert np.all(np.abs(got.astype(np.float64).sum(-1)) <= row_tol)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiny_sliced(dtype):
    rng = np.random.default_rng(21)
    N, g, V = 3, 5, 1024
    d = rng.normal(0, 2.0, (N, g, V)).astype(np.float32)
    t = (d + rng.normal(0, 0.8, (N, g, V))).astype(np.float32)
    d[1, 2, :100] = -np.inf
    inp = stats_case(d, t, teacher=rng.integers(100, V, (N, g)),
                     conf_logits=rng.normal(0, 1.5, (N, g)), block_mask=np.array([1, 0, 1], np.uint8),
                     dtype=dtype)
    check(inp, scale=0.37)


@pytest.mark.parametrize("V,dtype", [(1000, "bf16"), (999, "bf16"), (1001, "f32"), (1, "f32"),
                                     (2052, "f32")])
def test_ragged_vocab(V, dtype):
    rng = np.random.default_rng(V)
    N, g = 4, 3
    d = rng.normal(0, 2.0, (N, g, V)).astype(np.float32)
    t = (d + rng.normal(0, 1.0, (N, g, V))).astype(np.float32)
    inp = stats_case(d, t, teacher=rng.integers(0, V, (N, g)), conf_logits=rng.normal(0, 1, (N, g)),
                     dtype=dtype)
    check(inp)


def test_identical_and_disjoint_rows():
    rng = np.random.default_rng(8)
    g, V = 2, 4096
    d = rng.normal(0, 2, (2, g, V)).astype(np.float32)
    t = d.copy()
    t[1] = -np.inf
    t[1, :, ::2] = rng.normal(0, 2, (g, V // 2))
    d[1, :, ::2] = -np.inf  # block 1: disjoint supports
    inp = stats_case(d, t, teacher=np.ones((2, g), np.int64), dtype="bf16")
    check(inp, w=dict(w_ce=0.0, w_l1=1.0, w_conf=1.0))
    got, _ = run(inp, w_ce=0.0, w_l1=1.0, w_conf=1.0)
    assert np.all(got[0] == 0.0)  # P == T exactly: sign 0 everywhere
    assert np.abs(got[1]).max() < 1e-6  # L1 == 2: flat


@pytest.mark.parametrize("path", ["sliced", "row"])
def test_near_rows_full_vocab(path):
    """Row pairs from equal to disjoint at V=129280 (the rows of the plain
    statistics' test): the signs of P - T agree with the oracle's wherever
    |P - T| exceeds 1e-6 of max(P, T), on the sliced path (aligned rows) and
    on the row path (rows 2 bytes off 16-byte alignment)."""
    from tests.test_gpu_parity import _misaligned, _near_rows
    si = _near_rows(2, 7, 129280, 99)
    got = None
    if path == "row":
        out = ds.dspark_accept_stats_backward(_misaligned(G.logits(si["draft"], "bf16")),
                                              _misaligned(G.logits(si["target"], "bf16")),
                                              G.i32(si["teacher"]), G.f32(si["conf_logits"]), **W)
        torch.cuda.synchronize()
        got = (out["grad_draft"].float().cpu().numpy(), out["grad_conf"].cpu().numpy())
    check(si, near_rel=1e-6, got=got)


def test_full_vocab_sliced():
    si = stats_inputs(blocks=list(range(6)), mask_every=4)
    check(si, scale=1.0 / 42)


def test_full_vocab_row_path_sampled():
    # more than 2048 row pairs: one workgroup per pair; the oracle checks a
    # sample of blocks, the row sums are checked on all of them
    cfg = dict(seed=77, N=420, gamma=5, V=129280, dtype="bf16", draft_std=3.0, noise_std=1.0)
    si = stats_inputs(cfg)
    got, gotc = run(si, **W)
    assert np.all(np.isfinite(got))
    # every row sums to 0 up to the bf16 rounding of its elements
    g64 = got.astype(np.float64)
    assert np.all(np.abs(g64.sum(-1)) <= 2.0 ** -8 * np.abs(g64).sum(-1) + 1e-6)
    for blocks in ([0, 1], [209, 419]):
        sub = stats_inputs(cfg, blocks=blocks)
        ref = O.accept_stats_backward(sub, **W)
        tol = tolerance(sub, ref["grad_draft"], 1.0, W)
        assert np.all(np.abs(got[blocks] - ref["grad_draft"]) <= tol)
        assert np.allclose(gotc[blocks], ref["grad_conf"], rtol=1e-4, atol=1e-6)


def test_empty_batch():
    z = torch.zeros((0, 5, 64), dtype=torch.float32, device=G.DEV)
    out = ds.dspark_accept_stats_backward(z, z, torch.zeros((0, 5), dtype=torch.int32, device=G.DEV),
                                          torch.zeros((0, 5), dtype=torch.float32, device=G.DEV))
    torch.cuda.synchronize()
    assert out["grad_draft"].numel() == 0
