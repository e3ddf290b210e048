"""GPU parity of the HIP library against the CPU oracle (needs an MI355X).

Every input comes from the seeded generator (workloads.py) or from the oracle
itself (the verify's proposals and q are the oracle Markov's, rounded to fp32);
nothing the GPU computes is fed back to the oracle.

Bars: tokens, accept lengths and integer flags bit-exact, except where the
oracle flags a decision within 1e-6 of its threshold (then the rest of that
chain is not compared); floating-point outputs within 1e-4 relative.
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
from tests._cases import decode_case, per_request_threaded, request_subset, stats_case  # noqa: E402
from workloads import STATS_CONFIG, bf16_to_f32, decode_inputs, stats_inputs, to_bf16  # noqa: E402

RTOL = 1e-4
DATA_FLAGS = O.F_NONFINITE | O.F_EMPTY


def first_flag(flags):
    """Per request, index of the first row the oracle flags NEAR (g if none)."""
    near = (flags & O.F_NEAR) != 0
    g = flags.shape[1]
    return np.where(near.any(1), near.argmax(1), g)


def check_markov(inp, got, ref, rows=None, strict=False):
    """Compare up to each request's first oracle NEAR row (strict: every row)."""
    B, g = ref["draft_tokens"].shape
    ff = np.full(B, g) if strict else first_flag(ref["flags"])
    sampled = (inp["mode"] != 0)
    n_cmp = 0
    for b in range(B):
        for k in range(g):
            if k > ff[b]:
                break  # chain may legitimately diverge after a flagged draw
            # quantities that depend only on x_{k-1}: compare up to the flagged row
            assert np.isclose(got["confidence"][b, k], ref["confidence"][b, k], rtol=RTOL, atol=1e-6), (b, k)
            if sampled[b]:
                gz, rz = got["q_logits"][b, k], ref["q_z"][b, k]
                assert np.allclose(gz, rz, rtol=RTOL, atol=1e-5), (b, k, np.abs(gz - rz).max())
                assert np.isclose(got["q_lse"][b, k], ref["q_lse"][b, k], rtol=RTOL, atol=1e-6), (b, k)
                gt, rt = got["q_thr"][b, k], ref["q_thr"][b, k]
                assert (gt == rt == -np.inf) or np.isclose(gt, rt, rtol=RTOL, atol=1e-6), (b, k, gt, rt)
            if k == ff[b]:
                break
            assert got["draft_tokens"][b, k] == ref["draft_tokens"][b, k], (b, k)
            assert np.isclose(got["q_tok"][b, k], ref["q_tok"][b, k], rtol=RTOL, atol=1e-12), (b, k)
            assert (got["flags"][b, k] & DATA_FLAGS) == (ref["flags"][b, k] & DATA_FLAGS), (b, k)
            n_cmp += 1
    return n_cmp


def check_verify(got, ref):
    flagged = (ref["flags"] & O.F_NEAR).any(1)
    ok = ~flagged
    assert np.array_equal(got["accept_len"][ok], ref["accept_len"][ok])
    assert np.array_equal(got["out_tokens"][ok], ref["out_tokens"][ok])
    assert np.array_equal(got["flags"][ok] & (DATA_FLAGS | O.F_RESID_ZERO | O.F_BAD_POLICY),
                          ref["flags"][ok] & (DATA_FLAGS | O.F_RESID_ZERO | O.F_BAD_POLICY))
    return int(flagged.sum())


# ------------------------------------------------------------------ tiny ----
@pytest.mark.parametrize("mode", ["greedy", "sampled"])
def test_markov_tiny(mode):
    inp = decode_inputs("tiny", mode=mode)
    ref = O.markov_sample(inp)
    got = G.markov(inp)
    assert check_markov(inp, got, ref) >= inp["B"] * inp["gamma"] - 2


@pytest.mark.parametrize("mode", ["greedy", "sampled"])
def test_verify_tiny(mode):
    inp = decode_inputs("tiny", mode=mode)
    mk = O.markov_sample(inp)
    q = G.q_of(mk) if mode == "sampled" else None
    ref = O.verify(inp, mk["draft_tokens"], **(q or {}))
    got = G.verify(inp, mk["draft_tokens"], q)
    assert check_verify(got, ref) == 0


def test_stats_tiny_f32_and_bf16_masked():
    for dtype, mask in [("f32", 0), ("bf16", 3)]:
        si = stats_inputs(dict(seed=11, N=9, gamma=5, V=1024, dtype=dtype, draft_std=2.0,
                               noise_std=0.5), mask_every=mask)
        ref = O.accept_stats(si)
        got = G.stats(si)
        for key in ["l1", "accept_rate", "ce", "bce", "tau"]:
            assert np.allclose(got[key], ref[key], rtol=RTOL, atol=1e-6), key
        assert np.allclose(got["sums"], ref["sums"], rtol=RTOL, atol=1e-6)


# --------------------------------------------------------- decode, full V ----
def test_markov_decode_full_size(decode_full):
    """The decode batch at full size (B = 64, V = 129280, rank 256): every
    request against the oracle (threaded over request chunks)."""
    inp = decode_full
    got = G.markov(inp)
    ref = per_request_threaded(O.markov_sample, inp)
    assert check_markov(inp, got, ref) >= inp["B"] * inp["gamma"] - 2
    assert np.all((got["draft_tokens"] >= 0) & (got["draft_tokens"] < inp["V"]))
    assert np.all((got["q_tok"] > 0) & (got["q_tok"] <= 1))
    assert np.all((got["flags"] & DATA_FLAGS) == 0)


def test_verify_decode_full_size(decode_full):
    inp = decode_full
    mk = O.markov_sample(inp)  # all 64 requests: the proposals come from the oracle
    q = G.q_of(mk)
    ref = O.verify(inp, mk["draft_tokens"], **q)
    got = G.verify(inp, mk["draft_tokens"], q)
    assert check_verify(got, ref) <= 1
    rate = ref["accept_len"].mean() / inp["gamma"]
    assert 0.2 < rate < 0.95


def test_verify_wide_greedy_full_size():
    inp = decode_inputs("wide_greedy", with_embed=False)
    from workloads import bf16_to_f32

    # proposals: the draft rows' own argmax (input preparation, not the method)
    draft = bf16_to_f32(inp["backbone"]).argmax(-1).astype(np.int32)
    ref = O.verify(inp, draft)
    got = G.verify(inp, draft)
    assert check_verify(got, ref) == 0
    emitted = (got["out_tokens"] >= 0).sum(1)
    assert np.all((emitted >= 1) & (emitted <= 8))


def test_markov_wide_greedy_full_size():
    """The wide greedy tile (64 requests x gamma 7, V = 129280, rank 256):
    the Markov draft of every request against the oracle (greedy draws are
    argmaxes: bit-exact), then the verify of those proposals."""
    inp = decode_inputs("wide_greedy")
    got = G.markov(inp)
    ref = per_request_threaded(O.markov_sample, inp)
    assert check_markov(inp, got, ref, strict=True) == inp["B"] * inp["gamma"]
    assert np.all(got["q_tok"] == 1.0) and np.all(got["flags"] == 0)
    vref = O.verify(inp, ref["draft_tokens"])
    vgot = G.verify(inp, got["draft_tokens"])
    assert check_verify(vgot, vref) == 0


def test_stats_full_vocab():
    si = stats_inputs(blocks=list(range(16)), mask_every=8)
    ref = O.accept_stats(si)
    got = G.stats(si)
    for key in ["l1", "accept_rate", "ce", "bce", "tau"]:
        assert np.allclose(got[key], ref[key], rtol=RTOL, atol=1e-6), key
    assert np.allclose(got["sums"], ref["sums"], rtol=RTOL, atol=1e-6)


def test_stats_full_config_row_path():
    """The training statistics at their full shape (2048 blocks x gamma 7,
    V=129280, bf16, every 4th block masked: 14336 row pairs, the row path).
    Blocks 0, 1, 1023 and 2047 element by element against the oracle; tau
    and the sums against the call's own per-position outputs (fp64)."""
    cfg = dict(STATS_CONFIG)
    si = stats_inputs(cfg, mask_every=4)
    got = G.stats(si)
    del si
    blocks = [0, 1, 1023, 2047]
    sub = stats_inputs(cfg, blocks=blocks, mask_every=4)
    ref = O.accept_stats(sub)
    for key in ["l1", "accept_rate", "ce", "bce", "tau"]:
        assert np.allclose(got[key][blocks], ref[key], rtol=RTOL, atol=1e-6), key
    a = got["accept_rate"].astype(np.float64)
    tau = 1.0 + np.cumprod(a, axis=1).sum(1)
    assert np.allclose(got["tau"], tau, rtol=1e-6, atol=0)
    m = (np.arange(cfg["N"]) % 4 != 3)
    g = cfg["gamma"]
    w = np.exp(-np.arange(1, g + 1) / g)
    num = (m[:, None] * w[None, :] * (0.1 * got["ce"] + 0.9 * got["l1"] + 1.0 * got["bce"])).sum()
    n = g * m.sum()
    want = [num, n, (got["l1"] * m[:, None]).sum(), n, (a * m[:, None]).sum(), n,
            (tau * m).sum(), m.sum(), (got["ce"] * m[:, None]).sum(), n, (got["bce"] * m[:, None]).sum(), n]
    assert np.allclose(got["sums"], want, rtol=1e-5, atol=0)


def _near_rows(N, gamma, V, seed):
    """Row pairs at bf16 whose L1 spans 0 to 2: per position, in turn, equal
    rows; 300 logits moved by one bf16 step; every logit moved by
    bf16(N(0, 0.004^2)) noise (most round back, L1 about 4e-5); the row's
    maximum and 50 others moved by one step; disjoint supports; the target
    N(0, 1) away; the target offset by 100 (separate shifts); an empty
    target row; the target offset by +10.5 and by -9.75 exactly (logits on
    a 1/8 grid), with 300 logits moved by 1/8.  L1 is offset-invariant."""
    rng = np.random.default_rng(seed)
    d = rng.normal(0, 3.0, (N, gamma, V)).astype(np.float32)
    d = bf16_to_f32(to_bf16(d))
    t = d.copy()
    for i in range(N * gamma):
        b, k = divmod(i, gamma)
        x = d[b, k]
        kind = i % 10
        if kind == 1:
            idx = rng.choice(V, 300, replace=False)
            t[b, k, idx] = bf16_to_f32(to_bf16(x[idx] * np.float32(1 + 2.0 ** -7)))
        elif kind == 2:
            t[b, k] = bf16_to_f32(to_bf16(x + rng.normal(0, 0.004, V).astype(np.float32)))
        elif kind == 3:
            idx = np.concatenate([[np.argmax(x)], rng.choice(V, 50, replace=False)])
            t[b, k, idx] = bf16_to_f32(to_bf16(x[idx] * np.float32(1 + 2.0 ** -7)))
        elif kind == 4:
            t[b, k, 1::2] = -np.inf
            d[b, k, ::2] = -np.inf
        elif kind == 5:
            t[b, k] = x + rng.normal(0, 1.0, V).astype(np.float32)
        elif kind == 6:
            t[b, k] = x + np.float32(100.0)
        elif kind == 7:
            t[b, k] = -np.inf
        elif kind in (8, 9):
            g = np.clip(np.round(x * 8.0) / 8.0, -15.0, 15.0).astype(np.float32)
            d[b, k] = g
            t[b, k] = g + np.float32(10.5 if kind == 8 else -9.75)
            idx = rng.choice(V, 300, replace=False)
            t[b, k, idx] += np.float32(0.125) * rng.choice(np.array([-1.0, 1.0], np.float32), 300)
    teacher = rng.integers(0, V, (N, gamma))
    teacher[:, :] = np.argmax(np.where(np.isfinite(d), d, -1e30), axis=2)
    return stats_case(d, t, teacher=teacher, conf_logits=rng.normal(0, 1, (N, gamma)), dtype="bf16")


def _misaligned(x):
    """x (a device tensor) in storage that starts 2 bytes off a 16-byte boundary."""
    buf = torch.empty(x.numel() + 8, dtype=x.dtype, device=x.device)
    y = buf[1:1 + x.numel()].view(x.shape)
    y.copy_(x)
    assert y.is_contiguous() and y.data_ptr() % 16 != 0
    return y


@pytest.mark.parametrize("path", ["sliced", "row"])
def test_stats_near_rows_full_vocab(path):
    """L1 at V=129280 from 0 (equal rows) through 4e-5 (bf16 noise) to 2
    (disjoint), relative to L1 itself (1e-4), on the sliced path (28 pairs,
    aligned rows) and on the row path (the same rows 2 bytes off 16-byte
    alignment)."""
    si = _near_rows(4, 7, 129280, 2024)
    ref = O.accept_stats(si)
    if path == "sliced":
        got = G.stats(si)
    else:
        out = ds.dspark_accept_stats(_misaligned(G.logits(si["draft"], "bf16")),
                                     _misaligned(G.logits(si["target"], "bf16")),
                                     G.i32(si["teacher"]), G.f32(si["conf_logits"]))
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in out.items()}
    l1r, l1g = ref["l1"], got["l1"].astype(np.float64)
    bad = np.abs(l1g - l1r) > RTOL * l1r + 1e-9
    assert not bad.any(), (np.argwhere(bad), l1g[bad], l1r[bad])
    assert np.all(l1g.reshape(-1)[0::10] == 0.0)  # equal rows
    assert np.all(l1g.reshape(-1)[4::10] == 2.0)  # disjoint supports
    assert np.all(l1g.reshape(-1)[7::10] == 1.0)  # empty target row
    assert 1e-5 < l1r.reshape(-1)[2::10].max() < 1e-3
    assert np.all(l1r.reshape(-1)[8::10] < 1e-2) and np.all(l1r.reshape(-1)[9::10] < 1e-2)
    for key in ["accept_rate", "bce", "tau"]:
        assert np.allclose(got[key], ref[key], rtol=RTOL, atol=1e-6), key
    ce_ok = np.isfinite(ref["ce"])
    assert np.allclose(got["ce"][ce_ok], ref["ce"][ce_ok], rtol=RTOL, atol=1e-6)


# ---------------------------------------------------------- flag rate -------
def test_flag_rate_many_draws():
    """Sampled Markov + verify over ~1e5 draws on the tiny shape: unflagged
    draws bit-exact, flagged share below 1e-4."""
    inp = decode_inputs("tiny", B=8192, mode="sampled", with_embed=True)
    ref = O.markov_sample(inp)
    got = G.markov(inp)
    check_markov(inp, got, ref)
    vref = O.verify(inp, ref["draft_tokens"], **G.q_of(ref))
    vgot = G.verify(inp, ref["draft_tokens"], G.q_of(ref))
    check_verify(vgot, vref)
    draws = inp["B"] * inp["gamma"] + int((vref["accept_len"] + 1).sum())
    flagged = int(((ref["flags"] & O.F_NEAR) != 0).sum() + ((vref["flags"] & O.F_NEAR) != 0).sum())
    assert draws > 60000
    assert flagged / draws < 1e-4


# ---------------------------------------------------------- edge cases ------
def test_empty_batch():

    inp = decode_inputs("tiny", B=0, with_embed=True)
    out = G.verify(inp, np.zeros((0, inp["gamma"]), np.int32))
    assert out["accept_len"].shape == (0,)
    si = stats_case(np.zeros((0, 3, 16), np.float32), np.zeros((0, 3, 16), np.float32))
    got = G.stats(si)
    assert np.all(got["sums"] == 0)
    assert ds.dspark_workspace_size(ds.DSPARK_OP_VERIFY, 0, 5, 1024) >= 0


@pytest.mark.parametrize("V,dtype,B", [(999, "f32", 5), (1000, "bf16", 70), (1, "f32", 2)])
def test_ragged_shapes(V, dtype, B):
    cfg = dict(seed=77, B=B, gamma=3, V=V, r=16, d=24, dtype=dtype, draft_std=2.0,
               noise_std=0.5, w_std=0.3, mode="mixed")
    inp = decode_inputs(cfg)
    ref = O.markov_sample(inp)
    got = G.markov(inp)
    check_markov(inp, got, ref)
    vref = O.verify(inp, ref["draft_tokens"], **G.q_of(ref))
    vgot = G.verify(inp, ref["draft_tokens"], G.q_of(ref))
    assert check_verify(vgot, vref) <= 1


def test_max_gamma_and_rank():
    """The largest draft width (gamma = DSPARK_MAX_GAMMA) with the largest
    rank, mixed greedy / sampled requests: Markov, verify and the statistics
    of the same rows."""
    cfg = dict(seed=91, B=9, gamma=ds.DSPARK_MAX_GAMMA, V=2048, r=ds.DSPARK_MAX_RANK, d=64, dtype="bf16",
               draft_std=2.0, noise_std=0.5, w_std=0.05, mode="mixed")
    inp = decode_inputs(cfg)
    ref = O.markov_sample(inp)
    got = G.markov(inp)
    check_markov(inp, got, ref)
    vref = O.verify(inp, ref["draft_tokens"], **G.q_of(ref))
    vgot = G.verify(inp, ref["draft_tokens"], G.q_of(ref))
    assert check_verify(vgot, vref) <= 1
    si = stats_inputs(dict(seed=92, N=9, gamma=ds.DSPARK_MAX_GAMMA, V=2048, dtype="bf16", draft_std=2.0,
                           noise_std=0.5), mask_every=3)
    sref = O.accept_stats(si)
    sgot = G.stats(si)
    for key in ["l1", "accept_rate", "ce", "bce", "tau"]:
        assert np.allclose(sgot[key], sref[key], rtol=RTOL, atol=1e-6), key
    assert np.allclose(sgot["sums"], sref["sums"], rtol=RTOL, atol=1e-6)


def test_n_draft_and_bad_rows():
    rng = np.random.default_rng(5)
    B, g, V = 6, 4, 700
    tgt = rng.normal(0, 2, (B, g + 1, V)).astype(np.float32)
    tgt[1, 2, 10] = np.nan         # request 1: NaN in row 2
    tgt[2, 0, :] = -np.inf         # request 2: empty row 0
    tgt[3, 1, 5] = np.inf          # request 3: +inf in row 1
    tgt[4, :, 7] = 50.0            # request 4: a clear argmax
    inp = decode_case(None, tgt, B=B, gamma=g, V=V, mode=[0, 0, 0, 1, 0, 1])
    draft = rng.integers(0, V, (B, g)).astype(np.int32)
    draft[4] = 7
    n_draft = np.array([4, 3, 2, 4, 1, 0], np.int32)
    kq, zq, lq, tq, _ = O.policy_row(np.zeros(V), 1.0, 0, 1.0)
    q = dict(q_z=np.zeros((B, g, V), np.float32), q_lse=np.full((B, g), lq, np.float32),
             q_thr=np.full((B, g), -np.inf, np.float32), q_tok=np.full((B, g), 1.0 / V, np.float32))
    ref = O.verify(inp, draft, n_draft=n_draft, **q)
    got = G.verify(inp, draft, q, n_draft=n_draft)
    assert np.array_equal(got["flags"] & DATA_FLAGS, ref["flags"] & DATA_FLAGS)
    clean = [0, 4, 5]  # requests without a bad row
    assert np.array_equal(got["accept_len"][clean], ref["accept_len"][clean])
    assert np.array_equal(got["out_tokens"][clean], ref["out_tokens"][clean])
    assert got["accept_len"][4] == 1 and got["out_tokens"][4, 1] == 7


def test_greedy_ties_lowest_index():
    V = 20000  # three row slices in the fp32 vector path
    tgt = np.zeros((2, 3, V), np.float32)
    tgt[:, :, [17000, 9000, 3000, 17]] = 5.0  # equal maxima in different slices
    inp = decode_case(None, tgt, B=2, gamma=2, V=V, mode=0)
    got = G.verify(inp, np.array([[17, 17], [3000, 17]], np.int32))
    assert list(got["out_tokens"][0]) == [17, 17, 17]
    assert list(got["out_tokens"][1]) == [17, -1, -1]


@pytest.mark.parametrize("N,gamma,V,dtype", [(300, 7, 512, "bf16"), (5, 3, 1001, "f32"),
                                             (2, 7, 129280, "bf16")])
def test_stats_paths(N, gamma, V, dtype):
    """Both stats paths: item-sliced (small batches) and one workgroup per row
    pair (>= 2048 pairs, or rows not 16-byte aligned)."""
    si = stats_inputs(dict(seed=21, N=N, gamma=gamma, V=V, dtype=dtype, draft_std=3.0,
                           noise_std=1.0), mask_every=4)
    ref = O.accept_stats(si)
    got = G.stats(si)
    for key in ["l1", "accept_rate", "ce", "bce", "tau"]:
        assert np.allclose(got[key], ref[key], rtol=RTOL, atol=1e-6), key
    assert np.allclose(got["sums"], ref["sums"], rtol=RTOL, atol=1e-6)


@pytest.mark.parametrize("N,gamma,V,dtype", [(6, 5, 4096, "bf16"), (300, 7, 512, "bf16"),
                                             (4, 3, 2000, "f32")])
def test_stats_identical_near_and_disjoint_rows(N, gamma, V, dtype):
    """Both stats paths on rows whose L1 is 0 (identical), tiny (the target
    perturbed by 1e-3 to 3e-2) or 2 (disjoint supports): the kernels form L1
    as 2 (1 - sum min(P, T)), so these check its rounding where L1 is small,
    against the oracle's direct sum |P - T| (binary64)."""
    rng = np.random.default_rng(N * V)
    d = rng.normal(0, 3.0, (N, gamma, V)).astype(np.float32)
    scale = np.array([0.0, 1e-3, 1e-2, 3e-2])[np.arange(N * gamma) % 4].reshape(N, gamma, 1)
    t = (d + scale * rng.normal(0, 1.0, d.shape)).astype(np.float32)
    t[0, 0] = d[0, 0]
    t[-1, -1] = -np.inf
    t[-1, -1, ::2] = rng.normal(0, 3.0, V - V // 2)
    d[-1, -1, ::2] = -np.inf  # disjoint supports
    teacher = rng.integers(1, V, (N, gamma))
    teacher[-1, -1] = 1  # a token the disjoint row's draft keeps
    si = stats_case(d, t, teacher=teacher, conf_logits=rng.normal(0, 1, (N, gamma)), dtype=dtype)
    ref = O.accept_stats(si)
    got = G.stats(si)
    for key in ["l1", "accept_rate", "ce", "bce", "tau"]:
        assert np.allclose(got[key], ref[key], rtol=RTOL, atol=1e-6), key
    assert np.allclose(got["sums"], ref["sums"], rtol=RTOL, atol=1e-6)
    assert got["l1"][0, 0] <= 1e-6 and got["accept_rate"][0, 0] >= 1 - 1e-6
    assert got["l1"][-1, -1] == 2.0 and got["accept_rate"][-1, -1] == 0.0


@pytest.mark.parametrize("config", ["decode", "truncated"])
def test_markov_plans_agree(config, decode_full, truncated_full):
    """The launch plans agree at full size: the untruncated one-launch kernel
    (no truncation arrays; ordinary and cooperative launch), the truncating
    one-launch kernel (arrays passed, all off for the decode batch) and the
    per-step kernels.  Tokens, flags, z and thresholds bit for bit; the
    log-normalisers up to the order of their fp32 partial sums (the plans
    combine partials over different workgroup shapes)."""

    inp = decode_full if config == "decode" else truncated_full
    prev = ds.markov_plan(ds.MARKOV_AUTO)
    try:
        fused = G.markov(inp)
        fused_arrays = G.markov(inp, arrays=True)
        ds.markov_plan(ds.MARKOV_COOPERATIVE)
        coop = G.markov(inp)
        ds.markov_plan(ds.MARKOV_REQUEST_GROUPS)
        groups = G.markov(inp)
        ds.markov_plan(ds.MARKOV_PER_STEP)
        step = G.markov(inp)
    finally:
        ds.markov_plan(prev)
    samp = inp["mode"] != 0
    for other in (coop, groups):
        # the whole-step kernel (ordinary and cooperative launch) and the
        # request-group kernel (decode batch) form the same records and
        # combine them alike
        for k in ("draft_tokens", "q_thr", "confidence", "flags", "q_lse", "q_tok"):
            assert np.array_equal(fused[k], other[k]), k
        assert np.array_equal(fused["q_logits"][samp], other["q_logits"][samp])
    for other in (step, fused_arrays):
        for k in ("draft_tokens", "q_thr", "confidence", "flags"):
            assert np.array_equal(fused[k], other[k]), k
        for k in ("q_lse", "q_tok"):
            assert np.allclose(fused[k], other[k], rtol=1e-6, atol=0), k
        assert np.array_equal(fused["q_logits"][samp], other["q_logits"][samp])
    for o in (fused, fused_arrays, coop, groups, step):
        assert not np.any(o["flags"] & (1 << 5))  # no wait gave up


@pytest.mark.parametrize("B,V,dtype", [(33, 5000, "f32"), (48, 4096, "bf16"), (100, 2049, "bf16"),
                                       (256, 1536, "f32")])
def test_markov_request_groups(B, V, dtype):
    """The request-group one-launch kernel (MARKOV_REQUEST_GROUPS without
    truncation arrays, 33..256 requests) against the oracle on every request,
    and bit for bit against the whole-step kernel (AUTO): full and partly
    absent groups (B % 16), slices past the vocabulary, greedy and sampled
    requests side by side, per-request temperatures."""
    cfg = dict(seed=91 + B, B=B, gamma=5, V=V, r=32, d=24, dtype=dtype, draft_std=2.0,
               noise_std=0.5, w_std=0.3, mode="mixed")
    inp = decode_inputs(cfg)
    inp["temperature"] = np.random.default_rng(B).uniform(0.5, 1.5, B).astype(np.float32)
    ref = O.markov_sample(inp)
    prev = ds.markov_plan(ds.MARKOV_REQUEST_GROUPS)
    try:
        got = G.markov(inp)
        ds.markov_plan(ds.MARKOV_AUTO)
        whole = G.markov(inp)
    finally:
        ds.markov_plan(prev)
    assert check_markov(inp, got, ref) >= B * inp["gamma"] // 2
    samp = inp["mode"] != 0
    for k in ("draft_tokens", "q_lse", "q_thr", "q_tok", "confidence", "flags"):
        assert np.array_equal(got[k], whole[k]), k
    assert np.array_equal(got["q_logits"][samp], whole["q_logits"][samp])
    assert not np.any(got["flags"] & (1 << 5))  # no wait gave up


def test_markov_untruncated_256_full_size(truncated_full):
    """256 requests at full size (V = 129280, rank 256, the truncated
    workload's policies with truncation switched off, so no truncation
    arrays): the whole-step kernel's four 64-request tiles and the
    request-group kernel's sixteen groups.  Requests in every tile and at
    the tile and group edges against the oracle, and the two plans bit for
    bit on every request."""
    inp = dict(truncated_full)
    inp["top_k"] = np.zeros_like(inp["top_k"])
    inp["top_p"] = np.ones_like(inp["top_p"])
    assert not G.truncates(inp)
    prev = ds.markov_plan(ds.MARKOV_AUTO)
    try:
        whole = G.markov(inp)
        ds.markov_plan(ds.MARKOV_REQUEST_GROUPS)
        groups = G.markov(inp)
    finally:
        ds.markov_plan(prev)
    reqs = np.array([0, 5, 15, 16, 63, 64, 100, 127, 128, 150, 191, 192, 224, 255])
    sub = request_subset(inp, reqs)
    ref = per_request_threaded(O.markov_sample, sub)
    got = {k: v[reqs] for k, v in whole.items()}
    assert check_markov(sub, got, ref) >= len(reqs) * inp["gamma"] - 2
    samp = inp["mode"] != 0
    for k in ("draft_tokens", "q_lse", "q_thr", "q_tok", "confidence", "flags"):
        assert np.array_equal(groups[k], whole[k]), k
    assert np.array_equal(groups["q_logits"][samp], whole["q_logits"][samp])
    assert not np.any(whole["flags"] & (1 << 5)) and not np.any(groups["flags"] & (1 << 5))


def test_markov_stale_workspace(decode_full):
    """A one-launch call accepts only words tagged with its own epoch: a
    workspace left by earlier calls of the other one-launch kernel and of the
    per-step kernels (same buffer, other layouts) changes nothing."""
    inp = decode_full
    prev = ds.markov_plan(ds.MARKOV_AUTO)
    try:
        ref = G.markov(inp)
        G.markov(inp, arrays=True)  # truncating kernel: chunk records in the same area
        ds.markov_plan(ds.MARKOV_PER_STEP)
        G.markov(inp)  # untagged chunk records in the same area
        ds.markov_plan(ds.MARKOV_AUTO)
        again = G.markov(inp)
    finally:
        ds.markov_plan(prev)
    for k in ref:
        assert np.array_equal(ref[k], again[k]), k


def test_markov_concurrent_streams(decode_full):
    """Two one-launch Markov calls enqueued at once on two streams: the
    library chains its one-launch grids on the device, so neither grid waits
    on compute units the other holds, and the binding gives each stream its
    own workspace; both end with a lone call's results and no wait gives
    up."""

    inp = decode_full
    ref = G.markov(inp)
    args = (G.logits(inp["backbone"], inp["dtype"]), G.i32(inp["anchor"]), G.bf(inp["w1"]),
            G.bf(inp["w2"]), G.bf(inp["hidden"]), G.bf(inp["embed"]), G.f32(inp["conf_w"]),
            G.policy(inp))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        o1 = ds.dspark_markov_sample(*args, seed=inp["seed"])
    with torch.cuda.stream(s2):
        o2 = ds.dspark_markov_sample(*args, seed=inp["seed"])
    torch.cuda.synchronize()
    for o in (o1, o2):
        got = {k: v.cpu().numpy() for k, v in o.items()}
        for k in ("draft_tokens", "q_thr", "confidence", "flags", "q_lse", "q_tok"):
            assert np.array_equal(got[k], ref[k]), k
        assert not np.any(got["flags"] & (1 << 5))

def test_markov_repeatable(truncated_full):
    """Two calls on the truncated batch (candidate cuts for top-k rows, the
    weight histogram for spread top-p rows) give bit-identical outputs: the
    kept-set sums are exact integer sums and every other reduction has a
    fixed order."""
    a = G.markov(truncated_full)
    b = G.markov(truncated_full)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k
