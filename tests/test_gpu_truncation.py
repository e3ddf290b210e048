"""GPU parity of truncated sampling (top-k / top-p on both p and q).

The kept set of a row is decided on device by a candidate cut (chunk maxima
bound the cut, the candidates are sorted and cut exactly) with a radix select
over the whole row as the fallback; these cases reach both: value ties at the
top-k and top-p boundaries, top_k = 1 / V - 1 / >= V, top_p = 0 / tiny,
near-flat rows whose kept set overflows the candidate buffer, rows of more
chunks than the bound sorts, unaligned rows, and the truncated batch at its
full size (256 requests, V = 129280, mixed greedy / sampled policies).
"""

from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from oracle import oracle as O  # noqa: E402
from tests import _gpu as G  # noqa: E402
from tests._cases import decode_case, per_request_threaded  # noqa: E402
from tests.test_gpu_parity import check_markov, check_verify  # noqa: E402

# (temperature, top_k, top_p) per request
POLICIES = [(1.0, 1, 1.0), (1.0, 5, 1.0), (0.7, 20, 1.0), (1.0, 0, 0.9), (1.0, 0, 0.0),
            (1.3, 0, 0.5), (0.5, 50, 0.8), (1.0, -1, 1.0), (1.0, 0, 1e-6), (2.0, 7, 0.3),
            (1.0, 10**9, 0.95), (0.9, 3, 0.999)]


def _policy_case(V, dtype, quant, std, seed, policies=POLICIES, gamma=3):
    """Sampled requests with the given policies; zero Markov weights (z = l / T
    exactly on both sides); logits N(0, std^2), rounded to multiples of quant
    (0: not rounded) so that equal values meet the cut boundaries."""
    rng = np.random.default_rng(seed)
    B = len(policies)
    bb = rng.normal(0, std, (B, gamma, V))
    tg = np.concatenate([bb, rng.normal(0, std, (B, 1, V))], 1) + rng.normal(0, std / 3, (B, gamma + 1, V))
    if quant:
        bb, tg = np.round(bb / quant) * quant, np.round(tg / quant) * quant
    T = [p[0] for p in policies]
    tk = [V - 1 if p[1] == -1 else p[1] for p in policies]
    tp = [p[2] for p in policies]
    return decode_case(bb, tg, dtype=dtype, mode=1, temperature=T, top_k=tk, top_p=tp,
                       request_id=np.arange(B) * 7 + 3, seed=seed)


CASES = {
    "ties_f32": dict(V=3000, dtype="f32", quant=0.5, std=2.0, seed=11),
    "ties_bf16": dict(V=4096, dtype="bf16", quant=0.25, std=2.0, seed=12),
    "smooth_f32": dict(V=6000, dtype="f32", quant=0.0, std=3.0, seed=13),
    "unaligned_f32": dict(V=999, dtype="f32", quant=0.5, std=2.0, seed=14),
    # near-flat rows: the top-p kept set holds thousands of tokens
    "flat_bf16": dict(V=20000, dtype="bf16", quant=0.0, std=0.05, seed=15),
    # thousands of tokens tie at the top value: the candidates overflow
    "tied_flat_f32": dict(V=20000, dtype="f32", quant=0.5, std=0.3, seed=17),
    # more chunks than the bound sorts (radix select only)
    "wide_f32": dict(V=270000, dtype="f32", quant=0.0, std=2.0, seed=16,
                     policies=[(1.0, 50, 1.0), (0.8, 0, 0.9), (1.0, 20, 0.8)], gamma=2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_truncation_cases(name):
    inp = _policy_case(**CASES[name])
    print(f"# truncation case {name}: B={inp['B']} V={inp['V']} {inp['dtype']}", flush=True)
    ref = O.markov_sample(inp)
    got = G.markov(inp)
    # z is l / T on both sides, so ties are ties on both: compare every row
    assert check_markov(inp, got, ref, strict=True) == inp["B"] * inp["gamma"]
    assert np.all(np.isfinite(ref["q_thr"][[i for i, p in enumerate(_pol(inp)) if p]]))
    q = G.q_of(ref)
    vref = O.verify(inp, ref["draft_tokens"], **q)
    vgot = G.verify(inp, ref["draft_tokens"], q)
    assert check_verify(vgot, vref) <= 1


def _pol(inp):
    """Per request: is its policy truncating?"""
    V = inp["V"]
    return [(0 < k < V) or p < 1.0 for k, p in zip(inp["top_k"], inp["top_p"])]


def test_truncated_full_size(truncated_full):
    """The 256-request mixed-policy truncated batch at full size: Markov and
    verify on every request against the oracle (threaded over request
    chunks), the verify fed the oracle's proposals."""
    inp = truncated_full
    B, g, V = inp["B"], inp["gamma"], inp["V"]
    print(f"# truncated batch B={B} V={V}: oracle on every request", flush=True)
    ref = per_request_threaded(O.markov_sample, inp)

    got = G.markov(inp)
    assert check_markov(inp, got, ref) >= B * g - 8
    assert np.all((got["draft_tokens"] >= 0) & (got["draft_tokens"] < V))
    samp = inp["mode"] != 0
    assert np.all((got["q_tok"][samp] > 0) & (got["q_tok"][samp] <= 1))
    trunc = np.array(_pol(inp)) & samp
    assert np.all(np.isfinite(got["q_thr"][trunc])) and np.all(got["q_thr"][samp & ~trunc] == -np.inf)

    qs = G.q_of(ref)
    vgot = G.verify(inp, ref["draft_tokens"], qs)
    vref = per_request_threaded(lambda s, d, qz, ql, qt, qk: O.verify(s, d, qz, ql, qt, qk), inp,
                                extra=(ref["draft_tokens"], qs["q_z"], qs["q_lse"], qs["q_thr"], qs["q_tok"]))
    assert check_verify(vgot, vref) <= 2
    assert np.all((vgot["accept_len"] >= 0) & (vgot["accept_len"] <= g))
    last = vgot["out_tokens"][np.arange(B), vgot["accept_len"]]
    assert np.all((last >= 0) & (last < V))
