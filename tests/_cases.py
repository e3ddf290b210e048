"""Hand-built inputs and statistics helpers for the tests.

Builds input dicts of the same layout as workloads.decode_inputs /
stats_inputs from explicit arrays, so tests can construct the special cases
they pin (one-hot rows, chains, disjoint supports).  Holds none of the
method's arithmetic.
"""

from __future__ import annotations

import numpy as np
from scipy import stats

from workloads import to_bf16


def decode_case(backbone=None, target=None, *, B=None, gamma=None, V=None, r=16, d=8,
                dtype="f32", anchor=None, w1=None, w2=None, hidden=None, embed=None,
                conf_w=None, mode=1, temperature=1.0, top_k=0, top_p=1.0,
                request_id=None, position=None, seed=0):
    """Input dict for the Markov sampler / verify built from explicit arrays.

    backbone [B,gamma,V] and target [B,gamma+1,V] are float arrays (rounded to
    bf16 if dtype == "bf16"); missing weights are zero; scalars broadcast."""
    if backbone is not None:
        B, gamma, V = backbone.shape
    elif target is not None:
        B, g1, V = target.shape
        gamma = g1 - 1
    assert B is not None and gamma is not None and V is not None

    def lg(x, shape):
        x = np.zeros(shape, np.float32) if x is None else np.asarray(x, np.float32)
        x = np.broadcast_to(x, shape)
        return to_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x)

    def vec(x, dt):
        return np.ascontiguousarray(np.broadcast_to(np.asarray(x, dt), (B,)))

    def bf(x, shape):
        x = np.zeros(shape, np.float32) if x is None else np.asarray(x, np.float32)
        return to_bf16(np.broadcast_to(x, shape))

    return dict(
        backbone=lg(backbone, (B, gamma, V)), target=lg(target, (B, gamma + 1, V)),
        anchor=vec(0 if anchor is None else anchor, np.int32),
        w1=bf(w1, (V, r)), w2=bf(w2, (V, r)), hidden=bf(hidden, (B, gamma, d)),
        embed=bf(embed, (V, d)),
        conf_w=np.ascontiguousarray(np.broadcast_to(
            np.zeros(2 * d, np.float32) if conf_w is None else np.asarray(conf_w, np.float32),
            (2 * d,))),
        mode=vec(mode, np.uint8), temperature=vec(temperature, np.float32),
        top_k=vec(top_k, np.int32), top_p=vec(top_p, np.float32),
        request_id=vec(np.arange(B) if request_id is None else request_id, np.uint32),
        position=vec(100 if position is None else position, np.int32),
        seed=seed, B=B, gamma=gamma, V=V, r=r, d=d, dtype=dtype,
    )


def stats_case(draft, target, teacher=None, conf_logits=None, block_mask=None, dtype="f32"):
    N, g, V = draft.shape
    conv = to_bf16 if dtype == "bf16" else (lambda x: np.ascontiguousarray(x, np.float32))
    return dict(draft=conv(np.asarray(draft, np.float32)),
                target=conv(np.asarray(target, np.float32)),
                teacher=np.zeros((N, g), np.int32) if teacher is None else np.asarray(teacher, np.int32),
                conf_logits=np.zeros((N, g), np.float32) if conf_logits is None
                else np.asarray(conf_logits, np.float32),
                block_mask=block_mask, N=N, gamma=g, V=V, dtype=dtype)


def softmax64(z):
    z = np.asarray(z, np.float64)
    m = np.max(z[np.isfinite(z)])
    e = np.where(np.isfinite(z), np.exp(z - m), 0.0)
    return e / e.sum()


def chisq_pvalue(samples, probs, min_expected=5.0):
    """Pearson chi-square p-value of integer samples against probabilities.

    Categories with expected count below min_expected are pooled together;
    a sample outside the support (probability 0) gives p-value 0."""
    probs = np.asarray(probs, np.float64)
    n = len(samples)
    counts = np.bincount(np.asarray(samples), minlength=probs.size).astype(np.float64)
    if counts.size > probs.size or np.any(counts[probs == 0] > 0):
        return 0.0
    exp = probs * n
    big = exp >= min_expected
    obs_b, exp_b = list(counts[big]), list(exp[big])
    if (~big).any() and exp[~big].sum() > 0:
        obs_b.append(counts[~big].sum())
        exp_b.append(exp[~big].sum())
    if len(obs_b) < 2:
        return 1.0
    return float(stats.chisquare(obs_b, exp_b).pvalue)


def binom_pvalue(k, n, p):
    return float(stats.binomtest(int(k), int(n), float(p)).pvalue)


# Per-request arrays of the decode input dicts (leading axis B); every other
# key is shared by all requests.
_PER_REQUEST = ("backbone", "target", "anchor", "hidden", "mode", "temperature", "top_k", "top_p",
                "request_id", "position")


def request_subset(inp, reqs):
    """The input dict restricted to the requests reqs (in that order)."""
    reqs = np.asarray(reqs)
    out = {k: (v[reqs] if k in _PER_REQUEST else v) for k, v in inp.items()}
    out["B"] = len(reqs)
    return out


def per_request_threaded(fn, inp, extra=(), nthreads=None, chunk=8):
    """fn(sub, *extra_sub) over request chunks of inp on a thread pool (the
    oracle's calls release the GIL); the per-request outputs concatenated.
    extra holds per-request arrays (leading axis B) sliced alongside."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    B = inp["B"]
    parts = [list(range(s, min(s + chunk, B))) for s in range(0, B, chunk)]
    nthreads = nthreads or min(16, os.cpu_count() or 1)

    def run(reqs):
        return fn(request_subset(inp, reqs), *[np.asarray(x)[reqs] for x in extra])

    with ThreadPoolExecutor(max_workers=nthreads) as ex:
        outs = list(ex.map(run, parts))
    return {k: np.concatenate([o[k] for o in outs], axis=0) for k in outs[0]}
