"""The Python binding's argument checks: every call rejects a tensor of the
wrong length, dtype, layout or device with DSparkError before anything is
launched (the library reads and writes exactly the extents it is given, so a
short tensor would otherwise be read or written past its end).  These need
GPU tensors: on the CPU the device check fires first.  Each case also checks
that the valid call next to it succeeds, so a rejection is the check's and
not a broken fixture's.
"""

from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import dspark_draft_sampling_amd as ds  # noqa: E402

DEV = torch.device("cuda:0")
B, G, V, R, D = 4, 3, 300, 16, 16


def _policy(b=B, truncate=True, **over):
    f = dict(mode=torch.ones(b, dtype=torch.uint8, device=DEV),
             temperature=torch.ones(b, dtype=torch.float32, device=DEV),
             top_k=torch.zeros(b, dtype=torch.int32, device=DEV) if truncate else None,
             top_p=torch.ones(b, dtype=torch.float32, device=DEV) if truncate else None,
             request_id=torch.arange(b, dtype=torch.int32, device=DEV),
             position=torch.zeros(b, dtype=torch.int32, device=DEV))
    f.update(over)
    return ds.Policy(**f)


def _markov_args():
    g = torch.Generator().manual_seed(5)
    bf = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).to(DEV)  # noqa: E731
    return dict(backbone=bf(B, G, V), anchor=torch.arange(B, dtype=torch.int32, device=DEV),
                markov_w1=bf(V, R), markov_w2=bf(V, R), hidden=bf(B, G, D), embed=bf(V, D),
                conf_w=torch.randn(2 * D, generator=g).to(DEV), policy=_policy())


def _verify_args():
    g = torch.Generator().manual_seed(6)
    return dict(target=torch.randn(B, G + 1, V, generator=g).to(torch.bfloat16).to(DEV),
                draft_tokens=torch.randint(0, V, (B, G), generator=g, dtype=torch.int32).to(DEV),
                policy=_policy())


def _stats_args():
    g = torch.Generator().manual_seed(7)
    return dict(draft=torch.randn(B, G, V, generator=g).to(DEV),
                target=torch.randn(B, G, V, generator=g).to(DEV),
                teacher=torch.randint(0, V, (B, G), generator=g, dtype=torch.int32).to(DEV),
                conf_logits=torch.randn(B, G, generator=g).to(DEV))


def _short(t):
    return t.flatten()[:-1].clone() if t.dim() == 1 else t[..., :-1].contiguous()


def _raises(fn, **kw):
    with pytest.raises(ds.DSparkError):
        fn(**kw)


def test_markov_sample_rejects_bad_args():
    a = _markov_args()
    ds.dspark_markov_sample(**a)
    torch.cuda.synchronize()
    for name in ["anchor", "markov_w1", "markov_w2", "hidden", "embed", "conf_w"]:
        _raises(ds.dspark_markov_sample, **{**a, name: _short(a[name])})
    _raises(ds.dspark_markov_sample, **{**a, "markov_w2": a["markov_w2"].float()})
    _raises(ds.dspark_markov_sample, **{**a, "anchor": a["anchor"].long()})
    _raises(ds.dspark_markov_sample, **{**a, "backbone": a["backbone"].half()})
    _raises(ds.dspark_markov_sample, **{**a, "hidden": a["hidden"].transpose(0, 1)})
    _raises(ds.dspark_markov_sample, **{**a, "embed": a["embed"].cpu()})
    for field in ["mode", "temperature", "top_k", "top_p", "request_id", "position"]:
        _raises(ds.dspark_markov_sample,
                **{**a, "policy": _policy(**{field: _short(getattr(a["policy"], field))})})
    _raises(ds.dspark_markov_sample, **{**a, "policy": _policy(top_k=None)})
    # consistent shapes the library itself refuses: a rank that is not a multiple of 16
    _raises(ds.dspark_markov_sample, **{**a, "markov_w1": a["markov_w1"][:, :8].contiguous(),
                                        "markov_w2": a["markov_w2"][:, :8].contiguous()})
    out = ds.dspark_markov_sample(**a)
    for name in out:
        bad = dict(out)
        bad[name] = _short(out[name])
        _raises(ds.dspark_markov_sample, **a, out=bad)
    bad = dict(out)
    del bad["q_tok"]
    _raises(ds.dspark_markov_sample, **a, out=bad)


def test_verify_rejects_bad_args():
    a = _verify_args()
    mk = ds.dspark_markov_sample(**_markov_args())
    a["draft_tokens"] = mk["draft_tokens"]
    q = {name: mk[name] for name in ["q_logits", "q_lse", "q_thr", "q_tok"]}
    nd = torch.full((B,), G, dtype=torch.int32, device=DEV)
    out = ds.dspark_verify(**a, **q, n_draft=nd)
    torch.cuda.synchronize()
    for fn in (ds.dspark_verify,
               lambda **kw: ds.dspark_verify_noalloc(out=dict(out), **kw)):
        _raises(fn, **{**a, "draft_tokens": _short(a["draft_tokens"])})
        for name in q:
            _raises(fn, **a, **{**q, name: _short(q[name])})
        _raises(fn, **a, **q, n_draft=_short(nd))
        _raises(fn, **a, **q, n_draft=nd.long())
        _raises(fn, **{**a, "policy": _policy(b=B - 1)})
    for name in out:
        bad = dict(out)
        bad[name] = _short(out[name])
        _raises(ds.dspark_verify, **a, out=bad)
        _raises(ds.dspark_verify_noalloc, **a, out=bad)


def test_stats_rejects_bad_args():
    a = _stats_args()
    mask = torch.ones(B, dtype=torch.uint8, device=DEV)
    out = ds.dspark_accept_stats(**a, block_mask=mask)
    grads = ds.dspark_accept_stats_backward(**a, block_mask=mask)
    torch.cuda.synchronize()
    for fn in (ds.dspark_accept_stats, ds.dspark_accept_stats_backward):
        for name in ["target", "teacher", "conf_logits"]:
            _raises(fn, **{**a, name: _short(a[name])})
        _raises(fn, **a, block_mask=_short(mask))
        _raises(fn, **a, block_mask=mask.bool())
        _raises(fn, **{**a, "target": a["target"].to(torch.bfloat16)})
    for name in out:
        bad = dict(out)
        bad[name] = _short(out[name])
        _raises(ds.dspark_accept_stats, **a, out=bad)
    for name in grads:
        bad = dict(grads)
        bad[name] = _short(grads[name])
        _raises(ds.dspark_accept_stats_backward, **a, out=bad)
    _raises(ds.dspark_accept_stats_backward, **a,
            grad_scale=torch.ones(2, dtype=torch.float32, device=DEV))


def test_stats_markov_rejects_bad_args():
    a = _stats_args()
    g = torch.Generator().manual_seed(8)
    m = dict(backbone=a["draft"].to(torch.bfloat16), target=a["target"].to(torch.bfloat16),
             anchor=torch.arange(B, dtype=torch.int32, device=DEV),
             markov_w1=torch.randn(V, R, generator=g).to(torch.bfloat16).to(DEV),
             markov_w2=torch.randn(V, R, generator=g).to(torch.bfloat16).to(DEV),
             teacher=a["teacher"], conf_logits=a["conf_logits"])
    ds.dspark_accept_stats_markov(**m)
    torch.cuda.synchronize()
    for name in ["anchor", "markov_w1", "markov_w2", "teacher", "conf_logits"]:
        _raises(ds.dspark_accept_stats_markov, **{**m, name: _short(m[name])})
    _raises(ds.dspark_accept_stats_markov, **{**m, "target": m["target"].float()})
    _raises(ds.dspark_accept_stats_markov, **{**m, "markov_w1": m["markov_w1"][:, :R - 2].contiguous(),
                                              "markov_w2": m["markov_w2"]})


def test_select_width_rejects_bad_args():
    conf = torch.rand(B, G, device=DEV)
    cost = torch.ones(G + 2, device=DEV)
    ds.dspark_select_width(conf, cost)
    torch.cuda.synchronize()
    _raises(ds.dspark_select_width, confidence=conf, cost=_short(cost))
    _raises(ds.dspark_select_width, confidence=conf.double(), cost=cost)
    _raises(ds.dspark_select_width, confidence=conf, cost=cost,
            out=dict(n_draft=torch.empty(B - 1, dtype=torch.int32, device=DEV)))
    _raises(ds.dspark_select_width, confidence=conf, cost=cost,
            out=dict(n_draft=torch.empty(B, dtype=torch.int32, device=DEV),
                     expected=torch.empty(B + 1, dtype=torch.float32, device=DEV)))
