"""The decode step (Markov sample, verify, accept stats) captured in a HIP
graph and replayed: every replay gives the eager step's outputs bit for bit.

A captured Markov call runs its one-launch kernel (whole-step, request-group
or truncating) with the hand-off tag taken from its workspace, since a graph
replays its launch arguments; the eager reference runs the same kernel with
a host tag (the one-launch kernels agree bit for bit; the per-step plan sums
its records in another order).  Eager steps with the default
plan, on the same stream and workspaces, run between the replays, with
synchronisations, as a caller's own work would: their words (host tags) and
the replays' (workspace tags) meet in one workspace.
"""

from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import dspark_draft_sampling_amd as ds  # noqa: E402
from tests import _gpu as G  # noqa: E402
from workloads import decode_inputs, stats_markov_inputs  # noqa: E402


def _host(d):
    # bf16 tensors as their bit patterns (numpy has no bfloat16)
    return {k: (v.view(torch.int16) if v.dtype == torch.bfloat16 else v).cpu().numpy().copy()
            for k, v in d.items()}


@pytest.mark.parametrize("mode,plan,arrays", [("sampled", "auto", False), ("mixed", "auto", False),
                                               ("mixed", "groups", False), ("mixed", "auto", True)])
def test_decode_step_graph_replays(mode, plan, arrays):
    cfg = dict(seed=404, B=48, gamma=5, V=4096, r=32, d=32, dtype="bf16", draft_std=3.0,
               noise_std=1.0, w_std=0.05, mode=mode)
    inp = decode_inputs(cfg)
    g = inp["gamma"]
    backbone, target = G.logits(inp["backbone"], "bf16"), G.logits(inp["target"], "bf16")
    tgt_rows = target[:, :g].contiguous()
    anchor, w1, w2 = G.i32(inp["anchor"]), G.bf(inp["w1"]), G.bf(inp["w2"])
    hidden, embed, conf_w = G.bf(inp["hidden"]), G.bf(inp["embed"]), G.f32(inp["conf_w"])
    # a second set of draft logits: replays alternate between the two, so a
    # replay that took the previous replay's hand-off words for its own would
    # show it
    srcs = [backbone.clone(), G.logits(decode_inputs(dict(cfg, seed=405))["backbone"], "bf16")]
    pol = G.policy(inp, arrays)  # arrays: the truncating kernel (no request truncates)
    rng = np.random.default_rng(5)
    teacher = G.i32(rng.integers(0, inp["V"], (inp["B"], g)))
    conf_logits = G.f32(rng.standard_normal((inp["B"], g)))

    def step():
        mk = ds.dspark_markov_sample(backbone, anchor, w1, w2, hidden, embed, conf_w, pol, seed=11)
        vf = ds.dspark_verify(target, mk["draft_tokens"], pol, mk["q_logits"], mk["q_lse"], mk["q_thr"],
                              mk["q_tok"], seed=11)
        st = ds.dspark_accept_stats(backbone, tgt_rows, teacher, conf_logits)
        return mk, vf, st

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    prev = ds.markov_plan(ds.MARKOV_REQUEST_GROUPS if plan == "groups" else ds.MARKOV_AUTO)
    try:
        refs = []
        for src in srcs:  # eager, the same plan (host tag)
            with torch.cuda.stream(s):
                backbone.copy_(src)
                refs.append([_host(x) for x in step()])
            torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=s):
            outs = step()
    finally:
        ds.markov_plan(prev)
    samp = inp["mode"] != 0
    assert not np.array_equal(refs[0][0]["draft_tokens"], refs[1][0]["draft_tokens"])
    for rep in range(4):
        with torch.cuda.stream(s):
            backbone.copy_(srcs[rep % 2])
            gr.replay()
        torch.cuda.synchronize()
        got = [_host(x) for x in outs]
        for r, o in zip(refs[rep % 2], got):
            for k in r:
                if k == "q_logits":
                    assert np.array_equal(r[k][samp], o[k][samp]), (rep, k)
                else:
                    assert np.array_equal(r[k], o[k]), (rep, k)
        with torch.cuda.stream(s):
            step()  # the caller's own eager work between replays (default plan)
        torch.cuda.synchronize()
    assert not np.any(got[0]["flags"] & (1 << 5))  # no wait gave up


@pytest.mark.parametrize("N", [24, 2100])
def test_training_calls_graph_replays(N):
    """The training-side calls captured in one HIP graph: the statistics,
    their backward, the teacher-forced Markov statistics and the width
    choice.  Replays alternate between two sets of logits (copied into the
    captured tensors) and match the eager calls bit for bit.  N = 24 takes
    the sliced statistics kernels, N = 2100 (above 2048 row pairs at gamma
    1) the row kernels."""
    g = 5 if N < 2048 else 1
    sets = [stats_markov_inputs(dict(seed=60 + i, N=N, gamma=g, V=2048, dtype="bf16", draft_std=2.0,
                                     noise_std=0.6), r=32, w_std=0.1, mask_every=3) for i in range(2)]
    inp = sets[0]
    draft = G.logits(inp["backbone"], "bf16")
    target = G.logits(inp["target"], "bf16")
    srcs = [(G.logits(s["backbone"], "bf16"), G.logits(s["target"], "bf16")) for s in sets]
    teacher, conf = G.i32(inp["teacher"]), G.f32(inp["conf_logits"])
    anchor, w1, w2 = G.i32(inp["anchor"]), G.bf(inp["w1"]), G.bf(inp["w2"])
    mask = torch.from_numpy(np.ascontiguousarray(inp["block_mask"], np.uint8)).to(G.DEV)
    cost = G.f32(np.array([3.0] + [1.0 + 0.2 * k for k in range(g + 1)], np.float32))

    def calls():
        st = ds.dspark_accept_stats(draft, target, teacher, conf, mask)
        gr_ = ds.dspark_accept_stats_backward(draft, target, teacher, conf, mask)
        sm = ds.dspark_accept_stats_markov(draft, target, anchor, w1, w2, teacher, conf, mask)
        wd = ds.dspark_select_width(torch.sigmoid(conf), cost)
        return st, gr_, sm, wd

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    refs = []
    for d_, t_ in srcs:
        with torch.cuda.stream(s):
            draft.copy_(d_)
            target.copy_(t_)
            refs.append([_host({k: v for k, v in x.items() if v is not None}) for x in calls()])
        torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        outs = calls()
    for rep in range(4):
        d_, t_ = srcs[rep % 2]
        with torch.cuda.stream(s):
            draft.copy_(d_)
            target.copy_(t_)
            graph.replay()
        torch.cuda.synchronize()
        got = [_host({k: v for k, v in x.items() if v is not None}) for x in outs]
        for r, o in zip(refs[rep % 2], got):
            for k in r:
                assert np.array_equal(r[k], o[k], equal_nan=True), (rep, k)
        with torch.cuda.stream(s):
            calls()  # eager work between replays
        torch.cuda.synchronize()


def test_verify_noalloc_graph_replays():
    """dspark_verify_noalloc, for callers that cannot allocate, captured in a
    HIP graph (caller-owned outputs, the library's static scratch): replays
    alternating between two sets of target logits match dspark_verify run
    eagerly on each set, bit for bit."""
    cfg = dict(seed=808, B=48, gamma=5, V=4096, r=32, d=32, dtype="bf16", draft_std=3.0,
               noise_std=1.0, w_std=0.05, mode="mixed")
    inp = decode_inputs(cfg)
    pol = G.policy(inp)
    mk = ds.dspark_markov_sample(G.logits(inp["backbone"], "bf16"), G.i32(inp["anchor"]), G.bf(inp["w1"]),
                                 G.bf(inp["w2"]), G.bf(inp["hidden"]), G.bf(inp["embed"]), G.f32(inp["conf_w"]),
                                 pol, seed=3)
    q = dict(q_logits=mk["q_logits"], q_lse=mk["q_lse"], q_thr=mk["q_thr"], q_tok=mk["q_tok"])
    srcs = [G.logits(inp["target"], "bf16"), G.logits(decode_inputs(dict(cfg, seed=809))["target"], "bf16")]
    target = srcs[0].clone()
    B, g1 = target.shape[0], target.shape[1]
    outs = dict(accept_len=torch.zeros((B,), dtype=torch.int32, device=G.DEV),
                out_tokens=torch.zeros((B, g1), dtype=torch.int32, device=G.DEV),
                flags=torch.zeros((B, g1), dtype=torch.uint8, device=G.DEV))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    refs = []
    for src in srcs:
        with torch.cuda.stream(s):
            refs.append(_host(ds.dspark_verify(src, mk["draft_tokens"], pol, seed=3, **q)))
            ds.dspark_verify_noalloc(target, mk["draft_tokens"], pol, outs, seed=3, **q)  # warm
        torch.cuda.synchronize()
    assert not np.array_equal(refs[0]["out_tokens"], refs[1]["out_tokens"])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        ds.dspark_verify_noalloc(target, mk["draft_tokens"], pol, outs, seed=3, **q)
    for rep in range(4):
        with torch.cuda.stream(s):
            target.copy_(srcs[rep % 2])
            graph.replay()
        torch.cuda.synchronize()
        got = _host(outs)
        for k, v in refs[rep % 2].items():
            assert np.array_equal(got[k], v), (rep, k)
