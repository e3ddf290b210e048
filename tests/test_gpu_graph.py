"""The decode step (Markov sample, verify, accept stats) captured in a HIP
graph and replayed: every replay gives the eager step's outputs bit for bit.

A captured Markov call runs the per-step plan (a one-launch grid would keep
one call's hand-off tag for all of its replays), so the eager reference runs
that plan too.  Eager steps with the default plan, on the same stream and
workspaces, run between the replays, with synchronisations, as a caller's
own work would.
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
from workloads import decode_inputs  # noqa: E402


def _host(d):
    return {k: v.cpu().numpy().copy() for k, v in d.items()}


@pytest.mark.parametrize("mode", ["sampled", "mixed"])
def test_decode_step_graph_replays(mode):
    cfg = dict(seed=404, B=48, gamma=5, V=4096, r=32, d=32, dtype="bf16", draft_std=3.0,
               noise_std=1.0, w_std=0.05, mode=mode)
    inp = decode_inputs(cfg)
    g = inp["gamma"]
    backbone, target = G.logits(inp["backbone"], "bf16"), G.logits(inp["target"], "bf16")
    tgt_rows = target[:, :g].contiguous()
    anchor, w1, w2 = G.i32(inp["anchor"]), G.bf(inp["w1"]), G.bf(inp["w2"])
    hidden, embed, conf_w = G.bf(inp["hidden"]), G.bf(inp["embed"]), G.f32(inp["conf_w"])
    pol = G.policy(inp)
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
    prev = ds.markov_plan(ds.MARKOV_PER_STEP)
    try:
        with torch.cuda.stream(s):
            ref = [_host(x) for x in step()]  # eager, the plan a capture runs
    finally:
        ds.markov_plan(prev)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        outs = step()
    samp = inp["mode"] != 0
    for rep in range(3):
        with torch.cuda.stream(s):
            gr.replay()
        torch.cuda.synchronize()
        got = [_host(x) for x in outs]
        for r, o in zip(ref, got):
            for k in r:
                if k == "q_logits":
                    assert np.array_equal(r[k][samp], o[k][samp]), (rep, k)
                else:
                    assert np.array_equal(r[k], o[k]), (rep, k)
        with torch.cuda.stream(s):
            step()  # the caller's own eager work between replays (default plan)
        torch.cuda.synchronize()
    assert not np.any(got[0]["flags"] & (1 << 5))  # no wait gave up
