"""dspark_verify_noalloc (the verify on the library's own per-GPU scratch,
for callers that cannot allocate) against dspark_verify on the same device
inputs, bit for bit, on two calls in a row: the decode batch (B = 64, gamma
5, V = 129280, bf16, sampled, the Markov sampler's q) and then a smaller one
(B = 8, gamma 3, V = 1000, fp32, every other request greedy, truncation
arrays on); plus the size check.  Both sides are the HIP library; the
oracle is not involved.
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


def _outs(B, g1, fill):
    return {"accept_len": torch.full((B,), fill, dtype=torch.int32, device=G.DEV),
            "out_tokens": torch.full((B, g1), fill, dtype=torch.int32, device=G.DEV),
            "flags": torch.full((B, g1), fill & 0xFF, dtype=torch.uint8, device=G.DEV)}


def _both(inp, arrays=None):
    """Markov proposals on the device, then both verify entry points on them."""
    pol = G.policy(inp, arrays)
    mk = ds.dspark_markov_sample(G.logits(inp["backbone"], inp["dtype"]), G.i32(inp["anchor"]),
                                 G.bf(inp["w1"]), G.bf(inp["w2"]), G.bf(inp["hidden"]), G.bf(inp["embed"]),
                                 G.f32(inp["conf_w"]), pol, seed=inp["seed"])
    tgt = G.logits(inp["target"], inp["dtype"])
    q = dict(q_logits=mk["q_logits"], q_lse=mk["q_lse"], q_thr=mk["q_thr"], q_tok=mk["q_tok"])
    B, g1 = tgt.shape[0], tgt.shape[1]
    ref = ds.dspark_verify(tgt, mk["draft_tokens"], pol, seed=inp["seed"], **q)
    got = ds.dspark_verify_noalloc(tgt, mk["draft_tokens"], pol, _outs(B, g1, 77), seed=inp["seed"], **q)
    torch.cuda.synchronize()
    return ({k: v.cpu().numpy() for k, v in ref.items()}, {k: v.cpu().numpy() for k, v in got.items()})


def test_noalloc_matches_verify_twice():
    ref, got = _both(decode_inputs("decode"))
    for k in ref:
        assert np.array_equal(got[k], ref[k]), k
    assert (ref["out_tokens"] >= 0).sum() >= 64  # one token per request at least
    # second call, smaller: the scratch keeps the first call's contents
    small = decode_inputs("tiny", B=8, gamma=3, V=1000, mode="mixed", policy="random")
    ref, got = _both(small, arrays=True)
    for k in ref:
        assert np.array_equal(got[k], ref[k]), k


def test_noalloc_size_limit():
    # B = 65535 rows of gamma 16 over V = 129280 need more than the scratch:
    # EWORKSPACE on the host, nothing launched (the tensors are never read)
    assert ds.dspark_workspace_size(ds.DSPARK_OP_VERIFY, 65535, 16, 129280) > ds.DSPARK_NOALLOC_SCRATCH_BYTES
    tiny = torch.zeros(1, dtype=torch.int32, device=G.DEV)
    pol = ds.dspark_policy(tiny.data_ptr(), tiny.data_ptr(), None, None, tiny.data_ptr(), tiny.data_ptr())
    rc = ds.lib().dspark_verify_noalloc(ds._p(tiny), 1, ds._p(tiny), None, None, None, None, None, pol, 0,
                                        65535, 16, 129280, ds._p(tiny), ds._p(tiny), ds._p(tiny), None)
    assert rc == ds.DSPARK_EWORKSPACE
