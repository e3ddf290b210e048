"""Helpers of the GPU tests: move generator dicts to the device and call the
library through its Python binding (argument marshalling only)."""

from __future__ import annotations

import numpy as np
import torch

import dspark_draft_sampling_amd as ds

DEV = torch.device("cuda:0")


def bf(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)


def logits(x, dtype):
    return bf(x) if dtype == "bf16" else torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x).astype(np.int64).astype(np.int32))).to(DEV)


def f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)


def truncates(inp):
    """True if some request of the input has top-k or top-p switched on."""
    V = inp["V"]
    tk = np.asarray(inp["top_k"])
    return bool(np.any((tk > 0) & (tk < V)) or np.any(np.asarray(inp["top_p"]) < 1.0))


def policy(inp, arrays=None):
    """The input's policy as device tensors.  arrays=None passes the
    truncation arrays only when some request truncates (None otherwise: the
    library's untruncated paths); True / False force either form."""
    if arrays is None:
        arrays = truncates(inp)
    return ds.Policy(mode=torch.from_numpy(np.ascontiguousarray(inp["mode"], np.uint8)).to(DEV),
                     temperature=f32(inp["temperature"]),
                     top_k=i32(inp["top_k"]) if arrays else None,
                     top_p=f32(inp["top_p"]) if arrays else None,
                     request_id=torch.from_numpy(np.ascontiguousarray(inp["request_id"], np.uint32)
                                                 .view(np.int32)).to(DEV),
                     position=i32(inp["position"]))


def markov(inp, arrays=None):
    out = ds.dspark_markov_sample(logits(inp["backbone"], inp["dtype"]), i32(inp["anchor"]),
                                  bf(inp["w1"]), bf(inp["w2"]), bf(inp["hidden"]), bf(inp["embed"]),
                                  f32(inp["conf_w"]), policy(inp, arrays), seed=inp["seed"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def verify(inp, draft_tokens, q=None, n_draft=None, arrays=None):
    q = q or {}
    out = ds.dspark_verify(logits(inp["target"], inp["dtype"]), i32(draft_tokens), policy(inp, arrays),
                           q_logits=f32(q["q_z"]) if "q_z" in q else None,
                           q_lse=f32(q["q_lse"]) if "q_lse" in q else None,
                           q_thr=f32(q["q_thr"]) if "q_thr" in q else None,
                           q_tok=f32(q["q_tok"]) if "q_tok" in q else None,
                           n_draft=None if n_draft is None else i32(n_draft), seed=inp["seed"])
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def stats(inp, **kw):
    out = ds.dspark_accept_stats(logits(inp["draft"], inp["dtype"]), logits(inp["target"], inp["dtype"]),
                                 i32(inp["teacher"]), f32(inp["conf_logits"]),
                                 None if inp.get("block_mask") is None else
                                 torch.from_numpy(np.ascontiguousarray(inp["block_mask"], np.uint8)).to(DEV),
                                 **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def q_of(ref):
    """The oracle Markov's proposal side in the library's stored fp32 format."""
    return dict(q_z=ref["q_z"].astype(np.float32), q_lse=ref["q_lse"].astype(np.float32),
                q_thr=ref["q_thr"].astype(np.float32), q_tok=ref["q_tok"].astype(np.float32))
