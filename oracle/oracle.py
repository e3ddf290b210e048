"""ctypes view of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The GPU library never does, and the oracle shares no code with it:
the arithmetic lives in dspark_oracle.cpp (binary64 throughout); this file only
marshals numpy arrays.

Inputs are the dicts produced by workloads.decode_inputs / stats_inputs.
Outputs are numpy arrays in binary64 (token and flag arrays in int32 / uint8).
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdspark_oracle.so")

_lib = None

DTYPES = {"bf16": 1, "f32": 2}

F_NEAR, F_NONFINITE, F_RESID_ZERO, F_EMPTY, F_BAD_POLICY = 1, 2, 4, 8, 16
(TAG_DRAFT_TOKEN, TAG_ACCEPT, TAG_TARGET_TOKEN, TAG_DRAFT_CHUNK, TAG_TARGET_CHUNK, TAG_DRAFT_SUB,
 TAG_TARGET_SUB) = 0, 1, 2, 3, 4, 5, 6
CHUNK, SUB = 256, 16  # tokens per level-1 chunk and per level-2 sub-chunk of the sampler


def lib():
    """Load the oracle library, building it first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b  # noqa: PLC0415

            _b.build()
        _lib = C.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


def _declare(L):
    P = C.c_void_p
    i32, u32, u64, f64 = C.c_int32, C.c_uint32, C.c_uint64, C.c_double
    L.oracle_philox4x32_10.argtypes = [P, P, P]
    L.oracle_philox4x32_10.restype = None
    L.oracle_philox_word.argtypes = [u64, u32, i32, u32, u32]
    L.oracle_philox_word.restype = u32
    L.oracle_gumbel.argtypes = [u64, u32, i32, u32, u32]
    L.oracle_gumbel.restype = f64
    L.oracle_accept_uniform.argtypes = [u64, i32, u32]
    L.oracle_accept_uniform.restype = f64
    L.oracle_sample_three_level.argtypes = [P, i32, u64, u32, i32, u32, u32, u32, P]
    L.oracle_sample_three_level.restype = i32
    L.oracle_policy_row.argtypes = [P, i32, f64, i32, f64, i32, P, P, P, P, P]
    L.oracle_policy_row.restype = i32
    L.oracle_markov_sample.argtypes = [P, i32, P, P, P, P, P, P, P, P, P, P, P, P,
                                       u64, i32, i32, i32, i32, i32, P, P, P, P, P,
                                       P, P, P]
    L.oracle_markov_sample.restype = i32
    L.oracle_verify.argtypes = [P, i32, P, P, P, P, P, P, P, P, P, P, P, P, u64,
                                i32, i32, i32, P, P, P, P]
    L.oracle_verify.restype = i32
    L.oracle_accept_stats.argtypes = [P, P, i32, P, P, P, i32, i32, i32, f64, f64,
                                      f64, P, P, P, P, P, P]
    L.oracle_accept_stats.restype = i32
    L.oracle_accept_stats2.argtypes = [P, i32, P, i32, P, P, P, i32, i32, i32, f64, f64, f64,
                                       P, P, P, P, P, P]
    L.oracle_accept_stats2.restype = i32
    L.oracle_accept_stats_markov.argtypes = [P, P, i32, P, P, P, i32, P, P, P, i32, i32, i32, f64,
                                             f64, f64, P, P, P, P, P, P]
    L.oracle_accept_stats_markov.restype = i32
    L.oracle_accept_stats_backward.argtypes = [P, P, i32, P, P, P, i32, i32, i32, f64, f64,
                                               f64, f64, P, P]
    L.oracle_accept_stats_backward.restype = i32
    L.oracle_select_width.argtypes = [P, P, i32, i32, P, P]
    L.oracle_select_width.restype = i32


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


# ---- primitives -----------------------------------------------------------
def philox4x32_10(ctr, key):
    c = _c(ctr, np.uint32)
    k = _c(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().oracle_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def philox_word(seed, i, position, request, tag):
    return int(lib().oracle_philox_word(seed, i, position, request, tag))


def gumbel(seed, i, position, request, tag):
    return float(lib().oracle_gumbel(seed, i, position, request, tag))


def accept_uniform(seed, position, request):
    return float(lib().oracle_accept_uniform(seed, position, request))


def sample_three_level(lw, seed, request, position, tag_chunk=TAG_DRAFT_CHUNK,
                       tag_sub=TAG_DRAFT_SUB, tag_token=TAG_DRAFT_TOKEN):
    """Three-level Gumbel-max draw (chunk, sub-chunk, token) from log-weights lw
    (-inf = excluded).  Returns (token or -1, near flag)."""
    a = _c(lw, np.float64)
    near = C.c_int32(0)
    v = lib().oracle_sample_three_level(_p(a), a.size, seed, request, position,
                                        tag_chunk, tag_sub, tag_token, C.byref(near))
    return int(v), bool(near.value)


def policy_row(l, T=1.0, top_k=0, top_p=1.0, exact_order=True):
    """Row policy: returns (kept uint8[V], z[V], lse, thr, near)."""
    a = _c(l, np.float64)
    V = a.size
    kept = np.zeros(V, np.uint8)
    z = np.zeros(V, np.float64)
    lse, thr, near = C.c_double(), C.c_double(), C.c_int32()
    lib().oracle_policy_row(_p(a), V, float(T), int(top_k), float(top_p),
                            int(bool(exact_order)), _p(kept), _p(z),
                            C.byref(lse), C.byref(thr), C.byref(near))
    return kept, z, lse.value, thr.value, bool(near.value)


# ---- the three calls ------------------------------------------------------
def _logits(x, dtype):
    return _c(x, np.uint16 if dtype == "bf16" else np.float32)


def markov_sample(inp, forced_tokens=None, want_q=True):
    """Oracle of the Markov draft sampler on an input dict.

    Returns draft_tokens [B,g] int32, q_z [B,g,V] (or None), q_lse, q_thr,
    q_tok, confidence [B,g] float64, flags [B,g] uint8.
    """
    B, g, V, r, d = inp["B"], inp["gamma"], inp["V"], inp["r"], inp["d"]
    bb = _logits(inp["backbone"], inp["dtype"])
    assert bb.shape == (B, g, V)
    out = dict(
        draft_tokens=np.zeros((B, g), np.int32),
        q_z=np.zeros((B, g, V), np.float64) if want_q else None,
        q_lse=np.zeros((B, g)), q_thr=np.zeros((B, g)), q_tok=np.zeros((B, g)),
        confidence=np.zeros((B, g)), flags=np.zeros((B, g), np.uint8),
    )
    arrs = [_c(inp["anchor"], np.int32), _c(inp["w1"], np.uint16), _c(inp["w2"], np.uint16),
            _c(inp["hidden"], np.uint16), _c(inp["embed"], np.uint16),
            _c(inp["conf_w"], np.float32), _c(inp["mode"], np.uint8),
            _c(inp["temperature"], np.float32), _c(inp["top_k"], np.int32),
            _c(inp["top_p"], np.float32), _c(inp["request_id"], np.uint32),
            _c(inp["position"], np.int32)]
    ft = _c(forced_tokens, np.int32)
    rc = lib().oracle_markov_sample(
        _p(bb), DTYPES[inp["dtype"]], *[_p(a) for a in arrs], int(inp["seed"]),
        B, g, V, r, d, _p(ft), _p(out["draft_tokens"]), _p(out["q_z"]),
        _p(out["q_lse"]), _p(out["q_thr"]), _p(out["q_tok"]), _p(out["confidence"]),
        _p(out["flags"]))
    assert rc == 0
    return out


def verify(inp, draft_tokens, q_z=None, q_lse=None, q_thr=None, q_tok=None, n_draft=None):
    """Oracle of the exact verify.

    q_* are the proposal side in the library's stored fp32 format; they are
    rounded to float32 here if given in binary64.  Returns accept_len [B],
    out_tokens [B,g+1], flags [B,g+1], p_tok [B,g] (p_{k-1}(x_k) where tested).
    """
    B, g, V = inp["B"], inp["gamma"], inp["V"]
    tg = _logits(inp["target"], inp["dtype"])
    assert tg.shape == (B, g + 1, V)
    if q_tok is None:
        q_tok = np.ones((B, g), np.float32)
    if q_z is None:
        q_z = np.zeros((B, g, V), np.float32)
        q_lse = np.zeros((B, g), np.float32)
        q_thr = np.zeros((B, g), np.float32)
    arrs = [_c(draft_tokens, np.int32), _c(q_z, np.float32), _c(q_lse, np.float32),
            _c(q_thr, np.float32), _c(q_tok, np.float32), _c(n_draft, np.int32),
            _c(inp["mode"], np.uint8), _c(inp["temperature"], np.float32),
            _c(inp["top_k"], np.int32), _c(inp["top_p"], np.float32),
            _c(inp["request_id"], np.uint32), _c(inp["position"], np.int32)]
    out = dict(accept_len=np.zeros(B, np.int32),
               out_tokens=np.zeros((B, g + 1), np.int32),
               flags=np.zeros((B, g + 1), np.uint8),
               p_tok=np.full((B, g), np.nan))
    rc = lib().oracle_verify(_p(tg), DTYPES[inp["dtype"]], *[_p(a) for a in arrs],
                             int(inp["seed"]), B, g, V, _p(out["accept_len"]),
                             _p(out["out_tokens"]), _p(out["flags"]), _p(out["p_tok"]))
    assert rc == 0
    return out


def accept_stats(inp, w_ce=0.1, w_l1=0.9, w_conf=1.0):
    """Oracle of the training-side acceptance statistics."""
    N, g, V = inp["N"], inp["gamma"], inp["V"]
    dr = _logits(inp["draft"], inp["dtype"])
    tg = _logits(inp["target"], inp["dtype"])
    assert dr.shape == (N, g, V) and tg.shape == (N, g, V)
    te = _c(inp["teacher"], np.int32)
    cl = _c(inp["conf_logits"], np.float32)
    bm = _c(inp.get("block_mask"), np.uint8)
    out = dict(l1=np.zeros((N, g)), accept_rate=np.zeros((N, g)), ce=np.zeros((N, g)),
               bce=np.zeros((N, g)), tau=np.zeros(N), sums=np.zeros(12))
    rc = lib().oracle_accept_stats(_p(dr), _p(tg), DTYPES[inp["dtype"]], _p(te), _p(cl),
                                   _p(bm), N, g, V, w_ce, w_l1, w_conf, _p(out["l1"]),
                                   _p(out["accept_rate"]), _p(out["ce"]), _p(out["bce"]),
                                   _p(out["tau"]), _p(out["sums"]))
    assert rc == 0
    return out


def _stats_out(N, g):
    return dict(l1=np.zeros((N, g)), accept_rate=np.zeros((N, g)), ce=np.zeros((N, g)),
                bce=np.zeros((N, g)), tau=np.zeros(N), sums=np.zeros(12))


def accept_stats_f64_draft(draft64, inp, w_ce=0.1, w_l1=0.9, w_conf=1.0):
    """The statistics with binary64 draft rows (test helper: feeds rows the
    oracle itself produced, such as Markov z rows, without rounding)."""
    N, g, V = inp["N"], inp["gamma"], inp["V"]
    dr = np.ascontiguousarray(draft64, np.float64)
    assert dr.shape == (N, g, V)
    tg = _logits(inp["target"], inp["dtype"])
    out = _stats_out(N, g)
    rc = lib().oracle_accept_stats2(_p(dr), 3, _p(tg), DTYPES[inp["dtype"]], _p(_c(inp["teacher"], np.int32)),
                                    _p(_c(inp["conf_logits"], np.float32)),
                                    _p(_c(inp.get("block_mask"), np.uint8)), N, g, V, w_ce, w_l1,
                                    w_conf, _p(out["l1"]), _p(out["accept_rate"]), _p(out["ce"]),
                                    _p(out["bce"]), _p(out["tau"]), _p(out["sums"]))
    assert rc == 0
    return out


def accept_stats_markov(inp, w_ce=0.1, w_l1=0.9, w_conf=1.0):
    """Oracle of the statistics of the teacher-forced Markov draft: inp holds
    backbone (the parallel logits, in place of draft), target, anchor, w1, w2,
    r, teacher, conf_logits, block_mask, N, gamma, V, dtype."""
    N, g, V, r = inp["N"], inp["gamma"], inp["V"], inp["r"]
    bb = _logits(inp["backbone"], inp["dtype"])
    tg = _logits(inp["target"], inp["dtype"])
    assert bb.shape == (N, g, V) and tg.shape == (N, g, V)
    out = _stats_out(N, g)
    rc = lib().oracle_accept_stats_markov(
        _p(bb), _p(tg), DTYPES[inp["dtype"]], _p(_c(inp["anchor"], np.int32)),
        _p(_c(inp["w1"], np.uint16)), _p(_c(inp["w2"], np.uint16)), r,
        _p(_c(inp["teacher"], np.int32)), _p(_c(inp["conf_logits"], np.float32)),
        _p(_c(inp.get("block_mask"), np.uint8)), N, g, V, w_ce, w_l1, w_conf, _p(out["l1"]),
        _p(out["accept_rate"]), _p(out["ce"]), _p(out["bce"]), _p(out["tau"]), _p(out["sums"]))
    assert rc == 0
    return out


def accept_stats_backward(inp, w_ce=0.1, w_l1=0.9, w_conf=1.0, scale=1.0):
    """Oracle of the gradient of the statistics' loss numerator (times
    scale): dict grad_draft [N,g,V] and grad_conf [N,g], binary64."""
    N, g, V = inp["N"], inp["gamma"], inp["V"]
    dr = _logits(inp["draft"], inp["dtype"])
    tg = _logits(inp["target"], inp["dtype"])
    assert dr.shape == (N, g, V) and tg.shape == (N, g, V)
    te = _c(inp["teacher"], np.int32)
    cl = _c(inp["conf_logits"], np.float32)
    bm = _c(inp.get("block_mask"), np.uint8)
    out = dict(grad_draft=np.zeros((N, g, V)), grad_conf=np.zeros((N, g)))
    rc = lib().oracle_accept_stats_backward(_p(dr), _p(tg), DTYPES[inp["dtype"]], _p(te), _p(cl),
                                            _p(bm), N, g, V, w_ce, w_l1, w_conf, scale,
                                            _p(out["grad_draft"]), _p(out["grad_conf"]))
    assert rc == 0
    return out


def select_width(confidence, cost):
    """Oracle of the confidence-scheduled draft width.

    confidence: [B, gamma] per-proposal acceptance predictions; cost: the
    gamma + 2 values {D, V(0), ..., V(gamma)}.  Returns (n_draft int32 [B],
    expected float64 [B]).
    """
    c = _c(confidence, np.float32)
    assert c.ndim == 2
    B, g = c.shape
    co = _c(cost, np.float32)
    assert co.shape == (g + 2,)
    n = np.zeros(B, np.int32)
    e = np.zeros(B)
    rc = lib().oracle_select_width(_p(c), _p(co), B, g, _p(n), _p(e))
    assert rc == 0
    return n, e

