"""Python binding of the DSpark sampling / verification library (libdspark.so).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the stream (the current stream of the
tensors' device).  The functions carry the C ABI's names:

  dspark_markov_sample  Markov draft sampler + confidence head
  dspark_verify         exact greedy / sampled verify
  dspark_accept_stats   training-side analytic acceptance statistics

Outputs are allocated with torch on the inputs' device (or passed in through
`out=`).  A status other than DSPARK_OK raises DSparkError.  There is no CPU
fallback: without the built library every call raises.
"""

from __future__ import annotations

import atexit
import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdspark.so")

DSPARK_OK, DSPARK_EINVAL, DSPARK_EDTYPE, DSPARK_ESHAPE, DSPARK_EWORKSPACE, DSPARK_EDEVICE = range(6)
DSPARK_BF16, DSPARK_F32 = 1, 2
DSPARK_OP_MARKOV, DSPARK_OP_VERIFY, DSPARK_OP_STATS, DSPARK_OP_STATS_BACKWARD = 1, 2, 3, 4
DSPARK_OP_STATS_MARKOV = 5
DSPARK_NOALLOC_SCRATCH_BYTES = 32 << 20  # per-GPU scratch of dspark_verify_noalloc
DSPARK_MAX_GAMMA, DSPARK_MAX_RANK, DSPARK_MAX_VERIFY_BATCH = 16, 256, 65535  # as include/dspark.h
FLAG_NEAR, FLAG_NONFINITE, FLAG_RESIDUAL_ZERO, FLAG_EMPTY_ROW, FLAG_BAD_POLICY = 1, 2, 4, 8, 16

__all__ = ["DSparkError", "Policy", "lib", "dspark_markov_sample", "dspark_verify",
           "dspark_verify_noalloc",
           "dspark_accept_stats", "dspark_accept_stats_backward", "dspark_accept_stats_markov",
           "dspark_select_width", "dspark_workspace_size", "profile_enable",
           "profile_summary", "DSPARK_MAX_GAMMA", "DSPARK_MAX_RANK",
           "DSPARK_MAX_VERIFY_BATCH"]


class DSparkError(RuntimeError):
    pass


class dspark_policy(C.Structure):
    _fields_ = [("mode", C.c_void_p), ("temperature", C.c_void_p), ("top_k", C.c_void_p),
                ("top_p", C.c_void_p), ("request_id", C.c_void_p), ("position", C.c_void_p)]


_lib = None


def lib():
    """The loaded libdspark.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise DSparkError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(there is no CPU fallback)")
        L = C.CDLL(LIB_PATH)
        P, i32, u64, f32, sz = C.c_void_p, C.c_int32, C.c_uint64, C.c_float, C.c_size_t
        L.dspark_workspace_size.argtypes = [C.c_int, i32, i32, i32, i32, i32]
        L.dspark_workspace_size.restype = sz
        L.dspark_status_string.argtypes = [C.c_int]
        L.dspark_status_string.restype = C.c_char_p
        L.dspark_version.restype = C.c_int
        L.dspark_markov_sample.argtypes = [P, C.c_int, P, P, P, P, P, P, dspark_policy, u64, i32,
                                           i32, i32, i32, i32, P, P, P, P, P, P, P, P, sz, P]
        L.dspark_markov_sample.restype = C.c_int
        L.dspark_verify.argtypes = [P, C.c_int, P, P, P, P, P, P, dspark_policy, u64, i32, i32,
                                    i32, P, P, P, P, sz, P]
        L.dspark_verify.restype = C.c_int
        L.dspark_verify_noalloc.argtypes = L.dspark_verify.argtypes[:16] + [P]
        L.dspark_verify_noalloc.restype = C.c_int
        L.dspark_accept_stats.argtypes = [P, P, C.c_int, P, P, P, i32, i32, i32, f32, f32, f32,
                                          P, P, P, P, P, P, P, sz, P]
        L.dspark_accept_stats.restype = C.c_int
        L.dspark_accept_stats_markov.argtypes = [P, P, C.c_int, P, P, P, i32, P, P, P, i32, i32, i32,
                                                 f32, f32, f32, P, P, P, P, P, P, P, sz, P]
        L.dspark_accept_stats_markov.restype = C.c_int
        L.dspark_accept_stats_backward.argtypes = [P, P, C.c_int, P, P, P, i32, i32, i32, f32, f32,
                                                   f32, P, P, P, P, sz, P]
        L.dspark_accept_stats_backward.restype = C.c_int
        L.dspark_select_width.argtypes = [P, P, i32, i32, P, P, P]
        L.dspark_select_width.restype = C.c_int
        L.dspark_profile_enable.argtypes = [C.c_int]
        L.dspark_profile_enable.restype = C.c_int
        L.dspark_markov_plan.argtypes = [C.c_int]
        L.dspark_markov_plan.restype = C.c_int
        L.dspark_profile_summary.argtypes = [C.c_char_p, sz]
        L.dspark_profile_summary.restype = C.c_int
        L.dspark_release.argtypes = []
        L.dspark_release.restype = C.c_int
        _lib = L
        # the library's HIP objects go before the runtime's own teardown
        atexit.register(_release_at_exit)
    return _lib


def _release_at_exit():
    if _lib is not None:
        _lib.dspark_release()


def _check(rc):
    if rc != DSPARK_OK:
        raise DSparkError(f"dspark status {rc}: {lib().dspark_status_string(rc).decode()}")


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dev_tensor(t, dtype, name, shape=None, device=None):
    """Check that t is a contiguous GPU tensor of this dtype (and shape and
    device, when given): the library reads and writes exactly that extent."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise DSparkError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise DSparkError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise DSparkError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise DSparkError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise DSparkError(f"{name} must be on {device}, got {t.device}")
    return t


def _check_out(out, spec, device, what):
    """Check every caller-supplied output tensor against (name, dtype, shape)."""
    for name, dtype, shape in spec:
        if name not in out or out[name] is None:
            raise DSparkError(f"{what}: out is missing {name}")
        _dev_tensor(out[name], dtype, f"out[{name!r}]", shape, device)


def _logits_dtype(t, name):
    if t.dtype == torch.bfloat16:
        return DSPARK_BF16
    if t.dtype == torch.float32:
        return DSPARK_F32
    raise DSparkError(f"{name} must be bfloat16 or float32")


_ws = {}


def _workspace(op, device, nbytes):
    """A cached scratch buffer of at least nbytes per (device, stream, op).

    Calls on one stream are ordered, so they can share a buffer; calls on
    different streams may overlap, so each stream gets its own.  The buffer is
    allocated while its stream is current, so when a larger one replaces it,
    torch's allocator reuses the old memory only after that stream's pending
    work."""
    key = (device, torch.cuda.current_stream(device).cuda_stream, op)
    buf = _ws.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws[key] = buf
    return buf


def dspark_workspace_size(op, B, gamma, V, r=0, d=0):
    return int(lib().dspark_workspace_size(op, B, gamma, V, r, d))


@dataclass
class Policy:
    """Per-request sampling policy as device tensors of length B.

    top_k and top_p are both given or both None; None means that no request of
    the call truncates (the library then skips every truncation pass and the
    Markov sampler takes its untruncated one-launch kernel)."""

    mode: torch.Tensor                    # uint8: 0 greedy, 1 sampled
    temperature: torch.Tensor             # float32
    top_k: Optional[torch.Tensor]         # int32 (0 = off), or None
    top_p: Optional[torch.Tensor]         # float32 (>= 1 = off), or None
    request_id: torch.Tensor              # int32 holding the uint32 request ids
    position: torch.Tensor                # int32: absolute position of the anchor

    def c(self, B, device):
        _dev_tensor(self.mode, torch.uint8, "mode", (B,), device)
        _dev_tensor(self.temperature, torch.float32, "temperature", (B,), device)
        if (self.top_k is None) != (self.top_p is None):
            raise DSparkError("policy: top_k and top_p must both be given or both be None")
        if self.top_k is not None:
            _dev_tensor(self.top_k, torch.int32, "top_k", (B,), device)
            _dev_tensor(self.top_p, torch.float32, "top_p", (B,), device)
        _dev_tensor(self.request_id, torch.int32, "request_id", (B,), device)
        _dev_tensor(self.position, torch.int32, "position", (B,), device)
        return dspark_policy(self.mode.data_ptr(), self.temperature.data_ptr(),
                             None if self.top_k is None else self.top_k.data_ptr(),
                             None if self.top_p is None else self.top_p.data_ptr(),
                             self.request_id.data_ptr(), self.position.data_ptr())


def _stream(device):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def dspark_markov_sample(backbone, anchor, markov_w1, markov_w2, hidden, embed, conf_w,
                         policy: Policy, seed=0, out=None):
    """Markov draft sampling; returns a dict of device tensors
    draft_tokens [B,g] int32, q_logits [B,g,V] f32, q_lse, q_thr, q_tok,
    confidence [B,g] f32, flags [B,g] uint8."""
    dt = _logits_dtype(backbone, "backbone")
    _dev_tensor(backbone, backbone.dtype, "backbone")
    if backbone.dim() != 3:
        raise DSparkError("markov_sample: backbone must be [B, gamma, V]")
    B, g, V = backbone.shape
    dev = backbone.device
    _dev_tensor(markov_w1, torch.bfloat16, "markov_w1", device=dev)
    if markov_w1.dim() != 2 or hidden.dim() != 3:
        raise DSparkError("markov_sample: markov_w1 must be [V, r] and hidden [B, gamma, d]")
    r = markov_w1.shape[1]
    d = hidden.shape[2]
    _dev_tensor(markov_w1, torch.bfloat16, "markov_w1", (V, r), dev)
    _dev_tensor(markov_w2, torch.bfloat16, "markov_w2", (V, r), dev)
    _dev_tensor(hidden, torch.bfloat16, "hidden", (B, g, d), dev)
    _dev_tensor(embed, torch.bfloat16, "embed", (V, d), dev)
    _dev_tensor(conf_w, torch.float32, "conf_w", (2 * d,), dev)
    _dev_tensor(anchor, torch.int32, "anchor", (B,), dev)
    pol = policy.c(B, dev)
    spec = [("draft_tokens", torch.int32, (B, g)), ("q_logits", torch.float32, (B, g, V)),
            ("q_lse", torch.float32, (B, g)), ("q_thr", torch.float32, (B, g)),
            ("q_tok", torch.float32, (B, g)), ("confidence", torch.float32, (B, g)),
            ("flags", torch.uint8, (B, g))]
    if out is None:
        out = {name: torch.empty(shape, dtype=dtype, device=dev) for name, dtype, shape in spec}
    else:
        _check_out(out, spec, dev, "markov_sample")
    nb = dspark_workspace_size(DSPARK_OP_MARKOV, B, g, V, r, d)
    ws = _workspace(DSPARK_OP_MARKOV, dev, nb)
    rc = lib().dspark_markov_sample(
        _p(backbone), dt, _p(anchor), _p(markov_w1), _p(markov_w2), _p(hidden), _p(embed),
        _p(conf_w), pol, int(seed), B, g, V, r, d, _p(out["draft_tokens"]),
        _p(out["q_logits"]), _p(out["q_lse"]), _p(out["q_thr"]), _p(out["q_tok"]),
        _p(out["confidence"]), _p(out["flags"]), _p(ws), ws.numel(), _stream(dev))
    _check(rc)
    return out


def dspark_verify(target, draft_tokens, policy: Policy, q_logits=None, q_lse=None, q_thr=None,
                  q_tok=None, n_draft=None, seed=0, out=None):
    """Exact verify; returns dict accept_len [B] int32, out_tokens [B,g+1]
    int32, flags [B,g+1] uint8 (device tensors)."""
    dt = _logits_dtype(target, "target")
    _dev_tensor(target, target.dtype, "target")
    if target.dim() != 3:
        raise DSparkError("verify: target must be [B, gamma + 1, V]")
    B, g1, V = target.shape
    g = g1 - 1
    dev = target.device
    _dev_tensor(draft_tokens, torch.int32, "draft_tokens", (B, g), dev)
    for name, t, shape in [("q_logits", q_logits, (B, g, V)), ("q_lse", q_lse, (B, g)),
                           ("q_thr", q_thr, (B, g)), ("q_tok", q_tok, (B, g))]:
        if t is not None:
            _dev_tensor(t, torch.float32, name, shape, dev)
    if n_draft is not None:
        _dev_tensor(n_draft, torch.int32, "n_draft", (B,), dev)
    pol = policy.c(B, dev)
    spec = [("accept_len", torch.int32, (B,)), ("out_tokens", torch.int32, (B, g1)),
            ("flags", torch.uint8, (B, g1))]
    if out is None:
        out = {name: torch.empty(shape, dtype=dtype, device=dev) for name, dtype, shape in spec}
    else:
        _check_out(out, spec, dev, "verify")
    nb = dspark_workspace_size(DSPARK_OP_VERIFY, B, g, V)
    ws = _workspace(DSPARK_OP_VERIFY, dev, nb)
    rc = lib().dspark_verify(_p(target), dt, _p(draft_tokens), _p(q_logits), _p(q_lse),
                             _p(q_thr), _p(q_tok), _p(n_draft), pol, int(seed), B, g, V,
                             _p(out["accept_len"]), _p(out["out_tokens"]), _p(out["flags"]),
                             _p(ws), ws.numel(), _stream(dev))
    _check(rc)
    return out


def dspark_verify_noalloc(target, draft_tokens, policy: Policy, out, q_logits=None, q_lse=None,
                          q_thr=None, q_tok=None, n_draft=None, seed=0):
    """dspark_verify on the library's own per-GPU scratch: no workspace and no
    allocation (the caller passes out: accept_len [B] int32, out_tokens
    [B,g+1] int32, flags [B,g+1] uint8).  Calls that overlap on one GPU race."""
    dt = _logits_dtype(target, "target")
    _dev_tensor(target, target.dtype, "target")
    if target.dim() != 3:
        raise DSparkError("verify: target must be [B, gamma + 1, V]")
    B, g1, V = target.shape
    g = g1 - 1
    dev = target.device
    _dev_tensor(draft_tokens, torch.int32, "draft_tokens", (B, g), dev)
    for name, t, shape in [("q_logits", q_logits, (B, g, V)), ("q_lse", q_lse, (B, g)),
                           ("q_thr", q_thr, (B, g)), ("q_tok", q_tok, (B, g))]:
        if t is not None:
            _dev_tensor(t, torch.float32, name, shape, dev)
    if n_draft is not None:
        _dev_tensor(n_draft, torch.int32, "n_draft", (B,), dev)
    pol = policy.c(B, dev)
    _check_out(out, [("accept_len", torch.int32, (B,)), ("out_tokens", torch.int32, (B, g1)),
                     ("flags", torch.uint8, (B, g1))], dev, "verify_noalloc")
    rc = lib().dspark_verify_noalloc(_p(target), dt, _p(draft_tokens), _p(q_logits), _p(q_lse),
                                     _p(q_thr), _p(q_tok), _p(n_draft), pol, int(seed), B, g, V,
                                     _p(out["accept_len"]), _p(out["out_tokens"]), _p(out["flags"]),
                                     _stream(dev))
    _check(rc)
    return out


_STATS_OUT = ["l1", "accept_rate", "ce", "bce"]


def _stats_args(what, target, draft, teacher, conf_logits, block_mask, out, dev):
    """Checks shared by the statistics calls; returns the output dict."""
    N, g, V = draft.shape
    _dev_tensor(target, draft.dtype, "target", (N, g, V), dev)
    _dev_tensor(teacher, torch.int32, "teacher", (N, g), dev)
    _dev_tensor(conf_logits, torch.float32, "conf_logits", (N, g), dev)
    if block_mask is not None:
        _dev_tensor(block_mask, torch.uint8, "block_mask", (N,), dev)
    spec = [(name, torch.float32, (N, g)) for name in _STATS_OUT]
    spec += [("tau", torch.float32, (N,)), ("sums", torch.float32, (12,))]
    if out is None:
        return {name: torch.empty(shape, dtype=dtype, device=dev) for name, dtype, shape in spec}
    _check_out(out, spec, dev, what)
    return out


def dspark_accept_stats(draft, target, teacher, conf_logits, block_mask=None, w_ce=0.1,
                        w_l1=0.9, w_conf=1.0, out=None):
    """Acceptance statistics; returns dict l1, accept_rate, ce, bce [N,g],
    tau [N], sums [12] (float32 device tensors)."""
    dt = _logits_dtype(draft, "draft")
    _dev_tensor(draft, draft.dtype, "draft")
    if draft.dim() != 3:
        raise DSparkError("accept_stats: draft must be [N, gamma, V]")
    N, g, V = draft.shape
    dev = draft.device
    out = _stats_args("accept_stats", target, draft, teacher, conf_logits, block_mask, out, dev)
    nb = dspark_workspace_size(DSPARK_OP_STATS, N, g, V)
    ws = _workspace(DSPARK_OP_STATS, dev, nb) if nb > 0 else None
    rc = lib().dspark_accept_stats(_p(draft), _p(target), dt, _p(teacher), _p(conf_logits),
                                   _p(block_mask), N, g, V, float(w_ce), float(w_l1),
                                   float(w_conf), _p(out["l1"]), _p(out["accept_rate"]),
                                   _p(out["ce"]), _p(out["bce"]), _p(out["tau"]),
                                   _p(out["sums"]), _p(ws), 0 if ws is None else ws.numel(),
                                   _stream(dev))
    _check(rc)
    return out


def dspark_accept_stats_markov(backbone, target, anchor, markov_w1, markov_w2, teacher, conf_logits,
                               block_mask=None, w_ce=0.1, w_l1=0.9, w_conf=1.0, out=None):
    """Statistics of the teacher-forced Markov draft (backbone + W1[x] W2^T,
    x the anchor then the teacher tokens); returns the same dict as
    dspark_accept_stats."""
    dt = _logits_dtype(backbone, "backbone")
    _dev_tensor(backbone, backbone.dtype, "backbone")
    if backbone.dim() != 3:
        raise DSparkError("accept_stats_markov: backbone must be [N, gamma, V]")
    N, g, V = backbone.shape
    dev = backbone.device
    _dev_tensor(anchor, torch.int32, "anchor", (N,), dev)
    _dev_tensor(markov_w1, torch.bfloat16, "markov_w1", device=dev)
    if markov_w1.dim() != 2:
        raise DSparkError("accept_stats_markov: markov_w1 must be [V, r]")
    r = markov_w1.shape[1]
    _dev_tensor(markov_w1, torch.bfloat16, "markov_w1", (V, r), dev)
    _dev_tensor(markov_w2, torch.bfloat16, "markov_w2", (V, r), dev)
    out = _stats_args("accept_stats_markov", target, backbone, teacher, conf_logits, block_mask, out,
                      dev)
    nb = dspark_workspace_size(DSPARK_OP_STATS_MARKOV, N, g, V, r)
    ws = _workspace(DSPARK_OP_STATS_MARKOV, dev, nb) if nb > 0 else None
    rc = lib().dspark_accept_stats_markov(_p(backbone), _p(target), dt, _p(anchor), _p(markov_w1),
                                          _p(markov_w2), r, _p(teacher), _p(conf_logits),
                                          _p(block_mask), N, g, V, float(w_ce), float(w_l1),
                                          float(w_conf), _p(out["l1"]), _p(out["accept_rate"]),
                                          _p(out["ce"]), _p(out["bce"]), _p(out["tau"]),
                                          _p(out["sums"]), _p(ws), 0 if ws is None else ws.numel(),
                                          _stream(dev))
    _check(rc)
    return out


def dspark_accept_stats_backward(draft, target, teacher, conf_logits, block_mask=None, w_ce=0.1,
                                 w_l1=0.9, w_conf=1.0, grad_scale=None, out=None):
    """Gradient of grad_scale x the statistics' loss numerator; returns dict
    grad_draft [N,g,V] (the logits dtype) and grad_conf [N,g] float32 (device
    tensors).  grad_scale: a one-element float32 device tensor or None (1)."""
    dt = _logits_dtype(draft, "draft")
    _dev_tensor(draft, draft.dtype, "draft")
    if draft.dim() != 3:
        raise DSparkError("accept_stats_backward: draft must be [N, gamma, V]")
    N, g, V = draft.shape
    dev = draft.device
    _dev_tensor(target, draft.dtype, "target", (N, g, V), dev)
    _dev_tensor(teacher, torch.int32, "teacher", (N, g), dev)
    _dev_tensor(conf_logits, torch.float32, "conf_logits", (N, g), dev)
    if block_mask is not None:
        _dev_tensor(block_mask, torch.uint8, "block_mask", (N,), dev)
    if grad_scale is not None:
        _dev_tensor(grad_scale, torch.float32, "grad_scale", device=dev)
        if grad_scale.numel() != 1:
            raise DSparkError("accept_stats_backward: grad_scale must hold one value")
    spec = [("grad_draft", draft.dtype, (N, g, V)), ("grad_conf", torch.float32, (N, g))]
    if out is None:
        out = {name: torch.empty(shape, dtype=dtype, device=dev) for name, dtype, shape in spec}
    else:
        _check_out(out, spec, dev, "accept_stats_backward")
    nb = dspark_workspace_size(DSPARK_OP_STATS_BACKWARD, N, g, V)
    ws = _workspace(DSPARK_OP_STATS_BACKWARD, dev, nb) if nb > 0 else None
    rc = lib().dspark_accept_stats_backward(_p(draft), _p(target), dt, _p(teacher), _p(conf_logits),
                                            _p(block_mask), N, g, V, float(w_ce), float(w_l1),
                                            float(w_conf), _p(grad_scale), _p(out["grad_draft"]),
                                            _p(out["grad_conf"]), _p(ws),
                                            0 if ws is None else ws.numel(), _stream(dev))
    _check(rc)
    return out


def dspark_select_width(confidence, cost, want_expected=True, out=None):
    """Confidence-scheduled draft width; returns dict n_draft int32 [B] and
    expected float32 [B] (or None) as device tensors.  cost is the device
    float32 table {D, V(0), ..., V(gamma)}."""
    _dev_tensor(confidence, torch.float32, "confidence")
    if confidence.dim() != 2:
        raise DSparkError("select_width: confidence must be [B, gamma]")
    B, g = confidence.shape
    dev = confidence.device
    _dev_tensor(cost, torch.float32, "cost", (g + 2,), dev)
    if out is None:
        out = dict(n_draft=torch.empty((B,), dtype=torch.int32, device=dev),
                   expected=torch.empty((B,), dtype=torch.float32, device=dev)
                   if want_expected else None)
    else:
        _check_out(out, [("n_draft", torch.int32, (B,))], dev, "select_width")
        if out.get("expected") is not None:
            _dev_tensor(out["expected"], torch.float32, "out['expected']", (B,), dev)
    rc = lib().dspark_select_width(_p(confidence), _p(cost), B, g, _p(out["n_draft"]),
                                   _p(out["expected"]), _stream(dev))
    _check(rc)
    return out


def profile_enable(on=True):
    lib().dspark_profile_enable(1 if on else 0)


MARKOV_AUTO, MARKOV_PER_STEP, MARKOV_COOPERATIVE, MARKOV_REQUEST_GROUPS = 0, 1, 2, 3


def markov_plan(plan):
    """Set the Markov launch plan (MARKOV_AUTO, MARKOV_PER_STEP,
    MARKOV_COOPERATIVE or MARKOV_REQUEST_GROUPS, process-wide); returns the
    previous one."""
    prev = lib().dspark_markov_plan(int(plan))
    if prev < 0:
        raise DSparkError(f"unknown Markov plan {plan}")
    return prev


def profile_summary():
    """{kernel: (launches, total_ms)} of the launches recorded since the last call."""
    buf = C.create_string_buffer(1 << 16)
    _check(lib().dspark_profile_summary(buf, len(buf)))
    res = {}
    for line in buf.value.decode().splitlines():
        name, n, ms = line.split()
        res[name] = (int(n), float(ms))
    return res
