"""The C-ABI library on the CPU: it loads, exports every call the header
declares, and validates arguments on the host before touching the device
(no compute call is made here)."""

from __future__ import annotations

import ctypes as C
import os
import re

import pytest

import dspark_draft_sampling_amd as ds

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")

FAKE = C.c_void_p(4096)  # a non-NULL, 16-byte aligned pointer that is never dereferenced


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ds.LIB_PATH):
        pytest.skip("libdspark.so not built")
    return ds.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_\w+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert {"dspark_markov_sample", "dspark_verify", "dspark_accept_stats",
            "dspark_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def policy():
    return ds.dspark_policy(4096, 4096, 4096, 4096, 4096, 4096)


def verify(L, target=FAKE, dtype=1, B=4, gamma=5, V=1024, ws=FAKE, wsb=1 << 30, pol=None, out=FAKE):
    return L.dspark_verify(target, dtype, FAKE, FAKE, FAKE, FAKE, FAKE, None, pol or policy(), 0,
                           B, gamma, V, out, FAKE, FAKE, ws, wsb, None)


def markov(L, B=4, gamma=5, V=1024, r=16, d=64, w1=FAKE, wsb=1 << 30, dtype=1):
    return L.dspark_markov_sample(FAKE, dtype, FAKE, w1, FAKE, FAKE, FAKE, FAKE, policy(), 0, B,
                                  gamma, V, r, d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  wsb, None)


def stats(L, N=4, gamma=5, V=1024, dtype=1, sums=FAKE):
    return L.dspark_accept_stats(FAKE, FAKE, dtype, FAKE, FAKE, None, N, gamma, V, 0.1, 0.9, 1.0,
                                 FAKE, FAKE, FAKE, FAKE, FAKE, sums, None, 0, None)


def stats_bwd(L, N=4, gamma=5, V=1024, dtype=1, grad=FAKE, ws=FAKE, wsb=1 << 30):
    return L.dspark_accept_stats_backward(FAKE, FAKE, dtype, FAKE, FAKE, None, N, gamma, V, 0.1, 0.9,
                                          1.0, None, grad, FAKE, ws, wsb, None)


def test_stats_backward_validation(L):
    assert stats_bwd(L, N=-1) == ds.DSPARK_EINVAL
    assert stats_bwd(L, gamma=0) == ds.DSPARK_EINVAL
    assert stats_bwd(L, dtype=9) == ds.DSPARK_EDTYPE
    assert stats_bwd(L, gamma=17) == ds.DSPARK_ESHAPE
    assert stats_bwd(L, grad=None) == ds.DSPARK_EINVAL
    assert stats_bwd(L, ws=None) == ds.DSPARK_EWORKSPACE
    assert stats_bwd(L, wsb=16) == ds.DSPARK_EWORKSPACE
    assert stats_bwd(L, N=0, grad=None, ws=None) == ds.DSPARK_OK
    # the row path (many pairs) needs no workspace
    assert ds.dspark_workspace_size(ds.DSPARK_OP_STATS_BACKWARD, 2048, 7, 129280) == 0
    assert ds.dspark_workspace_size(ds.DSPARK_OP_STATS_BACKWARD, 64, 5, 129280) > 0


def stats_mk(L, N=4, gamma=5, V=1024, r=16, w1=FAKE, anchor=FAKE, ws=FAKE, wsb=1 << 30):
    return L.dspark_accept_stats_markov(FAKE, FAKE, 1, anchor, w1, FAKE, r, FAKE, FAKE, None, N, gamma,
                                        V, 0.1, 0.9, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, wsb,
                                        None)


def test_stats_markov_validation(L):
    assert stats_mk(L, N=-1) == ds.DSPARK_EINVAL
    assert stats_mk(L, r=0) == ds.DSPARK_EINVAL
    assert stats_mk(L, r=24) == ds.DSPARK_ESHAPE
    assert stats_mk(L, r=512) == ds.DSPARK_ESHAPE
    assert stats_mk(L, gamma=17) == ds.DSPARK_ESHAPE
    assert stats_mk(L, anchor=None) == ds.DSPARK_EINVAL
    assert stats_mk(L, w1=None) == ds.DSPARK_EINVAL
    assert stats_mk(L, w1=C.c_void_p(4098)) == ds.DSPARK_EINVAL  # misaligned factor
    assert stats_mk(L, ws=None) == ds.DSPARK_EWORKSPACE
    assert stats_mk(L, wsb=16) == ds.DSPARK_EWORKSPACE
    assert ds.dspark_workspace_size(ds.DSPARK_OP_STATS_MARKOV, 4, 5, 1024, 16) > 0


def width(L, B=4, gamma=5, conf=FAKE, cost=FAKE, out=FAKE):
    return L.dspark_select_width(conf, cost, B, gamma, out, None, None)


def test_select_width_validation(L):
    assert width(L, B=-1) == ds.DSPARK_EINVAL
    assert width(L, gamma=0) == ds.DSPARK_EINVAL
    assert width(L, gamma=17) == ds.DSPARK_ESHAPE
    assert width(L, conf=None) == ds.DSPARK_EINVAL
    assert width(L, cost=None) == ds.DSPARK_EINVAL
    assert width(L, out=None) == ds.DSPARK_EINVAL
    assert width(L, B=0, conf=None, out=None) == ds.DSPARK_OK  # empty batch: no-op
    assert width(L, B=0, cost=None) == ds.DSPARK_EINVAL


def test_verify_validation(L):
    assert verify(L, B=-1) == ds.DSPARK_EINVAL
    assert verify(L, gamma=0) == ds.DSPARK_EINVAL
    assert verify(L, V=0) == ds.DSPARK_EINVAL
    assert verify(L, dtype=7) == ds.DSPARK_EDTYPE
    assert verify(L, gamma=17) == ds.DSPARK_ESHAPE
    assert verify(L, V=(1 << 30) + 1) == ds.DSPARK_ESHAPE
    assert verify(L, B=65536) == ds.DSPARK_ESHAPE  # the decide grid's row limit
    assert verify(L, target=None) == ds.DSPARK_EINVAL
    assert verify(L, out=None) == ds.DSPARK_EINVAL
    assert verify(L, pol=ds.dspark_policy(4096, None, 4096, 4096, 4096, 4096)) == ds.DSPARK_EINVAL
    # top_k and top_p: both given or both NULL (no request truncates)
    assert verify(L, pol=ds.dspark_policy(4096, 4096, None, 4096, 4096, 4096)) == ds.DSPARK_EINVAL
    assert verify(L, pol=ds.dspark_policy(4096, 4096, 4096, None, 4096, 4096)) == ds.DSPARK_EINVAL
    assert verify(L, pol=ds.dspark_policy(4096, 4096, None, None, 4096, 4096),
                  ws=None) == ds.DSPARK_EWORKSPACE  # the policy itself passes
    assert verify(L, ws=None) == ds.DSPARK_EWORKSPACE
    assert verify(L, wsb=16) == ds.DSPARK_EWORKSPACE
    assert verify(L, B=0, target=None, out=None, ws=None) == ds.DSPARK_OK  # empty batch: no-op


def test_markov_validation(L):
    assert markov(L, r=24) == ds.DSPARK_ESHAPE
    assert markov(L, r=512) == ds.DSPARK_ESHAPE
    assert markov(L, r=0) == ds.DSPARK_EINVAL
    assert markov(L, d=0) == ds.DSPARK_EINVAL
    assert markov(L, d=70000) == ds.DSPARK_ESHAPE
    assert markov(L, w1=C.c_void_p(4104)) == ds.DSPARK_EINVAL  # weights must be 16-byte aligned
    assert markov(L, w1=None) == ds.DSPARK_EINVAL
    assert markov(L, wsb=8) == ds.DSPARK_EWORKSPACE
    assert markov(L, dtype=0) == ds.DSPARK_EDTYPE
    assert markov(L, B=0) == ds.DSPARK_OK


def test_stats_validation(L):
    assert stats(L, N=-1) == ds.DSPARK_EINVAL
    assert stats(L, sums=None) == ds.DSPARK_EINVAL
    assert stats(L, gamma=0) == ds.DSPARK_EINVAL
    assert stats(L, dtype=3) == ds.DSPARK_EDTYPE


def test_workspace_sizes(L):
    for op in (ds.DSPARK_OP_MARKOV, ds.DSPARK_OP_VERIFY):
        a = ds.dspark_workspace_size(op, 64, 5, 129280, 256, 4096)
        b = ds.dspark_workspace_size(op, 256, 5, 129280, 256, 4096)
        assert 0 < a <= b
    assert ds.dspark_workspace_size(99, 64, 5, 129280) == 0
    assert ds.dspark_workspace_size(ds.DSPARK_OP_VERIFY, 64, 0, 129280) == 0


def test_status_strings(L):
    for s in range(6):
        assert L.dspark_status_string(s)
    assert L.dspark_version() >= 100


def test_binding_refuses_cpu_tensors(L):
    import torch

    with pytest.raises(ds.DSparkError):
        ds.dspark_accept_stats(torch.zeros(1, 1, 4), torch.zeros(1, 1, 4),
                               torch.zeros(1, 1, dtype=torch.int32), torch.zeros(1, 1))


def test_markov_plan_switch(L):
    prev = L.dspark_markov_plan(1)
    try:
        assert prev in (0, 1, 2)
        assert L.dspark_markov_plan(0) == 1
        assert L.dspark_markov_plan(2) == 0       # cooperative launch
        assert L.dspark_markov_plan(0) == 2
        assert L.dspark_markov_plan(7) == -1      # unknown: refused, unchanged
        assert L.dspark_markov_plan(0) == 0
    finally:
        L.dspark_markov_plan(prev)


def test_binding_constants_match_header():
    """The binding's limits, dtype and operation codes are the header's."""
    text = open(HEADER).read()
    defines = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(DSPARK_MAX_\w+)\s+(\d+)", text)}
    assert defines["DSPARK_MAX_GAMMA"] == ds.DSPARK_MAX_GAMMA
    assert defines["DSPARK_MAX_RANK"] == ds.DSPARK_MAX_RANK
    assert defines["DSPARK_MAX_VERIFY_BATCH"] == ds.DSPARK_MAX_VERIFY_BATCH
    enums = dict(re.findall(r"\b(DSPARK_(?:BF16|F32|OP_\w+))\s*=\s*(\d+)", text))
    for name, value in enums.items():
        assert getattr(ds, name) == int(value), name
