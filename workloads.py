"""Seeded synthetic inputs for the DSpark sampling / verification engine.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, and both the GPU library's tests/benchmark and the CPU
oracle read the same bytes from it.

Every array of request (or block) b is drawn from its own stream keyed by
(config seed, array id, b), so any subset of requests can be regenerated
exactly without drawing the rest.  bf16 arrays are returned as uint16 holding
the round-to-nearest-even upper half of the float32 value.

The shapes follow the pages' decode tiles and training blocks: gamma 5 with a
six-row verify span and gamma 7 with an eight-row tile ("[2/3] feat(dsv4):
implement exact DSpark speculative decoding", "End-to-end speculative cycle";
"DeepSeek V4 DSpark NPU Serving Dev Notes", "Speculative decoding (K=7)"),
up to 256 requests, and training blocks of gamma = 7 ("DSpark Speculative
Decoding (Draft Training) Design", "Semi-autoregressive draft").  They stand
in for the pages' end-to-end workloads, whose prompts and checkpoints are not
available.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "to_bf16",
    "bf16_to_f32",
    "DECODE_CONFIGS",
    "STATS_CONFIG",
    "decode_inputs",
    "stats_inputs",
    "width_inputs",
    "stats_markov_inputs",
]


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# Decode-side configurations (Markov sample + verify).
DECODE_CONFIGS = {
    # Tiny: fp32 logits, draft N(0,2^2), target = draft + N(0,0.5^2), rank 16,
    # d = 64, T = 1, no truncation; run greedy and sampled.
    "tiny": dict(seed=1001, B=4, gamma=5, V=1024, r=16, d=64, dtype="f32",
                 draft_std=2.0, noise_std=0.5, w_std=0.02, mode="sampled"),
    # Decode verify (the headline): bf16, draft N(0,3^2), target = draft +
    # N(0,1), rank 256, d = 4096, T = 1, no truncation, sampled.
    "decode": dict(seed=1002, B=64, gamma=5, V=129280, r=256, d=4096,
                   dtype="bf16", draft_std=3.0, noise_std=1.0, w_std=0.02,
                   mode="sampled"),
    # Truncated sampling at max batch: as "decode" with B = 256, Zipf(1.1)
    # shaped target offsets, per-request T ~ U[0.3,1.2], top-k in
    # {0,20,50}, top-p in {1,0.9,0.8}, even requests sampled, odd greedy.
    "truncated": dict(seed=1003, B=256, gamma=5, V=129280, r=256, d=4096,
                      dtype="bf16", draft_std=3.0, noise_std=1.0, w_std=0.02,
                      mode="mixed", zipf=1.1, policy="random"),
    # Wide greedy tile: 64 requests x 8 rows (anchor + 7), target = draft +
    # N(0,1.5^2), greedy.
    "wide_greedy": dict(seed=1004, B=64, gamma=7, V=129280, r=256, d=4096,
                        dtype="bf16", draft_std=3.0, noise_std=1.5,
                        w_std=0.02, mode="greedy"),
}

# Training acceptance statistics: 2048 blocks x gamma 7, bf16, target =
# draft + N(0,1), confidence logits N(0,1).
STATS_CONFIG = dict(seed=1005, N=2048, gamma=7, V=129280, dtype="bf16",
                    draft_std=3.0, noise_std=1.0)


def _policy(cfg: dict, b: int):
    """(mode, temperature, top_k, top_p) of request b."""
    mode = cfg.get("mode", "sampled")
    m = {"sampled": 1, "greedy": 0}.get(mode, 1 - (b & 1))
    if cfg.get("policy") == "random":
        g = _rng(cfg["seed"], 5, b)
        T = float(g.uniform(0.3, 1.2))
        top_k = int(g.choice([0, 20, 50]))
        top_p = float(g.choice([1.0, 0.9, 0.8]))
        return m, T, top_k, top_p
    return m, float(cfg.get("temperature", 1.0)), int(cfg.get("top_k", 0)), float(cfg.get("top_p", 1.0))


def decode_inputs(name_or_cfg="tiny", requests=None, with_embed=True, **overrides) -> dict:
    """Inputs of one decode step: Markov sample and verify.

    `requests` selects a subset of request indices (default all); the data of
    request b does not depend on which others are drawn.  Keys:
      backbone [n,gamma,V], target [n,gamma+1,V] (uint16 bf16 or float32),
      anchor [n] int32, w1 / w2 [V,r] bf16, hidden [n,gamma,d] bf16,
      embed [V,d] bf16, conf_w [2d] float32, mode uint8, temperature float32,
      top_k int32, top_p float32, request_id uint32, position int32 (all [n]),
      seed, and the sizes B (= n), gamma, V, r, d, dtype.
    The backbone row k-1 and the target row k-1 share one draft draw; target
    row gamma (the bonus row) uses draft row gamma of the same draw.
    """
    cfg = dict(DECODE_CONFIGS[name_or_cfg]) if isinstance(name_or_cfg, str) else dict(name_or_cfg)
    cfg.update(overrides)
    s, gamma, V, r, d = cfg["seed"], cfg["gamma"], cfg["V"], cfg["r"], cfg["d"]
    reqs = list(range(cfg["B"])) if requests is None else [int(b) for b in requests]
    n = len(reqs)
    bf = cfg["dtype"] == "bf16"
    edt = np.uint16 if bf else np.float32
    backbone = np.empty((n, gamma, V), edt)
    target = np.empty((n, gamma + 1, V), edt)
    hidden = np.empty((n, gamma, d), np.uint16)
    anchor = np.empty(n, np.int32)
    mode = np.empty(n, np.uint8)
    temperature = np.empty(n, np.float32)
    top_k = np.empty(n, np.int32)
    top_p = np.empty(n, np.float32)
    def one(i):
        b = reqs[i]
        draft = _rng(s, 1, b).standard_normal((gamma + 1, V), dtype=np.float32) * np.float32(cfg["draft_std"])
        tgt = draft + _rng(s, 2, b).standard_normal((gamma + 1, V), dtype=np.float32) * np.float32(cfg["noise_std"])
        if cfg.get("zipf"):
            perm = _rng(s, 6, b).permutation(V).astype(np.float32)
            tgt += (-np.float32(cfg["zipf"]) * np.log1p(perm)).astype(np.float32)[None, :]
        if bf:
            backbone[i] = to_bf16(draft[:gamma])
            target[i] = to_bf16(tgt)
        else:
            backbone[i] = draft[:gamma]
            target[i] = tgt
        hidden[i] = to_bf16(_rng(s, 3, b).standard_normal((gamma, d), dtype=np.float32))
        anchor[i] = _rng(s, 4, b).integers(0, V)
        mode[i], temperature[i], top_k[i], top_p[i] = _policy(cfg, b)

    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        list(ex.map(one, range(n)))
    out = dict(
        backbone=backbone, target=target, anchor=anchor, hidden=hidden,
        w1=to_bf16(_rng(s, 10).standard_normal((V, r), dtype=np.float32) * np.float32(cfg["w_std"])),
        w2=to_bf16(_rng(s, 11).standard_normal((V, r), dtype=np.float32) * np.float32(cfg["w_std"])),
        conf_w=(_rng(s, 13).standard_normal(2 * d, dtype=np.float32) * np.float32(0.02)),
        mode=mode, temperature=temperature, top_k=top_k, top_p=top_p,
        request_id=np.asarray(reqs, np.uint32),
        position=(100 + 16 * np.asarray(reqs, np.int64)).astype(np.int32),
        seed=int(cfg.get("philox_seed", 0)),
        B=n, gamma=gamma, V=V, r=r, d=d, dtype=cfg["dtype"],
    )
    if with_embed:
        out["embed"] = embed_table(cfg)
    return out


def embed_table(cfg) -> np.ndarray:
    """Shared token embedding [V, d] bf16 of a decode config.

    Rows are drawn in blocks of 1024, block j from its own stream (config seed,
    12, j), so the table is the same whatever the number of worker threads."""
    cfg = dict(DECODE_CONFIGS[cfg]) if isinstance(cfg, str) else cfg
    V, d = cfg["V"], cfg["d"]
    out = np.empty((V, d), np.uint16)
    rows = 1024

    def fill(j):
        lo, hi = j * rows, min(V, (j + 1) * rows)
        out[lo:hi] = to_bf16(_rng(cfg["seed"], 12, j).standard_normal((hi - lo, d), dtype=np.float32))

    nblk = (V + rows - 1) // rows
    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        list(ex.map(fill, range(nblk)))
    return out


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def stats_inputs(cfg=None, blocks=None, mask_every=0, **overrides) -> dict:
    """Inputs of the training-side acceptance statistics.

    Keys: draft, target [n,gamma,V] (bf16 or float32), teacher [n,gamma] int32
    (the target row's argmax: a stand-in for the teacher-forced next tokens),
    conf_logits [n,gamma] float32 N(0,1), block_mask [n] uint8 (every
    `mask_every`-th block zero if mask_every > 0), N, gamma, V, dtype.
    """
    cfg = dict(STATS_CONFIG if cfg is None else cfg)
    cfg.update(overrides)
    s, gamma, V = cfg["seed"], cfg["gamma"], cfg["V"]
    blks = list(range(cfg["N"])) if blocks is None else [int(b) for b in blocks]
    n = len(blks)
    bf = cfg["dtype"] == "bf16"
    edt = np.uint16 if bf else np.float32
    draft = np.empty((n, gamma, V), edt)
    target = np.empty((n, gamma, V), edt)
    teacher = np.empty((n, gamma), np.int32)
    conf = np.empty((n, gamma), np.float32)
    def one(i):
        b = blks[i]
        dr = _rng(s, 1, b).standard_normal((gamma, V), dtype=np.float32) * np.float32(cfg["draft_std"])
        tg = dr + _rng(s, 2, b).standard_normal((gamma, V), dtype=np.float32) * np.float32(cfg["noise_std"])
        if bf:
            draft[i] = to_bf16(dr)
            target[i] = to_bf16(tg)
            teacher[i] = np.argmax(bf16_to_f32(target[i]), axis=1)
        else:
            draft[i] = dr
            target[i] = tg
            teacher[i] = np.argmax(tg, axis=1)
        conf[i] = _rng(s, 4, b).standard_normal(gamma, dtype=np.float32)

    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        list(ex.map(one, range(n)))
    mask = np.ones(n, np.uint8)
    if mask_every > 0:
        mask[np.asarray(blks) % mask_every == mask_every - 1] = 0
    return dict(draft=draft, target=target, teacher=teacher, conf_logits=conf,
                block_mask=mask, N=n, gamma=gamma, V=V, dtype=cfg["dtype"])


# Draft-width selection: per-proposal acceptance predictions and a cost table
# {D, V(0), ..., V(gamma)} in arbitrary time units.  Confidences of request b
# decay along the block (c_j = s_b * u_j^(j / gamma), s_b ~ U[0.3, 1], u_j ~
# U[0.5, 1]) so that the chosen widths spread over 0..gamma; the costs model a
# fixed draft pass and a verify pass that grows with the rows it checks.
WIDTH_CONFIG = dict(seed=1006, B=64, gamma=5, draft_cost=1.0, verify_base=3.0,
                    verify_per_row=0.45)


def width_inputs(B=None, gamma=None, cfg=None, **overrides) -> dict:
    cfg = dict(WIDTH_CONFIG if cfg is None else cfg)
    cfg.update(overrides)
    if B is not None:
        cfg["B"] = B
    if gamma is not None:
        cfg["gamma"] = gamma
    B, g = cfg["B"], cfg["gamma"]
    conf = np.empty((B, g), np.float32)
    for b in range(B):
        r = _rng(cfg["seed"], 1, b)
        s_b = r.uniform(0.3, 1.0)
        u = r.uniform(0.5, 1.0, g)
        conf[b] = s_b * u ** (np.arange(1, g + 1) / g)
    cost = np.empty(g + 2, np.float32)
    cost[0] = cfg["draft_cost"]
    cost[1:] = cfg["verify_base"] + cfg["verify_per_row"] * (np.arange(g + 1) + 1)
    return dict(B=B, gamma=g, confidence=conf, cost=cost)


def stats_markov_inputs(cfg=None, blocks=None, r=256, w_std=0.02, mask_every=0, **overrides) -> dict:
    """Inputs of the statistics of the teacher-forced Markov draft: the
    statistics' rows, with the draft rows renamed `backbone` (the parallel
    logits the Markov bias is added to), plus per block an anchor token and
    the rank-r factors W1, W2 [V, r] (bf16, N(0, w_std^2)), drawn from
    streams keyed like the rest."""
    cfg = dict(STATS_CONFIG if cfg is None else cfg)
    cfg.update(overrides)
    inp = stats_inputs(cfg, blocks=blocks, mask_every=mask_every)
    s, V = cfg["seed"], cfg["V"]
    blks = list(range(cfg["N"])) if blocks is None else [int(b) for b in blocks]
    inp["backbone"] = inp.pop("draft")
    inp["anchor"] = np.array([_rng(s, 6, b).integers(0, V) for b in blks], np.int32)
    inp["w1"] = to_bf16(_rng(s, 7).standard_normal((V, r), dtype=np.float32) * np.float32(w_std))
    inp["w2"] = to_bf16(_rng(s, 8).standard_normal((V, r), dtype=np.float32) * np.float32(w_std))
    inp["r"] = r
    return inp

