"""Share of the oracle's draws flagged NEAR_THRESHOLD at the decode shape.

A measurement, not a test (pytest does not collect it): the decode
configuration's vocabulary and logits (V = 129280, bf16, draft ~ N(0, 3^2),
target = draft + N(0, 1), temperature 1, sampled, no truncation) with the
Markov rank reduced to 16 and the confidence width to 64 (the flags do not
involve the confidence head, and the bias only shifts the draft logits by
about 1e-3), run through the oracle's Markov sampler and verify.  Draws are
counted as in the GPU flag-rate test: every Markov draw (B gamma) plus every
verify accept test and final draw (sum of accept_len + 1); a draw is flagged
when its row carries the NEAR bit (a decision within 1e-6 of its threshold,
DSPARK_FLAG_NEAR_THRESHOLD).  Requests run in chunks over a thread pool (the
oracle's calls release the GIL).

    python3 tests/measure_near_share.py --requests 12800 --threads 8
"""

from __future__ import annotations

import argparse
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import oracle as O  # noqa: E402
from workloads import decode_inputs  # noqa: E402


def chunk(reqs):
    inp = decode_inputs("decode", requests=reqs, r=16, d=64)
    mk = O.markov_sample(inp)
    q = dict(q_z=mk["q_z"].astype(np.float32), q_lse=mk["q_lse"].astype(np.float32),
             q_thr=mk["q_thr"].astype(np.float32), q_tok=mk["q_tok"].astype(np.float32))
    vf = O.verify(inp, mk["draft_tokens"], **q)
    g = inp["gamma"]
    draws = len(reqs) * g + int((vf["accept_len"] + 1).sum())
    near_m = int(((mk["flags"] & O.F_NEAR) != 0).sum())
    near_v = int(((vf["flags"] & O.F_NEAR) != 0).sum())
    return draws, near_m, near_v


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--requests", type=int, default=12800)
    ap.add_argument("--chunk", type=int, default=64)
    ap.add_argument("--threads", type=int, default=max(1, min(8, os.cpu_count() or 1)))
    a = ap.parse_args()
    O.lib()
    parts = [list(range(i, min(i + a.chunk, a.requests))) for i in range(0, a.requests, a.chunk)]
    t = time.time()
    with ThreadPoolExecutor(max_workers=a.threads) as ex:
        res = list(ex.map(chunk, parts))
    draws = sum(r[0] for r in res)
    nm, nv = sum(r[1] for r in res), sum(r[2] for r in res)
    print(f"requests {a.requests}  draws {draws}  flagged {nm + nv} (Markov {nm}, verify {nv})  "
          f"share {(nm + nv) / draws:.3e}  ({time.time() - t:.0f} s, {a.threads} threads)")


if __name__ == "__main__":
    main()
