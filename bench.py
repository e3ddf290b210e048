"""Benchmark of the DSpark sampling / verification hot path on one MI355X.

One step is one pass of the whole path over one batch of the decode-verify
workload (B = 64 requests, gamma = 5, V = 129280, bf16 logits, Markov rank 256,
confidence width 4096, sampled at temperature 1 without truncation):
  dspark_markov_sample  (gamma Markov steps: bias GEMM + sampling + confidence;
                        one launch for all steps by default, --markov-plan)
  dspark_verify         (the oracle-free exact sampled verify of those proposals)
  dspark_accept_stats   (analytic acceptance of the same draft / target rows)
Inputs are synthetic (workloads.py) and resident in HBM before timing starts;
successive steps cycle through --rotate independent copies of the batch and
weights (about 1.5 GB each), so no step is served from the Infinity Cache by
an earlier step's reads.

Prints one JSON line: value = verified rows per second, B (gamma + 1) rows per
step; the roofline entry is the dominant kernel's algorithmic HBM bytes per
launch over its average launch time, measured here with HIP events around each
launch (the library's opt-in profiler, on the launch stream; for the
cooperative Markov launch the event pair also brackets its dispatch), and its
counter-measured traffic from the committed rocprofv3 summary while the kernel
sources match it; cpu_baseline is the oracle, single-threaded, on a bounded
sample of the same batch.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified rows/sec (B×(γ+1)×V logits) at V=129280,B=64,γ=5; % HBM roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=4,
                    help="independent copies of the batch (logits and weights) cycled step by "
                         "step, so that no step finds its inputs in the 256 MB Infinity Cache")
    ap.add_argument("--cpu-requests", type=int, default=64,
                    help="requests of the batch the oracle baseline runs on")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--workload", choices=["decode", "truncated", "wide_greedy", "adaptive", "stats",
                                           "train", "markov_stats"],
                    default="decode",
                    help="decode (default: the benchmark line); the other configurations "
                         "are measured the same way for reference")
    ap.add_argument("--markov-plan", choices=["auto", "per-step", "cooperative", "request-groups"], default="auto",
                    help="Markov launch plan: one launch for all steps when its grid fits "
                         "(auto), the same through cooperative launch, or two launches per step")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step (profiling runs)")
    ap.add_argument("--concurrent-stats", action="store_true",
                    help="run the accept stats on a second stream, after the Markov call and beside "
                         "the verify (they read neither's outputs)")
    ap.add_argument("--truncation-arrays", action="store_true",
                    help="pass the top-k / top-p arrays even when no request truncates (the "
                         "library then takes its truncating kernels)")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="instead of the benchmark, write the rocprofv3 summary of the "
                         "profiling run under DIR to profiles/")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run a plain device copy of MIB MiB "
                         "(the reference kernel for scaling HBM byte counters)")
    return ap.parse_args()


def copy_calibration(mib):
    """A plain device-to-device copy of known size, for counter calibration."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps(dict(copy_bytes_read=n * 4, copy_bytes_written=n * 4, launches=3)), flush=True)


def kernel_bytes(name, B, g, V, r, d, S, R):
    """Algorithmic (compulsory) HBM bytes of one launch of each kernel."""
    C = (V + 255) // 256
    if name in ("markov_fused", "markov_fast", "markov_pipe"):  # one launch for all gamma steps: backbone, q, W2 once, A rows
        return 2 * B * g * V + 4 * S * g * V + 2 * r * V + 2 * B * g * r
    if name == "markov_step":      # backbone row + q row written + W2 (once per call) + A rows
        return 2 * B * V + 4 * S * V + (2 * r * V) / g + 2 * B * r
    if name == "markov_confidence":  # h row + embedding row per draft row, w once
        return 4 * B * g * d + 8 * d
    if name == "markov_finalize":  # chunk partials + chosen-chunk z
        return 16 * B * C + 4 * 256 * S
    if name == "verify_rows":      # every target row once
        return 2 * B * (g + 1) * V
    if name == "verify_decide":    # the proposal row of each rejecting request
        return 4 * V * R
    if name == "verify_select":    # second look at truncated rows (cached): not compulsory
        return 0
    if name in ("stats_rows", "stats_part1"):  # draft + target row pairs, first look
        return 2 * 2 * B * g * V
    if name == "stats_part2":      # second look at the same rows: not compulsory
        return 0
    if name in ("stats_pairs", "stats_reduce"):
        return 16 * B * g
    if name == "stats_markov_look1":  # backbone and target rows, W2 once per token slice
        return 2 * 2 * B * g * V + 2 * r * V
    if name == "stats_markov_look2":  # second look: not compulsory
        return 0
    if name == "stats_grad_rows":  # row pair read once, gradient row written once (bf16)
        return 3 * 2 * B * g * V
    if name == "stats_grad_write":  # the gradient row written (its reads are the third look)
        return 2 * B * g * V
    if name == "stats_grad_part2":  # second look: not compulsory
        return 0
    if name == "select_width":     # confidences in, widths and expectations out
        return 4 * B * g + 4 * (g + 2) + 8 * B
    return 0


PROFILE = os.path.join(ROOT, "profiles", "decode_step_B64_g5_V129280.md")
# profile summaries per workload: (file, title, bench arguments of the run)
PROFILES = {
    "decode": (PROFILE, "Decode step (Markov sample + verify + accept stats), B=64, gamma=5, "
                        "V=129280, bf16, sampled", ""),
    "train": (os.path.join(ROOT, "profiles", "stats_train_N2048_g7_V129280.md"),
              "Training statistics and their gradient (dspark_accept_stats + "
              "dspark_accept_stats_backward), 2048 blocks x gamma 7, V=129280, bf16",
              " --workload train"),
    "markov_stats": (os.path.join(ROOT, "profiles", "stats_markov_N2048_g7_V129280_r256.md"),
                     "Statistics of the teacher-forced Markov draft (dspark_accept_stats_markov), "
                     "2048 blocks x gamma 7, V=129280, rank 256, bf16",
                     " --workload markov_stats"),
    "truncated": (os.path.join(ROOT, "profiles", "truncated_step_B256_g5_V129280.md"),
                  "Truncated decode step (Markov sample + verify + accept stats), B=256, gamma=5, "
                  "V=129280, bf16, per-request temperature, top-k, top-p, mixed greedy/sampled",
                  " --workload truncated"),
    "wide_greedy": (os.path.join(ROOT, "profiles", "wide_greedy_step_B64_g7_V129280.md"),
                    "Wide greedy decode step (Markov sample + verify + accept stats), 64 requests x "
                    "8 target rows (gamma=7), V=129280, bf16, greedy",
                    " --workload wide_greedy"),
}
# the SQ counter passes of a profile (each within one pass's limits: at most
# 8 SQ and 2 GRBM counters)
SQ_PASSES = (("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"),
             ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_WAVE_CYCLES"))
DEVICE_CUS = 256
DEVICE_XCDS = 8  # GRBM_GUI_ACTIVE is summed over the XCDs
CSRC = os.path.join(ROOT, "dspark_draft_sampling_amd", "csrc")


# the sources a workload's kernels are built from (the digest of a profile
# summary covers these; None: every kernel source)
DIGEST_SOURCES = {
    "decode": ("common.hpp", "internal.hpp", "l1norm.hpp", "markov.hip", "stats.hip", "truncate.hpp",
               "verify.hip"),
    "train": ("common.hpp", "internal.hpp", "l1norm.hpp", "stats.hip"),
    "markov_stats": ("common.hpp", "internal.hpp", "l1norm.hpp", "stats.hip", "stats_markov.hip"),
    "truncated": ("common.hpp", "internal.hpp", "l1norm.hpp", "markov.hip", "stats.hip", "truncate.hpp",
                  "verify.hip"),
    "wide_greedy": ("common.hpp", "internal.hpp", "l1norm.hpp", "markov.hip", "stats.hip", "truncate.hpp",
                    "verify.hip"),
}


def source_digest(workload="decode"):
    """sha256 over the kernel sources of `workload` (file names and
    contents, sorted)."""
    import hashlib

    want = DIGEST_SOURCES.get(workload)
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".hpp", ".h")) and (want is None or f in want):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def counter_traffic(kernel, workload="decode"):
    """L2-miss bytes (FETCH_SIZE + WRITE_SIZE, copy-calibrated: reads served by
    the Infinity Cache are counted too) per launch of `kernel` from the
    workload's committed counter summary, or None when that summary was taken
    on other kernel sources."""
    if workload not in PROFILES:
        return None
    try:
        text = open(PROFILES[workload][0]).read()
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(blob)
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest(workload):
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None
    return int(k["read_bytes"] + k["write_bytes"])


def summarize_profile(base, workload="decode"):
    """Write the rocprofv3 summary (kernel trace + copy-calibrated HBM
    counters) of a profiling run of `workload` whose outputs are under
    `base`."""
    import collections
    import csv

    def agg(path):
        d = collections.defaultdict(list)
        with open(path) as fh:
            for row in csv.DictReader(fh):
                d[row["Kernel_Name"]].append(float(row["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in d.items()}

    out, title, wl = PROFILES[workload]
    ours = ("markov", "verify", "stats", "select_width")
    with open(f"{base}/prof_kt/kt_kernel_stats.csv") as fh:
        stats = [r for r in csv.DictReader(fh) if r["Name"].startswith(ours)]
    fetch = agg(f"{base}/prof_FETCH_SIZE/p_counter_collection.csv")
    write = agg(f"{base}/prof_WRITE_SIZE/p_counter_collection.csv")
    copy = "__amd_rocclr_copyBuffer"
    cf = agg(f"{base}/prof_copy_FETCH_SIZE/p_counter_collection.csv")[copy]
    cw = agg(f"{base}/prof_copy_WRITE_SIZE/p_counter_collection.csv")[copy]
    true_kib = 256 * 1024
    sf, sw = true_kib / cf, true_kib / cw
    cmd = "python3 bench.py" + wl
    decode_like = workload in ("decode", "truncated", "wide_greedy")
    steps = " --steps 50 --warmup 5" if decode_like else " --steps 10 --warmup 2"
    ng = " --no-graph" if decode_like else ""
    lines = [
        f"# {title}",
        "",
        "Commands, from the repository root after `cd /tmp && export TMPDIR=/tmp` (paths "
        f"absolute on the run; $OUT is the output directory; `python3 bench.py{wl} --summarize-profile $OUT` "
        "wrote this file):",
        "",
        "```",
        f"rocprofv3 --kernel-trace --stats -T -f csv -d $OUT/prof_kt -o kt -- {cmd}{steps} --no-cpu{ng}",
        f"rocprofv3 --pmc FETCH_SIZE -T -f csv -d $OUT/prof_FETCH_SIZE -o p -- {cmd} --steps 2 --warmup 1 --no-cpu{ng}",
        f"rocprofv3 --pmc WRITE_SIZE -T -f csv -d $OUT/prof_WRITE_SIZE -o p -- {cmd} --steps 2 --warmup 1 --no-cpu{ng}",
        f"rocprofv3 --pmc FETCH_SIZE -T -f csv -d $OUT/prof_copy_FETCH_SIZE -o p -- {cmd} --copy-calibration 256",
        f"rocprofv3 --pmc WRITE_SIZE -T -f csv -d $OUT/prof_copy_WRITE_SIZE -o p -- {cmd} --copy-calibration 256",
        *[f"rocprofv3 --pmc {' '.join(ps)} -T -f csv -d $OUT/prof_SQ{i} -o p -- {cmd} --steps 2 --warmup 1 --no-cpu{ng}"
          for i, ps in enumerate(SQ_PASSES)],
        "```",
        "",
        "## Kernel time (`--kernel-trace --stats`)",
        "",
        "| kernel | calls | average µs | min µs | max µs | share % |",
        "|---|---|---|---|---|---|",
    ]
    for r in stats:
        lines.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    lines += [
        "",
        "## HBM bytes per dispatch (`--pmc FETCH_SIZE`, `--pmc WRITE_SIZE`)",
        "",
        f"Calibration: a 256 MiB device copy (`{copy}`) reads {cf:.0f} KiB of FETCH_SIZE and "
        f"{cw:.0f} KiB of WRITE_SIZE per dispatch against {true_kib} KiB moved each way, so "
        f"FETCH_SIZE is scaled by {sf:.3f} and WRITE_SIZE by {sw:.3f}.",
        "",
        "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |",
        "|---|---|---|---|---|",
    ]
    rec = dict(source_sha256=source_digest(workload), sources=list(DIGEST_SOURCES.get(workload) or []),
               fetch_scale=sf, write_scale=sw, kernels={})
    for k in sorted(fetch):
        if not k.startswith(ours):
            continue
        rd, wr = fetch[k] * sf * 1024, write.get(k, 0.0) * sw * 1024
        name = k.replace("_kernel", "")
        avg = next((float(r["AverageNs"]) / 1e3 for r in stats if r["Name"] == k), None)
        rec["kernels"][name] = dict(read_bytes=round(rd), write_bytes=round(wr), avg_us=avg)
        lines.append(f"| {k} | {fetch[k]:.0f} | {write.get(k, 0):.0f} | {rd / 1e6:.1f} | {wr / 1e6:.1f} |")
    lines += sq_section(base, ours, stats)
    lines += ["", "Machine-readable copy (bench.py fills `roofline.traffic` from it while the "
              "kernel sources still hash to `source_sha256`):", "", "```json",
              json.dumps(rec, indent=1), "```"]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def sq_section(base, ours, stats):
    """MFMA and VALU activity per kernel from the SQ counter passes (if run):
    per-dispatch averages and the usual ratios, with c = GRBM_GUI_ACTIVE /
    XCDs the kernel's active cycles (the counter is summed over the XCDs),
      MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (c x CUs x 4 SIMDs),
      VALU busy = SQ_ACTIVE_INST_VALU x 4 / (CUs x 4 SIMDs) / c,
      MFMA TFLOP/s = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / kernel time
    (the last cross-checks the first: one MFMA MOP is 512 flops)."""
    import collections
    import csv

    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for i in range(len(SQ_PASSES)):
        path = f"{base}/prof_SQ{i}/p_counter_collection.csv"
        if not os.path.exists(path):
            return []
        with open(path) as fh:
            for row in csv.DictReader(fh):
                vals[row["Kernel_Name"]][row["Counter_Name"]].append(float(row["Counter_Value"]))
    out = ["", "## MFMA and VALU activity per dispatch (`--pmc`, two SQ passes)", "",
           f"With c = GRBM_GUI_ACTIVE / {DEVICE_XCDS} (the counter is summed over the {DEVICE_XCDS} XCDs): "
           f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (c x {DEVICE_CUS} CUs x 4 SIMDs); "
           f"VALU busy = SQ_ACTIVE_INST_VALU x 4 / ({DEVICE_CUS} x 4) / c; MFMA TFLOP/s = "
           "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / the kernel's average time (kernel trace above), which "
           "cross-checks MFMA busy against the 2.5 PFLOP/s dense bf16 peak.", "",
           "| kernel | GRBM_GUI_ACTIVE | MFMA busy % | VALU busy % | VALU insts | MFMA insts | MFMA TFLOP/s |",
           "|---|---|---|---|---|---|---|"]
    for k in sorted(vals):
        if not k.startswith(ours):
            continue
        a = {c: sum(v) / len(v) for c, v in vals[k].items()}
        gui = a.get("GRBM_GUI_ACTIVE", 0.0)
        cyc = gui / DEVICE_XCDS
        mb = 100.0 * a.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * DEVICE_CUS * 4) if gui else 0.0
        vb = 100.0 * a.get("SQ_ACTIVE_INST_VALU", 0.0) * 4 / (DEVICE_CUS * 4) / cyc if gui else 0.0
        avg = next((float(r["AverageNs"]) for r in stats if r["Name"] == k), None)
        tf = a.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512 / (avg * 1e-9) / 1e12 if avg else 0.0
        out.append(f"| {k} | {gui:.0f} | {mb:.2f} | {vb:.1f} | {a.get('SQ_INSTS_VALU', 0):.3g} | "
                   f"{a.get('SQ_INSTS_MFMA', 0):.3g} | {tf:.1f} |")
    return out


def _timed(step, args, torch):
    """W untimed steps, then K timed steps bracketed by synchronisation;
    returns (ms_total, wall_s)."""
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1), time.perf_counter() - t_wall


def _step_percentiles(step, args, torch):
    """p10 / p50 / p90 of single-step durations (HIP events around each step,
    a separate pass after the timed one)."""
    n = max(20, min(args.steps, 200))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    evs[0].record()
    for i in range(n):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    us = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n)])
    return dict(steps=n, p10_us=round(float(np.percentile(us, 10)), 2),
                p50_us=round(float(np.percentile(us, 50)), 2), p90_us=round(float(np.percentile(us, 90)), 2))


def _graph_step(step, nsteps, args, torch, ds):
    """The step captured in a HIP graph (nsteps eager steps, one per rotated
    input set, recorded once) and replayed: microseconds per step, next to the
    same steps run eagerly on the same stream.  A captured Markov call runs
    the plan an eager one would (the cooperative plan as an ordinary launch),
    its one-launch kernel taking its hand-off tag from its workspace."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2 * nsteps):  # the stream's workspaces exist before the capture
            step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(nsteps):
            step()
    torch.cuda.synchronize()
    reps = max(10, min(args.steps, 50))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        g.replay()
        ev0.record()
        for _ in range(reps):
            g.replay()
        ev1.record()
    torch.cuda.synchronize()
    graph_us = ev0.elapsed_time(ev1) * 1e3 / (reps * nsteps)
    with torch.cuda.stream(s):
        step()
        ev0.record()
        for _ in range(reps * nsteps):
            step()
        ev1.record()
    torch.cuda.synchronize()
    eager_us = ev0.elapsed_time(ev1) * 1e3 / (reps * nsteps)
    del g
    plan = "cooperative as an ordinary launch" if args.markov_plan == "cooperative" else args.markov_plan
    if args.markov_plan != "per-step":
        plan += " (one-launch kernel: hand-off tag from its workspace)"
    return dict(step_us=round(graph_us, 2), eager_same_plan_step_us=round(eager_us, 2), markov_plan=plan)


def _kernels(step, args, torch, ds, bytes_of):
    """Per-kernel launch durations over a second pass in the same launch
    configuration (HIP events on the launch stream)."""
    prof_steps = max(10, min(args.steps, 50))
    ds.profile_enable(True)
    for _ in range(prof_steps):
        step()
    torch.cuda.synchronize()
    prof = ds.profile_summary()
    ds.profile_enable(False)
    kernels = {}
    for name, (n, ms) in prof.items():
        avg_us = ms / n * 1e3
        nbytes = bytes_of(name)
        kernels[name] = dict(launches_per_step=n / prof_steps, avg_us=round(avg_us, 3),
                             alg_bytes=int(nbytes), gbs=round(nbytes / (avg_us * 1e-6) / 1e9, 1))
    return kernels


def _roofline(kernels, workload):
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches_per_step"])
    ach = kernels[dom]["gbs"]
    return dict(bound="hbm", kernel=dom, achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(ach / HBM_PEAK_GBS, 4),
                traffic=counter_traffic(dom, workload) if workload else None)


def _roofline_mfma(kernels):
    """The dominant kernel against the dense bf16 MFMA peak when it carries a
    contraction (the teacher-forced looks), else against HBM."""
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches_per_step"])
    if "mfma_tflops" not in kernels[dom]:
        return _roofline(kernels, None)
    ach = kernels[dom]["mfma_tflops"]
    return dict(bound="mfma", kernel=dom, achieved=ach, peak=MFMA_BF16_TFLOPS, unit="TFLOP/s",
                frac=round(ach / MFMA_BF16_TFLOPS, 4), traffic=None)


def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.workload if args.workload in PROFILES else "decode")
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(one GPU's share of a sharded batch is the same kernels at a smaller shape)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import dspark_draft_sampling_amd as ds

    ds.markov_plan({"auto": ds.MARKOV_AUTO, "per-step": ds.MARKOV_PER_STEP,
                    "cooperative": ds.MARKOV_COOPERATIVE, "request-groups": ds.MARKOV_REQUEST_GROUPS}[args.markov_plan])
    if args.workload == "markov_stats":
        line = run_markov_stats(args, torch, ds)
    elif args.workload in ("stats", "train"):
        line = run_stats(args, torch, ds)
    else:
        line = run_decode(args, torch, ds)
    print(json.dumps(line), flush=True)


DECODE_WORKLOADS = {
    # name: (generator config, description)
    "decode": ("decode", "decode verify: Markov sample + sampled verify + accept stats"),
    "truncated": ("truncated", "truncated sampling at max batch: B=256, mixed greedy/sampled, "
                               "per-request T, top-k, top-p; Markov + verify + accept stats"),
    "wide_greedy": ("wide_greedy", "wide greedy tile: 64 requests x 8 rows, greedy Markov + verify "
                                   "+ accept stats"),
    "adaptive": ("decode", "decode verify with confidence-scheduled width: Markov + width choice + "
                           "verify of the chosen proposals + accept stats"),
}

# Draft-width cost table of the adaptive workload, in microseconds: a fixed
# draft pass and a verify pass that grows with the rows it checks (synthetic
# values of the order of this step's own kernels, not a live calibration).
ADAPTIVE_COST_US = dict(draft=140.0, verify_base=40.0, verify_per_row=12.0)


def run_decode(args, torch, ds):
    from workloads import decode_inputs

    cfg_name, desc = DECODE_WORKLOADS[args.workload]
    headline = args.workload == "decode"
    t0 = time.time()
    inp = decode_inputs(cfg_name)
    B, g, V, r, d = inp["B"], inp["gamma"], inp["V"], inp["r"], inp["d"]
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    # --rotate independent device copies of every per-step input and weight
    # (the same values; distinct memory), used round-robin by successive steps
    sets = []
    for _ in range(max(1, args.rotate)):
        backbone, target = bf(inp["backbone"]), bf(inp["target"])
        sets.append(dict(backbone=backbone, target=target, tgt_rows=target[:, :g].contiguous(),
                         w1=bf(inp["w1"]), w2=bf(inp["w2"]), hidden=bf(inp["hidden"]),
                         embed=bf(inp["embed"])))
    anchor = torch.from_numpy(inp["anchor"]).to(dev)
    conf_w = torch.from_numpy(inp["conf_w"]).to(dev)
    # truncation arrays only when some request truncates: the library then
    # skips every truncation pass (untruncated Markov kernel, no verify_select)
    trunc = args.truncation_arrays or bool(np.any((inp["top_k"] > 0) & (inp["top_k"] < V))
                                           or np.any(inp["top_p"] < 1))
    pol = ds.Policy(mode=torch.from_numpy(inp["mode"]).to(dev),
                    temperature=torch.from_numpy(inp["temperature"]).to(dev),
                    top_k=torch.from_numpy(inp["top_k"]).to(dev) if trunc else None,
                    top_p=torch.from_numpy(inp["top_p"]).to(dev) if trunc else None,
                    request_id=torch.from_numpy(inp["request_id"].view(np.int32)).to(dev),
                    position=torch.from_numpy(inp["position"]).to(dev))
    # the accept stats read the same rows: draft logits and the first gamma target rows
    rng = np.random.default_rng(1234)
    teacher = torch.from_numpy(rng.integers(0, V, (B, g)).astype(np.int32)).to(dev)
    conf_logits = torch.from_numpy(rng.standard_normal((B, g)).astype(np.float32)).to(dev)

    s0 = sets[0]
    mk_out = [ds.dspark_markov_sample(s0["backbone"], anchor, s0["w1"], s0["w2"], s0["hidden"],
                                      s0["embed"], conf_w, pol, seed=0) for _ in sets]
    vf_out = ds.dspark_verify(s0["target"], mk_out[0]["draft_tokens"], pol, mk_out[0]["q_logits"],
                              mk_out[0]["q_lse"], mk_out[0]["q_thr"], mk_out[0]["q_tok"], seed=0)
    st_out = ds.dspark_accept_stats(s0["backbone"], s0["tgt_rows"], teacher, conf_logits)
    adaptive = args.workload == "adaptive"
    if adaptive:
        c = ADAPTIVE_COST_US
        cost = torch.tensor([c["draft"]] + [c["verify_base"] + c["verify_per_row"] * (w + 1)
                                            for w in range(g + 1)], dtype=torch.float32, device=dev)
        wd_out = ds.dspark_select_width(mk_out[0]["confidence"], cost)
    it = [0]
    side = torch.cuda.Stream() if args.concurrent_stats else None
    if side is not None:
        with torch.cuda.stream(side):  # the side stream's workspace exists before timing
            ds.dspark_accept_stats(s0["backbone"], s0["tgt_rows"], teacher, conf_logits, out=st_out)
        torch.cuda.synchronize()

    def step():
        i = it[0] % len(sets)
        it[0] += 1
        x, mo = sets[i], mk_out[i]
        ds.dspark_markov_sample(x["backbone"], anchor, x["w1"], x["w2"], x["hidden"], x["embed"],
                                conf_w, pol, seed=0, out=mo)
        if side is not None:
            # after the Markov grid (which holds every compute unit), beside the verify
            main = torch.cuda.current_stream()
            side.wait_stream(main)
            with torch.cuda.stream(side):
                ds.dspark_accept_stats(x["backbone"], x["tgt_rows"], teacher, conf_logits, out=st_out)
        nd = None
        if adaptive:
            ds.dspark_select_width(mo["confidence"], cost, out=wd_out)
            nd = wd_out["n_draft"]
        ds.dspark_verify(x["target"], mo["draft_tokens"], pol, mo["q_logits"], mo["q_lse"],
                         mo["q_thr"], mo["q_tok"], n_draft=nd, seed=0, out=vf_out)
        if side is not None:
            main.wait_stream(side)
        else:
            ds.dspark_accept_stats(x["backbone"], x["tgt_rows"], teacher, conf_logits, out=st_out)

    ms_total, wall = _timed(step, args, torch)
    ms_per_step = ms_total / args.steps
    value = B * (g + 1) * args.steps / (ms_total / 1e3)
    print(f"# {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (events), wall {wall:.3f}s",
          file=sys.stderr, flush=True)

    S = int((inp["mode"] != 0).sum())
    R = int((vf_out["accept_len"] < g).sum().item())
    kernels = _kernels(step, args, torch, ds, lambda n: kernel_bytes(n, B, g, V, r, d, S, R))
    roofline = _roofline(kernels, args.workload)
    step_bytes = sum(k["alg_bytes"] * k["launches_per_step"] for k in kernels.values())
    pct = _step_percentiles(step, args, torch)
    graph = None if args.no_graph else _graph_step(step, len(sets), args, torch, ds)
    # decode-path rates from the per-kernel event times: verify alone, and
    # Markov + verify (the statistics are the training side of the path)
    t_of = lambda pre: sum(k["avg_us"] * k["launches_per_step"] for n, k in kernels.items()
                           if n.startswith(pre))
    t_verify, t_markov, t_stats = t_of("verify"), t_of("markov"), t_of("stats")
    acc = vf_out["accept_len"].double().cpu().numpy()
    reached = acc + (acc < g)  # proposals whose accept test ran

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(inp, min(args.cpu_requests, B) if headline else min(16, B), cfg_name)

    metric = METRIC if headline else f"verified rows/sec (B×(γ+1)×V logits) at {args.workload} (V={V},B={B},γ={g})"
    modes = "sampled" if S == B else ("greedy" if S == 0 else "mixed")
    truncation = "none" if not np.any((inp["top_k"] > 0) | (inp["top_p"] < 1.0)) else "top-k/top-p per request"
    return dict(metric=metric, value=round(value, 1), unit="rows/s", n_gpus=1, steps=args.steps,
                warmup=args.warmup, ms_per_step=round(ms_per_step, 5), higher_is_better=True,
                scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
                config=dict(workload=desc, B=B, gamma=g, V=V, r=r, d=d, logits="bf16",
                            temperature=1.0 if headline else "per request", truncation=truncation,
                            mode=modes, rotated_batches=len(sets), markov_plan=args.markov_plan,
                            schedule="stats on a second stream beside the verify" if side is not None
                            else "one stream"),
                roofline=roofline, cpu_baseline=cpu,
                verified_rows_s=round(B * (g + 1) / (t_verify * 1e-6), 1),
                step_rows_s=round(B * (g + 1) / ((t_markov + t_verify) * 1e-6), 1),
                step_us=dict(**pct, markov_us=round(t_markov, 2), verify_us=round(t_verify, 2),
                             stats_us=round(t_stats, 2), width_us=round(t_of("select_width"), 2)),
                hip_graph=graph,
                acceptance=dict(mean_accept_len=round(float(acc.mean()), 4),
                                accepted_per_proposal=round(float(acc.mean()) / g, 4),
                                per_position_accept_rate=round(float(acc.sum() / max(reached.sum(), 1)), 4),
                                tokens_per_step=round(float(acc.mean()) + 1.0, 4)),
                step=dict(alg_bytes=int(step_bytes),
                          alg_gbs=round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                          **(dict(mean_width=round(float(wd_out["n_draft"].float().mean().item()), 3),
                                  cost_us=ADAPTIVE_COST_US) if adaptive else {}),
                          kernels=kernels))


def run_stats(args, torch, ds):
    """Training-side acceptance statistics: 2048 blocks x gamma 7; with
    --workload train also their gradient (the forward and backward of the
    loss terms)."""
    from workloads import stats_inputs

    t0 = time.time()
    inp = stats_inputs()
    N, g, V = inp["N"], inp["gamma"], inp["V"]
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    sets = [dict(draft=bf(inp["draft"]), target=bf(inp["target"])) for _ in range(max(1, min(args.rotate, 2)))]
    teacher = torch.from_numpy(inp["teacher"]).to(dev)
    conf = torch.from_numpy(inp["conf_logits"]).to(dev)
    out = ds.dspark_accept_stats(sets[0]["draft"], sets[0]["target"], teacher, conf)
    train = args.workload == "train"
    if train:
        # the loss is the numerator over its token count: the upstream gradient
        scale = (1.0 / out["sums"][1:2]).contiguous()
        gout = ds.dspark_accept_stats_backward(sets[0]["draft"], sets[0]["target"], teacher, conf,
                                               grad_scale=scale)
    it = [0]

    def step():
        x = sets[it[0] % len(sets)]
        it[0] += 1
        ds.dspark_accept_stats(x["draft"], x["target"], teacher, conf, out=out)
        if train:
            ds.dspark_accept_stats_backward(x["draft"], x["target"], teacher, conf, grad_scale=scale,
                                            out=gout)

    ms_total, wall = _timed(step, args, torch)
    ms_per_step = ms_total / args.steps
    value = N * g * args.steps / (ms_total / 1e3)
    kernels = _kernels(step, args, torch, ds, lambda n: kernel_bytes(n, N, g, V, 0, 0, 0, 0))
    cpu = None
    if not args.no_cpu:
        from oracle import oracle as O

        nb = 4
        sub = stats_inputs(blocks=list(range(nb)))
        t = time.perf_counter()
        O.accept_stats(sub)
        sec = time.perf_counter() - t
        cpu = dict(value=round(nb * g / sec, 2), unit="rows/s", cores=1, kind="oracle",
                   sample=f"{nb} of the {N} blocks, {sec:.1f}s single-threaded")
    what = "stats forward + backward" if train else "stats"
    return dict(metric=f"{what} rows/sec (N×γ row pairs) at V={V},N={N},γ={g}", value=round(value, 1),
                unit="rows/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
                ms_per_step=round(ms_per_step, 5), higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="bf16", data="synthetic",
                config=dict(workload="training acceptance statistics" +
                            (" and their gradient" if train else ""), N=N, gamma=g, V=V,
                            logits="bf16", rotated_batches=len(sets)),
                roofline=_roofline(kernels, args.workload), cpu_baseline=cpu,
                step=dict(kernels=kernels))


def run_markov_stats(args, torch, ds):
    """Statistics of the teacher-forced Markov draft: 2048 blocks x gamma 7,
    V = 129280, rank 256 (the bias formed on MFMA inside both looks)."""
    from workloads import stats_markov_inputs

    t0 = time.time()
    inp = stats_markov_inputs()
    N, g, V, r = inp["N"], inp["gamma"], inp["V"], inp["r"]
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    sets = [dict(backbone=bf(inp["backbone"]), target=bf(inp["target"]))
            for _ in range(max(1, min(args.rotate, 2)))]
    anchor = torch.from_numpy(inp["anchor"]).to(dev)
    w1, w2 = bf(inp["w1"]), bf(inp["w2"])
    teacher = torch.from_numpy(inp["teacher"]).to(dev)
    conf = torch.from_numpy(inp["conf_logits"]).to(dev)
    out = ds.dspark_accept_stats_markov(sets[0]["backbone"], sets[0]["target"], anchor, w1, w2, teacher,
                                        conf)
    it = [0]

    def step():
        x = sets[it[0] % len(sets)]
        it[0] += 1
        ds.dspark_accept_stats_markov(x["backbone"], x["target"], anchor, w1, w2, teacher, conf, out=out)

    ms_total, wall = _timed(step, args, torch)
    ms_per_step = ms_total / args.steps
    value = N * g * args.steps / (ms_total / 1e3)
    kernels = _kernels(step, args, torch, ds, lambda n: kernel_bytes(n, N, g, V, r, 0, 0, 0))
    flops = 2.0 * N * g * V * r  # the bias of one look
    for name in ("stats_markov_look1", "stats_markov_look2"):
        if name in kernels:
            kernels[name]["mfma_tflops"] = round(flops / (kernels[name]["avg_us"] * 1e-6) / 1e12, 1)
    return dict(metric=f"teacher-forced Markov stats rows/sec (N×γ row pairs) at V={V},N={N},γ={g},r={r}",
                value=round(value, 1), unit="rows/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
                ms_per_step=round(ms_per_step, 5), higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="bf16", data="synthetic",
                config=dict(workload="acceptance statistics of the teacher-forced Markov draft", N=N,
                            gamma=g, V=V, r=r, logits="bf16", rotated_batches=len(sets)),
                roofline=_roofline_mfma(kernels), cpu_baseline=None,
                step=dict(kernels=kernels, bias_gflop_per_look=round(flops / 1e9, 1)))


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform's."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def _oracle_step(O, sub):
    """One pass of the whole path through the oracle on a request subset."""
    g = sub["gamma"]
    mk = O.markov_sample(sub)
    q = dict(q_z=mk["q_z"].astype(np.float32), q_lse=mk["q_lse"].astype(np.float32),
             q_thr=mk["q_thr"].astype(np.float32), q_tok=mk["q_tok"].astype(np.float32))
    O.verify(sub, mk["draft_tokens"], **q)
    n = sub["B"]
    O.accept_stats(dict(draft=sub["backbone"], target=np.ascontiguousarray(sub["target"][:, :g]),
                        teacher=np.zeros((n, g), np.int32), conf_logits=np.zeros((n, g), np.float32),
                        block_mask=None, N=n, gamma=g, V=sub["V"], dtype=sub["dtype"]))


def cpu_baseline(inp, nreq, cfg_name="decode"):
    """The oracle (single-threaded C++) on the first nreq requests of the
    batch: once on one core, then with the requests split over one thread per
    host core (up to 16, the machine's CPU share); the oracle's calls release the
    GIL, so the threads run in parallel."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as O
    from workloads import decode_inputs

    reqs = list(range(nreq))
    sub = decode_inputs(cfg_name, requests=reqs, with_embed=False)
    sub["embed"] = inp["embed"]
    g = sub["gamma"]
    t = time.perf_counter()
    _oracle_step(O, sub)
    sec = time.perf_counter() - t
    nth = max(1, min(16, os.cpu_count() or 1, nreq))
    parts = [reqs[i::nth] for i in range(nth)]
    subs = []
    for pr in parts:
        sp = decode_inputs(cfg_name, requests=pr, with_embed=False)
        sp["embed"] = inp["embed"]
        subs.append(sp)
    t = time.perf_counter()
    with ThreadPoolExecutor(max_workers=nth) as ex:
        list(ex.map(lambda sp: _oracle_step(O, sp), subs))
    sec_t = time.perf_counter() - t
    return dict(value=round(nreq * (g + 1) / sec, 2), unit="rows/s", cores=1, kind="oracle",
                sample=f"{nreq} of the {inp['B']} requests (Markov sample + verify + accept "
                       f"stats), {sec:.1f}s single-threaded",
                cpu_model=cpu_model(),
                threaded=dict(value=round(nreq * (g + 1) / sec_t, 2), unit="rows/s", cores=nth,
                              sample=f"the same {nreq} requests over {nth} threads, {sec_t:.1f}s"))


if __name__ == "__main__":
    main()
