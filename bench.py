#!/usr/bin/env python3
"""Throughput of the MI355X SSD varlen prefill scan (and the MTP state update).

One step = one ssd_combined_varlen call (chunk cumsum with bmm; chunk state with
state passing, here cut into 3 parallel segments per head and chained by a carry
step; chunk scan) over the single-sequence Mamba2 layer prefill:
L = 4096 tokens, 80 heads, headdim 64, d_state 128, 1 group, chunk 256, bf16
x/B/C/dt, fp32 A/D/state. Inputs are seeded synthetic draws, resident in HBM
before the timed region. `value` = tokens / s of that call (one layer).

The same JSON line also carries:
  roofline      the dominant prefill kernel's algorithmic bytes per launch over
                its HIP-event-timed average duration, against HBM peak
  kernels       every prefill kernel's average duration and achieved GB/s
  decode        the MTP verify state update (128 requests x 3 tokens, 128 heads,
                bf16 cache of 512 slots, intermediate states kept): updates / s
                and its roofline
  cpu_baseline  the CPU oracle (float64 recurrence) on the same prefill, timed on
                this host's cores

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # (200 timed steps of ~0.09 ms: long enough that the clocks have settled, as in a
    # serving loop; shorter runs read the clock ramp)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (for scaling HBM counters)")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other prefill shapes (used for the profiling runs, so that "
                         "every dispatch of a kernel has the headline shape)")
    ap.add_argument("--shape", choices=("cached_continuation_32x32", "mixed_varlen_8seq_ckpt"),
                    help="time only the combined call on this other prefill shape (for a kernel "
                         "trace of that shape); prints one JSON line for it")
    ap.add_argument("--summarize-shape-trace", nargs=2, metavar=("TRACE_DIR", "SHAPE"),
                    help="write profiles/kernel_trace_prefill_<SHAPE>.md from the rocprofv3 "
                         "kernel trace of `--shape SHAPE` (no GPU work)")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ summaries from rocprofv3 output of this script "
                         "(no GPU work)")
    return ap.parse_args()


# ---------------------------------------------------------------------------------------
# algorithmic bytes per launch of each prefill kernel (what the kernel must move at least)

def prefill_bytes(T, S, H, P, N, G, Q, nc, ex, es, s_init, checkpoints):
    st = nc * H * P * N * 4                 # chunk states (fp32)
    ent = nc * H * P * N * ex               # entering states (input dtype)
    per_chunk = 2 * H * nc * Q * 4          # dA_cumsum + dt per chunk position (fp32)
    cb = nc * G * (Q // 16) * (Q // 16 + 1) // 2 * 256 * ex   # causal 16x16 tiles of CB
    return {
        "chunk_cumsum": T * H * ex + per_chunk,
        "bmm_chunk": 2 * T * G * N * ex + cb,
        "chunk_state": T * H * P * ex + T * G * N * ex + per_chunk + st,
        "state_passing": st + ent + (s_init + S) * H * P * N * es
                         + (nc * H * P * N * es if checkpoints else 0),
        # fused chunk state + state passing: x and B in, entering states out; the
        # chunk states stay on chip
        "chunk_state_passing": T * H * P * ex + T * G * N * ex + per_chunk + ent
                               + (s_init + S) * H * P * N * es
                               + (nc * H * P * N * es if checkpoints else 0),
        "chunk_scan": 2 * T * H * P * ex + T * G * N * ex + per_chunk + cb + ent,
    }


# kernel name fragment (as rocprofv3 prints it) -> (name used here, source files it is built from)
_PRE = ["ssd_prefill.hip", "ssd_device.h", "ssd_launch.h"]
_DEC = ["ssd_decode.hip", "ssd_device.h", "ssd_launch.h", "ssd_ssu.h"]
KERNELS = {
    "chunk_prep_kernel": ("chunk_prep", _PRE),
    "chunk_cumsum_kernel": ("chunk_cumsum", _PRE),
    "bmm_kernel": ("bmm_chunk", _PRE),
    "state_scan_fast_kernel": ("chunk_state_passing", _PRE),
    "state_carry_kernel": ("state_carry", _PRE),
    "chunk_scan_fast_kernel": ("chunk_scan", _PRE),
    "state_update_kernel": ("selective_state_update", _DEC),
    "replay_update_fast_kernel": ("replay_update", ["ssd_replay.hip", "ssd_device.h",
                                                    "ssd_launch.h", "ssd_ssu.h"]),
}
CSRC = os.path.join("state_space_model_varlen_amd", "csrc")
CALIBRATION_BYTES = 256 << 20   # the --copy-calibration copy


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel):
    """HBM bytes per launch of a kernel from committed counter runs
    (profiles/traffic_<kernel>.json), valid only while the sources the kernel is
    built from are unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    srcs = rec.get("sources", [])
    if not srcs or not all(os.path.exists(os.path.join(ROOT, p)) for p in srcs):
        return None
    if source_sha(srcs) != rec.get("source_sha"):
        return None
    return rec.get("bytes_per_launch")


def summarize_profiles(trace_dir, fetch_dir, write_dir, cmds):
    """Turn the rocprofv3 output of the three profiling runs of this script
    (kernel trace; FETCH_SIZE; WRITE_SIZE, both with --copy-calibration) into the
    committed summaries: profiles/kernel_trace_*.md, profiles/hbm_traffic_*.md and
    one profiles/traffic_<kernel>.json per kernel. Counter values (KiB per
    dispatch) are scaled by what the same counter reads for the 256 MiB
    calibration copy (the last copy dispatch of the run)."""
    import csv
    import re

    def short(name):
        """Report name of a kernel; the variants of the segmented state pass that
        the combined call runs for this layer get their own rows."""
        for frag, (nm, _) in KERNELS.items():
            if frag in name:
                m = re.search(r"state_scan_fast_kernelILi\d+ELb[01]ELb1E", name) or \
                    re.search(r"chunk_scan_fast_kernelILi\d+ELb1E", name)
                return nm + "_segmented" if m else nm
        return None

    def sources(nm):
        base = nm[:-len("_segmented")] if nm.endswith("_segmented") else nm
        return [os.path.join(CSRC, p) for p in next(v[1] for v in KERNELS.values()
                                                    if v[0] == base)]

    stats = list(csv.DictReader(open(os.path.join(trace_dir, "c1_kernel_stats.csv"))))
    counters = {}
    scale = {}
    for ctr, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
        cal = max(copies, key=lambda r: int(r["Dispatch_Id"]))
        scale[ctr] = CALIBRATION_BYTES / (float(cal["Counter_Value"]) * 1024.0)
        per = {}
        for r in rows:
            nm = short(r["Kernel_Name"])
            if nm:
                per.setdefault(nm, []).append(float(r["Counter_Value"]))
        counters[ctr] = {k: sum(v) / len(v) for k, v in per.items()}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    lines = ["# Kernel trace: SSD prefill (L=4096, 80 heads) and MTP verify update (128 x 3 tokens)",
             "", "Command (MI355X, one GPU, from the repository root):", "```", cmds[0], "```",
             "Source: `c1_kernel_stats.csv` written by that command (rocprofv3 `--stats`). "
             "Prefill kernels run inside ssd_combined_varlen (warm-up + timed steps) and alone "
             "(per-kernel timing, the step-wise entry points); torch kernels (input casts, "
             "copies) omitted. For this layer (one sequence, 80 heads) the combined call cuts "
             "each head's chunk chain into 3 segments: its state pass, carry step and chunk "
             "scan are the `_segmented` / `state_carry` rows; the step-wise entry points run "
             "the unsegmented kernels (the plain rows).", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        nm = short(r["Name"])
        if nm:
            lines.append(f"| {nm} (`{r['Name'][:48]}...`) | {r['Calls']} | "
                         f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                         f"{float(r['MaxNs']) / 1e3:.2f} |")
    with open(os.path.join(ROOT, "profiles", "kernel_trace_prefill_L4096_and_mtp_verify.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    lines = ["# HBM traffic per dispatch: SSD prefill (L=4096, 80 heads) and MTP verify update",
             "", "Commands (MI355X, one GPU, from the repository root), one counter per run:", "```",
             cmds[1], cmds[2], "```",
             f"Scale factors from the 256 MiB calibration copy in the same runs: FETCH_SIZE x "
             f"{scale['FETCH_SIZE']:.4f}, WRITE_SIZE x {scale['WRITE_SIZE']:.4f}.", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes per launch (scaled) |",
             "|---|---|---|---|"]
    for nm in sorted(set(counters["FETCH_SIZE"]) & set(counters["WRITE_SIZE"])):
        f, w = counters["FETCH_SIZE"][nm], counters["WRITE_SIZE"][nm]
        fb, wb = f * 1024 * scale["FETCH_SIZE"], w * 1024 * scale["WRITE_SIZE"]
        lines.append(f"| {nm} | {f:.1f} | {w:.1f} | {fb + wb:.0f} |")
        srcs = sources(nm)
        with open(os.path.join(ROOT, "profiles", f"traffic_{nm}.json"), "w") as fh:
            json.dump({"kernel": nm, "sources": srcs, "source_sha": source_sha(srcs),
                       "fetch_bytes": round(fb), "write_bytes": round(wb),
                       "bytes_per_launch": round(fb + wb), "fetch_scale": scale["FETCH_SIZE"],
                       "write_scale": scale["WRITE_SIZE"], "commands": cmds[1:]}, fh, indent=1)
            fh.write("\n")
    with open(os.path.join(ROOT, "profiles", "hbm_traffic_prefill_L4096_and_mtp_verify.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def shape_only(args, sy, ssd, torch):
    """The combined call alone on one of the other prefill shapes: W warm-up and K
    timed calls, HIP events on the call's stream. Used for the kernel trace of that
    shape (prints its time per call and tokens/s)."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    ocfg = {"cached_continuation_32x32": sy.C2, "mixed_varlen_8seq_ckpt": sy.C3}[args.shape]
    oin = sy.make_prefill(ocfg)
    oT, oS, oH, oP, oN, oG, oQ = (ocfg.total_tokens, ocfg.num_seqs, ocfg.nheads, ocfg.headdim,
                                  ocfg.d_state, ocfg.ngroups, ocfg.chunk_size)
    op = ssd.make_problem(oT, oS, oH, oP, oN, oG, oQ, ocfg.num_slots, ocfg.in_dtype,
                          ocfg.state_dtype)
    ox, odt, oA, oB, oC, oD = (t.to(dev) for t in (oin.x, oin.dt, oin.A, oin.B, oin.C, oin.D))
    ocu, oidx = oin.cu_seqlens.to(dev), oin.state_indices.to(dev)
    ohi = oin.has_initial.to(dev) if oin.has_initial is not None else None
    gen = torch.Generator(device=dev).manual_seed(4)
    ocache = (torch.randn(ocfg.num_slots, oH, oP, oN, device=dev, generator=gen) * 0.03
              ).to(ocfg.state_dtype)
    ock = (torch.empty(ssd.max_chunks(op), oH, oP, oN, dtype=ocfg.state_dtype, device=dev)
           if ocfg.checkpoints else None)
    oy = torch.empty(oT, oH, oP, dtype=ocfg.in_dtype, device=dev)
    ows = ssd.alloc_workspace(op, dev)

    def call():
        ssd.ssd_combined_varlen(op, ox, odt, oA, oB, oC, oD, ocu, ocache, oidx, ohi, oy, ock, ows,
                                stream)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(20_000_000)
    a.record(stream)
    for _ in range(args.steps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / args.steps
    print(json.dumps({"shape": args.shape, "tokens": oT, "seqs": oS, "combined_us": round(us, 3),
                      "tokens_per_s": round(oT / (us * 1e-6), 1), "steps": args.steps,
                      "warmup": args.warmup}), flush=True)


def shape_trace_command(shape):
    return ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof/" + shape +
            " -o run -- python3 bench.py --shape " + shape + " --steps 200 --warmup 50")


def summarize_shape_trace(trace_dir, shape):
    """profiles/kernel_trace_prefill_<shape>.md from the kernel statistics of
    shape_trace_command(shape) (the library's kernels only)."""
    import csv
    stats = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))))
    lines = [f"# Kernel trace: SSD prefill, {shape} (the combined call alone)", "",
             "Command (MI355X, one GPU, from the repository root):", "```",
             shape_trace_command(shape), "```",
             "Source: `run_kernel_stats.csv` written by that command (rocprofv3 `--stats`): "
             "50 warm-up and 200 timed calls of ssd_combined_varlen; torch kernels (input "
             "generation, casts) omitted.", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        if "ssd" not in r["Name"]:
            continue
        lines.append(f"| `{r['Name'][:70]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    out = os.path.join(ROOT, "profiles", f"kernel_trace_prefill_{shape}.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


PROFILE_COMMANDS = [
    "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof/trace -o c1 -- "
    "python3 bench.py --steps 20 --warmup 3 --no-cpu-baseline --headline-only",
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof/fetch -o run -- "
    "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --headline-only --copy-calibration",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof/write -o run -- "
    "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --headline-only --copy-calibration",
]


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles, PROFILE_COMMANDS)
        return
    if args.summarize_shape_trace:
        summarize_shape_trace(*args.summarize_shape_trace)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported; the scan shards by heads or sequences with no exchange, so "
              "the one-GPU figure is the per-GPU figure.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ssd_synth as sy
    import state_space_model_varlen_amd as ssd

    if args.shape:
        shape_only(args, sy, ssd, torch)
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # ------------------------------------------------------------------ prefill inputs
    cfg = sy.C1
    inp = sy.make_prefill(cfg)
    T, S, H, P, N, G, Q = (cfg.total_tokens, cfg.num_seqs, cfg.nheads, cfg.headdim, cfg.d_state,
                           cfg.ngroups, cfg.chunk_size)
    p = ssd.make_problem(T, S, H, P, N, G, Q, 1, cfg.in_dtype, cfg.state_dtype)
    x, dt, A, B, C, D = (t.to(dev) for t in (inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D))
    cu, idx = inp.cu_seqlens.to(dev), inp.state_indices.to(dev)
    cache = torch.zeros(1, H, P, N, dtype=cfg.state_dtype, device=dev)
    y = torch.empty(T, H, P, dtype=cfg.in_dtype, device=dev)
    ws = ssd.alloc_workspace(p, dev)
    torch.cuda.synchronize()

    def step():
        ssd.ssd_combined_varlen(p, x, dt, A, B, C, D, cu, cache, idx, None, y, None, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    elapsed = max(wall, gpu_ms / 1e3)
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = T * args.steps / elapsed

    # the same call with the last-level cache (256 MB on MI355X) flushed before each
    # call by a 512 MiB device write, each call timed alone: how much of the warm
    # figure comes from inputs still cached from the previous call (context only)
    cold = None
    if not args.headline_only:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        ca_, cb_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        times = []
        for _ in range(max(args.steps // 4, 5)):
            flush.fill_(1)
            ca_.record(stream)
            step()
            cb_.record(stream)
            torch.cuda.synchronize()
            times.append(ca_.elapsed_time(cb_) * 1e3)
        del flush
        cold_us = float(np.median(times))
        cold = {"us_per_step": round(cold_us, 2), "tokens_per_s": round(T / (cold_us * 1e-6), 1),
                "calls": len(times), "flush_bytes": 512 << 20}

    # ------------------------------------------------------------------ per-kernel timing
    nc = int(np.ceil(T / Q))
    buf = ssd.alloc_step_buffers(p, dev)
    launches = {
        "chunk_cumsum": lambda: ssd.ssd_chunk_cumsum(p, dt, A, cu, buf["chunk_meta"],
                                                     buf["dA_cumsum"], buf["dt_chunk"], stream),
        "bmm_chunk": lambda: ssd.ssd_bmm_chunk(p, B, C, buf["chunk_meta"], buf["CB"], stream),
        # what ssd_combined_varlen runs for bf16 inputs with headdim 64, d_state 128
        "chunk_state_passing": lambda: ssd.ssd_chunk_state_passing(
            p, x, B, buf["chunk_meta"], buf["dA_cumsum"], buf["dt_chunk"], cache, idx, None,
            buf["entering"], None, stream),
        "chunk_scan": lambda: ssd.ssd_chunk_scan(p, x, C, D, buf["chunk_meta"], buf["dA_cumsum"],
                                                 buf["dt_chunk"], buf["CB"], buf["entering"], y,
                                                 stream),
    }
    for fn in launches.values():      # one pass to fill every intermediate
        fn()
    torch.cuda.synchronize()
    nb = prefill_bytes(T, S, H, P, N, G, Q, nc, 2, 4, 0, False)
    kernels = {}
    reps = max(args.steps, 10)
    def avg_us(fn):
        """Average duration of back-to-back launches of fn, from HIP events recorded on
        the stream the kernels run on. A spin kernel queued first keeps the GPU busy
        while the host enqueues every launch, so host-side call overhead does not
        show up as idle time between the events."""
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(20_000_000)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    for name, fn in launches.items():
        us = avg_us(fn)
        kernels[name] = {"avg_us": round(us, 3), "bytes": nb[name],
                         "GBps": round(nb[name] / (us * 1e-6) / 1e9, 1)}
    # the roofline is reported for the chunk scan: the largest kernel of the timed call
    # (the call cuts this layer's state pass into segments, which the step-wise
    # chunk_state_passing entry point timed above does not, so that entry point's
    # time is not the time the state pass takes inside the call)
    dom = "chunk_scan"
    dk = kernels[dom]
    traffic = load_traffic(dom)
    roofline = {"kernel": dom, "bound": "hbm", "achieved": dk["GBps"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(dk["GBps"] / HBM_PEAK_GBS, 4),
                "traffic": traffic}

    # ------------------------------------------------------------------ decode / MTP verify
    dcfg = sy.C4
    dd = sy.make_decode(dcfg)
    R, TT, DH, DP, DN, DG = (dcfg.num_reqs, dcfg.tokens_per_req, dcfg.nheads, dcfg.headdim,
                             dcfg.d_state, dcfg.ngroups)
    up = ssd.make_ssu_problem(R, TT, DH, DP, DN, DG, dcfg.num_slots, dcfg.in_dtype,
                              dcfg.state_dtype)
    gen = torch.Generator(device=dev).manual_seed(4)
    dcache = (torch.randn(dcfg.num_slots, DH, DP, DN, device=dev, generator=gen) * 0.03
              ).to(dcfg.state_dtype)
    dx, ddt, dA, dB, dC, dD = (t.to(dev) for t in (dd.x, dd.dt, dd.A, dd.B, dd.C, dd.D))
    didx = dd.state_indices.to(dev)
    dy = torch.empty(R, TT, DH, DP, dtype=dcfg.in_dtype, device=dev)
    inter = torch.empty(R, TT, DH, DP, DN, dtype=dcfg.state_dtype, device=dev)
    ssu_us = avg_us(lambda: ssd.selective_state_update(up, dcache, didx, dx, ddt, dA, dB, dC, dD,
                                                       dy, inter, stream))
    es = 2
    ssu_bytes = R * DH * DP * DN * es * (1 + TT) + R * TT * (2 * DH * DP + 2 * DG * DN + DH) * 2
    decode = {"workload": "mtp_verify R=128 T=3 H=128 P=64 N=128 G=8 bf16 cache 512 slots",
              "metric": "decode updates/s", "value": round(R * TT / (ssu_us * 1e-6), 1),
              "unit": "updates/s", "avg_us": round(ssu_us, 3),
              "roofline": {"kernel": "selective_state_update", "bound": "hbm",
                           "achieved": round(ssu_bytes / (ssu_us * 1e-6) / 1e9, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(ssu_bytes / (ssu_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                           "traffic": load_traffic("selective_state_update"),
                           "bytes": ssu_bytes}}

    # ------------------------------------------------------------------ ReplaySSM decode
    # The same MTP verify workload without stored draft states: checkpoint + input
    # rings per slot (16 entries: up to 13 history tokens and one 3-token window).
    # One step = verify + cursor move, over a seeded sequence of accepted counts,
    # timed after enough steps that every request's history is in its steady cycle.
    import dataclasses
    W = 16
    rings = ssd.alloc_replay_rings(up, W, dev)
    rck = dcache.clone()
    nsteps = 24
    acc_seq = [sy.make_decode(dataclasses.replace(dcfg, seed=dcfg.seed + 1000 * k)).num_accepted
               .to(dev) for k in range(nsteps)]
    ry = torch.empty_like(dy)

    def replay_step(k):
        ssd.ssd_replay_update(up, W, rck, rings["ring_x"], rings["ring_dt"], rings["ring_B"],
                              rings["cursor"], didx, dx, ddt, dA, dB, dC, dD, ry, stream)
        ssd.ssd_replay_advance(up, W, rings["cursor"], didx, acc_seq[k], stream)

    for k in range(nsteps):          # warm-up: histories reach their steady cycle
        replay_step(k)
    torch.cuda.synchronize()
    ra, rb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(20_000_000)
    ra.record(stream)
    for k in range(nsteps):
        replay_step(k)
    rb.record(stream)
    torch.cuda.synchronize()
    replay_us = ra.elapsed_time(rb) * 1e3 / nsteps
    # algorithmic bytes of the timed steps: the cursor rule replayed on the host
    L = W - TT
    hist = np.zeros(R, dtype=np.int64)
    per_tok = (DH * DP + DH + DG * DN) * 2            # x, dt, B of one token (bf16)
    state_b = DH * DP * DN * es
    replay_bytes, hist_sum = 0, 0
    for k in range(2 * nsteps):
        ck = hist + TT > L
        if k >= nsteps:
            hist_sum += int(hist.sum())
            replay_bytes += int(R * state_b + hist.sum() * per_tok
                                + R * TT * (DH * DP + DH + 2 * DG * DN + DH * DP) * 2
                                + R * TT * per_tok + ck.sum() * state_b)
        a = acc_seq[k % nsteps].cpu().numpy()
        hist = np.where(ck, 1 + a, hist + 1 + a)
    replay_bytes //= nsteps
    replay_kernel_us = avg_us(lambda: ssd.ssd_replay_update(
        up, W, rck, rings["ring_x"], rings["ring_dt"], rings["ring_B"], rings["cursor"], didx,
        dx, ddt, dA, dB, dC, dD, ry, stream))
    replay = {"workload": "mtp_verify_replayssm R=128 T=3 H=128 P=64 N=128 G=8 bf16, ring 16",
              "metric": "decode updates/s", "value": round(R * TT / (replay_us * 1e-6), 1),
              "unit": "updates/s", "avg_us_per_step": round(replay_us, 3),
              "mean_history_tokens": round(hist_sum / (nsteps * R), 2),
              "roofline": {"kernel": "replay_update + replay_advance", "bound": "hbm",
                           "achieved": round(replay_bytes / (replay_us * 1e-6) / 1e9, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(replay_bytes / (replay_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                           "bytes": replay_bytes,
                           "traffic": load_traffic("replay_update")},
              "verify_kernel_us_at_end_state": round(replay_kernel_us, 3)}
    del rings, rck

    # ------------------------------------------------------------------ steps either side
    # (context): the layer's dt preprocessing fused into the c1 call, the MTP verify as a
    # packed varlen batch (1-3 tokens per request), and fp16 states with Philox
    # stochastic rounding (the c4 verify with per-token states, 5 rounds)
    extras = {}
    if not args.headline_only:
        bias = torch.from_numpy(inp.dt_bias).float().to(dev)
        tf = ssd.make_dt_transform(bias, sy.DT_MIN, sy.DT_MAX)
        raw = inp.dt_raw.to(dev)
        fused_us = avg_us(lambda: ssd.ssd_combined_varlen_dt(p, tf, x, raw, A, B, C, D, cu, cache,
                                                             idx, None, y, None, ws, stream))
        extras["prefill_dt_fused_c1"] = {"combined_us": round(fused_us, 3),
                                         "tokens_per_s": round(T / (fused_us * 1e-6), 1)}
        counts = torch.from_numpy(np.random.default_rng(5).integers(1, TT + 1, size=R)
                                  .astype(np.int32))
        vcu = torch.zeros(R + 1, dtype=torch.int32)
        vcu[1:] = torch.cumsum(counts, 0)
        Tt = int(vcu[-1])
        flat = lambda t: t.reshape(-1, *t.shape[2:])[:Tt].contiguous()
        vx, vdt, vB, vC = flat(dx), flat(ddt), flat(dB), flat(dC)
        vy = torch.empty(Tt, DH, DP, dtype=dcfg.in_dtype, device=dev)
        vinter = torch.empty(Tt, DH, DP, DN, dtype=dcfg.state_dtype, device=dev)
        vcu = vcu.to(dev)
        var_us = avg_us(lambda: ssd.selective_state_update_varlen(up, vcu, dcache, didx, vx, vdt,
                                                                  dA, vB, vC, dD, vy, vinter,
                                                                  stream=stream))
        extras["decode_varlen_mtp"] = {"tokens": Tt, "avg_us": round(var_us, 3),
                                       "updates_per_s": round(Tt / (var_us * 1e-6), 1)}
        del vinter
        up16 = ssd.make_ssu_problem(R, TT, DH, DP, DN, DG, dcfg.num_slots, dcfg.in_dtype,
                                    torch.float16)
        c16 = dcache.to(torch.float16)
        i16 = torch.empty(R, TT, DH, DP, DN, dtype=torch.float16, device=dev)
        seed = torch.tensor([12345], dtype=torch.int64, device=dev)
        for name, opt in (("fp16_nearest", ssd.make_options()),
                          ("fp16_stochastic_philox5", ssd.make_options(sr_seed=seed, sr_rounds=5))):
            us16 = avg_us(lambda: ssd.selective_state_update_ex(up16, opt, c16, didx, dx, ddt, dA,
                                                                dB, dC, dD, dy, i16,
                                                                stream=stream))
            extras[f"decode_{name}"] = {"avg_us": round(us16, 3),
                                        "updates_per_s": round(R * TT / (us16 * 1e-6), 1)}
        del c16, i16

    # ------------------------------------------------------------------ other prefill shapes
    # (context, not the headline): the cached short continuation and the mixed varlen
    # batch with checkpoints - the whole combined call, and the step-wise state passing
    # kernel on its own bytes (chunk states in, entering states, initial / final states
    # and checkpoints)
    others = {}
    other_cfgs = () if args.headline_only else (("cached_continuation_32x32", sy.C2),
                                                  ("mixed_varlen_8seq_ckpt", sy.C3))
    for cname, ocfg in other_cfgs:
        oin = sy.make_prefill(ocfg)
        oT, oS, oH, oP, oN, oG, oQ = (ocfg.total_tokens, ocfg.num_seqs, ocfg.nheads, ocfg.headdim,
                                      ocfg.d_state, ocfg.ngroups, ocfg.chunk_size)
        op = ssd.make_problem(oT, oS, oH, oP, oN, oG, oQ, ocfg.num_slots, ocfg.in_dtype,
                              ocfg.state_dtype)
        ox, odt, oA, oB, oC, oD = (t.to(dev) for t in (oin.x, oin.dt, oin.A, oin.B, oin.C, oin.D))
        ocu, oidx = oin.cu_seqlens.to(dev), oin.state_indices.to(dev)
        ohi = oin.has_initial.to(dev) if oin.has_initial is not None else None
        ocache = (torch.randn(ocfg.num_slots, oH, oP, oN, device=dev, generator=gen) * 0.03
                  ).to(ocfg.state_dtype)
        omc = ssd.max_chunks(op)
        ock = (torch.empty(omc, oH, oP, oN, dtype=ocfg.state_dtype, device=dev)
               if ocfg.checkpoints else None)
        oy = torch.empty(oT, oH, oP, dtype=ocfg.in_dtype, device=dev)
        ows = ssd.alloc_workspace(op, dev)
        comb_us = avg_us(lambda: ssd.ssd_combined_varlen(op, ox, odt, oA, oB, oC, oD, ocu, ocache,
                                                         oidx, ohi, oy, ock, ows, stream))
        obuf = ssd.alloc_step_buffers(op, dev)
        ssd.ssd_chunk_cumsum(op, odt, oA, ocu, obuf["chunk_meta"], obuf["dA_cumsum"],
                             obuf["dt_chunk"], stream)
        ssd.ssd_chunk_state(op, ox, oB, obuf["chunk_meta"], obuf["dA_cumsum"], obuf["dt_chunk"],
                            obuf["chunk_states"], stream)
        sp_us = avg_us(lambda: ssd.ssd_state_passing(op, obuf["chunk_states"], obuf["dA_cumsum"],
                                                     obuf["chunk_meta"], ocache, oidx, ohi,
                                                     obuf["entering"], ock, stream))
        onc = int(np.sum(-(-np.diff(oin.cu_seqlens.numpy()) // oQ)))   # chunks, ceil per seq
        es_o = 2 if ocfg.state_dtype == torch.bfloat16 else 4
        s_init = int(oin.has_initial.sum()) if oin.has_initial is not None else 0
        sp_bytes = prefill_bytes(oT, oS, oH, oP, oN, oG, oQ, onc, 2, es_o, s_init,
                                 ocfg.checkpoints)["state_passing"]
        others[cname] = {
            "tokens": oT, "seqs": oS, "combined_us": round(comb_us, 3),
            "tokens_per_s": round(oT / (comb_us * 1e-6), 1),
            "state_passing_step": {"avg_us": round(sp_us, 3), "bytes": sp_bytes,
                                   "GBps": round(sp_bytes / (sp_us * 1e-6) / 1e9, 1),
                                   "frac": round(sp_bytes / (sp_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}}
        if cname == "mixed_varlen_8seq_ckpt":
            # the same batch in align mode: odd sequences follow 4224 cached tokens
            pre = torch.tensor([ocfg.prefix_len if int(oin.has_initial[s]) else 0
                                for s in range(oS)], dtype=torch.int32, device=dev)
            ack = torch.empty(ssd.max_chunks_aligned(op), oH, oP, oN, dtype=ocfg.state_dtype,
                              device=dev)
            aws = ssd.alloc_workspace_aligned(op, dev)
            al_us = avg_us(lambda: ssd.ssd_combined_varlen_aligned(
                op, pre, ox, odt, oA, oB, oC, oD, ocu, ocache, oidx, ohi, oy, ack, aws, stream))
            others[cname]["aligned_combined_us"] = round(al_us, 3)
            del ack, aws
        del ox, odt, oB, oC, oy, ows, obuf, ocache, ock

    # achievable HBM bandwidth on this machine, for context: a plain 1 GiB device copy
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    ca, cb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ca.record(stream)
    for _ in range(5):
        dst.copy_(src)
    cb.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 5 / (ca.elapsed_time(cb) * 1e-3) / 1e9
    del src, dst
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        nthreads = oracle.max_threads()
        xs, dts, Bs, Cs = (oracle.f64(t) for t in (inp.x, inp.dt, inp.B, inp.C))
        # a bounded sample of about 10 s of wall clock: the whole layer prefill run
        # back to back until 10 s have passed (at least 3 runs); rate = tokens / time
        runs, total = 0, 0.0
        while runs < 3 or total < 10.0:
            t1 = time.perf_counter()
            oracle.recurrence(xs, dts, inp.A, Bs, Cs, inp.D, inp.cu_seqlens.numpy(), Q,
                              nthreads=nthreads)
            total += time.perf_counter() - t1
            runs += 1
        cpu = {"value": round(T * runs / total, 1), "unit": "tokens/s", "cores": nthreads,
               "kind": "oracle",
               "sample": f"the whole layer prefill (4096 tokens x 80 heads, float64 recurrence) "
                         f"run {runs} times back to back, {total:.1f} s wall clock on "
                         f"{nthreads} threads"}

    out = {
        "metric": "SSD prefill tokens/s per layer + decode updates/s; % MFMA / HBM roofline",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mamba2_ssd_prefill_L4096_H80_P64_N128_G1_Q256",
                   "seq_len": T, "num_seqs": S, "nheads": H, "headdim": P, "d_state": N,
                   "ngroups": G, "chunk_size": Q, "inputs": "bf16 x/B/C/dt, fp32 A/D/state",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cold_cache": cold,
        "hbm_copy_GBps": round(copy_gbps, 1),
        "kernels": kernels,
        "decode": decode,
        "decode_replayssm": replay,
        "other_prefill_shapes": others,
        "steps_either_side": extras,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
