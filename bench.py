#!/usr/bin/env python3
"""Throughput of the MI355X SSD varlen prefill scan (and the MTP state update).

One step = one ssd_combined_varlen call over the single-sequence Mamba2 layer
prefill: L = 4096 tokens, 80 heads, headdim 64, d_state 128, 1 group, chunk 256,
bf16 x/B/C/dt, fp32 A/D/state. Inputs are seeded synthetic draws, resident in
HBM before the timed region. Each timed call starts with the caches holding none
of its data: a 512 MiB device read (outside the timed interval) evicts the 256 MB
last-level cache and the L2s, so nothing the call reads is left over from the
call before. `value` = tokens / s of the median call (one layer); `ms_per_step` =
that median. (A 512 MiB write instead would leave up to 256 MB of unrelated dirty
lines whose write-back the timed call would pay for; that median is reported
beside it as cold_after_write_flush.)

The same JSON line also carries:
  warm          the same call back to back on resident inputs (context)
  launches      every kernel launch of the timed call, timed by HIP events on
                which each launch records its own start and end (ssd_options.trace,
                hipExtLaunchKernelGGL), over cache-flushed calls: mean us each, its
                algorithmic bytes and flops
  roofline      the launch that takes longest (the dominant kernel): algorithmic
                bytes per launch over its mean duration against HBM peak, its
                algorithmic flops against bf16 MFMA peak, and the HBM traffic and
                MFMA work rocprofv3 counters read for it
  other_prefill_shapes  the cached short continuation (32 x 32 tokens) and the mixed
                varlen batch with checkpoints, timed the same way
  decode        the MTP verify state update (128 requests x 3 tokens, 128 heads,
                bf16 cache of 512 slots, intermediate states kept): updates / s
  cpu_baseline  the CPU oracle (float64 recurrence) on the same layer prefill,
                best of 3 runs on all host threads and on one

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, published
FLUSH_BYTES = 512 << 20         # twice the 256 MB last-level cache


def flush_caches(flush, write=False):
    """Evict every cache level: a read of the whole flush buffer (its lines stay
    clean), or with write a fill (which leaves them dirty)."""
    import torch
    if write:
        flush.fill_(1)
    else:
        flush.view(torch.int32).sum()
CALIBRATION_BYTES = 256 << 20   # the --copy-calibration copy


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (for scaling HBM counters)")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the cache-flushed layer calls, plain and traced (used for the "
                         "profiling runs, so that every dispatch of a kernel is one of those)")
    ap.add_argument("--shape", choices=("cached_continuation_32x32", "mixed_varlen_8seq_ckpt",
                                        "decode_c4"),
                    help="only the cache-flushed calls on this other prefill shape, or only the "
                         "MTP verify updates (decode_c4), for a kernel trace and counters of "
                         "that shape; prints one JSON line for it")
    ap.add_argument("--summarize-profiles", nargs=2, metavar=("SHAPE", "PROF_DIR"),
                    help="write profiles/ summaries for SHAPE (layer_L4096 or a --shape name) "
                         "from the rocprofv3 output of profile_commands(SHAPE) under PROF_DIR "
                         "(trace/, fetch/, write/, mfma/ and the runs' stdout run0..3.log; no "
                         "GPU work)")
    return ap.parse_args()


# ---------------------------------------------------------------------------------------
# what each launch must move and compute (algorithmic bytes and flops per launch)

class Work:
    """Sizes of one prefill batch: T tokens, S sequences, nc chunks, e_x / e_s
    bytes per input / state element, s_init sequences with a cached state."""

    def __init__(self, lens, H, P, N, G, Q, ex, es, s_init, ckpt, nseg=1):
        self.lens = [int(v) for v in lens]
        self.T, self.S = sum(self.lens), len(self.lens)
        self.H, self.P, self.N, self.G, self.Q = H, P, N, G, Q
        self.chunk_lens = [min(Q, L - k) for L in self.lens for k in range(0, L, Q)]
        self.nc = len(self.chunk_lens)
        self.ex, self.es, self.s_init, self.ckpt, self.nseg = ex, es, s_init, ckpt, nseg


def launch_bytes(name, w: Work, entering_bytes=None):
    """Algorithmic HBM bytes of one launch: every input read once, every output
    written once. The chunk scan's entering states count at `entering_bytes` per
    element (the kernels store them in the input dtype; the per-kernel table of
    the scope document counts them in float32)."""
    T, S, H, P, N, G, Q, nc = w.T, w.S, w.H, w.P, w.N, w.G, w.Q, w.nc
    ex, es = w.ex, w.es
    HPN = H * P * N
    per_chunk = 2 * H * nc * Q * 4                       # cumsum + dt per position (fp32)
    cb = nc * G * (Q // 16) * (Q // 16 + 1) // 2 * 256 * ex   # causal 16 x 16 tiles of CB
    x, bc = T * H * P * ex, T * G * N * ex
    ent = nc * HPN * (ex if entering_bytes is None else entering_bytes)
    cache_io = (w.s_init + S) * HPN * w.es + (nc * HPN * es if w.ckpt else 0)
    fin = S * w.nseg * HPN * 4                           # segment final states (fp32)
    carry = S * (w.nseg - 1) * HPN * ex                  # segment starting states read
    table = {
        "chunk_cumsum": T * H * ex + per_chunk,
        "chunk_prep": T * H * ex + per_chunk + 2 * bc + cb,
        "bmm_chunk": 2 * bc + cb,
        "bmm_chunk_pairs": 2 * bc + cb,
        "chunk_state_passing": x + bc + per_chunk + ent + cache_io,
        "chunk_state_passing_multi": x + bc + per_chunk + ent + cache_io,
        "chunk_state_passing_segmented": x + bc + per_chunk + ent + w.s_init * HPN * es + fin,
        # the same launches doing the cumsum themselves: dt read, cumsum and dt rows
        # written; unsegmented, CB as well (C read, CB written)
        "chunk_state_passing_segmented_prep":
            x + 2 * bc + T * H * ex + per_chunk + ent + w.s_init * HPN * es + fin + cb,
        "chunk_state_passing_prep_bmm": x + 2 * bc + T * H * ex + per_chunk + ent + cache_io + cb,
        "state_carry": fin + S * w.nseg * HPN * ex + S * HPN * es,
        "chunk_scan": 2 * x + bc + per_chunk + cb + ent,
        "chunk_scan_segmented": 2 * x + bc + per_chunk + cb + ent + carry,
        # the one-launch short-sequence path: x, dt, B, C in, y out, initial and
        # final states, checkpoints
        "short_scan": 2 * x + T * H * ex + 2 * bc + cache_io,
    }
    return table.get(name)


def launch_flops(name, w: Work):
    """Algorithmic flops of one launch (causal part of the Q x Q work only)."""
    H, P, N, G = w.H, w.P, w.N, w.G
    q = w.chunk_lens
    intra = sum(H * P * v * (v + 1) for v in q)          # (CB o L) x, causal
    state_term = sum(2 * H * P * N * v for v in q)       # exp(cum) C . H_in
    chunk_state = sum(2 * H * P * N * v for v in q)      # x^T (w B)
    cbf = sum(G * N * v * (v + 1) for v in q)            # C B^T, causal
    if name.startswith("chunk_scan"):
        return intra + state_term
    if name in ("chunk_state_passing_prep_bmm", "chunk_state_passing_segmented_prep"):
        return chunk_state + cbf
    if name.startswith("chunk_state_passing"):
        return chunk_state
    if name in ("bmm_chunk", "bmm_chunk_pairs", "chunk_prep"):
        return cbf
    return 0


def segments(cfg):
    """Segments per sequence of a segmented combined call: enough state blocks (two
    64-column slices per (sequence, head)) for about 512, at most 8, at most the
    chunk bound T / Q + S."""
    n = 512 // (cfg.num_seqs * cfg.nheads * 2)
    n = min(n, 8, cfg.total_tokens // cfg.chunk_size + cfg.num_seqs)
    return n if n > 1 else 1


def layer_work(cfg, nseg=1):
    import torch
    ex = 2 if cfg.in_dtype == torch.bfloat16 else 4
    es = {torch.bfloat16: 2, torch.float16: 2}.get(cfg.state_dtype, 4)
    s_init = sum(1 for v in cfg.has_initial[:cfg.num_seqs] if v) if cfg.any_initial else 0
    return Work(cfg.seqlens, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups, cfg.chunk_size,
                ex, es, s_init, cfg.checkpoints, nseg)


# ---------------------------------------------------------------------------------------
# committed counter summaries (profiles/), valid while the kernel's sources are unchanged

CSRC = os.path.join("state_space_model_varlen_amd", "csrc")
PREFILL_SOURCES = [os.path.join(CSRC, f) for f in ("ssd_prefill.hip", "ssd_device.h",
                                                   "ssd_launch.h")]
DECODE_SOURCES = [os.path.join(CSRC, f) for f in ("ssd_decode.hip", "ssd_device.h",
                                                  "ssd_launch.h", "ssd_ssu.h")]
REPLAY_SOURCES = [os.path.join(CSRC, f) for f in ("ssd_replay.hip", "ssd_device.h",
                                                  "ssd_launch.h", "ssd_ssu.h")]

# rocprofv3 kernel name -> launch name (the names the library's trace gives)
KERNEL_PATTERNS = [
    (r"chunk_cumsum_kernel", "chunk_cumsum", PREFILL_SOURCES),
    (r"chunk_prep_kernel", "chunk_prep", PREFILL_SOURCES),
    (r"bmm_pair_kernel", "bmm_chunk_pairs", PREFILL_SOURCES),
    (r"bmm_kernel", "bmm_chunk", PREFILL_SOURCES),
    (r"state_scan_multi_kernel", "chunk_state_passing_multi", PREFILL_SOURCES),
    (r"state_scan_fast_kernelILi\d+ELb[01]ELb1ELb1E|state_scan_fast_kernel<\d+, \w+, true, true",
     "chunk_state_passing_segmented_prep", PREFILL_SOURCES),
    (r"state_scan_fast_kernelILi\d+ELb[01]ELb0ELb1E|state_scan_fast_kernel<\d+, \w+, false, true",
     "chunk_state_passing_prep_bmm", PREFILL_SOURCES),
    (r"state_scan_fast_kernelILi\d+ELb[01]ELb1E|state_scan_fast_kernel<\d+, \w+, true",
     "chunk_state_passing_segmented", PREFILL_SOURCES),
    (r"state_scan_fast_kernel", "chunk_state_passing", PREFILL_SOURCES),
    (r"state_carry_kernel", "state_carry", PREFILL_SOURCES),
    (r"short_scan_kernel", "short_scan", PREFILL_SOURCES),
    (r"chunk_scan_fast_kernelILi\d+ELb1E|chunk_scan_fast_kernel<\d+, true",
     "chunk_scan_segmented", PREFILL_SOURCES),
    (r"chunk_scan_fast_kernel|chunk_scan_kernel", "chunk_scan", PREFILL_SOURCES),
    (r"state_passing_kernel", "state_passing", PREFILL_SOURCES),
    (r"chunk_state_fast_kernel|chunk_state_kernel", "chunk_state", PREFILL_SOURCES),
    (r"state_update_kernel", "selective_state_update", DECODE_SOURCES),
    (r"replay_update_wave_kernel|replay_update_kernel", "replay_update", REPLAY_SOURCES),
]


def launch_name(kernel):
    for pat, nm, srcs in KERNEL_PATTERNS:
        if re.search(pat, kernel) or kernel == nm:
            return nm, srcs
    return None, None


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_counters(shape, name):
    """Counter figures of one launch on one shape (profiles/counters_<shape>.json),
    or None once the kernel's sources have changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"counters_{shape}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh).get(name)
    if not rec or source_sha(rec["sources"]) != rec["source_sha"]:
        return None
    return rec


# ---------------------------------------------------------------------------------------
# profiling commands and their summaries

def profile_commands(shape):
    sel = "--headline-only" if shape == "layer_L4096" else f"--shape {shape}"
    out = f"prof_raw/{shape}"
    run = f"python3 bench.py {sel} --no-cpu-baseline"
    return [
        f"rocprofv3 --kernel-trace --stats --output-format csv -d {out}/trace -o run -- {run}",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/fetch -o run -- {run} "
        "--steps 3 --warmup 1 --copy-calibration",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/write -o run -- {run} "
        "--steps 3 --warmup 1 --copy-calibration",
        f"rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE "
        f"--output-format csv -d {out}/mfma -o run -- {run} --steps 3 --warmup 1",
    ]


def sources_sha():
    """Hashes of the sources each group of kernels is built from (printed by every
    run, so that counter summaries carry the sources they were taken with)."""
    return {"prefill": source_sha(PREFILL_SOURCES), "decode": source_sha(DECODE_SOURCES),
            "replay": source_sha(REPLAY_SOURCES)}


def _group(srcs):
    return {id(PREFILL_SOURCES): "prefill", id(DECODE_SOURCES): "decode",
            id(REPLAY_SOURCES): "replay"}[id(srcs)]


def summarize_profiles(shape, prof_dir):
    """As _summarize below, with the sources' hashes the profiled runs printed."""
    shas = []
    for i in range(4):
        lines = [l for l in open(os.path.join(prof_dir, f"run{i}.log")).read().splitlines()
                 if l.startswith("{")]
        shas.append(json.loads(lines[-1])["sources_sha"])
    if any(v != shas[0] for v in shas):
        raise SystemExit("the profiled runs were built from different sources")
    _summarize(shape, *(os.path.join(prof_dir, d) for d in ("trace", "fetch", "write", "mfma")),
               shas[0])


def _summarize(shape, trace_dir, fetch_dir, write_dir, mfma_dir, run_sha):
    """profiles/kernel_trace_<shape>.md, profiles/counters_<shape>.md and
    profiles/counters_<shape>.json from the four runs of profile_commands(shape).
    HBM counters (KiB per dispatch) are scaled by what the same counter reads for
    the 256 MiB calibration copy; MFMA work is SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512
    flops (SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE are collected in the same run
    but not reported: their ratio is not normalised the way this summary could
    check)."""
    import csv

    def rows(d, stem):
        return list(csv.DictReader(open(os.path.join(d, f"run_{stem}.csv"))))

    cmds = profile_commands(shape)
    stats = rows(trace_dir, "kernel_stats")
    trace_rows = ["| launch | kernel | calls | average us | min us | max us |",
                  "|---|---|---|---|---|---|"]
    durations = {}
    for r in stats:
        nm, _ = launch_name(r["Name"])
        if nm:
            durations[nm] = float(r["AverageNs"]) / 1e3
            trace_rows.append(f"| {nm} | `{r['Name'][:60]}` | {r['Calls']} | "
                              f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                              f"{float(r['MaxNs']) / 1e3:.2f} |")
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_{shape}.md"), "w") as fh:
        fh.write("\n".join([f"# Kernel trace: {shape}", "",
                            "Command (MI355X, one GPU, from the repository root):", "```",
                            cmds[0], "```",
                            "Source: `run_kernel_stats.csv` written by that command (rocprofv3 "
                            "`--stats`): every dispatch is a cache-flushed ssd_combined_varlen "
                            "call (warm-up, timed, traced); torch kernels omitted.", ""]
                           + trace_rows) + "\n")
    per = {}
    scale = {}
    for ctr, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rr = rows(d, "counter_collection")
        cal = max((r for r in rr if "copyBuffer" in r["Kernel_Name"]),
                  key=lambda r: int(r["Dispatch_Id"]))
        scale[ctr] = CALIBRATION_BYTES / (float(cal["Counter_Value"]) * 1024.0)
        for r in rr:
            nm, srcs = launch_name(r["Kernel_Name"])
            if nm:
                per.setdefault(nm, {"sources": srcs}).setdefault(ctr, []).append(
                    float(r["Counter_Value"]) * 1024.0 * scale[ctr])
    mfma = {}
    for r in rows(mfma_dir, "counter_collection"):
        nm, srcs = launch_name(r["Kernel_Name"])
        if nm:
            key = (r["Dispatch_Id"], nm)
            mfma.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    for (_, nm), v in mfma.items():
        rec = per.setdefault(nm, {"sources": launch_name(nm)[1]})
        rec.setdefault("MOPS", []).append(v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0))
    mean = lambda a: sum(a) / len(a) if a else None
    out, lines = {}, []
    lines += [f"# Counters per dispatch: {shape}", "", "Commands (MI355X, one GPU, from the "
              "repository root), one counter group per run:", "```"] + cmds[1:] + ["```",
              f"HBM bytes: FETCH_SIZE x {scale['FETCH_SIZE']:.4f} + WRITE_SIZE x "
              f"{scale['WRITE_SIZE']:.4f} (KiB -> bytes, scaled so that the 256 MiB calibration "
              "copy in the same run reads its true size). MFMA flops executed: "
              "SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512. Trace us: the kernel trace's average.", "",
              "| launch | HBM bytes per dispatch | bf16 MFMA flops executed | trace us |",
              "|---|---|---|---|"]
    for nm, rec in sorted(per.items()):
        fb, wb = mean(rec.get("FETCH_SIZE", [])), mean(rec.get("WRITE_SIZE", []))
        mops = mean(rec.get("MOPS", []))
        o = {"sources": rec["sources"], "source_sha": run_sha[_group(rec["sources"])],
             "fetch_bytes": None if fb is None else round(fb),
             "write_bytes": None if wb is None else round(wb),
             "hbm_bytes": None if fb is None or wb is None else round(fb + wb),
             "mfma_bf16_flops": None if mops is None else round(mops * 512),
             "trace_us": durations.get(nm), "commands": cmds}
        out[nm] = o
        lines.append(f"| {nm} | {o['hbm_bytes']} | {o['mfma_bf16_flops']} | "
                     f"{'-' if o['trace_us'] is None else round(o['trace_us'], 2)} |")
    with open(os.path.join(ROOT, "profiles", f"counters_{shape}.json"), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    with open(os.path.join(ROOT, "profiles", f"counters_{shape}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(trace_rows + [""] + lines))


# ---------------------------------------------------------------------------------------
# GPU timing

class Prefill:
    """One prefill workload resident on the GPU, with its combined call."""

    def __init__(self, cfg, sy, ssd, torch, dev, gen):
        self.cfg, self.ssd, self.torch = cfg, ssd, torch
        inp = sy.make_prefill(cfg)
        c = cfg
        self.p = ssd.make_problem(c.total_tokens, c.num_seqs, c.nheads, c.headdim, c.d_state,
                                  c.ngroups, c.chunk_size, c.num_slots, c.in_dtype,
                                  c.state_dtype)
        self.args = [t.to(dev) for t in (inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D,
                                         inp.cu_seqlens)]
        self.cache = (torch.randn(c.num_slots, c.nheads, c.headdim, c.d_state, device=dev,
                                  generator=gen) * 0.03).to(c.state_dtype)
        self.idx = inp.state_indices.to(dev)
        self.hi = inp.has_initial.to(dev) if inp.has_initial is not None else None
        self.y = torch.empty(c.total_tokens, c.nheads, c.headdim, dtype=c.in_dtype, device=dev)
        self.ck = (torch.empty(ssd.max_chunks(self.p), c.nheads, c.headdim, c.d_state,
                               dtype=c.state_dtype, device=dev) if c.checkpoints else None)
        self.ws = ssd.alloc_workspace(self.p, dev)
        self.inp = inp

    def call(self, stream, opt=None):
        x, dt, A, B, C, D, cu = self.args
        if opt is None:
            self.ssd.ssd_combined_varlen(self.p, x, dt, A, B, C, D, cu, self.cache, self.idx,
                                         self.hi, self.y, self.ck, self.ws, stream)
        else:
            self.ssd.ssd_combined_varlen_ex(self.p, opt, x, dt, A, B, C, D, cu, self.cache,
                                            self.idx, self.hi, self.y, self.ck, self.ws, stream)


def pct(vals, q):
    import numpy as np
    return float(np.percentile(np.asarray(vals), q))


def time_cold(pf, stream, flush, warmup, steps, torch, write_flush=False):
    """Cache-flushed calls: the flush, then the call between two events.
    Returns (per-call us list, wall seconds of the timed loop)."""
    for _ in range(warmup):
        flush_caches(flush, write_flush)
        pf.call(stream)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        flush_caches(flush, write_flush)
        a.record(stream)
        pf.call(stream)
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) * 1e3 for a, b in evs], wall


def trace_cold(pf, stream, flush, steps, ssd, torch):
    """Cache-flushed calls with the library's per-launch events: mean us per launch."""
    tr = ssd.LaunchTrace()
    opt = ssd.make_options(trace=tr)
    acc, names = {}, None
    for _ in range(steps):
        flush_caches(flush)
        pf.call(stream, opt)
        torch.cuda.synchronize()
        d = tr.durations_us()
        names = [n for n, _ in d]
        for n, us in d:
            acc.setdefault(n, []).append(us)
    return names, {n: sum(v) / len(v) for n, v in acc.items()}


def launch_table(names, means, w: Work):
    out = {}
    for n in names:
        b, f = launch_bytes(n, w), launch_flops(n, w)
        us = means[n]
        out[n] = {"avg_us": round(us, 3), "bytes": b, "flops": f,
                  "GBps": None if b is None else round(b / (us * 1e-6) / 1e9, 1),
                  "hbm_frac": None if b is None else round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                  "mfma_frac": round(f / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4) if f else None}
    return out


def roofline_of(name, means, w: Work, shape):
    """The dominant launch's roofline: HBM on the scope document's per-kernel bytes
    (entering states counted in float32 for the chunk scan), the kernel's own
    algorithmic bytes beside it, its algorithmic flops against bf16 MFMA peak, and
    the counters committed for it."""
    us = means[name]
    own = launch_bytes(name, w)
    ref = launch_bytes(name, w, entering_bytes=4) if name.startswith("chunk_scan") else own
    flops = launch_flops(name, w)
    ctr = load_counters(shape, name)
    mfma = {"algorithmic_flops": flops,
            "algorithmic_frac": round(flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS}
    if ctr and ctr.get("mfma_bf16_flops"):
        mfma["executed_flops_counter"] = ctr["mfma_bf16_flops"]
        mfma["executed_frac"] = round(ctr["mfma_bf16_flops"] / (us * 1e-6) / 1e12
                                      / MFMA_BF16_PEAK_TFLOPS, 4)
    achieved = ref / (us * 1e-6) / 1e9
    if ctr and ctr.get("trace_us"):
        mfma["rocprof_kernel_us"] = round(ctr["trace_us"], 3)
    return {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": ctr["hbm_bytes"] if ctr else None, "bytes": ref, "avg_us": round(us, 3),
            "own_bytes": own, "own_frac": round(own / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "rocprof_kernel_us": None if not ctr else ctr.get("trace_us"),
            "mfma": mfma, "timing": "HIP start/end events of the kernel's own launch "
                                    "(hipExtLaunchKernelGGL) in cache-flushed calls, mean"}


def decode_only(args, sy, ssd, torch):
    """The MTP verify update (intermediate states kept) and the ReplaySSM verify with
    its cursor move, back to back, for their kernel trace and counters."""
    import dataclasses
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
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
    us = spin_avg_us(lambda: ssd.selective_state_update(up, dcache, didx, dx, ddt, dA, dB, dC,
                                                        dD, dy, inter, stream),
                     args.steps, stream, torch)
    W = 16
    rings = ssd.alloc_replay_rings(up, W, dev)
    acc_seq = [sy.make_decode(dataclasses.replace(dcfg, seed=dcfg.seed + 1000 * k))
               .num_accepted.to(dev) for k in range(args.steps + args.warmup)]
    for k in range(args.steps + args.warmup):
        ssd.ssd_replay_update(up, W, dcache, rings["ring_x"], rings["ring_dt"], rings["ring_B"],
                              rings["cursor"], didx, dx, ddt, dA, dB, dC, dD, dy, stream)
        ssd.ssd_replay_advance(up, W, rings["cursor"], didx, acc_seq[k], stream)
    torch.cuda.synchronize()
    print(json.dumps({"shape": "decode_c4", "selective_state_update_us": round(us, 3),
                      "steps": args.steps, "warmup": args.warmup,
                      "sources_sha": sources_sha()}), flush=True)


def shape_only(args, sy, ssd, torch):
    """The cache-flushed combined call alone on another prefill shape (plain and
    traced), for that shape's kernel trace and counters."""
    if args.shape == "decode_c4":
        decode_only(args, sy, ssd, torch)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    cfg = {"cached_continuation_32x32": sy.C2, "mixed_varlen_8seq_ckpt": sy.C3}[args.shape]
    gen = torch.Generator(device=dev).manual_seed(4)
    pf = Prefill(cfg, sy, ssd, torch, dev, gen)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    times, _ = time_cold(pf, stream, flush, args.warmup, args.steps, torch)
    names, means = trace_cold(pf, stream, flush, args.steps, ssd, torch)
    w = layer_work(cfg)
    med = pct(times, 50)
    print(json.dumps({"shape": args.shape, "tokens": cfg.total_tokens, "seqs": cfg.num_seqs,
                      "combined_us_median": round(med, 3),
                      "tokens_per_s": round(cfg.total_tokens / (med * 1e-6), 1),
                      "launches": launch_table(names, means, w), "steps": args.steps,
                      "warmup": args.warmup, "sources_sha": sources_sha()}), flush=True)


def calibration_copy(args, torch, dev):
    """One plain 256 MiB device copy (--copy-calibration): the counter runs scale
    FETCH_SIZE / WRITE_SIZE by what they read for it."""
    if args.copy_calibration:
        src = torch.empty(CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()


def spin_avg_us(fn, reps, stream, torch):
    """Average duration of back-to-back launches of fn between two events, all queued
    behind a spin kernel so that host call overhead does not show as idle time."""
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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(inp, Q, T):
    """The float64 oracle over the whole layer prefill, best of 3 runs on all the
    threads this process may use, and best of 3 on one thread."""
    import oracle
    xs, dts, Bs, Cs = (oracle.f64(t) for t in (inp.x, inp.dt, inp.B, inp.C))
    cu = inp.cu_seqlens.numpy()
    allowed = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, min(allowed, oracle.max_threads()))
    best = {}
    for n in (threads, 1):
        runs = []
        for _ in range(3):
            t1 = time.perf_counter()
            oracle.recurrence(xs, dts, inp.A, Bs, Cs, inp.D, cu, Q, nthreads=n)
            runs.append(time.perf_counter() - t1)
        best[n] = min(runs)
    return {"value": round(T / best[threads], 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "single_thread_value": round(T / best[1], 1),
            "nproc": os.cpu_count(), "threads_allowed": allowed, "cpu_model": cpu_model(),
            "sample": f"the whole layer prefill (4096 tokens x 80 heads, float64 recurrence), "
                      f"best of 3 runs: {best[threads]:.3f} s on {threads} threads, "
                      f"{best[1]:.3f} s on 1 thread"}


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles)
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
        calibration_copy(args, torch, torch.device("cuda:0"))
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device=dev).manual_seed(4)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    # ------------------------------------------------------------------ the layer prefill
    cfg = sy.C1
    pf = Prefill(cfg, sy, ssd, torch, dev, gen)
    T, Q = cfg.total_tokens, cfg.chunk_size
    torch.cuda.synchronize()
    torch.cuda.synchronize()                      # (one process: the barrier is this sync)
    times, wall = time_cold(pf, stream, flush, args.warmup, args.steps, torch)
    med = pct(times, 50)
    names, means = trace_cold(pf, stream, flush, args.steps, ssd, torch)
    w = layer_work(cfg, segments(cfg) if "chunk_scan_segmented" in names else 1)
    launches = launch_table(names, means, w)
    dom = max(names, key=lambda n: means[n])
    roofline = roofline_of(dom, means, w, "layer_L4096")

    warm = dirty = None
    if not args.headline_only:
        wus = spin_avg_us(lambda: pf.call(stream), max(args.steps, 50), stream, torch)
        warm = {"us_per_step": round(wus, 3), "tokens_per_s": round(T / (wus * 1e-6), 1)}
        dt_, _ = time_cold(pf, stream, flush, 3, args.steps, torch, write_flush=True)
        dirty = {"median_us": round(pct(dt_, 50), 3),
                 "tokens_per_s": round(T / (pct(dt_, 50) * 1e-6), 1),
                 "flush": "512 MiB write before each call (its dirty lines are written back "
                          "during the call)"}

    decode = replay = None
    others, extras = {}, {}
    if not args.headline_only:
        # -------------------------------------------------------------- other prefill shapes
        for cname, ocfg in (("cached_continuation_32x32", sy.C2),
                            ("mixed_varlen_8seq_ckpt", sy.C3)):
            opf = Prefill(ocfg, sy, ssd, torch, dev, gen)
            ot, _ = time_cold(opf, stream, flush, args.warmup, args.steps, torch)
            onames, omeans = trace_cold(opf, stream, flush, args.steps, ssd, torch)
            ow = layer_work(ocfg)
            omed = pct(ot, 50)
            state = next((n for n in onames if n.startswith("chunk_state_passing")), None)
            others[cname] = {
                "tokens": ocfg.total_tokens, "seqs": ocfg.num_seqs,
                "combined_us_median": round(omed, 3),
                "tokens_per_s": round(ocfg.total_tokens / (omed * 1e-6), 1),
                "launches": launch_table(onames, omeans, ow),
                "state_pass_kernel": state}
            if cname == "mixed_varlen_8seq_ckpt":
                pre = torch.tensor([ocfg.prefix_len if int(opf.inp.has_initial[s]) else 0
                                    for s in range(ocfg.num_seqs)], dtype=torch.int32,
                                   device=dev)
                ack = torch.empty(ssd.max_chunks_aligned(opf.p), ocfg.nheads, ocfg.headdim,
                                  ocfg.d_state, dtype=ocfg.state_dtype, device=dev)
                aws = ssd.alloc_workspace_aligned(opf.p, dev)
                x, dt, A, B, C, D, cu = opf.args
                al = spin_avg_us(lambda: ssd.ssd_combined_varlen_aligned(
                    opf.p, pre, x, dt, A, B, C, D, cu, opf.cache, opf.idx, opf.hi, opf.y, ack,
                    aws, stream), 50, stream, torch)
                others[cname]["aligned_combined_us_warm"] = round(al, 3)
                del ack, aws
            del opf

        # -------------------------------------------------------------- decode / MTP verify
        dcfg = sy.C4
        dd = sy.make_decode(dcfg)
        R, TT, DH, DP, DN, DG = (dcfg.num_reqs, dcfg.tokens_per_req, dcfg.nheads, dcfg.headdim,
                                 dcfg.d_state, dcfg.ngroups)
        up = ssd.make_ssu_problem(R, TT, DH, DP, DN, DG, dcfg.num_slots, dcfg.in_dtype,
                                  dcfg.state_dtype)
        dcache = (torch.randn(dcfg.num_slots, DH, DP, DN, device=dev, generator=gen) * 0.03
                  ).to(dcfg.state_dtype)
        dx, ddt, dA, dB, dC, dD = (t.to(dev) for t in (dd.x, dd.dt, dd.A, dd.B, dd.C, dd.D))
        didx = dd.state_indices.to(dev)
        dy = torch.empty(R, TT, DH, DP, dtype=dcfg.in_dtype, device=dev)
        inter = torch.empty(R, TT, DH, DP, DN, dtype=dcfg.state_dtype, device=dev)
        ssu_us = spin_avg_us(lambda: ssd.selective_state_update(up, dcache, didx, dx, ddt, dA, dB,
                                                                dC, dD, dy, inter, stream),
                             max(args.steps, 50), stream, torch)
        es = 2
        ssu_bytes = R * DH * DP * DN * es * (1 + TT) + R * TT * (2 * DH * DP + 2 * DG * DN + DH) * 2
        ctr = load_counters("decode_c4", "selective_state_update")
        decode = {"workload": "mtp_verify R=128 T=3 H=128 P=64 N=128 G=8 bf16 cache 512 slots",
                  "metric": "decode updates/s", "value": round(R * TT / (ssu_us * 1e-6), 1),
                  "unit": "updates/s", "avg_us": round(ssu_us, 3),
                  "roofline": {"kernel": "selective_state_update", "bound": "hbm",
                               "achieved": round(ssu_bytes / (ssu_us * 1e-6) / 1e9, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(ssu_bytes / (ssu_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                               "traffic": ctr["hbm_bytes"] if ctr else None,
                               "bytes": ssu_bytes}}

        # -------------------------------------------------------------- ReplaySSM decode
        # The same MTP verify workload without stored draft states: checkpoint + input
        # rings per slot (16 entries: up to 13 history tokens and one 3-token window).
        # One step = verify + cursor move, over a seeded sequence of accepted counts,
        # timed after enough steps that every request's history is in its steady cycle.
        import dataclasses
        W = 16
        rings = ssd.alloc_replay_rings(up, W, dev)
        rck = dcache.clone()
        nsteps = 24
        acc_seq = [sy.make_decode(dataclasses.replace(dcfg, seed=dcfg.seed + 1000 * k))
                   .num_accepted.to(dev) for k in range(nsteps)]
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
        rctr = load_counters("decode_c4", "replay_update")
        replay = {"workload": "mtp_verify_replayssm R=128 T=3 H=128 P=64 N=128 G=8 bf16, ring 16",
                  "metric": "decode updates/s", "value": round(R * TT / (replay_us * 1e-6), 1),
                  "unit": "updates/s", "avg_us_per_step": round(replay_us, 3),
                  "mean_history_tokens": round(hist_sum / (nsteps * R), 2),
                  "roofline": {"kernel": "replay_update + replay_advance", "bound": "hbm",
                               "achieved": round(replay_bytes / (replay_us * 1e-6) / 1e9, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(replay_bytes / (replay_us * 1e-6) / 1e9
                                             / HBM_PEAK_GBS, 4),
                               "bytes": replay_bytes,
                               "traffic": rctr["hbm_bytes"] if rctr else None}}
        del rings, rck

        # -------------------------------------------------------------- steps either side
        # (context): the layer's dt preprocessing fused into the layer call, the MTP verify
        # as a packed varlen batch (1-3 tokens per request), and fp16 states with Philox
        # stochastic rounding (the verify with per-token states, 5 rounds)
        x, dt, A, B, C, D, cu = pf.args
        bias = torch.from_numpy(pf.inp.dt_bias).float().to(dev)
        tf = ssd.make_dt_transform(bias, sy.DT_MIN, sy.DT_MAX)
        raw = pf.inp.dt_raw.to(dev)
        fused_us = spin_avg_us(lambda: ssd.ssd_combined_varlen_dt(
            pf.p, tf, x, raw, A, B, C, D, cu, pf.cache, pf.idx, None, pf.y, None, pf.ws, stream),
            50, stream, torch)
        extras["prefill_dt_fused_layer_warm"] = {"combined_us": round(fused_us, 3),
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
        var_us = spin_avg_us(lambda: ssd.selective_state_update_varlen(
            up, vcu, dcache, didx, vx, vdt, dA, vB, vC, dD, vy, vinter, stream=stream),
            50, stream, torch)
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
            us16 = spin_avg_us(lambda: ssd.selective_state_update_ex(
                up16, opt, c16, didx, dx, ddt, dA, dB, dC, dD, dy, i16, stream=stream),
                50, stream, torch)
            extras[f"decode_{name}"] = {"avg_us": round(us16, 3),
                                        "updates_per_s": round(R * TT / (us16 * 1e-6), 1)}
        del c16, i16, inter

    # achievable HBM bandwidth on this machine, for context: a plain 1 GiB device copy
    copy_gbps = None
    if not args.headline_only:
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
        copy_gbps = round(2 * (1 << 30) * 5 / (ca.elapsed_time(cb) * 1e-3) / 1e9, 1)
        del src, dst
    calibration_copy(args, torch, dev)

    cpu = None if args.no_cpu_baseline else cpu_baseline(pf.inp, Q, T)

    out = {
        "metric": "SSD prefill tokens/s per layer + decode updates/s; % MFMA / HBM roofline",
        "value": round(T / (med * 1e-6), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mamba2_ssd_prefill_L4096_H80_P64_N128_G1_Q256",
                   "seq_len": T, "num_seqs": cfg.num_seqs, "nheads": cfg.nheads,
                   "headdim": cfg.headdim, "d_state": cfg.d_state, "ngroups": cfg.ngroups,
                   "chunk_size": Q, "inputs": "bf16 x/B/C/dt, fp32 A/D/state",
                   "timing": "median of the cache-flushed calls (512 MiB read before each)",
                   "parallelism": "single GPU"},
        "cold_stats_us": {"median": round(med, 3), "mean": round(sum(times) / len(times), 3),
                          "p10": round(pct(times, 10), 3), "p90": round(pct(times, 90), 3),
                          "calls": len(times), "timed_loop_wall_s": round(wall, 4)},
        "roofline": roofline,
        "launches": launches,
        "warm": warm,
        "cold_after_write_flush": dirty,
        "hbm_copy_GBps": copy_gbps,
        "other_prefill_shapes": others,
        "decode": decode,
        "decode_replayssm": replay,
        "steps_either_side": extras,
        "cpu_baseline": cpu,
        "sources_sha": sources_sha(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
