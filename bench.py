#!/usr/bin/env python3
"""Benchmark of the speculative-sampling verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline]

One step = the whole verify of one batch: row statistics of every target and
draft row, the accept scan and the residual or bonus draw, inputs resident in
HBM.  --path two_call (default, the fastest path on MI355X) runs it as
spec_softmax_stats then spec_verify_sample on one stream; --path three_call as
spec_softmax_stats, spec_verify, spec_residual_sample; --path fused as one
spec_verify_fused launch.  W untimed steps, then K timed steps bracketed by
device synchronisation, with nothing else on the stream.  Prints one JSON
line on stdout; progress goes to stderr.

Reported:
  value          verified sequences per second (B / seconds per step)
  roofline       the dominant kernel (two_call, three_call: the stats kernel,
                 every logit once + stats written; fused: the fused kernel,
                 the whole step's compulsory bytes) / its mean duration, timed
                 with an event pair around it on its stream in K further steps
                 right after the timed region (events recorded between two
                 kernels add a few microseconds to a step, so they are kept
                 out of the timed region).  traffic is the HBM bytes per
                 launch that rocprofv3's FETCH_SIZE and WRITE_SIZE counters
                 measured for that kernel and workload, scaled by a plain copy
                 of known size, read from a "traffic-record" line under
                 profiles/; null when no record matches the current kernel
                 sources
  cpu_baseline   the fp64 CPU oracle on a bounded sample of the same input
                 bytes (host threads), sequences per second

    python bench.py --mode greedy|sample [--steps K] [--warmup W]

times the other two entry points on the same workload instead, with their own
JSON line: spec_greedy_verify (greedy mode; value = verified sequences/s) or
spec_sample on the workload's B*K draft rows (draft-side sampling; value =
tokens/s); roofline = the call's algorithmic bytes (every logit row it needs
read once) / its mean duration.

    python bench.py --mode ksweep [--ks 1,2,4,8,16]

the K trade-off of the pages' fig. 1 on synthetic rows: for each K, the
three-call verify at the workload's B, V, T and draft noise (fresh inputs per
K), its time per call and the mean tokens emitted per sequence; one JSON line
with a "sweep" list.

    python bench.py --pmc-summary DIR [--path P] [--workload W] [--command CMD]

turns rocprofv3 --pmc CSV output (DIR/fetch, DIR/write, DIR/fetch_copy,
DIR/write_copy: FETCH_SIZE and WRITE_SIZE of the bench, then of
--copy-calibration 1024) into the markdown summary kept under profiles/,
including the traffic-record line.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

from speculative_sampling_verification_softmax_amd import binding, synth

HBM_PEAK_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "speculative_sampling_verification_softmax_amd", "csrc")
COPY_MIB = 1024
METRIC = "verified seqs/sec + achieved HBM GB/s (% of peak), B=256 K=8 V=128256 bf16"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stats_bytes(wl: synth.Workload) -> int:
    """Algorithmic bytes of one spec_softmax_stats launch: every logit read
    once plus 8 bytes of stats written per row."""
    rows = wl.B * (2 * wl.K + 1)
    return rows * wl.V * wl.elt + rows * 8


def step_bytes(wl: synth.Workload) -> int:
    """Compulsory bytes of one whole step: logits once, stats written and read
    back, tokens, uniforms, outputs (residual re-reads are not counted)."""
    B, K = wl.B, wl.K
    rows = B * (2 * K + 1)
    return (rows * wl.V * wl.elt + 2 * rows * 8 + B * K * 4 + B * (K + 1) * 4
            + B * 4 + B * (K + 1) * 4 + B * K * 8 + B * 4)


def kernel_sources_hash() -> str:
    """sha256 over the kernel sources: a traffic record is valid only for the
    sources it was measured with."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if f.endswith((".hpp", ".hip", ".h")):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def find_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a matching traffic-record line in profiles/."""
    want = {"kernel": kernel, "workload": workload, "sources": kernel_sources_hash()}
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(f) as fh:
            for line in fh:
                if not line.startswith("traffic-record:"):
                    continue
                kv = dict(t.split("=", 1) for t in line.split()[1:] if "=" in t)
                if all(kv.get(k) == v for k, v in want.items()):
                    return float(kv["bytes"])
    return None


def _pmc_kernels(path: str) -> dict:
    """{kernel short name: [counter values per dispatch]} from one rocprofv3 --pmc CSV."""
    out = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            name = r["Kernel_Name"].replace("void ", "").split("(")[0]
            out.setdefault(name, []).append(float(r["Counter_Value"]))
    return out


def pmc_summary(d: str, path: str, workload: str, command: str) -> str:
    f = lambda sub: _pmc_kernels(os.path.join(d, sub, "run_counter_collection.csv"))
    # pass directories: fetch, write (the stats kernel, two or three calls); fetch_fused, ...
    suffix = "" if path in ("two_call", "three_call") else "_" + path
    fetch, write = f("fetch" + suffix), f("write" + suffix)
    copy_bytes = COPY_MIB << 20
    def calib(sub):  # mean counter of the calibration copies (torch's own copies are far smaller)
        v = [x for k, xs in f(sub).items() if "copyBuffer" in k for x in xs]
        big = [x for x in v if x > 0.9 * max(v)]
        return sum(big) / len(big)
    cf, cw = calib("fetch_copy"), calib("write_copy")
    kf = copy_bytes / (cf * 1024)
    kw = copy_bytes / (cw * 1024)
    wl = synth.WORKLOADS[workload]
    dom = "fused_kernel" if path == "fused" else "stats_kernel"
    alg = step_bytes(wl) if path == "fused" else stats_bytes(wl)
    lines = [f"# HBM traffic per launch: {path} path, {workload} workload "
             f"(B={wl.B}, K={wl.K}, V={wl.V}, {wl.dtype}, T={wl.T})", "",
             "Commands (one MI355X, from the repository root; each pass is a run of its own):", "",
             "```", command, "```", "",
             f"Calibration: a plain device copy of {COPY_MIB} MiB reads and writes "
             f"{copy_bytes} bytes; FETCH_SIZE reads {cf:.1f} KiB and "
             f"WRITE_SIZE {cw:.1f} KiB per dispatch, so bytes = "
             f"FETCH_SIZE x {kf:.4f} x 1024 and WRITE_SIZE x {kw:.4f} x 1024.", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read bytes | HBM write bytes |",
             "|---|---|---|---|---|---|"]
    rec = None
    for k in sorted(fetch):
        if "spec::" not in k:
            continue
        fa = sum(fetch[k]) / len(fetch[k])
        wa = sum(write.get(k, [0.0])) / max(len(write.get(k, [0.0])), 1)
        rb, wb = fa * 1024 * kf, wa * 1024 * kw
        lines.append(f"| `{k}` | {len(fetch[k])} | {fa:.1f} | {wa:.1f} | {rb:.4g} | {wb:.4g} |")
        if dom in k:
            rec = rb + wb
    lines += ["", f"Algorithmic bytes of one `{dom}` launch: {alg}."]
    if rec is not None:
        lines += [f"Measured HBM bytes per launch: {rec:.6g} ({rec / alg:.4f} of algorithmic).", "",
                  f"traffic-record: kernel={dom} workload={workload} sources={kernel_sources_hash()} "
                  f"bytes={rec:.0f}"]
    return "\n".join(lines) + "\n"


def trace_summary(d: str, command: str) -> str:
    """Markdown table of this library's kernels from rocprofv3 --kernel-trace --stats output."""
    f = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    rows = []
    with open(f[0]) as fh:
        for r in csv.DictReader(fh):
            if "spec::" in r["Name"]:
                rows.append((r["Name"].replace("void ", "").split("(")[0], int(r["Calls"]),
                             float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"])))
    lines = ["Command (one MI355X, from the repository root):", "", "```", command, "```", "",
             "| kernel | calls | average (ns) | min (ns) | max (ns) |", "|---|---|---|---|---|"]
    lines += [f"| `{n}` | {c} | {a:.0f} | {lo:.0f} | {hi:.0f} |" for n, c, a, lo, hi in rows]
    lines += ["", "Calls include the warm-up steps; torch's input generation kernels are left out.",
              f"Kernel sources: {kernel_sources_hash()}."]
    return "\n".join(lines) + "\n"


def cpu_baseline(inp: dict, wl: synth.Workload, max_seqs: int, min_cpu_s: float = 12.0) -> dict:
    """The oracle on the first max_seqs sequences of the batch, repeated until
    about min_cpu_s CPU-seconds (wall time x threads) have been spent."""
    import oracle
    n = min(wl.B, max_seqs)
    idx = torch.arange(n, device=inp["target"].device)
    sub = dict(target=inp["target"][idx], draft=inp["draft"][idx], tokens=inp["tokens"][idx],
               uniforms=inp["uniforms"][idx], T=inp["T"])
    host = synth.to_host_arrays(sub)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    T = float(np.float32(wl.T))
    reps, wall = 0, 0.0
    while reps == 0 or (wall * threads < min_cpu_s and reps < 200):
        t0 = time.perf_counter()
        oracle.verify(host["target"], host["draft"], host["tokens"], host["uniforms"], T,
                      nthreads=threads)
        wall += time.perf_counter() - t0
        reps += 1
    return {"value": n * reps / wall, "unit": "seqs/s", "cores": threads, "kind": "oracle",
            "sample": f"the first {n} of {wl.B} sequences of the same {wl.name} batch, verified "
                      f"{reps} times (fp64; {threads} OpenMP threads; {wall:.2f} s wall, "
                      f"{wall * threads:.1f} CPU-s)"}


def timed(step, steps: int, warmup: int, stream) -> tuple[float, float]:
    """(ms per step over the timed region, mean ms of the event pair that a
    step records around its main call).  The timed region holds `steps`
    steps and nothing else; the call's duration comes from `steps` further
    steps that record the pair."""
    torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, float(np.mean([a.elapsed_time(b) for a, b in evs]))


def repeat_cpu(fn, units: int, unit: str, threads: int, what: str, min_cpu_s: float = 12.0):
    reps, wall = 0, 0.0
    while reps == 0 or (wall * threads < min_cpu_s and reps < 200):
        t0 = time.perf_counter()
        fn()
        wall += time.perf_counter() - t0
        reps += 1
    return {"value": units * reps / wall, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{what}, {reps} times (fp64; {threads} OpenMP threads; {wall:.2f} s wall, "
                      f"{wall * threads:.1f} CPU-s)"}


def extra_mode(args, wl: synth.Workload, inp: dict, stream) -> dict:
    """--mode greedy / sample / filter / filtered: one JSON record for that entry point."""
    import oracle
    B, K, V = wl.B, wl.K, wl.V
    dev = inp["target"].device
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    if args.mode == "greedy":
        tgt, tok = inp["target"], inp["tokens"]
        am = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        nacc = torch.empty(B, dtype=torch.int32, device=dev)
        out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        ne = torch.empty(B, dtype=torch.int32, device=dev)

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            binding.greedy_verify(tgt, tok, am, nacc, out, ne, stream=stream)
            if ev is not None:
                ev[1].record(stream)
        ms, call_ms = timed(step, args.steps, args.warmup, stream)
        rows = B * (K + 1)
        alg = rows * V * wl.elt + rows * 4 + B * K * 4 + B * (K + 1) * 4 + 2 * B * 4
        units, unit, metric = B, "seqs/s", f"greedy verified seqs/sec, B={B} K={K} V={V} {wl.dtype}"
        kernel = "argmax_kernel + greedy_scan_kernel"
        host = synth.to_host_arrays(inp)
        cpu = None
        if args.cpu_seqs > 0:
            cpu = repeat_cpu(lambda: oracle.greedy_verify(host["target"], host["tokens"],
                                                          nthreads=threads),
                             B, "seqs/s", threads, f"the whole {wl.name} batch ({B} sequences)")
    elif args.mode == "filter":
        tgt, dft = inp["target"], inp["draft"]
        ft, fd = torch.empty_like(tgt), torch.empty_like(dft)
        tt = torch.empty(B * (K + 1), dtype=torch.float32, device=dev)
        td = torch.empty(B * K, dtype=torch.float32, device=dev)

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            binding.filter_rows(tgt, wl.T, args.top_k, args.top_p, out=ft, thresholds=tt,
                                stream=stream)
            binding.filter_rows(dft, wl.T, args.top_k, args.top_p, out=fd, thresholds=td,
                                stream=stream)
            if ev is not None:
                ev[1].record(stream)
        ms, call_ms = timed(step, args.steps, args.warmup, stream)
        R = B * (2 * K + 1)
        alg = 2 * R * V * wl.elt + R * 4  # each row read once and written once
        units, unit = B, "seqs/s"
        metric = (f"filtered seqs/sec (top-k {args.top_k}, top-p {args.top_p}, target and draft "
                  f"rows), B={B} K={K} V={V} {wl.dtype}")
        kernel = "filter_kernel x2"
        cpu = None
        if args.cpu_seqs > 0:
            n = min(B * K, 64)
            rows = dft.reshape(B * K, V)[:n].contiguous().cpu()
            lh = (rows.view(torch.int16).numpy().view(np.uint16) if rows.dtype == torch.bfloat16
                  else rows.numpy())
            T32, p32 = float(np.float32(wl.T)), float(np.float32(args.top_p))

            def cpu_rows():
                for r in range(n):
                    oracle.filter_threshold(lh[r], T32, top_k=args.top_k, top_p=p32)
            cpu = repeat_cpu(cpu_rows, n / (2 * K + 1), "seqs/s", 1,
                             f"thresholds of the first {n} draft rows (one thread), "
                             f"scaled to {2 * K + 1} rows per sequence")
    elif args.mode == "filtered":
        tgt, dft, tok, uni = inp["target"], inp["draft"], inp["tokens"], inp["uniforms"]
        ft, fd = torch.empty_like(tgt), torch.empty_like(dft)
        tt = torch.empty(B * (K + 1), dtype=torch.float32, device=dev)
        td = torch.empty(B * K, dtype=torch.float32, device=dev)
        st = torch.empty((B, K + 1, 2), dtype=torch.float32, device=dev)
        sd = torch.empty((B, K, 2), dtype=torch.float32, device=dev)
        nacc = torch.empty(B, dtype=torch.int32, device=dev)
        out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        ne = torch.empty(B, dtype=torch.int32, device=dev)

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            binding.filter_rows(tgt, wl.T, args.top_k, args.top_p, out=ft, thresholds=tt,
                                stats=st, stream=stream)
            binding.filter_rows(dft, wl.T, args.top_k, args.top_p, out=fd, thresholds=td,
                                stats=sd, stream=stream)
            binding.verify_sample(ft, fd, tok, uni, st, sd, wl.T, nacc, out, False, ne,
                                  stream=stream)
            if ev is not None:
                ev[1].record(stream)
        ms, call_ms = timed(step, args.steps, args.warmup, stream)
        R = B * (2 * K + 1)
        alg = 2 * R * V * wl.elt + R * 12  # rows read once and written once; thresholds, stats
        units, unit = B, "seqs/s"
        metric = (f"verified seqs/sec with top-k {args.top_k} and top-p {args.top_p} on both p "
                  f"and q (filter with stats, then spec_verify_sample), B={B} K={K} V={V} "
                  f"{wl.dtype}")
        kernel = "filter_kernel x2 + verify_draw_kernel"
        cpu = None
        if args.cpu_seqs > 0:
            n = min(B, 8)
            host = synth.to_host_arrays(inp)
            T32, p32 = float(np.float32(wl.T)), float(np.float32(args.top_p))
            cpu = repeat_cpu(lambda: oracle.verify_filtered(
                host["target"][:n], host["draft"][:n], host["tokens"][:n], host["uniforms"][:n],
                T32, top_k=args.top_k, top_p=p32, nthreads=threads), n, "seqs/s", threads,
                f"the first {n} of the {B} sequences (the thresholds on one thread, the verify "
                f"on all)")
    else:
        logits = inp["draft"]
        R = B * K
        g = torch.Generator(device=dev).manual_seed(args.seed + 1)
        u = (torch.randint(0, 1 << 24, (R,), generator=g, device=dev).to(torch.float64)
             * 2.0 ** -24).to(torch.float32)
        st = torch.empty((R, 2), dtype=torch.float32, device=dev)
        tk = torch.empty(R, dtype=torch.int32, device=dev)

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            binding.sample(logits, u, wl.T, st, tk, stream=stream)
            if ev is not None:
                ev[1].record(stream)
        ms, call_ms = timed(step, args.steps, args.warmup, stream)
        alg = R * V * wl.elt + R * 4 + R * 8 + R * 4
        units, unit = R, "tokens/s"
        metric = f"draft tokens sampled/sec, {R} rows of V={V} {wl.dtype}, T={wl.T}"
        kernel = "stats_kernel + sample_kernel"
        cpu = None
        if args.cpu_seqs > 0:
            n = min(R, 256)
            rows = logits.reshape(R, V)[:n].contiguous().cpu()
            lh = (rows.view(torch.int16).numpy().view(np.uint16) if rows.dtype == torch.bfloat16
                  else rows.numpy())
            uh = u[:n].cpu().numpy()
            T32 = float(np.float32(wl.T))
            cpu = repeat_cpu(lambda: oracle.sample_rows(lh, uh, T32, nthreads=threads), n,
                             "tokens/s", threads, f"the first {n} of the {R} draft rows")
    achieved = alg / (call_ms * 1e-3) / 1e9
    log(f"[bench] {args.mode}: {ms * 1e3:.1f} us/step, call {call_ms * 1e3:.1f} us")
    return {
        "metric": metric, "value": units / (ms * 1e-3), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32" if args.mode == "greedy" else "f64",
        "data": "synthetic",
        "config": {"workload": wl.name, "mode": args.mode, "B": B, "K": K, "V": V,
                   "logits": wl.dtype, "T": wl.T, "seed": args.seed},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None, "launch_us": call_ms * 1e3, "bytes_per_launch": alg},
        "cpu_baseline": cpu,
    }


def ksweep(args, base: synth.Workload) -> dict:
    """Verify time and emitted tokens per sequence as K varies (fig. 1 analogue)."""
    out = []
    stream = torch.cuda.current_stream()
    for K in [int(k) for k in args.ks.split(",")]:
        wl = synth.workload(base.name, K=K)
        inp = synth.make_inputs(wl, seed=args.seed, device="cuda")
        tgt, dft, tok, uni = inp["target"], inp["draft"], inp["tokens"], inp["uniforms"]
        B = wl.B
        ts = torch.empty((B, K + 1, 2), dtype=torch.float32, device="cuda")
        ds = torch.empty((B, K, 2), dtype=torch.float32, device="cuda")
        nacc = torch.empty(B, dtype=torch.int32, device="cuda")
        o = torch.empty((B, K + 1), dtype=torch.int32, device="cuda")
        pr = torch.empty((B, K, 2), dtype=torch.float32, device="cuda")
        ne = torch.empty(B, dtype=torch.int32, device="cuda")

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            binding.softmax_stats(tgt, dft, wl.T, ts, ds, stream=stream)
            binding.verify(tgt, dft, tok, uni, ts, ds, wl.T, nacc, o, pr, stream=stream)
            binding.residual_sample(tgt, dft, uni, ts, ds, nacc, wl.T, o, ne, stream=stream)
            if ev is not None:
                ev[1].record(stream)
        ms, _ = timed(step, args.steps, args.warmup, stream)
        emitted = float(ne.double().mean().item())
        out.append({"K": K, "us_per_call": ms * 1e3, "emitted_per_seq": emitted,
                    "emitted_tokens_per_s": B * emitted / (ms * 1e-3),
                    "GBps": step_bytes(wl) / (ms * 1e-3) / 1e9})
        log(f"[bench] K={K}: {ms * 1e3:.1f} us, {emitted:.3f} tokens/seq")
        del inp, tgt, dft
        torch.cuda.empty_cache()
    return {"metric": f"verify time and emitted tokens per sequence vs K, B={base.B} "
                      f"V={base.V} {base.dtype} T={base.T}",
            "unit": "per K", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "data": "synthetic", "config": {"workload": base.name, "mode": "ksweep"},
            "sweep": out}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="headline", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--mode", default="verify",
                    choices=["verify", "greedy", "sample", "filter", "filtered", "ksweep"],
                    help="verify (the headline step), time spec_greedy_verify / spec_sample, or "
                         "sweep K")
    ap.add_argument("--ks", default="1,2,3,4,6,8,12,16", help="K values for --mode ksweep")
    ap.add_argument("--top-k", type=int, default=50, help="top-k for --mode filter (0: off)")
    ap.add_argument("--top-p", type=float, default=0.9, help="nucleus top_p for --mode filter")
    ap.add_argument("--path", default="two_call", choices=["three_call", "two_call", "fused"],
                    help="three_call: spec_softmax_stats, spec_verify, spec_residual_sample; "
                         "two_call: spec_softmax_stats, spec_verify_sample; "
                         "fused: spec_verify_fused (one launch)")
    ap.add_argument("--cpu-seqs", type=int, default=256,
                    help="sequences in the CPU oracle sample (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times "
                         "(a known-size reference for HBM byte counters) and exit")
    ap.add_argument("--pmc-summary", default=None, metavar="DIR",
                    help="print the markdown summary of rocprofv3 --pmc output under DIR and exit")
    ap.add_argument("--trace-summary", default=None, metavar="DIR",
                    help="print the markdown table of rocprofv3 --kernel-trace --stats output "
                         "under DIR and exit")
    ap.add_argument("--command", default="", help="with --pmc-summary / --trace-summary: the "
                                                  "commands that made DIR")
    args = ap.parse_args()

    if args.pmc_summary:
        print(pmc_summary(args.pmc_summary, args.path, args.workload, args.command), end="")
        return 0
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.command), end="")
        return 0

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {n} bytes three times")
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the verify shards by sequence and needs "
              "no collective; multi-GPU runs are not part of this build", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        return 2

    binding.load()
    wl = synth.WORKLOADS[args.workload]
    if args.mode == "ksweep":
        print(json.dumps(ksweep(args, wl)), flush=True)
        return 0
    log(f"[bench] generating {wl.name}: B={wl.B} K={wl.K} V={wl.V} {wl.dtype} T={wl.T}")
    inp = synth.make_inputs(wl, seed=args.seed, device="cuda")
    tgt, dft, tok, uni, T = inp["target"], inp["draft"], inp["tokens"], inp["uniforms"], wl.T
    B, K = wl.B, wl.K
    dev = tgt.device
    ts = torch.empty((B, K + 1, 2), dtype=torch.float32, device=dev)
    ds = torch.empty((B, K, 2), dtype=torch.float32, device=dev)
    nacc = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    probs = torch.empty((B, K, 2), dtype=torch.float32, device=dev)
    nemit = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    if args.mode != "verify":
        print(json.dumps(extra_mode(args, wl, inp, stream)), flush=True)
        return 0

    ws = binding.new_workspace(B, K, wl.V, tgt.dtype, dev)

    def step_fused(ev=None):
        if ev is not None:
            ev[0].record(stream)
        binding.verify_fused(tgt, dft, tok, uni, T, ws, ts, ds, nacc, out, probs, nemit,
                             stream=stream)
        if ev is not None:
            ev[1].record(stream)

    def step_three(ev=None):
        if ev is not None:
            ev[0].record(stream)
        binding.softmax_stats(tgt, dft, T, ts, ds, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        binding.verify(tgt, dft, tok, uni, ts, ds, T, nacc, out, probs, stream=stream)
        binding.residual_sample(tgt, dft, uni, ts, ds, nacc, T, out, nemit, stream=stream)

    def step_two(ev=None):
        if ev is not None:
            ev[0].record(stream)
        binding.softmax_stats(tgt, dft, T, ts, ds, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        binding.verify_sample(tgt, dft, tok, uni, ts, ds, T, nacc, out, probs, nemit,
                              stream=stream)

    step = {"fused": step_fused, "two_call": step_two, "three_call": step_three}[args.path]

    log(f"[bench] warmup {args.warmup}, then {args.steps} timed steps")
    ms, dom_ms = timed(step, args.steps, args.warmup, stream)
    if args.path == "fused":
        dom_kernel, dom_bytes = "fused_kernel", step_bytes(wl)
    else:
        dom_kernel, dom_bytes = "stats_kernel", stats_bytes(wl)
    log(f"[bench] {args.path}: {ms * 1e3:.1f} us/step, {dom_kernel} {dom_ms * 1e3:.1f} us")

    seqs_per_s = B / (ms * 1e-3)
    gbps_step = step_bytes(wl) / (ms * 1e-3) / 1e9
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    hist = torch.bincount(nacc.clamp(min=0).long(), minlength=K + 1).cpu().tolist()

    cpu = None
    if args.cpu_seqs > 0:
        log(f"[bench] cpu_baseline: oracle on {min(B, args.cpu_seqs)} sequences")
        cpu = cpu_baseline(inp, wl, args.cpu_seqs)

    rec = {
        "metric": METRIC,
        "value": seqs_per_s,
        "unit": "seqs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "K": K, "V": wl.V, "logits": wl.dtype,
                   "T": wl.T, "seed": args.seed, "path": args.path},
        "draft_rows_per_s": B * K / (ms * 1e-3),
        "achieved_GBps": gbps_step,
        "pct_of_peak": 100.0 * gbps_step / HBM_PEAK_GBPS,
        "accepted_hist": hist,
        "roofline": {"bound": "hbm", "kernel": dom_kernel, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": find_traffic(dom_kernel, wl.name), "launch_us": dom_ms * 1e3,
                     "bytes_per_launch": dom_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
