#!/usr/bin/env python3
"""Benchmark of the speculative-sampling verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline]

One step = the whole verify of one batch: row statistics of every target and
draft row, the accept scan and the residual or bonus draw, inputs resident in
HBM.  --path three_call (default, the faster path on MI355X) runs it as
spec_softmax_stats, spec_verify, spec_residual_sample back to back on one
stream; --path fused as one spec_verify_fused launch.  W untimed steps, then K timed steps bracketed by device
synchronisation.  Prints one JSON line on stdout; progress goes to stderr.

Reported:
  value          verified sequences per second (B / seconds per step)
  roofline       the dominant kernel (fused: the fused kernel, algorithmic
                 bytes = the whole step's compulsory bytes; three_call: the
                 stats kernel, every logit once + stats written) / its mean
                 duration, timed with events on its stream in the timed region
  cpu_baseline   the fp64 CPU oracle on the same input bytes (whole batch,
                 all host threads), sequences per second
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

from speculative_sampling_verification_softmax_amd import binding, synth

HBM_PEAK_GBPS = 8000.0
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


def cpu_baseline(inp: dict, wl: synth.Workload, max_seqs: int) -> dict:
    import oracle
    n = min(wl.B, max_seqs)
    idx = torch.arange(n, device=inp["target"].device)
    sub = dict(target=inp["target"][idx], draft=inp["draft"][idx], tokens=inp["tokens"][idx],
               uniforms=inp["uniforms"][idx], T=inp["T"])
    host = synth.to_host_arrays(sub)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    T = float(np.float32(wl.T))
    t0 = time.perf_counter()
    oracle.verify(host["target"], host["draft"], host["tokens"], host["uniforms"], T,
                  nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "seqs/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {wl.B} sequences of the same {wl.name} batch "
                      f"(fp64, {threads} OpenMP threads, {dt:.2f} s wall)"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="headline", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--path", default="three_call", choices=["three_call", "fused"],
                    help="fused: spec_verify_fused (one launch); three_call: spec_softmax_stats, "
                         "spec_verify, spec_residual_sample")
    ap.add_argument("--cpu-seqs", type=int, default=256,
                    help="sequences in the CPU oracle sample (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times "
                         "(a known-size reference for HBM byte counters) and exit")
    args = ap.parse_args()

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

    step = step_fused if args.path == "fused" else step_three

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms = total_ms / args.steps
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
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
                     "traffic": None, "launch_us": dom_ms * 1e3,
                     "bytes_per_launch": dom_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
