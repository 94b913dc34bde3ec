#!/usr/bin/env python3
"""Benchmark of the KDA forward pass on one MI355X.

One step = one kda_chunk_fwd call (the whole chunkwise prefill path: L2 norm,
cumulative decay, A_kk + UT transform, A_qk, inter-chunk state update, output,
with the state carried on chip) over the long-prefill workload
B=1, H=96, T=65536, d_k=d_v=128 (bf16 q/k/v, fp32 g/beta/state), inputs
resident in HBM.  The decode step (kda_recurrent_step over N=256, H=96, 128
in-place steps) is timed separately and reported under "decode".

Prints ONE JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA fwd tokens/s (H=96,d=128,T=64K prefill) + decode step μs; % MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
B, T, H, D = 1, 65536, 96, 128
# algorithmic traffic per token-head: q, k, v, o in bf16 (4 * 2 * 128), g fp32 (4 * 128), beta fp32 (4)
BYTES_PER_TOKEN_HEAD = 2 * (2 * D + 2 * D) + 4 * D + 4
STATE_BYTES = 4 * D * D
# chunk-form flops per token-head (C = 64, d = 128, triangular-exact):
#   (C-1)d [A_kk] + (C+1)d [A_qk] + (C+1)(2d) [W, U] + (C+1)d [A_qk U~] + 6 d^2 [W S, Q S, K^T U~] + C^2/3 [UT]
C = 64
FLOPS_PER_TOKEN_HEAD = (C - 1) * D + (C + 1) * D + (C + 1) * 2 * D + (C + 1) * D + 6 * D * D + C * C / 3
DEC_N, DEC_H, DEC_STEPS = 256, 96, 128
DEC_BYTES_PER_CHAIN = 2 * 4 * D * D + 2 * 3 * D + 4 * D + 4 + 2 * D


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--cpu-sample-heads", type=int, default=96)
    p.add_argument("--cpu-sample-tokens", type=int, default=65536)
    return p.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_fwd_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, valid only
    for the kernel sources they were taken on."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def time_prefill(kda, torch, d, steps, warmup):
    stream = torch.cuda.current_stream()

    def call():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], o=d["o"], final_state=d["sT"],
                      workspace=d["ws"])

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = []
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        per.append((e0, e1))
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = ev0.elapsed_time(ev1)
    launches = [a.elapsed_time(b) for a, b in per]
    return total_ms, launches, wall


def time_decode(kda, torch, kda_inputs):
    w = kda_inputs.DECODE_WORKLOAD
    S0 = kda_inputs.decode_initial_state(w["seed"], DEC_N, DEC_H, D, w["s0_std"])
    state = torch.from_numpy(S0).cuda()
    del S0
    xs = []
    for s in range(8):  # 8 distinct seeded step inputs, cycled over the 128 steps
        x = kda_inputs.decode_step(w["seed"], s, DEC_N, DEC_H, D)
        xs.append(tuple(torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
                        if a.dtype == np.uint16 else torch.from_numpy(a).cuda()
                        for a in (x.q, x.k, x.v, x.g, x.beta)))
    o = torch.empty((DEC_N, DEC_H, D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    for s in range(4):
        kda.recurrent_step(*xs[s % 8], state, o=o)
    torch.cuda.synchronize()
    evs = []
    for s in range(DEC_STEPS):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kda.recurrent_step(*xs[s % 8], state, o=o)
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    med = float(np.median(us))
    bytes_step = DEC_BYTES_PER_CHAIN * DEC_N * DEC_H
    gbs = bytes_step / (med * 1e-6) / 1e9
    return {
        "workload": "decode N=256 H=96 d_k=d_v=128, bf16 q/k/v/o, fp32 g/beta/state in place, 128 steps",
        "us_per_step_median": med, "us_per_step_min": float(us.min()), "us_per_step_max": float(us.max()),
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": load_traffic("decode"),
                     "bytes_per_launch": bytes_step},
    }


def cpu_baseline(inp_full, heads, tokens):
    """The fp64 oracle on a bounded sample of the same workload, scaled to
    tokens/s of the full 96-head layer."""
    import oracle
    import kda_inputs
    sub = kda_inputs.PrefillInputs(
        B=1, T=tokens, H=heads, dk=D, dv=D, dtype="bf16",
        q=np.ascontiguousarray(inp_full.q[:, :tokens, :heads]), k=np.ascontiguousarray(inp_full.k[:, :tokens, :heads]),
        v=np.ascontiguousarray(inp_full.v[:, :tokens, :heads]), g=np.ascontiguousarray(inp_full.g[:, :tokens, :heads]),
        beta=np.ascontiguousarray(inp_full.beta[:, :tokens, :heads]),
        init_state=np.ascontiguousarray(inp_full.init_state[:, :heads]), cu_seqlens=None)
    threads = min(heads, os.cpu_count() or 1)
    t0 = time.perf_counter()
    oracle.forward(sub, threads=threads)
    dt = time.perf_counter() - t0
    token_heads_per_s = tokens * heads / dt
    return {"value": token_heads_per_s / H, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "first %d tokens x %d of 96 heads of the same workload (fp64 token recurrence, "
                      "OpenMP over heads); %.1f s wall; scaled to 96-head tokens/s" % (tokens, heads, dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    import kda_inputs
    import gated_delta_rule_fwd_amd as kda

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    kda.load()
    torch.manual_seed(0)

    inp = kda_inputs.workload("long_bf16")
    to = lambda a: (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
                    if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a)).cuda())
    d = {"q": to(inp.q), "k": to(inp.k), "v": to(inp.v), "g": to(inp.g), "beta": to(inp.beta),
         "s0": to(inp.init_state)}
    d["o"] = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    d["sT"] = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    # chunk-record workspace of the two-pass matrix-core path, allocated once
    d["ws"] = torch.empty(kda.workspace_bytes(B, T, H, D, D), dtype=torch.uint8, device="cuda")

    total_ms, launches, wall = time_prefill(kda, torch, d, args.steps, args.warmup)
    ms = total_ms / args.steps
    launch_ms = float(np.mean(launches))
    tokens_per_s = B * T / (ms * 1e-3)
    bytes_launch = BYTES_PER_TOKEN_HEAD * B * T * H + 2 * STATE_BYTES * B * H
    flops_launch = FLOPS_PER_TOKEN_HEAD * B * T * H
    gbs = bytes_launch / (launch_ms * 1e-3) / 1e9
    tfl = flops_launch / (launch_ms * 1e-3) / 1e12

    out = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "long prefill B=1 H=96 T=65536 d_k=d_v=128 (bf16 q/k/v/o, fp32 g/beta/state, "
                               "S0~N(0,0.02^2)), seed 2", "B": B, "T": T, "H": H, "d_k": D, "d_v": D, "chunk": C},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": load_traffic("chunk_fwd"), "bytes_per_launch": bytes_launch},
        "mfma": {"achieved_tflops_algorithmic": tfl, "peak_bf16_tflops": BF16_MFMA_PEAK_TFLOPS,
                 "frac": tfl / BF16_MFMA_PEAK_TFLOPS, "flops_per_launch": flops_launch},
        "launch_ms_mean": launch_ms, "launch_ms_min": float(np.min(launches)),
        "launch_ms_max": float(np.max(launches)), "wall_s_timed": wall,
    }
    del d
    torch.cuda.empty_cache()
    if not args.no_decode:
        out["decode"] = time_decode(kda, torch, kda_inputs)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_heads, args.cpu_sample_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
