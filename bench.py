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
    p.add_argument("--no-extra", action="store_true", help="skip the mid/varlen prefill timings and the copy kernel")
    p.add_argument("--sweep", action="store_true",
                   help="instead of the headline: a context-length sweep T = 2K..64K at H=16, d=128 (bf16), "
                        "one JSON line with ms and tokens/s per length")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="write profiles/traffic.json from two rocprofv3 --pmc runs of this bench "
                        "(FETCH_SIZE, then WRITE_SIZE) and exit; needs no GPU")
    p.add_argument("--workload", choices=sorted(WORKLOAD_LINES),
                   help="instead of the headline: time only this workload (for per-workload profiler runs) "
                        "and print its line")
    p.add_argument("--oracle-table", action="store_true",
                   help="instead of the headline: time the fp64 oracle on bounded samples of the five workloads, "
                        "on all host cores and on one core; needs no GPU")
    p.add_argument("--workspace-gib", type=float, default=None,
                   help="with --workload: cap the prefill workspace at this many GiB (never below the least one; "
                        "below the full size the windowed order runs)")
    p.add_argument("--long-context", action="store_true",
                   help="instead of the headline: prefill at 16 heads, T = 256K, 1M, 4M tokens, in a 1 GiB "
                        "workspace (and the full one up to 1M), inputs drawn on the device; one JSON line")
    p.add_argument("--mfma-from", metavar="DIR",
                   help="summarise a rocprofv3 --pmc run with SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES and "
                        "GRBM_GUI_ACTIVE (MFMA-busy fraction per kernel) and exit; needs no GPU")
    return p.parse_args()


# --workload names -> the bench line they time
WORKLOAD_LINES = {"tiny": "tiny_f32", "mid": "mid_bf16", "long": "long_bf16", "varlen": "varlen_bf16",
                  "decode": "decode"}


# the sources each measured path is built from (kernels, their headers, the launch code; the build
# script is hashed with them)
KERNEL_SOURCES = {
    "chunk_fwd": ("kda_chunk_two_pass.hip", "kda_stage_plan.h", "kda_mfma.h", "kda_kernels.h", "kda_device.h",
                  "kda_abi.hip"),
    "decode": ("kda_decode.hip", "kda_kernels.h", "kda_device.h", "kda_abi.hip"),
}


def kernel_source_hash(kernel: str) -> str:
    """Hash of the sources a path is built from and of the build script (its
    compiler options change the kernels too)."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "gated_delta_rule_fwd_amd")
    for name in sorted(KERNEL_SOURCES[kernel]):
        with open(os.path.join(pkg, "csrc", name), "rb") as f:
            h.update(name.encode() + f.read())
    with open(os.path.join(pkg, "build.py"), "rb") as f:
        h.update(b"build.py" + f.read())
    return h.hexdigest()[:16]


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def load_traffic(kernel: str, path: str = TRAFFIC_JSON):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, valid only
    for the kernel sources they were taken on."""
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(kernel):
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


def _dev(torch, a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def time_decode(kda, torch, kda_inputs, norm=False):
    w = kda_inputs.DECODE_WORKLOAD
    S0 = kda_inputs.decode_initial_state(w["seed"], DEC_N, DEC_H, D, w["s0_std"])
    state = torch.from_numpy(S0).cuda()
    del S0
    xs = []
    for s in range(8):  # 8 distinct seeded step inputs, cycled over the 128 steps
        x = kda_inputs.decode_step(w["seed"], s, DEC_N, DEC_H, D)
        xs.append(tuple(_dev(torch, a) for a in (x.q, x.k, x.v, x.g, x.beta)))
    kws = [{}] * 8
    if norm:
        wt = _dev(torch, kda_inputs.norm_weight(w["seed"], D))
        kws = [dict(out_gate=_dev(torch, kda_inputs.make_out_gate(w["seed"] + s, (DEC_N, DEC_H, D))),
                    norm_weight=wt, norm_eps=1e-5) for s in range(8)]
    o = torch.empty((DEC_N, DEC_H, D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    for s in range(4):
        kda.recurrent_step(*xs[s % 8], state, o=o, **kws[s % 8])
    torch.cuda.synchronize()
    evs = []
    for s in range(DEC_STEPS):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kda.recurrent_step(*xs[s % 8], state, o=o, **kws[s % 8])
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    med = float(np.median(us))
    bytes_step = (DEC_BYTES_PER_CHAIN + (2 * D if norm else 0)) * DEC_N * DEC_H
    gbs = bytes_step / (med * 1e-6) / 1e9
    line = {
        "workload": "decode N=256 H=96 d_k=d_v=128, bf16 q/k/v/o, fp32 g/beta/state in place, 128 steps" +
                    (", output norm fused (bf16 gate logits, fp32 gain)" if norm else ""),
        "us_per_step_median": med, "us_per_step_min": float(us.min()), "us_per_step_max": float(us.max()),
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "bytes_per_launch": bytes_step},
    }
    if not norm:
        line["roofline"]["traffic"] = load_traffic("decode")
    return line


def time_decode_layer(kda, torch, kda_inputs):
    """The decode step of the whole layer core: raw q, k, v through the short
    convolution (caches advanced in place), the decay gate from bf16 z, beta
    from logits, and the output norm; N=256 H=96 d=128, 128 steps."""
    w = kda_inputs.DECODE_WORKLOAD
    S0 = kda_inputs.decode_initial_state(w["seed"], DEC_N, DEC_H, D, w["s0_std"])
    state = torch.from_numpy(S0).cuda()
    del S0
    A_log, dt_bias = kda_inputs.gate_params(w["seed"], DEC_H, D)
    A_log, dt_bias = _dev(torch, A_log), _dev(torch, dt_bias)
    cw = tuple(_dev(torch, x) for x in kda_inputs.conv_weights(w["seed"], DEC_H, D, D))
    caches = tuple(_dev(torch, x) for x in kda_inputs.conv_states(w["seed"], DEC_N, DEC_H, D, D))
    wt = _dev(torch, kda_inputs.norm_weight(w["seed"], D))
    xs = []
    for s in range(8):
        x = kda_inputs.gated_decode_step(w["seed"], s, DEC_N, DEC_H, D)
        gate = _dev(torch, kda_inputs.make_out_gate(w["seed"] + s, (DEC_N, DEC_H, D)))
        xs.append((_dev(torch, x.q), _dev(torch, x.k), _dev(torch, x.v), _dev(torch, x.z),
                   _dev(torch, x.beta_logits), gate))
    o = torch.empty((DEC_N, DEC_H, D), dtype=torch.bfloat16, device="cuda")

    def step(x):
        kda.recurrent_step_gated(x[0], x[1], x[2], x[3], A_log, x[4], state, dt_bias=dt_bias, beta_logits=True,
                                 out_gate=x[5], norm_weight=wt, conv_weights=cw, conv_state=caches, o=o)

    for s in range(4):
        step(xs[s % 8])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = []
    for s in range(DEC_STEPS):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step(xs[s % 8])
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    med = float(np.median(us))
    # state in and out (fp32), raw q, k, v, z and the gate (bf16), beta logit, o (bf16), the three conv
    # caches read and written (3 rows of H*d bf16 each)
    per_chain = 2 * 4 * D * D + 2 * (4 * D + D) + 4 + 2 * D + 2 * 3 * 3 * 2 * D
    bytes_step = per_chain * DEC_N * DEC_H
    gbs = bytes_step / (med * 1e-6) / 1e9
    return {"workload": "decode step of the layer core: short convolution (caches in place) + gate prologue + "
                        "output norm, N=256 H=96 d=128, 128 steps",
            "us_per_step_median": med, "us_per_step_min": float(us.min()), "us_per_step_max": float(us.max()),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "bytes_per_launch": bytes_step}}


def context_sweep(kda, torch, kda_inputs, heads=16, lengths=(2048, 4096, 8192, 16384, 32768, 65536), reps=10):
    """Prefill time per call over context lengths at 16 heads, d = 128 (the
    head count and dims of the throughput comparison on the Complex KDA
    review page; the chunkwise page compares kernels over 2K..64K tokens).
    Synthetic bf16 inputs drawn like the long-prefill workload."""
    rows = []
    for T_ in lengths:
        inp = kda_inputs.make_prefill(20 + T_ // 2048, 1, T_, heads, D, D, gate="k3", s0_std=0.02)
        d = {k: _dev(torch, getattr(inp, k)) for k in ("q", "k", "v", "g", "beta", "init_state")}
        o = torch.empty((1, T_, heads, D), dtype=torch.bfloat16, device="cuda")
        sT = torch.empty((1, heads, D, D), dtype=torch.float32, device="cuda")
        ws = torch.empty(kda.workspace_bytes(1, T_, heads, D, D), dtype=torch.uint8, device="cuda")
        call = lambda: kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["init_state"], o=o,
                                     final_state=sT, workspace=ws)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        ts = []
        stream = torch.cuda.current_stream()
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        med = float(np.median(ts))
        gbs = (BYTES_PER_TOKEN_HEAD * T_ * heads + 2 * STATE_BYTES * heads) / (med * 1e-3) / 1e9
        rows.append({"T": T_, "ms_median": med, "tokens_per_s": T_ / (med * 1e-3), "algorithmic_gbs": gbs})
        del d, o, sT, ws
    return {"sweep": "prefill B=1 H=%d d_k=d_v=128 bf16, synthetic; median of %d calls" % (heads, reps),
            "rows": rows}


def long_context(kda, torch, heads=16, lengths=(262144, 1048576, 4194304), ws_gib=1.0, full_up_to=1048576,
                 reps=3, seed=5):
    """Prefill time per call at long contexts in a bounded workspace (the
    windowed order: memory independent of T) and, up to full_up_to tokens,
    with the full workspace.  Inputs are drawn on the device with torch's
    seeded generator, from the distributions of the long-prefill workload
    (q, k, v ~ N(0, 1) in bf16; g = -5 sigmoid(e^A_h z), A_h ~ U(-1, 1),
    z ~ N(0, 1); beta = sigmoid(N(0, 1)); S0 ~ N(0, 0.02^2)); they serve
    timing only."""
    gen = torch.Generator(device="cuda")
    rows = []
    for T_ in lengths:
        gen.manual_seed(seed + T_)
        shape = (1, T_, heads, D)
        x = {}
        for name in ("q", "k", "v"):
            x[name] = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        A = torch.rand((heads,), generator=gen, device="cuda") * 2 - 1
        g = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
        g.mul_(torch.exp(A)[None, None, :, None]).sigmoid_().mul_(-5.0)
        beta = torch.randn((1, T_, heads), generator=gen, device="cuda").sigmoid_()
        s0 = torch.randn((1, heads, D, D), generator=gen, device="cuda") * 0.02
        o = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        sT = torch.empty((1, heads, D, D), dtype=torch.float32, device="cuda")
        full = kda.workspace_bytes(1, T_, heads, D, D)
        least = kda.min_workspace_bytes(1, T_, heads, D, D)
        row = {"T": T_, "H": heads, "full_workspace_bytes": full, "least_workspace_bytes": least}
        for label, nbytes in (("bounded", max(least, min(full, int(ws_gib * (1 << 30))))),
                              ("full", full if T_ <= full_up_to else None)):
            if nbytes is None:
                continue
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            call = lambda: kda.chunk_fwd(x["q"], x["k"], x["v"], g, beta, s0, o=o, final_state=sT, workspace=ws)
            ts = _time_calls(torch, call, reps, 1)
            med = float(np.median(ts))
            row[label] = {"workspace_bytes": nbytes, "ms_median": med, "tokens_per_s": T_ / (med * 1e-3)}
            del ws
            torch.cuda.empty_cache()
        rows.append(row)
        del x, g, beta, s0, o, sT
        torch.cuda.empty_cache()
    return {"long_context": "prefill B=1 H=%d d_k=d_v=128 bf16, inputs drawn on the device; median of %d calls; "
                            "bounded workspace %.2f GiB" % (heads, reps, ws_gib), "rows": rows}


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
    # one core: one head, the first 16384 tokens
    one = kda_inputs.PrefillInputs(
        B=1, T=16384, H=1, dk=D, dv=D, dtype="bf16", q=np.ascontiguousarray(sub.q[:, :16384, :1]),
        k=np.ascontiguousarray(sub.k[:, :16384, :1]), v=np.ascontiguousarray(sub.v[:, :16384, :1]),
        g=np.ascontiguousarray(sub.g[:, :16384, :1]), beta=np.ascontiguousarray(sub.beta[:, :16384, :1]),
        init_state=np.ascontiguousarray(sub.init_state[:, :1]), cu_seqlens=None)
    t1 = time.perf_counter()
    oracle.forward(one, threads=1)
    dt1 = time.perf_counter() - t1
    return {"value": token_heads_per_s / H, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "first %d tokens x %d of 96 heads of the same workload (fp64 token recurrence, "
                      "OpenMP over heads); %.1f s wall; scaled to 96-head tokens/s" % (tokens, heads, dt),
            "one_core_tokens_per_s": 16384 / dt1 / H,
            "one_core_sample": "first 16384 tokens of head 0, 1 thread, %.2f s; scaled to 96-head tokens/s" % dt1,
            "host": host_info()}


def host_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "sched_affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def cpu_decode_baseline(n_sample=32):
    """The fp64 oracle's decode step on the first n_sample of the 256
    sequences (all 96 heads), scaled to ms per full step."""
    import oracle
    import kda_inputs
    w = kda_inputs.DECODE_WORKLOAD
    S0 = kda_inputs.decode_initial_state(w["seed"], n_sample, DEC_H, D, w["s0_std"]).astype(np.float64)
    x = kda_inputs.decode_step(w["seed"], 0, n_sample, DEC_H, D)
    f = lambda a: kda_inputs.bf16_to_f32(a) if a.dtype == np.uint16 else a
    threads = os.cpu_count() or 1
    q, k, v = f(x.q), f(x.k), f(x.v)
    S1 = np.ascontiguousarray(S0[:4])
    q1, k1, v1, g1, b1 = (np.ascontiguousarray(a[:4]) for a in (q, k, v, x.g, x.beta))
    t0 = time.perf_counter()
    oracle.decode_steps(S0, q, k, v, x.g, x.beta, threads=threads)
    dt = time.perf_counter() - t0
    # one core: the first 4 sequences
    t1 = time.perf_counter()
    oracle.decode_steps(S1, q1, k1, v1, g1, b1, threads=1)
    dt1 = time.perf_counter() - t1
    return {"ms_per_step": dt * 1e3 * DEC_N / n_sample, "cores": threads, "kind": "oracle",
            "sample": "%d of 256 sequences x 96 heads, one step, %.2f s; scaled to the full step" % (n_sample, dt),
            "one_core_ms_per_step": dt1 * 1e3 * DEC_N / 4,
            "one_core_sample": "4 of 256 sequences x 96 heads, one step, 1 thread, %.3f s; scaled to the full step" % dt1}


def _counter_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def write_traffic(fetch_dir, write_dir, path: str = TRAFFIC_JSON):
    """HBM bytes per call of each path from rocprofv3 FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch).  Each counter is scaled by what it reads for the bench's
    own device-to-device copy of COPY_BYTES, whose true traffic is COPY_BYTES
    read + COPY_BYTES written."""
    groups = {"chunk_fwd": ("chunk_prep_kernel", "chunk_scan_kernel"), "decode": ("decode_step_kernel",)}
    copy_names = ("copyBuffer", "copy_kernel", "CopyBuffer")
    out = {}
    scale = {}
    per = {}
    for ctr, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == ctr]
        copy = [float(r["Counter_Value"]) * 1024 for r in rows if any(c in r["Kernel_Name"] for c in copy_names)]
        if not copy:
            raise SystemExit("no copy-kernel dispatch with %s under %s" % (ctr, d))
        scale[ctr] = COPY_BYTES / max(copy)   # the largest copy is the bench's calibration copy
        for key, names in groups.items():
            vals = [float(r["Counter_Value"]) * 1024 for r in rows if any(n in r["Kernel_Name"] for n in names)]
            if key == "chunk_fwd":
                # a staged call dispatches each kernel once per stage: count
                # calls by pass-1 workgroups, B * ceil(T/64) * H per call
                wgs = sum(int(r["Grid_Size"]) // int(r["Workgroup_Size"]) for r in rows
                          if "chunk_prep_kernel" in r["Kernel_Name"])
                ncalls = max(1, round(wgs / (B * ((T + 63) // 64) * H)))
            else:
                ncalls = max(1, sum(1 for r in rows if names[0] in r["Kernel_Name"]))
            per.setdefault(key, {})[ctr] = sum(vals) / ncalls
    for key, v in per.items():
        if "FETCH_SIZE" in v and "WRITE_SIZE" in v:
            rd = v["FETCH_SIZE"] * scale["FETCH_SIZE"]
            wr = v["WRITE_SIZE"] * scale["WRITE_SIZE"]
            out[key] = {"source_hash": kernel_source_hash(key), "hbm_bytes_per_launch": rd + wr, "read_bytes": rd,
                        "write_bytes": wr, "fetch_scale": scale["FETCH_SIZE"], "write_scale": scale["WRITE_SIZE"]}
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(out, indent=1, sort_keys=True))
    return out


COPY_BYTES = 1 << 30


def copy_bandwidth(torch):
    """Achievable HBM rate of a plain device-to-device copy of 1 GiB."""
    x = torch.ones(COPY_BYTES // 4, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        y.copy_(x)
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    del x, y
    torch.cuda.empty_cache()
    return {"bytes_moved": 2 * COPY_BYTES, "ms_median": ms, "gbs": 2 * COPY_BYTES / (ms * 1e-3) / 1e9}


def _graph_replay_ms(torch, call, ins, o, sets, reps, warm):
    """Median time of `call` replayed from HIP graphs, one per input set, each
    first checked bit for bit (o) against its eager call."""
    refs = []
    for i in range(sets):
        call(ins[i])
        torch.cuda.synchronize()
        refs.append(o.clone())
    gs = []
    for i in range(sets):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            call(ins[i])
        gs.append(gr)
    torch.cuda.synchronize()
    for i in range(sets):
        o.zero_()
        gs[i].replay()
        torch.cuda.synchronize()
        if not torch.equal(o, refs[i]):
            raise RuntimeError("the graph replay differs from the eager call")
    for i in range(warm):
        gs[i % sets].replay()
    torch.cuda.synchronize()
    ts = []
    for i in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gs[i % sets].replay()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def time_workload(kda, torch, kda_inputs, name, sets, reps=20, warm=5, ws_gib=None, graphs=False):
    """Median call time of one prefill workload; with several input sets the
    calls rotate over them (a 200 MB working set would otherwise stay in the
    256 MB Infinity Cache).  ws_gib caps the workspace (not below the least
    one the call accepts).  With graphs, the same calls are also captured
    into HIP graphs (one per input set, each checked bit for bit against its
    eager call) and timed as replays: the host's launch work then leaves the
    timed region, which matters for calls of a few hundred microseconds."""
    to = lambda a: (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
                    if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a)).cuda())
    ins = []
    for k in range(sets):
        inp = kda_inputs.workload(name, seed=kda_inputs.WORKLOADS[name]["seed"] + 100 * k)
        d = {f: to(getattr(inp, f)) for f in ("q", "k", "v", "g", "beta")}
        d["cu"] = to(inp.cu_seqlens) if inp.cu_seqlens is not None else None
        d["s0"] = to(inp.init_state) if inp.init_state is not None else None
        ins.append(d)
    tokens, H = inp.B * inp.T, inp.H
    n_seq = (inp.cu_seqlens.shape[0] - 1) if inp.cu_seqlens is not None else inp.B
    f32 = inp.dtype == "f32"
    o = torch.empty((inp.B, inp.T, H, inp.dv), dtype=torch.float32 if f32 else torch.bfloat16, device="cuda")
    sT = torch.empty((n_seq, H, inp.dk, inp.dv), dtype=torch.float32, device="cuda")
    wkw = dict(num_seqs=n_seq if d["cu"] is not None else 0, in_bf16=not f32, out_bf16=not f32)
    ws_bytes = kda.workspace_bytes(inp.B, inp.T, H, inp.dk, inp.dv, **wkw)
    if ws_gib is not None:
        ws_bytes = max(kda.min_workspace_bytes(inp.B, inp.T, H, inp.dk, inp.dv, **wkw),
                       min(ws_bytes, int(ws_gib * (1 << 30))))
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device="cuda")
    call = lambda d: kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], d["cu"], o=o,
                                   final_state=sT, workspace=ws)
    for i in range(warm):
        call(ins[i % sets])
    torch.cuda.synchronize()
    ts = []
    for i in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call(ins[i % sets])
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    graph_ms = None
    if graphs:
        try:
            graph_ms = _graph_replay_ms(torch, call, ins, o, sets, reps, warm)
        except Exception as exc:   # an extra figure: never lose the bench line over it
            graph_ms = "not measured: %s" % exc
    if f32:   # fp32 q, k, v, o (4 bytes each per channel), fp32 g, beta; d_k, d_v of the workload
        algo = (4 * (2 * inp.dk + 2 * inp.dv) + 4 * inp.dk + 4) * tokens * H + 2 * 4 * inp.dk * inp.dv * n_seq * H
    else:
        algo = BYTES_PER_TOKEN_HEAD * tokens * H + 2 * STATE_BYTES * n_seq * H
    del ins, o, sT, ws
    torch.cuda.empty_cache()
    extra = {} if graph_ms is None else {"graph_replay_ms_median": graph_ms}
    return {"tokens": tokens, "heads": H, "sequences": n_seq, "input_sets": sets, "workspace_bytes": ws_bytes,
            "ms_median": ms, **extra,
            "ms_min": float(np.min(ts)), "ms_max": float(np.max(ts)), "tokens_per_s": tokens / (ms * 1e-3),
            "algorithmic_gbs": algo / (ms * 1e-3) / 1e9, "hbm_frac": algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


# gated prefill: bf16 decay logits z replace fp32 g (2 d instead of 4 d bytes), beta as fp32 logits
BYTES_PER_TOKEN_HEAD_GATED = 2 * (2 * D + 2 * D) + 2 * D + 4
# ... plus the output norm's bf16 gate logits (the gain is d_v floats per call)
BYTES_PER_TOKEN_HEAD_LAYER = BYTES_PER_TOKEN_HEAD_GATED + 2 * D


def _time_calls(torch, call, reps, warm):
    """Per-call HIP-event times (ms) on torch's current stream, which the
    binding launches on."""
    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    return ts


def _line(workload, ts, algo):
    ms = float(np.median(ts))
    return {"workload": workload, "ms_median": ms, "ms_min": float(np.min(ts)), "ms_max": float(np.max(ts)),
            "tokens_per_s": B * T / (ms * 1e-3), "bytes_per_launch": algo,
            "roofline": {"bound": "hbm", "achieved": algo / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}


def time_gated(kda, torch, kda_inputs, reps=20, warm=5, norm=False, conv=False):
    """The headline shape through the gated entry point (gate map and beta
    sigmoid in the kernel), same seed as the headline workload; with norm,
    also the output norm at the store of o; with conv, also the short
    convolution of q, k, v at their load (the whole fused layer core)."""
    gi = kda_inputs.make_gated_prefill(2, B, T, H, D, D, s0_std=0.02)
    d = {f: _dev(torch, getattr(gi, f)) for f in ("q", "k", "v", "z", "A_log", "dt_bias", "beta_logits",
                                                  "init_state")}
    del gi
    kw = {}
    if norm:
        kw = dict(out_gate=_dev(torch, kda_inputs.make_out_gate(2, (B, T, H, D))),
                  norm_weight=_dev(torch, kda_inputs.norm_weight(2, D)), norm_eps=1e-5)
    if conv:
        kw["conv_weights"] = tuple(_dev(torch, w) for w in kda_inputs.conv_weights(2, H, D, D))
        kw["conv_init"] = tuple(_dev(torch, c) for c in kda_inputs.conv_states(2, B, H, D, D))
        kw["conv_final"] = tuple(torch.empty_like(c) for c in kw["conv_init"])
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    sT = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.workspace_bytes(B, T, H, D, D, flags=kda.FLAG_QK_L2NORM | (kda.FLAG_OUT_NORM if norm else 0)),
                     dtype=torch.uint8, device="cuda")
    call = lambda: kda.chunk_fwd_gated(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["beta_logits"], d["init_state"],
                                       dt_bias=d["dt_bias"], beta_logits=True, o=o, final_state=sT, workspace=ws, **kw)
    ts = _time_calls(torch, call, reps, warm)
    del d, o, sT, ws, kw
    torch.cuda.empty_cache()
    if conv:
        return _line("long prefill B=1 H=96 T=65536 d=128, the fused layer core: short convolution + SiLU of raw bf16 "
                     "q, k, v with conv states in and out, decay-gate prologue, output norm (seed 2)",
                     ts, BYTES_PER_TOKEN_HEAD_LAYER * B * T * H + 2 * STATE_BYTES * B * H + 4 * D +
                     2 * 3 * 3 * H * D * 2 + 3 * 4 * 4 * H * D)
    if norm:
        return _line("long prefill B=1 H=96 T=65536 d=128, gated entry point with the output norm: bf16 decay "
                     "logits z, A_log, dt_bias, beta logits, bf16 output-gate logits, fp32 gain (seed 2)",
                     ts, BYTES_PER_TOKEN_HEAD_LAYER * B * T * H + 2 * STATE_BYTES * B * H + 4 * D)
    return _line("long prefill B=1 H=96 T=65536 d=128 via the gated entry point: bf16 decay logits z, A_log, "
                 "dt_bias, beta logits (seed 2)", ts, BYTES_PER_TOKEN_HEAD_GATED * B * T * H + 2 * STATE_BYTES * B * H)


def time_conv(kda, torch, kda_inputs, reps=20, warm=5):
    """The headline workload with the short convolution fused (raw q, k, v;
    conv states in and out); g and beta as in the headline call."""
    inp = kda_inputs.workload("long_bf16")
    d = {f: _dev(torch, getattr(inp, f)) for f in ("q", "k", "v", "g", "beta", "init_state")}
    del inp
    ws_ = tuple(_dev(torch, w) for w in kda_inputs.conv_weights(2, H, D, D))
    ci = tuple(_dev(torch, c) for c in kda_inputs.conv_states(2, B, H, D, D))
    cf = tuple(torch.empty_like(c) for c in ci)
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    sT = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.workspace_bytes(B, T, H, D, D), dtype=torch.uint8, device="cuda")
    call = lambda: kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["init_state"], o=o, final_state=sT,
                                 workspace=ws, conv_weights=ws_, conv_init=ci, conv_final=cf)
    ts = _time_calls(torch, call, reps, warm)
    del d, o, sT, ws
    torch.cuda.empty_cache()
    return _line("long prefill B=1 H=96 T=65536 d=128 with the short convolution + SiLU fused at the load of raw "
                 "bf16 q, k, v (conv states in and out; seed 2)", ts,
                 BYTES_PER_TOKEN_HEAD * B * T * H + 2 * STATE_BYTES * B * H + 2 * 3 * 3 * H * D * 2 + 3 * 4 * 4 * H * D)


def time_signed(kda, torch, kda_inputs, reps=20, warm=5):
    """The headline shape as Complex KDA (KDA_FLAG_SIGNED_ALPHA): signed
    decay alpha (a quarter of the entries negative), beta in (0, 2)."""
    si = kda_inputs.make_signed_prefill(2, B, T, H, D, D, s0_std=0.02)
    d = {f: _dev(torch, getattr(si, f)) for f in ("q", "k", "v", "g", "beta", "init_state")}
    del si
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    sT = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.workspace_bytes(B, T, H, D, D), dtype=torch.uint8, device="cuda")
    call = lambda: kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["init_state"], signed_alpha=True,
                                 o=o, final_state=sT, workspace=ws)
    ts = _time_calls(torch, call, reps, warm)
    del d, o, sT, ws
    torch.cuda.empty_cache()
    return _line("long prefill B=1 H=96 T=65536 d=128 as Complex KDA: signed alpha (25 % negative, |alpha| >= e^-5), "
                 "beta in (0, 2) (seed 2)", ts, BYTES_PER_TOKEN_HEAD * B * T * H + 2 * STATE_BYTES * B * H)


def oracle_table():
    """The fp64 oracle (test infrastructure, untuned) timed on bounded samples
    of the five workloads, on all host cores (OpenMP over chains) and on one
    core, each scaled to the workload's unit.  CPU only."""
    import oracle
    import kda_inputs
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)

    def sub(inp, tokens, heads):
        return kda_inputs.PrefillInputs(
            B=1, T=tokens, H=heads, dk=inp.dk, dv=inp.dv, dtype=inp.dtype,
            q=np.ascontiguousarray(inp.q[:, :tokens, :heads]), k=np.ascontiguousarray(inp.k[:, :tokens, :heads]),
            v=np.ascontiguousarray(inp.v[:, :tokens, :heads]), g=np.ascontiguousarray(inp.g[:, :tokens, :heads]),
            beta=np.ascontiguousarray(inp.beta[:, :tokens, :heads]),
            init_state=None if inp.init_state is None else np.ascontiguousarray(inp.init_state[:1, :heads]),
            cu_seqlens=None)

    def run(inp, threads):
        t0 = time.perf_counter()
        oracle.forward(inp, threads=threads)
        return time.perf_counter() - t0

    rows = {}
    for name, key, heads_all, heads_one, tokens_one in (("tiny", "tiny_f32", 2, 1, 256), ("mid", "mid_bf16", 32, 1, 4096),
                                                        ("long", "long_bf16", 96, 1, 16384)):
        inp = kda_inputs.workload(key) if name != "long" else kda_inputs.workload(key, T=16384)
        T_all = inp.T
        dt = run(inp, min(cores, heads_all))
        dt1 = run(sub(inp, tokens_one, heads_one), 1)
        T_full = kda_inputs.WORKLOADS[key]["T"]
        rows[name] = {"tokens_per_s_all_cores": T_all * heads_all / dt / kda_inputs.WORKLOADS[key]["H"],
                      "sample_all_cores": "%d tokens x %d heads, %d threads, %.2f s" % (T_all, heads_all,
                                                                                         min(cores, heads_all), dt),
                      "tokens_per_s_one_core": tokens_one * heads_one / dt1 / kda_inputs.WORKLOADS[key]["H"],
                      "sample_one_core": "%d tokens x %d head, 1 thread, %.2f s" % (tokens_one, heads_one, dt1),
                      "full_workload_tokens": T_full}
    # varlen: every sequence, the first 8 of 32 heads on all cores; the first
    # 4096 tokens of sequence 0, one head, on one core
    vin = kda_inputs.workload("varlen_bf16")
    hs = slice(0, 8)
    t0 = time.perf_counter()
    oracle.forward(vin, hs, threads=min(cores, 8 * len(vin.cu_seqlens)))
    dt = time.perf_counter() - t0
    dt1 = run(sub(vin, 4096, 1), 1)
    tot = int(vin.cu_seqlens[-1])
    rows["varlen"] = {"tokens_per_s_all_cores": tot * 8 / dt / vin.H,
                      "sample_all_cores": "all %d tokens x 8 of 32 heads, %.2f s" % (tot, dt),
                      "tokens_per_s_one_core": 4096 / dt1 / vin.H,
                      "sample_one_core": "first 4096 tokens of sequence 0, 1 head, 1 thread, %.2f s" % dt1}
    dec = cpu_decode_baseline()
    rows["decode"] = {"ms_per_step_all_cores": dec["ms_per_step"], "sample_all_cores": dec["sample"],
                      "ms_per_step_one_core": dec["one_core_ms_per_step"], "sample_one_core": dec["one_core_sample"]}
    return {"oracle_table": rows, "cores": cores, "host": host_info(),
            "note": "fp64 token recurrence (C, OpenMP over chains); tokens/s scaled to the workload's head count"}


def mfma_summary(d):
    """MFMA-busy per kernel from one rocprofv3 --pmc run: SQ_VALU_MFMA_BUSY_CYCLES
    over (GRBM_GUI_ACTIVE / 8 XCDs) x 256 CUs x 4 SIMDs, summed over the
    dispatches of each kernel name."""
    import collections
    rows = _counter_rows(d)
    acc = collections.defaultdict(lambda: collections.Counter())
    for r in rows:
        name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        acc[name][r["Counter_Name"]] += float(r["Counter_Value"])
        acc[name]["_dispatch:" + r.get("Dispatch_Id", "")] = 1
    out = {}
    for name, c in acc.items():
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in c or not c.get("GRBM_GUI_ACTIVE"):
            continue
        cycles = c["GRBM_GUI_ACTIVE"] / 8.0
        out[name] = {"dispatches": sum(1 for k in c if k.startswith("_dispatch:")),
                     "mfma_busy_frac": c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * 256 * 4),
                     "sq_busy_cycles": c.get("SQ_BUSY_CYCLES"), "gpu_cycles_per_xcd": cycles}
    print(json.dumps(out, indent=1, sort_keys=True))
    return out


def main():
    args = parse()
    if args.traffic_from:
        write_traffic(*args.traffic_from)
        return
    if args.mfma_from:
        mfma_summary(args.mfma_from)
        return
    if args.oracle_table:
        print(json.dumps(oracle_table()), flush=True)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (--gpus %d requested)" % args.gpus,
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
    if args.sweep:
        print(json.dumps(context_sweep(kda, torch, kda_inputs)))
        return
    if args.long_context:
        print(json.dumps(long_context(kda, torch)))
        return
    if args.workload:
        name = WORKLOAD_LINES[args.workload]
        if name == "decode":
            line = time_decode(kda, torch, kda_inputs)
        else:
            sets = 2 if name == "mid_bf16" else 1
            line = dict(workload=name, **time_workload(kda, torch, kda_inputs, name, sets=sets, reps=args.steps,
                                                       warm=args.warmup, ws_gib=args.workspace_gib))
        print(json.dumps({"workload_line": args.workload, **line}), flush=True)
        return

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
        "launch_ms_mean": launch_ms, "launch_ms_median": float(np.median(launches)),
        "launch_ms_min": float(np.min(launches)), "launch_ms_max": float(np.max(launches)), "wall_s_timed": wall,
    }
    if not args.no_extra:
        # the same call in a 1 GiB workspace (the windowed order, overlapped on the context's stream)
        ws1 = torch.empty(max(kda.min_workspace_bytes(B, T, H, D, D), 1 << 30), dtype=torch.uint8, device="cuda")
        t1 = _time_calls(torch, lambda: kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["s0"], o=d["o"],
                                                      final_state=d["sT"], workspace=ws1), 10, 2)
        out["prefill_long_1gib_workspace"] = {"workspace_bytes": ws1.numel(), "ms_median": float(np.median(t1)),
                                              "tokens_per_s": B * T / (float(np.median(t1)) * 1e-3)}
        del ws1
    del d
    torch.cuda.empty_cache()
    if not args.no_decode:
        out["decode"] = time_decode(kda, torch, kda_inputs)
        if not args.no_extra:
            out["decode_out_norm"] = time_decode(kda, torch, kda_inputs, norm=True)
            out["decode_layer_core"] = time_decode_layer(kda, torch, kda_inputs)
    if not args.no_extra:
        out["prefill_tiny"] = dict(workload="B=1 H=2 T=256 d=64 fp32 (exact fp32 path), seed 0",
                                   **time_workload(kda, torch, kda_inputs, "tiny_f32", sets=1, graphs=True))
        out["prefill_mid"] = dict(workload="B=1 H=32 T=4096 d=128 bf16, seed 1; two input sets rotated",
                                  **time_workload(kda, torch, kda_inputs, "mid_bf16", sets=2, graphs=True))
        out["prefill_varlen"] = dict(workload="16 packed sequences, lengths U[512,16384] from seed 3, H=32 d=128 bf16",
                                     **time_workload(kda, torch, kda_inputs, "varlen_bf16", sets=1, graphs=True))
        out["prefill_gated"] = time_gated(kda, torch, kda_inputs)
        out["prefill_gated_out_norm"] = time_gated(kda, torch, kda_inputs, norm=True)
        out["prefill_layer_core"] = time_gated(kda, torch, kda_inputs, norm=True, conv=True)
        out["prefill_conv"] = time_conv(kda, torch, kda_inputs)
        out["prefill_complex_kda"] = time_signed(kda, torch, kda_inputs)
    # the copy also calibrates rocprofv3's FETCH_SIZE / WRITE_SIZE (see --traffic-from)
    out["copy_kernel"] = copy_bandwidth(torch)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_sample_heads, args.cpu_sample_tokens)
        if not args.no_decode:
            out["decode"]["cpu_baseline"] = cpu_decode_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
