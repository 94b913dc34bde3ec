"""Seeded synthetic inputs for the KDA forward pass (prefill and decode).

This module only draws random tensors and quantises them; it holds none of the
recurrence's arithmetic.  Both the GPU path's tests/benchmark and the CPU
oracle take their inputs from here, so they always see identical values.

Recipe (one reading of the workloads; the pages print no data):
  * Every tensor is drawn blockwise along the token (or decode-step) axis from
    ``numpy.random.default_rng([seed, tensor_id, block])`` (PCG64), so large
    tensors can be generated in parallel and any block regenerated alone.
  * q, k, v ~ N(0, 1), drawn in fp32, then rounded to bf16 with
    round-to-nearest-even for the bf16 workloads.
  * Log-decay gate g (natural log of the per-key-channel retention), in fp32:
      'sigmoid':  g = -5 * sigmoid(z)               z ~ N(0,1) per (t, h, channel)
      'k3':       g = -5 * sigmoid(exp(A_h) * z)    A_h ~ U(-1, 1) per head
      'slow':     g = -5 * sigmoid(z - 4)           long memory probe
    This is the bounded decay map of "Kimi K3 模型结构（2）" (Q&A on the decay
    function) used as a data recipe; kernels take g itself.
  * beta = sigmoid(N(0,1)) per (t, h), fp32.
  * Initial state S0 ~ N(0, std^2) fp32 (std 0.02 where a workload asks for it).
  * Varlen lengths: integers U[512, 16384] from default_rng(3).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

BLOCK_T = 4096  # tokens per independently seeded block
_TENSOR_ID = {"q": 1, "k": 2, "v": 3, "z": 4, "beta": 5, "s0": 6, "A": 7, "dt_bias": 8, "sign": 9,
              "out_gate": 10, "norm_w": 11, "conv_w": 12, "conv_s": 13}


# ----------------------------------------------------------------------------
# bf16 helpers (storage format only)
# ----------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exactly widened fp32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _sigmoid32(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32, copy=False)
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x))).astype(np.float32)


def _rng(seed: int, name: str, block: int) -> np.random.Generator:
    return np.random.default_rng([seed, _TENSOR_ID[name], block])


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------
# Prefill inputs
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class PrefillInputs:
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: str                      # 'f32' or 'bf16' (storage of q, k, v)
    q: np.ndarray                   # [B,T,H,dk]  float32, or uint16 bf16 bits
    k: np.ndarray                   # [B,T,H,dk]
    v: np.ndarray                   # [B,T,H,dv]
    g: np.ndarray                   # [B,T,H,dk]  float32
    beta: np.ndarray                # [B,T,H]     float32
    init_state: Optional[np.ndarray]  # [N,H,dk,dv] float32 or None (zeros)
    cu_seqlens: Optional[np.ndarray]  # [N+1] int32 or None (dense batch)
    seed: int = 0

    @property
    def num_seqs(self) -> int:
        return self.B if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    def f32(self, name: str, heads: Optional[slice] = None) -> np.ndarray:
        """A tensor widened exactly to fp32, optionally restricted to heads."""
        a = getattr(self, name)
        if heads is not None:
            if name == "init_state":
                a = a[:, heads]
            else:
                a = a[:, :, heads]
        if a.dtype == np.uint16:
            return bf16_to_f32(a)
        return np.ascontiguousarray(a, dtype=np.float32)


def _fill_blocked(out: np.ndarray, seed: int, name: str, draw, T: int) -> None:
    """Fill out[:, t0:t1] block by block (axis 1 = tokens) in parallel."""
    nblk = (T + BLOCK_T - 1) // BLOCK_T

    def job(b):
        t0, t1 = b * BLOCK_T, min(T, (b + 1) * BLOCK_T)
        shape = (out.shape[0], t1 - t0) + out.shape[2:]
        out[:, t0:t1] = draw(_rng(seed, name, b), shape, t0, t1)

    if nblk == 1:
        job(0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(job, range(nblk)))


def make_prefill(seed: int, B: int, T: int, H: int, dk: int, dv: int, *,
                 dtype: str = "bf16", gate: str = "k3", s0_std: float = 0.0,
                 host_l2norm: bool = False, lengths=None) -> PrefillInputs:
    """Draw one prefill workload.  With ``lengths`` the sequences are packed
    (B must be 1, T = sum(lengths)) and cu_seqlens is returned."""
    cu = None
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        assert B == 1
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        T = int(cu[-1])
    N = B if cu is None else len(cu) - 1

    def normal(rng, shape, t0, t1):
        return rng.standard_normal(shape, dtype=np.float32)

    store = np.float32 if dtype == "f32" else np.uint16
    qkv = {}
    for name, d in (("q", dk), ("k", dk), ("v", dv)):
        arr = np.empty((B, T, H, d), dtype=store)

        def draw(rng, shape, t0, t1, name=name):
            x = rng.standard_normal(shape, dtype=np.float32)
            if host_l2norm and name in ("q", "k"):
                x = x / np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True)).astype(np.float32)
            return x if dtype == "f32" else bf16_bits(x)

        _fill_blocked(arr, seed, name, draw, T)
        qkv[name] = arr

    A = _rng(seed, "A", 0).uniform(-1.0, 1.0, size=H).astype(np.float32)
    g = np.empty((B, T, H, dk), dtype=np.float32)

    def draw_g(rng, shape, t0, t1):
        z = rng.standard_normal(shape, dtype=np.float32)
        if gate == "sigmoid":
            x = z
        elif gate == "k3":
            x = np.exp(A)[None, None, :, None].astype(np.float32) * z
        elif gate == "slow":
            x = z - np.float32(4.0)
        else:
            raise ValueError(gate)
        return (np.float32(-5.0) * _sigmoid32(x)).astype(np.float32)

    _fill_blocked(g, seed, "z", draw_g, T)

    beta = np.empty((B, T, H), dtype=np.float32)
    _fill_blocked(beta, seed, "beta",
                  lambda rng, shape, t0, t1: _sigmoid32(rng.standard_normal(shape, dtype=np.float32)), T)

    s0 = None
    if s0_std > 0:
        s0 = (_rng(seed, "s0", 0).standard_normal((N, H, dk, dv), dtype=np.float32)
              * np.float32(s0_std)).astype(np.float32)
    return PrefillInputs(B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype, q=qkv["q"], k=qkv["k"],
                         v=qkv["v"], g=g, beta=beta, init_state=s0, cu_seqlens=cu, seed=seed)


def varlen_lengths(seed: int = 3, n: int = 16, lo: int = 512, hi: int = 16384) -> np.ndarray:
    """Sequence lengths, integers uniform on [lo, hi] inclusive."""
    return np.random.default_rng(seed).integers(lo, hi, size=n, endpoint=True).astype(np.int64)


# ----------------------------------------------------------------------------
# Named workloads
# ----------------------------------------------------------------------------
WORKLOADS = {
    "tiny_f32": dict(seed=0, B=1, T=256, H=2, dk=64, dv=64, dtype="f32", gate="sigmoid",
                     s0_std=0.0, host_l2norm=True),
    "mid_bf16": dict(seed=1, B=1, T=4096, H=32, dk=128, dv=128, dtype="bf16", gate="k3", s0_std=0.0),
    "long_bf16": dict(seed=2, B=1, T=65536, H=96, dk=128, dv=128, dtype="bf16", gate="k3", s0_std=0.02),
    "varlen_bf16": dict(seed=3, B=1, T=0, H=32, dk=128, dv=128, dtype="bf16", gate="k3", s0_std=0.0),
}
DECODE_WORKLOAD = dict(seed=4, N=256, H=96, d=128, steps=128, s0_std=0.02)


def workload(name: str, **over) -> PrefillInputs:
    p = dict(WORKLOADS[name])
    p.update(over)
    if name == "varlen_bf16" and "lengths" not in p:
        p["lengths"] = varlen_lengths()
    return make_prefill(**p)


# ----------------------------------------------------------------------------
# Decode inputs (one token per sequence per step)
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class DecodeStep:
    q: np.ndarray      # [N,H,d] uint16 bf16 bits (or float32)
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray      # [N,H,d] float32
    beta: np.ndarray   # [N,H] float32


def decode_gate_scale(seed: int, H: int) -> np.ndarray:
    return _rng(seed, "A", 0).uniform(-1.0, 1.0, size=H).astype(np.float32)


def decode_initial_state(seed: int, N: int, H: int, d: int, std: float = 0.02) -> np.ndarray:
    """S0 ~ N(0, std^2), [N,H,d,d] fp32, drawn per sequence block."""
    out = np.empty((N, H, d, d), dtype=np.float32)
    blk = 16

    def job(b):
        n0, n1 = b * blk, min(N, (b + 1) * blk)
        out[n0:n1] = (_rng(seed, "s0", b).standard_normal((n1 - n0, H, d, d), dtype=np.float32)
                      * np.float32(std))

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(job, range((N + blk - 1) // blk)))
    return out


def decode_step(seed: int, step: int, N: int, H: int, d: int, dtype: str = "bf16") -> DecodeStep:
    A = decode_gate_scale(seed, H)
    blk = 1_000_000 + step  # step-indexed blocks, disjoint from prefill blocks

    def qkv(name):
        x = _rng(seed, name, blk).standard_normal((N, H, d), dtype=np.float32)
        return x if dtype == "f32" else bf16_bits(x)

    z = _rng(seed, "z", blk).standard_normal((N, H, d), dtype=np.float32)
    g = (np.float32(-5.0) * _sigmoid32(np.exp(A)[None, :, None].astype(np.float32) * z)).astype(np.float32)
    beta = _sigmoid32(_rng(seed, "beta", blk).standard_normal((N, H), dtype=np.float32))
    return DecodeStep(q=qkv("q"), k=qkv("k"), v=qkv("v"), g=g, beta=beta)


# ----------------------------------------------------------------------------
# Raw gate inputs (decay logits z, A_log, dt_bias, beta logits) for the gated
# entry points.  These are draws only: the gate map itself is applied by the
# code under test and by the oracle.
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class GatedPrefillInputs:
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: str
    q: np.ndarray                   # [B,T,H,dk] (bf16 bits or float32)
    k: np.ndarray
    v: np.ndarray
    z: np.ndarray                   # [B,T,H,dk] decay logits, same storage as q
    A_log: np.ndarray               # [H] float32
    dt_bias: np.ndarray             # [H,dk] float32
    beta_logits: np.ndarray         # [B,T,H] float32
    init_state: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]

    def f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return bf16_to_f32(a) if a.dtype == np.uint16 else a


def make_gated_prefill(seed: int, B: int, T: int, H: int, dk: int, dv: int, *, dtype: str = "bf16",
                       s0_std: float = 0.0, lengths=None, bias_std: float = 0.5) -> GatedPrefillInputs:
    """q, k, v, S0 and the packing as make_prefill (same streams); z ~ N(0,1)
    stored like q; A_log ~ U(-1, 1) per head; dt_bias ~ N(0, bias_std^2) per
    (head, channel); beta logits ~ N(0,1)."""
    base = make_prefill(seed, B, T, H, dk, dv, dtype=dtype, gate="sigmoid", s0_std=s0_std, lengths=lengths)
    T = base.T
    store = np.float32 if dtype == "f32" else np.uint16
    z = np.empty((B, T, H, dk), dtype=store)
    _fill_blocked(z, seed, "z", lambda rng, shape, t0, t1: (
        lambda x: x if dtype == "f32" else bf16_bits(x))(rng.standard_normal(shape, dtype=np.float32)), T)
    A_log = _rng(seed, "A", 0).uniform(-1.0, 1.0, size=H).astype(np.float32)
    dt_bias = (_rng(seed, "dt_bias", 0).standard_normal((H, dk), dtype=np.float32)
               * np.float32(bias_std)).astype(np.float32)
    bl = np.empty((B, T, H), dtype=np.float32)
    _fill_blocked(bl, seed, "beta", lambda rng, shape, t0, t1: rng.standard_normal(shape, dtype=np.float32), T)
    return GatedPrefillInputs(B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype, q=base.q, k=base.k, v=base.v, z=z,
                              A_log=A_log, dt_bias=dt_bias, beta_logits=bl, init_state=base.init_state,
                              cu_seqlens=base.cu_seqlens)


@dataclasses.dataclass
class GatedDecodeStep:
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    z: np.ndarray           # [N,H,d] decay logits, same storage as q
    beta_logits: np.ndarray  # [N,H] float32


def gated_decode_step(seed: int, step: int, N: int, H: int, d: int, dtype: str = "bf16") -> GatedDecodeStep:
    blk = 1_000_000 + step

    def draw(name, shape):
        x = _rng(seed, name, blk).standard_normal(shape, dtype=np.float32)
        return x if dtype == "f32" else bf16_bits(x)

    return GatedDecodeStep(q=draw("q", (N, H, d)), k=draw("k", (N, H, d)), v=draw("v", (N, H, d)),
                           z=draw("z", (N, H, d)),
                           beta_logits=_rng(seed, "beta", blk).standard_normal((N, H), dtype=np.float32))


def gate_params(seed: int, H: int, d: int, bias_std: float = 0.5):
    """A_log [H] ~ U(-1, 1) and dt_bias [H,d] ~ N(0, bias_std^2)."""
    A_log = _rng(seed, "A", 0).uniform(-1.0, 1.0, size=H).astype(np.float32)
    dt_bias = (_rng(seed, "dt_bias", 0).standard_normal((H, d), dtype=np.float32)
               * np.float32(bias_std)).astype(np.float32)
    return A_log, dt_bias


# ----------------------------------------------------------------------------
# Complex KDA inputs: signed decay alpha and beta in (0, 2)
# ----------------------------------------------------------------------------
def make_signed_prefill(seed: int, B: int, T: int, H: int, dk: int, dv: int, *, dtype: str = "bf16",
                        s0_std: float = 0.0, lengths=None, p_negative: float = 0.25) -> PrefillInputs:
    """As make_prefill (same streams), then the decay is given as a signed
    alpha: |alpha| = e^g with g from the bounded map (so |alpha| >= e^-5) and
    a negative sign with probability p_negative per (token, head, channel);
    beta = 2 sigmoid(N(0,1)) in (0, 2).  Returned in the g and beta fields."""
    base = make_prefill(seed, B, T, H, dk, dv, dtype=dtype, gate="k3", s0_std=s0_std, lengths=lengths)
    T = base.T
    alpha = np.exp(base.g).astype(np.float32)
    neg = np.empty(alpha.shape, dtype=bool)
    _fill_blocked(neg, seed, "sign", lambda rng, shape, t0, t1: rng.uniform(size=shape) < p_negative, T)
    alpha[neg] = -alpha[neg]
    base.g = alpha
    base.beta = (np.float32(2.0) * base.beta).astype(np.float32)
    return base


def signed_decode_step(seed: int, step: int, N: int, H: int, d: int, dtype: str = "bf16",
                       p_negative: float = 0.25) -> DecodeStep:
    """decode_step with the decay given as signed alpha and beta in (0, 2)."""
    x = decode_step(seed, step, N, H, d, dtype)
    alpha = np.exp(x.g).astype(np.float32)
    neg = _rng(seed, "sign", 1_000_000 + step).uniform(size=alpha.shape) < p_negative
    alpha[neg] = -alpha[neg]
    return DecodeStep(q=x.q, k=x.k, v=x.v, g=alpha, beta=(np.float32(2.0) * x.beta).astype(np.float32))


# ----------------------------------------------------------------------------
# Output-norm inputs: the output-gate logits and the norm's per-channel gain
# ----------------------------------------------------------------------------
def make_out_gate(seed: int, shape, dtype: str = "bf16") -> np.ndarray:
    """Output-gate logits ~ N(0, 1) of the shape of o ([B,T,H,d_v] or
    [N,H,d_v]), bf16 bits or fp32; drawn in token blocks like q, k, v."""
    out = np.empty(tuple(shape), np.float32)
    if len(shape) == 4:
        _fill_blocked(out, seed, "out_gate",
                      lambda rng, shp, t0, t1: rng.standard_normal(shp, dtype=np.float32), shape[1])
    else:
        out[:] = _rng(seed, "out_gate", 0).standard_normal(out.shape, dtype=np.float32)
    return bf16_bits(out) if dtype == "bf16" else out


def norm_weight(seed: int, dv: int) -> np.ndarray:
    """The norm's per-channel gain [d_v] ~ U(0.5, 1.5), fp32."""
    return _rng(seed, "norm_w", 0).uniform(0.5, 1.5, size=dv).astype(np.float32)


# ----------------------------------------------------------------------------
# Short-convolution inputs: per-channel taps and the 3-token conv state
# ----------------------------------------------------------------------------
def conv_weights(seed: int, H: int, dk: int, dv: int, std: float = 0.5):
    """Taps of the q, k and v convolutions, [H*d, 4] fp32 each ~ N(0, std^2)
    (oldest token first)."""
    rng = _rng(seed, "conv_w", 0)
    return tuple((rng.standard_normal((H * d, 4), dtype=np.float32) * np.float32(std)).astype(np.float32)
                 for d in (dk, dk, dv))


def conv_states(seed: int, N: int, H: int, dk: int, dv: int, dtype: str = "bf16"):
    """Conv states of q, k and v, [N, 3, H*d] ~ N(0, 1) (the 3 previous raw
    inputs of each sequence), bf16 bits or fp32."""
    rng = _rng(seed, "conv_s", 0)
    out = []
    for d in (dk, dk, dv):
        x = rng.standard_normal((N, 3, H * d), dtype=np.float32)
        out.append(bf16_bits(x) if dtype == "bf16" else x)
    return tuple(out)
