"""CPU oracle for the KDA forward pass -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding)
never imports, links or calls anything here, and this package imports nothing
from the product path: the two share no code.

Contents
  * ``forward`` / ``forward_arrays``: the fp64 token-by-token recurrence in C
    (kda_oracle.c, OpenMP over independent (sequence, head) chains).  It is
    the plain definition of the method: decay, erase, write, then read
    ("Kimi K3 の KDA ..." page, section 1.2.1; "GDN, KDA の整理", sections
    "Kimi Delta Attention" and "Online learning").
  * ``decode_steps``: the same recurrence, one token per call, carrying the
    fp64 state between calls (the recurrent form that the chunkwise page
    assigns to decode: "Kimi K3 模型结构（2）", Q&A on train/prefill/decode).
  * ``gate_map`` / ``beta_from_logits`` / ``forward_gated`` / ``decode_gated``:
    the gate prologue of the gated entry points, g = -5 sigmoid(e^{A_h} (z +
    dt_bias)) and beta = sigmoid(logit), evaluated in fp64 ("Kimi K3 模型结构
    （2）", Q&A on the scaled sigmoid with g_min = -5; "Kimi K3 の KDA ..."
    section 1.2.1 on A_log, dt_bias and the in-kernel sigmoid of beta), then
    the recurrence above.
  * ``forward_signed``: the same recurrence with the decay given as a signed
    alpha in [-1, 1] and beta in [0, 2] (Complex KDA, "[논문리뷰] Complex KDA
    ..." page).
  * ``short_conv`` / ``conv_qkv`` / ``forward_conv`` / ``decode_conv``: the
    causal width-4 depthwise convolution + SiLU that produces q, k, v from
    their projections, with its 3-token conv state ("Kimi K3 の KDA ..."
    section 1.2.1; "GDN, KDA の整理" on the conv cache), then the recurrence.
  * ``out_norm``: the gated RMSNorm that follows the kernel in the model,
    o / sqrt(mean(o^2) + eps) * w * sigmoid(gate) per (token, head) row
    ("Kimi K3 の KDA ..." section 1.2.1, the output gate).
  * ``product_form``: a second, independently written NumPy formulation that
    builds each transition matrix (I - beta k k^T) Diag(alpha) explicitly
    ("Kimi K3 の KDA ..." section 2.3.5: the state map is the ordered product of
    per-token transitions).  Used for tiny brute-force checks.

Every function here is pinned by tests in tests/test_oracle_pins.py against
identities the pages state and textbook linear algebra; see each test's
docstring for the passage it follows.  The one-token helpers (decode_steps,
decode_gated, decode_conv) and the per-head channel layout of conv_qkv are
pinned by the per-token hand-off of the affine maps ("Kimi K3 の KDA ..."
sections 2.3.4.2 and 2.3.4.5) with several sequences and heads, against
per-chain computations written out separately.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

EPS = 1e-6  # inside the square root of the L2 norm (the pages give no value)


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (host only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                               "-std=c99", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        for f in (lib.kda_oracle_forward, lib.kda_oracle_forward_signed):
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_int] * 5 + [ctypes.c_int, P] + [P] * 5 + [P, ctypes.c_double,
                                                                             ctypes.c_double, ctypes.c_int,
                                                                             P, P, ctypes.c_int]
        lib.kda_oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return _load().kda_oracle_num_threads()


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def forward_arrays(q, k, v, g, beta, init_state=None, cu_seqlens=None, *, scale=1.0, eps=EPS,
                   normalize=True, want_o=True, threads=0, alpha_given=False):
    """Run the recurrence.  q, k, g: [B,T,H,dk]; v: [B,T,H,dv]; beta: [B,T,H]
    (all converted to fp32, which is exact for bf16 values); init_state
    [N,H,dk,dv] (converted to fp64).  With alpha_given, g holds the signed
    decay alpha itself (Complex KDA).  Returns (o fp64 [B,T,H,dv] or None,
    final_state fp64 [N,H,dk,dv])."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and g.shape == q.shape and v.shape == (B, T, H, dv)
    assert beta.shape == (B, T, H)
    cu = None
    N = B
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        N = len(cu) - 1
    s0 = None
    if init_state is not None:
        s0 = np.ascontiguousarray(init_state, dtype=np.float64)
        assert s0.shape == (N, H, dk, dv)
    o = np.empty((B, T, H, dv), dtype=np.float64) if want_o else None
    sT = np.empty((N, H, dk, dv), dtype=np.float64)
    fn = lib.kda_oracle_forward_signed if alpha_given else lib.kda_oracle_forward
    rc = fn(B, T, H, dk, dv, N, _ptr(cu), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), float(scale),
            float(eps), int(bool(normalize)), _ptr(o), _ptr(sT), int(threads))
    if rc != 0:
        raise ValueError("kda_oracle_forward rejected its arguments")
    return o, sT


def forward(inp, heads: Optional[slice] = None, *, scale=1.0, want_o=True, threads=0):
    """Oracle on a kda_inputs.PrefillInputs, optionally on a subset of heads."""
    s0 = inp.f32("init_state", heads) if inp.init_state is not None else None
    return forward_arrays(inp.f32("q", heads), inp.f32("k", heads), inp.f32("v", heads),
                          inp.g if heads is None else inp.g[:, :, heads],
                          inp.beta if heads is None else inp.beta[:, :, heads],
                          s0, inp.cu_seqlens, scale=scale, want_o=want_o, threads=threads)


def forward_signed(q, k, v, alpha, beta, init_state=None, cu_seqlens=None, **kw):
    """Complex KDA: the recurrence with signed per-channel decay alpha in
    [-1, 1] and beta in [0, 2] ("[논문리뷰] Complex KDA ..." page, Method:
    the transition stays (I - beta k^ k^T) Diag(alpha))."""
    return forward_arrays(q, k, v, alpha, beta, init_state, cu_seqlens, alpha_given=True, **kw)


def decode_steps(state, q, k, v, g, beta, *, scale=1.0, threads=0, alpha_given=False):
    """One recurrent step for every (n, h): q, k, g [N,H,dk]; v [N,H,dv];
    beta [N,H]; state fp64 [N,H,dk,dv].  Returns (o [N,H,dv], new state)."""
    N, H, dk = np.shape(q)
    dv = np.shape(v)[-1]
    o, sT = forward_arrays(np.reshape(q, (N, 1, H, dk)), np.reshape(k, (N, 1, H, dk)),
                           np.reshape(v, (N, 1, H, dv)), np.reshape(g, (N, 1, H, dk)),
                           np.reshape(beta, (N, 1, H)), state, scale=scale, threads=threads, alpha_given=alpha_given)
    return o[:, 0], sT


# ----------------------------------------------------------------------------
# Gate prologue
# ----------------------------------------------------------------------------
def sigmoid(x):
    """1 / (1 + e^-x) in fp64, written so that neither branch overflows."""
    x = np.asarray(x, np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gate_map(z, A_log, dt_bias=None):
    """Per-channel log-decay of the bounded map: g = g_min sigmoid(e^A x) with
    g_min = -5 and x the decay logit ("Kimi K3 模型结构（2）", Q&A: K3 replaces
    the unbounded negative softplus by a scaled sigmoid with g_min = -5, range
    (-5, 0)).  A = A_log[h] is the per-head log-scale and dt_bias[h, c] the
    per-(head, channel) bias ("Kimi K3 の KDA ..." section 1.2.1).  Reading:
    the bias is added to the logit before the scale, x = z + dt_bias.
    z: [..., H, d_k]; A_log: [H]; dt_bias: [H, d_k] or None.  fp64 result."""
    z = np.asarray(z, np.float64)
    x = z if dt_bias is None else z + np.asarray(dt_bias, np.float64)
    return -5.0 * sigmoid(np.exp(np.asarray(A_log, np.float64))[:, None] * x)


def beta_from_logits(b):
    """beta = sigmoid(logit) ("Kimi K3 の KDA ..." section 1.2.1: the per-head
    write strength goes through a sigmoid inside the kernel)."""
    return sigmoid(b)


def forward_gated(inp, heads: Optional[slice] = None, *, beta_logits=True, scale=1.0, want_o=True, threads=0):
    """Oracle on a kda_inputs.GatedPrefillInputs: the gate map in fp64, then
    the recurrence (which reads g and beta as fp32, one rounding each)."""
    hs = slice(None) if heads is None else heads
    g = gate_map(inp.f32("z")[:, :, hs], inp.A_log[hs], inp.dt_bias[hs])
    b = beta_from_logits(inp.beta_logits[:, :, hs]) if beta_logits else inp.beta_logits[:, :, hs]
    s0 = inp.init_state[:, hs] if inp.init_state is not None else None
    return forward_arrays(inp.f32("q")[:, :, hs], inp.f32("k")[:, :, hs], inp.f32("v")[:, :, hs], g, b, s0,
                          inp.cu_seqlens, scale=scale, want_o=want_o, threads=threads)


def decode_gated(state, q, k, v, z, A_log, dt_bias, beta_logits, *, scale=1.0, threads=0):
    """One gated decode step: gate map on z [N,H,d_k], sigmoid on the beta
    logits [N,H], then decode_steps."""
    return decode_steps(state, q, k, v, gate_map(z, A_log, dt_bias), beta_from_logits(beta_logits),
                        scale=scale, threads=threads)


# ----------------------------------------------------------------------------
# Short convolution prologue
# ----------------------------------------------------------------------------
CONV_WIDTH = 4


def silu(x):
    """x sigmoid(x) in fp64."""
    x = np.asarray(x, np.float64)
    return x * sigmoid(x)


def short_conv(x, w, init=None, cu_seqlens=None):
    """Causal depthwise convolution of width 4 along the token axis, then SiLU
    ("Kimi K3 の KDA ..." section 1.2.1: each channel is independent and mixes
    the current token with the 3 before it; the SiLU follows).  Reading: tap j
    of channel c multiplies the input 3 - j tokens back (w[:, 3] is the
    current token), no bias; inputs before a sequence's first token come from
    its conv state (the previous 3 inputs, oldest first; "GDN, KDA の整理",
    section on the conv cache) or are zero.  Sequences never see each other.

    x: [B, T, C]; w: [C, 4]; init: [N, 3, C] or None; cu_seqlens: [N+1] with
    B = 1, or None (then N = B).  Returns (y fp64 [B, T, C], final [N, 3, C]):
    the SiLU of the convolution, and each sequence's last 3 inputs (drawn from
    init where the sequence is shorter than 3).  Tokens outside every packed
    sequence get y = 0."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    B, T, C = x.shape
    assert w.shape == (C, CONV_WIDTH)
    if cu_seqlens is None:
        segs = [(b, 0, T) for b in range(B)]
    else:
        assert B == 1
        cu = np.asarray(cu_seqlens)
        segs = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    y = np.zeros_like(x)
    final = np.empty((len(segs), CONV_WIDTH - 1, C))
    for n, (b, t0, t1) in enumerate(segs):
        prev = np.zeros((CONV_WIDTH - 1, C)) if init is None else np.asarray(init[n], np.float64)
        xs = np.concatenate([prev, x[b, t0:t1]], axis=0)            # token t0 + i sits at row i + 3
        L = t1 - t0
        pre = np.zeros((L, C))
        for j in range(CONV_WIDTH):
            pre += w[:, j] * xs[j:j + L]                             # row i + j = token t0 + i - (3 - j)
        y[b, t0:t1] = silu(pre)
        final[n] = xs[L:L + CONV_WIDTH - 1]
    return y, final


def conv_qkv(q, k, v, weights, inits=None, cu_seqlens=None):
    """short_conv on q, k [B,T,H,d_k] and v [B,T,H,d_v], each over its H*d
    channels with its own weights ([H*d, 4]) and state ([N, 3, H*d] or None).
    Returns ((q, k, v) fp64 in the input shapes, (final_q, final_k, final_v))."""
    outs, finals = [], []
    for i, x in enumerate((q, k, v)):
        x = np.asarray(x, np.float64)
        B, T, H, d = x.shape
        y, f = short_conv(x.reshape(B, T, H * d), weights[i], None if inits is None else inits[i], cu_seqlens)
        outs.append(y.reshape(B, T, H, d))
        finals.append(f)
    return tuple(outs), tuple(finals)


def forward_conv(q, k, v, g, beta, weights, conv_inits=None, init_state=None, cu_seqlens=None, *,
                 alpha_given=False, **kw):
    """The recurrence on conv-SiLU'd q, k, v (the inputs the kernel sees in
    the model once the short convolutions have run).  The convolved values
    reach the C recurrence rounded once to fp32.  Returns (o, final_state,
    conv finals)."""
    (qc, kc, vc), finals = conv_qkv(q, k, v, weights, conv_inits, cu_seqlens)
    o, sT = forward_arrays(qc, kc, vc, g, beta, init_state, cu_seqlens, alpha_given=alpha_given, **kw)
    return o, sT, finals


def decode_conv(caches, weights, q, k, v):
    """One decode token per sequence through the three short convolutions:
    q, k [N,H,d_k], v [N,H,d_v]; caches: 3 arrays [N, 3, H*d] (or None for
    zeros).  Returns ((q, k, v) convolved, new caches)."""
    outs, news = [], []
    for i, x in enumerate((q, k, v)):
        x = np.asarray(x, np.float64)
        N, H, d = x.shape
        y, f = short_conv(x.reshape(N, 1, H * d), weights[i], None if caches is None else caches[i])
        outs.append(y.reshape(N, H, d))
        news.append(f)
    return tuple(outs), tuple(news)


# ----------------------------------------------------------------------------
# Output norm epilogue
# ----------------------------------------------------------------------------
def out_norm(o, gate, weight=None, eps=1e-5):
    """The gated RMSNorm applied to the kernel's output ("Kimi K3 の KDA ..."
    section 1.2.1: per head, RMSNorm over the head's value dimension, a
    sigmoid on the output gate, and the elementwise product; the norm comes
    before the gate).  For every (token, head) row over the last axis c:

        y_c = o_c / sqrt(mean_c' o_c'^2 + eps) * weight_c * sigmoid(gate_c)

    Reading: weight is the norm's per-channel gain [d_v], shared by all heads
    (None means ones); eps is the caller's (the pages give none).  fp64."""
    o = np.asarray(o, np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    y = o / np.sqrt(ms + eps)
    if weight is not None:
        y = y * np.asarray(weight, np.float64)
    return y * sigmoid(gate)


# ----------------------------------------------------------------------------
# Second formulation: explicit transition matrices (tiny sizes only)
# ----------------------------------------------------------------------------
def transition(alpha, beta, k):
    """(I - beta k k^T) Diag(alpha) for one token, general real alpha and beta
    (the signed-gate / beta in [0, 2] range of the Complex KDA pages is
    allowed here so the worked rotation example can pin this function)."""
    alpha = np.asarray(alpha, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = k.shape[0]
    return (np.eye(d) - beta * np.outer(k, k)) @ np.diag(alpha)


def product_form(q, k, v, g, beta, S0=None, *, scale=1.0, eps=EPS, alpha_given=False):
    """One chain, explicit matrices: S_t = M_t S_{t-1} + beta_t k^_t v_t^T with
    M_t = (I - beta_t k^_t k^_t^T) Diag(alpha_t), alpha_t = exp g_t (or g_t
    itself with alpha_given); o_t = scale * S_t^T q^_t.
    q, k, g: [T, dk]; v: [T, dv]; beta: [T].  Returns (o [T, dv], S_T)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        qh = q[t] / np.sqrt(q[t] @ q[t] + eps)
        kh = k[t] / np.sqrt(k[t] @ k[t] + eps)
        M = transition(g[t] if alpha_given else np.exp(g[t]), beta[t], kh)
        S = M @ S + beta[t] * np.outer(kh, v[t])
        o[t] = scale * (S.T @ qh)
    return o, S
