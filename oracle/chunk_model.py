"""Chunkwise form of the KDA recurrence, in NumPy -- TEST INFRASTRUCTURE ONLY.

This is not the oracle's definition (that is the token recurrence in
kda_oracle.c); it is the chunk algebra the GPU design follows, written out
plainly so a test can check it against the token oracle, and so each matrix
product can be evaluated at a chosen precision to budget the GPU kernels'
arithmetic.  It shares no code with the HIP path.

For one chunk of L <= C tokens with start state S (d_k x d_v), and with
b_r = sum_{u<=r} g_u (running log-decay inside the chunk, per key channel),
Gamma_r = exp(b_r), gamma = Gamma_L:

  A_kk = StrictTril(Diag(beta) (K^ * Gamma)(K^ / Gamma)^T)
  Tm   = (I + A_kk)^-1                              (the UT transform)
  W    = Tm Diag(beta) (K^ * Gamma),  U = Tm Diag(beta) V,  Ut = U - W S
  A_qk = Tril((Q^ * Gamma)(K^ / Gamma)^T)           (diagonal kept: each token
                                                      reads the state after its
                                                      own write)
  O    = (Q^ * Gamma) S + A_qk Ut
  S'   = Diag(gamma) S + (K^ * gamma / Gamma)^T Ut

Sources: "Kimi K3 模型结构（2）：序列维度（下）" (Q&A on the chunkwise algorithm:
C = 64, WY representation, UT transform as one C x C triangular inverse; Q&A
on the intra-chunk matrix A[t] and the output O[t]); "Kimi K3 の KDA ..."
section 1.2.1 (inter-chunk path 1 / intra-chunk path 2, Tril keeps the
diagonal).  A_kk, W, U and S' are not printed on the pages; they follow from
the recurrence (the derivation is in the design notes) and the test
``test_chunk_model_matches_token_oracle`` pins them.

The ratio Gamma_r / Gamma_s is formed per 16-token sub-tile pair with a
reference point between s and r, so no factor leaves [e^-80, e^80] when
g >= -5 ("Kimi K3 の KDA ..." section 1.2.1 on the bounded decay; "Kimi K3 模型结构（2）" Q&A on
the -5 bound: 16 steps give at most e^80 < bf16 max).
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6
SUB = 16


# ----------------------------------------------------------------------------
# precision emulation of one matrix product
# ----------------------------------------------------------------------------
def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def _bf16(x):
    u = _f32(x).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)
    return r.astype(np.uint32).view(np.float32)


def _fp16(x):
    return _f32(x).astype(np.float16).astype(np.float32)


def _split(x, rnd):
    hi = rnd(x)
    lo = rnd(np.asarray(x, np.float64) - hi.astype(np.float64))
    return hi, lo


def mm(X, Y, mode="f64"):
    """X @ Y with operands rounded per ``mode``; accumulation in fp32 for the
    reduced modes (as a matrix core accumulates)."""
    if mode == "f64":
        return np.asarray(X, np.float64) @ np.asarray(Y, np.float64)
    if mode == "f32":
        return (_f32(X) @ _f32(Y)).astype(np.float64)
    rnd = {"bf16": _bf16, "fp16": _fp16}[mode.split("x")[0]]
    if mode in ("bf16", "fp16"):
        return (rnd(X) @ rnd(Y)).astype(np.float64)
    if mode.endswith("x2a"):           # X split hi/lo, Y rounded once
        xh, xl = _split(X, rnd)
        y = rnd(Y)
        return (xh @ y + xl @ y).astype(np.float64)
    if mode.endswith("x2b"):           # Y split hi/lo, X rounded once
        yh, yl = _split(Y, rnd)
        x = rnd(X)
        return (x @ yh + x @ yl).astype(np.float64)
    if mode.endswith("x3"):
        xh, xl = _split(X, rnd)
        yh, yl = _split(Y, rnd)
        return (xh @ yh + xh @ yl + xl @ yh).astype(np.float64)
    raise ValueError(mode)


DEFAULT_PREC = dict(akk="f64", aqk="f64", W="f64", U="f64", WS="f64", QS="f64", AU="f64", KU="f64",
                    KS="f64", TR="f64")


# ----------------------------------------------------------------------------
# the chunk algebra
# ----------------------------------------------------------------------------
def _tiled_pair_matrix(X, K, b, mode, strict):
    """M[r, s] = sum_i X[r,i] K[s,i] exp(b[r,i] - b[s,i]) for s <= r (s < r if
    strict), formed per SUB x SUB tile pair (row tile ti, column tile tj <= ti)
    as (X_r * exp(b_r - ref)) . (K_s * exp(ref - b_s)) with ref = b at the end
    of the tile before ti (0 for the first).  The row factor is <= 1; the
    column factor is <= 1 off the diagonal (where it can only underflow when
    the whole term is negligible) and <= exp(-SUB * min g) on it."""
    L = X.shape[0]
    M = np.zeros((L, L))
    nt = (L + SUB - 1) // SUB
    for ti in range(nt):
        r0, r1 = ti * SUB, min(L, (ti + 1) * SUB)
        ref = b[r0 - 1] if r0 > 0 else np.zeros(b.shape[1])
        rowf = X[r0:r1] * np.exp(b[r0:r1] - ref[None, :])
        for tj in range(ti + 1):
            s0, s1 = tj * SUB, min(L, (tj + 1) * SUB)
            colf = K[s0:s1] * np.exp(ref[None, :] - b[s0:s1])
            M[r0:r1, s0:s1] = mm(rowf, colf.T, mode)
    return np.tril(M, -1 if strict else 0)


def chunk_chain(q, k, v, g, beta, S0=None, *, C=64, scale=1.0, eps=EPS, prec=None, tinv="f64", form="WU"):
    """Chunkwise forward for one chain.  q, k, g: [T, dk]; v: [T, dv];
    beta: [T].  Returns (o [T, dv], S_T).

    form="WU": U~ = U - W S with U = Tm Diag(beta) V, W = Tm Diag(beta)(K^ Gamma);
    form="R":  U~ = (Tm Diag(beta)) (V - (K^ Gamma) S), the same quantity."""
    p = dict(DEFAULT_PREC)
    if prec:
        p.update(prec)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    T, dk = q.shape
    dv = v.shape[1]
    Qh = q / np.sqrt(np.sum(q * q, axis=1, keepdims=True) + eps)
    Kh = k / np.sqrt(np.sum(k * k, axis=1, keepdims=True) + eps)
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        L = c1 - c0
        Q, K, V, G, bt = Qh[c0:c1], Kh[c0:c1], v[c0:c1], g[c0:c1], beta[c0:c1]
        b = np.cumsum(G, axis=0)
        Gam = np.exp(b)
        gam = Gam[L - 1]
        Akk = bt[:, None] * _tiled_pair_matrix(K, K, b, p["akk"], strict=True)
        Aqk = _tiled_pair_matrix(Q, K, b, p["aqk"], strict=False)
        if tinv == "f64":
            Tm = np.linalg.inv(np.eye(L) + Akk)
        else:
            Tm = np.linalg.inv((np.eye(L) + Akk).astype(np.float32)).astype(np.float64)
        if form == "WU":
            W = mm(Tm, bt[:, None] * (K * Gam), p["W"])
            U = mm(Tm * bt[None, :], V, p["U"])
            Ut = U - mm(W, S, p["WS"])
        else:
            R = V - mm(K * Gam, S, p["KS"])
            Ut = mm(Tm * bt[None, :], R, p["TR"])
        o[c0:c1] = scale * (mm(Q * Gam, S, p["QS"]) + mm(Aqk, Ut, p["AU"]))
        Kg = K * np.exp(b[L - 1][None, :] - b)
        S = gam[:, None] * S + mm(Kg.T, Ut, p["KU"])
    return o, S
