"""Pins for the CPU oracle: every check compares it with something other than
itself -- a closed form, an identity the pages state, a worked example they
print, or a second formulation written independently.  CPU only."""
import json
import os

import numpy as np
import pytest

import kda_inputs
import oracle
from oracle import chunk_model

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng(1234)


def _rand_chain(rng, T, dk, dv, gate_lo=-5.0, beta_hi=1.0):
    q = rng.standard_normal((T, dk)).astype(np.float32)
    k = rng.standard_normal((T, dk)).astype(np.float32)
    v = rng.standard_normal((T, dv)).astype(np.float32)
    g = rng.uniform(gate_lo, 0.0, (T, dk)).astype(np.float32)
    beta = rng.uniform(0.0, beta_hi, T).astype(np.float32)
    return q, k, v, g, beta


def _run(q, k, v, g, beta, S0=None, eps=oracle.EPS, scale=1.0):
    """C oracle on one chain."""
    T, dk = q.shape
    dv = v.shape[1]
    o, sT = oracle.forward_arrays(q[None, :, None], k[None, :, None], v[None, :, None], g[None, :, None],
                                  beta[None, :, None], None if S0 is None else S0[None, None],
                                  eps=eps, scale=scale)
    return o[0, :, 0], sT[0, 0]


def _unit(x, eps=oracle.EPS):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(x @ x + eps)


# ---------------------------------------------------------------------------
# P1 -- brute force: the general solution of the affine recurrence as an
# ordered product of transitions ("Kimi K3 の KDA ..." section 2.3.5: the
# state map is prod_t T_t, later factors on the left; section 2.3.4.1: the
# composed write term of (A2,b2)o(A1,b1) is A2 b1 + b2).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d", [2, 3, 4, 8])
@pytest.mark.parametrize("T", [1, 5, 12])
def test_brute_force_transition_products(d, T):
    rng = np.random.default_rng(100 * d + T)
    q, k, v, g, beta = _rand_chain(rng, T, d, d + 1)
    S0 = rng.standard_normal((d, d + 1))
    o, sT = _run(q, k, v, g, beta, S0)
    kh = [_unit(k[t]) for t in range(T)]
    M = [oracle.transition(np.exp(g[t].astype(np.float64)), float(beta[t]), kh[t]) for t in range(T)]

    def prod(lo, hi):  # M_{hi-1} ... M_lo  (empty product = I)
        P = np.eye(d)
        for t in range(lo, hi):
            P = M[t] @ P
        return P

    for t in range(T):
        St = prod(0, t + 1) @ S0
        for s in range(t + 1):
            St = St + prod(s + 1, t + 1) @ (float(beta[s]) * np.outer(kh[s], v[s]))
        np.testing.assert_allclose(o[t], St.T @ _unit(q[t]), rtol=1e-12, atol=1e-12)
        if t == T - 1:
            np.testing.assert_allclose(sT, St, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# P2 -- the worked example printed with Figure 1 of the Complex KDA review
# ---------------------------------------------------------------------------
def test_worked_example_rotation():
    with open(os.path.join(GOLDEN, "rotation_90.json")) as f:
        ex = json.load(f)
    M = oracle.transition(ex["alpha"], ex["beta"], ex["k"])
    np.testing.assert_allclose(M, np.array(ex["expected_transition"]), atol=1e-15)
    assert abs(np.linalg.det(M) - 1.0) < 1e-14
    np.testing.assert_allclose(M.T @ M, np.eye(2), atol=1e-15)
    # rotates (1,0) by +90 degrees
    angle = np.degrees(np.arctan2(*(M @ np.array([1.0, 0.0]))[::-1]))
    assert abs(angle - ex["rotation_degrees"]) < 1e-12


def test_printed_constants():
    with open(os.path.join(GOLDEN, "printed_constants.json")) as f:
        c = json.load(f)
    assert abs(np.exp(-c["g_min"] * c["sub_tile"]) / c["exp80_approx"] - 1) < 0.01
    bf16_max = float(kda_inputs.bf16_to_f32(np.array([0x7F7F], np.uint16))[0])
    assert abs(bf16_max / c["bf16_max_approx"] - 1) < 0.01
    assert np.exp(-c["g_min"] * c["sub_tile"]) < bf16_max
    assert abs(np.exp(c["g_min"]) - c["exp_minus5_approx"]) < 5e-5
    assert chunk_model.SUB == c["sub_tile"]


# ---------------------------------------------------------------------------
# P3 -- GDN reduction ("GDN, KDA の整理", section "Kimi Delta Attention":
# D_t = alpha_t I gives Gated DeltaNet)
# ---------------------------------------------------------------------------
def test_gdn_reduction():
    rng = np.random.default_rng(3)
    T, dk, dv = 40, 16, 12
    q, k, v, _, beta = _rand_chain(rng, T, dk, dv)
    a = rng.uniform(-3.0, 0.0, T).astype(np.float32)
    g = np.repeat(a[:, None], dk, axis=1)
    o, sT = _run(q, k, v, g, beta)
    # scalar-gated delta rule, written in its own (GDN) form
    S = np.zeros((dk, dv))
    for t in range(T):
        kh = _unit(k[t])
        alpha = np.exp(np.float64(a[t]))
        S = alpha * (S - beta[t] * np.outer(kh, kh @ S)) + beta[t] * np.outer(kh, v[t])
        np.testing.assert_allclose(o[t], S.T @ _unit(q[t]), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sT, S, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# P4 -- beta = 0: pure decay, S_t = Diag(exp(sum_{u<=t} g_u)) S_0
# ("Kimi K3 の KDA ..." section 2.3.5, pure-decay approximation)
# ---------------------------------------------------------------------------
def test_beta_zero_closed_form():
    rng = np.random.default_rng(4)
    T, dk, dv = 33, 8, 5
    q, k, v, g, _ = _rand_chain(rng, T, dk, dv, gate_lo=-0.5)
    beta = np.zeros(T, np.float32)
    S0 = rng.standard_normal((dk, dv))
    o, sT = _run(q, k, v, g, beta, S0)
    cum = np.cumsum(g.astype(np.float64), axis=0)
    for t in range(T):
        St = np.exp(cum[t])[:, None] * S0
        np.testing.assert_allclose(o[t], St.T @ _unit(q[t]), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sT, np.exp(cum[-1])[:, None] * S0, rtol=1e-12)


# ---------------------------------------------------------------------------
# P5 -- non-expansiveness ("Kimi K3 の KDA ..." section 1.2.1: L2-normalised k keeps the
# erase operator's spectral norm <= 1; Complex KDA review, key terms)
# ---------------------------------------------------------------------------
def test_non_expansive():
    rng = np.random.default_rng(5)
    T, dk, dv = 50, 16, 8
    q, k, _, g, beta = _rand_chain(rng, T, dk, dv, gate_lo=-0.05)
    v = np.zeros((T, dv), np.float32)
    S0 = rng.standard_normal((dk, dv))
    norms = [np.linalg.norm(S0)]
    for t in range(1, T + 1):
        _, sT = _run(q[:t], k[:t], v[:t], g[:t], beta[:t], S0)
        norms.append(np.linalg.norm(sT))
    assert all(n2 <= n1 * (1 + 1e-13) for n1, n2 in zip(norms, norms[1:]))
    assert norms[-1] < norms[0]


@pytest.mark.parametrize("beta", [0.0, 0.3, 1.0])
def test_erase_operator_spectrum(beta):
    k = _unit(rng0.standard_normal(7), eps=0.0)
    E = np.eye(7) - beta * np.outer(k, k)
    ev = np.sort(np.linalg.eigvalsh(E))
    np.testing.assert_allclose(ev, np.sort([1.0 - beta] + [1.0] * 6), atol=1e-14)
    assert np.linalg.norm(E, 2) <= 1 + 1e-14


# ---------------------------------------------------------------------------
# P6 -- local loss: after the update the residual on k is (1-beta) times the
# pre-update one; beta = 1 recalls v exactly ("GDN, KDA の整理", 局所損失)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("b_last", [0.37, 1.0])
def test_residual_contraction(b_last):
    rng = np.random.default_rng(6)
    T, dk, dv = 20, 12, 9
    q, k, v, g, beta = _rand_chain(rng, T, dk, dv)
    beta[-1] = b_last
    _, s_prev = _run(q[:-1], k[:-1], v[:-1], g[:-1], beta[:-1], eps=0.0)
    _, s_T = _run(q, k, v, g, beta, eps=0.0)
    kh = _unit(k[-1], eps=0.0)
    S_tilde = np.exp(g[-1].astype(np.float64))[:, None] * s_prev
    r_pre = v[-1] - S_tilde.T @ kh
    r_post = v[-1] - s_T.T @ kh
    np.testing.assert_allclose(r_post, (1.0 - b_last) * r_pre, atol=1e-12)


# ---------------------------------------------------------------------------
# P7 -- a query orthogonal to k_t does not see the delta update
# ("GDN, KDA の整理", 局所損失, last paragraph)
# ---------------------------------------------------------------------------
def test_orthogonal_query():
    rng = np.random.default_rng(7)
    T, dk, dv = 15, 10, 6
    q, k, v, g, beta = _rand_chain(rng, T, dk, dv)
    kk = k[-1].astype(np.float64)
    qq = rng.standard_normal(dk)
    qq -= (qq @ kk) / (kk @ kk) * kk
    q[-1] = qq.astype(np.float32)
    qq = q[-1].astype(np.float64)
    assert abs(qq @ kk) < 1e-5 * np.linalg.norm(qq) * np.linalg.norm(kk)
    _, s_prev = _run(q[:-1], k[:-1], v[:-1], g[:-1], beta[:-1])
    o, _ = _run(q, k, v, g, beta)
    S_tilde = np.exp(g[-1].astype(np.float64))[:, None] * s_prev
    np.testing.assert_allclose(o[-1], S_tilde.T @ _unit(qq), atol=1e-6 * np.abs(o[-1]).max() + 1e-12)


# ---------------------------------------------------------------------------
# P8 -- fixed point of a repeated affine map x* = (I - A)^-1 b
# ("Kimi K3 の KDA ..." section 2.3.3, item 3)
# ---------------------------------------------------------------------------
def test_fixed_point_long_run():
    rng = np.random.default_rng(8)
    dk, dv, n = 8, 5, 40000
    k1 = rng.standard_normal(dk)
    v1 = rng.standard_normal(dv)
    g1 = np.full(dk, -1e-3)
    b1 = 0.5
    q = np.tile(rng.standard_normal(dk), (n, 1)).astype(np.float32)
    k = np.tile(k1, (n, 1)).astype(np.float32)
    v = np.tile(v1, (n, 1)).astype(np.float32)
    g = np.tile(g1, (n, 1)).astype(np.float32)
    beta = np.full(n, b1, np.float32)
    _, sT = _run(q, k, v, g, beta)
    kh = _unit(k[0])
    M = oracle.transition(np.exp(g[0].astype(np.float64)), float(beta[0]), kh)
    Sstar = np.linalg.solve(np.eye(dk) - M, float(beta[0]) * np.outer(kh, v[0]))
    np.testing.assert_allclose(sT, Sstar, rtol=1e-9, atol=1e-9)


# ---------------------------------------------------------------------------
# P9 / P10 -- associativity (split and hand-off) and the identity (empty
# segment) of the affine monoid ("Kimi K3 の KDA ..." sections 2.3.4.2,
# 2.3.4.3 and 2.3.4.5)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("split", [0, 1, 17, 63, 64, 65, 100, 130])
def test_split_handoff(split):
    rng = np.random.default_rng(9)
    T, dk, dv = 130, 16, 16
    q, k, v, g, beta = _rand_chain(rng, T, dk, dv)
    S0 = rng.standard_normal((dk, dv))
    o, sT = _run(q, k, v, g, beta, S0)
    o1, s1 = _run(q[:split], k[:split], v[:split], g[:split], beta[:split], S0)
    o2, s2 = _run(q[split:], k[split:], v[split:], g[split:], beta[split:], s1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s2, sT, rtol=1e-12, atol=1e-13)


def test_empty_sequence_is_identity_and_varlen_packing():
    rng = np.random.default_rng(10)
    H, dk, dv = 3, 8, 6
    lens = [5, 0, 70, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = rng.standard_normal((1, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((1, T, H, dk)).astype(np.float32)
    v = rng.standard_normal((1, T, H, dv)).astype(np.float32)
    g = rng.uniform(-5, 0, (1, T, H, dk)).astype(np.float32)
    beta = rng.uniform(0, 1, (1, T, H)).astype(np.float32)
    S0 = rng.standard_normal((len(lens), H, dk, dv))
    o, sT = oracle.forward_arrays(q, k, v, g, beta, S0, cu)
    np.testing.assert_array_equal(sT[1], S0[1])
    for n, L in enumerate(lens):
        a, b = cu[n], cu[n + 1]
        on, sn = oracle.forward_arrays(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], S0[n:n + 1])
        np.testing.assert_array_equal(sn[0], sT[n])
        np.testing.assert_array_equal(on[0], o[0, a:b])


# ---------------------------------------------------------------------------
# P11 -- column independence: the d_v columns are independent affine systems
# sharing one transition ("Kimi K3 の KDA ..." section 2.3.2)
# ---------------------------------------------------------------------------
def test_column_independence():
    rng = np.random.default_rng(11)
    T, dk, dv = 90, 12, 10
    q, k, v, g, beta = _rand_chain(rng, T, dk, dv)
    S0 = rng.standard_normal((dk, dv))
    o, sT = _run(q, k, v, g, beta, S0)
    J = [1, 4, 9]
    oj, sj = _run(q, k, np.ascontiguousarray(v[:, J]), g, beta, np.ascontiguousarray(S0[:, J]))
    np.testing.assert_array_equal(oj, o[:, J])
    np.testing.assert_array_equal(sj, sT[:, J])


# ---------------------------------------------------------------------------
# P12 -- non-commutativity: order matters ("Kimi K3 の KDA ..." section 2.3.4.6)
# ---------------------------------------------------------------------------
def test_order_sensitivity():
    rng = np.random.default_rng(12)
    T, dk, dv = 6, 6, 4
    q, k, v, g, beta = _rand_chain(rng, T, dk, dv)
    _, sT = _run(q, k, v, g, beta)
    perm = np.array([0, 1, 3, 2, 4, 5])
    _, sP = _run(q[perm], k[perm], v[perm], g[perm], beta[perm])
    assert np.abs(sT - sP).max() > 1e-3
    # the decay matrices alone commute
    a, b = np.diag(np.exp(g[2])), np.diag(np.exp(g[3]))
    np.testing.assert_allclose(a @ b, b @ a)


# ---------------------------------------------------------------------------
# P13 -- two formulations agree: innovation form (C) vs explicit product of
# transition matrices (NumPy) -- "Kimi K3 の KDA ..." section 1.2.1 (innovation) and
# "GDN, KDA の整理" section "Online learning" (gradient step on the decayed state)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("scale", [1.0, 0.125])
def test_innovation_vs_product_form(scale):
    rng = np.random.default_rng(13)
    T, dk, dv = 77, 32, 24
    q, k, v, g, beta = _rand_chain(rng, T, dk, dv)
    S0 = 0.1 * rng.standard_normal((dk, dv))
    o, sT = _run(q, k, v, g, beta, S0, scale=scale)
    op, sp = oracle.product_form(q, k, v, g, beta, S0, scale=scale)
    np.testing.assert_allclose(o, op, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(sT, sp, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------------------
# P14 -- the chunk algebra (WY/UT form with 16-token sub-tile references)
# equals the token recurrence, including partial chunks
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,gate", [(1, "k3"), (16, "k3"), (63, "sigmoid"), (64, "k3"),
                                    (65, "slow"), (200, "k3"), (257, "sigmoid")])
def test_chunk_model_matches_token_oracle(T, gate):
    inp = kda_inputs.make_prefill(21 + T, 1, T, 2, 32, 24, dtype="bf16", gate=gate, s0_std=0.02)
    o, sT = oracle.forward(inp)
    for h in range(2):
        oc, sc = chunk_model.chunk_chain(inp.f32("q")[0, :, h], inp.f32("k")[0, :, h], inp.f32("v")[0, :, h],
                                         inp.g[0, :, h], inp.beta[0, :, h], inp.f32("init_state")[0, h])
        scale = np.sqrt(np.mean(o[0, :, h] ** 2))
        assert np.abs(oc - o[0, :, h]).max() <= 1e-12 * max(scale, 1e-30) + 1e-15
        assert np.abs(sc - sT[0, h]).max() <= 1e-12


def test_chunk_model_bounded_factors_at_gmin():
    """All gates at the lower bound -5 (the worst case the pages allow): the
    sub-tile factors stay finite in fp32 and the model still matches."""
    rng = np.random.default_rng(14)
    T, dk, dv = 128, 16, 8
    q, k, v, _, beta = _rand_chain(rng, T, dk, dv)
    g = np.full((T, dk), -5.0, np.float32)
    o, sT = _run(q, k, v, g, beta)
    oc, sc = chunk_model.chunk_chain(q, k, v, g, beta, prec=dict(aqk="f32", akk="f32"))
    assert np.all(np.isfinite(oc))
    np.testing.assert_allclose(oc, o, rtol=1e-4, atol=1e-6)
    np.testing.assert_allclose(sc, sT, rtol=1e-4, atol=1e-6)


# ---------------------------------------------------------------------------
# input generator sanity (not a pin of the method)
# ---------------------------------------------------------------------------
def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], np.float32)
    bits = kda_inputs.bf16_bits(x)
    back = kda_inputs.bf16_to_f32(bits)
    assert back[0] == 1.0
    assert back[1] == 1.0                       # tie -> even (mantissa 0)
    assert back[2] == 1.0 + 4 * 2 ** -8         # tie -> even (round up)
    assert back[3] == -2.5


def test_generator_is_deterministic_and_blocked():
    a = kda_inputs.make_prefill(7, 1, 5000, 2, 16, 16, gate="k3", s0_std=0.02)
    b = kda_inputs.make_prefill(7, 1, 5000, 2, 16, 16, gate="k3", s0_std=0.02)
    for name in ("q", "k", "v", "g", "beta", "init_state"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    assert a.g.min() >= -5.0 and a.g.max() <= 0.0
    assert a.beta.min() > 0.0 and a.beta.max() < 1.0
    lens = kda_inputs.varlen_lengths()
    assert len(lens) == 16 and lens.min() >= 512 and lens.max() <= 16384


# ---------------------------------------------------------------------------
# Gate prologue of the gated entry points: g = -5 sigmoid(e^A (z + dt_bias)),
# beta = sigmoid(logit) ("Kimi K3 模型结构（2）", Q&A: the scaled sigmoid with
# g_min = -5 and range (-5, 0); "Kimi K3 の KDA ..." section 1.2.1: A_log,
# dt_bias and the in-kernel sigmoid of beta).  Each test checks a value the
# formula fixes without evaluating the formula the same way.
# ---------------------------------------------------------------------------
def _gate_case(seed=11, H=3, d=8, n=5):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((n, H, d))
    A = rng.uniform(-1, 1, H)
    b = rng.standard_normal((H, d))
    return z, A, b


def test_gate_map_midpoint_is_half_of_the_bound():
    # sigmoid(0) = 1/2: a logit that cancels the bias gives exactly g_min / 2
    _, A, b = _gate_case()
    g = oracle.gate_map(-b[None], A, b)
    np.testing.assert_array_equal(g, np.full(g.shape, -2.5))


def test_gate_map_reflection():
    # sigmoid(x) + sigmoid(-x) = 1  =>  g(x) + g(-x) = g_min for x = e^A (z + b)
    z, A, b = _gate_case()
    g_pos = oracle.gate_map(z, A, b)
    g_neg = oracle.gate_map(-z - 2 * b, A, b)          # z + b -> -(z + b)
    np.testing.assert_allclose(g_pos + g_neg, -5.0, rtol=0, atol=1e-14)


def test_gate_map_bounds_limits_and_monotonicity():
    z, A, b = _gate_case()
    g = oracle.gate_map(z, A, b)
    assert np.all(g < 0) and np.all(g > -5)             # the open range (-5, 0)
    big = np.full_like(z, 60.0)
    np.testing.assert_allclose(oracle.gate_map(big, A, None), -5.0, rtol=0, atol=1e-8)   # no-forget limit: -5
    np.testing.assert_allclose(oracle.gate_map(-big, A, None), 0.0, rtol=0, atol=1e-8)   # and 0 at -inf
    # strictly decreasing in z for every head scale e^A > 0
    np.testing.assert_array_less(oracle.gate_map(z + 1e-3, A, b), g)


def test_gate_map_scale_enters_as_exp_of_a_log():
    # e^(A + ln 2) (z/2 + b/2) = e^A (z + b): halving the logit and the bias
    # while adding ln 2 to A_log leaves g unchanged
    z, A, b = _gate_case()
    np.testing.assert_allclose(oracle.gate_map(z / 2, A + np.log(2.0), b / 2), oracle.gate_map(z, A, b),
                               rtol=1e-14, atol=1e-15)


def test_gate_map_without_bias_is_the_printed_k3_map():
    # with no bias the map is exactly g_min * sigmoid(e^A z), checked against
    # a logistic evaluated through tanh: sigmoid(x) = (1 + tanh(x/2)) / 2
    z, A, _ = _gate_case()
    x = np.exp(A)[:, None] * z
    np.testing.assert_allclose(oracle.gate_map(z, A, None), -5.0 * 0.5 * (1.0 + np.tanh(x / 2)), rtol=1e-14)


def test_beta_from_logits():
    assert oracle.beta_from_logits(0.0) == 0.5
    b = np.linspace(-30, 30, 61)
    np.testing.assert_allclose(oracle.beta_from_logits(b) + oracle.beta_from_logits(-b), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.beta_from_logits(b), 0.5 * (1.0 + np.tanh(b / 2)), rtol=1e-13, atol=1e-15)
    assert oracle.beta_from_logits(-1000.0) == 0.0 and oracle.beta_from_logits(1000.0) == 1.0   # no overflow


def test_gated_oracle_composes_map_and_recurrence():
    # the gated oracle equals the plain one fed with the mapped decay and
    # strength; and a logit of +inf-like size gives beta = 1, i.e. S^T k^ = v
    inp = kda_inputs.make_gated_prefill(5, 1, 70, 2, 8, 4, dtype="f32", s0_std=0.1)
    o1, s1 = oracle.forward_gated(inp)
    g = oracle.gate_map(inp.z, inp.A_log, inp.dt_bias)
    o2, s2 = oracle.forward_arrays(inp.q, inp.k, inp.v, g, oracle.beta_from_logits(inp.beta_logits),
                                   inp.init_state)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)
    inp.beta_logits[:] = 80.0
    _, sT = oracle.forward_gated(inp)
    kl = inp.k[0, -1].astype(np.float64)
    kh = kl / np.sqrt(np.sum(kl * kl, axis=-1, keepdims=True) + oracle.EPS)
    # |k^|^2 = 1 - eps / (|k|^2 + eps) leaves a residual of order 1e-7 here
    for h in range(2):
        np.testing.assert_allclose(sT[0, h].T @ kh[h], inp.v[0, -1, h], rtol=2e-6, atol=2e-6)


def test_gated_generator_draws_raw_inputs():
    a = kda_inputs.make_gated_prefill(7, 1, 300, 2, 16, 16, s0_std=0.02)
    b = kda_inputs.make_gated_prefill(7, 1, 300, 2, 16, 16, s0_std=0.02)
    for name in ("q", "k", "v", "z", "A_log", "dt_bias", "beta_logits", "init_state"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    assert a.z.dtype == np.uint16 and a.beta_logits.min() < 0 < a.beta_logits.max()   # raw logits, not sigmoids


# ---------------------------------------------------------------------------
# Complex KDA: signed decay alpha in [-1, 1], beta in [0, 2] ("[논문리뷰]
# Complex KDA ..." page: the gate range widened to [-1, 1] and beta to [0, 2];
# one update (I - beta k k^T) Diag(alpha) stays diagonal-plus-rank-one and
# non-expansive; Figure 1's 90 degree rotation).
# ---------------------------------------------------------------------------
def test_signed_oracle_runs_the_printed_rotation():
    # Figure 1 through the C recurrence: one token with v = 0 maps S0 = I to
    # the transition itself, the rotation by 90 degrees
    with open(os.path.join(GOLDEN, "rotation_90.json")) as f:
        ex = json.load(f)
    q = np.array([[[[1.0, 0.0]]]], np.float32)
    k = np.array([[[ex["k"]]]], np.float32)
    v = np.zeros((1, 1, 1, 2), np.float32)
    alpha = np.array([[[ex["alpha"]]]], np.float32)
    beta = np.full((1, 1, 1), ex["beta"], np.float32)
    _, sT = oracle.forward_signed(q, k, v, alpha, beta, np.eye(2)[None, None], eps=0.0)
    np.testing.assert_allclose(sT[0, 0], np.array(ex["expected_transition"]), atol=1e-7)


@pytest.mark.parametrize("d,T", [(2, 7), (3, 5), (8, 12)])
def test_signed_oracle_matches_explicit_products(d, T):
    rng = np.random.default_rng(100 + d)
    q = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    v = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    alpha = rng.uniform(-1, 1, (1, T, 1, d)).astype(np.float32)
    beta = rng.uniform(0, 2, (1, T, 1)).astype(np.float32)
    s0 = rng.standard_normal((1, 1, d, d))
    o, sT = oracle.forward_signed(q, k, v, alpha, beta, s0)
    op, sp = oracle.product_form(q[0, :, 0], k[0, :, 0], v[0, :, 0], alpha[0, :, 0], beta[0, :, 0], s0[0, 0],
                                 alpha_given=True)
    np.testing.assert_allclose(o[0, :, 0], op, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sT[0, 0], sp, rtol=1e-12, atol=1e-12)


def test_signed_transitions_are_non_expansive_and_orthogonal_at_the_ends():
    rng = np.random.default_rng(7)
    d, T = 6, 40
    q = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    v = np.zeros((1, T, 1, d), np.float32)
    s0 = rng.standard_normal((1, 1, d, d))
    # |alpha| <= 1, beta in [0, 2]: ||S_t||_F never grows (v = 0)
    alpha = rng.uniform(-1, 1, (1, T, 1, d)).astype(np.float32)
    beta = rng.uniform(0, 2, (1, T, 1)).astype(np.float32)
    norms = [np.linalg.norm(s0)]
    for t in range(1, T + 1):
        _, s = oracle.forward_signed(q[:, :t], k[:, :t], v[:, :t], alpha[:, :t], beta[:, :t], s0, eps=0.0)
        norms.append(np.linalg.norm(s))
    assert all(b <= a * (1 + 1e-12) for a, b in zip(norms, norms[1:]))
    # alpha in {-1, +1} and beta = 2: a reflection times a signed permutation-free
    # diagonal is orthogonal, so the norm is kept exactly
    alpha = np.where(rng.uniform(size=(1, T, 1, d)) < 0.5, -1.0, 1.0).astype(np.float32)
    beta = np.full((1, T, 1), 2.0, np.float32)
    _, s = oracle.forward_signed(q, k, v, alpha, beta, s0, eps=0.0)
    assert abs(np.linalg.norm(s) / np.linalg.norm(s0) - 1.0) < 1e-5


def test_signed_oracle_with_positive_alpha_is_the_log_oracle():
    inp = kda_inputs.make_prefill(3, 1, 90, 2, 8, 8, dtype="f32", s0_std=0.1)
    o1, s1 = oracle.forward_arrays(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state)
    alpha = np.exp(inp.g.astype(np.float64)).astype(np.float32)
    o2, s2 = oracle.forward_signed(inp.q, inp.k, inp.v, alpha, inp.beta, inp.init_state)
    # alpha rounded to fp32 once: agreement to fp32 rounding of the decay
    np.testing.assert_allclose(o2, o1, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(s2, s1, rtol=1e-5, atol=1e-6)


# ---------------------------------------------------------------------------
# Output norm ("Kimi K3 の KDA ..." section 1.2.1: per-head RMSNorm over the
# value dimension, sigmoid of the output gate, elementwise product; the norm
# before the gate)
# ---------------------------------------------------------------------------
def test_out_norm_worked_by_hand():
    # o = (1, 2, 2): mean square 3; with eps = 1 the scale is 1/sqrt(4) = 1/2,
    # so RMSNorm(o) = (0.5, 1, 1).  weight (2, 1, 0.5) and gate (0, ln 3,
    # -ln 3), whose sigmoids are (1/2, 3/4, 1/4), give (0.5, 0.75, 0.125).
    y = oracle.out_norm(np.array([1.0, 2.0, 2.0]), np.array([0.0, np.log(3.0), -np.log(3.0)]),
                        np.array([2.0, 1.0, 0.5]), eps=1.0)
    np.testing.assert_allclose(y, [0.5, 0.75, 0.125], rtol=1e-15, atol=0)


def test_out_norm_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(77)
    o = rng.standard_normal((5, 3, 16))
    gate = rng.standard_normal((5, 3, 16))
    y = oracle.out_norm(o, gate, eps=0.0)
    np.testing.assert_allclose(oracle.out_norm(7.5 * o, gate, eps=0.0), y, rtol=1e-14, atol=0)
    np.testing.assert_allclose(oracle.out_norm(-o, gate, eps=0.0), -y, rtol=1e-15, atol=0)
    # a saturated gate (sigmoid = 1) leaves the plain RMSNorm: unit RMS per row
    y1 = oracle.out_norm(o, np.full_like(o, 60.0), eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y1 * y1, axis=-1)), 1.0, rtol=1e-14, atol=0)
    # sigmoid(x) + sigmoid(-x) = 1: the two gates add up to the plain norm
    np.testing.assert_allclose(oracle.out_norm(o, gate, eps=0.0) + oracle.out_norm(o, -gate, eps=0.0), y1,
                               rtol=1e-13, atol=1e-15)
    # eps keeps a zero row at zero
    assert np.all(oracle.out_norm(np.zeros((2, 8)), np.zeros((2, 8)), eps=1e-5) == 0.0)


def test_out_norm_reduces_each_row_over_the_last_axis_with_a_shared_weight():
    rng = np.random.default_rng(78)
    u = rng.standard_normal(16)
    c = rng.uniform(0.1, 10.0, (4, 3, 1))
    y = oracle.out_norm(c * u, np.zeros((4, 3, 16)), eps=0.0)   # every row a positive multiple of u
    np.testing.assert_allclose(y, np.broadcast_to(y[0, 0], y.shape), rtol=1e-14, atol=0)
    w = np.zeros(16)
    w[5] = 2.0
    y = oracle.out_norm(rng.standard_normal((4, 3, 16)), rng.standard_normal((4, 3, 16)), w, eps=1e-5)
    assert np.all(np.delete(y, 5, axis=-1) == 0.0) and np.all(y[..., 5] != 0.0)


def test_out_norm_after_one_token_from_zero_state():
    # from S = 0 the first output is o = scale beta (k^ . q^) v, so its norm
    # with eps = 0 is sign(beta k^.q^) v / rms(v) * w * sigmoid(gate)
    rng = np.random.default_rng(79)
    d = 8
    q, k, v, g, beta = _rand_chain(rng, 1, d, d)
    o, _ = _run(q, k, v, g, beta, scale=0.5)
    gate = rng.standard_normal(d)
    w = rng.uniform(0.5, 1.5, d)
    vv = v[0].astype(np.float64)
    sign = np.sign(float(beta[0]) * float(_unit(k[0]) @ _unit(q[0])))
    expect = sign * vv / np.sqrt(np.mean(vv * vv)) * w / (1.0 + np.exp(-gate))
    np.testing.assert_allclose(oracle.out_norm(o[0], gate, w, eps=0.0), expect, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Short convolution ("Kimi K3 の KDA ..." section 1.2.1: causal, per channel,
# the current token and the 3 before it, then SiLU; "GDN, KDA の整理": the conv
# cache holds the previous 3 inputs)
# ---------------------------------------------------------------------------
def _silu(x):
    import math
    return x / (1.0 + math.exp(-x))


def test_short_conv_worked_by_hand():
    # one channel, taps (1, 2, 3, 4) oldest first, an impulse at t = 0: the
    # pre-activations walk the taps backwards, (4, 3, 2, 1, 0)
    w = np.array([[1.0, 2.0, 3.0, 4.0]])
    y, fin = oracle.short_conv(np.array([1.0, 0, 0, 0, 0])[None, :, None], w)
    np.testing.assert_allclose(y[0, :, 0], [_silu(4.0), _silu(3.0), _silu(2.0), _silu(1.0), 0.0], rtol=1e-15)
    assert np.all(fin == 0.0)
    # with a conv state (5, 6, 7) and one input 1: 1*5 + 2*6 + 3*7 + 4*1 = 42,
    # and the new state drops the oldest input
    y, fin = oracle.short_conv(np.array([[[1.0]]]), w, init=np.array([[[5.0], [6.0], [7.0]]]))
    np.testing.assert_allclose(y[0, 0, 0], _silu(42.0), rtol=1e-15)
    np.testing.assert_array_equal(fin[0, :, 0], [6.0, 7.0, 1.0])


def test_silu_closed_forms():
    x = np.linspace(-20, 20, 81)
    assert oracle.silu(0.0) == 0.0
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=0, atol=1e-14)
    np.testing.assert_allclose(oracle.silu(x), x / (1.0 + np.exp(-x)), rtol=1e-14, atol=1e-300)


def test_short_conv_identity_and_shift_taps():
    rng = np.random.default_rng(81)
    x = rng.standard_normal((2, 9, 5))
    init = rng.standard_normal((2, 3, 5))
    ident = np.tile([0.0, 0.0, 0.0, 1.0], (5, 1))
    y, fin = oracle.short_conv(x, ident, init)
    np.testing.assert_allclose(y, oracle.silu(x), rtol=0, atol=0)
    np.testing.assert_array_equal(fin, x[:, -3:])
    shift = np.tile([1.0, 0.0, 0.0, 0.0], (5, 1))                    # 3 tokens back
    y, _ = oracle.short_conv(x, shift, init)
    np.testing.assert_allclose(y[:, 3:], oracle.silu(x[:, :-3]), rtol=0, atol=0)
    np.testing.assert_allclose(y[:, :3], oracle.silu(init), rtol=0, atol=0)


def test_short_conv_is_causal_with_a_window_of_four():
    rng = np.random.default_rng(82)
    x = rng.standard_normal((1, 20, 3))
    w = rng.standard_normal((3, 4))
    y0, _ = oracle.short_conv(x, w)
    x2 = x.copy()
    x2[0, 9] += 1.0
    y1, _ = oracle.short_conv(x2, w)
    changed = np.any(y1 != y0, axis=(0, 2))
    assert not changed[:9].any() and changed[9:13].all() and not changed[13:].any()


def test_short_conv_state_carries_a_split_and_decode_steps():
    rng = np.random.default_rng(83)
    x = rng.standard_normal((1, 30, 6))
    w = rng.standard_normal((6, 4))
    init = rng.standard_normal((1, 3, 6))
    y, fin = oracle.short_conv(x, w, init)
    for cut in (1, 2, 3, 17):
        ya, fa = oracle.short_conv(x[:, :cut], w, init)
        yb, fb = oracle.short_conv(x[:, cut:], w, fa)
        np.testing.assert_allclose(np.concatenate([ya, yb], axis=1), y, rtol=1e-15, atol=1e-15)
        np.testing.assert_array_equal(fb, fin)
    st = init
    for t in range(30):                                             # one token per call
        yt, st = oracle.short_conv(x[:, t:t + 1], w, st)
        np.testing.assert_allclose(yt[0, 0], y[0, t], rtol=1e-15, atol=1e-15)
    # a sequence shorter than the window keeps part of its incoming state
    _, f2 = oracle.short_conv(x[:, :2], w, init)
    np.testing.assert_array_equal(f2[0], np.concatenate([init[0, 2:], x[0, :2]]))


def test_short_conv_packed_sequences_are_isolated():
    rng = np.random.default_rng(84)
    lens = [5, 0, 1, 12]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = rng.standard_normal((1, cu[-1], 4))
    w = rng.standard_normal((4, 4))
    init = rng.standard_normal((4, 3, 4))
    y, fin = oracle.short_conv(x, w, init, cu)
    for n in range(4):
        yn, fn = oracle.short_conv(x[:, cu[n]:cu[n + 1]], w, init[n:n + 1])
        np.testing.assert_array_equal(y[:, cu[n]:cu[n + 1]], yn)
        np.testing.assert_array_equal(fin[n], fn[0])
    np.testing.assert_array_equal(fin[1], init[1])                   # empty sequence: state passes through


def test_conv_then_recurrence_first_token_closed_form():
    # zero conv state and zero recurrent state: q, k, v become silu(w_3 x)
    # and the first output is scale beta (k^ . q^) v_c
    rng = np.random.default_rng(85)
    d = 8
    q, k, v, g, beta = _rand_chain(rng, 1, d, d)
    ws = [rng.standard_normal((d, 4)) for _ in range(3)]
    o, _, fin = oracle.forward_conv(q[None, :, None], k[None, :, None], v[None, :, None], g[None, :, None],
                                    beta[None, :, None], ws, scale=0.5)
    qc, kc, vc = (oracle.silu(ws[i][:, 3] * x[0].astype(np.float64)) for i, x in enumerate((q, k, v)))
    expect = 0.5 * float(beta[0]) * float(_unit(kc) @ _unit(qc)) * vc
    np.testing.assert_allclose(o[0, 0, 0], expect, rtol=1e-6, atol=1e-7)   # the conv output reaches fp32 once
    np.testing.assert_array_equal(fin[0][0], np.concatenate([np.zeros((2, d)), q[None, 0].astype(np.float64)]))


# ---------------------------------------------------------------------------
# Decode helpers: one token per call carries the state, so iterating them is
# the whole-sequence run split at every token ("Kimi K3 の KDA ..." sections
# 2.3.4.2 and 2.3.4.5: composing the per-segment affine maps in order gives
# the map of the concatenation; a segment may be a single token).  Each pin
# uses N >= 2 sequences and H >= 2 heads with distinct states and inputs, so
# a reshape that mixes the sequence, head or token axes changes the result,
# and each compares against a per-chain computation written out separately.
# ---------------------------------------------------------------------------
def _dec_inputs(rng, T, N, H, dk, dv):
    q = rng.standard_normal((T, N, H, dk)).astype(np.float32)
    k = rng.standard_normal((T, N, H, dk)).astype(np.float32)
    v = rng.standard_normal((T, N, H, dv)).astype(np.float32)
    g = rng.uniform(-5.0, 0.0, (T, N, H, dk)).astype(np.float32)
    beta = rng.uniform(0.0, 1.0, (T, N, H)).astype(np.float32)
    S0 = rng.standard_normal((N, H, dk, dv))
    return q, k, v, g, beta, S0


def test_decode_steps_iterated_is_the_sequence_run():
    rng = np.random.default_rng(91)
    T, N, H, dk, dv = 7, 3, 2, 4, 5
    q, k, v, g, beta, S0 = _dec_inputs(rng, T, N, H, dk, dv)
    st = S0.copy()
    o_steps = np.empty((T, N, H, dv))
    for t in range(T):
        o_steps[t], st = oracle.decode_steps(st, q[t], k[t], v[t], g[t], beta[t], scale=0.75)
    # the same tokens as N sequences of T tokens in one call
    o_seq, s_seq = oracle.forward_arrays(q.transpose(1, 0, 2, 3), k.transpose(1, 0, 2, 3), v.transpose(1, 0, 2, 3),
                                         g.transpose(1, 0, 2, 3), beta.transpose(1, 0, 2), S0, scale=0.75)
    np.testing.assert_allclose(o_steps.transpose(1, 0, 2, 3), o_seq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st, s_seq, rtol=1e-12, atol=1e-12)
    # and chain by chain through the explicit transition products
    for n in range(N):
        for h in range(H):
            o_ref, s_ref = oracle.product_form(q[:, n, h], k[:, n, h], v[:, n, h], g[:, n, h], beta[:, n, h],
                                               S0[n, h], scale=0.75)
            np.testing.assert_allclose(o_steps[:, n, h], o_ref, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(st[n, h], s_ref, rtol=1e-10, atol=1e-12)


def test_decode_gated_is_the_map_then_the_step():
    rng = np.random.default_rng(92)
    T, N, H, dk, dv = 4, 2, 3, 4, 3
    q, k, v, _, _, S0 = _dec_inputs(rng, T, N, H, dk, dv)
    z = rng.standard_normal((T, N, H, dk))
    bl = rng.standard_normal((T, N, H))
    A_log = np.array([-0.7, 0.2, 0.9])              # distinct per head
    dt_bias = rng.standard_normal((H, dk))           # distinct per (head, channel)
    st = S0.copy()
    outs = []
    for t in range(T):
        o, st = oracle.decode_gated(st, q[t], k[t], v[t], z[t], A_log, dt_bias, bl[t])
        outs.append(o)
    # per chain, with the bounded map and the sigmoid evaluated element by
    # element: g = -5 / (1 + exp(-e^A (z + bias))), beta = 1 / (1 + exp(-b))
    for n in range(N):
        for h in range(H):
            gg = np.array([[-5.0 / (1.0 + np.exp(-np.exp(A_log[h]) * (z[t, n, h, c] + dt_bias[h, c])))
                            for c in range(dk)] for t in range(T)])
            bb = np.array([1.0 / (1.0 + np.exp(-bl[t, n, h])) for t in range(T)])
            # the recurrence reads g and beta rounded once to fp32
            o_ref, s_ref = oracle.product_form(q[:, n, h], k[:, n, h], v[:, n, h], gg.astype(np.float32),
                                               bb.astype(np.float32), S0[n, h])
            np.testing.assert_allclose(np.array([o[n, h] for o in outs]), o_ref, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(st[n, h], s_ref, rtol=1e-10, atol=1e-12)


def _conv_by_hand(x, w, prev):
    """Causal width-4 convolution + SiLU of one channel written as a loop:
    y_t = silu(sum_j w[j] x_{t-3+j}), with x_{-3..-1} = prev."""
    xs = list(prev) + list(x)
    y = []
    for t in range(len(x)):
        a = sum(w[j] * xs[t + j] for j in range(4))
        y.append(a / (1.0 + np.exp(-a)))
    return np.array(y), np.array(xs[len(x):len(x) + 3])


def test_decode_conv_iterated_is_the_sequence_convolution():
    rng = np.random.default_rng(93)
    T, N, H, dk, dv = 6, 3, 2, 3, 2
    xs = [rng.standard_normal((T, N, H, d)) for d in (dk, dk, dv)]
    ws = [rng.standard_normal((H * d, 4)) for d in (dk, dk, dv)]
    caches = [rng.standard_normal((N, 3, H * d)) for d in (dk, dk, dv)]
    st = [c.copy() for c in caches]
    outs = []
    for t in range(T):
        y, st = oracle.decode_conv(st, ws, xs[0][t], xs[1][t], xs[2][t])
        outs.append(y)
    for i, d in enumerate((dk, dk, dv)):
        # whole sequences through short_conv: [N, T, H*d], one state per sequence
        seq = xs[i].transpose(1, 0, 2, 3).reshape(N, T, H * d)
        for n in range(N):
            y_seq, f_seq = oracle.short_conv(seq[n:n + 1], ws[i], caches[i][n:n + 1])
            y_dec = np.stack([outs[t][i][n].reshape(H * d) for t in range(T)])
            np.testing.assert_allclose(y_dec, y_seq[0], rtol=1e-13, atol=1e-13)
            np.testing.assert_array_equal(st[i][n], f_seq[0])
            for h in range(H):                         # channel h*d + c is (head h, channel c)
                for c in range(d):
                    yh, fh = _conv_by_hand(xs[i][:, n, h, c], ws[i][h * d + c], caches[i][n, :, h * d + c])
                    np.testing.assert_allclose(y_dec[:, h * d + c], yh, rtol=1e-13, atol=1e-13)
                    np.testing.assert_array_equal(st[i][n, :, h * d + c], fh)


def test_conv_qkv_convolves_each_head_slice_with_its_taps():
    rng = np.random.default_rng(94)
    B, T, H, dk, dv = 2, 9, 3, 4, 2
    xs = [rng.standard_normal((B, T, H, d)) for d in (dk, dk, dv)]
    ws = [rng.standard_normal((H * d, 4)) for d in (dk, dk, dv)]
    inits = [rng.standard_normal((B, 3, H * d)) for d in (dk, dk, dv)]
    (yq, yk, yv), finals = oracle.conv_qkv(xs[0], xs[1], xs[2], ws, inits)
    for i, (y, d) in enumerate(zip((yq, yk, yv), (dk, dk, dv))):
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            ys, fs = oracle.short_conv(xs[i][:, :, h], ws[i][sl], inits[i][:, :, sl])
            np.testing.assert_array_equal(y[:, :, h], ys)
            np.testing.assert_array_equal(finals[i][:, :, sl], fs)
            for b in range(B):
                for c in range(d):
                    yh, fh = _conv_by_hand(xs[i][b, :, h, c], ws[i][h * d + c], inits[i][b, :, h * d + c])
                    np.testing.assert_allclose(y[b, :, h, c], yh, rtol=1e-13, atol=1e-13)
                    np.testing.assert_array_equal(finals[i][b, :, h * d + c], fh)
