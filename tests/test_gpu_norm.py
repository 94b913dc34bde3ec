"""GPU parity of the fused output norm (o <- o / sqrt(mean(o^2) + eps) * w *
sigmoid(gate) per (token, head) row) against the fp64 oracle's recurrence
followed by its out_norm.  Every kernel family that can carry the norm is
covered: the matrix-core prefill (the sequential kernel normalises o as it
stores it, its two value-slice workgroups exchanging per-row sums of o^2),
the exact fp32 prefill (separate norm pass over fp32 o) and the decode step
(norm in the lanes that hold o).  Marked ``gpu``."""
import numpy as np
import pytest

import kda_inputs
import oracle
from gpu_util import check, check_state, dev, host64

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
EPS = 1e-5


@pytest.fixture(scope="module")
def kda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_fwd_amd as m
    m.load()
    return m


def _f64(a):
    return kda_inputs.bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _plain(kda, inp, gate, w, out_dtype, **kw):
    import torch
    o, s = kda.chunk_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state),
                         dev(inp.cu_seqlens), out_dtype=out_dtype, out_gate=dev(gate), norm_weight=dev(w),
                         norm_eps=EPS, **kw)
    torch.cuda.synchronize()
    return o, s


@pytest.mark.parametrize("use_w", [True, False])
def test_norm_matrix_core_prefill(kda, use_w):
    """bf16, d=128: the sequential kernel with the norm at the store of o
    (row sums exchanged between the two value slices); ragged T, both output
    dtypes, with and without the gain."""
    import torch
    inp = kda_inputs.make_prefill(31, 1, 1000, 8, 128, 128, s0_std=0.02)
    gate = kda_inputs.make_out_gate(31, inp.v.shape)
    w = kda_inputs.norm_weight(31, 128) if use_w else None
    o_ref, s_ref = oracle.forward(inp)
    y_ref = oracle.out_norm(o_ref, _f64(gate), w, EPS)
    for odt in (torch.bfloat16, torch.float32):
        o, s = _plain(kda, inp, gate, w, odt)
        check("norm_mfma_w%d/%s" % (use_w, str(odt).split(".")[-1]), host64(o), y_ref, host64(s), s_ref, TOL_BF16,
              bf16_store=(odt == torch.bfloat16))


def test_norm_matrix_core_batched_and_varlen(kda):
    import torch
    inp = kda_inputs.make_prefill(32, 2, 300, 4, 128, 128, s0_std=0.02)
    gate = kda_inputs.make_out_gate(32, inp.v.shape)
    w = kda_inputs.norm_weight(32, 128)
    o_ref, s_ref = oracle.forward(inp)
    o, s = _plain(kda, inp, gate, w, torch.float32)
    check("norm_mfma_B2", host64(o), oracle.out_norm(o_ref, _f64(gate), w, EPS), host64(s), s_ref, TOL_BF16,
          bf16_store=False)
    inp = kda_inputs.make_prefill(33, 1, 0, 4, 128, 128, lengths=[1, 65, 0, 130, 700, 64])
    gate = kda_inputs.make_out_gate(33, inp.v.shape)
    o_ref, s_ref = oracle.forward(inp)
    o, s = _plain(kda, inp, gate, w, torch.bfloat16)
    check("norm_mfma_varlen", host64(o), oracle.out_norm(o_ref, _f64(gate), w, EPS), host64(s), s_ref, TOL_BF16,
          bf16_store=True)


def test_norm_with_gate_prologue_is_the_fused_layer(kda):
    """Decay-gate prologue and output norm in one call (kda_chunk_fwd_fused
    with both), beta from logits."""
    import torch
    inp = kda_inputs.make_gated_prefill(34, 1, 777, 4, 128, 128, s0_std=0.02)
    gate = kda_inputs.make_out_gate(34, inp.v.shape)
    w = kda_inputs.norm_weight(34, 128)
    o_ref, s_ref = oracle.forward_gated(inp)
    y_ref = oracle.out_norm(o_ref, _f64(gate), w, EPS)
    for fp32_path in (False, True):
        o, s = kda.chunk_fwd_gated(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.z), dev(inp.A_log),
                                   dev(inp.beta_logits), dev(inp.init_state), dt_bias=dev(inp.dt_bias),
                                   beta_logits=True, out_dtype=torch.float32, out_gate=dev(gate), norm_weight=dev(w),
                                   norm_eps=EPS, fp32_path=fp32_path)
        torch.cuda.synchronize()
        check("norm_gated_fp32path%d" % fp32_path, host64(o), y_ref, host64(s), s_ref,
              TOL_F32 * 10 if fp32_path else TOL_BF16, bf16_store=False)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 128)])
def test_norm_fp32_path(kda, dk, dv):
    """fp32 inputs: the exact path writes fp32 o to the workspace and a
    second kernel applies the norm."""
    import torch
    inp = kda_inputs.make_prefill(35, 1, 300, 3, dk, dv, dtype="f32", s0_std=0.02)
    gate = kda_inputs.make_out_gate(35, inp.v.shape, dtype="f32")
    w = kda_inputs.norm_weight(35, dv)
    o_ref, s_ref = oracle.forward(inp)
    y_ref = oracle.out_norm(o_ref, gate.astype(np.float64), w, EPS)
    for odt in (torch.float32, torch.bfloat16):
        o, s = _plain(kda, inp, gate, w, odt)
        check("norm_fp32_%dx%d/%s" % (dk, dv, str(odt).split(".")[-1]), host64(o), y_ref, host64(s), s_ref,
              TOL_F32 if odt == torch.float32 else TOL_BF16, bf16_store=(odt == torch.bfloat16))


def test_norm_signed_alpha(kda):
    import torch
    inp = kda_inputs.make_signed_prefill(36, 1, 500, 4, 128, 128, s0_std=0.02)
    gate = kda_inputs.make_out_gate(36, inp.v.shape)
    o_ref, s_ref = oracle.forward_signed(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.g, inp.beta,
                                         inp.init_state)
    o, s = _plain(kda, inp, gate, None, torch.float32, signed_alpha=True)
    check("norm_signed", host64(o), oracle.out_norm(o_ref, _f64(gate), None, EPS), host64(s), s_ref, TOL_BF16,
          bf16_store=False)


def test_norm_with_validate(kda):
    import torch
    inp = kda_inputs.make_prefill(37, 1, 200, 2, 128, 128)
    gate = kda_inputs.make_out_gate(37, inp.v.shape)
    o_ref, s_ref = oracle.forward(inp)
    o, s = _plain(kda, inp, gate, None, torch.float32, validate=True)
    check("norm_validate", host64(o), oracle.out_norm(o_ref, _f64(gate), None, EPS), host64(s), s_ref, TOL_BF16,
          bf16_store=False)


@pytest.mark.parametrize("dtype,d,gated", [("bf16", 128, False), ("f32", 64, False), ("bf16", 128, True)])
def test_norm_decode_steps(kda, dtype, d, gated):
    """Eight decode steps carrying the state, each with the fused norm."""
    import torch
    N, H, steps = 16, 8, 8
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    S0 = kda_inputs.decode_initial_state(38, N, H, d, 0.02)
    A_log, dt_bias = kda_inputs.gate_params(38, H, d)
    w = kda_inputs.norm_weight(38, d)
    state = dev(S0)
    s_ref = S0.astype(np.float64)
    for step in range(steps):
        gate = kda_inputs.make_out_gate(1000 + step, (N, H, d), dtype=dtype)
        if gated:
            x = kda_inputs.gated_decode_step(38, step, N, H, d, dtype=dtype)
            o_ref, s_ref = oracle.decode_gated(s_ref, _f64(x.q), _f64(x.k), _f64(x.v), _f64(x.z), A_log, dt_bias,
                                               x.beta_logits)
            o = kda.recurrent_step_gated(dev(x.q), dev(x.k), dev(x.v), dev(x.z), dev(A_log), dev(x.beta_logits),
                                         state, dt_bias=dev(dt_bias), beta_logits=True, out_dtype=torch.float32,
                                         out_gate=dev(gate), norm_weight=dev(w), norm_eps=EPS)
        else:
            x = kda_inputs.decode_step(38, step, N, H, d, dtype=dtype)
            o_ref, s_ref = oracle.decode_steps(s_ref, _f64(x.q), _f64(x.k), _f64(x.v), x.g, x.beta)
            o = kda.recurrent_step(dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), state,
                                   out_dtype=torch.float32, out_gate=dev(gate), norm_weight=dev(w), norm_eps=EPS)
        torch.cuda.synchronize()
        check("norm_decode_%s_g%d/step%d" % (dtype, gated, step), host64(o),
              oracle.out_norm(o_ref, _f64(gate), w, EPS), None, None, tol, bf16_store=False)
    check_state("norm_decode_%s_g%d/final" % (dtype, gated), host64(state), s_ref, tol)


@pytest.mark.parametrize("odt_name", ["bfloat16", "float32"])
def test_norm_matrix_core_short_sequences(kda, odt_name):
    """The matrix-core norm finishes each chunk one chunk after its row sums
    are exchanged and flushes the last two at the end: packed sequences of
    one, two, three and more chunks (and empty ones), both output dtypes."""
    import torch
    odt = getattr(torch, odt_name)
    lens = [1, 64, 65, 128, 0, 129, 192, 193, 300, 17]
    inp = kda_inputs.make_prefill(41, 1, 0, 3, 128, 128, s0_std=0.02, lengths=lens)
    gate = kda_inputs.make_out_gate(41, inp.v.shape)
    w = kda_inputs.norm_weight(41, 128)
    o_ref, s_ref = oracle.forward(inp)
    y_ref = oracle.out_norm(o_ref, _f64(gate), w, EPS)
    o, s = _plain(kda, inp, gate, w, odt)
    check("norm_short/%s" % odt_name, host64(o), y_ref, host64(s), s_ref, TOL_BF16, bf16_store=(odt == torch.bfloat16))


def test_norm_matrix_core_workspace_reuse(kda):
    """Two calls with different inputs in one workspace: the second equals the
    same call in a fresh workspace bit for bit (the row-sum words the value
    slices exchange are cleared at the start of every call, so words a
    previous call left behind cannot pass for the current chunk's)."""
    import torch
    B, T, H = 1, 700, 4
    ins = [kda_inputs.make_prefill(42 + i, B, T, H, 128, 128, s0_std=0.02) for i in range(2)]
    gates = [dev(kda_inputs.make_out_gate(42 + i, (B, T, H, 128))) for i in range(2)]
    ws = torch.empty(kda.workspace_bytes(B, T, H, 128, 128, flags=kda.FLAG_QK_L2NORM | kda.FLAG_OUT_NORM),
                     dtype=torch.uint8, device="cuda")
    outs = []
    for i in (0, 1):
        x = ins[i]
        o, s = kda.chunk_fwd(dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), dev(x.init_state),
                             out_gate=gates[i], norm_eps=EPS, workspace=ws)
        torch.cuda.synchronize()
        outs.append((o, s))
    x = ins[1]
    o2, s2 = kda.chunk_fwd(dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), dev(x.init_state),
                           out_gate=gates[1], norm_eps=EPS)
    torch.cuda.synchronize()
    assert torch.equal(outs[1][0], o2) and torch.equal(outs[1][1], s2)
