"""GPU parity of the gated entry points (gate prologue fused into the forward
pass: g = -5 sigmoid(e^{A_h} (z + dt_bias)), beta = sigmoid(logit)) against
the fp64 oracle's gate map followed by its recurrence.  Marked ``gpu``."""
import numpy as np
import pytest

import kda_inputs
import oracle
from gpu_util import check, check_state, dev, host64

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


@pytest.fixture(scope="module")
def kda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_fwd_amd as m
    m.load()
    return m


def _run_gated(kda, inp, out_dtype, beta_logits=True, use_bias=True, **kw):
    import torch
    o, s = kda.chunk_fwd_gated(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.z), dev(inp.A_log),
                               dev(inp.beta_logits), dev(inp.init_state), dev(inp.cu_seqlens),
                               dt_bias=dev(inp.dt_bias) if use_bias else None, out_dtype=out_dtype,
                               beta_logits=beta_logits, **kw)
    torch.cuda.synchronize()
    return o, s


def _oracle(inp, use_bias=True):
    if not use_bias:
        inp = kda_inputs.GatedPrefillInputs(**{**inp.__dict__, "dt_bias": np.zeros_like(inp.dt_bias)})
    return oracle.forward_gated(inp)


@pytest.mark.parametrize("use_bias", [True, False])
def test_gated_prefill_matrix_core_path(kda, use_bias):
    """bf16, d=128 (two-pass matrix-core path), ragged T, both output dtypes."""
    import torch
    inp = kda_inputs.make_gated_prefill(21, 1, 1000, 8, 128, 128, s0_std=0.02)
    o_ref, s_ref = _oracle(inp, use_bias)
    for odt in (torch.bfloat16, torch.float32):
        o, s = _run_gated(kda, inp, odt, use_bias=use_bias)
        check("gated_mfma_bias%d/%s" % (use_bias, str(odt).split(".")[-1]), host64(o), o_ref, host64(s), s_ref,
              TOL_BF16, bf16_store=(odt == torch.bfloat16))


def test_gated_prefill_fp32_path(kda):
    """fp32 inputs, d=64 (exact fp32 path), and bf16 inputs forced onto it."""
    import torch
    inp = kda_inputs.make_gated_prefill(22, 1, 300, 2, 64, 64, dtype="f32", s0_std=0.02)
    o_ref, s_ref = _oracle(inp)
    o, s = _run_gated(kda, inp, torch.float32)
    check("gated_fp32_d64", host64(o), o_ref, host64(s), s_ref, TOL_F32, bf16_store=False)
    inp = kda_inputs.make_gated_prefill(23, 1, 400, 3, 128, 128, s0_std=0.02)
    o_ref, s_ref = _oracle(inp)
    o, s = _run_gated(kda, inp, torch.float32, fp32_path=True)
    check("gated_bf16_fp32path", host64(o), o_ref, host64(s), s_ref, TOL_F32 * 10, bf16_store=False)


def test_gated_prefill_varlen(kda):
    """Packed sequences with empty, one-token and partial-chunk members."""
    import torch
    inp = kda_inputs.make_gated_prefill(24, 1, 0, 4, 128, 128, lengths=[1, 65, 0, 130, 700, 64])
    o_ref, s_ref = _oracle(inp)
    for odt in (torch.bfloat16, torch.float32):
        o, s = _run_gated(kda, inp, odt)
        check("gated_varlen/%s" % str(odt).split(".")[-1], host64(o), o_ref, host64(s), s_ref, TOL_BF16,
              bf16_store=(odt == torch.bfloat16))


def test_beta_logits_on_the_plain_entry_point(kda):
    """KDA_FLAG_BETA_LOGITS with a given g: beta = sigmoid(logit) in the kernel."""
    import torch
    inp = kda_inputs.make_prefill(25, 1, 500, 4, 128, 128, s0_std=0.02)
    logits = np.log(inp.beta / (1.0 - inp.beta)).astype(np.float32)     # the same strengths as logits
    o_ref, s_ref = oracle.forward(inp)
    o, s = kda.chunk_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(logits), dev(inp.init_state),
                         out_dtype=torch.float32, beta_logits=True)
    torch.cuda.synchronize()
    check("plain_beta_logits", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)


def test_gated_validate_accepts_in_range_inputs(kda):
    import torch
    inp = kda_inputs.make_gated_prefill(26, 1, 200, 2, 128, 128)
    o_ref, s_ref = _oracle(inp)
    o, s = _run_gated(kda, inp, torch.float32, validate=True)
    check("gated_validate", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_gated_decode_steps(kda, dtype, d):
    """Eight gated decode steps carrying the state, against the oracle step."""
    import torch
    N, H, steps = 16, 8, 8
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    A_log, dt_bias = kda_inputs.gate_params(27, H, d)
    S0 = kda_inputs.decode_initial_state(27, N, H, d, 0.02)
    state = dev(S0)
    s_ref = S0.astype(np.float64)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for step in range(steps):
        x = kda_inputs.gated_decode_step(27, step, N, H, d, dtype=dtype)
        f = lambda a: kda_inputs.bf16_to_f32(a) if a.dtype == np.uint16 else a
        o_ref, s_ref = oracle.decode_gated(s_ref, f(x.q), f(x.k), f(x.v), f(x.z), A_log, dt_bias, x.beta_logits)
        o = kda.recurrent_step_gated(dev(x.q), dev(x.k), dev(x.v), dev(x.z), dev(A_log), dev(x.beta_logits), state,
                                     dt_bias=dev(dt_bias), out_dtype=torch.float32, beta_logits=True)
        torch.cuda.synchronize()
        check("gated_decode_%s/step%d" % (dtype, step), host64(o), o_ref, None, None, tol, bf16_store=False)
    check_state("gated_decode_%s/final" % dtype, host64(state), s_ref, tol)
    assert tdt in (torch.bfloat16, torch.float32)
