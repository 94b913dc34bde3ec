"""GPU parity of Complex KDA (KDA_FLAG_SIGNED_ALPHA: signed per-channel
decay alpha in [-1, 1], beta in [0, 2]) against the oracle's signed-alpha
recurrence.  Marked ``gpu``."""
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


def _oracle(inp):
    return oracle.forward_signed(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.g, inp.beta,
                                 inp.f32("init_state") if inp.init_state is not None else None, inp.cu_seqlens)


def _run(kda, inp, odt, **kw):
    import torch
    o, s = kda.chunk_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state),
                         dev(inp.cu_seqlens), out_dtype=odt, signed_alpha=True, **kw)
    torch.cuda.synchronize()
    return o, s


def test_signed_prefill_matrix_core_path(kda):
    """bf16, d=128: the two-pass path with the running sign folded in."""
    import torch
    inp = kda_inputs.make_signed_prefill(31, 1, 1100, 8, 128, 128, s0_std=0.02)
    o_ref, s_ref = _oracle(inp)
    for odt in (torch.bfloat16, torch.float32):
        o, s = _run(kda, inp, odt)
        check("signed_mfma/%s" % str(odt).split(".")[-1], host64(o), o_ref, host64(s), s_ref, TOL_BF16,
              bf16_store=(odt == torch.bfloat16))


def test_signed_prefill_fp32_path(kda):
    import torch
    inp = kda_inputs.make_signed_prefill(32, 1, 300, 2, 64, 64, dtype="f32", s0_std=0.02)
    o_ref, s_ref = _oracle(inp)
    o, s = _run(kda, inp, torch.float32)
    check("signed_fp32_d64", host64(o), o_ref, host64(s), s_ref, TOL_F32, bf16_store=False)
    inp = kda_inputs.make_signed_prefill(33, 1, 400, 3, 128, 128, s0_std=0.02)
    o_ref, s_ref = _oracle(inp)
    o, s = _run(kda, inp, torch.float32, fp32_path=True)
    check("signed_bf16_fp32path", host64(o), o_ref, host64(s), s_ref, TOL_F32 * 10, bf16_store=False)


def test_signed_prefill_varlen_and_validate(kda):
    import torch
    inp = kda_inputs.make_signed_prefill(34, 1, 0, 4, 128, 128, lengths=[1, 65, 0, 130, 700, 64])
    o_ref, s_ref = _oracle(inp)
    o, s = _run(kda, inp, torch.float32, validate=True)
    check("signed_varlen", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)


def test_signed_reflections_and_rotations(kda):
    """alpha in {-1, +1} with beta = 2: every transition is orthogonal (the
    page's rotation regime), over a long sequence on the matrix-core path."""
    import torch
    inp = kda_inputs.make_signed_prefill(35, 1, 2048, 4, 128, 128, s0_std=0.02)
    rng = np.random.default_rng(35)
    inp.g = np.where(rng.uniform(size=inp.g.shape) < 0.5, -1.0, 1.0).astype(np.float32)
    inp.beta = np.full(inp.beta.shape, 2.0, np.float32)
    o_ref, s_ref = _oracle(inp)
    o, s = _run(kda, inp, torch.float32)
    check("signed_orthogonal", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)


def test_signed_validate_rejects_out_of_range(kda):
    import torch
    inp = kda_inputs.make_signed_prefill(36, 1, 128, 2, 128, 128)
    bad = inp.g.copy()
    bad[0, 5, 1, 7] = 1e-3                      # |alpha| below e^-5
    with pytest.raises(kda.KDAError) as e:
        kda.chunk_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(bad), dev(inp.beta), signed_alpha=True,
                      validate=True, out_dtype=torch.float32)
    assert e.value.status == 4
    beta = inp.beta.copy()
    beta[0, 3, 0] = 2.5                           # beta above 2
    with pytest.raises(kda.KDAError) as e:
        kda.chunk_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(beta), signed_alpha=True,
                      validate=True, out_dtype=torch.float32)
    assert e.value.status == 4


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_signed_decode_steps(kda, dtype, d):
    import torch
    N, H, steps = 16, 8, 8
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    S0 = kda_inputs.decode_initial_state(37, N, H, d, 0.02)
    state = dev(S0)
    s_ref = S0.astype(np.float64)
    f = lambda a: kda_inputs.bf16_to_f32(a) if a.dtype == np.uint16 else a
    for step in range(steps):
        x = kda_inputs.signed_decode_step(37, step, N, H, d, dtype=dtype)
        o_ref, s_ref = oracle.decode_steps(s_ref, f(x.q), f(x.k), f(x.v), x.g, x.beta, alpha_given=True)
        o = kda.recurrent_step(dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), state, out_dtype=torch.float32,
                               signed_alpha=True)
        torch.cuda.synchronize()
        check("signed_decode_%s/step%d" % (dtype, step), host64(o), o_ref, None, None, tol, bf16_store=False)
    check_state("signed_decode_%s/final" % dtype, host64(state), s_ref, tol)
