"""GPU parity of the fused short convolution (q, k, v = silu(causal width-4
depthwise conv) of the raw projections, with a 3-token conv state) against the
fp64 oracle's short_conv followed by its recurrence.  Covers the matrix-core
prefill (conv in pass 1 for q, k and in the scan pass's V fetch), the exact
fp32 prefill, the decode step with its in-place cache, the conv states written
after a prefill (bit-exact: they are copies of raw inputs), and a prefill
continued by decode steps.  Marked ``gpu``."""
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


def _f(a):
    return kda_inputs.bf16_to_f32(a) if a.dtype == np.uint16 else a


def _empty_like_states(states):
    import torch
    return tuple(torch.empty(s.shape, dtype=torch.bfloat16 if s.dtype == np.uint16 else torch.float32, device="cuda")
                 for s in states)


def _check_conv_states(name, got, ref_states):
    for i, (gt, ref) in enumerate(zip(got, ref_states)):
        g = host64(gt)
        assert np.array_equal(g, np.asarray(ref, np.float64)), "%s: conv state %d differs (max %g)" % (
            name, i, np.abs(g - ref).max())


def _run_plain(kda, inp, ws, cs, out_dtype, use_init=True, **kw):
    import torch
    finals = _empty_like_states(cs)
    o, s = kda.chunk_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state),
                         dev(inp.cu_seqlens), out_dtype=out_dtype, conv_weights=tuple(dev(w) for w in ws),
                         conv_init=tuple(dev(c) for c in cs) if use_init else None, conv_final=finals, **kw)
    torch.cuda.synchronize()
    return o, s, finals


def _oracle(inp, ws, cs, use_init=True):
    return oracle.forward_conv(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.g, inp.beta, ws,
                               tuple(_f(c) for c in cs) if use_init else None, inp.init_state, inp.cu_seqlens)


@pytest.mark.parametrize("use_init", [True, False])
def test_conv_matrix_core_prefill(kda, use_init):
    """bf16, d=128: conv of q, k in pass 1 and of v in the scan pass; ragged T,
    both output dtypes; conv states in and out."""
    import torch
    inp = kda_inputs.make_prefill(41, 1, 1000, 8, 128, 128, s0_std=0.02)
    ws = kda_inputs.conv_weights(41, 8, 128, 128)
    cs = kda_inputs.conv_states(41, 1, 8, 128, 128)
    o_ref, s_ref, f_ref = _oracle(inp, ws, cs, use_init)
    for odt in (torch.bfloat16, torch.float32):
        o, s, fin = _run_plain(kda, inp, ws, cs, odt, use_init)
        check("conv_mfma_init%d/%s" % (use_init, str(odt).split(".")[-1]), host64(o), o_ref, host64(s), s_ref,
              TOL_BF16, bf16_store=(odt == torch.bfloat16))
        _check_conv_states("conv_mfma", fin, f_ref)


def test_conv_matrix_core_batched_and_varlen(kda):
    import torch
    inp = kda_inputs.make_prefill(42, 2, 200, 4, 128, 128, s0_std=0.02)
    ws = kda_inputs.conv_weights(42, 4, 128, 128)
    cs = kda_inputs.conv_states(42, 2, 4, 128, 128)
    o_ref, s_ref, f_ref = _oracle(inp, ws, cs)
    o, s, fin = _run_plain(kda, inp, ws, cs, torch.float32)
    check("conv_mfma_B2", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)
    _check_conv_states("conv_mfma_B2", fin, f_ref)
    # sequences shorter than the window keep part of their incoming state
    lens = [1, 2, 65, 0, 130, 700, 64, 3]
    inp = kda_inputs.make_prefill(43, 1, 0, 4, 128, 128, lengths=lens, s0_std=0.02)
    cs = kda_inputs.conv_states(43, len(lens), 4, 128, 128)
    o_ref, s_ref, f_ref = _oracle(inp, ws, cs)
    o, s, fin = _run_plain(kda, inp, ws, cs, torch.bfloat16)
    check("conv_mfma_varlen", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=True)
    _check_conv_states("conv_mfma_varlen", fin, f_ref)


def test_conv_state_in_place(kda):
    """conv_final aliasing conv_init: the outgoing state overwrites the
    incoming one only after every kernel that reads it."""
    import torch
    inp = kda_inputs.make_prefill(44, 1, 0, 4, 128, 128, lengths=[2, 70, 1], s0_std=0.02)
    ws = kda_inputs.conv_weights(44, 4, 128, 128)
    cs = kda_inputs.conv_states(44, 3, 4, 128, 128)
    o_ref, s_ref, f_ref = _oracle(inp, ws, cs)
    for fp32_path in (False, True):
        st = tuple(dev(c) for c in cs)
        o, s = kda.chunk_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state),
                             dev(inp.cu_seqlens), out_dtype=torch.float32, conv_weights=tuple(dev(w) for w in ws),
                             conv_init=st, conv_final=st, fp32_path=fp32_path)
        torch.cuda.synchronize()
        check("conv_inplace_fp32path%d" % fp32_path, host64(o), o_ref, host64(s), s_ref,
              TOL_F32 * 10 if fp32_path else TOL_BF16, bf16_store=False)
        _check_conv_states("conv_inplace", st, f_ref)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 128)])
def test_conv_fp32_path(kda, dk, dv):
    import torch
    inp = kda_inputs.make_prefill(45, 1, 0, 3, dk, dv, dtype="f32", lengths=[150, 2, 90], s0_std=0.02)
    ws = kda_inputs.conv_weights(45, 3, dk, dv)
    cs = kda_inputs.conv_states(45, 3, 3, dk, dv, dtype="f32")
    o_ref, s_ref, f_ref = _oracle(inp, ws, cs)
    o, s, fin = _run_plain(kda, inp, ws, cs, torch.float32)
    check("conv_fp32_%dx%d" % (dk, dv), host64(o), o_ref, host64(s), s_ref, TOL_F32, bf16_store=False)
    _check_conv_states("conv_fp32", fin, f_ref)


def test_conv_signed_alpha(kda):
    import torch
    inp = kda_inputs.make_signed_prefill(46, 1, 400, 4, 128, 128, s0_std=0.02)
    ws = kda_inputs.conv_weights(46, 4, 128, 128)
    cs = kda_inputs.conv_states(46, 1, 4, 128, 128)
    o_ref, s_ref, f_ref = oracle.forward_conv(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.g, inp.beta, ws,
                                              tuple(_f(c) for c in cs), inp.init_state, alpha_given=True)
    o, s, fin = _run_plain(kda, inp, ws, cs, torch.float32, signed_alpha=True)
    check("conv_signed", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)
    _check_conv_states("conv_signed", fin, f_ref)


def test_conv_gate_and_norm_the_whole_layer_core(kda):
    """All three fused steps in one call: conv prologue, decay-gate prologue,
    output norm; matrix-core path and fp32 path."""
    import torch
    inp = kda_inputs.make_gated_prefill(47, 1, 500, 4, 128, 128, s0_std=0.02)
    ws = kda_inputs.conv_weights(47, 4, 128, 128)
    cs = kda_inputs.conv_states(47, 1, 4, 128, 128)
    gate = kda_inputs.make_out_gate(47, inp.v.shape)
    w = kda_inputs.norm_weight(47, 128)
    g = oracle.gate_map(inp.f32("z"), inp.A_log, inp.dt_bias)
    o_ref, s_ref, f_ref = oracle.forward_conv(inp.f32("q"), inp.f32("k"), inp.f32("v"), g,
                                              oracle.beta_from_logits(inp.beta_logits), ws, tuple(_f(c) for c in cs),
                                              inp.init_state)
    y_ref = oracle.out_norm(o_ref, _f(gate).astype(np.float64), w, 1e-5)
    for fp32_path in (False, True):
        finals = _empty_like_states(cs)
        o, s = kda.chunk_fwd_gated(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.z), dev(inp.A_log),
                                   dev(inp.beta_logits), dev(inp.init_state), dt_bias=dev(inp.dt_bias),
                                   beta_logits=True, out_dtype=torch.float32, out_gate=dev(gate), norm_weight=dev(w),
                                   norm_eps=1e-5, conv_weights=tuple(dev(x) for x in ws),
                                   conv_init=tuple(dev(c) for c in cs), conv_final=finals, fp32_path=fp32_path)
        torch.cuda.synchronize()
        check("conv_layer_fp32path%d" % fp32_path, host64(o), y_ref, host64(s), s_ref,
              TOL_F32 * 10 if fp32_path else TOL_BF16, bf16_store=False)
        _check_conv_states("conv_layer", finals, f_ref)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_conv_decode_steps(kda, dtype, d):
    """Eight decode steps carrying the recurrent state and the conv cache
    (updated in place)."""
    import torch
    N, H, steps = 16, 8, 8
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    S0 = kda_inputs.decode_initial_state(48, N, H, d, 0.02)
    ws = kda_inputs.conv_weights(48, H, d, d)
    cs = kda_inputs.conv_states(48, N, H, d, d, dtype=dtype)
    state = dev(S0)
    cache = tuple(dev(c) for c in cs)
    s_ref = S0.astype(np.float64)
    c_ref = tuple(_f(c).astype(np.float64) for c in cs)
    for step in range(steps):
        x = kda_inputs.decode_step(48, step, N, H, d, dtype=dtype)
        (qc, kc, vc), c_ref = oracle.decode_conv(c_ref, ws, _f(x.q), _f(x.k), _f(x.v))
        o_ref, s_ref = oracle.decode_steps(s_ref, qc, kc, vc, x.g, x.beta)
        o = kda.recurrent_step(dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), state, out_dtype=torch.float32,
                               conv_weights=tuple(dev(w) for w in ws), conv_state=cache)
        torch.cuda.synchronize()
        check("conv_decode_%s/step%d" % (dtype, step), host64(o), o_ref, None, None, tol, bf16_store=False)
        _check_conv_states("conv_decode_%s/step%d" % (dtype, step), cache, c_ref)
    check_state("conv_decode_%s/final" % dtype, host64(state), s_ref, tol)


def test_prefill_then_decode_continues_the_sequence(kda):
    """A prefill of 300 tokens hands its recurrent state and conv states to
    decode steps; the outputs match the oracle run over the whole sequence."""
    import torch
    H, d, T, steps = 4, 128, 300, 6
    inp = kda_inputs.make_prefill(49, 1, T + steps, H, d, d, s0_std=0.02)
    ws = kda_inputs.conv_weights(49, H, d, d)
    o_all, s_all, f_all = oracle.forward_conv(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.g, inp.beta, ws, None,
                                              inp.init_state)
    head = lambda a: np.ascontiguousarray(a[:, :T])
    cache = tuple(torch.empty((1, 3, H * d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    o, s = kda.chunk_fwd(dev(head(inp.q)), dev(head(inp.k)), dev(head(inp.v)), dev(head(inp.g)), dev(head(inp.beta)),
                         dev(inp.init_state), out_dtype=torch.float32, conv_weights=tuple(dev(w) for w in ws),
                         conv_final=cache)
    torch.cuda.synchronize()
    check("prefill_part", host64(o), o_all[:, :T], None, None, TOL_BF16, bf16_store=False)
    for t in range(T, T + steps):
        row = lambda a: np.ascontiguousarray(a[:, t])
        ot = kda.recurrent_step(dev(row(inp.q)), dev(row(inp.k)), dev(row(inp.v)), dev(row(inp.g)),
                                dev(row(inp.beta)), s, out_dtype=torch.float32,
                                conv_weights=tuple(dev(w) for w in ws), conv_state=cache)
        torch.cuda.synchronize()
        check("decode_after_prefill/t%d" % t, host64(ot), o_all[:, t], None, None, TOL_BF16, bf16_store=False)
    check_state("decode_after_prefill/final", host64(s), s_all, TOL_BF16)
    _check_conv_states("decode_after_prefill", cache, f_all)


def test_layer_decode_step_conv_gate_and_norm(kda):
    """The whole decode step of the layer in one call: short convolution with
    its cache, decay-gate prologue, beta logits, the recurrence, output norm;
    eight steps carrying both states."""
    import torch
    N, H, d, steps = 8, 4, 128, 8
    S0 = kda_inputs.decode_initial_state(50, N, H, d, 0.02)
    ws = kda_inputs.conv_weights(50, H, d, d)
    cs = kda_inputs.conv_states(50, N, H, d, d)
    A_log, dt_bias = kda_inputs.gate_params(50, H, d)
    w = kda_inputs.norm_weight(50, d)
    state, cache = dev(S0), tuple(dev(c) for c in cs)
    s_ref, c_ref = S0.astype(np.float64), tuple(_f(c).astype(np.float64) for c in cs)
    for step in range(steps):
        x = kda_inputs.gated_decode_step(50, step, N, H, d)
        gate = kda_inputs.make_out_gate(2000 + step, (N, H, d))
        (qc, kc, vc), c_ref = oracle.decode_conv(c_ref, ws, _f(x.q), _f(x.k), _f(x.v))
        o_ref, s_ref = oracle.decode_gated(s_ref, qc, kc, vc, _f(x.z), A_log, dt_bias, x.beta_logits)
        y_ref = oracle.out_norm(o_ref, _f(gate).astype(np.float64), w, 1e-5)
        o = kda.recurrent_step_gated(dev(x.q), dev(x.k), dev(x.v), dev(x.z), dev(A_log), dev(x.beta_logits), state,
                                     dt_bias=dev(dt_bias), beta_logits=True, out_dtype=torch.float32,
                                     out_gate=dev(gate), norm_weight=dev(w), norm_eps=1e-5,
                                     conv_weights=tuple(dev(t) for t in ws), conv_state=cache)
        torch.cuda.synchronize()
        check("layer_decode/step%d" % step, host64(o), y_ref, None, None, TOL_BF16, bf16_store=False)
        _check_conv_states("layer_decode/step%d" % step, cache, c_ref)
    check_state("layer_decode/final", host64(state), s_ref, TOL_BF16)


def test_conv_with_validate(kda):
    import torch
    inp = kda_inputs.make_prefill(51, 1, 0, 2, 128, 128, lengths=[100, 0, 37])
    ws = kda_inputs.conv_weights(51, 2, 128, 128)
    cs = kda_inputs.conv_states(51, 3, 2, 128, 128)
    o_ref, s_ref, f_ref = _oracle(inp, ws, cs)
    o, s, fin = _run_plain(kda, inp, ws, cs, torch.float32, validate=True)
    check("conv_validate", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)
    _check_conv_states("conv_validate", fin, f_ref)


def test_layer_core_full_size_sampled_heads(kda):
    """The whole fused layer core at the long-prefill size (B=1, H=96,
    T=65536; the bench's launch): short convolution, gate prologue, output
    norm; the oracle runs on three sampled heads (the convolution, gate map
    and norm act per head and channel, so a head's slice of every input
    suffices)."""
    import torch
    H, d = 96, 128
    inp = kda_inputs.make_gated_prefill(2, 1, 65536, H, d, d, s0_std=0.02)
    ws = kda_inputs.conv_weights(2, H, d, d)
    cs = kda_inputs.conv_states(2, 1, H, d, d)
    gate = kda_inputs.make_out_gate(2, inp.v.shape)
    w = kda_inputs.norm_weight(2, d)
    finals = _empty_like_states(cs)
    o, s = kda.chunk_fwd_gated(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.z), dev(inp.A_log), dev(inp.beta_logits),
                               dev(inp.init_state), dt_bias=dev(inp.dt_bias), beta_logits=True,
                               out_gate=dev(gate), norm_weight=dev(w), norm_eps=1e-5,
                               conv_weights=tuple(dev(x) for x in ws), conv_init=tuple(dev(c) for c in cs),
                               conv_final=finals)
    torch.cuda.synchronize()
    for h in (0, 51, 95):
        hs, cols = slice(h, h + 1), slice(h * d, (h + 1) * d)
        g = oracle.gate_map(inp.f32("z")[:, :, hs], inp.A_log[hs], inp.dt_bias[hs])
        o_ref, s_ref, f_ref = oracle.forward_conv(
            inp.f32("q")[:, :, hs], inp.f32("k")[:, :, hs], inp.f32("v")[:, :, hs], g,
            oracle.beta_from_logits(inp.beta_logits[:, :, hs]), [x[cols] for x in ws],
            [_f(c)[:, :, cols] for c in cs], inp.init_state[:, hs])
        y_ref = oracle.out_norm(o_ref, _f(gate[:, :, hs]).astype(np.float64), w, 1e-5)
        check("layer_core_64k/h%d" % h, host64(o[:, :, hs]), y_ref, host64(s[:, hs]), s_ref, TOL_BF16,
              bf16_store=True)
        _check_conv_states("layer_core_64k/h%d" % h, [f[:, :, cols] for f in finals], f_ref)
