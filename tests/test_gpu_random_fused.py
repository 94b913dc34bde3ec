"""GPU parity of the fused entry points over seeded random configurations:
per case, the decay input (log-decay g, the gate prologue from logits, or the
signed alpha of Complex KDA), the short convolution (with or without incoming
conv states), the output norm (with or without a gain), the layout (dense or
packed, empty sequences included), head dims, input and output dtypes and the
fp32 path are drawn, and o, the final state and the outgoing conv states are
compared with the fp64 oracle.  Marked ``gpu``."""
import numpy as np
import pytest

import kda_inputs
import oracle
from gpu_util import check, dev, host64

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
CASES = 16
EPS = 1e-5


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


def _draw_case(i):
    r = np.random.default_rng(5000 + i)
    dtype = "f32" if r.random() < 0.2 else "bf16"
    dk, dv = (int(x) for x in r.choice([64, 128], size=2))
    if dtype == "bf16" and r.random() < 0.7:
        dk = dv = 128
    mode = str(r.choice(["plain", "gated", "signed"]))
    packed = r.random() < 0.5
    lengths = [int(x) if r.random() > 0.15 else 0 for x in r.integers(1, 240, size=int(r.integers(1, 5)))] \
        if packed else None
    return dict(dtype=dtype, dk=dk, dv=dv, H=int(r.integers(1, 4)), mode=mode,
                B=1 if packed else int(r.integers(1, 3)), T=0 if packed else int(r.integers(1, 260)),
                lengths=lengths, conv=bool(r.random() < 0.6), conv_init=bool(r.random() < 0.6),
                norm=bool(r.random() < 0.6), norm_w=bool(r.random() < 0.5), s0_std=float(r.choice([0.0, 0.02])),
                out=str(r.choice(["same", "f32"])),
                fp32_path=bool(dtype == "bf16" and dk == dv == 128 and r.random() < 0.3))


@pytest.mark.parametrize("i", range(CASES))
def test_random_fused_prefill(kda, i):
    import torch
    c = _draw_case(i)
    print("case", i, c, flush=True)
    seed = 6000 + i
    B, T, H, dk, dv = c["B"], c["T"], c["H"], c["dk"], c["dv"]
    if c["mode"] == "gated":
        inp = kda_inputs.make_gated_prefill(seed, B, T, H, dk, dv, dtype=c["dtype"], s0_std=c["s0_std"],
                                            lengths=c["lengths"])
        g_ref = oracle.gate_map(inp.f32("z"), inp.A_log, inp.dt_bias)
        b_ref = oracle.beta_from_logits(inp.beta_logits)
    elif c["mode"] == "signed":
        inp = kda_inputs.make_signed_prefill(seed, B, T, H, dk, dv, dtype=c["dtype"], s0_std=c["s0_std"],
                                             lengths=c["lengths"])
        g_ref, b_ref = inp.g, inp.beta
    else:
        inp = kda_inputs.make_prefill(seed, B, T, H, dk, dv, dtype=c["dtype"], s0_std=c["s0_std"],
                                      lengths=c["lengths"])
        g_ref, b_ref = inp.g, inp.beta
    N = B if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1
    T = inp.q.shape[1]
    signed = c["mode"] == "signed"

    ws = cs = None
    if c["conv"]:
        ws = kda_inputs.conv_weights(seed, H, dk, dv)
        cs = kda_inputs.conv_states(seed, N, H, dk, dv, dtype=c["dtype"]) if c["conv_init"] else None
        o_ref, s_ref, f_ref = oracle.forward_conv(inp.f32("q"), inp.f32("k"), inp.f32("v"), g_ref, b_ref, ws,
                                                  None if cs is None else tuple(_f(x) for x in cs),
                                                  inp.init_state, inp.cu_seqlens, alpha_given=signed)
    else:
        o_ref, s_ref = oracle.forward_arrays(inp.f32("q"), inp.f32("k"), inp.f32("v"), g_ref, b_ref,
                                             inp.init_state, inp.cu_seqlens, alpha_given=signed)
    gate = w = None
    if c["norm"]:
        gate = kda_inputs.make_out_gate(seed, (B, T, H, dv), dtype=c["dtype"])
        w = kda_inputs.norm_weight(seed, dv) if c["norm_w"] else None
        o_ref = oracle.out_norm(o_ref, _f(gate).astype(np.float64), w, EPS)

    odt = torch.float32 if (c["out"] == "f32" or c["dtype"] == "f32") else torch.bfloat16
    kw = dict(out_dtype=odt, fp32_path=c["fp32_path"])
    finals = None
    if c["conv"]:
        finals = tuple(torch.empty((N, 3, H * d), dtype=torch.bfloat16 if c["dtype"] == "bf16" else torch.float32,
                                   device="cuda") for d in (dk, dk, dv))
        kw.update(conv_weights=tuple(dev(x) for x in ws), conv_final=finals,
                  conv_init=None if cs is None else tuple(dev(x) for x in cs))
    if c["norm"]:
        kw.update(out_gate=dev(gate), norm_weight=dev(w), norm_eps=EPS)
    if c["mode"] == "gated":
        o, s = kda.chunk_fwd_gated(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.z), dev(inp.A_log),
                                   dev(inp.beta_logits), dev(inp.init_state), dev(inp.cu_seqlens),
                                   dt_bias=dev(inp.dt_bias), beta_logits=True, **kw)
    else:
        o, s = kda.chunk_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state),
                             dev(inp.cu_seqlens), signed_alpha=signed, **kw)
    torch.cuda.synchronize()

    tol = TOL_F32 if (c["dtype"] == "f32" and odt == torch.float32) else TOL_BF16
    if o_ref.size == 0:
        assert o.numel() == 0
        np.testing.assert_array_equal(host64(s), s_ref)
    else:
        check("fused%d" % i, host64(o), o_ref, host64(s), s_ref, tol, bf16_store=(odt == torch.bfloat16))
    if c["conv"]:
        # the outgoing conv states are copies of raw inputs (or of the incoming states): exact
        for x, (got, ref) in enumerate(zip(finals, f_ref)):
            assert np.array_equal(host64(got), np.asarray(ref, np.float64)), "conv state %d" % x


@pytest.mark.parametrize("i", range(8))
def test_random_fused_decode(kda, i):
    """Four decode steps per case with the decay input, the short convolution
    (cache advanced in place) and the output norm drawn per case, carrying
    the fp32 state and the conv cache; the oracle carries them in fp64."""
    import torch
    r = np.random.default_rng(7000 + i)
    N, H = int(r.integers(1, 7)), int(r.integers(1, 4))
    d = int(r.choice([64, 128]))
    dtype = "f32" if r.random() < 0.25 else "bf16"
    mode = str(r.choice(["plain", "gated", "signed"]))
    use_conv, use_norm = bool(r.random() < 0.6), bool(r.random() < 0.6)
    seed = 8000 + i
    print("case", i, dict(N=N, H=H, d=d, dtype=dtype, mode=mode, conv=use_conv, norm=use_norm), flush=True)
    S0 = kda_inputs.decode_initial_state(seed, N, H, d, 0.02)
    state, s_ref = dev(S0), S0.astype(np.float64)
    ws = kda_inputs.conv_weights(seed, H, d, d) if use_conv else None
    cache = c_ref = None
    if use_conv:
        cs = kda_inputs.conv_states(seed, N, H, d, d, dtype=dtype)
        cache, c_ref = tuple(dev(c) for c in cs), tuple(_f(c).astype(np.float64) for c in cs)
    A_log, dt_bias = kda_inputs.gate_params(seed, H, d)
    w = kda_inputs.norm_weight(seed, d) if use_norm else None
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    for step in range(4):
        if mode == "gated":
            x = kda_inputs.gated_decode_step(seed, step, N, H, d, dtype=dtype)
        elif mode == "signed":
            x = kda_inputs.signed_decode_step(seed, step, N, H, d, dtype=dtype)
        else:
            x = kda_inputs.decode_step(seed, step, N, H, d, dtype=dtype)
        q, k, v = _f(x.q), _f(x.k), _f(x.v)
        if use_conv:
            (q, k, v), c_ref = oracle.decode_conv(c_ref, ws, q, k, v)
        if mode == "gated":
            o_ref, s_ref = oracle.decode_gated(s_ref, q, k, v, _f(x.z), A_log, dt_bias, x.beta_logits)
        else:
            o_ref, s_ref = oracle.decode_steps(s_ref, q, k, v, x.g, x.beta, alpha_given=(mode == "signed"))
        kw = dict(out_dtype=torch.float32)
        if use_conv:
            kw.update(conv_weights=tuple(dev(t) for t in ws), conv_state=cache)
        if use_norm:
            gate = kda_inputs.make_out_gate(seed + 100 + step, (N, H, d), dtype=dtype)
            o_ref = oracle.out_norm(o_ref, _f(gate).astype(np.float64), w, EPS)
            kw.update(out_gate=dev(gate), norm_weight=dev(w), norm_eps=EPS)
        if mode == "gated":
            o = kda.recurrent_step_gated(dev(x.q), dev(x.k), dev(x.v), dev(x.z), dev(A_log), dev(x.beta_logits),
                                         state, dt_bias=dev(dt_bias), beta_logits=True, **kw)
        else:
            o = kda.recurrent_step(dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), state,
                                   signed_alpha=(mode == "signed"), **kw)
        torch.cuda.synchronize()
        check("fdecode%d/step%d" % (i, step), host64(o), o_ref, host64(state), s_ref, tol, bf16_store=False)
        if use_conv:
            for x_, (got, ref) in enumerate(zip(cache, c_ref)):
                assert np.array_equal(host64(got), np.asarray(ref, np.float64)), "conv cache %d" % x_
