"""GPU parity over seeded random configurations that reach the segmented and
windowed orders of the matrix-core prefill: few chains and thousands of
tokens (dense batches or packed sequences of mixed lengths), a workspace
that is the full one, the least one or a random size between, with or
without a context, through the fused entry point with a random decay input
(log-decay, the gate prologue, or the signed alpha of Complex KDA), short
convolution and output norm.  o, the final state and the outgoing conv
states are compared with the fp64 oracle.  Marked ``gpu``."""
import numpy as np
import pytest

import kda_inputs
import oracle
from gpu_util import check, dev, host64

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
CASES = 10
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
    r = np.random.default_rng(7000 + i)
    packed = r.random() < 0.4
    H = int(r.integers(1, 7))
    if packed:
        n = int(r.integers(1, 5))
        lengths = [int(x) if r.random() > 0.15 else 0 for x in r.integers(1, 12000, size=n)]
        B, T = 1, 0
    else:
        lengths = None
        B, T = int(r.integers(1, 3)), int(r.integers(3000, 14000))
    return dict(B=B, T=T, H=H, lengths=lengths, mode=str(r.choice(["plain", "gated", "signed"])),
                conv=bool(r.random() < 0.4), norm=bool(r.random() < 0.4), s0_std=float(r.choice([0.0, 0.02])),
                out=str(r.choice(["bf16", "f32"])), ws=str(r.choice(["full", "least", "between"], p=[0.45, 0.25, 0.3])),
                ws_frac=float(r.uniform(0.05, 0.9)), context=bool(r.random() < 0.7))


@pytest.mark.parametrize("i", range(CASES))
def test_random_orders(kda, i):
    import torch
    c = _draw_case(i)
    print("case", i, c, flush=True)
    seed = 8000 + i
    B, T, H = c["B"], c["T"], c["H"]
    if c["mode"] == "gated":
        inp = kda_inputs.make_gated_prefill(seed, B, T, H, 128, 128, s0_std=c["s0_std"], lengths=c["lengths"])
        g_ref = oracle.gate_map(inp.f32("z"), inp.A_log, inp.dt_bias)
        b_ref = oracle.beta_from_logits(inp.beta_logits)
    elif c["mode"] == "signed":
        inp = kda_inputs.make_signed_prefill(seed, B, T, H, 128, 128, s0_std=c["s0_std"], lengths=c["lengths"])
        g_ref, b_ref = inp.g, inp.beta
    else:
        inp = kda_inputs.make_prefill(seed, B, T, H, 128, 128, s0_std=c["s0_std"], lengths=c["lengths"])
        g_ref, b_ref = inp.g, inp.beta
    N = B if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1
    T = inp.q.shape[1]
    signed = c["mode"] == "signed"

    ws = cs = None
    if c["conv"]:
        ws = kda_inputs.conv_weights(seed, H, 128, 128)
        cs = kda_inputs.conv_states(seed, N, H, 128, 128)
        o_ref, s_ref, f_ref = oracle.forward_conv(inp.f32("q"), inp.f32("k"), inp.f32("v"), g_ref, b_ref, ws,
                                                  tuple(_f(x) for x in cs), inp.init_state, inp.cu_seqlens,
                                                  alpha_given=signed)
    else:
        o_ref, s_ref = oracle.forward_arrays(inp.f32("q"), inp.f32("k"), inp.f32("v"), g_ref, b_ref,
                                             inp.init_state, inp.cu_seqlens, alpha_given=signed)
    gate = None
    if c["norm"]:
        gate = kda_inputs.make_out_gate(seed, (B, T, H, 128))
        o_ref = oracle.out_norm(o_ref, _f(gate).astype(np.float64), None, EPS)

    flags = kda.FLAG_QK_L2NORM | (kda.FLAG_OUT_NORM if c["norm"] else 0)
    nseq = N if inp.cu_seqlens is not None else 0
    full = kda.workspace_bytes(B, T, H, 128, 128, num_seqs=nseq, flags=flags)
    least = kda.min_workspace_bytes(B, T, H, 128, 128, num_seqs=nseq, flags=flags)
    nbytes = {"full": full, "least": least,
              "between": least + int(c["ws_frac"] * (full - least)) // 256 * 256}[c["ws"]]
    workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    odt = torch.float32 if c["out"] == "f32" else torch.bfloat16
    kw = dict(out_dtype=odt, workspace=workspace, context="default" if c["context"] else None)
    finals = None
    if c["conv"]:
        finals = tuple(torch.empty((N, 3, H * 128), dtype=torch.bfloat16, device="cuda") for _ in range(3))
        kw.update(conv_weights=tuple(dev(x) for x in ws), conv_final=finals, conv_init=tuple(dev(x) for x in cs))
    if c["norm"]:
        kw.update(out_gate=dev(gate), norm_eps=EPS)
    if c["mode"] == "gated":
        o, s = kda.chunk_fwd_gated(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.z), dev(inp.A_log),
                                   dev(inp.beta_logits), dev(inp.init_state), dev(inp.cu_seqlens),
                                   dt_bias=dev(inp.dt_bias), beta_logits=True, **kw)
    else:
        o, s = kda.chunk_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state),
                             dev(inp.cu_seqlens), signed_alpha=signed, **kw)
    torch.cuda.synchronize()
    check("orders%d" % i, host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=(odt == torch.bfloat16))
    if c["conv"]:
        for x_, (got, ref) in enumerate(zip(finals, f_ref)):
            assert np.array_equal(host64(got), np.asarray(ref, np.float64)), "conv state %d" % x_
