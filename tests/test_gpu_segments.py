"""GPU parity of the segmented sequential pass: a dense batch with few chains
and many chunks splits every chain into P segments, summarises the middle
segments as affine maps S -> M S + B, chains the segments' initial states and
reruns the segments with outputs ("Kimi K3 の KDA ..." sections 2.3.4.2-
2.3.4.5).  The shapes here make the library take that order on a 256-CU
MI355X (3 to 32 segments; the plan itself is checked on the CPU in
test_stage_plan.py); o and the final state are compared with the fp64 oracle
at the same tolerances as the plain order.  Marked ``gpu``."""
import numpy as np
import pytest

import kda_inputs
import oracle
from gpu_util import check, dev, host64

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
EPS = 1e-5


@pytest.fixture(scope="module")
def kda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_fwd_amd as m
    m.load()
    if torch.cuda.get_device_properties(0).multi_processor_count < 256:
        pytest.skip("segment counts below are those of a 256-CU device")
    return m


def _f(a):
    return kda_inputs.bf16_to_f32(a) if a.dtype == np.uint16 else a


def _run(kda, inp, odt, **kw):
    import torch
    o, s = kda.chunk_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state),
                         dev(inp.cu_seqlens), out_dtype=odt, **kw)
    torch.cuda.synchronize()
    return o, s


@pytest.mark.parametrize("shape", [(1, 8192 + 37, 2), (2, 16384, 4), (1, 6144 + 5, 1), (1, 4096 + 100, 16),
                                   (1, 3072 + 5, 32)],
                         ids=["P8_ragged", "P8_B2", "P6_one_chain", "P4_16_chains", "P3_32_chains"])
def test_segments_plain(kda, shape):
    """8 segments over 129 chunks (the last one partial) and over 256 chunks
    of 8 chains, 6 segments of one chain, 4 segments of 16 chains, 3 of 32
    chains; nonzero initial state, both output dtypes."""
    import torch
    B, T, H = shape
    inp = kda_inputs.make_prefill(51, B, T, H, 128, 128, s0_std=0.02)
    o_ref, s_ref = oracle.forward(inp)
    for odt in (torch.bfloat16, torch.float32):
        o, s = _run(kda, inp, odt)
        check("seg_%dx%dx%d/%s" % (B, T, H, str(odt).split(".")[-1]), host64(o), o_ref, host64(s), s_ref,
              TOL_BF16, bf16_store=(odt == torch.bfloat16))


def test_segments_zero_initial_state_and_no_final_state(kda):
    import torch
    inp = kda_inputs.make_prefill(52, 1, 8192, 2, 128, 128)
    o_ref, s_ref = oracle.forward(inp)
    o, s = _run(kda, inp, torch.float32)
    check("seg_s0_zero", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)
    o2, s2 = _run(kda, inp, torch.float32, output_final_state=False)
    assert s2 is None
    assert torch.equal(o2, o)


def test_segments_initial_state_aliasing_final_state(kda):
    """init_state and final_state the same buffer (allowed by the ABI): phase C
    starts segment 0 from phase A's copy of the initial state, so the last
    segment's write of the final state in the same launch cannot reach it;
    equal bit for bit to the call with separate buffers."""
    import torch
    inp = kda_inputs.make_prefill(58, 1, 8192 + 9, 4, 128, 128, s0_std=0.02)
    a = [dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta)]
    s0 = dev(inp.init_state)
    o1, s1 = kda.chunk_fwd(*a, s0.clone(), out_dtype=torch.float32)
    st = s0.clone()
    o2, s2 = kda.chunk_fwd(*a, st, final_state=st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, st)


def test_segments_signed(kda):
    """Complex KDA: signed decays inside the segment maps."""
    import torch
    inp = kda_inputs.make_signed_prefill(53, 1, 8192 + 100, 2, 128, 128, s0_std=0.02)
    o_ref, s_ref = oracle.forward_signed(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.g, inp.beta,
                                         inp.init_state, inp.cu_seqlens)
    o, s = _run(kda, inp, torch.bfloat16, signed_alpha=True)
    check("seg_signed", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=True)


def test_segments_conv_and_norm(kda):
    """Short convolution (the value rows of a segment's first chunk reach back
    into the previous segment) and the output norm (row-sum words per
    segment unit) together."""
    import torch
    B, T, H = 1, 6144 + 70, 2
    inp = kda_inputs.make_prefill(54, B, T, H, 128, 128, s0_std=0.02)
    ws = kda_inputs.conv_weights(54, H, 128, 128)
    cs = kda_inputs.conv_states(54, B, H, 128, 128)
    gate = kda_inputs.make_out_gate(54, inp.v.shape)
    w = kda_inputs.norm_weight(54, 128)
    o_ref, s_ref, _ = oracle.forward_conv(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.g, inp.beta, ws,
                                          tuple(_f(c) for c in cs), inp.init_state, inp.cu_seqlens)
    y_ref = oracle.out_norm(o_ref, _f(gate).astype(np.float64), w, EPS)
    for odt in (torch.bfloat16, torch.float32):
        o, s = _run(kda, inp, odt, conv_weights=tuple(dev(x) for x in ws), conv_init=tuple(dev(c) for c in cs),
                    out_gate=dev(gate), norm_weight=dev(w), norm_eps=EPS)
        check("seg_conv_norm/%s" % str(odt).split(".")[-1], host64(o), y_ref, host64(s), s_ref, TOL_BF16,
              bf16_store=(odt == torch.bfloat16))


def test_segments_paired_and_unpaired_summaries(kda):
    """16 chains of 129 chunks: without the short convolution the summary
    units run two per CU and the chain takes 8 segments, with it one per CU
    and 5 segments; both against the oracle."""
    import torch
    B, T, H = 1, 8192 + 70, 16
    inp = kda_inputs.make_prefill(58, B, T, H, 128, 128, s0_std=0.02)
    o_ref, s_ref = oracle.forward(inp)
    o, s = _run(kda, inp, torch.bfloat16)
    check("seg_paired", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=True)
    ws = kda_inputs.conv_weights(58, H, 128, 128)
    cs = kda_inputs.conv_states(58, B, H, 128, 128)
    o_ref, s_ref, _ = oracle.forward_conv(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.g, inp.beta, ws,
                                          tuple(_f(c) for c in cs), inp.init_state, inp.cu_seqlens)
    o, s = _run(kda, inp, torch.float32, conv_weights=tuple(dev(x) for x in ws), conv_init=tuple(dev(c) for c in cs))
    check("seg_unpaired_conv", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)


@pytest.mark.parametrize("shape", [(1, 64 * 600 + 17, 1), (2, 64 * 520, 2)], ids=["P32_one_chain", "P32_four_chains"])
def test_segments_many(kda, shape):
    """Few chains of many chunks take up to 32 segments (at most 128
    segment-chains in all): 32 segments of 19 chunks for one chain, of 17
    for four; against the oracle, with the output norm too (its row-sum
    words indexed per segment unit)."""
    import torch
    B, T, H = shape
    inp = kda_inputs.make_prefill(59, B, T, H, 128, 128, s0_std=0.02)
    o_ref, s_ref = oracle.forward(inp)
    o, s = _run(kda, inp, torch.bfloat16)
    check("seg_many_%dx%d" % (B, H), host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=True)
    gate = kda_inputs.make_out_gate(59, inp.v.shape)
    y_ref = oracle.out_norm(o_ref, _f(gate).astype(np.float64), None, EPS)
    o, s = _run(kda, inp, torch.float32, out_gate=dev(gate), norm_eps=EPS)
    check("seg_many_norm_%dx%d" % (B, H), host64(o), y_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)


def test_segments_many_with_the_short_convolution(kda):
    """Four chains of 520 chunks with the short convolution: the summaries
    run one per CU, so 17 segments; against the oracle."""
    import torch
    B, T, H = 2, 64 * 520, 2
    inp = kda_inputs.make_prefill(60, B, T, H, 128, 128, s0_std=0.02)
    ws = kda_inputs.conv_weights(60, H, 128, 128)
    cs = kda_inputs.conv_states(60, B, H, 128, 128)
    o_ref, s_ref, _ = oracle.forward_conv(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.g, inp.beta, ws,
                                          tuple(_f(c) for c in cs), inp.init_state, inp.cu_seqlens)
    o, s = _run(kda, inp, torch.float32, conv_weights=tuple(dev(x) for x in ws), conv_init=tuple(dev(c) for c in cs))
    check("seg_many_conv", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)


def test_segments_packed(kda):
    """Packed sequences of mixed lengths (one empty, one of a single token):
    each chain cuts its own chunk range into the 5 segments (24 chains,
    ceil(T/64) = 361); an empty sequence passes its initial state through
    bit for bit."""
    import torch
    lens = [8000, 3000, 0, 64, 12000, 1]
    inp = kda_inputs.make_prefill(56, 1, 0, 4, 128, 128, s0_std=0.02, lengths=lens)
    d = [dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state), dev(inp.cu_seqlens)]
    o_ref, s_ref = oracle.forward(inp)
    for odt in (torch.bfloat16, torch.float32):
        o, s = kda.chunk_fwd(*d, out_dtype=odt)
        torch.cuda.synchronize()
        check("seg_packed/%s" % str(odt).split(".")[-1], host64(o), o_ref, host64(s), s_ref, TOL_BF16,
              bf16_store=(odt == torch.bfloat16))
        np.testing.assert_array_equal(host64(s[2]), inp.init_state[2].astype(np.float64))


def test_segments_packed_conv_norm(kda):
    """Two long packed sequences, 3 heads (6 chains, 8 segments each) with
    the short convolution and the output norm."""
    import torch
    lens = [5000, 7000]
    H = 3
    inp = kda_inputs.make_prefill(57, 1, 0, H, 128, 128, s0_std=0.02, lengths=lens)
    ws = kda_inputs.conv_weights(57, H, 128, 128)
    cs = kda_inputs.conv_states(57, len(lens), H, 128, 128)
    gate = kda_inputs.make_out_gate(57, inp.v.shape)
    w = kda_inputs.norm_weight(57, 128)
    o_ref, s_ref, _ = oracle.forward_conv(inp.f32("q"), inp.f32("k"), inp.f32("v"), inp.g, inp.beta, ws,
                                          tuple(_f(c) for c in cs), inp.init_state, inp.cu_seqlens)
    y_ref = oracle.out_norm(o_ref, _f(gate).astype(np.float64), w, EPS)
    o, s = kda.chunk_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state),
                         dev(inp.cu_seqlens), out_dtype=torch.float32, conv_weights=tuple(dev(x) for x in ws),
                         conv_init=tuple(dev(c) for c in cs), out_gate=dev(gate), norm_weight=dev(w), norm_eps=EPS)
    torch.cuda.synchronize()
    check("seg_packed_conv_norm", host64(o), y_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)


def test_segments_long_sampled_heads(kda):
    """64K tokens x 16 heads (8 segments of 128 chunks), oracle on two
    sampled heads; with the default context the last segment's pass 1 runs
    on the context's stream beside phase A, without one after it: the same
    bits."""
    import torch
    inp = kda_inputs.workload("long_bf16", H=16)
    o, s = _run(kda, inp, torch.bfloat16)
    o2, s2 = _run(kda, inp, torch.bfloat16, context=None)
    assert torch.equal(o, o2) and torch.equal(s, s2)
    del o2, s2
    for h in (0, 15):
        hs = slice(h, h + 1)
        o_ref, s_ref = oracle.forward(inp, hs)
        check("seg_long16/h%d" % h, host64(o[:, :, hs]), o_ref, host64(s[:, hs]), s_ref, TOL_BF16, bf16_store=True)


@pytest.mark.parametrize("shape", [(1, 4096 + 33, 8), (1, 16384 + 50, 32)], ids=["serial", "tail_overlapped"])
def test_segments_in_a_graph(kda, shape):
    """A segmented call (with the output norm, so the row-sum words are
    cleared by the fill kernel inside the graph) captured with its buffers;
    replays after the inputs are overwritten eagerly reproduce the eager
    results bit for bit, and the eager results equal those of context=None.
    The second shape (257 chunks, 32 chains) runs the last segment's pass 1
    on the context's stream beside phase A, so the capture records that fork
    and its join."""
    import torch
    B, T, H = shape
    inps = [kda_inputs.make_prefill(55 + i, B, T, H, 128, 128, s0_std=0.02) for i in range(2)]
    gate = dev(kda_inputs.make_out_gate(55, (B, T, H, 128)))
    bufs = {k: dev(getattr(inps[0], k)).clone() for k in ("q", "k", "v", "g", "beta", "init_state")}
    o = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device="cuda")
    st = torch.empty((B, H, 128, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(kda.workspace_bytes(B, T, H, 128, 128, flags=kda.FLAG_QK_L2NORM | kda.FLAG_OUT_NORM),
                     dtype=torch.uint8, device="cuda")

    def call(context="default"):
        kda.chunk_fwd(bufs["q"], bufs["k"], bufs["v"], bufs["g"], bufs["beta"], bufs["init_state"], out_gate=gate,
                      norm_eps=EPS, o=o, final_state=st, workspace=ws, context=context)

    refs = []
    for inp in inps:
        for k in bufs:
            bufs[k].copy_(dev(getattr(inp, k)))
        call()
        torch.cuda.synchronize()
        refs.append((o.clone(), st.clone()))
        call(None)
        torch.cuda.synchronize()
        assert torch.equal(o, refs[-1][0]) and torch.equal(st, refs[-1][1])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        i = rep % 2
        for k in bufs:
            bufs[k].copy_(dev(getattr(inps[i], k)))
        o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, refs[i][0]), "replay %d: o" % rep
        assert torch.equal(st, refs[i][1]), "replay %d: final state" % rep
