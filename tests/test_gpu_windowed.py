"""GPU tests of the windowed order (constant-memory long context): with a
workspace below kda_chunk_fwd_workspace_bytes the matrix-core path runs the
chunks in windows, pass 1 then pass 2 per window, the state carried between
windows in fp32 ("Kimi K3 模型结构（2）", Q&A on the chunkwise algorithm:
one state per chain, updated once per chunk).  The windows change no
arithmetic, so a windowed call must equal the unwindowed two-pass order bit
for bit (the plain, staged and packed orders), whatever the window; against
the segmented order (few chains) it is compared with the fp64 oracle.
Marked ``gpu``."""
import numpy as np
import pytest

import kda_inputs
import oracle
from gpu_util import check, dev, host64

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
EPS = 1e-5
RECORD = 74240
STATE = 128 * 128 * 4


@pytest.fixture(scope="module")
def kda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_fwd_amd as m
    m.load()
    return m


def _ws(nseq, H, window, norm=False):
    """Workspace bytes of a window of `window` chunks of every sequence."""
    chains = nseq * H
    return chains * (window * RECORD + STATE + (4096 if norm else 0))


def _ws_seg(nseq, H, window, nck):
    """Workspace bytes of a window of `window` chunks with room for the
    segmented order inside it: 3P - 3 state-sized blocks per chain for the
    most segments P a sequence of nck chunks may take, min(32, 128 // chains,
    nck // 16)."""
    chains = nseq * H
    return chains * (window * RECORD + STATE + (3 * _seg_cap(chains, nck) - 3) * STATE)


def _seg_cap(chains, nck):
    return min(32, 128 // chains, nck // 16)


def _args(inp):
    return [dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state)]


@pytest.mark.parametrize("window", [1, 7, 40])
def test_windowed_equals_full_dense(kda, window):
    """96 chains (the plain order with the full workspace), a ragged last
    chunk, windows of 1, 7 and 40 chunks of the 79 per sequence."""
    import torch
    B, T, H = 2, 5000, 48
    inp = kda_inputs.make_prefill(61, B, T, H, 128, 128, s0_std=0.02)
    a = _args(inp)
    o1, s1 = kda.chunk_fwd(*a)
    o2, s2 = kda.chunk_fwd(*a, workspace_limit=_ws(B, H, window))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_windowed_against_oracle_and_min_workspace(kda):
    """The least workspace (one chunk per window) on a short batch, against
    the oracle; the binding allocates exactly min_workspace_bytes."""
    import torch
    B, T, H = 1, 700, 4
    inp = kda_inputs.make_prefill(62, B, T, H, 128, 128, s0_std=0.02)
    assert kda.min_workspace_bytes(B, T, H, 128, 128) == _ws(B, H, 1)
    ws = torch.empty(kda.min_workspace_bytes(B, T, H, 128, 128), dtype=torch.uint8, device="cuda")
    o, s = kda.chunk_fwd(*_args(inp), workspace=ws, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.forward(inp)
    check("windowed_min", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)


def test_windowed_few_chains_against_oracle(kda):
    """Few chains: the full workspace takes the segmented order, a small one
    the windowed order; both against the oracle, and two window sizes
    against each other bit for bit."""
    import torch
    B, T, H = 1, 8192 + 21, 2
    inp = kda_inputs.make_prefill(63, B, T, H, 128, 128, s0_std=0.02)
    a = _args(inp)
    o_ref, s_ref = oracle.forward(inp)
    runs = []
    for lim in (None, _ws(B, H, 5), _ws(B, H, 33)):
        o, s = kda.chunk_fwd(*a, workspace_limit=lim)
        torch.cuda.synchronize()
        check("few_chains/%s" % lim, host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=True)
        runs.append((o, s))
    assert torch.equal(runs[1][0], runs[2][0]) and torch.equal(runs[1][1], runs[2][1])


@pytest.mark.parametrize("window", [100, 64])
def test_windowed_segments_against_oracle(kda, window):
    """Few chains and windows long enough for the segmented order inside each
    window (6 and 4 segments of the 100- and 64-chunk windows; the last,
    shorter window of 57 chunks takes 3, or the plain order at 1 chunk):
    against the oracle, with the output norm too."""
    import torch
    B, T, H = 1, 16384 + 33, 2
    inp = kda_inputs.make_prefill(69, B, T, H, 128, 128, s0_std=0.02)
    gate = kda_inputs.make_out_gate(69, inp.v.shape)
    o_ref, s_ref = oracle.forward(inp)
    nck = (T + 63) // 64
    o, s = kda.chunk_fwd(*_args(inp), workspace_limit=_ws_seg(B, H, window, nck))
    torch.cuda.synchronize()
    check("win_seg%d" % window, host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=True)
    y_ref = oracle.out_norm(o_ref, kda_inputs.bf16_to_f32(gate).astype(np.float64), None, EPS)
    o, s = kda.chunk_fwd(*_args(inp), out_gate=dev(gate), norm_eps=EPS, out_dtype=torch.float32,
                         workspace_limit=_ws_seg(B, H, window, nck) + B * H * _seg_cap(B * H, nck) * 4096)
    torch.cuda.synchronize()
    check("win_seg%d_norm" % window, host64(o), y_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)


def test_windowed_equals_full_packed(kda):
    """Packed sequences of mixed lengths (one empty, one shorter than a
    chunk): windows by chunk index within each sequence; sequences that
    ended before a window pass their state through it."""
    import torch
    inp = kda_inputs.make_prefill(64, 1, 0, 4, 128, 128, s0_std=0.02, lengths=[300, 0, 1000, 40, 2000, 64])
    d = [dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state), dev(inp.cu_seqlens)]
    o1, s1 = kda.chunk_fwd(*d)
    for window in (1, 3, 16):
        o2, s2 = kda.chunk_fwd(*d, workspace_limit=_ws(6, 4, window))
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2), window
    o_ref, s_ref = oracle.forward(inp)
    check("windowed_packed", host64(o2), o_ref, host64(s2), s_ref, TOL_BF16, bf16_store=True)


def test_windowed_equals_full_fused_variants(kda):
    """Gate prologue + short convolution + output norm, and Complex KDA,
    windowed against the full workspace (packed sequences: the plain order)."""
    import torch
    lens = [500, 1300, 0, 777]
    H = 3
    gin = kda_inputs.make_gated_prefill(65, 1, 0, H, 128, 128, s0_std=0.02, lengths=lens)
    T = gin.T
    ws = tuple(dev(x) for x in kda_inputs.conv_weights(65, H, 128, 128))
    cs = tuple(dev(c) for c in kda_inputs.conv_states(65, len(lens), H, 128, 128))
    gate = dev(kda_inputs.make_out_gate(65, (1, T, H, 128)))
    w = dev(kda_inputs.norm_weight(65, 128))
    outs = []
    for lim in (None, _ws(len(lens), H, 2, norm=True)):
        fin = tuple(torch.empty_like(c) for c in cs)
        o, s = kda.chunk_fwd_gated(dev(gin.q), dev(gin.k), dev(gin.v), dev(gin.z), dev(gin.A_log),
                                   dev(gin.beta_logits), dev(gin.init_state), dev(gin.cu_seqlens),
                                   dt_bias=dev(gin.dt_bias), beta_logits=True, conv_weights=ws, conv_init=cs,
                                   conv_final=fin, out_gate=gate, norm_weight=w, norm_eps=EPS, workspace_limit=lim)
        torch.cuda.synchronize()
        outs.append((o, s, fin))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert all(torch.equal(x, y) for x, y in zip(outs[0][2], outs[1][2]))

    sin = kda_inputs.make_signed_prefill(66, 1, 0, H, 128, 128, s0_std=0.02, lengths=lens)
    d = [dev(sin.q), dev(sin.k), dev(sin.v), dev(sin.g), dev(sin.beta), dev(sin.init_state), dev(sin.cu_seqlens)]
    o1, s1 = kda.chunk_fwd(*d, signed_alpha=True)
    o2, s2 = kda.chunk_fwd(*d, signed_alpha=True, workspace_limit=_ws(len(lens), H, 3))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_windowed_equals_staged(kda):
    """A shape that runs in stages with the full workspace (48 chains, 256
    chunks per sequence): windowed with a 1/8 workspace, equal bit for bit."""
    import torch
    B, T, H = 1, 16384, 48
    inp = kda_inputs.make_prefill(67, B, T, H, 128, 128, s0_std=0.02)
    a = _args(inp)
    full = kda.workspace_bytes(B, T, H, 128, 128)
    o1, s1 = kda.chunk_fwd(*a)
    o2, s2 = kda.chunk_fwd(*a, workspace_limit=full // 8)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_windowed_in_a_graph(kda):
    """A windowed call captured with its buffers (the norm's words cleared
    by the fill kernel inside the graph); replays after eager input changes
    reproduce the eager results."""
    import torch
    inps = [kda_inputs.make_prefill(68 + i, 1, 0, 2, 128, 128, s0_std=0.02, lengths=[900, 130, 0])
            for i in range(2)]
    T = inps[0].T
    bufs = {k: dev(getattr(inps[0], k)).clone() for k in ("q", "k", "v", "g", "beta", "init_state", "cu_seqlens")}
    gate = dev(kda_inputs.make_out_gate(68, (1, T, 2, 128)))
    o = torch.empty((1, T, 2, 128), dtype=torch.bfloat16, device="cuda")
    st = torch.empty((3, 2, 128, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(_ws(3, 2, 2, norm=True), dtype=torch.uint8, device="cuda")

    def call():
        kda.chunk_fwd(bufs["q"], bufs["k"], bufs["v"], bufs["g"], bufs["beta"], bufs["init_state"], bufs["cu_seqlens"],
                      out_gate=gate, norm_eps=EPS, o=o, final_state=st, workspace=ws)

    refs = []
    for inp in inps:
        for k in bufs:
            bufs[k].copy_(dev(getattr(inp, k)))
        call()
        torch.cuda.synchronize()
        refs.append((o.clone(), st.clone()))
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


def test_windowed_overlap_orders_and_graph(kda):
    """48 chains, 258 chunks per sequence, a ring of 80 chunks: with the
    context the windows overlap their passes (two ring halves of 40 chunks,
    7 stages), without it they run one after the other; both equal the full
    workspace's staged call bit for bit, and so does every replay of the
    overlapped call captured in a graph."""
    import torch
    B, T, H = 1, 16384 + 100, 48
    inps = [kda_inputs.make_prefill(70 + i, B, T, H, 128, 128, s0_std=0.02) for i in range(2)]
    bufs = {k: dev(getattr(inps[0], k)).clone() for k in ("q", "k", "v", "g", "beta", "init_state")}
    o = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device="cuda")
    st = torch.empty((B, H, 128, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(_ws(B, H, 80), dtype=torch.uint8, device="cuda")

    def call(context="default", workspace=ws):
        kda.chunk_fwd(bufs["q"], bufs["k"], bufs["v"], bufs["g"], bufs["beta"], bufs["init_state"], o=o,
                      final_state=st, workspace=workspace, context=context)

    refs = []
    for inp in inps:
        for k in bufs:
            bufs[k].copy_(dev(getattr(inp, k)))
        call(workspace=None)
        torch.cuda.synchronize()
        refs.append((o.clone(), st.clone()))
        for ctx in ("default", None):
            o.zero_()
            call(ctx)
            torch.cuda.synchronize()
            assert torch.equal(o, refs[-1][0]) and torch.equal(st, refs[-1][1]), ctx
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


def test_windowed_million_tokens_against_oracle(kda):
    """One sequence of 2^20 + 37 tokens, 2 heads, in a 64 MiB workspace
    (windows of ~430 chunks, 8 segments inside each), against the fp64
    oracle over every token and the final state: the constant-memory order
    at a length whose full record area (2.3 GiB here) it never allocates."""
    import torch
    B, T, H = 1, (1 << 20) + 37, 2
    inp = kda_inputs.make_prefill(72, B, T, H, 128, 128, s0_std=0.02)
    assert kda.workspace_bytes(B, T, H, 128, 128) > 2 * (1 << 30)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    o, s = kda.chunk_fwd(*_args(inp), workspace=ws, out_dtype=torch.float32)
    torch.cuda.synchronize()
    print("million-token call done", flush=True)
    o_ref, s_ref = oracle.forward(inp)
    check("windowed_1M", host64(o), o_ref, host64(s), s_ref, TOL_BF16, bf16_store=False)
