"""The staged order of the matrix-core prefill: a dense batch long enough to
be split into stages (the chunk-parallel kernel of one stage overlapping the
sequential kernel of the stage before, on a second stream) gives the same
bits as the unstaged order, which the same sequences take when passed as
packed sequences (cu_seqlens) or when the call is captured into a graph.
Covered: plain, gate prologue, short convolution, output norm, Complex KDA,
two host threads with a stream each, and a staged call against the oracle.
Marked ``gpu``."""
import threading

import pytest

import kda_inputs
import oracle
from gpu_util import check, dev, host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_fwd_amd as m
    m.load()
    return m


def _packed(x, B, T):
    """[B, T, ...] viewed as one packed batch [1, B*T, ...]."""
    return None if x is None else x.reshape(1, B * T, *x.shape[2:])


def _run_both(kda, fwd, args, kw, B, T):
    """(o, final state) of the dense call and of the same sequences packed."""
    import torch
    o1, s1 = fwd(*args, **kw)
    torch.cuda.synchronize()
    seq_args = [_packed(a, B, T) if (a is not None and a.dim() >= 3 and a.shape[:2] == (B, T)) else a for a in args]
    cu = torch.tensor([b * T for b in range(B + 1)], dtype=torch.int32, device="cuda")
    kw2 = dict(kw)
    if "out_gate" in kw2:
        kw2["out_gate"] = _packed(kw2["out_gate"], B, T)
    o2, s2 = fwd(*seq_args, cu_seqlens=cu, **kw2)
    torch.cuda.synchronize()
    return (o1, s1), (o2.reshape(o1.shape), s2)


# Every shape here is above the staging threshold: at least 256 chunks per
# sequence, at least 8K (chunk, chain) pairs, and few enough chains (B*H <= 112)
# to leave CUs idle during the sequential pass; more than 42 chains, below
# which a dense batch takes the segmented sequential pass instead.
@pytest.mark.parametrize("B,T,H", [(1, 16384, 48), (2, 17000, 24)])
def test_staged_equals_unstaged_plain(kda, B, T, H):
    import torch
    inp = kda_inputs.make_prefill(80 + B, B, T, H, 128, 128, s0_std=0.02)
    args = [dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state)]
    (o1, s1), (o2, s2) = _run_both(kda, kda.chunk_fwd, args, {}, B, T)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_staged_equals_unstaged_gated_conv_norm(kda):
    """The whole layer core: gate prologue, short convolution, output norm."""
    import torch
    B, T, H = 1, 16500, 48
    gin = kda_inputs.make_gated_prefill(83, B, T, H, 128, 128, s0_std=0.02)
    ws = kda_inputs.conv_weights(83, H, 128, 128)
    gate = dev(kda_inputs.make_out_gate(83, (B, T, H, 128)))
    w = dev(kda_inputs.norm_weight(83, 128))
    cs = tuple(dev(c) for c in kda_inputs.conv_states(83, B, H, 128, 128))
    outs = []
    for packed in (False, True):
        fin = tuple(torch.empty((B, 3, H * 128), dtype=torch.bfloat16, device="cuda") for _ in range(3))
        kw = dict(dt_bias=dev(gin.dt_bias), beta_logits=True, conv_weights=tuple(dev(x) for x in ws), conv_init=cs,
                  conv_final=fin, out_gate=gate, norm_weight=w)
        cu = torch.tensor([0, T], dtype=torch.int32, device="cuda") if packed else None
        o, s = kda.chunk_fwd_gated(dev(gin.q), dev(gin.k), dev(gin.v), dev(gin.z), dev(gin.A_log),
                                   dev(gin.beta_logits), dev(gin.init_state), cu, **kw)
        torch.cuda.synchronize()
        outs.append((o, s, fin))
    (o1, s1, f1), (o2, s2, f2) = outs
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    for a, b in zip(f1, f2):
        assert torch.equal(a, b)


def test_staged_equals_unstaged_signed(kda):
    import torch
    B, T, H = 1, 16384, 48
    inp = kda_inputs.make_signed_prefill(84, B, T, H, 128, 128, s0_std=0.02)
    args = [dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state)]
    (o1, s1), (o2, s2) = _run_both(kda, kda.chunk_fwd, args, dict(signed_alpha=True), B, T)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_staged_against_oracle(kda):
    """A staged call with a ragged last chunk against the fp64 oracle."""
    import torch
    B, T, H = 1, 16400, 48
    inp = kda_inputs.make_prefill(85, B, T, H, 128, 128, s0_std=0.02)
    o, s = kda.chunk_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state),
                         out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.forward(inp)
    check("staged", host64(o), o_ref, host64(s), s_ref, 2e-2, bf16_store=False)


def test_staged_call_in_a_graph_and_on_two_threads(kda):
    """Captured and replayed (staged inside the graph: the thread's default
    context exists from the eager calls, so the capture records the fork and
    the join), captured on a fresh thread (no context yet, and none is made
    inside a capture: the graph holds the unstaged order), and run from two
    host threads on streams and contexts of their own: all equal the eager
    staged call bit for bit."""
    import torch
    B, T, H = 1, 16384, 48
    inps = [kda_inputs.make_prefill(86 + i, B, T, H, 128, 128, s0_std=0.02) for i in range(2)]
    devs = [[dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), dev(x.init_state)] for x in inps]
    bufs = []
    for _ in range(2):
        bufs.append(dict(o=torch.empty((B, T, H, 128), dtype=torch.bfloat16, device="cuda"),
                         s=torch.empty((B, H, 128, 128), dtype=torch.float32, device="cuda"),
                         ws=torch.empty(kda.workspace_bytes(B, T, H, 128, 128), dtype=torch.uint8, device="cuda")))
    refs = []
    for i in range(2):
        kda.chunk_fwd(*devs[i], o=bufs[i]["o"], final_state=bufs[i]["s"], workspace=bufs[i]["ws"])
        torch.cuda.synchronize()
        refs.append((bufs[i]["o"].clone(), bufs[i]["s"].clone()))

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.chunk_fwd(*devs[0], o=bufs[0]["o"], final_state=bufs[0]["s"], workspace=bufs[0]["ws"])
    torch.cuda.synchronize()
    for rep in range(3):
        bufs[0]["o"].zero_()
        bufs[0]["s"].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs[0]["o"], refs[0][0]) and torch.equal(bufs[0]["s"], refs[0][1]), "replay %d" % rep

    # a capture on a thread that has made no staged call yet
    errors = []

    def capture_fresh():
        try:
            g2 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g2):
                kda.chunk_fwd(*devs[1], o=bufs[1]["o"], final_state=bufs[1]["s"], workspace=bufs[1]["ws"])
            torch.cuda.synchronize()
            for _ in range(2):
                bufs[1]["o"].zero_()
                bufs[1]["s"].zero_()
                torch.cuda.synchronize()
                g2.replay()
                torch.cuda.synchronize()
                if not (torch.equal(bufs[1]["o"], refs[1][0]) and torch.equal(bufs[1]["s"], refs[1][1])):
                    errors.append("fresh-thread graph replay differs")
        except Exception as e:   # reported by the main thread
            errors.append(e)

    t = threading.Thread(target=capture_fresh)
    t.start()
    t.join()
    assert not errors, errors

    for b in bufs:
        b["o"].zero_()
        b["s"].zero_()
    torch.cuda.synchronize()

    def worker(i):
        try:
            st = torch.cuda.Stream()   # default priority
            with torch.cuda.stream(st):
                for _ in range(3):
                    kda.chunk_fwd(*devs[i], o=bufs[i]["o"], final_state=bufs[i]["s"], workspace=bufs[i]["ws"])
            st.synchronize()
        except Exception as e:   # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i in range(2):
        assert torch.equal(bufs[i]["o"], refs[i][0]) and torch.equal(bufs[i]["s"], refs[i][1]), "thread %d" % i


@pytest.mark.parametrize("i", range(4))
def test_random_staged_against_oracle(kda, i):
    """Seeded random dense batches long enough to run in stages (ragged last
    chunk, one or two sequences, few heads, each gate distribution) against
    the fp64 oracle on every head."""
    import numpy as np
    import torch
    r = np.random.default_rng(9000 + i)
    B = int(r.integers(1, 3))
    T = int(r.integers(16384, 24000))
    H = int(r.integers(44, 65)) // B          # 44..64 chains: staged
    gate = str(r.choice(["k3", "slow", "sigmoid"]))
    print("case", i, dict(B=B, T=T, H=H, gate=gate), flush=True)
    inp = kda_inputs.make_prefill(9100 + i, B, T, H, 128, 128, gate=gate, s0_std=0.02)
    o, s = kda.chunk_fwd(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), dev(inp.init_state))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.forward(inp)
    check("random_staged%d" % i, host64(o), o_ref, host64(s), s_ref, 2e-2, bf16_store=True)


def test_context_ownership(kda):
    """The staged order needs a caller-owned context: an explicit Context and
    context=None (one kernel after the other on the call's stream) give the
    same bits; while the context's stream is part of an open graph capture,
    an eager call on another stream with the same context takes the unstaged
    order on its own stream (nothing of it enters the graph), and both the
    eager result and every replay of the graph equal the reference."""
    import torch
    B, T, H = 1, 16384, 48
    inps = [kda_inputs.make_prefill(88 + i, B, T, H, 128, 128, s0_std=0.02) for i in range(2)]
    devs = [[dev(x.q), dev(x.k), dev(x.v), dev(x.g), dev(x.beta), dev(x.init_state)] for x in inps]
    ws = kda.workspace_bytes(B, T, H, 128, 128)
    bufs = [dict(o=torch.empty((B, T, H, 128), dtype=torch.bfloat16, device="cuda"),
                 s=torch.empty((B, H, 128, 128), dtype=torch.float32, device="cuda"),
                 ws=torch.empty(ws, dtype=torch.uint8, device="cuda")) for _ in range(2)]
    with kda.Context() as ctx:
        refs = []
        for i in range(2):
            kda.chunk_fwd(*devs[i], o=bufs[i]["o"], final_state=bufs[i]["s"], workspace=bufs[i]["ws"], context=None)
            torch.cuda.synchronize()
            refs.append((bufs[i]["o"].clone(), bufs[i]["s"].clone()))
            bufs[i]["o"].zero_()
            kda.chunk_fwd(*devs[i], o=bufs[i]["o"], final_state=bufs[i]["s"], workspace=bufs[i]["ws"], context=ctx)
            torch.cuda.synchronize()
            assert torch.equal(bufs[i]["o"], refs[i][0]) and torch.equal(bufs[i]["s"], refs[i][1]), "explicit %d" % i
        for b in bufs:
            b["o"].zero_()
            b["s"].zero_()
        torch.cuda.synchronize()
        other = torch.cuda.Stream()   # default priority
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, capture_error_mode="relaxed"):
            kda.chunk_fwd(*devs[0], o=bufs[0]["o"], final_state=bufs[0]["s"], workspace=bufs[0]["ws"], context=ctx)
            with torch.cuda.stream(other):
                kda.chunk_fwd(*devs[1], o=bufs[1]["o"], final_state=bufs[1]["s"], workspace=bufs[1]["ws"],
                              context=ctx)
        other.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(bufs[1]["o"], refs[1][0]) and torch.equal(bufs[1]["s"], refs[1][1]), "eager beside capture"
        assert not bufs[0]["o"].any(), "captured work ran eagerly"
        for rep in range(2):
            bufs[1]["o"].zero_()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(bufs[0]["o"], refs[0][0]) and torch.equal(bufs[0]["s"], refs[0][1]), "replay %d" % rep
            assert not bufs[1]["o"].any(), "the eager call entered the graph"
        del graph
