"""The entry points on the caller's stream: results on a side stream equal
the default-stream results bit for bit, and the prefill and decode calls
can be captured into a graph (they only launch kernels; KDA_FLAG_VALIDATE,
which synchronises, is the exception) whose replays, with eager work and
synchronisations between them, reproduce the eager results bit for bit.
Marked ``gpu``."""
import numpy as np
import pytest

import kda_inputs
from gpu_util import dev, inputs_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_fwd_amd as m
    m.load()
    return m


def _prefill_buffers(kda, inp):
    import torch
    d = inputs_to_device(inp)
    B, T, H, dk = inp.q.shape
    dv = inp.v.shape[-1]
    N = B if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1
    d["o"] = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device="cuda")
    d["final_state"] = torch.empty((N, H, dk, dv), dtype=torch.float32, device="cuda")
    d["workspace"] = torch.empty(kda.workspace_bytes(B, T, H, dk, dv, num_seqs=0 if inp.cu_seqlens is None else N),
                                 dtype=torch.uint8, device="cuda")
    return d


def _prefill(kda, d):
    return kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["init_state"], d["cu_seqlens"], o=d["o"],
                         final_state=d["final_state"], workspace=d["workspace"])


def test_side_stream_matches_default_stream(kda):
    import torch
    inp = kda_inputs.make_prefill(71, 1, 0, 3, 128, 128, s0_std=0.02, lengths=[300, 0, 129])
    d = _prefill_buffers(kda, inp)
    _prefill(kda, d)
    torch.cuda.synchronize()
    o_ref, s_ref = d["o"].clone(), d["final_state"].clone()
    d["o"].zero_()
    d["final_state"].zero_()
    side = torch.cuda.Stream()   # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _prefill(kda, d)
    side.synchronize()
    assert torch.equal(d["o"], o_ref) and torch.equal(d["final_state"], s_ref)

    # decode on the side stream
    N, H, D = 4, 3, 128
    S0 = dev(kda_inputs.decode_initial_state(72, N, H, D))
    x = kda_inputs.decode_step(72, 0, N, H, D)
    args = [dev(a) for a in (x.q, x.k, x.v, x.g, x.beta)]
    s1 = S0.clone()
    o1 = kda.recurrent_step(*args, s1)
    torch.cuda.synchronize()
    s2 = S0.clone()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o2 = kda.recurrent_step(*args, s2)
    side.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_stream_argument_without_a_stream_context(kda):
    """stream= names a side stream while the current stream stays the
    default one: the buffers the call allocates (o, the final state and the
    record workspace) belong to the side stream, and the results equal the
    default-stream ones bit for bit (a staged prefill and a decode step)."""
    import torch
    inp = kda_inputs.make_prefill(75, 1, 16384, 48, 128, 128, s0_std=0.02)
    d = inputs_to_device(inp)
    args = [d[k] for k in ("q", "k", "v", "g", "beta", "init_state")]
    o1, s1 = kda.chunk_fwd(*args)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()   # default priority
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):   # freed buffers of one call are reused by the next only behind the side stream
        o2, s2 = kda.chunk_fwd(*args, stream=side)
    side.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)

    N, H, D = 4, 3, 128
    S0 = dev(kda_inputs.decode_initial_state(76, N, H, D))
    x = kda_inputs.decode_step(76, 0, N, H, D)
    xa = [dev(a) for a in (x.q, x.k, x.v, x.g, x.beta)]
    st1 = S0.clone()
    o1 = kda.recurrent_step(*xa, st1)
    torch.cuda.synchronize()
    st2 = S0.clone()
    side.wait_stream(torch.cuda.current_stream())
    o2 = kda.recurrent_step(*xa, st2, stream=side)
    side.synchronize()
    assert torch.equal(o1, o2) and torch.equal(st1, st2)


def test_decode_steps_in_a_graph(kda):
    """Eight decode steps captured once, replayed three times from a reset
    state with eager work in between; every replay equals the eager run."""
    import torch
    N, H, D, steps = 8, 4, 128, 8
    S0 = dev(kda_inputs.decode_initial_state(73, N, H, D))
    xs = []
    for s in range(steps):
        x = kda_inputs.decode_step(73, s, N, H, D)
        xs.append([dev(a) for a in (x.q, x.k, x.v, x.g, x.beta)])
    outs = [torch.empty((N, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(steps)]

    state = S0.clone()
    for s in range(steps):
        kda.recurrent_step(*xs[s], state, o=outs[s])
    torch.cuda.synchronize()
    o_ref = [o.clone() for o in outs]
    s_ref = state.clone()

    state.copy_(S0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(steps):
            kda.recurrent_step(*xs[s], state, o=outs[s])
    torch.cuda.synchronize()
    for rep in range(3):
        state.copy_(S0)                       # eager work between replays
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, s_ref), "replay %d: state" % rep
        for s in range(steps):
            assert torch.equal(outs[s], o_ref[s]), "replay %d: o of step %d" % (rep, s)


def test_prefill_in_a_graph(kda):
    """One packed prefill call captured with its workspace; replays after the
    inputs are overwritten (eagerly) reproduce the eager results for them."""
    import torch
    lens = [200, 65, 0, 130]
    inps = [kda_inputs.make_prefill(74 + i, 1, 0, 2, 128, 128, s0_std=0.02, lengths=lens) for i in range(2)]
    d = _prefill_buffers(kda, inps[0])
    refs = []
    for inp in inps:
        e = inputs_to_device(inp)
        for key in ("q", "k", "v", "g", "beta", "init_state"):
            d[key].copy_(e[key])
        _prefill(kda, d)
        torch.cuda.synchronize()
        refs.append((d["o"].clone(), d["final_state"].clone()))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _prefill(kda, d)
    torch.cuda.synchronize()
    for rep in range(4):
        i = rep % 2
        e = inputs_to_device(inps[i])
        for key in ("q", "k", "v", "g", "beta", "init_state"):
            d[key].copy_(e[key])
        d["o"].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(d["o"], refs[i][0]), "replay %d: o" % rep
        assert torch.equal(d["final_state"], refs[i][1]), "replay %d: final state" % rep
