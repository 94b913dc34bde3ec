"""kda_chunk_fwd_noalloc through the C ABI: two calls in a row (the second
smaller, on the scratch the first left behind) each equal kda_chunk_fwd on
the same inputs bit for bit, against the fp64 oracle too; a call whose full
workspace exceeds the fixed area runs in the windowed order there and still
equals kda_chunk_fwd bit for bit; a call whose least workspace exceeds it is
refused before any launch.  Named to be collected last.  Marked ``gpu``."""
import numpy as np
import pytest

import kda_inputs
import oracle
from gpu_util import check, host64, inputs_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_fwd_amd as m
    m.load()
    return m


def _both(kda, inp):
    import torch
    d = inputs_to_device(inp)
    args = [d[k] for k in ("q", "k", "v", "g", "beta", "init_state", "cu_seqlens")]
    o_ref, s_ref = kda.chunk_fwd(*args, context=None)
    B, T, H, _ = inp.q.shape
    N = B if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1
    o = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device="cuda")
    s = torch.empty((N, H, 128, 128), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    kda.chunk_fwd_noalloc(*args, o=o, final_state=s)
    torch.cuda.synchronize()
    return (o_ref, s_ref), (o, s)


def test_noalloc_matches_chunk_fwd_on_two_calls(kda):
    import torch
    big = kda_inputs.make_prefill(61, 1, 2048, 8, 128, 128, s0_std=0.02)                  # 256 records: 19 MB
    small = kda_inputs.make_prefill(62, 1, 0, 3, 128, 128, s0_std=0.02, lengths=[300, 0, 129])
    assert kda.workspace_bytes(1, 2048, 8, 128, 128) <= kda.NOALLOC_SCRATCH_BYTES
    for name, inp in (("first", big), ("second_smaller", small)):
        (o_ref, s_ref), (o, s) = _both(kda, inp)
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref), name
        ro, rs = oracle.forward(inp)
        check("noalloc/" + name, host64(o), ro, host64(s), rs, 2e-2, bf16_store=True)


def test_noalloc_windowed_beyond_the_scratch(kda):
    import torch
    B, T, H = 1, 4096, 64                                                               # 4096 records: 304 MB
    assert kda.workspace_bytes(B, T, H, 128, 128) > kda.NOALLOC_SCRATCH_BYTES
    assert kda.min_workspace_bytes(B, T, H, 128, 128) <= kda.NOALLOC_SCRATCH_BYTES
    inp = kda_inputs.make_prefill(63, B, T, H, 128, 128, s0_std=0.02)
    (o_ref, s_ref), (o, s) = _both(kda, inp)
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)


def test_noalloc_refuses_a_call_beyond_the_scratch(kda):
    import torch
    B, T, H = 1, 64, 512                                # one chunk of 512 chains: 71.6 MB at least
    assert kda.min_workspace_bytes(B, T, H, 128, 128) > kda.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, T, H, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((B, T, H, 128), dtype=torch.float32, device="cuda")
    beta = torch.zeros((B, T, H), dtype=torch.float32, device="cuda")
    o = torch.full((B, T, H, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kda.KDAError) as ei:
        kda.chunk_fwd_noalloc(q, q, q, g, beta, o=o)
    assert ei.value.status == 6
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())                                                       # nothing was launched
