"""Parity past 2^31 elements per tensor: at T = 65536 and H = 320 the bf16 q,
k, v and o hold 2.7e9 elements (byte offsets up to 5.4e9) and the fp32 g
byte offsets reach 1.07e10, so any 32-bit index arithmetic in the kernels
would read or write the wrong rows.  A 64-head prefill of 270,000 tokens
does the same through the staged order, and the decode state at N = 512, H = 320
holds 2.7e9 fp32 values likewise.

The inputs are four seeded chains tiled over the heads (head h carries chain
h mod 4): every head is then checked bit for bit against its chain's
representative (a property that holds at any size and covers every head's
output and state region), and the first and last four heads are checked
against the fp64 oracle on those four chains.  Marked ``gpu``."""
import numpy as np
import pytest

import kda_inputs
import oracle
from gpu_util import check, host64

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
CHAINS = 4


@pytest.fixture(scope="module")
def kda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_fwd_amd as m
    m.load()
    return m


def _tile(base, axis, count):
    """base repeated along ``axis`` so that index h holds base index h % CHAINS."""
    import torch
    idx = torch.arange(count, device=base.device) % CHAINS
    return base.index_select(axis, idx).contiguous()


def _dev(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _same_as_representatives(x, axis, count):
    """Every index along ``axis`` equals index (h mod CHAINS), bit for bit."""
    import torch
    shape = list(x.shape)
    grouped = x.view(*shape[:axis], count // CHAINS, CHAINS, *shape[axis + 1:])
    rep = x.narrow(axis, 0, CHAINS).unsqueeze(axis)
    return bool(torch.equal(grouped, rep.expand_as(grouped)))


def test_prefill_past_2_31_elements(kda):
    import torch
    T, H, d = 65536, 320, 128
    assert T * H * d > 2 ** 31
    print("large prefill T=%d H=%d" % (T, H), flush=True)
    base = kda_inputs.make_prefill(91, 1, T, CHAINS, d, d, dtype="bf16", s0_std=0.02)
    o_ref, s_ref = oracle.forward(base)

    q, k, v = (_tile(_dev(getattr(base, n)), 2, H) for n in ("q", "k", "v"))
    g = _tile(_dev(base.g), 2, H)
    beta = _tile(_dev(base.beta), 2, H)
    s0 = _tile(_dev(base.init_state), 1, H)
    o, s = kda.chunk_fwd(q, k, v, g, beta, s0)
    torch.cuda.synchronize()
    del q, k, v, g, beta

    assert _same_as_representatives(o, 2, H), "o of a head differs from its chain's representative"
    assert _same_as_representatives(s, 1, H), "final state of a head differs from its chain's representative"
    for heads in (range(CHAINS), range(H - CHAINS, H)):
        sel = torch.tensor(list(heads), device="cuda")
        o_h = host64(o.index_select(2, sel))
        s_h = host64(s.index_select(1, sel))
        for j, h in enumerate(heads):
            c = h % CHAINS
            check("large_prefill/h%d" % h, o_h[:, :, j], o_ref[:, :, c], s_h[:, j], s_ref[:, c], TOL_BF16,
                  bf16_store=True)


def test_staged_prefill_past_2_31_elements(kda):
    """A dense prefill that runs in stages (64 heads leave CUs idle during the
    sequential pass) at T = 270,000 tokens: 2.2e9 elements per bf16 tensor and
    4,219 chunks per chain.  Every head against its representative bit for
    bit, the four representatives against the oracle on the first and last
    65,536 tokens and on the final state."""
    import torch
    T, H, d = 270_000, 64, 128
    assert T * H * d > 2 ** 31
    print("large staged prefill T=%d H=%d" % (T, H), flush=True)
    base = kda_inputs.make_prefill(93, 1, T, CHAINS, d, d, dtype="bf16", s0_std=0.02)
    o_ref, s_ref = oracle.forward(base)
    q, k, v = (_tile(_dev(getattr(base, n)), 2, H) for n in ("q", "k", "v"))
    g = _tile(_dev(base.g), 2, H)
    beta = _tile(_dev(base.beta), 2, H)
    s0 = _tile(_dev(base.init_state), 1, H)
    o, s = kda.chunk_fwd(q, k, v, g, beta, s0)
    torch.cuda.synchronize()
    del q, k, v, g, beta
    assert _same_as_representatives(o, 2, H), "o of a head differs from its chain's representative"
    assert _same_as_representatives(s, 1, H), "final state of a head differs from its chain's representative"
    W = 65536
    for h in range(CHAINS):
        s_h = host64(s[:, h])
        for t0 in (0, T - W):
            o_h = host64(o[:, t0:t0 + W, h])
            check("large_staged/h%d/t%d" % (h, t0), o_h, o_ref[:, t0:t0 + W, h], s_h, s_ref[:, h], TOL_BF16,
                  bf16_store=True)


def test_decode_state_past_2_31_elements(kda):
    import torch
    N, H, d = 512, 320, 128
    chains = N * H
    assert chains * d * d > 2 ** 31
    print("large decode N=%d H=%d" % (N, H), flush=True)
    S0 = kda_inputs.decode_initial_state(92, 1, CHAINS, d)          # [1, 4, d, d]
    state = _tile(_dev(S0[0]), 0, chains).view(N, H, d, d)
    s_ref = S0[0].astype(np.float64)[None]                          # [1, 4, d, d]
    for step in range(2):
        x = kda_inputs.decode_step(92, step, 1, CHAINS, d)
        args = [_tile(_dev(a[0]), 0, chains).view(N, H, *a.shape[2:]) for a in (x.q, x.k, x.v, x.g, x.beta)]
        o = kda.recurrent_step(*args, state, out_dtype=torch.float32)
        torch.cuda.synchronize()
        f = kda_inputs.bf16_to_f32
        o_ref, s_ref = oracle.decode_steps(s_ref, f(x.q), f(x.k), f(x.v), x.g, x.beta)
        flat_o, flat_s = o.view(chains, d), state.view(chains, d, d)
        assert _same_as_representatives(flat_o, 0, chains), "step %d: o" % step
        assert _same_as_representatives(flat_s, 0, chains), "step %d: state" % step
        for c0 in (0, chains - CHAINS):
            for j in range(CHAINS):
                c = c0 + j
                check("large_decode/step%d/chain%d" % (step, c), host64(flat_o[c]), o_ref[0, c % CHAINS],
                      host64(flat_s[c]), s_ref[0, c % CHAINS], TOL_BF16, bf16_store=False)
