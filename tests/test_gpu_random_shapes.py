"""GPU parity over seeded random shapes: batch size, ragged lengths (zero
included), head count, head dims, input dtype, packed or dense layout, the
initial state, the gate distribution and the entry-point flags drawn per
case, each compared with the fp64 oracle.  Marked ``gpu``."""
import numpy as np
import pytest

import kda_inputs
import oracle
from gpu_util import check, host64, inputs_to_device

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
CASES = 24


@pytest.fixture(scope="module")
def kda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_fwd_amd as m
    m.load()
    return m


def _draw_case(i):
    """One random configuration, drawn from its own seed."""
    r = np.random.default_rng(1000 + i)
    dtype = "f32" if r.random() < 0.25 else "bf16"
    dk, dv = (int(x) for x in r.choice([64, 128], size=2))
    if dtype == "bf16" and r.random() < 0.6:
        dk = dv = 128                        # the matrix-core path
    H = int(r.integers(1, 5))
    packed = r.random() < 0.5
    if packed:
        n = int(r.integers(1, 6))
        lengths = [int(x) if r.random() > 0.15 else 0 for x in r.integers(1, 260, size=n)]
        B, T = 1, 0
    else:
        lengths = None
        B, T = int(r.integers(1, 4)), int(r.integers(1, 330))
    gate = str(r.choice(["k3", "slow", "sigmoid"]))
    s0_std = float(r.choice([0.0, 0.02, 0.1]))
    out = str(r.choice(["same", "f32"]))
    fp32_path = bool(dtype == "bf16" and dk == dv == 128 and r.random() < 0.35)
    return dict(dtype=dtype, dk=dk, dv=dv, H=H, B=B, T=T, lengths=lengths, gate=gate, s0_std=s0_std,
                out=out, fp32_path=fp32_path)


@pytest.mark.parametrize("i", range(CASES))
def test_random_prefill(kda, i):
    import torch
    c = _draw_case(i)
    inp = kda_inputs.make_prefill(2000 + i, c["B"], c["T"], c["H"], c["dk"], c["dv"], dtype=c["dtype"],
                                  gate=c["gate"], s0_std=c["s0_std"], lengths=c["lengths"])
    print("case", i, c, flush=True)
    o_ref, s_ref = oracle.forward(inp)
    d = inputs_to_device(inp)
    odt = torch.float32 if (c["out"] == "f32" or c["dtype"] == "f32") else torch.bfloat16
    o, s = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["init_state"], d["cu_seqlens"],
                         out_dtype=odt, fp32_path=c["fp32_path"])
    torch.cuda.synchronize()
    tol = TOL_F32 if c["dtype"] == "f32" else TOL_BF16
    if o_ref.size == 0:
        assert o.numel() == 0
        np.testing.assert_array_equal(host64(s), s_ref)
        return
    check("random%d" % i, host64(o), o_ref, host64(s), s_ref, tol, bf16_store=(odt == torch.bfloat16))
    # zero-length sequences hand their initial state back unchanged
    if c["lengths"] is not None:
        for n, L in enumerate(c["lengths"]):
            if L == 0:
                want = 0.0 if inp.init_state is None else inp.init_state[n].astype(np.float64)
                np.testing.assert_array_equal(host64(s[n]), np.broadcast_to(want, s_ref[n].shape))


@pytest.mark.parametrize("i", range(8))
def test_random_decode_steps(kda, i):
    """A few consecutive decode steps on random (N, H, d, dtype) against the
    oracle's recurrence carried in fp64."""
    import torch
    r = np.random.default_rng(3000 + i)
    N, H = int(r.integers(1, 9)), int(r.integers(1, 5))
    d = int(r.choice([64, 128]))
    dtype = "f32" if r.random() < 0.3 else "bf16"
    S0 = kda_inputs.decode_initial_state(3000 + i, N, H, d, std=float(r.choice([0.0, 0.02, 0.1])))
    state = torch.from_numpy(np.ascontiguousarray(S0)).cuda()
    s_ref = S0.astype(np.float64)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    for step in range(3):
        x = kda_inputs.decode_step(3000 + i, step, N, H, d, dtype=dtype)
        f = (lambda a: kda_inputs.bf16_to_f32(a)) if dtype == "bf16" else (lambda a: a)
        o_ref, s_ref = oracle.decode_steps(s_ref, f(x.q), f(x.k), f(x.v), x.g, x.beta)
        dv = {name: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
              if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a)).cuda()
              for name, a in (("q", x.q), ("k", x.k), ("v", x.v), ("g", x.g), ("beta", x.beta))}
        o = kda.recurrent_step(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], state, out_dtype=torch.float32)
        torch.cuda.synchronize()
        check("rdecode%d/step%d" % (i, step), host64(o), o_ref, host64(state), s_ref, tol, bf16_store=False)
