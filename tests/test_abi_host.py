"""Host-side checks of the C ABI (CPU only, no GPU): the library loads, exports
every entry point include/kda.h declares, and rejects bad arguments before
launching anything.  Device pointers here are fake addresses that the
library never dereferences, because every call below fails its host checks."""
import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_fwd_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"KDA_API\s+[\w\s\*]+?\b(kda_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.lib_path()):
        pytest.skip("libkda.so not built")
    return kda.load()


def test_header_declares_expected_entry_points():
    assert _declared() == sorted(["kda_chunk_fwd", "kda_chunk_fwd_gated", "kda_chunk_fwd_fused",
                                  "kda_chunk_fwd_workspace_bytes", "kda_recurrent_step", "kda_recurrent_step_gated",
                                  "kda_recurrent_step_fused", "kda_status_str", "kda_last_hip_error", "kda_version",
                                  "kda_context_create", "kda_context_destroy", "kda_chunk_fwd_noalloc",
                                  "kda_chunk_fwd_min_workspace_bytes"])


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", kda.lib_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(kda_\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    for code in range(7):
        assert lib.kda_status_str(code) and lib.kda_status_str(code) != b"unknown status"
    assert b"ok" == lib.kda_status_str(0)
    assert lib.kda_version().startswith(b"kda-mi355x")
    assert lib.kda_last_hip_error() == 0


def test_noalloc_host_checks(lib):
    # rejected on the host before any device is touched: no descriptor, the
    # validate flag (it reads counters back to the host)
    P = [ctypes.c_void_p(FAKE + 0x100000 * i) for i in range(9)]
    assert lib.kda_chunk_fwd_noalloc(None, *P, None) == 1
    d = _desc(flags=kda.FLAG_QK_L2NORM | kda.FLAG_VALIDATE)
    assert lib.kda_chunk_fwd_noalloc(ctypes.byref(d), *P, None) == 2


def test_context_arguments(lib):
    assert lib.kda_context_create(None) == 1                   # nowhere to put the handle
    assert lib.kda_context_destroy(None) == 0                  # releasing nothing is a no-op


LAYOUT_DRIVER = r"""
#include <stddef.h>
#include <stdio.h>
#include "kda.h"
int main(void)
{
    printf("%zu %zu %zu %zu %zu\n", sizeof(kda_chunk_desc), offsetof(kda_chunk_desc, scale),
           offsetof(kda_chunk_desc, flags), offsetof(kda_chunk_desc, context), sizeof(kda_out_norm));
    return 0;
}
"""


def test_descriptor_layout_matches_the_header(tmp_path):
    """The binding's ctypes structures have the C layout of include/kda.h
    (compiled here with the host C compiler)."""
    import shutil
    cc = shutil.which("gcc") or shutil.which("cc")
    if not cc or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("no host C compiler or HIP headers")
    src, exe = tmp_path / "layout.c", tmp_path / "layout"
    src.write_text(LAYOUT_DRIVER)
    subprocess.run([cc, "-std=c99", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
                    "-I/opt/rocm/include", str(src), "-o", str(exe)], check=True, capture_output=True)
    size, off_scale, off_flags, off_ctx, norm_size = map(int, subprocess.run([str(exe)], capture_output=True,
                                                                             text=True, check=True).stdout.split())
    assert size == ctypes.sizeof(kda.ChunkDesc)
    assert off_scale == kda.ChunkDesc.scale.offset
    assert off_flags == kda.ChunkDesc.flags.offset
    assert off_ctx == kda.ChunkDesc.context.offset
    assert norm_size == ctypes.sizeof(kda.OutNorm)


def _desc(**kw):
    base = dict(B=1, T=64, H=2, d_k=128, d_v=128, num_seqs=0, in_dtype=1, out_dtype=1, scale=1.0,
                flags=kda.FLAG_QK_L2NORM)
    base.update(kw)
    return kda.ChunkDesc(**base)


FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def _call(lib, d, ptrs=None, ws=None, ws_bytes=0, cu=None):
    p = [FAKE + 0x100000 * i for i in range(9)]
    if ptrs:
        for i, val in ptrs.items():
            p[i] = val
    args = [ctypes.c_void_p(x) if x is not None else None for x in p]
    # slots: q k v g beta init o final
    return lib.kda_chunk_fwd(None if d is None else ctypes.byref(d), args[0], args[1], args[2], args[3], args[4],
                             args[5], None if cu is None else ctypes.c_void_p(cu), args[6], args[7],
                             None if ws is None else ctypes.c_void_p(ws), ctypes.c_size_t(ws_bytes), None)


def test_chunk_fwd_rejects_bad_arguments(lib):
    assert _call(lib, None) == 1
    assert _call(lib, _desc(d_k=96)) == 2                     # unsupported head dim
    assert _call(lib, _desc(d_v=32)) == 2
    assert _call(lib, _desc(in_dtype=7)) == 2                 # unknown dtype
    assert _call(lib, _desc(flags=0x80)) == 2                 # unknown flag
    assert _call(lib, _desc(B=0)) == 1
    assert _call(lib, _desc(H=0)) == 1
    assert _call(lib, _desc(T=-1)) == 1
    assert _call(lib, _desc(), ptrs={0: None}) == 1           # null q
    assert _call(lib, _desc(), ptrs={3: FAKE + 4}) == 1       # misaligned g
    assert _call(lib, _desc(), ptrs={4: FAKE + 2}) == 1       # misaligned beta
    assert _call(lib, _desc(B=2, num_seqs=2), cu=FAKE) == 1   # varlen needs B == 1
    assert _call(lib, _desc(B=1, num_seqs=-1), cu=FAKE) == 1
    d = _desc(flags=kda.FLAG_QK_L2NORM | kda.FLAG_VALIDATE)
    need = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert _call(lib, d, ws=FAKE, ws_bytes=need - 1) == 3      # workspace too small
    assert _call(lib, d, ws=None, ws_bytes=need) == 3
    assert lib.kda_chunk_fwd_workspace_bytes(None) == ctypes.c_size_t(-1).value
    assert _call(lib, _desc()) == 3                            # matrix-core path needs its record workspace


def test_size_limits(lib):
    # prefill: B*T*H <= 2^31 token-heads and N*H <= 2^22 chains (fp32 path: no workspace needed)
    f32 = dict(in_dtype=0, out_dtype=0)
    assert _call(lib, _desc(B=1, T=2 ** 29, H=5, **f32)) == 1
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(_desc(B=1, T=2 ** 29, H=5))) == 0
    assert _call(lib, _desc(B=4096, T=1, H=1025, **f32)) == 1
    # matrix-core path: 2^24 or more (chunk, head) records run in windows,
    # so such a call is not refused and its least workspace stays small
    d = _desc(B=1, T=2 ** 30, H=1)
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(d)) == 2 ** 24 * RECORD + STATE + seg_blocks(1, 2 ** 24) * STATE
    assert lib.kda_chunk_fwd_min_workspace_bytes(ctypes.byref(d)) == RECORD + STATE
    assert _call(lib, d, ws=FAKE, ws_bytes=RECORD + STATE - 16) == 3
    # decode: N*H <= 2^24 - 1 chains
    P = [ctypes.c_void_p(FAKE + 0x100000 * i) for i in range(7)]
    assert lib.kda_recurrent_step(2 ** 12, 2 ** 12, 128, 128, 1, 1, 1.0, kda.FLAG_QK_L2NORM, *P, None) == 1


RECORD = 74240   # bytes of chunk-local operands per (64-token chunk, head)
STATE = 128 * 128 * 4   # fp32 state of one chain, carried between the stages of a dense batch
# a batch of at most 42 chains and at least 48 chunks per sequence may take
# the segmented sequential pass: 3P - 3 state-sized blocks per chain for the
# most segments P it may take on any device, min(32, 128 // chains,
# chunks // 16) (segment 0's end state, B_s and M_s of the middle segments,
# the initial states of segments 1 .. P-1, a copy of the chain's initial
# state), 256-byte aligned after the rest


def seg_cap(chains, nck):
    return min(32, 128 // chains, nck // 16)


def seg_blocks(chains, nck):
    return 3 * seg_cap(chains, nck) - 3


def test_workspace_sizes(lib):
    size = lambda **kw: lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(_desc(**kw)))
    # fp32 arithmetic paths need nothing
    assert size(in_dtype=0) == 0
    assert size(d_k=64, d_v=64) == 0
    assert size(flags=kda.FLAG_QK_L2NORM | kda.FLAG_FP32_PATH) == 0
    # dense batch: B * ceil(T / 64) chunk records per head, then the state of every chain
    assert size(B=3, T=130, H=5) == 3 * 3 * 5 * RECORD + 3 * 5 * STATE
    # packed sequences: num_seqs + T // 64 slots per head plus one int32 per slot (256-byte rounded);
    # the descriptor does not say which layout is coming, so the larger need is reported
    slots = 7 + 1000 // 64
    assert size(B=1, T=1000, H=4, num_seqs=7) == max(slots * 4 * RECORD + 256, 16 * 4 * RECORD + 4 * STATE)
    assert size(B=1, T=64 * 40, H=2, num_seqs=3) == 40 * 2 * RECORD + 256 + 3 * 2 * RECORD
    # both readings may take the segmented pass here (at least 48 chunks, few chains): the packed one
    # (53 slots, 6 chains) needs more
    assert size(B=1, T=64 * 50, H=2, num_seqs=3) == 53 * 2 * RECORD + 256 + 6 * seg_blocks(6, 50) * STATE
    # segment states: chains <= 42 and ceil(T / 64) >= 48 (dense only)
    assert size(B=1, T=96 * 64, H=42) == 96 * 42 * RECORD + 42 * STATE + 42 * seg_blocks(42, 96) * STATE
    assert size(B=1, T=96 * 64, H=43) == 96 * 43 * RECORD + 43 * STATE
    assert size(B=1, T=47 * 64, H=2) == 47 * 2 * RECORD + 2 * STATE
    assert size(B=1, T=47 * 64 + 1, H=2) == 48 * 2 * RECORD + 2 * STATE + 2 * seg_blocks(2, 48) * STATE
    assert size(B=2, T=6100, H=3) == 2 * 96 * 3 * RECORD + 6 * STATE + 6 * seg_blocks(6, 96) * STATE
    # few chains of a long sequence: up to 32 segments, 93 blocks per chain
    assert size(B=1, T=64 * 4096, H=1) == 4096 * RECORD + STATE + 93 * STATE
    assert size(B=1, T=64 * 4096, H=4) == 4 * 4096 * RECORD + 4 * STATE + 4 * 93 * STATE
    assert size(B=1, T=64 * 4096, H=16) == 16 * 4096 * RECORD + 16 * STATE + 16 * 21 * STATE
    # validation counters come first
    assert size(B=2, T=64, H=1, flags=kda.FLAG_QK_L2NORM | kda.FLAG_VALIDATE) == 256 + 2 * RECORD + 2 * STATE
    # a misaligned workspace is refused before anything runs
    d = _desc(B=1, T=64, H=1)
    assert _call(lib, d, ws=FAKE + 8, ws_bytes=RECORD + STATE) == 1


def test_min_workspace_sizes(lib):
    """The least workspace: records for one chunk of every sequence, the
    carried states, the norm's words; never above the full figure; the
    same for every T on the matrix-core path."""
    mn = lambda **kw: lib.kda_chunk_fwd_min_workspace_bytes(ctypes.byref(_desc(**kw)))
    full = lambda **kw: lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(_desc(**kw)))
    assert lib.kda_chunk_fwd_min_workspace_bytes(None) == 2 ** 64 - 1
    assert mn(B=3, T=130, H=5) == 3 * 5 * RECORD + 15 * STATE
    for T in (1000, 10 ** 5, 10 ** 7):
        assert mn(B=2, T=T, H=4) == 2 * 4 * (RECORD + STATE)
    assert mn(B=2, T=10 ** 5, H=4, flags=kda.FLAG_QK_L2NORM | kda.FLAG_OUT_NORM) == 2 * 4 * (RECORD + STATE + 4096)
    assert mn(B=2, T=10 ** 5, H=4, flags=kda.FLAG_QK_L2NORM | kda.FLAG_VALIDATE) == 256 + 2 * 4 * (RECORD + STATE)
    # one chunk per sequence: nothing to window
    assert mn(B=3, T=64, H=5) == full(B=3, T=64, H=5)
    assert mn(B=3, T=0, H=5) == full(B=3, T=0, H=5)
    # packed: one chunk of each of the num_seqs sequences and their carried states;
    # the larger of the dense and the packed reading is reported
    assert mn(B=1, T=100000, H=4, num_seqs=7) == 7 * 4 * (RECORD + STATE)
    # fp32 path: nothing, or the fp32 staging of o for the norm (not windowed)
    assert mn(B=2, T=100, H=3, d_k=64, d_v=64) == 0
    assert mn(B=2, T=100, H=3, d_k=64, d_v=64, flags=kda.FLAG_QK_L2NORM | kda.FLAG_OUT_NORM) == 2 * 100 * 3 * 64 * 4
    for kw in (dict(B=3, T=130, H=5), dict(B=1, T=5000, H=2), dict(B=1, T=1000, H=4, num_seqs=7)):
        assert mn(**kw) <= full(**kw)
    # below the least size the call is refused before anything runs
    d = _desc(B=2, T=10 ** 5, H=4)
    assert _call(lib, d, ws=FAKE, ws_bytes=2 * 4 * (RECORD + STATE) - 16) == 3


def test_chunk_fwd_empty_batch_is_a_no_op(lib):
    # zero packed sequences: nothing to compute, no launch, no pointer touched
    assert _call(lib, _desc(B=1, T=0, num_seqs=0), ptrs={i: None for i in range(8)}, cu=FAKE) == 0


def test_recurrent_step_rejects_bad_arguments(lib):
    P = [ctypes.c_void_p(FAKE + 0x100000 * i) for i in range(7)]

    def call(N=4, H=2, dk=128, dv=128, it=1, ot=1, flags=kda.FLAG_QK_L2NORM, ptrs=P):
        return lib.kda_recurrent_step(N, H, dk, dv, it, ot, 1.0, flags, *ptrs, None)

    assert call(dk=32) == 2
    assert call(it=3) == 2
    assert call(flags=kda.FLAG_VALIDATE) == 2
    assert call(N=-1) == 1
    assert call(H=0) == 1
    assert call(ptrs=[None] + P[1:]) == 1
    assert call(ptrs=P[:5] + [ctypes.c_void_p(FAKE + 8)] + P[6:]) == 1   # misaligned state
    assert call(N=0, ptrs=[None] * 7) == 0                               # nothing to do


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(kda, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(kda, "_lib", None)
    with pytest.raises(ImportError):
        kda.load()


def _call_gated(lib, d, z=FAKE + 0x900000, a_log=FAKE + 0xA00000, dt_bias=None, beta=FAKE + 0xB00000, ws=None,
                ws_bytes=0):
    p = [ctypes.c_void_p(FAKE + 0x100000 * i) for i in range(3)]
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.kda_chunk_fwd_gated(ctypes.byref(d), p[0], p[1], p[2], vp(z), vp(a_log), vp(dt_bias), vp(beta),
                                   None, None, ctypes.c_void_p(FAKE + 0xC00000), None, vp(ws),
                                   ctypes.c_size_t(ws_bytes), None)


def test_gated_entry_points_reject_bad_arguments(lib):
    d = _desc(flags=kda.FLAG_QK_L2NORM | kda.FLAG_BETA_LOGITS)
    need = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert _call_gated(lib, d, z=None, ws=FAKE, ws_bytes=need) == 1          # z required
    assert _call_gated(lib, d, a_log=None, ws=FAKE, ws_bytes=need) == 1      # A_log required
    assert _call_gated(lib, d, z=FAKE + 8, ws=FAKE, ws_bytes=need) == 1      # z misaligned
    assert _call_gated(lib, d, a_log=FAKE + 2, ws=FAKE, ws_bytes=need) == 1  # A_log misaligned
    assert _call_gated(lib, d, dt_bias=FAKE + 4, ws=FAKE, ws_bytes=need) == 1
    assert _call_gated(lib, d, ws=None, ws_bytes=0) == 3                     # same workspace rule
    assert _call_gated(lib, _desc(flags=0x80)) == 2
    assert _call_gated(lib, _desc(flags=kda.FLAG_QK_L2NORM | kda.FLAG_SIGNED_ALPHA), ws=FAKE, ws_bytes=need) == 2
    P = [ctypes.c_void_p(FAKE + 0x100000 * i) for i in range(9)]

    def step(z=P[3], a_log=P[4], flags=kda.FLAG_QK_L2NORM):
        return lib.kda_recurrent_step_gated(4, 2, 128, 128, 1, 1, 1.0, flags, P[0], P[1], P[2], z, a_log, None,
                                            P[5], P[6], P[7], None)

    assert step(z=None) == 1
    assert step(a_log=None) == 1
    assert step(flags=kda.FLAG_VALIDATE) == 2
    assert lib.kda_recurrent_step_gated(0, 2, 128, 128, 1, 1, 1.0, 1, *([None] * 9), None) == 0


def test_workspace_for_the_output_norm(lib):
    size = lambda **kw: lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(_desc(**kw)))
    on = kda.FLAG_QK_L2NORM | kda.FLAG_OUT_NORM
    # matrix-core path: the two value slices of each chain exchange per-row
    # sums of o^2 through 2 x 4 x 64 words of 8 bytes per chain, after the
    # records; o itself is normalised as it is stored (bf16 or fp32)
    words = 2 * 4 * 64 * 8
    assert size(B=2, T=100, H=3, flags=on) == size(B=2, T=100, H=3) + 2 * 3 * words
    assert size(B=2, T=100, H=3, out_dtype=0, flags=on) == size(B=2, T=100, H=3) + 2 * 3 * words
    assert size(B=1, T=1000, H=2, num_seqs=5, flags=on) == size(B=1, T=1000, H=2, num_seqs=5) + 5 * 2 * words
    # a batch that may take the segmented pass: words for each of the up to
    # P segment units of the phase with outputs per chain, then the segment states
    assert size(B=1, T=96 * 64, H=2, flags=on) == (96 * 2 * RECORD + 2 * STATE + 2 * seg_cap(2, 96) * words +
                                                   2 * seg_blocks(2, 96) * STATE)
    # fp32 path: a bf16 o is staged in fp32 for the norm pass; an fp32 o is
    # normalised in place
    assert size(B=2, T=100, H=3, d_k=64, d_v=64, flags=on) == 2 * 100 * 3 * 64 * 4
    assert size(B=2, T=100, H=3, d_k=64, d_v=64, out_dtype=0, flags=on) == 0
    assert size(B=1, T=10, H=1, in_dtype=0, out_dtype=0, flags=on | kda.FLAG_VALIDATE) == 256


def _call_fused(lib, d, g=FAKE + 0x300000, dg=None, norm=None, ws=FAKE, ws_bytes=1 << 40, conv=None):
    p = [ctypes.c_void_p(FAKE + 0x100000 * i) for i in range(3)]
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.kda_chunk_fwd_fused(ctypes.byref(d), p[0], p[1], p[2], vp(g), None if dg is None else ctypes.byref(dg),
                                   ctypes.c_void_p(FAKE + 0x400000), None, None,
                                   None if conv is None else ctypes.byref(conv),
                                   None if norm is None else ctypes.byref(norm), ctypes.c_void_p(FAKE + 0x600000),
                                   None, vp(ws), ctypes.c_size_t(ws_bytes), None)


def _conv(weights=(FAKE + 0xD00000, FAKE + 0xD10000, FAKE + 0xD20000), inits=(None,) * 3, finals=(None,) * 3):
    sc = kda.ShortConv()
    for i in range(3):
        sc.weight[i], sc.init_state[i], sc.final_state[i] = weights[i], inits[i], finals[i]
    return sc


def test_fused_entry_points_reject_bad_arguments(lib):
    on = kda.FLAG_QK_L2NORM | kda.FLAG_OUT_NORM
    good = kda.OutNorm(FAKE + 0x800000, None, 1e-5)
    assert _call_fused(lib, _desc(flags=on), norm=None) == 1                        # flag without a norm
    assert _call_fused(lib, _desc(), norm=good) == 1                               # norm without the flag
    assert _call_fused(lib, _desc(flags=on), norm=kda.OutNorm(None, None, 1e-5)) == 1        # gate required
    assert _call_fused(lib, _desc(flags=on), norm=kda.OutNorm(FAKE + 8, None, 1e-5)) == 1    # gate misaligned
    assert _call_fused(lib, _desc(flags=on), norm=kda.OutNorm(FAKE + 0x800000, FAKE + 4, 1e-5)) == 1
    assert _call_fused(lib, _desc(flags=on), norm=kda.OutNorm(FAKE + 0x800000, None, -1.0)) == 1
    assert _call_fused(lib, _desc(flags=on), norm=kda.OutNorm(FAKE + 0x800000, None, float("nan"))) == 1
    assert _call_fused(lib, _desc(flags=on), norm=kda.OutNorm(FAKE + 0x600000, None, 1e-5)) == 1  # gate is o
    dg = kda.DecayGate(FAKE + 0x900000, FAKE + 0xA00000, None)
    assert _call_fused(lib, _desc(), dg=dg) == 1                                   # g and a decay gate
    assert _call_fused(lib, _desc(flags=on), g=None, dg=kda.DecayGate(FAKE + 0x900000, None, None),
                       norm=good) == 1                                             # A_log required
    assert _call_fused(lib, _desc(flags=on), norm=good, ws=None, ws_bytes=0) == 3  # same workspace rule
    assert _call_fused(lib, _desc(flags=on | kda.FLAG_SIGNED_ALPHA), g=None, dg=dg, norm=good) == 2
    P = [ctypes.c_void_p(FAKE + 0x100000 * i) for i in range(9)]

    def step(flags=on, norm=good, g=P[3], dg=None, N=4, conv=None):
        return lib.kda_recurrent_step_fused(N, 2, 128, 128, 1, 1, 1.0, flags, P[0], P[1], P[2], g,
                                            None if dg is None else ctypes.byref(dg), P[4],
                                            None if conv is None else ctypes.byref(conv),
                                            None if norm is None else ctypes.byref(norm), P[5], P[6], None)

    assert step(norm=None) == 1
    assert step(flags=kda.FLAG_QK_L2NORM) == 1
    assert step(norm=kda.OutNorm(None, None, 0.0)) == 1
    assert step(norm=kda.OutNorm(FAKE + 0x800000, None, float("inf"))) == 1
    assert step(dg=dg) == 1
    assert step(flags=on | kda.FLAG_VALIDATE) == 2
    assert step(N=0) == 0
    assert _call(lib, _desc(flags=on), ws=FAKE, ws_bytes=1 << 40) == 1      # the plain entry points take no norm
    # short convolution: every weight required, every pointer 16-byte aligned
    plain = kda.FLAG_QK_L2NORM
    assert _call_fused(lib, _desc(), conv=_conv(weights=(FAKE, None, FAKE))) == 1
    assert _call_fused(lib, _desc(), conv=_conv(weights=(FAKE, FAKE + 4, FAKE))) == 1
    assert _call_fused(lib, _desc(), conv=_conv(inits=(None, FAKE + 8, None))) == 1
    assert _call_fused(lib, _desc(), conv=_conv(finals=(None, None, FAKE + 2))) == 1
    assert _call_fused(lib, _desc(), conv=_conv(), ws=None, ws_bytes=0) == 3      # same workspace rule
    assert step(flags=plain, norm=None, conv=_conv(weights=(None, FAKE, FAKE))) == 1
    assert step(flags=plain, norm=None, conv=_conv(inits=(FAKE + 4, None, None))) == 1
    assert step(flags=plain, norm=None, conv=_conv(), N=0) == 0
