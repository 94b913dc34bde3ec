"""gated_delta_rule_fwd_amd -- Python binding of libkda.so (KDA forward on MI355X).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI declared in include/kda.h.  PyTorch provides device
memory and the current stream.  There is no CPU fallback: if libkda.so is not
built, importing the library raises.

  chunk_fwd(q, k, v, g, beta, init_state=None, cu_seqlens=None, ...)
      -> (o, final_state)                       [kda_chunk_fwd]
  recurrent_step(q, k, v, g, beta, state, ...)
      -> o   (state updated in place)           [kda_recurrent_step]
  chunk_fwd_gated(q, k, v, z, A_log, beta, ..., dt_bias=None)
      -> (o, final_state)                       [kda_chunk_fwd_gated]
  recurrent_step_gated(q, k, v, z, A_log, beta, state, ..., dt_bias=None)
      -> o                                      [kda_recurrent_step_gated]

Each of them takes ``out_gate=`` (with ``norm_weight=``, ``norm_eps=``) to
apply the output norm o <- RMSNorm(o) * norm_weight * sigmoid(out_gate), and ``conv_weights=(w_q, w_k, w_v)`` to fuse the short
convolution + SiLU at the load of q, k, v (then raw projections); the
prefill calls take ``conv_init=`` / ``conv_final=`` (three [N, 3, H*d]
tensors each, entries may be None), the decode calls ``conv_state=`` (updated
in place).  Such calls go through kda_chunk_fwd_fused /
kda_recurrent_step_fused.

A long dense prefill overlaps its two kernels on the stream of a caller-owned
``Context`` (kda_context_create / kda_context_destroy).  By default the
prefill calls use one Context per host thread and device, made on first use
outside a graph capture and released with the thread; ``context=None`` runs
the kernels one after the other on the call's stream.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import threading

__all__ = ["chunk_fwd", "recurrent_step", "chunk_fwd_gated", "recurrent_step_gated", "workspace_bytes", "lib_path",
           "Context", "default_context", "chunk_fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "min_workspace_bytes",
           "load", "KDAError", "FLAG_QK_L2NORM", "FLAG_VALIDATE", "FLAG_FP32_PATH", "FLAG_BETA_LOGITS",
           "FLAG_SIGNED_ALPHA", "FLAG_OUT_NORM", "STATUS"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkda.so")

FLAG_QK_L2NORM = 0x1
FLAG_VALIDATE = 0x2
FLAG_FP32_PATH = 0x4
FLAG_BETA_LOGITS = 0x8
FLAG_SIGNED_ALPHA = 0x10
FLAG_OUT_NORM = 0x20
KDA_F32, KDA_BF16 = 0, 1
STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED", 3: "KDA_ERR_WORKSPACE",
          4: "KDA_ERR_RANGE", 5: "KDA_ERR_HIP", 6: "KDA_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20   # KDA_NOALLOC_SCRATCH_BYTES


class KDAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s (%d): %s" % (STATUS.get(status, "?"), status, msg))
        self.status = status


class ChunkDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int), ("d_k", ctypes.c_int),
                ("d_v", ctypes.c_int), ("num_seqs", ctypes.c_int), ("in_dtype", ctypes.c_int),
                ("out_dtype", ctypes.c_int), ("scale", ctypes.c_float), ("flags", ctypes.c_uint),
                ("context", ctypes.c_void_p)]


class DecayGate(ctypes.Structure):
    _fields_ = [("z", ctypes.c_void_p), ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p)]


class ShortConv(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p * 3), ("init_state", ctypes.c_void_p * 3),
                ("final_state", ctypes.c_void_p * 3)]


class OutNorm(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("weight", ctypes.c_void_p), ("eps", ctypes.c_float)]


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libkda.so is not built (%s); run python gated_delta_rule_fwd_amd/build.py" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, U, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint, ctypes.c_size_t
    lib.kda_chunk_fwd.restype = I
    lib.kda_chunk_fwd.argtypes = [ctypes.POINTER(ChunkDesc)] + [P] * 9 + [P, S, P]
    lib.kda_chunk_fwd_workspace_bytes.restype = S
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [ctypes.POINTER(ChunkDesc)]
    lib.kda_chunk_fwd_min_workspace_bytes.restype = S
    lib.kda_chunk_fwd_min_workspace_bytes.argtypes = [ctypes.POINTER(ChunkDesc)]
    lib.kda_recurrent_step.restype = I
    lib.kda_recurrent_step.argtypes = [I, I, I, I, I, I, F, U] + [P] * 7 + [P]
    lib.kda_chunk_fwd_gated.restype = I
    lib.kda_chunk_fwd_gated.argtypes = [ctypes.POINTER(ChunkDesc)] + [P] * 11 + [P, S, P]
    lib.kda_recurrent_step_gated.restype = I
    lib.kda_recurrent_step_gated.argtypes = [I, I, I, I, I, I, F, U] + [P] * 9 + [P]
    lib.kda_chunk_fwd_fused.restype = I
    lib.kda_chunk_fwd_fused.argtypes = [ctypes.POINTER(ChunkDesc)] + [P] * 4 + [ctypes.POINTER(DecayGate)] + \
        [P] * 3 + [ctypes.POINTER(ShortConv), ctypes.POINTER(OutNorm)] + [P, P, P, S, P]
    lib.kda_recurrent_step_fused.restype = I
    lib.kda_recurrent_step_fused.argtypes = [I, I, I, I, I, I, F, U] + [P] * 4 + [
        ctypes.POINTER(DecayGate), P, ctypes.POINTER(ShortConv), ctypes.POINTER(OutNorm), P, P, P]
    lib.kda_status_str.restype = ctypes.c_char_p
    lib.kda_status_str.argtypes = [I]
    lib.kda_last_hip_error.restype = I
    lib.kda_last_hip_error.argtypes = []
    lib.kda_version.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_chunk_fwd_noalloc.restype = I
    lib.kda_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(ChunkDesc)] + [P] * 9 + [P]
    lib.kda_context_create.restype = I
    lib.kda_context_create.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.kda_context_destroy.restype = I
    lib.kda_context_destroy.argtypes = [P]
    _lib = lib
    return lib


_exiting = False


@atexit.register
def _mark_exit():
    global _exiting
    _exiting = True


class Context:
    """A kda_context: the second HIP stream and the events with which a long
    dense prefill overlaps its two kernels, on the device that is current
    (or ``device``) when it is made.  Serves one call at a time; release it
    with close() (or by dropping it)."""

    def __init__(self, device=None):
        torch = _torch()
        lib = load()
        h = ctypes.c_void_p()
        with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
            self.device = torch.cuda.current_device()
            _check(lib.kda_context_create(ctypes.byref(h)))
        self._h = h.value

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("context is closed")
        return self._h

    def close(self):
        h, self._h = getattr(self, "_h", None), None
        if h is not None and not _exiting:
            _check(load().kda_context_destroy(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


_tls = threading.local()


def default_context(device=None):
    """This thread's Context for ``device`` (default: the current device),
    made on first use; None while the current stream is capturing a graph and
    none exists yet (no stream or event is made inside a capture)."""
    torch = _torch()
    if isinstance(device, torch.device):
        device = device.index
    dev = torch.cuda.current_device() if device is None else int(device)
    ctxs = getattr(_tls, "contexts", None)
    if ctxs is None:
        ctxs = _tls.contexts = {}
    c = ctxs.get(dev)
    if c is None and not torch.cuda.is_current_stream_capturing():
        c = ctxs[dev] = Context(dev)
    return c


def _check(status: int):
    if status != 0:
        lib = load()
        msg = lib.kda_status_str(status).decode()
        if status == 5:
            msg += " (hipError %d)" % lib.kda_last_hip_error()
        raise KDAError(status, msg)


def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.bfloat16:
        return KDA_BF16
    if dt == torch.float32:
        return KDA_F32
    raise TypeError("unsupported dtype %s (bf16 or fp32)" % dt)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype=None, shape=None):
    if t is None:
        raise ValueError("%s is required" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _desc(B, T, H, dk, dv, num_seqs, in_dt, out_dt, scale, flags, context=None) -> ChunkDesc:
    return ChunkDesc(B, T, H, dk, dv, num_seqs, in_dt, out_dt, float(scale), flags,
                     None if context is None else context.handle)


def workspace_bytes(B, T, H, dk, dv, *, num_seqs=0, in_bf16=True, out_bf16=True, scale=1.0, flags=FLAG_QK_L2NORM):
    """kda_chunk_fwd_workspace_bytes: the workspace of the fastest order."""
    d = _desc(B, T, H, dk, dv, num_seqs, KDA_BF16 if in_bf16 else KDA_F32, KDA_BF16 if out_bf16 else KDA_F32,
              scale, flags)
    return int(load().kda_chunk_fwd_workspace_bytes(ctypes.byref(d)))


def min_workspace_bytes(B, T, H, dk, dv, *, num_seqs=0, in_bf16=True, out_bf16=True, scale=1.0,
                        flags=FLAG_QK_L2NORM):
    """kda_chunk_fwd_min_workspace_bytes: the least workspace a call accepts
    (the windowed order; independent of T on the matrix-core path)."""
    d = _desc(B, T, H, dk, dv, num_seqs, KDA_BF16 if in_bf16 else KDA_F32, KDA_BF16 if out_bf16 else KDA_F32,
              scale, flags)
    return int(load().kda_chunk_fwd_min_workspace_bytes(ctypes.byref(d)))


def chunk_fwd(q, k, v, g, beta, init_state=None, cu_seqlens=None, *, out_dtype=None, scale=1.0,
              normalize=True, output_final_state=True, validate=False, fp32_path=False, beta_logits=False,
              signed_alpha=False, out_gate=None, norm_weight=None, norm_eps=1e-5, conv_weights=None,
              conv_init=None, conv_final=None, o=None, final_state=None, workspace=None, stream=None,
              context="default", workspace_limit=None):
    """Chunkwise KDA forward (prefill).  q, k, g: [B,T,H,d_k]; v: [B,T,H,d_v];
    beta: [B,T,H]; init_state: [N,H,d_k,d_v] fp32 or None; cu_seqlens: int32
    [N+1] device tensor or None (then N = B).  With signed_alpha (Complex KDA)
    g holds the signed decay alpha in [-1, 1] and beta may lie in [0, 2].
    out_gate ([B,T,H,d_v], q's dtype) fuses the output norm, with norm_weight
    ([d_v] fp32 or None) and norm_eps.  conv_weights ([H*d,4] fp32 for q, k,
    v) fuses the short convolution: q, k, v are then the raw projections,
    conv_init / conv_final the [N,3,H*d] conv states read / written.
    context: a Context, None (no overlap of the two kernels) or "default"
    (this thread's Context for the device).  o, final_state and the
    workspace, when not given, are allocated on ``stream``; the workspace
    at most workspace_limit bytes when that is given (but never below
    min_workspace_bytes: the windowed order, bit-identical and slower).
    Returns (o, final_state)."""
    return _chunk(q, k, v, g, None, beta, init_state, cu_seqlens, out_dtype, scale, normalize, output_final_state,
                  validate, fp32_path, beta_logits, o, final_state, workspace, stream, signed_alpha,
                  (out_gate, norm_weight, norm_eps), (conv_weights, conv_init, conv_final), context, workspace_limit)


def chunk_fwd_noalloc(q, k, v, g, beta, init_state=None, cu_seqlens=None, *, o, final_state=None, scale=1.0,
                      normalize=True, fp32_path=False, beta_logits=False, signed_alpha=False, stream=None,
                      context=None):
    """kda_chunk_fwd_noalloc: chunk_fwd for callers that cannot allocate.
    Nothing is allocated here or in the library: the caller passes o (and
    final_state, if wanted); the kernels' scratch is the library's fixed
    per-device area of NOALLOC_SCRATCH_BYTES (a call needing more runs in the
    windowed order; KDAError KDA_ERR_SCRATCH when even min_workspace_bytes
    exceeds it).  Calls that overlap on one GPU race on that area.
    Returns (o, final_state)."""
    torch = _torch()
    lib = load()
    _need(q, "q")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _need(k, "k", q.dtype, q.shape)
    _need(v, "v", q.dtype, (B, T, H, dv))
    _need(g, "g", torch.float32, (B, T, H, dk))
    _need(beta, "beta", torch.float32, (B, T, H))
    N = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        N = cu_seqlens.numel() - 1
    if init_state is not None:
        _need(init_state, "init_state", torch.float32, (N, H, dk, dv))
    _need(o, "o", None, (B, T, H, dv))
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, H, dk, dv))
    if context is not None and context.device != q.device.index:
        raise ValueError("context belongs to device %d, tensors to %s" % (context.device, q.device))
    flags = (FLAG_QK_L2NORM if normalize else 0) | (FLAG_FP32_PATH if fp32_path else 0) | \
        (FLAG_BETA_LOGITS if beta_logits else 0) | (FLAG_SIGNED_ALPHA if signed_alpha else 0)
    d = _desc(B, T, H, dk, dv, N if cu_seqlens is not None else 0, _dtype_code(q.dtype), _dtype_code(o.dtype),
              scale, flags, context)
    _check(lib.kda_chunk_fwd_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(init_state), _ptr(cu_seqlens), _ptr(o), _ptr(final_state),
                                     _stream(stream)))
    return o, final_state


def chunk_fwd_gated(q, k, v, z, A_log, beta, init_state=None, cu_seqlens=None, *, dt_bias=None, out_dtype=None,
                    scale=1.0, normalize=True, output_final_state=True, validate=False, fp32_path=False,
                    beta_logits=False, out_gate=None, norm_weight=None, norm_eps=1e-5, conv_weights=None,
                    conv_init=None, conv_final=None, o=None, final_state=None, workspace=None, stream=None,
                    context="default", workspace_limit=None):
    """As chunk_fwd, with g = -5 sigmoid(exp(A_log[h]) (z + dt_bias[h, c]))
    computed in the kernel: z [B,T,H,d_k] in q's dtype, A_log [H] fp32,
    dt_bias [H,d_k] fp32 or None."""
    return _chunk(q, k, v, None, (z, A_log, dt_bias), beta, init_state, cu_seqlens, out_dtype, scale, normalize,
                  output_final_state, validate, fp32_path, beta_logits, o, final_state, workspace, stream, False,
                  (out_gate, norm_weight, norm_eps), (conv_weights, conv_init, conv_final), context, workspace_limit)


def _norm_args(norm, o_shape, in_dtype, dv):
    """Checks the output-norm tensors; returns an OutNorm or None."""
    torch = _torch()
    out_gate, weight, eps = norm if norm is not None else (None, None, 0.0)
    if out_gate is None:
        if weight is not None:
            raise ValueError("norm_weight needs out_gate")
        return None
    _need(out_gate, "out_gate", in_dtype, o_shape)
    if weight is not None:
        _need(weight, "norm_weight", torch.float32, (dv,))
    return OutNorm(out_gate.data_ptr(), None if weight is None else weight.data_ptr(), float(eps))


def _conv_args(conv, N, H, dk, dv, dtype):
    """Checks the short-convolution tensors; returns a ShortConv or None."""
    torch = _torch()
    weights, inits, finals = conv if conv is not None else (None, None, None)
    if weights is None:
        if inits is not None or finals is not None:
            raise ValueError("conv states need conv_weights")
        return None
    inits = inits or (None, None, None)
    finals = finals or (None, None, None)
    sc = ShortConv()
    for i, (name, d) in enumerate((("q", dk), ("k", dk), ("v", dv))):
        _need(weights[i], "conv weight of " + name, torch.float32, (H * d, 4))
        sc.weight[i] = weights[i].data_ptr()
        for lst, field, what in ((inits, sc.init_state, "conv_init"), (finals, sc.final_state, "conv_final")):
            if lst[i] is not None:
                _need(lst[i], "%s of %s" % (what, name), dtype, (N, 3, H * d))
                field[i] = lst[i].data_ptr()
    return sc


def _chunk(q, k, v, g, gate, beta, init_state, cu_seqlens, out_dtype, scale, normalize, output_final_state,
           validate, fp32_path, beta_logits, o, final_state, workspace, stream, signed_alpha=False, norm=None,
           conv=None, context="default", workspace_limit=None):
    torch = _torch()
    lib = load()
    if stream is not None and stream != torch.cuda.current_stream(q.device):
        # the buffers this call allocates belong to `stream`: the caching
        # allocator then reuses them only behind that stream's work
        with torch.cuda.stream(stream):
            return _chunk(q, k, v, g, gate, beta, init_state, cu_seqlens, out_dtype, scale, normalize,
                          output_final_state, validate, fp32_path, beta_logits, o, final_state, workspace, None,
                          signed_alpha, norm, conv, context, workspace_limit)
    if isinstance(context, str):
        if context != "default":
            raise ValueError("context must be a Context, None or 'default'")
        context = default_context(q.device)
    _need(q, "q")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _need(k, "k", q.dtype, q.shape)
    _need(v, "v", q.dtype, (B, T, H, dv))
    if gate is None:
        _need(g, "g", torch.float32, (B, T, H, dk))
    else:
        z, A_log, dt_bias = gate
        _need(z, "z", q.dtype, (B, T, H, dk))
        _need(A_log, "A_log", torch.float32, (H,))
        if dt_bias is not None:
            _need(dt_bias, "dt_bias", torch.float32, (H, dk))
    _need(beta, "beta", torch.float32, (B, T, H))
    N = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        N = cu_seqlens.numel() - 1
    if init_state is not None:
        _need(init_state, "init_state", torch.float32, (N, H, dk, dv))
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=q.device)
    _need(o, "o", out_dtype, (B, T, H, dv))
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (N, H, dk, dv))
    on = _norm_args(norm, (B, T, H, dv), q.dtype, dv)
    sc = _conv_args(conv, N, H, dk, dv, q.dtype)
    flags = (FLAG_QK_L2NORM if normalize else 0) | (FLAG_VALIDATE if validate else 0) | \
        (FLAG_FP32_PATH if fp32_path else 0) | (FLAG_BETA_LOGITS if beta_logits else 0) | \
        (FLAG_SIGNED_ALPHA if signed_alpha else 0) | (FLAG_OUT_NORM if on is not None else 0)
    if context is not None and context.device != q.device.index:
        raise ValueError("context belongs to device %d, tensors to %s" % (context.device, q.device))
    d = _desc(B, T, H, dk, dv, N if cu_seqlens is not None else 0, _dtype_code(q.dtype), _dtype_code(out_dtype),
              scale, flags, context)
    ws = int(lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(d)))
    if workspace_limit is not None and ws > workspace_limit:
        ws = max(int(lib.kda_chunk_fwd_min_workspace_bytes(ctypes.byref(d))), int(workspace_limit))
    if ws > 0 and workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace")
    wsb = ctypes.c_size_t(0 if workspace is None else workspace.numel() * workspace.element_size())
    if on is not None or sc is not None:
        dg = None if gate is None else ctypes.byref(DecayGate(z.data_ptr(), A_log.data_ptr(),
                                                              None if dt_bias is None else dt_bias.data_ptr()))
        st = lib.kda_chunk_fwd_fused(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), dg, _ptr(beta),
                                     _ptr(init_state), _ptr(cu_seqlens), None if sc is None else ctypes.byref(sc),
                                     None if on is None else ctypes.byref(on), _ptr(o), _ptr(final_state),
                                     _ptr(workspace), wsb, _stream(stream))
    elif gate is None:
        st = lib.kda_chunk_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(init_state),
                               _ptr(cu_seqlens), _ptr(o), _ptr(final_state), _ptr(workspace), wsb, _stream(stream))
    else:
        st = lib.kda_chunk_fwd_gated(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A_log), _ptr(dt_bias),
                                     _ptr(beta), _ptr(init_state), _ptr(cu_seqlens), _ptr(o), _ptr(final_state),
                                     _ptr(workspace), wsb, _stream(stream))
    _check(st)
    return o, final_state


def recurrent_step(q, k, v, g, beta, state, *, out_dtype=None, scale=1.0, normalize=True, beta_logits=False,
                   signed_alpha=False, out_gate=None, norm_weight=None, norm_eps=1e-5, conv_weights=None,
                   conv_state=None, o=None, stream=None):
    """One fused decode step.  q, k, g: [N,H,d_k]; v: [N,H,d_v]; beta: [N,H];
    state: [N,H,d_k,d_v] fp32, updated in place.  With signed_alpha g holds
    the signed decay alpha.  out_gate [N,H,d_v] fuses the output norm;
    conv_weights the short convolution, with conv_state (three [N,3,H*d]
    caches, or None for zeros and no update) advanced in place.
    Returns o [N,H,d_v]."""
    return _step(q, k, v, g, None, beta, state, out_dtype, scale, normalize, beta_logits, o, stream, signed_alpha,
                 (out_gate, norm_weight, norm_eps), (conv_weights, conv_state, conv_state))


def recurrent_step_gated(q, k, v, z, A_log, beta, state, *, dt_bias=None, out_dtype=None, scale=1.0, normalize=True,
                         beta_logits=False, out_gate=None, norm_weight=None, norm_eps=1e-5, conv_weights=None,
                         conv_state=None, o=None, stream=None):
    """As recurrent_step, with g computed in the kernel from z [N,H,d_k],
    A_log [H] and dt_bias [H,d_k] (or None)."""
    return _step(q, k, v, None, (z, A_log, dt_bias), beta, state, out_dtype, scale, normalize, beta_logits, o, stream,
                 False, (out_gate, norm_weight, norm_eps), (conv_weights, conv_state, conv_state))


def _step(q, k, v, g, gate, beta, state, out_dtype, scale, normalize, beta_logits, o, stream, signed_alpha=False,
          norm=None, conv=None):
    torch = _torch()
    lib = load()
    if stream is not None and stream != torch.cuda.current_stream(q.device):
        with torch.cuda.stream(stream):   # o, when allocated here, belongs to `stream`
            return _step(q, k, v, g, gate, beta, state, out_dtype, scale, normalize, beta_logits, o, None,
                         signed_alpha, norm, conv)
    _need(q, "q")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _need(k, "k", q.dtype, q.shape)
    _need(v, "v", q.dtype, (N, H, dv))
    if gate is None:
        _need(g, "g", torch.float32, (N, H, dk))
    else:
        z, A_log, dt_bias = gate
        _need(z, "z", q.dtype, (N, H, dk))
        _need(A_log, "A_log", torch.float32, (H,))
        if dt_bias is not None:
            _need(dt_bias, "dt_bias", torch.float32, (H, dk))
    _need(beta, "beta", torch.float32, (N, H))
    _need(state, "state", torch.float32, (N, H, dk, dv))
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dtype, device=q.device)
    _need(o, "o", out_dtype, (N, H, dv))
    on = _norm_args(norm, (N, H, dv), q.dtype, dv)
    sc = _conv_args(conv, N, H, dk, dv, q.dtype)
    flags = (FLAG_QK_L2NORM if normalize else 0) | (FLAG_BETA_LOGITS if beta_logits else 0) | \
        (FLAG_SIGNED_ALPHA if signed_alpha else 0) | (FLAG_OUT_NORM if on is not None else 0)
    if on is not None or sc is not None:
        dg = None if gate is None else ctypes.byref(DecayGate(z.data_ptr(), A_log.data_ptr(),
                                                              None if dt_bias is None else dt_bias.data_ptr()))
        st = lib.kda_recurrent_step_fused(N, H, dk, dv, _dtype_code(q.dtype), _dtype_code(out_dtype), float(scale),
                                          flags, _ptr(q), _ptr(k), _ptr(v), _ptr(g), dg, _ptr(beta),
                                          None if sc is None else ctypes.byref(sc),
                                          None if on is None else ctypes.byref(on), _ptr(state), _ptr(o),
                                          _stream(stream))
    elif gate is None:
        st = lib.kda_recurrent_step(N, H, dk, dv, _dtype_code(q.dtype), _dtype_code(out_dtype), float(scale), flags,
                                    _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
                                    _stream(stream))
    else:
        st = lib.kda_recurrent_step_gated(N, H, dk, dv, _dtype_code(q.dtype), _dtype_code(out_dtype), float(scale),
                                          flags, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A_log), _ptr(dt_bias),
                                          _ptr(beta), _ptr(state), _ptr(o), _stream(stream))
    _check(st)
    return o
