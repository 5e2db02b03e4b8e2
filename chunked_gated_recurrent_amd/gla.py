"""Thin Python binding of libgla.so (the C ABI in include/gla.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs and workspace are allocated with torch, and the raw
device pointers plus torch's current HIP stream go to the library. Every step
of the computation runs in the library's HIP kernels; there is no fallback
of any kind. If libgla.so has not been built the first call raises.

Functions mirror the C entry points:
    gla_chunk_fwd(q, k, v, decay, ...)          -> (o, s_final)
    gla_chunk_fwd_varlen(q, k, v, cu, decay, ...) -> (o, s_final)
    gla_chunk_fwd_varlen_noalloc(q, k, v, cu, decay, out, ...) -> (out, s_final)
    gla_decode_step(q, k, v, decay, state, ...)  -> o   (state updated in place)
    gla_chunk_fwd_gated(q, k, v, g, decay, gate, ...) -> (o * act(g), s_final)
      (and g=, gate= on gla_chunk_fwd_varlen and gla_decode_step: the gated calls)
    gla_decode_step_pool(q, k, v, decay, state_pool, slots, ...) -> o
    gla_chunk_bwd(q, k, v, decay, dout, ...)    -> (dq, dk, dv, ds0)
    gla_chunk_bwd_varlen(q, k, v, cu, decay, dout, ...) -> (dq, dk, dv, ds0)
    short_conv_fwd(x, w, bias, window_in, ...)  -> (y, window_out)
    short_conv_decode_step(x, w, bias, window)  -> y   (window updated in place)
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgla.so")

GLA_F32, GLA_BF16 = 0, 1
# the output gate's activation (gla_gate)
GATES = {"sigmoid": 1, "silu": 2}
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGS = {
    "gla_abi_version": ([], _I),
    "gla_status_str": ([_I], ctypes.c_char_p),
    "gla_chunk_fwd_workspace_bytes": ([_I] * 7, ctypes.c_size_t),
    "gla_chunk_fwd": ([_I] * 7 + [_P, _P, _P, _P, ctypes.c_float, _P, _P, _P,
                                  _P, ctypes.c_size_t, _P], _I),
    "gla_chunk_bwd_workspace_bytes": ([_I] * 7, ctypes.c_size_t),
    "gla_chunk_bwd": ([_I] * 7 + [_P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P, _P,
                                  _P, _P, _P, ctypes.c_size_t, _P], _I),
    "gla_chunk_bwd_varlen_workspace_bytes": ([_I] * 7, ctypes.c_size_t),
    "gla_chunk_bwd_varlen": ([_I] * 7 + [_P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P,
                                         _P, _P, _P, _P, ctypes.c_size_t, _P], _I),
    "gla_chunk_fwd_varlen_workspace_bytes": ([_I] * 7, ctypes.c_size_t),
    "gla_chunk_fwd_varlen": ([_I] * 7 + [_P, _P, _P, _P, _P, ctypes.c_float, _P,
                                         _P, _P, _P, ctypes.c_size_t, _P], _I),
    "gla_chunk_fwd_varlen_noalloc": ([_I] * 7 + [_P, _P, _P, _P, _P, ctypes.c_float, _P,
                                                 _P, _P, _P], _I),
    "gla_linear_attn_fwd_workspace_bytes": ([_I] * 7, ctypes.c_size_t),
    "gla_linear_attn_fwd": ([_I] * 7 + [_P] * 9 + [ctypes.c_size_t, _P], _I),
    "gla_linear_attn_decode_step": ([_I] * 5 + [_P] * 7, _I),
    "gla_linear_attn_fwd_varlen_workspace_bytes": ([_I] * 7, ctypes.c_size_t),
    "gla_linear_attn_fwd_varlen": ([_I] * 7 + [_P] * 10 + [ctypes.c_size_t, _P], _I),
    "gla_decode_step": ([_I] * 5 + [_P, _P, _P, _P, ctypes.c_float, _P, _P, _P], _I),
    "gla_chunk_fwd_gated": ([_I] * 7 + [_P, _P, _P, _P, _I, _P, ctypes.c_float, _P, _P, _P,
                                        _P, ctypes.c_size_t, _P], _I),
    "gla_chunk_fwd_varlen_gated": ([_I] * 7 + [_P, _P, _P, _P, _P, _I, _P, ctypes.c_float,
                                               _P, _P, _P, _P, ctypes.c_size_t, _P], _I),
    "gla_decode_step_gated": ([_I] * 5 + [_P, _P, _P, _P, _I, _P, ctypes.c_float, _P, _P,
                                          _P], _I),
    "gla_short_conv_fwd": ([_I] * 4 + [_P] * 7, _I),
    "gla_short_conv_decode_step": ([_I] * 3 + [_P] * 6, _I),
    "gla_decode_step_pool": ([_I] * 5 + [_P, _P, _P, _P, ctypes.c_float, _P, _I, _P, _P, _P], _I),
}
EXPORTS = tuple(_SIGS)


class GlaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s: %s (status %d)" % (where, status_str(code), code))


def bind(L):
    """Declare the C signatures of every exported entry point on a loaded
    ctypes library handle; returns it."""
    for name, (args, res) in _SIGS.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libgla.so is not built (%s); run "
                "`python -m chunked_gated_recurrent_amd.build`" % LIB_PATH)
        import torch  # noqa: F401  -- bind to the HIP runtime torch loaded
        _lib = bind(ctypes.CDLL(LIB_PATH))
    return _lib


def abi_version() -> int:
    return lib().gla_abi_version()


def status_str(code: int) -> str:
    return lib().gla_status_str(code).decode()


def _dt(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GLA_BF16
    if t.dtype == torch.float32:
        return GLA_F32
    raise TypeError("q, k, v must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _decay_array(decay, H):
    d = np.ascontiguousarray(np.asarray(decay, dtype=np.float32).reshape(-1))
    if d.shape[0] != H:
        raise ValueError("decay must have H = %d entries" % H)
    return d, d.ctypes.data_as(ctypes.c_void_p)


def _check(t, name, dev, dtype=None, shape=None):
    if t.device != dev or dev.type != "cuda":
        raise ValueError("%s must be on the GPU of q (%s), got %s" % (name, dev, t.device))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and t.shape != shape:
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(dev):
    """torch's current stream on `dev` (a device with an index), as the
    hipStream_t the library launches on."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return ctypes.c_void_p(raw(dev.index))
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _gate_code(gate):
    if gate not in GATES:
        raise ValueError("gate must be one of %s, got %r" % (tuple(GATES), gate))
    return GATES[gate]


def _chunk_fwd(q, k, v, decay, scale, initial_state, output_final_state, chunk, out,
               final_state, workspace, g=None, gate=None):
    import torch
    dev = q.device
    B, T, H, dk = q.shape
    dv = v.shape[3]
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (B, T, H, dk))
    _check(v, "v", dev, q.dtype, (B, T, H, dv))
    if g is not None:
        _check(g, "g", dev, q.dtype, (B, T, H, dv))
    dt = _dt(q)
    if initial_state is not None:
        _check(initial_state, "initial_state", dev, torch.float32, (B, H, dk, dv))
    o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev) if out is None else out
    _check(o, "out", dev, q.dtype, (B, T, H, dv))
    sf = final_state
    if sf is None and output_final_state:
        sf = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if sf is not None:
        _check(sf, "final_state", dev, torch.float32, (B, H, dk, dv))
    L = lib()
    need = L.gla_chunk_fwd_workspace_bytes(dt, B, T, H, dk, dv, chunk)
    ws = workspace
    if need > 0 and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _d, dptr = _decay_array(decay, H)
    if g is None:
        rc = L.gla_chunk_fwd(dt, B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v),
                             dptr, float(scale), _ptr(initial_state), _ptr(o),
                             _ptr(sf), _ptr(ws), wsb, _stream(dev))
        where = "gla_chunk_fwd"
    else:
        rc = L.gla_chunk_fwd_gated(dt, B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(g), _gate_code(gate), dptr, float(scale),
                                   _ptr(initial_state), _ptr(o), _ptr(sf), _ptr(ws), wsb,
                                   _stream(dev))
        where = "gla_chunk_fwd_gated"
    if rc != 0:
        raise GlaError(rc, where)
    return o, sf


def gla_chunk_fwd(q, k, v, decay, scale: float = 1.0, initial_state=None,
                  output_final_state: bool = True, chunk: int = 0, out=None,
                  final_state=None, workspace=None):
    """Chunked forward of a fixed-length batch.

    q, k: [B, T, H, dk]; v: [B, T, H, dv] (bf16 or fp32, same dtype);
    decay: H floats on the host; initial_state: [B, H, dk, dv] fp32 or None.
    Returns (o [B, T, H, dv], s_final [B, H, dk, dv] fp32 or None).
    `final_state` may be `initial_state` itself (updated in place).
    """
    return _chunk_fwd(q, k, v, decay, scale, initial_state, output_final_state, chunk, out,
                      final_state, workspace)


def gla_chunk_fwd_gated(q, k, v, g, decay, gate: str, scale: float = 1.0,
                        initial_state=None, output_final_state: bool = True, chunk: int = 0,
                        out=None, final_state=None, workspace=None):
    """gla_chunk_fwd with the output gate: o * act(g) elementwise, act
    "sigmoid" or "silu"; g: [B, T, H, dv] in q's dtype. The final state is the
    ungated call's."""
    return _chunk_fwd(q, k, v, decay, scale, initial_state, output_final_state, chunk, out,
                      final_state, workspace, g, gate)


def linear_attn_fwd(q, k, v, initial_state=None, initial_z=None,
                    output_final_state: bool = True, chunk: int = 0, out=None,
                    final_state=None, final_z=None, workspace=None):
    """Normalised causal linear attention with ReLU features (no decay):
    o_t = phi(q_t) S_t / (phi(q_t) . z_t + 1e-6), S and z running sums of
    phi(k)^T v and phi(k).

    q, k: [B, T, H, dk]; v: [B, T, H, dv] (bf16 or fp32); initial_state
    [B, H, dk, dv] and initial_z [B, H, dk] fp32 or None. Returns
    (o, s_final or None, z_final or None).
    """
    import torch
    dev = q.device
    B, T, H, dk = q.shape
    dv = v.shape[3]
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (B, T, H, dk))
    _check(v, "v", dev, q.dtype, (B, T, H, dv))
    dt = _dt(q)
    if initial_state is not None:
        _check(initial_state, "initial_state", dev, torch.float32, (B, H, dk, dv))
    if initial_z is not None:
        _check(initial_z, "initial_z", dev, torch.float32, (B, H, dk))
    o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev) if out is None else out
    _check(o, "out", dev, q.dtype, (B, T, H, dv))
    sf, zf = final_state, final_z
    if output_final_state:
        if sf is None:
            sf = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        if zf is None:
            zf = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
    if sf is not None:
        _check(sf, "final_state", dev, torch.float32, (B, H, dk, dv))
    if zf is not None:
        _check(zf, "final_z", dev, torch.float32, (B, H, dk))
    L = lib()
    need = L.gla_linear_attn_fwd_workspace_bytes(dt, B, T, H, dk, dv, chunk)
    ws = workspace
    if need > 0 and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    rc = L.gla_linear_attn_fwd(dt, B, T, H, dk, dv, chunk, _ptr(q), _ptr(k), _ptr(v),
                               _ptr(initial_state), _ptr(initial_z), _ptr(o), _ptr(sf),
                               _ptr(zf), _ptr(ws), wsb, _stream(dev))
    if rc != 0:
        raise GlaError(rc, "gla_linear_attn_fwd")
    return o, sf, zf


def linear_attn_fwd_varlen(q, k, v, cu_seqlens, initial_state=None, initial_z=None,
                           output_final_state: bool = True, chunk: int = 0, out=None,
                           final_state=None, final_z=None, workspace=None):
    """linear_attn_fwd over packed sequences: q, k [total_T, H, dk], v
    [total_T, H, dv], cu_seqlens [N+1] int32 on the device; initial_state
    [N, H, dk, dv], initial_z [N, H, dk] fp32 or None. Returns
    (o, s_final or None, z_final or None)."""
    import torch
    dev = q.device
    total, H, dk = q.shape
    dv = v.shape[2]
    N = cu_seqlens.shape[0] - 1
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (total, H, dk))
    _check(v, "v", dev, q.dtype, (total, H, dv))
    _check(cu_seqlens, "cu_seqlens", dev, torch.int32, (N + 1,))
    if initial_state is not None:
        _check(initial_state, "initial_state", dev, torch.float32, (N, H, dk, dv))
    if initial_z is not None:
        _check(initial_z, "initial_z", dev, torch.float32, (N, H, dk))
    o = torch.empty((total, H, dv), dtype=q.dtype, device=dev) if out is None else out
    _check(o, "out", dev, q.dtype, (total, H, dv))
    sf, zf = final_state, final_z
    if output_final_state:
        if sf is None:
            sf = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        if zf is None:
            zf = torch.empty((N, H, dk), dtype=torch.float32, device=dev)
    if sf is not None:
        _check(sf, "final_state", dev, torch.float32, (N, H, dk, dv))
    if zf is not None:
        _check(zf, "final_z", dev, torch.float32, (N, H, dk))
    L = lib()
    dt = _dt(q)
    need = L.gla_linear_attn_fwd_varlen_workspace_bytes(dt, N, total, H, dk, dv, chunk)
    ws = workspace
    if need > 0 and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    rc = L.gla_linear_attn_fwd_varlen(dt, N, total, H, dk, dv, chunk, _ptr(cu_seqlens),
                                      _ptr(q), _ptr(k), _ptr(v), _ptr(initial_state),
                                      _ptr(initial_z), _ptr(o), _ptr(sf), _ptr(zf), _ptr(ws),
                                      wsb, _stream(dev))
    if rc != 0:
        raise GlaError(rc, "gla_linear_attn_fwd_varlen")
    return o, sf, zf


def linear_attn_decode_step(q, k, v, state, z, out=None):
    """One decode step of the normalised linear attention: q, k [N, H, dk],
    v [N, H, dv]; state [N, H, dk, dv] and z [N, H, dk] fp32, updated in
    place. Returns o [N, H, dv]."""
    import torch
    dev = q.device
    N, H, dk = q.shape
    dv = v.shape[2]
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (N, H, dk))
    _check(v, "v", dev, q.dtype, (N, H, dv))
    _check(state, "state", dev, torch.float32, (N, H, dk, dv))
    _check(z, "z", dev, torch.float32, (N, H, dk))
    o = torch.empty((N, H, dv), dtype=q.dtype, device=dev) if out is None else out
    _check(o, "out", dev, q.dtype, (N, H, dv))
    rc = lib().gla_linear_attn_decode_step(_dt(q), N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(state), _ptr(z), _ptr(o), _stream(dev))
    if rc != 0:
        raise GlaError(rc, "gla_linear_attn_decode_step")
    return o


def gla_chunk_fwd_varlen(q, k, v, cu_seqlens, decay, scale: float = 1.0,
                         initial_state=None, output_final_state: bool = True,
                         chunk: int = 0, out=None, final_state=None,
                         workspace=None, g=None, gate=None):
    """Chunked forward of N packed sequences.

    q, k: [total_T, H, dk]; v: [total_T, H, dv]; cu_seqlens: [N+1] int32 on
    the device. Returns (o [total_T, H, dv], s_final [N, H, dk, dv] or None).
    With g ([total_T, H, dv], q's dtype) and gate ("sigmoid" or "silu"):
    the gated call gla_chunk_fwd_varlen_gated, o * act(g).
    """
    import torch
    dev = q.device
    total, H, dk = q.shape
    dv = v.shape[2]
    N = cu_seqlens.shape[0] - 1
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (total, H, dk))
    _check(v, "v", dev, q.dtype, (total, H, dv))
    _check(cu_seqlens, "cu_seqlens", dev, torch.int32)
    if g is not None:
        _check(g, "g", dev, q.dtype, (total, H, dv))
    dt = _dt(q)
    if initial_state is not None:
        _check(initial_state, "initial_state", dev, torch.float32, (N, H, dk, dv))
    o = torch.empty((total, H, dv), dtype=q.dtype, device=dev) if out is None else out
    _check(o, "out", dev, q.dtype, (total, H, dv))
    sf = final_state
    if sf is None and output_final_state:
        sf = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if sf is not None:
        _check(sf, "final_state", dev, torch.float32, (N, H, dk, dv))
    L = lib()
    need = L.gla_chunk_fwd_varlen_workspace_bytes(dt, N, total, H, dk, dv, chunk)
    ws = workspace
    if need > 0 and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _d, dptr = _decay_array(decay, H)
    if g is None:
        rc = L.gla_chunk_fwd_varlen(dt, N, total, H, dk, dv, chunk, _ptr(cu_seqlens),
                                    _ptr(q), _ptr(k), _ptr(v), dptr, float(scale),
                                    _ptr(initial_state), _ptr(o), _ptr(sf), _ptr(ws),
                                    wsb, _stream(dev))
        where = "gla_chunk_fwd_varlen"
    else:
        rc = L.gla_chunk_fwd_varlen_gated(dt, N, total, H, dk, dv, chunk, _ptr(cu_seqlens),
                                          _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                          _gate_code(gate), dptr, float(scale),
                                          _ptr(initial_state), _ptr(o), _ptr(sf), _ptr(ws),
                                          wsb, _stream(dev))
        where = "gla_chunk_fwd_varlen_gated"
    if rc != 0:
        raise GlaError(rc, where)
    return o, sf


def gla_chunk_fwd_varlen_noalloc(q, k, v, cu_seqlens, decay, out, scale: float = 1.0,
                                 initial_state=None, final_state=None, chunk: int = 0):
    """gla_chunk_fwd_varlen without a workspace: the library's fixed
    per-GPU scratch array serves instead, and nothing is allocated here
    either, so the outputs come in: out [total_T, H, dv] (dtype of q) and
    final_state [N, H, dk, dv] fp32 or None. Calls that overlap in time on
    one GPU share that array and must not be issued. Returns (out,
    final_state)."""
    import torch
    dev = q.device
    total, H, dk = q.shape
    dv = v.shape[2]
    N = cu_seqlens.shape[0] - 1
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (total, H, dk))
    _check(v, "v", dev, q.dtype, (total, H, dv))
    _check(cu_seqlens, "cu_seqlens", dev, torch.int32)
    dt = _dt(q)
    if initial_state is not None:
        _check(initial_state, "initial_state", dev, torch.float32, (N, H, dk, dv))
    _check(out, "out", dev, q.dtype, (total, H, dv))
    if final_state is not None:
        _check(final_state, "final_state", dev, torch.float32, (N, H, dk, dv))
    _d, dptr = _decay_array(decay, H)
    rc = lib().gla_chunk_fwd_varlen_noalloc(dt, N, total, H, dk, dv, chunk,
                                            _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                                            dptr, float(scale), _ptr(initial_state),
                                            _ptr(out), _ptr(final_state), _stream(dev))
    if rc != 0:
        raise GlaError(rc, "gla_chunk_fwd_varlen_noalloc")
    return out, final_state


def gla_decode_step(q, k, v, decay, state, scale: float = 1.0, out=None, g=None, gate=None):
    """One decode step: state [N, H, dk, dv] fp32 is updated in place;
    returns o [N, H, dv]. With g ([N, H, dv], q's dtype) and gate ("sigmoid"
    or "silu"): the gated step gla_decode_step_gated, o * act(g)."""
    import torch
    dev = q.device
    N, H, dk = q.shape
    dv = v.shape[2]
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (N, H, dk))
    _check(v, "v", dev, q.dtype, (N, H, dv))
    _check(state, "state", dev, torch.float32, (N, H, dk, dv))
    if g is not None:
        _check(g, "g", dev, q.dtype, (N, H, dv))
    dt = _dt(q)
    o = torch.empty((N, H, dv), dtype=q.dtype, device=dev) if out is None else out
    _check(o, "out", dev, q.dtype, (N, H, dv))
    _d, dptr = _decay_array(decay, H)
    if g is None:
        rc = lib().gla_decode_step(dt, N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), dptr,
                                   float(scale), _ptr(state), _ptr(o), _stream(dev))
        where = "gla_decode_step"
    else:
        rc = lib().gla_decode_step_gated(dt, N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                         _gate_code(gate), dptr, float(scale), _ptr(state),
                                         _ptr(o), _stream(dev))
        where = "gla_decode_step_gated"
    if rc != 0:
        raise GlaError(rc, where)
    return o


def gla_decode_step_pool(q, k, v, decay, state_pool, slots, scale: float = 1.0, out=None):
    """One decode step against a state pool: row n of q [N, H, dk], k, v
    [N, H, dv] updates state_pool[slots[n]] ([P, H, dk, dv] fp32, in place);
    slots is an int32 tensor [N] on the device, and a slot outside [0, P)
    marks a padding row (o row zero, no state touched). Returns o [N, H, dv]."""
    import torch
    dev = q.device
    N, H, dk = q.shape
    dv = v.shape[2]
    P = state_pool.shape[0]
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (N, H, dk))
    _check(v, "v", dev, q.dtype, (N, H, dv))
    _check(state_pool, "state_pool", dev, torch.float32, (P, H, dk, dv))
    _check(slots, "slots", dev, torch.int32, (N,))
    dt = _dt(q)
    o = torch.empty((N, H, dv), dtype=q.dtype, device=dev) if out is None else out
    _check(o, "out", dev, q.dtype, (N, H, dv))
    _d, dptr = _decay_array(decay, H)
    rc = lib().gla_decode_step_pool(dt, N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), dptr,
                                    float(scale), _ptr(slots), P, _ptr(state_pool),
                                    _ptr(o), _stream(dev))
    if rc != 0:
        raise GlaError(rc, "gla_decode_step_pool")
    return o


def gla_chunk_bwd(q, k, v, decay, dout, scale: float = 1.0, initial_state=None,
                  ds_final=None, want_ds0: bool = True, chunk: int = 0,
                  dq=None, dk=None, dv=None, ds0=None, workspace=None):
    """Backward of gla_chunk_fwd: q, k [B, T, H, dk], v and dout [B, T, H, dv]
    (bf16 or fp32), decay H floats, initial_state and ds_final [B, H, dk, dv] fp32 or
    None. Returns (dq, dk, dv, ds0) with ds0 None unless want_ds0 or given."""
    import torch
    dev = q.device
    B, T, H, dk_ = q.shape
    dv_ = v.shape[3]
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (B, T, H, dk_))
    _check(v, "v", dev, q.dtype, (B, T, H, dv_))
    _check(dout, "dout", dev, q.dtype, (B, T, H, dv_))
    dt = _dt(q)
    for name, t in (("initial_state", initial_state), ("ds_final", ds_final)):
        if t is not None:
            _check(t, name, dev, torch.float32, (B, H, dk_, dv_))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check(dq, "dq", dev, q.dtype, (B, T, H, dk_))
    _check(dk, "dk", dev, q.dtype, (B, T, H, dk_))
    _check(dv, "dv", dev, q.dtype, (B, T, H, dv_))
    if ds0 is None and want_ds0:
        ds0 = torch.empty((B, H, dk_, dv_), dtype=torch.float32, device=dev)
    if ds0 is not None:
        _check(ds0, "ds0", dev, torch.float32, (B, H, dk_, dv_))
    L = lib()
    need = L.gla_chunk_bwd_workspace_bytes(dt, B, T, H, dk_, dv_, chunk)
    ws = workspace
    if need > 0 and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _d, dptr = _decay_array(decay, H)
    rc = L.gla_chunk_bwd(dt, B, T, H, dk_, dv_, chunk, _ptr(q), _ptr(k), _ptr(v), dptr,
                         float(scale), _ptr(initial_state), _ptr(dout), _ptr(ds_final),
                         _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ds0), _ptr(ws), wsb,
                         _stream(dev))
    if rc != 0:
        raise GlaError(rc, "gla_chunk_bwd")
    return dq, dk, dv, ds0


def gla_chunk_bwd_varlen(q, k, v, cu_seqlens, decay, dout, scale: float = 1.0,
                         initial_state=None, ds_final=None, want_ds0: bool = True,
                         chunk: int = 0, dq=None, dk=None, dv=None, ds0=None,
                         workspace=None):
    """Backward of gla_chunk_fwd_varlen: q, k [total_T, H, dk], v and dout
    [total_T, H, dv] (bf16 or fp32), cu_seqlens [N+1] int32 on the device,
    initial_state and ds_final [N, H, dk, dv] fp32 or None. Returns
    (dq, dk, dv, ds0)."""
    import torch
    dev = q.device
    total, H, dk_ = q.shape
    dv_ = v.shape[2]
    N = cu_seqlens.shape[0] - 1
    _check(q, "q", dev)
    _check(k, "k", dev, q.dtype, (total, H, dk_))
    _check(v, "v", dev, q.dtype, (total, H, dv_))
    _check(dout, "dout", dev, q.dtype, (total, H, dv_))
    _check(cu_seqlens, "cu_seqlens", dev, torch.int32, (N + 1,))
    dt = _dt(q)
    for name, t in (("initial_state", initial_state), ("ds_final", ds_final)):
        if t is not None:
            _check(t, name, dev, torch.float32, (N, H, dk_, dv_))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check(dq, "dq", dev, q.dtype, (total, H, dk_))
    _check(dk, "dk", dev, q.dtype, (total, H, dk_))
    _check(dv, "dv", dev, q.dtype, (total, H, dv_))
    if ds0 is None and want_ds0:
        ds0 = torch.empty((N, H, dk_, dv_), dtype=torch.float32, device=dev)
    if ds0 is not None:
        _check(ds0, "ds0", dev, torch.float32, (N, H, dk_, dv_))
    L = lib()
    need = L.gla_chunk_bwd_varlen_workspace_bytes(dt, N, total, H, dk_, dv_, chunk)
    ws = workspace
    if need > 0 and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _d, dptr = _decay_array(decay, H)
    rc = L.gla_chunk_bwd_varlen(dt, N, total, H, dk_, dv_, chunk, _ptr(cu_seqlens), _ptr(q),
                                _ptr(k), _ptr(v), dptr, float(scale), _ptr(initial_state),
                                _ptr(dout), _ptr(ds_final), _ptr(dq), _ptr(dk), _ptr(dv),
                                _ptr(ds0), _ptr(ws), wsb, _stream(dev))
    if rc != 0:
        raise GlaError(rc, "gla_chunk_bwd_varlen")
    return dq, dk, dv, ds0


def short_conv_fwd(x, w, bias=None, window_in=None, want_window: bool = True,
                   out=None, window_out=None):
    """Causal width-4 depthwise convolution + SiLU: x [B, T, D] (bf16 or
    fp32), w [D, 4] fp32, bias [D] fp32 or None, window_in [B, 4, D] fp32 or
    None. Returns (y [B, T, D], window_out [B, 4, D] fp32 or None)."""
    import torch
    dev = x.device
    B, T, D = x.shape
    _check(x, "x", dev)
    _check(w, "w", dev, torch.float32, (D, 4))
    if bias is not None:
        _check(bias, "bias", dev, torch.float32, (D,))
    if window_in is not None:
        _check(window_in, "window_in", dev, torch.float32, (B, 4, D))
    y = torch.empty_like(x) if out is None else out
    _check(y, "out", dev, x.dtype, (B, T, D))
    if window_out is None and want_window:
        window_out = torch.empty((B, 4, D), dtype=torch.float32, device=dev)
    if window_out is not None:
        _check(window_out, "window_out", dev, torch.float32, (B, 4, D))
    rc = lib().gla_short_conv_fwd(_dt(x), B, T, D, _ptr(x), _ptr(w), _ptr(bias),
                                  _ptr(window_in), _ptr(y), _ptr(window_out), _stream(dev))
    if rc != 0:
        raise GlaError(rc, "gla_short_conv_fwd")
    return y, window_out


def short_conv_decode_step(x, w, bias, window, out=None):
    """One decode step of the convolution: x [N, D], window [N, 4, D] fp32
    (shifted in place). Returns y [N, D]."""
    import torch
    dev = x.device
    N, D = x.shape
    _check(x, "x", dev)
    _check(w, "w", dev, torch.float32, (D, 4))
    if bias is not None:
        _check(bias, "bias", dev, torch.float32, (D,))
    _check(window, "window", dev, torch.float32, (N, 4, D))
    y = torch.empty_like(x) if out is None else out
    _check(y, "out", dev, x.dtype, (N, D))
    rc = lib().gla_short_conv_decode_step(_dt(x), N, D, _ptr(x), _ptr(w), _ptr(bias),
                                          _ptr(window), _ptr(y), _stream(dev))
    if rc != 0:
        raise GlaError(rc, "gla_short_conv_decode_step")
    return y
