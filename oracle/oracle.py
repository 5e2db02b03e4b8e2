"""Python front end of the fp64 CPU oracle (``gla_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this module; the GPU library and its binding never
import it. It takes numpy arrays, widens bf16 bit patterns to fp32 exactly,
and calls the plain token-by-token fp64 recurrence of the Laplace 3B /
Trainium2 page, section "GLA mixer" (S_t = lambda_h S_{t-1} + k_t^T v_t,
o_t = scale * q_t S_t, readout after the update), its backward, and, in
plain numpy, the short causal convolution in front of the mixer and the
normalised causal linear attention of the linear-attention tutorial page.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gla_oracle.c with gcc into oracle/liboracle.so (plain C11, -O2,
    generic x86-64 so the same file runs on any host of the image)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fno-fast-math",
             "-Wall", "-Wextra", "-o", tmp, _SRC, "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # a sanitizer build of the same source (the host sanitizer tests run
        # the oracle's pins against one), else the regular build
        path = os.environ.get("GLA_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB):
                build(force=False)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.oracle_gla_varlen.argtypes = [
            ctypes.c_int, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            P, P, P, P, ctypes.c_double, P, P, P, ctypes.c_int]
        lib.oracle_gla_varlen.restype = ctypes.c_int
        lib.oracle_gla_decode.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            P, P, P, P, ctypes.c_double, P, P, ctypes.c_int]
        lib.oracle_gla_decode.restype = ctypes.c_int
        lib.oracle_gla_bwd_varlen.argtypes = [
            ctypes.c_int, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            P, P, P, P, ctypes.c_double, P, P, P, P, P, P, P, ctypes.c_int]
        lib.oracle_gla_bwd_varlen.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    """Threads for the oracle: OMP_NUM_THREADS when set, else the visible
    cores capped at 16."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    return max(1, min(16, os.cpu_count() or 1))


def widen(x) -> np.ndarray:
    """Exact widening to fp32: a uint16 array is taken as bf16 bit patterns
    (bits << 16); float arrays are cast to fp32 (they must hold fp32 values)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(x, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def gla_varlen(cu_seqlens, q, k, v, decay, scale=1.0, s0=None,
               want_o=True, want_state=True, threads=None):
    """Packed variable-length recurrence in fp64.

    q, k: [total, H, dk]; v: [total, H, dv] (fp32 values or bf16 bits as
    uint16); cu_seqlens: [N+1] ints; decay: [H] fp32; s0: [N, H, dk, dv]
    (fp32, or fp64 for a state carried out of an earlier oracle call) or
    None. Returns (o [total, H, dv] fp64 or None, s_final [N, H, dk, dv]
    fp64 or None).
    """
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    q, k, v = widen(q), widen(k), widen(v)
    total, H, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    if k.shape != (total, H, dk) or v.shape[:2] != (total, H) or cu[-1] != total:
        raise ValueError("shape mismatch")
    lam = np.ascontiguousarray(np.asarray(decay, dtype=np.float32))
    if lam.shape != (H,):
        raise ValueError("decay must be [H]")
    s0a = None
    if s0 is not None:
        s0 = np.asarray(s0)
        s0a = s0 if s0.dtype == np.float64 else widen(s0).astype(np.float64)
        s0a = np.ascontiguousarray(s0a.reshape(N, H, dk, dv))
    o = np.zeros((total, H, dv), np.float64) if want_o else None
    sf = np.zeros((N, H, dk, dv), np.float64) if want_state else None
    rc = _load().oracle_gla_varlen(
        N, _ptr(cu), H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(lam),
        float(scale), _ptr(s0a), _ptr(o), _ptr(sf),
        int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle_gla_varlen failed: %d" % rc)
    return o, sf


def gla_fwd(q, k, v, decay, scale=1.0, s0=None, want_o=True, want_state=True,
            threads=None):
    """Fixed-length batch [B, T, H, d] through the same recurrence
    (sequence b owns tokens b*T .. b*T+T-1 of the flattened batch)."""
    q, k, v = widen(q), widen(k), widen(v)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    cu = np.arange(B + 1, dtype=np.int64) * T
    o, sf = gla_varlen(cu, q.reshape(B * T, H, dk), k.reshape(B * T, H, dk),
                       v.reshape(B * T, H, dv), decay, scale, s0,
                       want_o, want_state, threads)
    return (None if o is None else o.reshape(B, T, H, dv)), sf


def gla_bwd_varlen(cu_seqlens, q, k, v, decay, dout, scale=1.0, s0=None,
                   ds_final=None, threads=None):
    """Backward of the packed recurrence in fp64 (chain rule written out
    token by token: a forward sweep for dq, a reverse sweep carrying
    dL/dS for dk, dv and dS0; the training backward of the Laplace 3B /
    Trainium2 page, section "Challenge 3").

    dout: [total, H, dv] (fp32 or bf16 bits); ds_final: [N, H, dk, dv] or
    None (zero). Returns (dq, dk [total, H, dk], dv [total, H, dv],
    ds0 [N, H, dk, dv]), all fp64."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    q, k, v, dout = widen(q), widen(k), widen(v), widen(dout)
    total, H, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    if k.shape != (total, H, dk) or v.shape != (total, H, dv) or \
            dout.shape != (total, H, dv) or cu[-1] != total:
        raise ValueError("shape mismatch")
    lam = np.ascontiguousarray(np.asarray(decay, dtype=np.float32))
    if lam.shape != (H,):
        raise ValueError("decay must be [H]")

    def state(x):
        if x is None:
            return None
        x = np.asarray(x)
        x = x if x.dtype == np.float64 else widen(x).astype(np.float64)
        return np.ascontiguousarray(x.reshape(N, H, dk, dv))
    s0a, dsf = state(s0), state(ds_final)
    dq = np.zeros((total, H, dk), np.float64)
    dk_ = np.zeros((total, H, dk), np.float64)
    dv_ = np.zeros((total, H, dv), np.float64)
    ds0 = np.zeros((N, H, dk, dv), np.float64)
    rc = _load().oracle_gla_bwd_varlen(
        N, _ptr(cu), H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(lam),
        float(scale), _ptr(s0a), _ptr(dout), _ptr(dsf), _ptr(dq), _ptr(dk_),
        _ptr(dv_), _ptr(ds0), int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle_gla_bwd_varlen failed: %d" % rc)
    return dq, dk_, dv_, ds0


def gla_bwd(q, k, v, decay, dout, scale=1.0, s0=None, ds_final=None, threads=None):
    """Backward of a fixed-length batch [B, T, H, d]; returns (dq, dk, dv
    [B, T, H, d], ds0 [B, H, dk, dv]) in fp64."""
    q, k, v, dout = widen(q), widen(k), widen(v), widen(dout)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    cu = np.arange(B + 1, dtype=np.int64) * T
    dq, dk_, dv_, ds0 = gla_bwd_varlen(
        cu, q.reshape(B * T, H, dk), k.reshape(B * T, H, dk), v.reshape(B * T, H, dv),
        decay, dout.reshape(B * T, H, dv), scale, s0, ds_final, threads)
    return (dq.reshape(B, T, H, dk), dk_.reshape(B, T, H, dk),
            dv_.reshape(B, T, H, dv), ds0)


def gla_decode(q, k, v, decay, state, scale=1.0, threads=None):
    """One decode step. q, k: [N, H, dk]; v: [N, H, dv]; state: [N, H, dk, dv]
    fp64, updated IN PLACE. Returns o [N, H, dv] fp64."""
    q, k, v = widen(q), widen(k), widen(v)
    N, H, dk = q.shape
    dv = v.shape[2]
    if state.dtype != np.float64 or not state.flags.c_contiguous or \
            state.shape != (N, H, dk, dv):
        raise ValueError("state must be a C-contiguous fp64 [N,H,dk,dv] array")
    lam = np.ascontiguousarray(np.asarray(decay, dtype=np.float32))
    o = np.zeros((N, H, dv), np.float64)
    rc = _load().oracle_gla_decode(
        N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(lam), float(scale),
        _ptr(state), _ptr(o), int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle_gla_decode failed: %d" % rc)
    return o


def gla_decode_pool(q, k, v, decay, pool, slots, scale=1.0, threads=None):
    """One decode step against a pool of per-sequence state pages (Laplace
    3B / Trainium2 page, inference section: each sequence keeps a fixed
    state page, batches are padded to fixed widths). Row n updates pool
    entry slots[n]; a slot outside [0, P) is a padding row whose output is
    zero and which touches no state. The valid slots must be distinct.
    pool: [P, H, dk, dv] fp64, updated IN PLACE. Returns o [N, H, dv] fp64.

    Written as the plain definition: gather the named pages, run the direct
    decode step on them, scatter them back."""
    slots = np.asarray(slots, dtype=np.int64).reshape(-1)
    P = pool.shape[0]
    valid = np.nonzero((slots >= 0) & (slots < P))[0]
    if np.unique(slots[valid]).size != valid.size:
        raise ValueError("valid slots must be distinct")
    q, k, v = widen(q), widen(k), widen(v)
    N, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((N, H, dv), np.float64)
    if valid.size:
        pages = np.ascontiguousarray(pool[slots[valid]])
        o[valid] = gla_decode(q[valid], k[valid], v[valid], decay, pages, scale, threads)
        pool[slots[valid]] = pages
    return o


def short_conv(x, w, bias=None, window=None):
    """Causal depthwise convolution of width K followed by SiLU, in fp64
    (Laplace 3B / Trainium2 page, section on the layer's normalisation and
    convolution: every channel of the residual stream passes through a
    causal Conv1d of width 4 with SiLU, a 4-gram summary per position).

    x: [B, T, D]; w: [D, K] (tap j multiplies the input K-1-j tokens back,
    so tap K-1 is the current token); bias: [D] or None; window: [B, K, D]
    or None, the K most recent inputs before x, oldest first (zeros when
    None). Returns (y [B, T, D], window_out [B, K, D]): y_t = SiLU(z_t),
    z_t[c] = bias[c] + sum_j w[c, j] x_{t-K+1+j}[c], SiLU(z) = z / (1 + e^-z),
    and window_out the K most recent inputs after x."""
    x = widen(x).astype(np.float64)
    w = np.asarray(w, np.float64)
    B, T, D = x.shape
    K = w.shape[1]
    hist = np.zeros((B, K, D)) if window is None else np.asarray(window, np.float64)
    X = np.concatenate([hist, x], axis=1)          # [B, K + T, D]
    y = np.zeros((B, T, D))
    for t in range(T):
        z = np.zeros((B, D)) if bias is None else np.broadcast_to(
            np.asarray(bias, np.float64), (B, D)).copy()
        for j in range(K):
            z += w[:, j] * X[:, t + 1 + j]
        y[:, t] = z / (1.0 + np.exp(-z))
    return y, X[:, T:T + K].copy()


def short_conv_decode(x, w, bias, window):
    """One decode step of short_conv: window [N, K, D] fp64 is shifted by one
    token IN PLACE (the oldest input drops out, x enters last) and
    y = SiLU(bias + sum_j w[:, j] window[:, j]) is returned, [N, D] fp64."""
    x = widen(x).astype(np.float64)
    w = np.asarray(w, np.float64)
    window[:, :-1] = window[:, 1:].copy()
    window[:, -1] = x
    z = (window * w.T[None]).sum(axis=1)
    if bias is not None:
        z = z + np.asarray(bias, np.float64)
    return z / (1.0 + np.exp(-z))


LINEAR_ATTN_EPS = 1e-6


def linear_attention(q, k, v, s0=None, z0=None, eps=LINEAR_ATTN_EPS):
    """Normalised causal linear attention in fp64, token by token (the
    tutorial page on RNNs without recurrence, section 6.1, "core logic of
    linear attention"): with the non-negative feature map phi = ReLU,

        S_t = S_{t-1} + phi(k_t)^T v_t,    z_t = z_{t-1} + phi(k_t),
        o_t = phi(q_t) S_t / (phi(q_t) . z_t + eps),

    eps = 1e-6 added to the denominator as in the page's demonstration
    module (section 6.2); the page fixes no decay, so the state is a plain
    running sum. Every head runs the recurrence on its own.

    q, k: [B, T, H, dk]; v: [B, T, H, dv] (fp32 values or bf16 bits as
    uint16); s0: [B, H, dk, dv] and z0: [B, H, dk] or None (zeros): the
    sums carried in from earlier tokens. Returns (o [B, T, H, dv],
    s_final [B, H, dk, dv], z_final [B, H, dk]), all fp64."""
    q = widen(q).astype(np.float64)
    k = widen(k).astype(np.float64)
    v = widen(v).astype(np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != (B, T, H):
        raise ValueError("shape mismatch")
    S = np.zeros((B, H, dk, dv)) if s0 is None else np.array(s0, np.float64).reshape(B, H, dk, dv)
    z = np.zeros((B, H, dk)) if z0 is None else np.array(z0, np.float64).reshape(B, H, dk)
    fq = np.maximum(q, 0.0)
    fk = np.maximum(k, 0.0)
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        S += fk[:, t, :, :, None] * v[:, t, :, None, :]
        z += fk[:, t]
        num = np.einsum("bhd,bhde->bhe", fq[:, t], S)
        den = np.einsum("bhd,bhd->bh", fq[:, t], z) + eps
        o[:, t] = num / den[:, :, None]
    return o, S, z


GATES = ("sigmoid", "silu")


def gate_activation(g, act):
    """The output gate's activation in fp64, from its definition:
    sigmoid(z) = 1 / (1 + e^-z) and SiLU(z) = z / (1 + e^-z). g: fp32 values
    or bf16 bits (uint16)."""
    z = widen(g).astype(np.float64)
    with np.errstate(over="ignore"):
        e = np.exp(-z)  # e^-z overflows to inf for very negative z: act -> 0
    if act == "sigmoid":
        return 1.0 / (1.0 + e)
    if act == "silu":
        return z / (1.0 + e)
    raise ValueError("act must be one of %s" % (GATES,))


def output_gate(o, g, act):
    """The mixer output gated elementwise by its gate vector (Laplace 3B /
    Trainium2 page, section "QKVG projection": the fused projection yields
    g beside q, k and v, and g is applied after the mixer; the page gives no
    activation, so the caller names one): y = o * act(g), in fp64.
    o: fp64 (or fp32) array; g: the same shape (fp32 or bf16 bits)."""
    return np.asarray(o, np.float64) * gate_activation(g, act)


def gla_fwd_gated(q, k, v, g, decay, act, scale=1.0, s0=None, threads=None):
    """The chunked forward's result with the output gate applied:
    (o * act(g) [B, T, H, dv], s_final) in fp64; the state is the ungated
    recurrence's."""
    o, sf = gla_fwd(q, k, v, decay, scale, s0, threads=threads)
    return output_gate(o, g, act), sf


def gla_varlen_gated(cu_seqlens, q, k, v, g, decay, act, scale=1.0, s0=None, threads=None):
    o, sf = gla_varlen(cu_seqlens, q, k, v, decay, scale, s0, threads=threads)
    return output_gate(o, g, act), sf


def gla_decode_gated(q, k, v, g, decay, act, state, scale=1.0, threads=None):
    """One gated decode step: state updated in place as by gla_decode;
    returns o * act(g) [N, H, dv] fp64."""
    return output_gate(gla_decode(q, k, v, decay, state, scale, threads), g, act)
