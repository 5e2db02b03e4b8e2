"""Seeded synthetic inputs for Simple GLA, shared by the tests, the smoke check
and the benchmark. This module only draws numbers and rounds them to the
storage dtype; it holds none of the recurrence's arithmetic.

Shapes follow the Laplace 3B / Trainium2 page ("Beyond the KV cache"): H = 16
heads with dk = 96 and dv = 192 (section "QKVG projection"), prefill length
2,048 = 16 chunks x 128 tokens (section "Challenge 1"), and 1,280 concurrent
decode sequences (section "Inference optimisation on Trainium2"). The page's
datasets and weights are not used; normal draws stand in for activations.

Recipe (all draws fp32 from numpy's PCG64 ``default_rng``):
  * q, k, v ~ N(0, 1); q and k are multiplied by dk**-0.5 in fp32; bf16
    workloads then round each value once to bf16, round-to-nearest-even.
  * initial states are fp32 N(0, sigma^2) with the sigma of the workload.
  * variable-length workloads draw their lengths first.
  * decode draws its state from rng([seed, 0]) and the tokens of step s from
    rng([seed, s + 1]), so any step can be regenerated on its own.
Per-head decays are fixed numbers, not draws: computed in fp64 and rounded
once to fp32, and both the GPU and the oracle receive those fp32 values.
"""
from __future__ import annotations

import numpy as np

DK_LAPLACE, DV_LAPLACE, H_LAPLACE = 96, 192, 16


# ----------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------
def bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even); returns the uint16
    bit patterns. NaN stays NaN (quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    one = np.uint32(1)
    # finite values cannot overflow 32 bits here (largest: 0xFF7FFFFF + 0x8000)
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & one))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# per-head decays
# ----------------------------------------------------------------------------
def geometric_decays(H: int = H_LAPLACE) -> np.ndarray:
    """lambda_h = 1 - 2**-(5 + 7h/(H-1)): memory lengths 1/(1-lambda) spaced
    geometrically from 32 to 4,096 tokens across the heads (the page fixes
    the decays at initialisation, geometric across heads; its formula image
    is lost, so this schedule is a stated reading)."""
    h = np.arange(H, dtype=np.float64)
    span = max(H - 1, 1)
    return (1.0 - 2.0 ** -(5.0 + 7.0 * h / span)).astype(np.float32)


def tiny_decays(H: int = 2) -> np.ndarray:
    """lambda_h = 1 - 2**-(3+h): 0.875, 0.9375, ... for the tiny check."""
    h = np.arange(H, dtype=np.float64)
    return (1.0 - 2.0 ** -(3.0 + h)).astype(np.float32)


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
WORKLOADS = {
    # tiny fp32 check that the oracle finishes instantly
    "tiny_fp32": dict(kind="prefill", seed=1, B=1, T=256, H=2, dk=16, dv=32,
                      dtype="f32", s0_sigma=None, chunk=32, decays="tiny"),
    # one Laplace-shaped layer of prefill
    "laplace_prefill": dict(kind="prefill", seed=2, B=8, T=2048, H=16, dk=96,
                            dv=192, dtype="bf16", s0_sigma=None, chunk=64,
                            decays="geometric"),
    # one 65,536-token sequence from a random initial state
    "long_context": dict(kind="prefill", seed=3, B=1, T=65536, H=16, dk=96,
                         dv=192, dtype="bf16", s0_sigma=0.1, chunk=64,
                         decays="geometric"),
    # 1,280 sequences, one token each per step, 100 steps
    "batched_decode": dict(kind="decode", seed=4, N=1280, H=16, dk=96, dv=192,
                           steps=100, state_sigma=float(np.sqrt(0.1)),
                           decays="geometric"),
    # 32 packed sequences with lengths uniform in [1, 8192]
    "varlen": dict(kind="varlen", seed=5, N=32, max_len=8192, H=16, dk=96,
                   dv=192, dtype="bf16", s0_sigma=0.1, chunk=64,
                   decays="geometric"),
}


def decays_for(spec: dict) -> np.ndarray:
    return tiny_decays(spec["H"]) if spec["decays"] == "tiny" else geometric_decays(spec["H"])


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def _qkv(rng, lead, H, dk, dv, dtype, prescale=True):
    sc = np.float32(1.0 / np.sqrt(dk)) if prescale else np.float32(1.0)
    q = rng.standard_normal(lead + (H, dk), dtype=np.float32) * sc
    k = rng.standard_normal(lead + (H, dk), dtype=np.float32) * sc
    v = rng.standard_normal(lead + (H, dv), dtype=np.float32)
    return _store(q, dtype), _store(k, dtype), _store(v, dtype)


def prefill_inputs(seed: int, B: int, T: int, H: int, dk: int, dv: int,
                   dtype: str = "bf16", s0_sigma=None, decays=None,
                   prescale: bool = True) -> dict:
    """q, k: [B, T, H, dk]; v: [B, T, H, dv] (uint16 bf16 bits or fp32);
    s0: [B, H, dk, dv] fp32 or None; decay: [H] fp32. prescale=False leaves
    q and k at N(0, 1) (for a caller that passes dk**-0.5 as the scale)."""
    rng = np.random.default_rng(seed)
    q, k, v = _qkv(rng, (B, T), H, dk, dv, dtype, prescale)
    s0 = None
    if s0_sigma is not None:
        s0 = rng.standard_normal((B, H, dk, dv), dtype=np.float32) * np.float32(s0_sigma)
    lam = geometric_decays(H) if decays is None else np.asarray(decays, np.float32)
    return dict(q=q, k=k, v=v, s0=s0, decay=lam, dtype=dtype)


def varlen_lengths(seed: int, N: int, max_len: int) -> np.ndarray:
    return np.random.default_rng(seed).integers(1, max_len + 1, size=N)


def varlen_inputs(seed: int, N: int, max_len: int, H: int, dk: int, dv: int,
                  dtype: str = "bf16", s0_sigma=0.1, decays=None,
                  lengths=None, prescale: bool = True) -> dict:
    """Lengths are drawn first (uniform integers in [1, max_len]) unless
    given; q, k: [total, H, dk]; v: [total, H, dv]; cu_seqlens: [N+1] int32;
    s0: [N, H, dk, dv] fp32 or None."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = rng.integers(1, max_len + 1, size=N)
    lengths = np.asarray(lengths, dtype=np.int64)
    N = lengths.shape[0]
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    total = int(cu[-1])
    q, k, v = _qkv(rng, (total,), H, dk, dv, dtype, prescale)
    s0 = None
    if s0_sigma is not None:
        s0 = rng.standard_normal((N, H, dk, dv), dtype=np.float32) * np.float32(s0_sigma)
    lam = geometric_decays(H) if decays is None else np.asarray(decays, np.float32)
    return dict(q=q, k=k, v=v, s0=s0, cu_seqlens=cu, lengths=lengths,
                decay=lam, dtype=dtype)


def decode_state(seed: int, N: int, H: int, dk: int, dv: int,
                 sigma: float) -> np.ndarray:
    rng = np.random.default_rng([seed, 0])
    return rng.standard_normal((N, H, dk, dv), dtype=np.float32) * np.float32(sigma)


def decode_tokens(seed: int, step: int, N: int, H: int, dk: int, dv: int,
                  dtype: str = "bf16", prescale: bool = True):
    """q, k: [N, H, dk]; v: [N, H, dv] for decode step `step`."""
    rng = np.random.default_rng([seed, step + 1])
    return _qkv(rng, (N,), H, dk, dv, dtype, prescale)


def spec_inputs(name: str, **overrides) -> dict:
    """Inputs of a named workload (prefill / varlen kinds)."""
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    lam = decays_for(spec)
    if spec["kind"] == "prefill":
        return prefill_inputs(spec["seed"], spec["B"], spec["T"], spec["H"],
                              spec["dk"], spec["dv"], spec["dtype"],
                              spec["s0_sigma"], lam)
    if spec["kind"] == "varlen":
        return varlen_inputs(spec["seed"], spec["N"], spec["max_len"], spec["H"],
                             spec["dk"], spec["dv"], spec["dtype"],
                             spec["s0_sigma"], lam)
    raise ValueError("decode workloads use decode_state / decode_tokens")


# ----------------------------------------------------------------------------
# torch plumbing (device memory only)
# ----------------------------------------------------------------------------
def as_torch(x, device="cuda"):
    """numpy -> torch on `device`: uint16 arrays become bfloat16 tensors with
    the same bits, float32 stays float32, int32 stays int32."""
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(x)
    return t.to(device)


def to_numpy_bits(t) -> np.ndarray:
    """torch tensor -> numpy; bfloat16 comes back as uint16 bit patterns."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def device_normal_inputs(seed: int, lead, H: int, dk: int, dv: int, device,
                         s0_shape=None, s0_sigma=None):
    """The same recipe drawn on the device with torch's seeded generator
    (for timing runs of large workloads, where host generation would dominate
    the wall clock): bf16 q, k, v ~ N(0,1) with q, k scaled by dk**-0.5 in
    fp32 before rounding; optional fp32 initial state N(0, sigma^2)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    sc = 1.0 / float(np.sqrt(dk))
    lead = tuple(lead)

    def draw(shape, s):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if s != 1.0:
            x.mul_(s)
        return x

    q = draw(lead + (H, dk), sc).to(torch.bfloat16)
    k = draw(lead + (H, dk), sc).to(torch.bfloat16)
    v = draw(lead + (H, dv), 1.0).to(torch.bfloat16)
    s0 = None
    if s0_shape is not None:
        s0 = draw(tuple(s0_shape), float(s0_sigma))
    return q, k, v, s0
