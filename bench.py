#!/usr/bin/env python3
"""Benchmark of the Simple GLA hot path on one MI355X.

A step is one call of the chunked forward on the Laplace-shaped prefill
workload (B=8, T=2048, H=16, dk=96, dv=192, bf16, C=64, geometric decays):
16,384 tokens through all 16 heads of one layer, inputs resident in HBM.
The headline `value` is tokens per second over exactly `--steps` timed
steps. Four input/output buffer sets are rotated so that no step finds its
inputs in the 256 MB last-level cache.

The same JSON line also carries:
  roofline      the dominant kernel (the MFMA chunk kernel; HBM-bound):
                algorithmic bytes per launch / mean launch duration from one
                HIP event pair on the launch stream around the timed steps;
  cpu_baseline  the fp64 oracle timed on this host's cores on a bounded
                sample of the same workload;
  secondary     long_context (B1 T65536), batched_decode (1,280 sequences,
                100 consecutive steps) and varlen (32 packed sequences),
                each with its own throughput and HBM roofline.

The GPU reaches its steady clocks only after a while under load, so every
timed region follows the W warm-up steps (400 by default for the headline)
and, if those took less, untimed steps up to at least 0.5 s of work.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       [--no-secondary] [--only {prefill,long,decode,decode_pool,varlen,backward,
                                 long_backward,short_conv,linear_attn,sweep,cpu}]
       [--sweep-part {forward,decode,backward}]
(--only sweep: the shape sweep, one JSON line per case; --only cpu: the
oracle's CPU baseline alone.)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GLA fwd tokens/s (H16,dk96,dv192) + decode seq-steps/s; % MFMA / HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MIN_WARM_S = 0.5               # untimed work before every timed region, at least
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
H, DK, DV = 16, 96, 192
# algorithmic bytes per token (all heads): q, k, v read once, o written once, bf16
PREFILL_BYTES_PER_TOKEN = H * (DK + DK + DV + DV) * 2
STATE_BYTES = H * DK * DV * 4  # one sequence's fp32 state, all heads
# chunked-form flops per token at C = 64 (causal triangle counted once)
PREFILL_FLOPS_PER_TOKEN = H * (65 * (DK + DV) + 4 * DK * DV)
# decode bytes per seq-step: state read + write, bf16 q, k, v in and o out
DECODE_BYTES_PER_SEQSTEP = 2 * STATE_BYTES + H * (DK + DK + DV) * 2 + H * DV * 2
DECODE_FLOPS_PER_SEQSTEP = H * DK * DV * 5


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed(fn, steps, warmup):
    """Run fn(i) for warmup + steps iterations; time exactly `steps` between
    two device synchronisations, with one HIP event pair on the current
    stream (the stream the library launches on) around the same region.
    Returns (wall_s, event_ms_per_step). Events around every call would put
    two marker packets between consecutive kernels and slow the stream down,
    so the per-launch duration is the event span over the steps (it includes
    the few-microsecond gaps between back-to-back launches)."""
    import torch
    for i in range(warmup):
        fn(i)
    # The W warm-up steps can be as short as a few tens of milliseconds; a GPU
    # coming out of idle (e.g. after the process's own start-up) has been seen
    # to need longer to reach its steady clocks, so keep warming (untimed)
    # until at least MIN_WARM_S of the workload has run.
    torch.cuda.synchronize()
    t_w = time.perf_counter()
    n = 0
    while time.perf_counter() - t_w < MIN_WARM_S:
        for j in range(8):
            fn(warmup + n + j)
        n += 8
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        fn(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, e0.elapsed_time(e1) / steps


def roofline(bytes_per_launch, launch_ms, bound="hbm"):
    ach = bytes_per_launch / (launch_ms * 1e-3) / 1e9
    return {"bound": bound, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}


# ---------------------------------------------------------------------------
def bench_prefill(steps, warmup):
    import torch
    from chunked_gated_recurrent_amd import gla
    from chunked_gated_recurrent_amd import workloads as W
    spec = W.WORKLOADS["laplace_prefill"]
    B, T = spec["B"], spec["T"]
    lam = W.decays_for(spec)
    x = W.spec_inputs("laplace_prefill")
    dev = torch.device("cuda")
    sets = []
    for r in range(4):  # rotate buffer sets past the last-level cache
        q, k, v = (W.as_torch(x[n], dev) for n in ("q", "k", "v"))
        if r:
            q, k, v = q.clone(), k.clone(), v.clone()
        o = torch.empty(B, T, H, DV, dtype=torch.bfloat16, device=dev)
        sf = torch.empty(B, H, DK, DV, dtype=torch.float32, device=dev)
        sets.append((q, k, v, o, sf))
    ws = gla.lib().gla_chunk_fwd_workspace_bytes(1, B, T, H, DK, DV, 64)
    assert ws == 0, "the headline shape runs as one kernel without scratch"

    def step(i):
        q, k, v, o, sf = sets[i % 4]
        gla.gla_chunk_fwd(q, k, v, lam, chunk=64, out=o, final_state=sf)

    wall, ev_ms = timed(step, steps, warmup)
    tokens = B * T
    bytes_call = tokens * PREFILL_BYTES_PER_TOKEN + B * STATE_BYTES
    flops_call = tokens * PREFILL_FLOPS_PER_TOKEN
    res = dict(value=tokens * steps / wall, ms_per_step=wall / steps * 1e3,
               event_ms=ev_ms, bytes=bytes_call, flops=flops_call, x=x, lam=lam)
    res["roofline"] = roofline(bytes_call, ev_ms)
    res["mfma_frac"] = flops_call / (ev_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS
    return res


def bench_long(steps, warmup):
    import torch
    from chunked_gated_recurrent_amd import gla
    from chunked_gated_recurrent_amd import workloads as W
    spec = W.WORKLOADS["long_context"]
    B, T = spec["B"], spec["T"]
    lam = W.decays_for(spec)
    dev = torch.device("cuda")
    sets = []
    for r in range(2):
        q, k, v, s0 = W.device_normal_inputs(spec["seed"] + 100 * r, (B, T), H, DK, DV, dev,
                                             (B, H, DK, DV), spec["s0_sigma"])
        o = torch.empty(B, T, H, DV, dtype=torch.bfloat16, device=dev)
        sf = torch.empty(B, H, DK, DV, dtype=torch.float32, device=dev)
        sets.append((q, k, v, s0, o, sf))
    need = gla.lib().gla_chunk_fwd_workspace_bytes(1, B, T, H, DK, DV, 64)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def step(i):
        q, k, v, s0, o, sf = sets[i % 2]
        gla.gla_chunk_fwd(q, k, v, lam, initial_state=s0, chunk=64, out=o,
                          final_state=sf, workspace=ws)

    wall, ev_ms = timed(step, steps, warmup)
    tokens = B * T
    bytes_call = tokens * PREFILL_BYTES_PER_TOKEN + 2 * B * STATE_BYTES
    return {"workload": "long_context", "config": {"B": B, "T": T, "chunk": 64},
            "value": round(tokens * steps / wall, 1), "unit": "tokens/s",
            "ms_per_call": round(wall / steps * 1e3, 4),
            "roofline": dict(roofline(bytes_call, ev_ms),
                             kernel="whole call (state pass + combine + outputs)",
                             traffic=measured_traffic("whole call@long_context")),
            "mfma_frac": round(tokens * PREFILL_FLOPS_PER_TOKEN / (ev_ms * 1e-3) / 1e12
                               / BF16_PEAK_TFLOPS, 4),
            "workspace_bytes": need}


def bench_decode(warmup_runs=1):
    import torch
    from chunked_gated_recurrent_amd import gla
    from chunked_gated_recurrent_amd import workloads as W
    spec = W.WORKLOADS["batched_decode"]
    N, steps = spec["N"], spec["steps"]
    lam = W.decays_for(spec)
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(spec["seed"])
    state = torch.randn(N, H, DK, DV, generator=g, device=dev).mul_(spec["state_sigma"])
    q, k, v, _ = W.device_normal_inputs(spec["seed"] + 1, (steps, N), H, DK, DV, dev)
    o = torch.empty(N, H, DV, dtype=torch.bfloat16, device=dev)

    def step(i):
        t = i % steps
        gla.gla_decode_step(q[t], k[t], v[t], lam, state, out=o)

    wall, ev_ms = timed(step, steps, warmup_runs * steps)
    return {"workload": "batched_decode", "config": {"N": N, "steps": steps},
            "value": round(N * steps / wall, 1), "unit": "seq-steps/s",
            "ms_per_step": round(wall / steps * 1e3, 4),
            "roofline": dict(roofline(N * DECODE_BYTES_PER_SEQSTEP, ev_ms),
                             kernel="decode_kernel<bf16,16>",
                             traffic=measured_traffic("decode_kernel<bf16,16>@batched_decode")),
            "tokens_per_s_all_heads": round(N * steps / wall, 1)}


def bench_decode_pool(warmup_runs=1, pool_pages=2048):
    """Decode against a pool of per-sequence state pages: the 1,280
    sequences of the decode workload live in a scattered subset of 2,048
    pages (a seeded permutation), 100 steps."""
    import numpy as np
    import torch
    from chunked_gated_recurrent_amd import gla
    from chunked_gated_recurrent_amd import workloads as W
    spec = W.WORKLOADS["batched_decode"]
    N, steps = spec["N"], spec["steps"]
    lam = W.decays_for(spec)
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(spec["seed"])
    pool = torch.randn(pool_pages, H, DK, DV, generator=g, device=dev).mul_(spec["state_sigma"])
    slots = torch.from_numpy(np.random.default_rng(spec["seed"]).permutation(pool_pages)[:N]
                             .astype(np.int32)).to(dev)
    q, k, v, _ = W.device_normal_inputs(spec["seed"] + 1, (steps, N), H, DK, DV, dev)
    o = torch.empty(N, H, DV, dtype=torch.bfloat16, device=dev)

    def step(i):
        t = i % steps
        gla.gla_decode_step_pool(q[t], k[t], v[t], lam, pool, slots, out=o)

    wall, ev_ms = timed(step, steps, warmup_runs * steps)
    return {"workload": "batched_decode_pool", "config": {"N": N, "pool_pages": pool_pages,
                                                          "steps": steps},
            "value": round(N * steps / wall, 1), "unit": "seq-steps/s",
            "ms_per_step": round(wall / steps * 1e3, 4),
            "roofline": dict(roofline(N * DECODE_BYTES_PER_SEQSTEP, ev_ms),
                             kernel="decode_kernel<bf16,16> (slot table)",
                             traffic=measured_traffic(
                                 "decode_kernel<bf16,16> (slot table)@batched_decode_pool"))}


BACKWARD_BYTES_PER_TOKEN = 16 * (96 + 96 + 192 + 192) * 2 + 16 * (96 + 96 + 192) * 2


def bench_backward(steps, warmup, workload="laplace_prefill"):
    """Backward of a prefill workload (default the Laplace-shaped B8 T2048
    H16 96/192): dq, dk, dv and dS0 from dO and dS_final, zero initial state."""
    import torch
    from chunked_gated_recurrent_amd import gla
    from chunked_gated_recurrent_amd import workloads as W
    spec = W.WORKLOADS[workload]
    B, T = spec["B"], spec["T"]
    lam = W.decays_for(spec)
    dev = torch.device("cuda")
    sets = []
    for r in range(2):
        q, k, v, _ = W.device_normal_inputs(spec["seed"] + 50 + r, (B, T), H, DK, DV, dev)
        g = torch.Generator(device=dev)
        g.manual_seed(spec["seed"] + 60 + r)
        do = torch.randn(B, T, H, DV, generator=g, device=dev).to(torch.bfloat16)
        dsf = torch.randn(B, H, DK, DV, generator=g, device=dev)
        outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                torch.empty(B, H, DK, DV, dtype=torch.float32, device=dev))
        sets.append((q, k, v, do, dsf, outs))
    need = gla.lib().gla_chunk_bwd_workspace_bytes(1, B, T, H, DK, DV, 64)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def step(i):
        q, k, v, do, dsf, (dq, dk, dv, ds0) = sets[i % 2]
        gla.gla_chunk_bwd(q, k, v, lam, do, 1.0, None, dsf, chunk=64, dq=dq, dk=dk,
                          dv=dv, ds0=ds0, workspace=ws)

    wall, ev_ms = timed(step, steps, warmup)
    tokens = B * T
    bytes_call = tokens * BACKWARD_BYTES_PER_TOKEN + 2 * B * STATE_BYTES
    name = "laplace_backward" if workload == "laplace_prefill" else workload + "_backward"
    # no scratch: whole sequences, both walks in one launch; else time segments
    if need == 0:
        key = label = "bwd_fused_wide_kernel"
        label += " (dq walk and reverse walk in one launch)"
    else:
        key = "whole call"
        label = "whole call (segment boundaries + scans + dq pass + dk/dv pass)"
    return {"workload": name, "config": {"B": B, "T": T, "chunk": 64},
            "value": round(tokens * steps / wall, 1), "unit": "tokens/s",
            "ms_per_call": round(wall / steps * 1e3, 4),
            "roofline": dict(roofline(bytes_call, ev_ms), kernel=label,
                             traffic=measured_traffic(key + "@" + name)),
            "workspace_bytes": need}


def bench_short_conv(steps, warmup):
    """Short causal convolution + SiLU on the residual stream of the
    Laplace-shaped batch (B8 T2048 D3072 bf16) and one decode step for 1,280
    sequences."""
    import torch
    from chunked_gated_recurrent_amd import gla
    dev = torch.device("cuda")
    B, T, D, N = 8, 2048, 3072, 1280
    g = torch.Generator(device=dev)
    g.manual_seed(9)
    xs = [torch.randn(B, T, D, generator=g, device=dev).to(torch.bfloat16) for _ in range(2)]
    w = torch.randn(D, 4, generator=g, device=dev) * 0.5
    bias = torch.randn(D, generator=g, device=dev) * 0.1
    y = torch.empty_like(xs[0])
    wo = torch.empty(B, 4, D, dtype=torch.float32, device=dev)
    wall, ev_ms = timed(lambda i: gla.short_conv_fwd(xs[i % 2], w, bias, None, out=y,
                                                     window_out=wo), steps, warmup)
    bytes_pre = B * T * D * 2 * 2 + B * 4 * D * 4
    xd = torch.randn(N, D, generator=g, device=dev).to(torch.bfloat16)
    win = torch.randn(N, 4, D, generator=g, device=dev)
    yd = torch.empty_like(xd)
    wall_d, ev_d = timed(lambda i: gla.short_conv_decode_step(xd, w, bias, win, out=yd),
                         steps, warmup)
    bytes_dec = N * D * (2 * 2 + 3 * 4 + 4 * 4)
    return {"workload": "short_conv", "config": {"B": B, "T": T, "D": D, "decode_N": N},
            "value": round(B * T * steps / wall, 1), "unit": "tokens/s",
            "ms_per_call": round(wall / steps * 1e3, 4),
            "roofline": dict(roofline(bytes_pre, ev_ms), kernel="short_conv_fwd_kernel<bf16>",
                             traffic=measured_traffic("short_conv_fwd_kernel<bf16>@short_conv")),
            "decode": {"value": round(N * steps / wall_d, 1), "unit": "seq-steps/s",
                       "ms_per_step": round(wall_d / steps * 1e3, 4),
                       "roofline": dict(roofline(bytes_dec, ev_d),
                                        kernel="short_conv_decode_kernel<bf16>",
                                        traffic=measured_traffic(
                                            "short_conv_decode_kernel<bf16>@short_conv"))}}


def bench_linear_attn(steps, warmup):
    """Normalised causal linear attention (ReLU features, no decay) on the
    prefill batch shape B8 T2048 H16 dk96 dv192 bf16, final sums S and z
    written."""
    import torch
    from chunked_gated_recurrent_amd import gla
    dev = torch.device("cuda")
    B, T = 8, 2048
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    sets = []
    for r in range(4):  # rotate buffer sets past the last-level cache
        q, k = (torch.randn(B, T, H, DK, generator=g, device=dev).to(torch.bfloat16)
                for _ in range(2))
        v = torch.randn(B, T, H, DV, generator=g, device=dev).to(torch.bfloat16)
        o = torch.empty(B, T, H, DV, dtype=torch.bfloat16, device=dev)
        sf = torch.empty(B, H, DK, DV, dtype=torch.float32, device=dev)
        zf = torch.empty(B, H, DK, dtype=torch.float32, device=dev)
        sets.append((q, k, v, o, sf, zf))
    assert gla.lib().gla_linear_attn_fwd_workspace_bytes(1, B, T, H, DK, DV, 64) == 0

    def step(i):
        q, k, v, o, sf, zf = sets[i % 4]
        gla.linear_attn_fwd(q, k, v, chunk=64, out=o, final_state=sf, final_z=zf)

    wall, ev_ms = timed(step, steps, warmup)
    bytes_call = B * T * PREFILL_BYTES_PER_TOKEN + B * (STATE_BYTES + H * DK * 4)
    del sets
    # one decode step for 1,280 sequences from running sums (S, z), in place
    N = 1280
    st = torch.randn(N, H, DK, DV, generator=g, device=dev) * 0.3
    zs = torch.rand(N, H, DK, generator=g, device=dev) * 10.0
    qd, kd = (torch.randn(N, H, DK, generator=g, device=dev).to(torch.bfloat16)
              for _ in range(2))
    vd = torch.randn(N, H, DV, generator=g, device=dev).to(torch.bfloat16)
    od = torch.empty(N, H, DV, dtype=torch.bfloat16, device=dev)
    dsteps = max(10, steps // 10)
    wall_d, ev_d = timed(lambda i: gla.linear_attn_decode_step(qd, kd, vd, st, zs, out=od),
                         dsteps, max(3, warmup // 10))
    bytes_dec = N * (DECODE_BYTES_PER_SEQSTEP + 2 * H * DK * 4)
    return {"workload": "linear_attention", "config": {"B": B, "T": T, "H": H, "dk": DK,
                                                       "dv": DV, "decode_N": N},
            "value": round(B * T * steps / wall, 1), "unit": "tokens/s",
            "ms_per_call": round(wall / steps * 1e3, 4),
            "roofline": dict(roofline(bytes_call, ev_ms), kernel="fwd_out_kernel<96, true, 96>",
                             traffic=measured_traffic("fwd_out_kernel<96, true, 96>@linear_attention")),
            "decode": {"value": round(N * dsteps / wall_d, 1), "unit": "seq-steps/s",
                       "ms_per_step": round(wall_d / dsteps * 1e3, 4),
                       "roofline": dict(roofline(bytes_dec, ev_d),
                                        kernel="decode_kernel<bf16,16,true>",
                                        traffic=measured_traffic(
                                            "decode_kernel<bf16,16,true>@linear_attention"))}}


def bench_varlen(steps, warmup):
    import torch
    from chunked_gated_recurrent_amd import gla
    from chunked_gated_recurrent_amd import workloads as W
    spec = W.WORKLOADS["varlen"]
    lam = W.decays_for(spec)
    lens = W.varlen_lengths(spec["seed"], spec["N"], spec["max_len"])
    import numpy as np
    cu_np = np.zeros(len(lens) + 1, np.int32)
    cu_np[1:] = np.cumsum(lens)
    total = int(cu_np[-1])
    N = len(lens)
    dev = torch.device("cuda")
    q, k, v, s0 = W.device_normal_inputs(spec["seed"], (total,), H, DK, DV, dev,
                                         (N, H, DK, DV), spec["s0_sigma"])
    cu = torch.from_numpy(cu_np).to(dev)
    o = torch.empty(total, H, DV, dtype=torch.bfloat16, device=dev)
    sf = torch.empty(N, H, DK, DV, dtype=torch.float32, device=dev)
    need = gla.lib().gla_chunk_fwd_varlen_workspace_bytes(1, N, total, H, DK, DV, 64)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def step(i):
        gla.gla_chunk_fwd_varlen(q, k, v, cu, lam, initial_state=s0, chunk=64, out=o,
                                 final_state=sf, workspace=ws)

    wall, ev_ms = timed(step, steps, warmup)
    bytes_call = total * PREFILL_BYTES_PER_TOKEN + 2 * N * STATE_BYTES
    return {"workload": "varlen", "config": {"N": N, "total_tokens": total,
                                             "max_len": int(lens.max()), "chunk": 64},
            "value": round(total * steps / wall, 1), "unit": "tokens/s",
            "ms_per_call": round(wall / steps * 1e3, 4),
            "roofline": dict(roofline(bytes_call, ev_ms), kernel="whole call (order + outputs)",
                             traffic=measured_traffic("whole call@varlen")),
            "workspace_bytes": need}


# ---------------------------------------------------------------------------
# Shape sweep (--only sweep): the same calls across head shapes, dtypes, head
# counts, batch sizes and sequence lengths; for each case the time per call
# and its HBM roofline fraction (algorithmic bytes per call / time / 8 TB/s;
# every call is HBM-bound at these shapes), one JSON line per case. Inputs
# are seeded synthetic draws on the device (q, k, v ~ N(0, 1), q and k
# scaled by dk^-1/2, geometric decays); two or more input sets are rotated so
# that small cases do not run out of the last-level cache, and every timed
# region follows at least SWEEP_WARM_S of untimed calls.
SWEEP_WARM_S = 0.3


def _sweep_elt(dtype):
    return 2 if dtype == "bf16" else 4


def _sweep_time(fn, n_sets, min_calls=20):
    import torch
    i = 0
    torch.cuda.synchronize()
    t = time.perf_counter()
    while time.perf_counter() - t < SWEEP_WARM_S or i < 3:
        fn(i % n_sets)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    per = (time.perf_counter() - t) / i
    calls = max(min_calls, int(0.5 / max(per, 1e-6)))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for j in range(calls):
        fn(j % n_sets)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / calls * 1e3  # microseconds


def _sweep_inputs(lead, H, dk, dv, dtype, seed):
    import torch
    from chunked_gated_recurrent_amd import workloads as W
    dev = torch.device("cuda")
    q, k, v, _ = W.device_normal_inputs(seed, lead, H, dk, dv, dev)
    if dtype == "f32":
        q, k, v = q.float(), k.float(), v.float()
    return q, k, v


def _sweep_sets(nbytes):
    """Input sets to rotate: enough to exceed the 256 MB last-level cache."""
    return max(2, min(8, int(1.2e9 // max(nbytes, 1)) + 1))


def _sweep_line(call, dtype, shape, us, nbytes, **extra):
    gbs = nbytes / (us * 1e-6) / 1e9
    d = {"call": call, "dtype": dtype}
    d.update(shape)
    d.update({"us": round(us, 1), "GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 3)})
    d.update(extra)
    print(json.dumps(d), flush=True)


def sweep_forward():
    import torch
    from chunked_gated_recurrent_amd import gla
    from chunked_gated_recurrent_amd import workloads as W
    cases = [  # dtype, B, T, H, dk, dv
        ("bf16", 8, 2048, 16, 96, 192), ("bf16", 1, 2048, 16, 96, 192),
        ("bf16", 8, 512, 16, 96, 192), ("bf16", 32, 2048, 16, 96, 192),
        ("bf16", 8, 8192, 16, 96, 192), ("bf16", 1, 65536, 16, 96, 192),
        ("bf16", 8, 2048, 8, 96, 192), ("bf16", 8, 2048, 32, 96, 192),
        ("bf16", 8, 2048, 16, 96, 64), ("bf16", 8, 2048, 16, 96, 128),
        ("bf16", 8, 2048, 16, 96, 256),
        ("bf16", 8, 2048, 16, 64, 128), ("bf16", 8, 2048, 16, 128, 128),
        ("f32", 8, 2048, 16, 96, 192),
    ]
    for dtype, B, T, H, dk, dv in cases:
        lam = W.geometric_decays(H)
        e = _sweep_elt(dtype)
        nbytes = B * T * H * (2 * dk + 2 * dv) * e + B * H * dk * dv * 4
        sets = []
        for r in range(_sweep_sets(nbytes)):
            q, k, v = _sweep_inputs((B, T), H, dk, dv, dtype, 40 + r)
            o = torch.empty(B, T, H, dv, dtype=q.dtype, device=q.device)
            sf = torch.empty(B, H, dk, dv, device=q.device)
            sets.append((q, k, v, o, sf))
        need = gla.lib().gla_chunk_fwd_workspace_bytes(1 if dtype == "bf16" else 0, B, T, H,
                                                       dk, dv, 0)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=sets[0][0].device)

        def call(i):
            q, k, v, o, sf = sets[i]
            gla.gla_chunk_fwd(q, k, v, lam, out=o, final_state=sf, workspace=ws)

        us = _sweep_time(call, len(sets))
        _sweep_line("gla_chunk_fwd", dtype, dict(B=B, T=T, H=H, dk=dk, dv=dv), us, nbytes,
              tokens_per_s=round(B * T / (us * 1e-6), 1), workspace_bytes=need)
        del sets, ws
        torch.cuda.empty_cache()


def sweep_decode():
    import torch
    from chunked_gated_recurrent_amd import gla
    from chunked_gated_recurrent_amd import workloads as W
    cases = [("bf16", 1280, 16, 96, 192), ("bf16", 64, 16, 96, 192),
             ("bf16", 1280, 16, 96, 128), ("bf16", 1280, 16, 64, 128),
             ("f32", 1280, 16, 96, 192)]
    for dtype, N, H, dk, dv in cases:
        lam = W.geometric_decays(H)
        e = _sweep_elt(dtype)
        nbytes = N * H * (2 * dk * dv * 4 + (2 * dk + 2 * dv) * e)
        n_sets = _sweep_sets(nbytes)
        dev = torch.device("cuda")
        states = [torch.randn(N, H, dk, dv, device=dev) * 0.3 for _ in range(n_sets)]
        q, k, v = _sweep_inputs((n_sets, N), H, dk, dv, dtype, 60)
        o = torch.empty(N, H, dv, dtype=q.dtype, device=dev)

        def call(i):
            gla.gla_decode_step(q[i], k[i], v[i], lam, states[i], out=o)

        us = _sweep_time(call, n_sets)
        _sweep_line("gla_decode_step", dtype, dict(N=N, H=H, dk=dk, dv=dv), us, nbytes,
              seq_steps_per_s=round(N / (us * 1e-6), 1))
        del states
        torch.cuda.empty_cache()


def sweep_backward():
    import torch
    from chunked_gated_recurrent_amd import gla
    from chunked_gated_recurrent_amd import workloads as W
    cases = [("bf16", 8, 2048, 16, 96, 192), ("bf16", 32, 2048, 16, 96, 192),
             ("bf16", 8, 2048, 16, 96, 128), ("bf16", 8, 2048, 16, 96, 256),
             ("bf16", 8, 2048, 16, 64, 128), ("bf16", 8, 2048, 16, 128, 128),
             ("bf16", 8, 2048, 16, 128, 256), ("f32", 8, 2048, 16, 96, 192)]
    for dtype, B, T, H, dk, dv in cases:
        lam = W.geometric_decays(H)
        e = _sweep_elt(dtype)
        nbytes = B * T * H * (4 * dk + 3 * dv) * e + 2 * B * H * dk * dv * 4
        sets = []
        gen = torch.Generator(device="cuda")
        gen.manual_seed(70)
        for r in range(_sweep_sets(nbytes)):
            q, k, v = _sweep_inputs((B, T), H, dk, dv, dtype, 80 + r)
            do = torch.randn(B, T, H, dv, generator=gen, device=q.device).to(q.dtype)
            dsf = torch.randn(B, H, dk, dv, generator=gen, device=q.device)
            outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                    torch.empty(B, H, dk, dv, device=q.device))
            sets.append((q, k, v, do, dsf, outs))
        need = gla.lib().gla_chunk_bwd_workspace_bytes(1 if dtype == "bf16" else 0, B, T, H,
                                                       dk, dv, 0)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=sets[0][0].device)

        def call(i):
            q, k, v, do, dsf, (dq, dk_, dv_, ds0) = sets[i]
            gla.gla_chunk_bwd(q, k, v, lam, do, 1.0, None, dsf, dq=dq, dk=dk_, dv=dv_, ds0=ds0,
                              workspace=ws)

        us = _sweep_time(call, len(sets))
        _sweep_line("gla_chunk_bwd", dtype, dict(B=B, T=T, H=H, dk=dk, dv=dv), us, nbytes,
              tokens_per_s=round(B * T / (us * 1e-6), 1), workspace_bytes=need)
        del sets, ws
        torch.cuda.empty_cache()



def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(x, lam, budget_s=8.0, decode_budget_s=4.0):
    """The fp64 oracle on this host's cores, untuned, parallel only across
    independent (sequence, head) chains:
      * the headline: the whole Laplace-shaped prefill workload (8 x 2,048
        tokens x 16 heads), repeated for about `budget_s` seconds;
      * decode: steps of the batched-decode recipe (fp32 states N(0, 0.1),
        fresh bf16 tokens per step) on the first 160 of its 1,280 sequences
        (all 16 heads), for about `decode_budget_s` seconds;
      * one pass over the long-context workload (1 x 65,536 tokens) and one
        over the packed 32-sequence workload.
    `threads` is what the oracle ran with: OMP_NUM_THREADS when set, else
    the visible cores capped at 16, the CPU share a job on one GPU gets on
    these hosts; `host_cores` is what the operating system reports."""
    import numpy as np
    from chunked_gated_recurrent_amd import workloads as W
    from oracle import oracle as O
    threads = O.default_threads()
    host_cores = os.cpu_count()
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = host_cores
    B, T = x["q"].shape[0], x["q"].shape[1]
    t0 = time.perf_counter()
    calls = 0
    while True:
        O.gla_fwd(x["q"], x["k"], x["v"], lam, threads=threads)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    out = {"value": round(calls * B * T / el, 1), "unit": "tokens/s", "cores": threads,
           "threads": threads, "host_cores": host_cores, "usable_cores": usable,
           "kind": "oracle", "cpu_model": _cpu_model(),
           "sample": "%d passes over the laplace_prefill workload (B=%d, T=%d, 16 heads), "
                     "fp64 token-by-token recurrence, %.1f s wall" % (calls, B, T, el)}
    # decode: the batched-decode recipe on a bounded subset of its sequences
    spec = W.WORKLOADS["batched_decode"]
    Nd = 160
    # the first Nd sequences of the recipe's state draw (numpy fills the array
    # in order, so a draw of Nd sequences is that prefix)
    state = W.decode_state(spec["seed"], Nd, spec["H"], spec["dk"], spec["dv"],
                           spec["state_sigma"]).astype(np.float64)
    lam_d = W.decays_for(spec)
    steps = 0
    el = 0.0
    while el < decode_budget_s and steps < spec["steps"]:
        q, k, v = W.decode_tokens(spec["seed"], steps, spec["N"], spec["H"], spec["dk"],
                                  spec["dv"])
        q, k, v = q[:Nd].copy(), k[:Nd].copy(), v[:Nd].copy()
        t1 = time.perf_counter()
        O.gla_decode(q, k, v, lam_d, state, threads=threads)
        el += time.perf_counter() - t1
        steps += 1
    out["decode"] = {"value": round(Nd * steps / el, 1), "unit": "seq-steps/s",
                     "sample": "%d consecutive steps of the batched_decode recipe on %d of "
                               "its 1280 sequences (16 heads each), fp64 state in place, "
                               "%.1f s of oracle time" % (steps, Nd, el)}
    del state
    # one pass each over the long-context and the packed workloads
    for name in ("long_context", "varlen"):
        xs = W.spec_inputs(name)
        t1 = time.perf_counter()
        if name == "varlen":
            O.gla_varlen(xs["cu_seqlens"], xs["q"], xs["k"], xs["v"], xs["decay"], 1.0,
                         xs["s0"], threads=threads)
            tokens = int(xs["cu_seqlens"][-1])
        else:
            O.gla_fwd(xs["q"], xs["k"], xs["v"], xs["decay"], 1.0, xs["s0"], threads=threads)
            tokens = xs["q"].shape[0] * xs["q"].shape[1]
        el = time.perf_counter() - t1
        out[name] = {"value": round(tokens / el, 1), "unit": "tokens/s",
                     "sample": "one pass over the whole %s workload (%d tokens, 16 heads), "
                               "%.1f s wall" % (name, tokens, el)}
        del xs
    return out


def copy_bandwidth(gib=1.0):
    """Achievable HBM bandwidth of a plain device copy (read + write), for
    context beside the datasheet peak."""
    import torch
    n = int(gib * (1 << 30)) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    return round(2 * n * 4 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)


def mfma_achievable(n=8192):
    """Achievable dense bf16 matrix-core rate of a plain library GEMM
    (n x n x n, fp32 accumulate), TFLOP/s, for context beside the datasheet
    peak."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    a = torch.randn(n, n, generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, generator=g, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    del c
    return round(2.0 * n ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)


def measured_traffic(key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken with the current kernel source (else None)."""
    f = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        from chunked_gated_recurrent_amd.profiling import source_sha256
        with open(f) as fh:
            rec = json.load(fh).get(key)
        if rec and rec.get("source_sha256") == source_sha256(rec.get("source_files")):
            return int(rec["traffic_bytes"])
    except (OSError, ValueError, KeyError):
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--only", choices=["prefill", "long", "decode", "decode_pool", "varlen",
                                       "backward", "long_backward", "short_conv",
                                       "linear_attn", "sweep", "cpu"])
    ap.add_argument("--sweep-part", choices=["forward", "decode", "backward"],
                    help="with --only sweep: one part of the shape sweep")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    if args.only == "cpu":  # the oracle alone: no GPU needed
        from chunked_gated_recurrent_amd import workloads as W
        x = W.spec_inputs("laplace_prefill")
        print(json.dumps(cpu_baseline(x, x["decay"])))
        return
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from chunked_gated_recurrent_amd import gla
    gla.lib()

    if args.only == "sweep":
        for name, fn in (("forward", sweep_forward), ("decode", sweep_decode),
                         ("backward", sweep_backward)):
            if args.sweep_part in (None, name):
                fn()
        return
    if args.only:
        fn = {"prefill": lambda: bench_prefill(args.steps, args.warmup),
              "long": lambda: bench_long(args.steps, args.warmup),
              "decode": lambda: bench_decode(),
              "decode_pool": lambda: bench_decode_pool(),
              "backward": lambda: bench_backward(args.steps, args.warmup),
              "short_conv": lambda: bench_short_conv(args.steps, args.warmup),
              "linear_attn": lambda: bench_linear_attn(args.steps, args.warmup),
              "long_backward": lambda: bench_backward(args.steps, args.warmup, "long_context"),
              "varlen": lambda: bench_varlen(args.steps, args.warmup)}[args.only]
        r = fn()
        r.pop("x", None)
        r.pop("lam", None)
        print(json.dumps(r, default=float))
        return

    log("prefill: laplace_prefill B8 T2048 ...")
    pre = bench_prefill(args.steps, args.warmup)
    secondary = {}
    if not args.no_secondary:
        log("long_context ...")
        secondary["long_context"] = bench_long(max(10, args.steps // 10), max(3, args.warmup // 10))
        log("batched_decode ...")
        secondary["batched_decode"] = bench_decode()
        log("batched_decode_pool ...")
        secondary["batched_decode_pool"] = bench_decode_pool()
        log("laplace_backward ...")
        secondary["laplace_backward"] = bench_backward(max(10, args.steps // 10),
                                                       max(3, args.warmup // 10))
        log("short_conv ...")
        secondary["short_conv"] = bench_short_conv(max(10, args.steps // 10),
                                                   max(3, args.warmup // 10))
        log("linear_attention ...")
        secondary["linear_attention"] = bench_linear_attn(max(10, args.steps // 10),
                                                          max(3, args.warmup // 10))
        log("varlen ...")
        secondary["varlen"] = bench_varlen(max(10, args.steps // 10), max(3, args.warmup // 10))
    copy_bw = copy_bandwidth()
    mfma_tf = mfma_achievable()
    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(pre["x"], pre["lam"])
    line = {
        "metric": METRIC,
        "value": round(pre["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "laplace_prefill", "B": 8, "T": 2048, "H": H, "dk": DK,
                   "dv": DV, "chunk": 64, "decays": "geometric, memory 32..4096 tokens",
                   "initial_state": "zero", "buffer_sets": 4},
        "roofline": dict(pre["roofline"], kernel="fwd_out_kernel<96, false, 96>",
                         traffic=measured_traffic("fwd_out_kernel<96, false, 96>@laplace_prefill"),
                         bytes_per_launch=pre["bytes"], launch_ms=round(pre["event_ms"], 5)),
        "hbm_copy_GBps": copy_bw,
        "hbm_frac_of_copy": round(pre["roofline"]["achieved"] / copy_bw, 4) if copy_bw else None,
        "mfma_frac": round(pre["mfma_frac"], 4),
        "mfma_bf16_gemm_TFLOPs": mfma_tf,
        "mfma_frac_of_gemm": round(pre["mfma_frac"] * BF16_PEAK_TFLOPS / mfma_tf, 4),
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
