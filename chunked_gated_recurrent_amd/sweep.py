"""Shape sweep of the library's calls on one GPU.

bench.py measures the benchmark shapes; this times the same calls across
head shapes, dtypes, head counts, batch sizes and sequence lengths, and
reports for each case the time per call and its HBM roofline fraction
(algorithmic bytes per call / time / 8 TB/s; every call is HBM-bound at
these shapes). One JSON line per case on stdout.

Inputs are seeded synthetic draws on the device (bf16 or fp32 q, k, v ~
N(0, 1) with q, k scaled by dk^-1/2; geometric decays); two or more input
sets are rotated so that small cases do not run out of the last-level
cache. Every timed region follows at least 0.3 s of untimed calls.

Usage: python -m chunked_gated_recurrent_amd.sweep [--only forward|decode|backward]
"""
from __future__ import annotations

import argparse
import json
import sys
import time

PEAK_GBS = 8000.0
MIN_WARM_S = 0.3


def _elt(dtype):
    return 2 if dtype == "bf16" else 4


def _time(fn, n_sets, min_calls=20):
    import torch
    i = 0
    torch.cuda.synchronize()
    t = time.perf_counter()
    while time.perf_counter() - t < MIN_WARM_S or i < 3:
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


def _inputs(lead, H, dk, dv, dtype, seed):
    import torch
    from . import workloads as W
    dev = torch.device("cuda")
    q, k, v, _ = W.device_normal_inputs(seed, lead, H, dk, dv, dev)
    if dtype == "f32":
        q, k, v = q.float(), k.float(), v.float()
    return q, k, v


def _sets(nbytes):
    """Input sets to rotate: enough to exceed the 256 MB last-level cache."""
    return max(2, min(8, int(1.2e9 // max(nbytes, 1)) + 1))


def _line(call, dtype, shape, us, nbytes, **extra):
    gbs = nbytes / (us * 1e-6) / 1e9
    d = {"call": call, "dtype": dtype}
    d.update(shape)
    d.update({"us": round(us, 1), "GBps": round(gbs, 1), "frac": round(gbs / PEAK_GBS, 3)})
    d.update(extra)
    print(json.dumps(d), flush=True)


def sweep_forward():
    import torch
    from . import gla
    from . import workloads as W
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
        e = _elt(dtype)
        nbytes = B * T * H * (2 * dk + 2 * dv) * e + B * H * dk * dv * 4
        sets = []
        for r in range(_sets(nbytes)):
            q, k, v = _inputs((B, T), H, dk, dv, dtype, 40 + r)
            o = torch.empty(B, T, H, dv, dtype=q.dtype, device=q.device)
            sf = torch.empty(B, H, dk, dv, device=q.device)
            sets.append((q, k, v, o, sf))
        need = gla.lib().gla_chunk_fwd_workspace_bytes(1 if dtype == "bf16" else 0, B, T, H,
                                                       dk, dv, 0)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=sets[0][0].device)

        def call(i):
            q, k, v, o, sf = sets[i]
            gla.gla_chunk_fwd(q, k, v, lam, out=o, final_state=sf, workspace=ws)

        us = _time(call, len(sets))
        _line("gla_chunk_fwd", dtype, dict(B=B, T=T, H=H, dk=dk, dv=dv), us, nbytes,
              tokens_per_s=round(B * T / (us * 1e-6), 1), workspace_bytes=need)
        del sets, ws
        torch.cuda.empty_cache()


def sweep_decode():
    import torch
    from . import gla
    from . import workloads as W
    cases = [("bf16", 1280, 16, 96, 192), ("bf16", 64, 16, 96, 192),
             ("bf16", 1280, 16, 96, 128), ("bf16", 1280, 16, 64, 128),
             ("f32", 1280, 16, 96, 192)]
    for dtype, N, H, dk, dv in cases:
        lam = W.geometric_decays(H)
        e = _elt(dtype)
        nbytes = N * H * (2 * dk * dv * 4 + (2 * dk + 2 * dv) * e)
        n_sets = _sets(nbytes)
        dev = torch.device("cuda")
        states = [torch.randn(N, H, dk, dv, device=dev) * 0.3 for _ in range(n_sets)]
        q, k, v = _inputs((n_sets, N), H, dk, dv, dtype, 60)
        o = torch.empty(N, H, dv, dtype=q.dtype, device=dev)

        def call(i):
            gla.gla_decode_step(q[i], k[i], v[i], lam, states[i], out=o)

        us = _time(call, n_sets)
        _line("gla_decode_step", dtype, dict(N=N, H=H, dk=dk, dv=dv), us, nbytes,
              seq_steps_per_s=round(N / (us * 1e-6), 1))
        del states
        torch.cuda.empty_cache()


def sweep_backward():
    import torch
    from . import gla
    from . import workloads as W
    cases = [("bf16", 8, 2048, 16, 96, 192), ("bf16", 32, 2048, 16, 96, 192),
             ("bf16", 8, 2048, 16, 96, 128), ("bf16", 8, 2048, 16, 96, 256),
             ("bf16", 8, 2048, 16, 64, 128), ("bf16", 8, 2048, 16, 128, 128),
             ("bf16", 8, 2048, 16, 128, 256), ("f32", 8, 2048, 16, 96, 192)]
    for dtype, B, T, H, dk, dv in cases:
        lam = W.geometric_decays(H)
        e = _elt(dtype)
        nbytes = B * T * H * (4 * dk + 3 * dv) * e + 2 * B * H * dk * dv * 4
        sets = []
        gen = torch.Generator(device="cuda")
        gen.manual_seed(70)
        for r in range(_sets(nbytes)):
            q, k, v = _inputs((B, T), H, dk, dv, dtype, 80 + r)
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

        us = _time(call, len(sets))
        _line("gla_chunk_bwd", dtype, dict(B=B, T=T, H=H, dk=dk, dv=dv), us, nbytes,
              tokens_per_s=round(B * T / (us * 1e-6), 1), workspace_bytes=need)
        del sets, ws
        torch.cuda.empty_cache()


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--only", choices=["forward", "decode", "backward"])
    args = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        sys.exit("the sweep needs a GPU")
    from . import gla
    gla.lib()  # fail loudly when the library is missing
    for name, fn in (("forward", sweep_forward), ("decode", sweep_decode),
                     ("backward", sweep_backward)):
        if args.only in (None, name):
            fn()


if __name__ == "__main__":
    main()
