"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph on
ROCm). Every entry point only launches kernels on the caller's stream: it
allocates nothing, never synchronises and records no memset (fills are
kernels), so a serving or training loop can capture it once and replay it.
Each test captures a sequence of calls, then replays the graph several times
with eager work and synchronisations in between, and checks every replay bit
for bit against the same calls made eagerly (the kernels are deterministic)."""
import pytest
import torch

from chunked_gated_recurrent_amd import gla
from chunked_gated_recurrent_amd import workloads as W

pytestmark = pytest.mark.gpu

DK, DV = 96, 192


def _capture_and_replay(run, outputs, replays=3):
    """run() issues the calls; outputs are the tensors they write."""
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(replays):
        for t in outputs:          # eager work between replays
            t.fill_(float("nan") if t.is_floating_point() else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, (t, r) in enumerate(zip(outputs, ref)):
            assert torch.equal(t, r), ("replay", rep, "output", n)


def test_graph_prefill_then_decode_steps():
    """Fixed-batch prefill (one kernel), then four decode steps on its final
    state and two pooled decode steps."""
    dev = torch.device("cuda")
    B, T, H, P = 2, 300, 4, 5
    lam = W.geometric_decays(H)
    q, k, v, s0 = W.device_normal_inputs(1500, (B, T), H, DK, DV, dev, (B, H, DK, DV), 0.1)
    qd, kd, vd, _ = W.device_normal_inputs(1501, (4, B), H, DK, DV, dev)
    pool0 = torch.randn(P, H, DK, DV, device=dev) * 0.3
    slots = torch.tensor([3, 0], dtype=torch.int32, device=dev)
    o = torch.empty(B, T, H, DV, dtype=torch.bfloat16, device=dev)
    S = torch.empty(B, H, DK, DV, device=dev)
    od = torch.empty(4, B, H, DV, dtype=torch.bfloat16, device=dev)
    pool = torch.empty_like(pool0)
    op = torch.empty(2, B, H, DV, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(gla.lib().gla_chunk_fwd_workspace_bytes(1, B, T, H, DK, DV, 0), 1),
                     dtype=torch.uint8, device=dev)

    def run():
        pool.copy_(pool0)
        gla.gla_chunk_fwd(q, k, v, lam, initial_state=s0, out=o, final_state=S, workspace=ws)
        for t in range(4):
            gla.gla_decode_step(qd[t], kd[t], vd[t], lam, S, out=od[t])
        for t in range(2):
            gla.gla_decode_step_pool(qd[t], kd[t], vd[t], lam, pool, slots, out=op[t])

    _capture_and_replay(run, [o, S, od, pool, op])


def test_graph_long_sequence_forward_and_backward():
    """One 4,096-token sequence: time segments (state pass, combine, output
    pass) and the segmented backward (boundary pass, scans, dq and dk/dv)."""
    dev = torch.device("cuda")
    B, T, H = 1, 4096, 4
    lam = W.geometric_decays(H)
    q, k, v, s0 = W.device_normal_inputs(1510, (B, T), H, DK, DV, dev, (B, H, DK, DV), 0.1)
    g = torch.Generator(device=dev)
    g.manual_seed(1511)
    do = torch.randn(B, T, H, DV, generator=g, device=dev).to(torch.bfloat16)
    dsf = torch.randn(B, H, DK, DV, generator=g, device=dev)
    L = gla.lib()
    wf = torch.empty(max(L.gla_chunk_fwd_workspace_bytes(1, B, T, H, DK, DV, 0), 1),
                     dtype=torch.uint8, device=dev)
    wb = torch.empty(max(L.gla_chunk_bwd_workspace_bytes(1, B, T, H, DK, DV, 0), 1),
                     dtype=torch.uint8, device=dev)
    assert wf.numel() > 1 and wb.numel() > 1, "expected the segmented paths"
    o = torch.empty(B, T, H, DV, dtype=torch.bfloat16, device=dev)
    S = torch.empty(B, H, DK, DV, device=dev)
    dq, dk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ds0 = torch.empty(B, H, DK, DV, device=dev)

    def run():
        gla.gla_chunk_fwd(q, k, v, lam, initial_state=s0, out=o, final_state=S, workspace=wf)
        gla.gla_chunk_bwd(q, k, v, lam, do, 1.0, s0, dsf, dq=dq, dk=dk, dv=dvv, ds0=ds0,
                          workspace=wb)

    _capture_and_replay(run, [o, S, dq, dk, dvv, ds0])


@pytest.mark.parametrize("dk,dv", [(96, 128), (128, 128), (64, 192)])
def test_graph_other_head_shapes(dk, dv):
    """Time segments at other head shapes: the forward's state pass (d_k 128
    scales k in registers), the backward's boundary pass and the per-head
    backward kernels."""
    dev = torch.device("cuda")
    B, T, H = 1, 3000, 4
    lam = W.geometric_decays(H)
    q, k, v, s0 = W.device_normal_inputs(1530 + dk, (B, T), H, dk, dv, dev, (B, H, dk, dv), 0.1)
    g = torch.Generator(device=dev)
    g.manual_seed(1531)
    do = torch.randn(B, T, H, dv, generator=g, device=dev).to(torch.bfloat16)
    dsf = torch.randn(B, H, dk, dv, generator=g, device=dev)
    L = gla.lib()
    wf = torch.empty(max(L.gla_chunk_fwd_workspace_bytes(1, B, T, H, dk, dv, 0), 1),
                     dtype=torch.uint8, device=dev)
    wb = torch.empty(max(L.gla_chunk_bwd_workspace_bytes(1, B, T, H, dk, dv, 0), 1),
                     dtype=torch.uint8, device=dev)
    assert wf.numel() > 1 and wb.numel() > 1, "expected the segmented paths"
    o = torch.empty(B, T, H, dv, dtype=torch.bfloat16, device=dev)
    S = torch.empty(B, H, dk, dv, device=dev)
    dq, dk_, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ds0 = torch.empty(B, H, dk, dv, device=dev)

    def run():
        gla.gla_chunk_fwd(q, k, v, lam, initial_state=s0, out=o, final_state=S, workspace=wf)
        gla.gla_chunk_bwd(q, k, v, lam, do, 1.0, s0, dsf, dq=dq, dk=dk_, dv=dvv, ds0=ds0,
                          workspace=wb)

    _capture_and_replay(run, [o, S, dq, dk_, dvv, ds0])


def test_graph_packed_sequences():
    """Packed input with device-side planning (order kernel) and its
    backward, plus the short convolution's prefill and decode step."""
    dev = torch.device("cuda")
    H = 4
    lengths = [700, 3, 129, 0, 64, 2000]
    x = W.varlen_inputs(1520, len(lengths), 0, H, DK, DV, "bf16", 0.1, W.geometric_decays(H),
                        lengths=lengths)
    q, k, v = (W.as_torch(x[n], dev) for n in ("q", "k", "v"))
    s0 = W.as_torch(x["s0"], dev)
    cu = W.as_torch(x["cu_seqlens"], dev)
    lam = x["decay"]
    total, N = q.shape[0], len(lengths)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1521)
    do = torch.randn(total, H, DV, generator=gen, device=dev).to(torch.bfloat16)
    L = gla.lib()
    wf = torch.empty(max(L.gla_chunk_fwd_varlen_workspace_bytes(1, N, total, H, DK, DV, 0), 1),
                     dtype=torch.uint8, device=dev)
    wb = torch.empty(max(L.gla_chunk_bwd_varlen_workspace_bytes(1, N, total, H, DK, DV, 0), 1),
                     dtype=torch.uint8, device=dev)
    o = torch.empty(total, H, DV, dtype=torch.bfloat16, device=dev)
    S = torch.empty(N, H, DK, DV, device=dev)
    dq, dk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ds0 = torch.empty(N, H, DK, DV, device=dev)
    D = 3072
    xc = torch.randn(2, 40, D, generator=gen, device=dev).to(torch.bfloat16)
    xt = torch.randn(2, D, generator=gen, device=dev).to(torch.bfloat16)
    w = torch.randn(D, 4, generator=gen, device=dev) * 0.3
    b = torch.randn(D, generator=gen, device=dev) * 0.1
    yc = torch.empty_like(xc)
    win = torch.empty(2, 4, D, device=dev)
    yt = torch.empty_like(xt)

    def run():
        gla.gla_chunk_fwd_varlen(q, k, v, cu, lam, initial_state=s0, out=o, final_state=S,
                                 workspace=wf)
        gla.gla_chunk_bwd_varlen(q, k, v, cu, lam, o, 1.0, s0, S, dq=dq, dk=dk, dv=dvv,
                                 ds0=ds0, workspace=wb)
        gla.short_conv_fwd(xc, w, b, out=yc, window_out=win)
        gla.short_conv_decode_step(xt, w, b, win, out=yt)

    _capture_and_replay(run, [o, S, dq, dk, dvv, ds0, yc, win, yt])
