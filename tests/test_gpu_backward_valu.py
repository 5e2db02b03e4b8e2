"""GPU parity of the vector-ALU backward (fp32 inputs, head sizes off the
matrix-core path, 32-token chunks requested explicitly) against the fp64
oracle's backward. Bar per output (dq, dk, dv, dS0): max|gpu - oracle| <=
1e-4 * max|oracle| for fp32 inputs, 1e-2 for bf16."""
import numpy as np
import pytest
import torch

from chunked_gated_recurrent_amd import gla
from chunked_gated_recurrent_amd import workloads as W
from oracle import oracle as O
from gla_testutil import TOL, dev, host, rel_err

pytestmark = pytest.mark.gpu


def _case(seed, B, T, H, dk, dv, dtype, with_s0=True, with_dsf=True):
    x = W.prefill_inputs(seed, B, T, H, dk, dv, dtype, 0.1 if with_s0 else None,
                         W.geometric_decays(H))
    rng = np.random.default_rng(seed + 1000)
    do = rng.standard_normal((B, T, H, dv), dtype=np.float32)
    if dtype == "bf16":
        do = W.bf16_bits(do)
    dsf = (rng.standard_normal((B, H, dk, dv), dtype=np.float32) * np.float32(0.5)
           if with_dsf else None)
    return x, do, dsf


def _check(name, dtype, got, ref):
    names = ("dq", "dk", "dv", "dS0")
    errs = [rel_err(g, r) for g, r in zip(got, ref)]
    print("%s: " % name + "  ".join("%s %.2e" % (n, e) for n, e in zip(names, errs)))
    for n, g, e in zip(names, got, errs):
        assert np.isfinite(g).all(), n
        assert e <= TOL[dtype], (name, n, e)


def _run(x, do, dsf, chunk=0, scale=1.0):
    q, k, v, s0 = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["s0"])
    out = gla.gla_chunk_bwd(q, k, v, x["decay"], dev(do), scale, s0, dev(dsf), chunk=chunk)
    torch.cuda.synchronize()
    return tuple(host(t) for t in out)


def _oracle(x, do, dsf, scale=1.0):
    return O.gla_bwd(x["q"], x["k"], x["v"], x["decay"], do, scale, x["s0"], dsf)


@pytest.mark.parametrize("dtype,dk,dv,T,chunk", [
    ("f32", 32, 64, 130, 0), ("f32", 16, 32, 70, 32), ("f32", 128, 256, 70, 0),
    ("f32", 96, 192, 100, 0), ("f32", 32, 48, 95, 0), ("f32", 48, 80, 33, 0),
    ("bf16", 64, 80, 100, 0), ("bf16", 96, 192, 100, 32)])
def test_valu_backward_shapes(dtype, dk, dv, T, chunk):
    x, do, dsf = _case(1100 + dk + dv + T, 2, T, 2, dk, dv, dtype)
    _check("valu bwd %s dk%d dv%d T%d C%d" % (dtype, dk, dv, T, chunk), dtype,
           _run(x, do, dsf, chunk), _oracle(x, do, dsf))


def test_valu_backward_defaults_and_scale():
    x, do, dsf = _case(1150, 2, 77, 3, 32, 32, "f32", with_s0=False, with_dsf=False)
    _check("valu bwd no s0/dsf, scale 0.3", "f32", _run(x, do, dsf, scale=0.3),
           _oracle(x, do, dsf, 0.3))


def test_valu_backward_time_segments():
    """One sequence, two heads of 32 x 32: cut into time segments (forward
    state pass + combine, carry pass + reverse combine)."""
    x, do, dsf = _case(1160, 1, 3000, 2, 32, 32, "f32")
    need = gla.lib().gla_chunk_bwd_workspace_bytes(0, 1, 3000, 2, 32, 32, 0)
    plain = 2 * 1 * 2 * 3000 * 32 * 4  # partials of one dv tile, dq and dk
    assert need > plain
    _check("valu bwd segments T3000", "f32", _run(x, do, dsf), _oracle(x, do, dsf))


@pytest.mark.parametrize("lengths", [[5, 0, 130, 1, 64, 65, 300], [2500, 3]])
def test_valu_backward_varlen(lengths):
    H, dk, dv = 2, 32, 64
    x = W.varlen_inputs(1170 + len(lengths), len(lengths), 0, H, dk, dv, "f32", 0.1,
                        W.geometric_decays(H), lengths=lengths)
    total = int(x["cu_seqlens"][-1])
    rng = np.random.default_rng(1171)
    do = rng.standard_normal((total, H, dv), dtype=np.float32)
    dsf = rng.standard_normal((len(lengths), H, dk, dv), dtype=np.float32)
    q, k, v, s0 = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["s0"])
    out = gla.gla_chunk_bwd_varlen(q, k, v, dev(x["cu_seqlens"]), x["decay"], dev(do), 1.0,
                                   s0, dev(dsf))
    torch.cuda.synchronize()
    got = tuple(host(t) for t in out)
    ref = O.gla_bwd_varlen(x["cu_seqlens"], x["q"], x["k"], x["v"], x["decay"], do, 1.0,
                           x["s0"], dsf)
    _check("valu bwd varlen %s" % lengths, "f32", got, ref)
    for n, L in enumerate(lengths):
        if L == 0:
            np.testing.assert_array_equal(got[3][n], dsf[n].astype(np.float64))
