"""The `scale` argument on every forward path, against the fp64 oracle called
with the same fp32 scale: 0.37 on the usual pre-scaled inputs, and
dk**-0.5 on raw N(0, 1) queries and keys (the scaling moved from the inputs
into the call). A scale that a kernel dropped, or applied twice, fails the
1e-2 / 1e-4 bars by a wide margin at either value."""
import numpy as np
import pytest
import torch

from chunked_gated_recurrent_amd import gla
from chunked_gated_recurrent_amd import workloads as W
from oracle import oracle as O
from gla_testutil import TOL, dev, env, host, rel_err

pytestmark = pytest.mark.gpu

SCALES = ["0.37", "dk^-1/2"]


def scale_for(kind, dk):
    """(fp32 scale value both sides receive, whether the inputs are pre-scaled)"""
    if kind == "0.37":
        return float(np.float32(0.37)), True
    return float(np.float32(1.0 / np.sqrt(dk))), False


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gla.lib()
    yield
    torch.cuda.synchronize()


def _check(name, got, ref, tol):
    e = rel_err(got, ref)
    print("%s: err %.3e (tol %.0e)" % (name, e, tol))
    assert np.isfinite(got).all() and e <= tol, (name, e)


# (name, dtype, dk, dv, T, chunk, segmented)
FWD_CASES = [
    ("mfma dk96", "bf16", 96, 192, 200, 0, False),
    ("mfma dk64", "bf16", 64, 128, 130, 0, False),
    ("mfma dk128", "bf16", 128, 128, 130, 0, False),
    ("mfma segmented", "bf16", 96, 192, 1000, 0, True),
    ("valu f32", "f32", 32, 64, 150, 0, False),
    ("valu bf16 chunk32", "bf16", 96, 192, 90, 32, False),
]


@pytest.mark.parametrize("kind", SCALES)
@pytest.mark.parametrize("case", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_scale(case, kind):
    name, dtype, dk, dv, T, chunk, seg = case
    scale, pre = scale_for(kind, dk)
    x = W.prefill_inputs(300 + dk + T, 2, T, 3, dk, dv, dtype, 0.1, W.geometric_decays(3),
                         prescale=pre)
    knob = dict(GLA_TARGET_WGS=100000) if seg else {}
    with env(**knob):
        if seg:
            assert gla.lib().gla_chunk_fwd_workspace_bytes(
                1, 2, T, 3, dk, dv, chunk) > 0, "time segments expected"
        o, sf = gla.gla_chunk_fwd(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["decay"],
                                  scale=scale, initial_state=dev(x["s0"]), chunk=chunk)
        torch.cuda.synchronize()
    ro, rs = O.gla_fwd(x["q"], x["k"], x["v"], x["decay"], scale, x["s0"])
    _check("%s scale %s o" % (name, kind), host(o), ro, TOL[dtype])
    _check("%s scale %s S" % (name, kind), host(sf), rs, TOL[dtype])


@pytest.mark.parametrize("kind", SCALES)
@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 96, 192), ("f32", 32, 64)])
def test_varlen_scale(dtype, dk, dv, kind):
    scale, pre = scale_for(kind, dk)
    x = W.varlen_inputs(320 + dk, 5, 300, 3, dk, dv, dtype, 0.1, W.geometric_decays(3),
                        lengths=[130, 0, 64, 257, 1], prescale=pre)
    o, sf = gla.gla_chunk_fwd_varlen(dev(x["q"]), dev(x["k"]), dev(x["v"]),
                                     dev(x["cu_seqlens"]), x["decay"], scale=scale,
                                     initial_state=dev(x["s0"]))
    torch.cuda.synchronize()
    ro, rs = O.gla_varlen(x["cu_seqlens"], x["q"], x["k"], x["v"], x["decay"], scale,
                          x["s0"])
    _check("varlen %s scale %s o" % (dtype, kind), host(o), ro, TOL[dtype])
    _check("varlen %s scale %s S" % (dtype, kind), host(sf), rs, TOL[dtype])


@pytest.mark.parametrize("kind", SCALES)
@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 96, 192), ("f32", 32, 64)])
def test_decode_scale(dtype, dk, dv, kind):
    """Three decode steps (the second and third read states the kernel
    wrote), on the unrolled 16-rows-per-thread kernel (96/192) and the
    generic one (32/64)."""
    scale, pre = scale_for(kind, dk)
    N, H = 37, 4
    lam = W.geometric_decays(H)
    S = W.decode_state(330 + dk, N, H, dk, dv, 0.3)
    ref = S.astype(np.float64)
    state = dev(S)
    for t in range(3):
        q, k, v = W.decode_tokens(331 + dk, t, N, H, dk, dv, dtype, prescale=pre)
        o = gla.gla_decode_step(dev(q), dev(k), dev(v), lam, state, scale=scale)
        torch.cuda.synchronize()
        ro = O.gla_decode(q, k, v, lam, ref, scale)
        _check("decode %s step %d scale %s" % (dtype, t, kind), host(o), ro, TOL[dtype])
    _check("decode %s state scale %s" % (dtype, kind), host(state), ref, TOL[dtype])


@pytest.mark.parametrize("kind", SCALES)
def test_decode_pool_scale(kind):
    scale, pre = scale_for(kind, 96)
    N, H, dk, dv, P = 9, 4, 96, 192, 16
    lam = W.geometric_decays(H)
    pool = W.decode_state(340, P, H, dk, dv, 0.3)
    ref = pool.astype(np.float64)
    slots = np.array([3, 15, -1, 0, 7, 16, 9, 2, 11], np.int32)  # two padding rows
    dpool = dev(pool)
    q, k, v = W.decode_tokens(341, 0, N, H, dk, dv, "bf16", prescale=pre)
    o = gla.gla_decode_step_pool(dev(q), dev(k), dev(v), lam, dpool, dev(slots), scale=scale)
    torch.cuda.synchronize()
    ro = O.gla_decode_pool(q, k, v, lam, ref, slots, scale)
    _check("pool scale %s o" % kind, host(o), ro, TOL["bf16"])
    _check("pool scale %s pages" % kind, host(dpool), ref, TOL["bf16"])
