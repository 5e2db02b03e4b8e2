"""GPU parity of the output gate (y = o * act(g), act sigmoid or SiLU) on every
forward path and on decode, against the fp64 oracle's gated results on the
same seeded inputs. Bars as everywhere: max|gpu - oracle| <= 1e-2 *
max|oracle| for bf16 inputs, 1e-4 for fp32 inputs, on outputs and states
(the state must be the ungated recurrence's)."""
import numpy as np
import pytest
import torch

from chunked_gated_recurrent_amd import gla
from chunked_gated_recurrent_amd import workloads as W
from oracle import oracle as O
from gla_testutil import TOL, dev, env, host, rel_err

pytestmark = pytest.mark.gpu


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


def _gate_values(seed, shape, dtype):
    """Gate pre-activations ~ N(0, 4): both saturated ends and the middle of
    the activations are exercised."""
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(2.0)
    return W.bf16_bits(x) if dtype == "bf16" else x


# (name, dtype, dk, dv, T, chunk, segmented)
CASES = [
    ("mfma dk96", "bf16", 96, 192, 200, 0, False),
    ("mfma dk96 dv64", "bf16", 96, 64, 130, 0, False),
    ("mfma dk64", "bf16", 64, 128, 130, 0, False),
    ("mfma dk128", "bf16", 128, 128, 70, 0, False),
    ("mfma segmented", "bf16", 96, 192, 1000, 0, True),
    ("valu f32", "f32", 32, 64, 150, 0, False),
    ("valu bf16 chunk32", "bf16", 96, 192, 90, 32, False),
]


@pytest.mark.parametrize("act", ["sigmoid", "silu"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gated_forward(case, act):
    name, dtype, dk, dv, T, chunk, seg = case
    x = W.prefill_inputs(400 + dk + dv + T, 2, T, 3, dk, dv, dtype, 0.1, W.geometric_decays(3))
    g = _gate_values(401 + T, (2, T, 3, dv), dtype)
    with env(**(dict(GLA_TARGET_WGS=100000) if seg else {})):
        o, sf = gla.gla_chunk_fwd_gated(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(g),
                                        x["decay"], act, scale=0.5,
                                        initial_state=dev(x["s0"]), chunk=chunk)
        torch.cuda.synchronize()
    ro, rs = O.gla_fwd_gated(x["q"], x["k"], x["v"], g, x["decay"], act, 0.5, x["s0"])
    _check("%s %s o" % (name, act), host(o), ro, TOL[dtype])
    _check("%s %s S" % (name, act), host(sf), rs, TOL[dtype])


@pytest.mark.parametrize("act", ["sigmoid", "silu"])
def test_gated_forward_laplace_shape_full(act):
    """The Laplace-shaped batch (B8 T2048 H16 96/192), every output."""
    x = W.spec_inputs("laplace_prefill")
    g = _gate_values(410, (8, 2048, 16, 192), "bf16")
    o, sf = gla.gla_chunk_fwd_gated(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(g), x["decay"],
                                    act)
    torch.cuda.synchronize()
    ro, rs = O.gla_fwd_gated(x["q"], x["k"], x["v"], g, x["decay"], act)
    _check("laplace gated %s o" % act, host(o), ro, TOL["bf16"])
    _check("laplace gated %s S" % act, host(sf), rs, TOL["bf16"])


@pytest.mark.parametrize("act", ["sigmoid", "silu"])
@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 96, 192), ("f32", 32, 64)])
def test_gated_varlen(dtype, dk, dv, act):
    x = W.varlen_inputs(420 + dk, 5, 0, 3, dk, dv, dtype, 0.1, W.geometric_decays(3),
                        lengths=[130, 0, 64, 1000, 1])
    total = int(x["cu_seqlens"][-1])
    g = _gate_values(421, (total, 3, dv), dtype)
    o, sf = gla.gla_chunk_fwd_varlen(dev(x["q"]), dev(x["k"]), dev(x["v"]),
                                     dev(x["cu_seqlens"]), x["decay"],
                                     initial_state=dev(x["s0"]), g=dev(g), gate=act)
    torch.cuda.synchronize()
    ro, rs = O.gla_varlen_gated(x["cu_seqlens"], x["q"], x["k"], x["v"], g, x["decay"], act,
                                1.0, x["s0"])
    _check("varlen %s %s o" % (dtype, act), host(o), ro, TOL[dtype])
    _check("varlen %s %s S" % (dtype, act), host(sf), rs, TOL[dtype])


@pytest.mark.parametrize("act", ["sigmoid", "silu"])
@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 96, 192), ("f32", 32, 64)])
def test_gated_decode(dtype, dk, dv, act):
    N, H = 40, 4
    lam = W.geometric_decays(H)
    S = W.decode_state(430 + dk, N, H, dk, dv, 0.3)
    ref = S.astype(np.float64)
    state = dev(S)
    for t in range(3):
        q, k, v = W.decode_tokens(431 + dk, t, N, H, dk, dv, dtype)
        g = _gate_values(432 + t, (N, H, dv), dtype)
        o = gla.gla_decode_step(dev(q), dev(k), dev(v), lam, state, g=dev(g), gate=act)
        torch.cuda.synchronize()
        ro = O.gla_decode_gated(q, k, v, g, lam, act, ref)
        _check("decode %s %s step %d" % (dtype, act, t), host(o), ro, TOL[dtype])
    _check("decode %s %s state" % (dtype, act), host(state), ref, TOL[dtype])


def test_gate_saturation():
    """A gate of +40 is the identity under sigmoid: the gated output equals
    the ungated one bit for bit (the activation rounds to 1.0 in fp32); a gate
    of -1000 zeroes every output under either activation, with no NaN."""
    x = W.prefill_inputs(440, 2, 150, 3, 96, 192, "bf16", 0.1, W.geometric_decays(3))
    q, k, v, s0 = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["s0"])
    o_plain, s_plain = gla.gla_chunk_fwd(q, k, v, x["decay"], initial_state=s0)
    hi = torch.full((2, 150, 3, 192), 40.0, device="cuda").to(torch.bfloat16)
    lo = torch.full((2, 150, 3, 192), -1000.0, device="cuda").to(torch.bfloat16)
    o_hi, s_hi = gla.gla_chunk_fwd_gated(q, k, v, hi, x["decay"], "sigmoid", initial_state=s0)
    torch.cuda.synchronize()
    assert torch.equal(o_hi, o_plain) and torch.equal(s_hi, s_plain)
    for act in ("sigmoid", "silu"):
        o_lo, _ = gla.gla_chunk_fwd_gated(q, k, v, lo, x["decay"], act, initial_state=s0)
        torch.cuda.synchronize()
        assert torch.all(o_lo.float() == 0.0), act
