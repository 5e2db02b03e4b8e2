"""GPU parity of the normalised causal linear attention (ReLU features, no
decay, eps = 1e-6 in the denominator) against the fp64 oracle on seeded
inputs: the matrix-core path (bf16, dk = 96, dv tiles of 96 and 64), the
vector-ALU path (the tutorial page's single-head d_k = 32 shape in fp32,
bf16 dk = 64), time segments, carried sums, and the degenerate cases.

Bar: max|gpu - oracle| <= 1e-2 * max|oracle| for bf16 inputs, 1e-4 for fp32,
on the output and on the final sums S and z."""
import numpy as np
import pytest
import torch

from chunked_gated_recurrent_amd import gla
from chunked_gated_recurrent_amd import workloads as W
from oracle import oracle as O
from gla_testutil import TOL, dev, host, rel_err

pytestmark = pytest.mark.gpu


def _case(seed, B, T, H, dk, dv, dtype):
    rng = np.random.default_rng(seed)
    xs = [rng.standard_normal((B, T, H, d), dtype=np.float32) for d in (dk, dk, dv)]
    if dtype == "bf16":
        xs = [W.bf16_bits(x) for x in xs]
    return xs


def _run(q, k, v, s0=None, z0=None, chunk=0):
    o, sf, zf = gla.linear_attn_fwd(dev(q), dev(k), dev(v), dev(s0), dev(z0), chunk=chunk)
    torch.cuda.synchronize()
    return host(o), host(sf), host(zf)


def _check(dtype, got, ref, what):
    errs = [rel_err(g, r) for g, r in zip(got, ref)]
    print("%s: o %.2e  S %.2e  z %.2e" % ((what,) + tuple(errs)))
    assert max(errs) <= TOL[dtype], errs


@pytest.mark.parametrize("dv", [192, 128, 256])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200, 321])
def test_matrix_core_path(T, dv):
    q, k, v = _case(900 + T + dv, 2, T, 3, 96, dv, "bf16")
    _check("bf16", _run(q, k, v), O.linear_attention(q, k, v), "mfma T%d dv%d" % (T, dv))


@pytest.mark.parametrize("dtype,dk,dv,chunk", [("f32", 32, 32, 0), ("f32", 32, 32, 32),
                                               ("bf16", 64, 64, 0), ("f32", 96, 48, 0)])
def test_vector_alu_path(dtype, dk, dv, chunk):
    """The page's demonstration shape (one head, d_k = 32 for q, k and v) and
    other head sizes off the matrix-core path."""
    q, k, v = _case(950 + dk + dv + chunk, 2, 150, 1 if dk == 32 else 2, dk, dv, dtype)
    _check(dtype, _run(q, k, v, chunk=chunk), O.linear_attention(q, k, v),
           "valu %s dk%d dv%d C%d" % (dtype, dk, dv, chunk))


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 96, 192), ("f32", 32, 32)])
def test_carried_sums_continue_the_sequence(dtype, dk, dv):
    """First 100 tokens, then the remaining 133 from the returned (S, z):
    equal to the oracle over all 233 tokens."""
    q, k, v = _case(970 + dk, 2, 233, 2, dk, dv, dtype)
    o1, s1, z1 = gla.linear_attn_fwd(dev(q[:, :100]), dev(k[:, :100]), dev(v[:, :100]))
    o2, s2, z2 = gla.linear_attn_fwd(dev(q[:, 100:]), dev(k[:, 100:]), dev(v[:, 100:]), s1, z1)
    torch.cuda.synchronize()
    ro, rs, rz = O.linear_attention(q, k, v)
    got = (np.concatenate([host(o1), host(o2)], axis=1), host(s2), host(z2))
    _check(dtype, got, (ro, rs, rz), "carried %s" % dtype)


@pytest.mark.parametrize("dtype,dk,dv,T", [("bf16", 96, 192, 4000), ("f32", 32, 32, 1500)])
def test_time_segments(dtype, dk, dv, T):
    """One batch entry, few heads: the sequence is cut into time segments
    whose local sums (S and z) are combined before the outputs."""
    assert gla.lib().gla_linear_attn_fwd_workspace_bytes(
        1 if dtype == "bf16" else 0, 1, T, 2, dk, dv, 0) > 0
    q, k, v = _case(990 + T, 1, T, 2, dk, dv, dtype)
    _, s0, z0 = O.linear_attention(*_case(992, 1, 50, 2, dk, dv, dtype))
    got = _run(q, k, v, s0.astype(np.float32), z0.astype(np.float32))
    ref = O.linear_attention(q, k, v, s0.astype(np.float32), z0.astype(np.float32))
    _check(dtype, got, ref, "segments %s T%d" % (dtype, T))


def test_laplace_shape_full():
    """B8 T2048 H16 dk96 dv192 bf16 (the prefill batch shape): every head of
    every batch entry against the oracle."""
    B, T, H = 8, 2048, 16
    q, k, v = _case(1000, B, T, H, 96, 192, "bf16")
    o, sf, zf = _run(q, k, v)
    _check("bf16", (o, sf, zf), O.linear_attention(q, k, v), "laplace B8 T2048 all heads")


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 96, 192), ("f32", 32, 32)])
def test_degenerate_features(dtype, dk, dv):
    """phi(q) = 0 everywhere gives o = 0 exactly; phi(k) = 0 everywhere gives
    S = z = 0 and o = 0 (the denominator is eps alone)."""
    q, k, v = _case(1010, 2, 70, 2, dk, dv, dtype)
    neg = (lambda x: x | np.uint16(0x8000)) if dtype == "bf16" else (lambda x: -np.abs(x))
    o, sf, zf = _run(neg(q), k, v)
    assert np.all(o == 0.0)
    o, sf, zf = _run(q, neg(k), v)
    assert np.all(o == 0.0) and np.all(sf == 0.0) and np.all(zf == 0.0)


def test_empty_sequence_copies_the_sums():
    B, H, dk, dv = 2, 3, 96, 192
    rng = np.random.default_rng(1020)
    s0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    z0 = np.abs(rng.standard_normal((B, H, dk))).astype(np.float32)
    e = torch.empty((B, 0, H, dk), dtype=torch.bfloat16, device="cuda")
    ev = torch.empty((B, 0, H, dv), dtype=torch.bfloat16, device="cuda")
    o, sf, zf = gla.linear_attn_fwd(e, e, ev, dev(s0), dev(z0))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(sf), s0)
    np.testing.assert_array_equal(host(zf), z0)
    o, sf, zf = gla.linear_attn_fwd(e, e, ev)
    torch.cuda.synchronize()
    assert np.all(host(sf) == 0.0) and np.all(host(zf) == 0.0)


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 96, 192), ("f32", 32, 32), ("bf16", 64, 128),
                                         ("bf16", 128, 64)])
def test_decode_steps_continue_the_prefill(dtype, dk, dv):
    """Prefill 37 tokens, then 5 decode steps from the returned (S, z): equal
    to the oracle over all 42 tokens, outputs and final sums."""
    B, T0, T, H = 3, 37, 42, 2
    q, k, v = _case(1030 + dk, B, T, H, dk, dv, dtype)
    o, sf, zf = gla.linear_attn_fwd(dev(q[:, :T0]), dev(k[:, :T0]), dev(v[:, :T0]))
    outs = [host(o)]
    for t in range(T0, T):
        ot = gla.linear_attn_decode_step(dev(np.ascontiguousarray(q[:, t])),
                                         dev(np.ascontiguousarray(k[:, t])),
                                         dev(np.ascontiguousarray(v[:, t])), sf, zf)
        outs.append(host(ot)[:, None])
    torch.cuda.synchronize()
    ro, rs, rz = O.linear_attention(q, k, v)
    _check(dtype, (np.concatenate(outs, axis=1), host(sf), host(zf)), (ro, rs, rz),
           "decode after prefill %s dk%d" % (dtype, dk))


def test_causality_and_determinism():
    """Changing tokens after position 100 leaves outputs 0..100 bitwise
    unchanged; two identical calls agree bitwise (no atomics feed an
    output)."""
    q, k, v = _case(1040, 2, 200, 3, 96, 192, "bf16")
    a = _run(q, k, v)
    b = _run(q, k, v)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    rng = np.random.default_rng(1041)
    for arr in (q2, k2, v2):
        arr[:, 101:] = W.bf16_bits(rng.standard_normal(arr[:, 101:].shape, dtype=np.float32))
    c = _run(q2, k2, v2)
    np.testing.assert_array_equal(c[0][:, :101], a[0][:, :101])
    assert not np.array_equal(c[0][:, 101:], a[0][:, 101:])


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 96, 192), ("f32", 32, 32)])
@pytest.mark.parametrize("lengths", [[5, 0, 130, 1, 64, 65, 300], [3000, 1, 700]])
def test_packed_sequences(dtype, dk, dv, lengths):
    """Packed sequences (empty, one-token, chunk-aligned, ragged; a few long
    ones cut into time segments by the device planner), each from its own
    carried sums: every sequence equals the oracle run on it alone."""
    H = 2
    N = len(lengths)
    cu = np.zeros(N + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    total = int(cu[-1])
    q, k, v = (x[0] for x in _case(1050 + total, 1, total, H, dk, dv, dtype))
    rng = np.random.default_rng(1051)
    s0 = (rng.standard_normal((N, H, dk, dv)) * 0.3).astype(np.float32)
    z0 = np.abs(rng.standard_normal((N, H, dk))).astype(np.float32)
    o, sf, zf = gla.linear_attn_fwd_varlen(dev(q), dev(k), dev(v), dev(cu), dev(s0), dev(z0))
    torch.cuda.synchronize()
    o, sf, zf = host(o), host(sf), host(zf)
    worst = [0.0, 0.0, 0.0]
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        ro, rs, rz = O.linear_attention(q[None, a:b], k[None, a:b], v[None, a:b],
                                        s0[n:n + 1], z0[n:n + 1])
        if b > a:
            worst[0] = max(worst[0], rel_err(o[a:b], ro[0]))
        worst[1] = max(worst[1], rel_err(sf[n], rs[0]))
        worst[2] = max(worst[2], rel_err(zf[n], rz[0]))
        if b == a:
            np.testing.assert_array_equal(sf[n], s0[n])
            np.testing.assert_array_equal(zf[n], z0[n])
    print("packed %s %s: o %.2e  S %.2e  z %.2e" % ((dtype, lengths) + tuple(worst)))
    assert max(worst) <= TOL[dtype], worst


def test_max_heads():
    q, k, v = _case(1060, 1, 90, 64, 96, 192, "bf16")
    _check("bf16", _run(q, k, v), O.linear_attention(q, k, v), "H64")


def test_packed_all_empty_copies_the_sums():
    N, H, dk, dv = 3, 2, 96, 192
    rng = np.random.default_rng(1070)
    s0 = rng.standard_normal((N, H, dk, dv)).astype(np.float32)
    z0 = np.abs(rng.standard_normal((N, H, dk))).astype(np.float32)
    e = torch.empty((0, H, dk), dtype=torch.bfloat16, device="cuda")
    ev = torch.empty((0, H, dv), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    o, sf, zf = gla.linear_attn_fwd_varlen(e, e, ev, cu, dev(s0), dev(z0))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(sf), s0)
    np.testing.assert_array_equal(host(zf), z0)
