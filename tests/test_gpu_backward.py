"""GPU parity of the backward (gla_chunk_bwd) against the fp64 oracle's
backward on the same seeded inputs and upstream gradients. Bar, per output
(dq, dk, dv, dS0): max|gpu - oracle| <= 1e-2 * max|oracle| (bf16 inputs)."""
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


def _inputs(seed, B, T, H, dv, with_s0=True, with_dsf=True, dk=96):
    x = W.prefill_inputs(seed, B, T, H, dk, dv, "bf16", 0.1 if with_s0 else None,
                         W.geometric_decays(H))
    rng = np.random.default_rng(seed + 1000)
    do = W.bf16_bits(rng.standard_normal((B, T, H, dv), dtype=np.float32))
    dsf = (rng.standard_normal((B, H, dk, dv), dtype=np.float32) * np.float32(0.5)
           if with_dsf else None)
    return x, do, dsf


def _run(x, do, dsf, scale=1.0, heads=None):
    q, k, v, s0 = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["s0"])
    dq, dk, dv, ds0 = gla.gla_chunk_bwd(q, k, v, x["decay"], dev(do), scale, s0, dev(dsf))
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv), host(ds0)


def _oracle(x, do, dsf, scale=1.0, heads=None):
    q, k, v, s0, d, lam = x["q"], x["k"], x["v"], x["s0"], do, x["decay"]
    f = dsf
    if heads is not None:
        q, k, v, d = q[:, :, heads], k[:, :, heads], v[:, :, heads], d[:, :, heads]
        s0 = None if s0 is None else s0[:, heads]
        f = None if f is None else f[:, heads]
        lam = lam[heads]
    return O.gla_bwd(q, k, v, lam, d, scale, s0, f)


def _check(name, got, ref):
    names = ("dq", "dk", "dv", "dS0")
    errs = [rel_err(g, r) for g, r in zip(got, ref)]
    print("%s: " % name + "  ".join("%s %.2e" % (n, e) for n, e in zip(names, errs)))
    for n, g, e in zip(names, got, errs):
        assert np.isfinite(g).all(), n
        assert e <= TOL["bf16"], (name, n, e)


@pytest.mark.parametrize("T", [1, 17, 64, 65, 130, 200])
@pytest.mark.parametrize("dv", [192, 128, 64])
def test_backward_ragged_lengths(T, dv):
    x, do, dsf = _inputs(700 + T, 2, T, 3, dv)
    _check("bwd T%d dv%d" % (T, dv), _run(x, do, dsf), _oracle(x, do, dsf))


def test_backward_widest_value_head():
    """dv = 256, the widest head: four dv tiles of 64 columns, four
    partial sums per dq and dk element."""
    x, do, dsf = _inputs(705, 2, 150, 2, 256)
    _check("bwd dv256", _run(x, do, dsf), _oracle(x, do, dsf))


@pytest.mark.parametrize("dv", [192, 128, 64])
def test_backward_two_segments_joined_on_load(dv):
    """8 x 8 units of 256 tokens: two time segments per sequence, whose
    local states and carries the wide kernels (one workgroup over all of
    d_v) join with S0 and dL/dS_final as they load them (no scan launch)."""
    x, do, dsf = _inputs(707 + dv, 8, 256, 8, dv)
    need = gla.lib().gla_chunk_bwd_workspace_bytes(1, 8, 256, 8, 96, dv, 0)
    assert need == 2 * (8 * 2 * 8 * 96 * dv * 4)  # two segments' states and carries
    _check("bwd two segments dv%d" % dv, _run(x, do, dsf), _oracle(x, do, dsf))


@pytest.mark.parametrize("dv", [192, 128, 64])
def test_backward_both_walks_in_one_launch(dv):
    """8 x 16 units of 256 tokens fill the GPU with both walks in one launch:
    no time segments, no scratch."""
    x, do, dsf = _inputs(709 + dv, 8, 256, 16, dv)
    assert gla.lib().gla_chunk_bwd_workspace_bytes(1, 8, 256, 16, 96, dv, 0) == 0
    _check("bwd one launch dv%d" % dv, _run(x, do, dsf), _oracle(x, do, dsf))


@pytest.mark.parametrize("T,dv", [(1000, 192), (2048, 128), (300, 192), (64, 192)])
def test_backward_tail_share_changes_no_bit(T, dv):
    """In the one-launch backward the dq walk's workgroups form the dk and dv
    rows of the last chunks of each sequence (GLA_BWD_TAIL: the share of
    chunks moved, 0 to 0.5) while the reverse walk only carries the gradient
    through them. Every carry is formed by the same operations in the same
    order either way, so every output equals the one-walk result bit for bit;
    and it matches the oracle."""
    x, do, dsf = _inputs(716 + T + dv, 8, T, 16, dv)
    assert gla.lib().gla_chunk_bwd_workspace_bytes(1, 8, T, 16, 96, dv, 0) == 0
    with env(GLA_BWD_TAIL="0"):
        base = _run(x, do, dsf)
    for share in ("0.1875", "0.25", "0.5"):
        with env(GLA_BWD_TAIL=share):
            got = _run(x, do, dsf)
        for n, u, w in zip(("dq", "dk", "dv", "dS0"), base, got):
            np.testing.assert_array_equal(u, w, err_msg="%s share %s" % (n, share))
    if T <= 1000:
        _check("bwd tail share T%d dv%d" % (T, dv), got, _oracle(x, do, dsf))


def test_backward_max_heads_with_lambda_one():
    """64 heads, one of them without decay."""
    H = 64
    lam = np.concatenate([[1.0], W.geometric_decays(H - 1)]).astype(np.float32)
    x = W.prefill_inputs(706, 1, 90, H, 96, 192, "bf16", 0.1, lam)
    rng = np.random.default_rng(1706)
    do = W.bf16_bits(rng.standard_normal((1, 90, H, 192), dtype=np.float32))
    dsf = rng.standard_normal((1, H, 96, 192), dtype=np.float32) * np.float32(0.5)
    _check("bwd H64", _run(x, do, dsf), _oracle(x, do, dsf))


def test_backward_without_initial_state_or_final_gradient():
    x, do, dsf = _inputs(710, 2, 150, 4, 192, with_s0=False, with_dsf=False)
    _check("bwd no s0 / dS_final", _run(x, do, dsf), _oracle(x, do, dsf))


def test_backward_scale():
    x, do, dsf = _inputs(711, 1, 130, 2, 192)
    _check("bwd scale 0.37", _run(x, do, dsf, 0.37), _oracle(x, do, dsf, 0.37))


def test_backward_laplace_prefill_full():
    """The Laplace-shaped batch (B8 T2048 H16 96/192): every head of every
    sequence, all four gradients."""
    spec = W.WORKLOADS["laplace_prefill"]
    x = W.spec_inputs("laplace_prefill")
    rng = np.random.default_rng(712)
    B, T, H, dv = spec["B"], spec["T"], spec["H"], spec["dv"]
    do = W.bf16_bits(rng.standard_normal((B, T, H, dv), dtype=np.float32))
    _check("bwd laplace B8 T2048 all heads", _run(x, do, None), _oracle(x, do, None))


def test_backward_empty_sequence_passes_gradient_through():
    x, do, dsf = _inputs(713, 2, 0, 2, 192)
    q, k, v, s0 = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["s0"])
    _, _, _, ds0 = gla.gla_chunk_bwd(q, k, v, x["decay"], dev(do), 1.0, s0, dev(dsf))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(ds0), dsf.astype(np.float64))


def test_backward_is_bitwise_deterministic():
    x, do, dsf = _inputs(714, 2, 300, 4, 192)
    a = _run(x, do, dsf)
    b = _run(x, do, dsf)
    for u, w in zip(a, b):
        np.testing.assert_array_equal(u, w)


DK_DV_OFF96 = [(64, 64), (64, 192), (64, 256), (128, 64), (128, 128), (128, 192), (128, 256)]


@pytest.mark.parametrize("T", [17, 130])
@pytest.mark.parametrize("dk,dv", DK_DV_OFF96)
def test_backward_dk64_dk128(dk, dv, T):
    """Key heads of 64 and 128 on the matrix cores: one workgroup over all
    of d_v where its tiles fit the LDS (d_v 64 and 128, and 192 at dk 64),
    else d_v tiles of 64 columns at dk 64 and of 32 at dk 128 (as the
    forward) with one partial sum per tile."""
    x, do, dsf = _inputs(760 + dk + dv + T, 2, T, 3, dv, dk=dk)
    _check("bwd dk%d dv%d T%d" % (dk, dv, T), _run(x, do, dsf), _oracle(x, do, dsf))


@pytest.mark.parametrize("dk,dv", [(64, 128), (64, 192), (128, 64), (128, 192)])
def test_backward_dk64_dk128_time_segments_and_packed(dk, dv):
    """dk 64 and 128: a fixed batch cut into time segments (boundary pass
    and both scans), then packed sequences with empty, short and long
    lengths (device planner)."""
    from gla_testutil import env
    x, do, dsf = _inputs(770 + dk, 2, 700, 3, dv, dk=dk)
    with env(GLA_TARGET_WGS=4096):
        got = _run(x, do, dsf)
    _check("bwd segmented dk%d dv%d" % (dk, dv), got, _oracle(x, do, dsf))
    lengths = [5, 0, 130, 1, 2000, 65, 300]
    x, do, dsf = _varlen_case(780 + dk, lengths, dv=dv, dk=dk)
    got = _run_varlen(x, do, dsf)
    ref = O.gla_bwd_varlen(x["cu_seqlens"], x["q"], x["k"], x["v"], x["decay"], do, 1.0,
                           x["s0"], dsf)
    _check("bwd varlen dk%d dv%d" % (dk, dv), got, ref)
    np.testing.assert_array_equal(got[3][1], dsf[1].astype(np.float64))


@pytest.mark.parametrize("T,dv", [(700, 192), (1000, 192), (700, 128), (1000, 64)])
def test_backward_time_segments(T, dv):
    """Few chains and a high workgroup target force time segments: the
    forward state pass and combine give each segment its incoming state,
    the carry pass and reverse combine its incoming gradient."""
    from gla_testutil import env
    x, do, dsf = _inputs(720 + T + dv, 2, T, 3, dv)
    with env(GLA_TARGET_WGS=4096):
        got = _run(x, do, dsf)
    _check("bwd segmented T%d dv%d" % (T, dv), got, _oracle(x, do, dsf))


def test_backward_long_context_full():
    """B1 T65536 (time segments by default): every head over the whole
    sequence, all four gradients."""
    spec = W.WORKLOADS["long_context"]
    x = W.spec_inputs("long_context")
    rng = np.random.default_rng(721)
    B, T, H, dv = spec["B"], spec["T"], spec["H"], spec["dv"]
    do = W.bf16_bits(rng.standard_normal((B, T, H, dv), dtype=np.float32))
    dsf = rng.standard_normal((B, H, 96, dv), dtype=np.float32) * np.float32(0.5)
    _check("bwd long_context T65536 all heads", _run(x, do, dsf), _oracle(x, do, dsf))


def _varlen_case(seed, lengths, H=3, dv=192, dk=96):
    x = W.varlen_inputs(seed, len(lengths), 0, H, dk, dv, "bf16", 0.1,
                        W.geometric_decays(H), lengths=lengths)
    total = int(x["cu_seqlens"][-1])
    rng = np.random.default_rng(seed + 1000)
    do = W.bf16_bits(rng.standard_normal((total, H, dv), dtype=np.float32))
    dsf = rng.standard_normal((len(lengths), H, dk, dv), dtype=np.float32) * np.float32(0.5)
    return x, do, dsf


def _run_varlen(x, do, dsf):
    q, k, v, s0 = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["s0"])
    cu = dev(x["cu_seqlens"])
    dq, dk, dv, ds0 = gla.gla_chunk_bwd_varlen(q, k, v, cu, x["decay"], dev(do), 1.0, s0,
                                               dev(dsf))
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv), host(ds0)


@pytest.mark.parametrize("lengths,dv", [([5, 0, 130, 1, 64, 65, 300], 192),
                                        ([2000, 1, 700], 192),
                                        ([5, 0, 130, 1, 2000, 65, 300], 128)])
def test_backward_varlen_matches_oracle(lengths, dv):
    """Packed sequences with empty, one-token, chunk-aligned and ragged
    lengths (one workgroup per sequence), and a few long sequences (time
    segments from the device planner)."""
    x, do, dsf = _varlen_case(730 + len(lengths), lengths, dv=dv)
    got = _run_varlen(x, do, dsf)
    ref = O.gla_bwd_varlen(x["cu_seqlens"], x["q"], x["k"], x["v"], x["decay"], do, 1.0,
                           x["s0"], dsf)
    _check("bwd varlen %s" % lengths, got, ref)
    for n, L in enumerate(lengths):
        if L == 0:
            np.testing.assert_array_equal(got[3][n], dsf[n].astype(np.float64))


def test_backward_varlen_tail_share_changes_no_bit():
    """The same over packed sequences of mixed lengths (empty, one token,
    ragged, long) in the one-launch backward."""
    x, do, dsf = _varlen_case(741, [300, 1, 0, 1000, 64, 129, 700, 5], H=16)
    with env(GLA_BWD_TAIL="0"):
        base = _run_varlen(x, do, dsf)
    with env(GLA_BWD_TAIL="0.5"):
        got = _run_varlen(x, do, dsf)
    for n, u, w in zip(("dq", "dk", "dv", "dS0"), base, got):
        np.testing.assert_array_equal(u, w, err_msg=n)
    ref = O.gla_bwd_varlen(x["cu_seqlens"], x["q"], x["k"], x["v"], x["decay"], do, 1.0,
                           x["s0"], dsf)
    _check("bwd varlen tail share", got, ref)


def test_backward_varlen_equals_fixed_batch():
    """Equal lengths packed: bitwise the fixed-batch backward on the same
    tokens (both split each sequence into the same two time segments)."""
    B, T, H = 4, 300, 16
    x, do, dsf = _inputs(740, B, T, H, 192)
    got_f = _run(x, do, dsf)
    cu = np.arange(B + 1, dtype=np.int32) * T
    q, k, v = (dev(x[n].reshape(B * T, H, -1)) for n in ("q", "k", "v"))
    dq, dk, dv, ds0 = gla.gla_chunk_bwd_varlen(q, k, v, dev(cu), x["decay"],
                                               dev(do.reshape(B * T, H, -1)), 1.0,
                                               dev(x["s0"]), dev(dsf))
    torch.cuda.synchronize()
    got_v = (host(dq).reshape(B, T, H, -1), host(dk).reshape(B, T, H, -1),
             host(dv).reshape(B, T, H, -1), host(ds0))
    for a, b in zip(got_f, got_v):
        np.testing.assert_array_equal(a, b)
