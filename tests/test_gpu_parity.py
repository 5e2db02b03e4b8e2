"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs. Bar: max|gpu - oracle| <= 1e-2 * max|oracle| for bf16
inputs and <= 1e-4 for fp32 inputs, for outputs and final states.

Full-size workloads are run in full on the GPU and compared in full: every
head of every sequence, every decode row at every step (the threaded fp64
oracle takes seconds for each of them)."""
import numpy as np
import pytest
import torch

from chunked_gated_recurrent_amd import gla
from chunked_gated_recurrent_amd import workloads as W
from oracle import oracle as O
from gla_testutil import TOL, dev, env, host, oracle_fixed, oracle_varlen, per_head, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gla.lib()
    yield
    torch.cuda.synchronize()


def run_fixed(x, chunk=0, s_in_place=False):
    q, k, v, s0 = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["s0"])
    if s_in_place:
        o, sf = gla.gla_chunk_fwd(q, k, v, x["decay"], initial_state=s0,
                                  final_state=s0, chunk=chunk)
    else:
        o, sf = gla.gla_chunk_fwd(q, k, v, x["decay"], initial_state=s0, chunk=chunk)
    torch.cuda.synchronize()
    return host(o), host(sf)


def check(name, got_o, ref_o, got_s, ref_s, tol, head_axis_o=2, head_axis_s=1):
    eo, es = rel_err(got_o, ref_o), rel_err(got_s, ref_s)
    print("%s: o err %.3e  S err %.3e  (tol %.0e)" % (name, eo, es, tol))
    if ref_o.size and ref_o.ndim > head_axis_o:
        print("  per-head o:", " ".join("%.1e" % e for e in per_head(got_o, ref_o, head_axis_o)))
    assert np.isfinite(got_o).all() and np.isfinite(got_s).all()
    assert eo <= tol, (name, "o", eo)
    assert es <= tol, (name, "S", es)


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------
def test_tiny_fp32_workload():
    x = W.spec_inputs("tiny_fp32")
    o, s = run_fixed(x, chunk=32)
    ro, rs = oracle_fixed(x)
    check("tiny_fp32", o, ro, s, rs, TOL["f32"])


def test_laplace_prefill_full():
    x = W.spec_inputs("laplace_prefill")
    o, s = run_fixed(x)
    ro, rs = oracle_fixed(x)
    check("laplace_prefill B8 T2048", o, ro, s, rs, TOL["bf16"])


def test_long_context_full():
    """B1 T65536 from a random initial state (segmented carry on the GPU):
    every head over the whole sequence, outputs and final states."""
    x = W.spec_inputs("long_context")
    o, s = run_fixed(x, chunk=64)
    ro, rs = oracle_fixed(x)
    check("long_context T65536 all heads", o, ro, s, rs, TOL["bf16"])


def test_varlen_workload_full():
    """32 packed sequences with lengths uniform in [1, 8192]: every head of
    every sequence."""
    x = W.spec_inputs("varlen")
    q, k, v, s0 = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["s0"])
    cu = dev(x["cu_seqlens"])
    o, sf = gla.gla_chunk_fwd_varlen(q, k, v, cu, x["decay"], initial_state=s0)
    torch.cuda.synchronize()
    ro, rs = oracle_varlen(x)
    check("varlen N32 all heads", host(o), ro, host(sf), rs, TOL["bf16"], head_axis_o=1)


def test_batched_decode_100_steps_full():
    """1,280 sequences x 16 heads, 100 consecutive steps in place: every
    output row at every step, and every state after the last step."""
    spec = W.WORKLOADS["batched_decode"]
    N, H, dk, dv, steps = spec["N"], spec["H"], spec["dk"], spec["dv"], spec["steps"]
    seed = spec["seed"]
    lam = W.decays_for(spec)
    S = W.decode_state(seed, N, H, dk, dv, spec["state_sigma"])
    ref_state = S.astype(np.float64)
    state = dev(S)
    del S
    worst = 0.0
    for t in range(steps):
        q, k, v = W.decode_tokens(seed, t, N, H, dk, dv)
        o = gla.gla_decode_step(dev(q), dev(k), dev(v), lam, state)
        ro = O.gla_decode(q, k, v, lam, ref_state)
        e = rel_err(host(o), ro)
        worst = max(worst, e)
        assert e <= TOL["bf16"], (t, e)
    es = rel_err(host(state), ref_state)
    print("decode N1280 x100: worst o err %.3e, S err %.3e" % (worst, es))
    assert es <= TOL["bf16"]


# ---------------------------------------------------------------------------
# edge shapes on the MFMA path (dk 96) and the vector-ALU path
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 17, 63, 64, 65, 200])
@pytest.mark.parametrize("with_s0", [False, True])
def test_ragged_lengths_mfma(T, with_s0):
    x = W.prefill_inputs(100 + T, 2, T, 3, 96, 192, "bf16", 0.1 if with_s0 else None,
                         W.geometric_decays(3))
    o, s = run_fixed(x)
    ro, rs = oracle_fixed(x)
    check("mfma T%d s0=%s" % (T, with_s0), o, ro, s, rs, TOL["bf16"])


@pytest.mark.parametrize("T", [1, 63, 65, 200])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 192), (64, 256), (128, 64), (128, 192), (128, 256)])
def test_ragged_lengths_mfma_dk64_dk128(T, dk, dv):
    """d_k = 64 (d_v tiles of 64 columns) and 128 (tiles of 32) on the
    matrix cores."""
    x = W.prefill_inputs(140 + T + dk + dv, 2, T, 3, dk, dv, "bf16", 0.1, W.geometric_decays(3))
    o, s = run_fixed(x)
    ro, rs = oracle_fixed(x)
    check("mfma dk%d dv%d T%d" % (dk, dv, T), o, ro, s, rs, TOL["bf16"])


@pytest.mark.parametrize("dk", [64, 128])
def test_dk64_dk128_time_segments_and_packed_sequences(dk):
    """d_k = 64 and 128: one long sequence cut into time segments (state
    pass, combine, output pass), and packed sequences with and without
    segments."""
    x = W.prefill_inputs(160 + dk, 1, 3000, 2, dk, 128, "bf16", 0.1, W.geometric_decays(2))
    assert gla.lib().gla_chunk_fwd_workspace_bytes(1, 1, 3000, 2, dk, 128, 0) > 0
    o, s = run_fixed(x)
    ro, rs = oracle_fixed(x)
    check("mfma dk%d segmented T3000" % dk, o, ro, s, rs, TOL["bf16"])
    lens = [0, 1, 63, 65, 300, 1000]
    x = W.varlen_inputs(161 + dk, 0, 0, 4, dk, 192, "bf16", 0.1, W.geometric_decays(4),
                        lengths=lens)
    ro, rs = oracle_varlen(x)
    for knob in ({}, dict(GLA_TARGET_WGS=100000)):
        with env(**knob):
            q, k, v, s0 = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["s0"])
            o, sf = gla.gla_chunk_fwd_varlen(q, k, v, dev(x["cu_seqlens"]), x["decay"],
                                             initial_state=s0)
            torch.cuda.synchronize()
            check("mfma dk%d varlen %s" % (dk, knob), host(o), ro, host(sf), rs, TOL["bf16"],
                  head_axis_o=1)


@pytest.mark.parametrize("dtype,dk,dv,T,chunk", [
    ("bf16", 16, 32, 100, 32), ("f32", 32, 64, 130, 64), ("f32", 128, 256, 70, 0),
    ("bf16", 64, 128, 129, 0), ("f32", 96, 192, 257, 64), ("bf16", 96, 128, 150, 0),
    ("bf16", 96, 64, 150, 0), ("bf16", 96, 256, 150, 0), ("bf16", 128, 256, 90, 0)])
def test_shapes(dtype, dk, dv, T, chunk):
    x = W.prefill_inputs(7 + dk + T, 2, T, 2, dk, dv, dtype, 0.1, np.array([0.9, 0.995], np.float32))
    o, s = run_fixed(x, chunk=chunk)
    ro, rs = oracle_fixed(x)
    check("%s dk%d dv%d T%d C%d" % (dtype, dk, dv, T, chunk), o, ro, s, rs, TOL[dtype])


def test_max_heads_and_lambda_one():
    lam = np.concatenate([[1.0], W.geometric_decays(63)]).astype(np.float32)
    x = W.prefill_inputs(55, 1, 96, 64, 96, 192, "bf16", 0.1, lam)
    o, s = run_fixed(x)
    ro, rs = oracle_fixed(x)
    check("H64 with lambda=1", o, ro, s, rs, TOL["bf16"])


@pytest.mark.parametrize("T", [63, 300])
def test_extreme_decays(T):
    """Decays from nearly instant forgetting (powers underflow to zero within
    a chunk) to none at all, with time segments forced so that the carried
    state crosses segment boundaries; forward and backward."""
    from gla_testutil import env
    lam = np.array([1e-6, 1e-3, 0.25, 0.5, 0.9999, 1.0], np.float32)
    x = W.prefill_inputs(56 + T, 2, T, 6, 96, 192, "bf16", 0.1, lam)
    with env(GLA_TARGET_WGS=4096):
        o, s = run_fixed(x)
    ro, rs = oracle_fixed(x)
    check("extreme decays T%d" % T, o, ro, s, rs, TOL["bf16"])
    rng = np.random.default_rng(57 + T)
    do = W.bf16_bits(rng.standard_normal((2, T, 6, 192), dtype=np.float32))
    q, k, v, s0 = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["s0"])
    with env(GLA_TARGET_WGS=4096):
        g = gla.gla_chunk_bwd(q, k, v, lam, dev(do), 1.0, s0)
    torch.cuda.synchronize()
    ref = O.gla_bwd(x["q"], x["k"], x["v"], lam, do, 1.0, x["s0"])
    for name, a, b in zip(("dq", "dk", "dv", "dS0"), g, ref):
        e = rel_err(host(a), b)
        print("  bwd %s %.2e" % (name, e))
        assert np.isfinite(host(a)).all() and e <= TOL["bf16"], (name, e)


def test_empty_sequence_passes_state_through():
    x = W.prefill_inputs(3, 2, 0, 4, 96, 192, "bf16", 0.1, W.geometric_decays(4))
    s0 = dev(x["s0"])
    o, sf = gla.gla_chunk_fwd(dev(x["q"]), dev(x["k"]), dev(x["v"]), x["decay"], initial_state=s0)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert torch.equal(sf, s0)


# ---------------------------------------------------------------------------
# invariants of the recurrence, checked on the GPU path
# ---------------------------------------------------------------------------
def test_segmented_carry_matches_oracle_and_in_place_state():
    """Force time segmentation on a batch (and write the final state over the
    initial one) and compare with the oracle."""
    x = W.prefill_inputs(21, 2, 1000, 4, 96, 192, "bf16", 0.1, W.geometric_decays(4))
    ro, rs = oracle_fixed(x)
    with env(GLA_TARGET_WGS=100000):
        need = gla.lib().gla_chunk_fwd_workspace_bytes(1, 2, 1000, 4, 96, 192, 0)
        assert need > 0
        o, s = run_fixed(x)
        check("segmented", o, ro, s, rs, TOL["bf16"])
        o2, s2 = run_fixed(x, s_in_place=True)
        check("segmented in place", o2, ro, s2, rs, TOL["bf16"])
    o3, s3 = run_fixed(x, s_in_place=True)
    check("unsegmented in place", o3, ro, s3, rs, TOL["bf16"])


def test_chunk_sizes_agree():
    """The two chunk sizes the library runs (32 on the vector ALUs, 64 on
    the matrix cores) both meet the bar; 0 is the default 64 (bitwise the
    same call) and 128, which no kernel runs, is refused."""
    x = W.prefill_inputs(31, 1, 300, 2, 96, 192, "bf16", 0.1, np.array([0.97, 0.999], np.float32))
    ro, rs = oracle_fixed(x)
    res = {}
    for c in (0, 32, 64):
        res[c] = run_fixed(x, chunk=c)
        check("chunk %d" % c, res[c][0], ro, res[c][1], rs, TOL["bf16"])
    assert np.array_equal(res[0][0], res[64][0]) and np.array_equal(res[0][1], res[64][1])
    with pytest.raises(gla.GlaError) as e:
        run_fixed(x, chunk=128)
    assert e.value.code == 6  # GLA_ERR_UNSUPPORTED


@pytest.mark.parametrize("T1", [1, 63, 64, 65, 255])
def test_split_invariance(T1):
    x = W.prefill_inputs(41, 2, 256, 3, 96, 192, "bf16", 0.1, W.geometric_decays(3))
    q, k, v, s0 = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["s0"])
    o, s = gla.gla_chunk_fwd(q, k, v, x["decay"], initial_state=s0)
    oa, sa = gla.gla_chunk_fwd(q[:, :T1].contiguous(), k[:, :T1].contiguous(),
                               v[:, :T1].contiguous(), x["decay"], initial_state=s0)
    ob, sb = gla.gla_chunk_fwd(q[:, T1:].contiguous(), k[:, T1:].contiguous(),
                               v[:, T1:].contiguous(), x["decay"], initial_state=sa)
    torch.cuda.synchronize()
    ro, rs = oracle_fixed(x)
    check("split at %d" % T1, np.concatenate([host(oa), host(ob)], axis=1), ro,
          host(sb), rs, TOL["bf16"])
    check("unsplit", host(o), ro, host(s), rs, TOL["bf16"])


def test_decode_steps_equal_chunked_and_handoff():
    """T decode steps from S0 equal one chunked call; a prefill followed by
    decode steps equals one longer prefill."""
    T, Tp = 40, 25
    x = W.prefill_inputs(51, 3, T, 4, 96, 192, "bf16", 0.1, W.geometric_decays(4))
    q, k, v, s0 = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["s0"])
    ro, rs = oracle_fixed(x)
    state = s0.clone()
    outs = []
    for t in range(T):
        outs.append(host(gla.gla_decode_step(q[:, t].contiguous(), k[:, t].contiguous(),
                                             v[:, t].contiguous(), x["decay"], state)))
    check("decode x%d" % T, np.stack(outs, axis=1), ro, host(state), rs, TOL["bf16"])
    op, sp = gla.gla_chunk_fwd(q[:, :Tp].contiguous(), k[:, :Tp].contiguous(),
                               v[:, :Tp].contiguous(), x["decay"], initial_state=s0)
    outs = [host(op)]
    for t in range(Tp, T):
        outs.append(host(gla.gla_decode_step(q[:, t].contiguous(), k[:, t].contiguous(),
                                             v[:, t].contiguous(), x["decay"], sp))[:, None])
    check("prefill %d + decode" % Tp, np.concatenate(outs, axis=1), ro, host(sp), rs, TOL["bf16"])


@pytest.mark.parametrize("segmented", [False, True])
def test_varlen_ragged_and_empty_sequences(segmented):
    lens = [0, 1, 63, 64, 65, 300, 0, 1000]
    x = W.varlen_inputs(61, 0, 0, 4, 96, 192, "bf16", 0.1, W.geometric_decays(4), lengths=lens)
    ro, rs = oracle_varlen(x)
    knob = dict(GLA_TARGET_WGS=100000) if segmented else {}
    with env(**knob):
        q, k, v, s0 = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["s0"])
        o, sf = gla.gla_chunk_fwd_varlen(q, k, v, dev(x["cu_seqlens"]), x["decay"], initial_state=s0)
        torch.cuda.synchronize()
        check("varlen ragged seg=%s" % segmented, host(o), ro, host(sf), rs, TOL["bf16"], head_axis_o=1)
        # sequences are independent: each equals its own fixed-length call
        cu = x["cu_seqlens"]
        for n, L in enumerate(lens):
            if L == 0:
                assert torch.equal(sf[n], s0[n])
                continue
            a, b = int(cu[n]), int(cu[n + 1])
            on, sn = gla.gla_chunk_fwd(q[None, a:b], k[None, a:b], v[None, a:b], x["decay"],
                                       initial_state=s0[n:n + 1].contiguous())
            torch.cuda.synchronize()
            assert rel_err(host(on)[0], host(o)[a:b]) <= TOL["bf16"]
            assert rel_err(host(sn)[0], host(sf)[n]) <= TOL["bf16"]


def test_varlen_fp32_path():
    x = W.varlen_inputs(62, 0, 0, 2, 32, 64, "f32", 0.1, np.array([0.9, 0.99], np.float32),
                        lengths=[5, 0, 130, 64])
    o, sf = gla.gla_chunk_fwd_varlen(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["cu_seqlens"]),
                                     x["decay"], initial_state=dev(x["s0"]))
    torch.cuda.synchronize()
    ro, rs = oracle_varlen(x)
    check("varlen fp32", host(o), ro, host(sf), rs, TOL["f32"], head_axis_o=1)


def test_causality_future_tokens_do_not_leak():
    """Changing tokens after t0 leaves outputs up to t0 unchanged; NaN placed
    in the next chunk never reaches earlier outputs. (A NaN inside the same
    chunk would reach them through 0 * NaN in the masked product.)"""
    T, t0 = 192, 100
    x = W.prefill_inputs(71, 1, T, 2, 96, 192, "bf16", None, W.geometric_decays(2))
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    o, _ = gla.gla_chunk_fwd(q, k, v, x["decay"])
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    for t in (q2, k2, v2):
        t[:, t0 + 1:] = 7.0
    o2, _ = gla.gla_chunk_fwd(q2, k2, v2, x["decay"])
    torch.cuda.synchronize()
    assert torch.equal(o[:, :t0 + 1], o2[:, :t0 + 1])
    for t in (q2, k2, v2):
        t[:, 128:] = float("nan")
    o3, _ = gla.gla_chunk_fwd(q2, k2, v2, x["decay"])
    torch.cuda.synchronize()
    assert torch.isfinite(o3[:, :128]).all()
    assert torch.equal(o[:, :t0 + 1], o3[:, :t0 + 1])


def test_run_to_run_bitwise_determinism():
    x = W.prefill_inputs(81, 1, 3000, 16, 96, 192, "bf16", 0.1)
    q, k, v, s0 = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["s0"])
    o1, s1 = gla.gla_chunk_fwd(q, k, v, x["decay"], initial_state=s0)
    o2, s2 = gla.gla_chunk_fwd(q, k, v, x["decay"], initial_state=s0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


# ---------------------------------------------------------------------------
# closed forms at the long-context size (any-size properties, no oracle run)
# ---------------------------------------------------------------------------
def _long_inputs(seed, s0_sigma=None):
    T, H = 65536, 16
    x = W.prefill_inputs(seed, 1, T, H, 96, 192, "bf16", s0_sigma, W.geometric_decays(H))
    return x, T, H


def test_constant_tokens_geometric_series_long():
    """k_t = k and v_t = v for every token, zero initial state: the state is
    a geometric series, S_t = (1 - lam^(t+1)) / (1 - lam) k^T v, so
    o_t = (q_t . k) (1 - lam^(t+1)) / (1 - lam) v. Checked for every token
    of T = 65,536 (segmented carry over 1,024 chunks), all 16 heads."""
    x, T, H = _long_inputs(300)
    k0 = x["k"][:, :1].copy()
    v0 = x["v"][:, :1].copy()
    x["k"][:] = k0
    x["v"][:] = v0
    o, s = run_fixed(x, chunk=64)
    lam = x["decay"].astype(np.float64)
    qf = W.bf16_to_f32(x["q"][0]).astype(np.float64)          # [T, H, dk]
    kf = W.bf16_to_f32(k0[0, 0]).astype(np.float64)            # [H, dk]
    vf = W.bf16_to_f32(v0[0, 0]).astype(np.float64)            # [H, dv]
    t = np.arange(T, dtype=np.float64)
    worst_o = worst_s = 0.0
    den_o = den_s = 0.0
    errs = []
    for h in range(H):
        g = (1.0 - lam[h] ** (t + 1.0)) / (1.0 - lam[h])
        ref = ((qf[:, h] @ kf[h]) * g)[:, None] * vf[h][None, :]
        got = o[0, :, h]
        err = np.max(np.abs(got - ref))
        den = np.max(np.abs(ref))
        errs.append(err / den)
        worst_o, den_o = max(worst_o, err), max(den_o, den)
        sref = np.outer(kf[h], vf[h]) * (1.0 - lam[h] ** T) / (1.0 - lam[h])
        worst_s = max(worst_s, np.max(np.abs(s[0, h] - sref)))
        den_s = max(den_s, np.max(np.abs(sref)))
    print("constant tokens T65536: o err %.3e  S err %.3e" % (worst_o / den_o, worst_s / den_s))
    print("  per-head o:", " ".join("%.1e" % e for e in errs))
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert worst_o / den_o <= TOL["bf16"]
    assert worst_s / den_s <= TOL["bf16"]


def test_decay_only_long():
    """v = 0: nothing is added to the state, so S_T = lam^T S0 and
    o_t = lam^(t+1) q_t S0 for every token of T = 65,536 (the carried state
    crosses 1,024 chunks and every time segment)."""
    x, T, H = _long_inputs(301, s0_sigma=0.1)
    x["v"][:] = 0
    o, s = run_fixed(x, chunk=64)
    lam = x["decay"].astype(np.float64)
    qf = W.bf16_to_f32(x["q"][0]).astype(np.float64)
    s0 = x["s0"][0].astype(np.float64)
    t = np.arange(T, dtype=np.float64)
    worst_o = den_o = 0.0
    worst_s = den_s = 0.0
    for h in range(H):
        ref = (lam[h] ** (t + 1.0))[:, None] * (qf[:, h] @ s0[h])
        worst_o = max(worst_o, np.max(np.abs(o[0, :, h] - ref)))
        den_o = max(den_o, np.max(np.abs(ref)))
        sref = lam[h] ** T * s0[h]
        worst_s = max(worst_s, np.max(np.abs(s[0, h] - sref)))
        den_s = max(den_s, np.max(np.abs(sref)))
    print("decay only T65536: o err %.3e  S err %.3e (max|S_ref| %.2e)"
          % (worst_o / den_o, worst_s / den_s, den_s))
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert worst_o / den_o <= TOL["bf16"]
    assert worst_s / den_s <= TOL["bf16"]


# ---------------------------------------------------------------------------
# decode against a state pool (per-sequence pages, padded batches)
# ---------------------------------------------------------------------------
def _pool_slots(rng, N, P, n_pad):
    """Distinct valid slots for N - n_pad rows, padding rows get -1 or a
    value >= P."""
    slots = rng.permutation(P)[:N].astype(np.int32)
    pad = rng.permutation(N)[:n_pad]
    slots[pad] = np.where(rng.random(n_pad) < 0.5, -1, P + rng.integers(0, 5, n_pad))
    return slots


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_pool_matches_oracle_over_steps(dtype):
    rng = np.random.default_rng(40)
    N, H, dk, dv, P, steps = 48, 4, 96, 192, 100, 6
    lam = W.geometric_decays(H)
    pool0 = (rng.standard_normal((P, H, dk, dv)) * 0.3).astype(np.float32)
    ref = pool0.astype(np.float64)
    pool = dev(pool0)
    touched = np.zeros(P, bool)
    tol = TOL[dtype]
    for t in range(steps):
        x = W.prefill_inputs(500 + t, 1, N, H, dk, dv, dtype, None, lam)
        q, k, v = x["q"][0], x["k"][0], x["v"][0]
        slots = _pool_slots(rng, N, P, 7)
        o = gla.gla_decode_step_pool(dev(q), dev(k), dev(v), lam, pool, dev(slots))
        ro = O.gla_decode_pool(q, k, v, lam, ref, slots)
        got = host(o)
        valid = (slots >= 0) & (slots < P)
        touched[slots[valid]] = True
        assert not got[~valid].any(), "padding rows must read zero"
        e = rel_err(got[valid], ro[valid])
        print("pool step %d: o err %.3e" % (t, e))
        assert e <= tol, (t, e)
    fin = host(pool)
    assert rel_err(fin[touched], ref[touched]) <= tol
    np.testing.assert_array_equal(fin[~touched], pool0[~touched].astype(np.float64))


def test_decode_pool_is_bitwise_the_direct_step():
    """The pool step on a permuted pool equals the direct step on the same
    states gathered into batch order, bit for bit (same kernel arithmetic)."""
    rng = np.random.default_rng(41)
    N, H, dk, dv, P = 64, 16, 96, 192, 96
    lam = W.geometric_decays(H)
    x = W.prefill_inputs(600, 1, N, H, dk, dv, "bf16", None, lam)
    q, k, v = dev(x["q"][0]), dev(x["k"][0]), dev(x["v"][0])
    slots = rng.permutation(P)[:N].astype(np.int32)
    pool = torch.randn(P, H, dk, dv, device="cuda") * 0.3
    direct = pool[torch.from_numpy(slots).long().cuda()].contiguous()
    o_pool = gla.gla_decode_step_pool(q, k, v, lam, pool, dev(slots))
    o_dir = gla.gla_decode_step(q, k, v, lam, direct)
    torch.cuda.synchronize()
    assert torch.equal(o_pool, o_dir)
    assert torch.equal(pool[torch.from_numpy(slots).long().cuda()], direct)


def test_decode_pool_full_size():
    """1,280 rows (128 of them padding) against a pool of 2,048 pages at the
    Laplace head shape: every row's output and every page against the
    oracle's pooled step (untouched pages bit-identical)."""
    rng = np.random.default_rng(42)
    spec = W.WORKLOADS["batched_decode"]
    N, H, dk, dv = spec["N"], spec["H"], spec["dk"], spec["dv"]
    P = 2048
    lam = W.decays_for(spec)
    pool = torch.randn(P, H, dk, dv, device="cuda").mul_(spec["state_sigma"])
    slots = _pool_slots(rng, N, P, 128)
    valid = np.nonzero((slots >= 0) & (slots < P))[0]
    before = W.to_numpy_bits(pool)  # fp32 copy of the whole pool
    ref = before.astype(np.float64)
    q, k, v = W.decode_tokens(spec["seed"], 0, N, H, dk, dv)
    o = host(gla.gla_decode_step_pool(dev(q), dev(k), dev(v), lam, pool, dev(slots)))
    ro = O.gla_decode_pool(q, k, v, lam, ref, slots)
    got = W.to_numpy_bits(pool)
    e = rel_err(o, ro)
    es = rel_err(got[slots[valid]], ref[slots[valid]])
    print("pool decode N1280 P2048: o err %.3e  S err %.3e" % (e, es))
    pad = np.setdiff1d(np.arange(N), valid)
    assert not o[pad].any()
    untouched = np.setdiff1d(np.arange(P), slots[valid])
    np.testing.assert_array_equal(got[untouched], before[untouched])
    assert e <= TOL["bf16"] and es <= TOL["bf16"]
