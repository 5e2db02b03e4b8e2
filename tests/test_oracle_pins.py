"""Pins of the fp64 oracle against facts fixed by the pages and by algebra,
not against the oracle itself. CPU only.

Each pin targets a plausible mistake:
  * hand-worked examples and exact rational brute force: any wrong term,
    sign, index or transposition changes an exactly known number;
  * O(T^2) masked form: the decay exponent (lambda^(t-s), inclusive
    diagonal) and the initial-state term lambda^(t+1) q_t S0;
  * lambda = 1: the prefix-sum / cumulative linear attention special case
    (tutorial page on recurrence-free sequence models, sections 3.2 and 6.1);
  * T = 1: the readout happens after the update;
  * split invariance, decode == forward, varlen == separate calls: the
    state hand-over;
  * constant tokens and decay only: closed-form geometric series at long
    range;
  * linearity, head permutation, causality (tutorial page, section 8).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O
from chunked_gated_recurrent_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _rand(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def brute_masked(q, k, v, lam, scale=1.0, s0=None):
    """O(T^2) unrolled form of one sequence, fp64:
    o_t = scale * (sum_{s<=t} lam^(t-s) (q_t . k_s) v_s + lam^(t+1) q_t S0)
    S_T = lam^T S0 + sum_s lam^(T-1-s) k_s^T v_s
    q, k: [T, H, dk]; v: [T, H, dv]; s0: [H, dk, dv] or None."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    T, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((T, H, dv))
    S = np.zeros((H, dk, dv))
    t = np.arange(T)[:, None]
    s = np.arange(T)[None, :]
    for h in range(H):
        lh = float(np.float32(lam[h]))
        D = np.where(t >= s, lh ** np.maximum(t - s, 0), 0.0)
        A = (q[:, h, :] @ k[:, h, :].T) * D
        o[:, h, :] = A @ v[:, h, :]
        w = lh ** (T - 1 - np.arange(T))
        S[h] = (k[:, h, :] * w[:, None]).T @ v[:, h, :]
        if s0 is not None:
            S0 = np.asarray(s0[h], np.float64)
            o[:, h, :] += (lh ** (np.arange(T) + 1))[:, None] * (q[:, h, :] @ S0)
            S[h] += lh ** T * S0
    return scale * o, S


# ---------------------------------------------------------------------------
# hand-worked examples (exact)
# ---------------------------------------------------------------------------
def test_hand_worked_examples_exact():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], np.float32)[None]
        k = np.array(c["k"], np.float32)[None]
        v = np.array(c["v"], np.float32)[None]
        s0 = None if c["s0"] is None else np.array(c["s0"], np.float32)[None]
        o, sf = O.gla_fwd(q, k, v, c["decay"], 1.0, s0)
        np.testing.assert_array_equal(o[0], np.array(c["o"]), err_msg=c["name"])
        np.testing.assert_array_equal(sf[0], np.array(c["s_final"]), err_msg=c["name"])


def test_exact_rational_brute_force():
    """Dyadic inputs and lambda = 3/4: every fp64 intermediate is exact, so the
    oracle must equal the rational-arithmetic unrolled sum bit for bit."""
    rng = np.random.default_rng(11)
    T, dk, dv = 6, 3, 2
    vals = np.array([-2, -1, -0.5, 0, 0.5, 1, 2], np.float32)
    q = rng.choice(vals, (T, 1, dk))
    k = rng.choice(vals, (T, 1, dk))
    v = rng.choice(vals, (T, 1, dv))
    s0 = rng.choice(vals, (1, dk, dv))
    lam = Fraction(3, 4)
    F = lambda x: Fraction(float(x))  # noqa: E731
    o_ref = np.zeros((T, dv))
    for t in range(T):
        for j in range(dv):
            acc = Fraction(0)
            for s in range(t + 1):
                dot = sum(F(q[t, 0, i]) * F(k[s, 0, i]) for i in range(dk))
                acc += lam ** (t - s) * dot * F(v[s, 0, j])
            acc += lam ** (t + 1) * sum(F(q[t, 0, i]) * F(s0[0, i, j]) for i in range(dk))
            o_ref[t, j] = float(acc)
    S_ref = np.zeros((dk, dv))
    for i in range(dk):
        for j in range(dv):
            acc = lam ** T * F(s0[0, i, j])
            for s in range(T):
                acc += lam ** (T - 1 - s) * F(k[s, 0, i]) * F(v[s, 0, j])
            S_ref[i, j] = float(acc)
    o, sf = O.gla_fwd(q[None], k[None], v[None], [0.75], 1.0, s0[None])
    np.testing.assert_array_equal(o[0, :, 0, :], o_ref)
    np.testing.assert_array_equal(sf[0, 0], S_ref)


# ---------------------------------------------------------------------------
# O(T^2) masked form on random inputs
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,H,dk,dv,with_s0,scale", [
    (1, 1, 4, 4, False, 1.0), (17, 2, 8, 16, False, 1.0), (64, 3, 16, 8, True, 1.0),
    (40, 2, 5, 7, True, 0.37)])
def test_brute_masked_form(T, H, dk, dv, with_s0, scale):
    rng = np.random.default_rng(T * 100 + dk)
    q, k, v = _rand(rng, (T, H, dk), 0.3), _rand(rng, (T, H, dk), 0.3), _rand(rng, (T, H, dv))
    s0 = _rand(rng, (H, dk, dv)) if with_s0 else None
    lam = np.array([0.875, 0.5, 0.999][:H], np.float32)
    o, sf = O.gla_fwd(q[None], k[None], v[None], lam, scale,
                      None if s0 is None else s0[None])
    o_ref, S_ref = brute_masked(q, k, v, lam, scale, s0)
    assert np.max(np.abs(o[0] - o_ref)) <= 1e-12 * max(1.0, np.max(np.abs(o_ref)))
    assert np.max(np.abs(sf[0] - S_ref)) <= 1e-12 * max(1.0, np.max(np.abs(S_ref)))


def test_tiny_workload_matches_brute_force():
    """The tiny fp32 workload (B1 H2 T256 dk16 dv32) in full."""
    spec = W.WORKLOADS["tiny_fp32"]
    x = W.spec_inputs("tiny_fp32")
    o, sf = O.gla_fwd(x["q"], x["k"], x["v"], x["decay"])
    o_ref, S_ref = brute_masked(x["q"][0], x["k"][0], x["v"][0], x["decay"])
    assert o.shape == (1, spec["T"], spec["H"], spec["dv"])
    assert np.max(np.abs(o[0] - o_ref)) <= 1e-12 * np.max(np.abs(o_ref))
    assert np.max(np.abs(sf[0] - S_ref)) <= 1e-12 * np.max(np.abs(S_ref))


def test_decay_is_taken_as_the_given_fp32_value():
    """lambda = 0.1 is not representable: the oracle must use float32(0.1)."""
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, (30, 1, 4)), _rand(rng, (30, 1, 4)), _rand(rng, (30, 1, 3))
    o, _ = O.gla_fwd(q[None], k[None], v[None], [0.1])
    o32, _ = brute_masked(q, k, v, np.array([0.1], np.float32))
    o64 = np.zeros_like(o32)
    for t in range(30):  # same sum with the fp64 value 0.1
        for s in range(t + 1):
            o64[t, 0] += 0.1 ** (t - s) * (q[t, 0] @ k[s, 0].astype(np.float64)) * v[s, 0]
    assert np.max(np.abs(o[0] - o32)) <= 1e-13 * np.max(np.abs(o32))
    assert np.max(np.abs(o[0] - o64)) > 1e-10 * np.max(np.abs(o64))


# ---------------------------------------------------------------------------
# lambda = 1: cumulative linear attention
# ---------------------------------------------------------------------------
def test_lambda_one_is_cumulative_linear_attention():
    rng = np.random.default_rng(3)
    T, H, dk, dv = 50, 2, 6, 5
    q, k, v = _rand(rng, (T, H, dk)), _rand(rng, (T, H, dk)), _rand(rng, (T, H, dv))
    o, sf = O.gla_fwd(q[None], k[None], v[None], [1.0, 1.0])
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    kv = k64[:, :, :, None] * v64[:, :, None, :]          # per-token outer products
    kv_cum = np.cumsum(kv, axis=0)                          # prefix sums over time
    ref = np.einsum("thd,thde->the", q64, kv_cum)           # numerator of the page's form
    assert np.max(np.abs(o[0] - ref)) <= 1e-12 * np.max(np.abs(ref))
    np.testing.assert_allclose(sf[0], kv_cum[-1], rtol=0, atol=1e-12 * np.max(np.abs(kv_cum)))


# ---------------------------------------------------------------------------
# T = 1
# ---------------------------------------------------------------------------
def test_single_token():
    rng = np.random.default_rng(4)
    H, dk, dv = 3, 7, 5
    q, k, v = _rand(rng, (1, H, dk)), _rand(rng, (1, H, dk)), _rand(rng, (1, H, dv))
    lam = np.array([0.9, 0.5, 1.0], np.float32)
    o, sf = O.gla_fwd(q[None], k[None], v[None], lam)
    q64, k64, v64 = (x[0].astype(np.float64) for x in (q, k, v))
    for h in range(H):
        np.testing.assert_allclose(o[0, 0, h], (q64[h] @ k64[h]) * v64[h], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(sf[0, h], np.outer(k64[h], v64[h]), rtol=1e-15, atol=0)
    s0 = _rand(rng, (H, dk, dv))
    o, sf = O.gla_fwd(q[None], k[None], v[None], lam, 1.0, s0[None])
    for h in range(H):
        S = float(lam[h]) * s0[h].astype(np.float64) + np.outer(k64[h], v64[h])
        np.testing.assert_allclose(o[0, 0, h], q64[h] @ S, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(sf[0, h], S, rtol=1e-15, atol=1e-15)


# ---------------------------------------------------------------------------
# state hand-over
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T1", [1, 31, 32, 33, 69])
def test_split_invariance(T1):
    rng = np.random.default_rng(7)
    T, H, dk, dv = 70, 2, 8, 6
    q, k, v = _rand(rng, (1, T, H, dk)), _rand(rng, (1, T, H, dk)), _rand(rng, (1, T, H, dv))
    s0 = _rand(rng, (1, H, dk, dv))
    lam = np.array([0.9, 0.97], np.float32)
    o, sf = O.gla_fwd(q, k, v, lam, 1.0, s0)
    oa, sa = O.gla_fwd(q[:, :T1], k[:, :T1], v[:, :T1], lam, 1.0, s0)
    ob, sb = O.gla_fwd(q[:, T1:], k[:, T1:], v[:, T1:], lam, 1.0, sa)
    np.testing.assert_array_equal(np.concatenate([oa, ob], axis=1), o)
    np.testing.assert_array_equal(sb, sf)


def test_decode_steps_equal_forward():
    rng = np.random.default_rng(8)
    T, N, H, dk, dv = 12, 3, 2, 5, 4
    q, k, v = _rand(rng, (N, T, H, dk)), _rand(rng, (N, T, H, dk)), _rand(rng, (N, T, H, dv))
    s0 = _rand(rng, (N, H, dk, dv))
    lam = np.array([0.8, 0.95], np.float32)
    o, sf = O.gla_fwd(q, k, v, lam, 0.5, s0)
    state = s0.astype(np.float64)
    for t in range(T):
        ot = O.gla_decode(q[:, t], k[:, t], v[:, t], lam, state, 0.5)
        np.testing.assert_array_equal(ot, o[:, t])
    np.testing.assert_array_equal(state, sf)


def test_decode_pool_equals_forward_per_sequence_and_leaves_the_rest():
    """A state pool with per-sequence pages and padded batches: three
    sequences live in pages 4, 1 and 3 of a 6-page pool and get tokens in a
    batch of 4 rows whose row order changes each step; unused rows are padding
    (slot -1 or >= P). Each page must end as the chunked forward over the
    tokens its sequence received (and each output must equal that forward's
    output at the same position); pages 0, 2 and 5 stay bit-identical and
    padding rows read zero."""
    rng = np.random.default_rng(21)
    H, dk, dv, P, steps = 2, 5, 4, 6, 5
    lam = np.array([0.7, 0.97], np.float32)
    page = {0: 4, 1: 1, 2: 3}
    pool0 = _rand(rng, (P, H, dk, dv)).astype(np.float64)
    pool = pool0.copy()
    hist = {n: [] for n in page}  # per sequence: (q, k, v, o) per step it ran
    for t in range(steps):
        seqs = [n for n in page if rng.random() < 0.8]
        rows = list(rng.permutation(4))
        slots = np.full(4, -1, np.int64)
        slots[rows[3]] = P + 2                     # out of range: padding too
        for n, r in zip(seqs, rows):
            slots[r] = page[n]
        q, k, v = _rand(rng, (4, H, dk)), _rand(rng, (4, H, dk)), _rand(rng, (4, H, dv))
        o = O.gla_decode_pool(q, k, v, lam, pool, slots, 0.5)
        for r in range(4):
            if not (0 <= slots[r] < P):
                assert not o[r].any()
        for n, r in zip(seqs, rows):
            hist[n].append((q[r], k[r], v[r], o[r]))
    for n, pg in page.items():
        if not hist[n]:
            np.testing.assert_array_equal(pool[pg], pool0[pg])
            continue
        qs = np.stack([h[0] for h in hist[n]])[None]
        ks = np.stack([h[1] for h in hist[n]])[None]
        vs = np.stack([h[2] for h in hist[n]])[None]
        of, sf = O.gla_fwd(qs, ks, vs, lam, 0.5, pool0[pg][None].astype(np.float32))
        np.testing.assert_allclose(np.stack([h[3] for h in hist[n]]), of[0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(pool[pg], sf[0], rtol=1e-12, atol=1e-12)
    for pg in (0, 2, 5):
        np.testing.assert_array_equal(pool[pg], pool0[pg])
    with pytest.raises(ValueError):
        O.gla_decode_pool(q, k, v, lam, pool, np.array([1, 1, -1, -1]))


def test_varlen_equals_separate_calls_and_empty_sequences():
    rng = np.random.default_rng(9)
    lens = [5, 0, 17, 1, 0]
    H, dk, dv = 2, 4, 3
    cu = np.concatenate([[0], np.cumsum(lens)])
    tot = cu[-1]
    q, k, v = _rand(rng, (tot, H, dk)), _rand(rng, (tot, H, dk)), _rand(rng, (tot, H, dv))
    s0 = _rand(rng, (len(lens), H, dk, dv))
    lam = np.array([0.9, 0.6], np.float32)
    o, sf = O.gla_varlen(cu, q, k, v, lam, 1.0, s0)
    for n, L in enumerate(lens):
        a, b = cu[n], cu[n + 1]
        if L == 0:
            np.testing.assert_array_equal(sf[n], s0[n].astype(np.float64))
            continue
        on, sn = O.gla_fwd(q[None, a:b], k[None, a:b], v[None, a:b], lam, 1.0, s0[n:n + 1])
        np.testing.assert_array_equal(o[a:b], on[0])
        np.testing.assert_array_equal(sf[n], sn[0])


# ---------------------------------------------------------------------------
# closed forms at long range
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("lam", [0.96875, 0.999755859375, 1.0])
def test_constant_tokens_geometric_series(lam):
    """k_t = k, v_t = v, S0 = 0: S_t = (sum_{n<=t} lam^n) k^T v, so
    o_t = (q_t . k) * (1 - lam^(t+1)) / (1 - lam) * v   (t+1 terms when lam=1)."""
    rng = np.random.default_rng(12)
    T, dk, dv = 4096, 4, 3
    kk, vv = _rand(rng, (dk,), 0.5), _rand(rng, (dv,))
    q = _rand(rng, (T, 1, dk), 0.5)
    k = np.broadcast_to(kk, (T, 1, dk)).copy()
    v = np.broadcast_to(vv, (T, 1, dv)).copy()
    o, sf = O.gla_fwd(q[None], k[None], v[None], [lam])
    t = np.arange(T, dtype=np.float64)
    lam64 = float(np.float32(lam))
    geo = (t + 1) if lam64 == 1.0 else (1 - lam64 ** (t + 1)) / (1 - lam64)
    ref = (q[:, 0].astype(np.float64) @ kk.astype(np.float64))[:, None] * geo[:, None] * vv
    assert np.max(np.abs(o[0, :, 0] - ref)) <= 1e-10 * np.max(np.abs(ref))
    np.testing.assert_allclose(sf[0, 0], geo[-1] * np.outer(kk.astype(np.float64), vv), rtol=1e-10, atol=0)


def test_decay_only():
    """v = 0: S_T = lam^T S0 and o_t = lam^(t+1) q_t S0."""
    rng = np.random.default_rng(13)
    T, H, dk, dv = 2000, 2, 5, 6
    q, k = _rand(rng, (1, T, H, dk)), _rand(rng, (1, T, H, dk))
    v = np.zeros((1, T, H, dv), np.float32)
    s0 = _rand(rng, (1, H, dk, dv))
    lam = np.array([0.999, 0.99], np.float32)
    o, sf = O.gla_fwd(q, k, v, lam, 1.0, s0)
    for h in range(H):
        lh = float(lam[h])
        S0 = s0[0, h].astype(np.float64)
        ref = (lh ** (np.arange(T) + 1.0))[:, None] * (q[0, :, h].astype(np.float64) @ S0)
        assert np.max(np.abs(o[0, :, h] - ref)) <= 1e-11 * np.max(np.abs(ref))
        np.testing.assert_allclose(sf[0, h], lh ** T * S0, rtol=1e-11)


# ---------------------------------------------------------------------------
# structure: linearity, permutation, causality
# ---------------------------------------------------------------------------
def test_linearity_in_v_and_state_and_q():
    rng = np.random.default_rng(14)
    T, H, dk, dv = 33, 2, 4, 5
    grid = lambda shape: (rng.integers(-16, 17, shape) / 8).astype(np.float32)  # noqa: E731
    q, k = grid((1, T, H, dk)), grid((1, T, H, dk))
    v1, v2 = grid((1, T, H, dv)), grid((1, T, H, dv))
    s1, s2 = grid((1, H, dk, dv)), grid((1, H, dk, dv))
    lam = np.array([0.75, 0.5], np.float32)
    oa, sa = O.gla_fwd(q, k, v1, lam, 1.0, s1)
    ob, sb = O.gla_fwd(q, k, v2, lam, 1.0, s2)
    oc, sc = O.gla_fwd(q, k, 2 * v1 - 3 * v2, lam, 1.0, 2 * s1 - 3 * s2)
    tol = 1e-12 * max(np.max(np.abs(oc)), 1)
    assert np.max(np.abs(oc - (2 * oa - 3 * ob))) <= tol
    assert np.max(np.abs(sc - (2 * sa - 3 * sb))) <= 1e-12 * max(np.max(np.abs(sc)), 1)
    od, _ = O.gla_fwd(-2 * q, k, v1, lam, 1.0, s1)
    assert np.max(np.abs(od + 2 * oa)) <= tol


def test_head_permutation_and_batch_independence():
    rng = np.random.default_rng(15)
    B, T, H, dk, dv = 3, 20, 4, 3, 5
    q, k, v = _rand(rng, (B, T, H, dk)), _rand(rng, (B, T, H, dk)), _rand(rng, (B, T, H, dv))
    s0 = _rand(rng, (B, H, dk, dv))
    lam = np.array([0.5, 0.9, 0.99, 1.0], np.float32)
    o, sf = O.gla_fwd(q, k, v, lam, 1.0, s0)
    p = np.array([2, 0, 3, 1])
    op, sp = O.gla_fwd(q[:, :, p], k[:, :, p], v[:, :, p], lam[p], 1.0, s0[:, p])
    np.testing.assert_array_equal(op, o[:, :, p])
    np.testing.assert_array_equal(sp, sf[:, p])
    o1, s1 = O.gla_fwd(q[1:2], k[1:2], v[1:2], lam, 1.0, s0[1:2])
    np.testing.assert_array_equal(o1[0], o[1])
    np.testing.assert_array_equal(s1[0], sf[1])


def test_causality_future_tokens_do_not_leak():
    """Changing, or NaN-filling, tokens after t0 leaves outputs up to t0
    bit-identical and finite."""
    rng = np.random.default_rng(16)
    T, H, dk, dv, t0 = 40, 2, 4, 4, 23
    q, k, v = _rand(rng, (1, T, H, dk)), _rand(rng, (1, T, H, dk)), _rand(rng, (1, T, H, dv))
    lam = np.array([0.9, 0.6], np.float32)
    o, _ = O.gla_fwd(q, k, v, lam)
    for fill in (np.nan, 1e3):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        q2[:, t0 + 1:] = fill
        k2[:, t0 + 1:] = fill
        v2[:, t0 + 1:] = fill
        o2, _ = O.gla_fwd(q2, k2, v2, lam)
        np.testing.assert_array_equal(o2[:, :t0 + 1], o[:, :t0 + 1])
        assert np.isfinite(o2[:, :t0 + 1]).all()


# ---------------------------------------------------------------------------
# the shared input generator (storage rounding only)
# ---------------------------------------------------------------------------
def test_bf16_rounding_is_round_to_nearest_even():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 0.1, 3.0e38], np.float32)
    b = W.bf16_bits(x)
    assert b[0] == 0x3F80 and b[1] == 0x3F80          # tie -> even
    assert W.bf16_to_f32(b)[2] == np.float32(1 + 2 ** -6)  # tie -> even (up)
    assert W.bf16_to_f32(b)[3] == np.float32(-2.5)
    np.testing.assert_array_equal(O.widen(b), W.bf16_to_f32(b))
    import torch
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, tb)
    assert np.isnan(W.bf16_to_f32(W.bf16_bits(np.array([np.nan], np.float32)))).all()


def test_generators_are_seeded_and_shaped():
    a = W.spec_inputs("tiny_fp32")
    b = W.spec_inputs("tiny_fp32")
    np.testing.assert_array_equal(a["q"], b["q"])
    assert a["q"].shape == (1, 256, 2, 16) and a["v"].shape == (1, 256, 2, 32)
    assert a["q"].dtype == np.float32 and a["s0"] is None
    np.testing.assert_array_equal(a["decay"], np.array([0.875, 0.9375], np.float32))
    lam = W.geometric_decays(16)
    assert lam[0] == np.float32(0.96875) and lam[-1] == np.float32(1 - 2 ** -12)
    assert np.all(np.diff(lam) > 0)
    x = W.varlen_inputs(5, 6, 100, 2, 16, 32)
    assert x["cu_seqlens"][0] == 0 and x["cu_seqlens"][-1] == x["q"].shape[0]
    assert x["q"].dtype == np.uint16 and (x["lengths"] >= 1).all() and (x["lengths"] <= 100).all()
    s1 = W.decode_tokens(4, 3, 2, 2, 16, 32)
    s2 = W.decode_tokens(4, 3, 2, 2, 16, 32)
    np.testing.assert_array_equal(s1[2], s2[2])
