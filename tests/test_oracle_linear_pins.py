"""Pins of the oracle's normalised causal linear attention (CPU only).

The oracle runs the recurrence of the tutorial page on RNNs without
recurrence (section 6.1: S_t = S_{t-1} + phi(k_t)^T v_t, z_t = z_{t-1} +
phi(k_t), o_t = phi(q_t) S_t / (phi(q_t) . z_t + eps), phi = ReLU, eps = 1e-6
from the demonstration module of section 6.2) token by token. Pinned against
things other than itself:

* the page's own parallel form: prefix sums (numpy.cumsum) of the per-token
  outer products and keys, contracted with the queries;
* the attention form the page derives it from: o_t is a weighted mean of
  v_1..v_t with kernel weights w_tj = phi(q_t) . phi(k_j), an O(T^2) matrix
  product with a lower-triangular mask;
* the already pinned Simple GLA oracle (C, token by token) at lambda = 1 and
  scale 1 on phi(q), phi(k): the numerator with v, the denominator with a
  value column of ones;
* closed forms: one token, constant values, non-positive queries;
* split invariance with (S, z) carried between calls.
"""
import numpy as np

from oracle import oracle as O

EPS = 1e-6


def _case(seed, B=2, T=19, H=3, dk=8, dv=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    return q, k, v


def test_matches_prefix_sum_form():
    q, k, v = _case(1)
    o, S, z = O.linear_attention(q, k, v)
    fq = np.maximum(q.astype(np.float64), 0)
    fk = np.maximum(k.astype(np.float64), 0)
    kv = fk[..., :, None] * v.astype(np.float64)[..., None, :]   # [B,T,H,dk,dv]
    kv_cum = np.cumsum(kv, axis=1)
    k_cum = np.cumsum(fk, axis=1)
    num = (fq[..., :, None] * kv_cum).sum(axis=3)
    den = (fq * k_cum).sum(axis=3) + EPS
    np.testing.assert_allclose(o, num / den[..., None], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S, kv_cum[:, -1], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(z, k_cum[:, -1], rtol=1e-13, atol=1e-13)


def test_matches_masked_kernel_attention():
    q, k, v = _case(2, B=1, T=31, H=2)
    o, _, _ = O.linear_attention(q, k, v)
    for h in range(q.shape[2]):
        fq = np.maximum(q[0, :, h].astype(np.float64), 0)
        fk = np.maximum(k[0, :, h].astype(np.float64), 0)
        W = np.tril(fq @ fk.T)                       # w_tj, j <= t
        ref = (W @ v[0, :, h].astype(np.float64)) / (W.sum(axis=1) + EPS)[:, None]
        np.testing.assert_allclose(o[0, :, h], ref, rtol=1e-12, atol=1e-13)


def test_numerator_and_denominator_are_simple_gla_at_unit_decay():
    q, k, v = _case(3)
    B, T, H, dk = q.shape
    rng = np.random.default_rng(33)
    s0 = rng.standard_normal((B, H, dk, v.shape[3]))
    z0 = np.abs(rng.standard_normal((B, H, dk)))
    o, S, z = O.linear_attention(q, k, v, s0, z0)
    fq = np.maximum(q, 0).astype(np.float32)
    fk = np.maximum(k, 0).astype(np.float32)
    one = np.ones(H, np.float32)
    num, s_num = O.gla_fwd(fq, fk, v, one, 1.0, s0)
    den, s_den = O.gla_fwd(fq, fk, np.ones((B, T, H, 1), np.float32), one, 1.0,
                           z0[..., None])
    np.testing.assert_allclose(o, num / (den + EPS), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, s_num, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, s_den[..., 0], rtol=1e-12, atol=1e-12)


def test_single_token_closed_form_and_eps():
    # tiny features so that eps is a visible part of the denominator
    q = np.full((1, 1, 1, 4), 1e-3, np.float32)
    k = np.full((1, 1, 1, 4), 5e-4, np.float32)
    k[..., 1] = -2.0                                  # phi drops it
    v = np.array([[[[3.0, -1.0]]]], np.float32)
    o, S, z = O.linear_attention(q, k, v)
    a = 3 * np.float64(np.float32(1e-3)) * np.float64(np.float32(5e-4))
    np.testing.assert_allclose(o[0, 0, 0], a / (a + EPS) * np.array([3.0, -1.0]), rtol=1e-14)
    np.testing.assert_array_equal(z[0, 0], np.float64(np.float32(5e-4)) * np.array([1, 0, 1, 1]))


def test_constant_values_and_nonpositive_queries():
    q, k, _ = _case(4)
    c = np.array([0.5, -2.0, 4.0], np.float32)
    v = np.broadcast_to(c, q.shape[:3] + (3,)).copy()
    o, _, z = O.linear_attention(q, k, v)
    fq = np.maximum(q.astype(np.float64), 0)
    a = (fq * np.cumsum(np.maximum(k.astype(np.float64), 0), axis=1)).sum(axis=3)
    np.testing.assert_allclose(o, (a / (a + EPS))[..., None] * c, rtol=1e-13, atol=1e-14)
    o2, _, _ = O.linear_attention(-np.abs(q), k, v)
    assert np.all(o2 == 0.0)


def test_split_invariance():
    q, k, v = _case(5, T=40)
    o, S, z = O.linear_attention(q, k, v)
    o1, S1, z1 = O.linear_attention(q[:, :17], k[:, :17], v[:, :17])
    o2, S2, z2 = O.linear_attention(q[:, 17:], k[:, 17:], v[:, 17:], S1, z1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S2, S, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(z2, z, rtol=1e-13, atol=1e-13)


def test_bf16_bits_widen_exactly():
    q, k, v = _case(6, T=7)
    bits = [(x.view(np.uint32) >> 16).astype(np.uint16) for x in (q, k, v)]
    vals = [(b.astype(np.uint32) << 16).view(np.float32) for b in bits]
    np.testing.assert_array_equal(O.linear_attention(*bits)[0], O.linear_attention(*vals)[0])
