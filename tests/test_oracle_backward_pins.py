"""Pins of the oracle's backward (CPU only).

The backward is the chain rule through the recurrence S_t = lambda S_{t-1} +
k_t^T v_t, o_t = scale * q_t S_t (Laplace 3B / Trainium2 page, sections "GLA
mixer" and "Challenge 3": training differentiates through every sequential
state update). It is pinned against things other than itself:

* central finite differences of the oracle FORWARD (itself pinned in
  test_oracle_pins.py). The loss sum(W_o * o) + sum(W_s * S_final) is linear
  in every single input element (o and S_final are multilinear in q, k, v,
  S0), and the inputs and steps are exact binary fractions, so the central
  difference equals the derivative up to fp64 rounding: a tight pin;
* the gradients of the O(T^2) masked form
      o_t = scale * (sum_{u<=t} lambda^(t-u) (q_t . k_u) v_u + lambda^(t+1) q_t S0),
      S_final = lambda^T S0 + sum_u lambda^(T-1-u) k_u^T v_u,
  derived by hand as matrix products over the decay-masked score matrices
  (a different derivation from the oracle's reverse sweep);
* T = 0 and varlen = separate calls.
"""
import numpy as np
import pytest

from oracle import oracle as O


def _dyadic(rng, shape, bits=8):
    """Values that are exact binary fractions (k / 2^bits), so x +- 2^-bits
    is exact in fp32."""
    return (rng.integers(-2 ** bits, 2 ** bits, size=shape) / 2.0 ** bits).astype(np.float32)


def _loss(q, k, v, s0, lam, scale, Wo, Ws):
    o, sf = O.gla_fwd(q, k, v, lam, scale, s0)
    return float(np.sum(Wo * o) + np.sum(Ws * sf))


def test_backward_equals_central_differences_of_the_forward():
    rng = np.random.default_rng(30)
    B, T, H, dk, dv = 2, 7, 2, 3, 4
    q, k, v = _dyadic(rng, (B, T, H, dk)), _dyadic(rng, (B, T, H, dk)), _dyadic(rng, (B, T, H, dv))
    s0 = _dyadic(rng, (B, H, dk, dv))
    lam = np.array([0.75, 0.9375], np.float32)   # exact binary fractions
    scale = 0.625
    Wo = _dyadic(rng, (B, T, H, dv)).astype(np.float64)
    Ws = _dyadic(rng, (B, H, dk, dv)).astype(np.float64)
    dq, dk_, dv_, ds0 = O.gla_bwd(q, k, v, lam, Wo.astype(np.float32), scale, s0,
                                  Ws.astype(np.float32))
    eps = np.float32(2.0 ** -8)
    args = {"q": q, "k": k, "v": v, "s0": s0}
    grads = {"q": dq, "k": dk_, "v": dv_, "s0": ds0}
    worst = 0.0
    for name, x in args.items():
        g = grads[name]
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            a = dict(args)
            a[name] = xp
            lp = _loss(a["q"], a["k"], a["v"], a["s0"], lam, scale, Wo, Ws)
            a[name] = xm
            lm = _loss(a["q"], a["k"], a["v"], a["s0"], lam, scale, Wo, Ws)
            fd = (lp - lm) / (2.0 * float(eps))
            worst = max(worst, abs(fd - g[idx]))
    assert worst < 1e-9, worst


def _masked_form_grads(q, k, v, s0, lam, scale, dO, dSf):
    """Gradients of the O(T^2) masked form of one (sequence, head) chain,
    as matrix products: A = (Q K^T) * D, Bm = (dO V^T) * D with
    D[t, u] = lam^(t-u) for t >= u."""
    T = q.shape[0]
    t = np.arange(T)
    D = np.where(t[:, None] >= t[None, :], float(lam) ** (t[:, None] - t[None, :]).clip(0), 0.0)
    A = (q @ k.T) * D
    Bm = (dO @ v.T) * D
    lt1 = float(lam) ** (t + 1.0)
    lrev = float(lam) ** (T - 1.0 - t)
    dq = scale * (Bm @ k) + scale * lt1[:, None] * (dO @ s0.T)
    dk = scale * (Bm.T @ q) + lrev[:, None] * (v @ dSf.T)
    dv = scale * (A.T @ dO) + lrev[:, None] * (k @ dSf)
    ds0 = scale * (q * lt1[:, None]).T @ dO + float(lam) ** T * dSf
    return dq, dk, dv, ds0


@pytest.mark.parametrize("T", [1, 5, 33])
def test_backward_equals_masked_form_gradients(T):
    rng = np.random.default_rng(31 + T)
    H, dk, dv = 2, 6, 5
    q = rng.standard_normal((1, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((1, T, H, dk)).astype(np.float32)
    v = rng.standard_normal((1, T, H, dv)).astype(np.float32)
    dO = rng.standard_normal((1, T, H, dv)).astype(np.float32)
    s0 = rng.standard_normal((1, H, dk, dv)).astype(np.float32)
    dSf = rng.standard_normal((1, H, dk, dv)).astype(np.float32)
    lam = np.array([0.8, 1.0], np.float32)
    scale = 0.3
    dq, dk_, dv_, ds0 = O.gla_bwd(q, k, v, lam, dO, scale, s0, dSf)
    for h in range(H):
        f64 = lambda a: a.astype(np.float64)
        r = _masked_form_grads(f64(q[0, :, h]), f64(k[0, :, h]), f64(v[0, :, h]),
                               f64(s0[0, h]), lam[h], scale, f64(dO[0, :, h]), f64(dSf[0, h]))
        for got, ref in zip((dq[0, :, h], dk_[0, :, h], dv_[0, :, h], ds0[0, h]), r):
            np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


def test_backward_without_final_gradient_and_initial_state():
    """ds_final None is zero and s0 None is zero: equal to passing zeros."""
    rng = np.random.default_rng(32)
    T, H, dk, dv = 9, 1, 4, 3
    q, k = rng.standard_normal((1, T, H, dk)), rng.standard_normal((1, T, H, dk))
    v, dO = rng.standard_normal((1, T, H, dv)), rng.standard_normal((1, T, H, dv))
    q, k, v, dO = (a.astype(np.float32) for a in (q, k, v, dO))
    lam = np.array([0.9], np.float32)
    a = O.gla_bwd(q, k, v, lam, dO)
    z = np.zeros((1, H, dk, dv), np.float32)
    b = O.gla_bwd(q, k, v, lam, dO, 1.0, z, z)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_backward_varlen_equals_separate_calls_and_empty_sequences():
    rng = np.random.default_rng(33)
    lens = [4, 0, 11, 1]
    H, dk, dv = 2, 3, 5
    cu = np.concatenate([[0], np.cumsum(lens)])
    tot = int(cu[-1])
    q, k = rng.standard_normal((tot, H, dk)), rng.standard_normal((tot, H, dk))
    v, dO = rng.standard_normal((tot, H, dv)), rng.standard_normal((tot, H, dv))
    q, k, v, dO = (a.astype(np.float32) for a in (q, k, v, dO))
    s0 = rng.standard_normal((len(lens), H, dk, dv)).astype(np.float32)
    dsf = rng.standard_normal((len(lens), H, dk, dv)).astype(np.float32)
    lam = np.array([0.7, 0.99], np.float32)
    dq, dk_, dv_, ds0 = O.gla_bwd_varlen(cu, q, k, v, lam, dO, 0.5, s0, dsf)
    for n, L in enumerate(lens):
        a, b = cu[n], cu[n + 1]
        r = O.gla_bwd(q[a:b][None], k[a:b][None], v[a:b][None], lam, dO[a:b][None], 0.5,
                      s0[n:n + 1], dsf[n:n + 1])
        np.testing.assert_array_equal(dq[a:b], r[0][0])
        np.testing.assert_array_equal(dk_[a:b], r[1][0])
        np.testing.assert_array_equal(dv_[a:b], r[2][0])
        np.testing.assert_array_equal(ds0[n], r[3][0])
        if L == 0:  # no tokens: the gradient passes straight through
            np.testing.assert_array_equal(ds0[n], dsf[n].astype(np.float64))
