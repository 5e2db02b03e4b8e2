"""Pins of the oracle's short causal convolution + SiLU (CPU only).

The layer in front of the mixer (Laplace 3B / Trainium2 page, section on
normalisation and convolution: a causal, per-channel Conv1d of width 4 with
SiLU). Pinned against library routines and its own structure:

* numpy.convolve per channel (the library's discrete convolution) on the
  history-padded input, and scipy.special.expit for the sigmoid of SiLU;
* a single tap on the current token reduces to SiLU of the input;
* decode steps equal the prefill token by token, and split invariance with
  the window carried between calls.
"""
import numpy as np
from scipy.special import expit

from oracle import oracle as O


def _case(seed, B=2, T=23, D=40, K=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, T, D)).astype(np.float32)
    w = rng.standard_normal((D, K))
    b = rng.standard_normal(D)
    win = rng.standard_normal((B, K, D))
    return x, w, b, win


def test_matches_numpy_convolve_and_expit():
    x, w, b, win = _case(1)
    B, T, D = x.shape
    K = w.shape[1]
    y, wout = O.short_conv(x, w, b, win)
    for n in range(B):
        for c in range(D):
            seq = np.concatenate([win[n, :, c], x[n, :, c].astype(np.float64)])
            # 'valid' convolution with the reversed taps: sum_j w[j] seq[t + 1 + j]
            z = np.convolve(seq[1:], w[c][::-1], mode="valid") + b[c]
            np.testing.assert_allclose(y[n, :, c], z * expit(z), rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(wout[n], np.concatenate(
            [win[n], x[n].astype(np.float64)])[-K:])


def test_single_current_tap_is_silu():
    x, w, _, _ = _case(2)
    w = np.zeros_like(w)
    w[:, -1] = 1.0
    y, _ = O.short_conv(x, w)
    xf = x.astype(np.float64)
    np.testing.assert_allclose(y, xf * expit(xf), rtol=1e-13, atol=1e-15)
    assert O.short_conv(np.zeros((1, 3, 5), np.float32), w[:5])[0].sum() == 0.0


def test_decode_steps_equal_prefill_and_split_invariance():
    x, w, b, win = _case(3)
    y, wout = O.short_conv(x, w, b, win)
    state = win.copy()
    for t in range(x.shape[1]):
        yt = O.short_conv_decode(x[:, t], w, b, state)
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(state, wout)
    for t1 in (1, 3, 4, 10):
        ya, wa = O.short_conv(x[:, :t1], w, b, win)
        yb, wb = O.short_conv(x[:, t1:], w, b, wa)
        np.testing.assert_allclose(np.concatenate([ya, yb], axis=1), y, rtol=1e-13, atol=1e-13)
        np.testing.assert_array_equal(wb, wout)
