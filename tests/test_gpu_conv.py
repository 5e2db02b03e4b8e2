"""GPU parity of the short causal convolution + SiLU (prefill and decode)
against the fp64 oracle on seeded inputs. Bar: max|gpu - oracle| <=
1e-2 * max|oracle| for bf16, 1e-4 for fp32; windows compared exactly (they
hold input values)."""
import numpy as np
import pytest
import torch

from chunked_gated_recurrent_amd import gla
from chunked_gated_recurrent_amd import workloads as W
from oracle import oracle as O
from gla_testutil import TOL, dev, host, rel_err

pytestmark = pytest.mark.gpu


def _case(seed, B, T, D, dtype, with_bias=True, with_window=True):
    rng = np.random.default_rng(seed)
    xf = rng.standard_normal((B, T, D), dtype=np.float32)
    x = W.bf16_bits(xf) if dtype == "bf16" else xf
    w = (rng.standard_normal((D, 4)) * 0.5).astype(np.float32)
    b = (rng.standard_normal(D) * 0.1).astype(np.float32) if with_bias else None
    win = rng.standard_normal((B, 4, D)).astype(np.float32) if with_window else None
    return x, w, b, win


def _t(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [0, 1, 3, 31, 32, 33, 200])
def test_short_conv_prefill(dtype, T):
    x, w, b, win = _case(800 + T, 2, T, 3072 if dtype == "bf16" else 520, dtype)
    y, wo = gla.short_conv_fwd(dev(x), _t(w), _t(b), _t(win))
    torch.cuda.synchronize()
    ry, rwo = O.short_conv(x, w, b, win)
    e = rel_err(host(y), ry) if T else 0.0
    print("short conv %s T%d: err %.2e" % (dtype, T, e))
    assert e <= TOL[dtype]
    np.testing.assert_array_equal(host(wo), rwo)


def test_short_conv_without_bias_or_window_and_laplace_size():
    x, w, _, _ = _case(810, 8, 2048, 3072, "bf16", False, False)
    y, wo = gla.short_conv_fwd(dev(x), _t(w))
    torch.cuda.synchronize()
    ry, rwo = O.short_conv(x, w)          # every token of every channel
    assert rel_err(host(y), ry) <= TOL["bf16"]
    np.testing.assert_array_equal(host(wo), rwo)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_short_conv_decode_steps_continue_the_prefill(dtype):
    """Prefill 37 tokens, then 5 decode steps from its window: equal to the
    oracle over the whole 42 tokens."""
    D = 3072
    x, w, b, win = _case(820, 3, 42, D, dtype)
    y0, wo = gla.short_conv_fwd(dev(x[:, :37]), _t(w), _t(b), _t(win))
    ys = [host(y0)]
    for t in range(37, 42):
        ys.append(host(gla.short_conv_decode_step(dev(x[:, t]), _t(w), _t(b), wo))[:, None])
    torch.cuda.synchronize()
    ry, rwo = O.short_conv(x, w, b, win)
    assert rel_err(np.concatenate(ys, axis=1), ry) <= TOL[dtype]
    np.testing.assert_array_equal(host(wo), rwo)


@pytest.mark.parametrize("dtype,N", [("bf16", 1280), ("f32", 1280), ("bf16", 700)])
def test_short_conv_decode_full_size(dtype, N):
    """One decode step at the decode workload's width (3,072 channels) for
    1,280 sequences and a ragged 700: every sequence against the oracle
    (each thread walks several sequences of one channel group, so every row
    is checked), and the window is shifted exactly."""
    D = 3072
    rng = np.random.default_rng(830 + N)
    x = rng.standard_normal((N, D), dtype=np.float32)
    if dtype == "bf16":
        x = W.bf16_bits(x)
    w = (rng.standard_normal((D, 4)) * 0.5).astype(np.float32)
    b = (rng.standard_normal(D) * 0.1).astype(np.float32)
    win = rng.standard_normal((N, 4, D)).astype(np.float32)
    wd = _t(win)
    y = gla.short_conv_decode_step(dev(x), _t(w), _t(b), wd)
    torch.cuda.synchronize()
    rw = win.astype(np.float64)
    ry = O.short_conv_decode(x, w, b, rw)
    assert rel_err(host(y), ry) <= TOL[dtype]
    np.testing.assert_array_equal(host(wd), rw)


def test_short_conv_causality_and_determinism():
    x, w, b, win = _case(840, 2, 200, 3072, "bf16")
    y1, w1 = gla.short_conv_fwd(dev(x), _t(w), _t(b), _t(win))
    y2, w2 = gla.short_conv_fwd(dev(x), _t(w), _t(b), _t(win))
    x3 = x.copy()
    x3[:, 120:] ^= np.uint16(0x0040)          # perturb every later token
    y3, _ = gla.short_conv_fwd(dev(x3), _t(w), _t(b), _t(win))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(y1), host(y2))
    np.testing.assert_array_equal(host(w1), host(w2))
    np.testing.assert_array_equal(host(y3)[:, :120], host(y1)[:, :120])
    assert not np.array_equal(host(y3)[:, 120:], host(y1)[:, 120:])
