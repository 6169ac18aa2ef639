"""Pins of the PLE conv / grouped RMSNorm oracle — no GPU.

The convolution is pinned to torch.nn.functional.conv1d (depthwise, dilated,
left zero padding) in fp64 on the CPU and to the pure-shift closed form of a
one-hot kernel; the halo form to the full-sequence result (context-parallel
shards); backwards to finite differences and to autograd of the library
convolution.  The norm is pinned to its invariants (unit RMS, scale and sign
symmetry, the constant-group closed form) and its backward to finite
differences."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ple_ref as P


def conv_library(x, w, bias, dilation):
    B, S, C = x.shape
    K = w.shape[1]
    xt = torch.from_numpy(x).permute(0, 2, 1)
    xt = F.pad(xt, ((K - 1) * dilation, 0))
    y = F.conv1d(xt, torch.from_numpy(w).reshape(C, 1, K), None if bias is None else torch.from_numpy(bias),
                 dilation=dilation, groups=C)
    return y.permute(0, 2, 1).numpy()


@pytest.mark.parametrize("K,d", [(4, 3), (4, 1), (2, 5), (1, 3)])
def test_conv_equals_library(K, d):
    rng = np.random.default_rng(K * 10 + d)
    x = rng.standard_normal((2, 37, 6))
    w = rng.standard_normal((6, K))
    b = rng.standard_normal(6)
    np.testing.assert_allclose(P.short_conv(x, w, b, d), conv_library(x, w, b, d), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(P.short_conv(x, w, None, d), conv_library(x, w, None, d), rtol=1e-12, atol=1e-12)


def test_one_hot_kernel_is_a_shift():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 20, 4))
    for k in range(4):
        w = np.zeros((4, 4))
        w[:, k] = 1.0
        back = (4 - 1 - k) * 3
        expect = np.zeros_like(x)
        expect[:, back:] = x[:, :20 - back]
        assert np.array_equal(P.short_conv(x, w, None, 3), expect)


def test_zero_start_gives_bias():
    x = np.random.default_rng(2).standard_normal((2, 5, 3))
    assert np.array_equal(P.short_conv(x, np.zeros((3, 4)), np.array([1.0, -2.0, 0.5])),
                          np.broadcast_to([1.0, -2.0, 0.5], x.shape))


def test_halo_reproduces_full_sequence():
    """A shard [t0, t1) with the nine preceding tokens as halo equals the full result."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 50, 5))
    w = rng.standard_normal((5, 4))
    full = P.short_conv(x, w, None, 3)
    for t0 in (9, 10, 23):
        part = P.short_conv(x[:, t0:40], w, None, 3, halo=x[:, t0 - 9:t0])
        np.testing.assert_allclose(part, full[:, t0:40], rtol=1e-13, atol=1e-13)


def numeric_grad(f, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        hi = f(x)
        x[i] = old - eps
        lo = f(x)
        x[i] = old
        g[i] = (hi - lo) / (2 * eps)
    return g


def test_conv_backward_finite_differences_and_autograd():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 13, 3))
    w = rng.standard_normal((3, 4))
    halo = rng.standard_normal((2, 9, 3))
    dy = rng.standard_normal((2, 13, 3))
    dx, dw, db, dh = P.short_conv_backward(x, dy, w, 3, halo)
    loss = lambda xx: float((P.short_conv(xx, w, None, 3, halo) * dy).sum())
    np.testing.assert_allclose(dx, numeric_grad(loss, x.copy()), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(dw, numeric_grad(lambda ww: float((P.short_conv(x, ww, None, 3, halo) * dy).sum()),
                                                w.copy()), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(dh, numeric_grad(lambda hh: float((P.short_conv(x, w, None, 3, hh) * dy).sum()),
                                                halo.copy()), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(db, dy.sum(axis=(0, 1)), rtol=1e-12)
    # autograd of the library convolution (zero history)
    xt = torch.from_numpy(x).requires_grad_()
    wt = torch.from_numpy(w).requires_grad_()
    y = F.conv1d(F.pad(xt.permute(0, 2, 1), (9, 0)), wt.reshape(3, 1, 4), dilation=3, groups=3).permute(0, 2, 1)
    (y * torch.from_numpy(dy)).sum().backward()
    dx0, dw0, _, _ = P.short_conv_backward(x, dy, w, 3)
    np.testing.assert_allclose(dx0, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw0, wt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_norm_invariants():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 12)) * 3
    zero = np.zeros(12)
    y = P.grouped_rms_norm(x, zero, 4, eps=0.0)
    rms = np.sqrt((y.reshape(7, 3, 4) ** 2).mean(axis=-1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-13)
    np.testing.assert_allclose(P.grouped_rms_norm(5.0 * x, zero, 4, eps=0.0), y, rtol=1e-13)
    np.testing.assert_allclose(P.grouped_rms_norm(-x, zero, 4), -P.grouped_rms_norm(x, zero, 4), rtol=1e-15)
    w = rng.standard_normal(12)
    a = np.full((1, 12), 0.25)
    expect = 0.25 / np.sqrt(0.0625 + 1e-6) * (1 + w)
    np.testing.assert_allclose(P.grouped_rms_norm(a, w, 4)[0], expect, rtol=1e-14)
    # groups are independent: changing one group leaves the others
    x2 = x.copy()
    x2[:, 4:8] *= 10
    np.testing.assert_allclose(P.grouped_rms_norm(x2, w, 4)[:, :4], P.grouped_rms_norm(x, w, 4)[:, :4], rtol=1e-15)


def test_norm_backward_finite_differences():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 8))
    w = rng.standard_normal(8)
    dy = rng.standard_normal((3, 8))
    dx, dw = P.grouped_rms_norm_backward(x, dy, w, 4, eps=1e-3)
    np.testing.assert_allclose(dx, numeric_grad(lambda xx: float((P.grouped_rms_norm(xx, w, 4, 1e-3) * dy).sum()),
                                                x.copy()), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dw, numeric_grad(lambda ww: float((P.grouped_rms_norm(x, ww, 4, 1e-3) * dy).sum()),
                                                w.copy()), rtol=1e-6, atol=1e-8)
