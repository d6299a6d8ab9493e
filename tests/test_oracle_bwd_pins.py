"""Pins for the oracle's backward of the depthwise 1-D convolution (CPU only).

The backward pass of the (batch, steps, channels) depthwise conv is the next step
the speechbrain issue #2733 thread takes (its author's follow-up comments).  The
oracle writes the chain-rule sums out; none of these tests retype them.  They
check the oracle against:

* the adjoint identities of a linear map, using the (separately pinned) forward
  oracle: <conv(x; w), dy> = <x, dx(dy; w)> and <conv(x; w), dy> = <w, dw(x, dy)>;
* torch's CPU autograd of F.conv1d in float64 (the library route);
* closed forms: the bias gradient is the sum of dy over batch and steps; for stride
  1 the input gradient is the forward conv of dy with the filter reversed and
  padding (K-1)*d - p; a 1-tap filter makes both gradients elementwise.
"""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GEOMS = [  # B, T, C, K, stride, pad, dilation
    (2, 13, 3, 3, 1, 1, 1),
    (1, 20, 4, 5, 2, 2, 1),
    (2, 17, 2, 3, 2, 0, 2),
    (1, 9, 3, 4, 1, 3, 1),      # even K, asymmetric reach
    (3, 31, 2, 31, 1, 15, 1),   # the Conformer filter length
    (2, 5, 2, 7, 1, 3, 1),      # sequence shorter than the filter
    (1, 40, 2, 5, 3, 4, 2),     # stride 3 with dilation
]


def _inputs(seed, B, T, C, K, s, p, d):
    rng = np.random.default_rng(seed)
    To = oracle.out_len(T, K, s, p, d)
    return rng.standard_normal((B, T, C)), rng.standard_normal((C, 1, K)), rng.standard_normal((B, To, C))


@pytest.mark.parametrize("gi", range(len(GEOMS)))
def test_bwd_data_is_the_adjoint_of_forward(gi):
    B, T, C, K, s, p, d = GEOMS[gi]
    x, w, dy = _inputs(100 + gi, B, T, C, K, s, p, d)
    y = oracle.dwconv1d_btc(x, w, None, s, p, d)
    dx = oracle.dwconv1d_btc_bwd_data(dy, w, T, s, p, d)
    lhs, rhs = float((y * dy).sum()), float((x * dx).sum())
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs))


@pytest.mark.parametrize("gi", range(len(GEOMS)))
def test_bwd_filter_is_the_adjoint_of_forward_in_w(gi):
    B, T, C, K, s, p, d = GEOMS[gi]
    x, w, dy = _inputs(200 + gi, B, T, C, K, s, p, d)
    y = oracle.dwconv1d_btc(x, w, None, s, p, d)
    dw, _ = oracle.dwconv1d_btc_bwd_filter(x, dy, K, s, p, d)
    lhs, rhs = float((y * dy).sum()), float((w * dw).sum())
    assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(lhs))


@pytest.mark.parametrize("gi", range(len(GEOMS)))
def test_bwd_matches_torch_autograd(gi):
    B, T, C, K, s, p, d = GEOMS[gi]
    x, w, dy = _inputs(300 + gi, B, T, C, K, s, p, d)
    b = np.random.default_rng(400 + gi).standard_normal(C)
    xt = torch.tensor(x.transpose(0, 2, 1).copy(), requires_grad=True)    # (B, C, T)
    wt = torch.tensor(w, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    yt = F.conv1d(xt, wt, bt, stride=s, padding=p, dilation=d, groups=C)
    yt.backward(torch.tensor(dy.transpose(0, 2, 1).copy()))
    dx = oracle.dwconv1d_btc_bwd_data(dy, w, T, s, p, d)
    dw, db = oracle.dwconv1d_btc_bwd_filter(x, dy, K, s, p, d)
    np.testing.assert_allclose(dx, xt.grad.numpy().transpose(0, 2, 1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=0, atol=1e-11)


def test_bias_gradient_is_the_sum_of_dy():
    x, w, dy = _inputs(7, 3, 12, 4, 3, 1, 1, 1)
    _, db = oracle.dwconv1d_btc_bwd_filter(x, dy, 3, 1, 1, 1)
    np.testing.assert_allclose(db, dy.sum(axis=(0, 1)), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("K,p,d", [(3, 1, 1), (31, 15, 1), (5, 0, 1), (3, 2, 2), (4, 1, 1)])
def test_stride1_bwd_data_is_forward_with_reversed_filter(K, p, d):
    B, T, C = 2, 23, 3
    x, w, dy = _inputs(500 + K + p, B, T, C, K, 1, p, d)
    dx = oracle.dwconv1d_btc_bwd_data(dy, w, T, 1, p, d)
    ref = oracle.dwconv1d_btc(dy, w[:, :, ::-1], None, 1, (K - 1) * d - p, d)
    assert ref.shape == dx.shape
    np.testing.assert_allclose(dx, ref, rtol=0, atol=1e-13)


def test_one_tap_filter_is_elementwise():
    x, w, dy = _inputs(9, 2, 11, 5, 1, 1, 0, 1)
    dx = oracle.dwconv1d_btc_bwd_data(dy, w, 11, 1, 0, 1)
    dw, _ = oracle.dwconv1d_btc_bwd_filter(x, dy, 1, 1, 0, 1)
    np.testing.assert_allclose(dx, dy * w[:, 0, 0], rtol=1e-15, atol=0)
    np.testing.assert_allclose(dw[:, 0, 0], (dy * x).sum(axis=(0, 1)), rtol=1e-13, atol=1e-13)


def test_bwd_data_at_equals_full():
    B, T, C, K, s, p, d = 2, 19, 3, 5, 2, 2, 1
    x, w, dy = _inputs(11, B, T, C, K, s, p, d)
    dx = oracle.dwconv1d_btc_bwd_data(dy, w, T, s, p, d)
    idx = np.arange(dx.size)
    np.testing.assert_array_equal(oracle.dwconv1d_btc_bwd_data_at(dy, w, T, idx, s, p, d), dx.ravel())


def test_bwd_invalid_arguments_raise():
    x, w, dy = _inputs(12, 1, 8, 2, 3, 1, 1, 1)
    with pytest.raises(ValueError):
        oracle.dwconv1d_btc_bwd_data(dy, w, 9, 1, 1, 1)      # dy length does not match T
    with pytest.raises(ValueError):
        oracle.dwconv1d_btc_bwd_filter(x, dy[:, :-1], 3, 1, 1, 1)
