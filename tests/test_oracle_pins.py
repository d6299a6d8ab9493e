"""Pins for the fp64 oracle (CPU only).

The oracle is the plain definition of grouped convolution (neon issue "Grouped
convolutions", thestew42's reply: groups of channels/filters/outputs that are not
connected; F.conv2d semantics from the discuss.pytorch.org thread's test script;
depthwise (batch, steps, channels) conv from speechbrain issue #2733).  None of
these tests retype the oracle's formula: each one checks it against a library
routine (scipy, numpy, torch in float64), a structural invariant (block-diagonal
dense equivalence, per-group slicing and independence, stride = subsampling,
dilation = zero-inserted kernel, padding = explicit zero pad, linearity), or a
closed form (constant input, delta kernels, 1x1 = per-group matmul).
"""
import itertools

import numpy as np
import pytest
import scipy.signal
import torch
import torch.nn.functional as F

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def rnd(rng, *shape):
    return rng.standard_normal(shape)


def t64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


# ---------------------------------------------------------------- output size

def test_out_len_matches_enumeration():
    """Output length = number of window start positions that fit in the padded
    input, counted one by one."""
    for L, K, s, p, d in itertools.product(range(1, 11), range(1, 5), range(1, 4), range(0, 4), range(1, 4)):
        count = 0
        o = 0
        while o * s <= L + 2 * p:
            lo = o * s - p
            hi = lo + d * (K - 1)
            if lo >= -p and hi <= L + p - 1:
                count += 1
            o += 1
        assert oracle.out_len(L, K, s, p, d) == count, (L, K, s, p, d)


def test_page_workload_shape_golden():
    """The p2 layer from tests/golden: F.conv2d with padding 3//2 keeps 256x256."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_workload_shapes.json")))
    for case in g["cases"]:
        x, w = case["x_shape"], case["w_shape"]
        p = case["padding"]
        oh = oracle.out_len(x[2], w[2], 1, p, 1)
        ow = oracle.out_len(x[3], w[3], 1, p, 1)
        assert [x[0], w[0], oh, ow] == case["y_shape"]
        assert x[1] // case["groups"] == w[1]


# ---------------------------------------------------------------- dense core

@pytest.mark.parametrize("seed", range(4))
def test_g1_equals_scipy_correlate2d(seed):
    """g=1: y[n,o] = sum_ci correlate2d(pad(x[n,ci]), w[o,ci], 'valid').
    scipy.signal.correlate2d does not flip the kernel."""
    rng = np.random.default_rng(seed)
    N, C, H, W = 2, int(rng.integers(1, 5)), int(rng.integers(3, 9)), int(rng.integers(3, 9))
    Co, KH, KW = int(rng.integers(1, 5)), int(rng.integers(1, 4)), int(rng.integers(1, 4))
    p = int(rng.integers(0, 3))
    x, w = rnd(rng, N, C, H, W), rnd(rng, Co, C, KH, KW)
    y = oracle.conv2d(x, w, padding=p)
    ref = np.zeros_like(y)
    for n in range(N):
        for o in range(Co):
            for c in range(C):
                ref[n, o] += scipy.signal.correlate2d(np.pad(x[n, c], p), w[o, c], mode="valid")
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_g1_equals_sliding_window_einsum():
    rng = np.random.default_rng(11)
    x, w = rnd(rng, 2, 3, 7, 6), rnd(rng, 4, 3, 3, 2)
    y = oracle.conv2d(x, w, padding=(1, 0))
    xp = np.pad(x, ((0, 0), (0, 0), (1, 1), (0, 0)))
    win = np.lib.stride_tricks.sliding_window_view(xp, (3, 2), axis=(2, 3))  # n c oh ow kh kw
    ref = np.einsum("ncijhw,ochw->noij", win, w)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(8))
def test_matches_torch_conv2d_float64(seed):
    """Library pin: torch.nn.functional.conv2d in float64 on the CPU, with groups,
    stride, padding, dilation and bias drawn at random."""
    rng = np.random.default_rng(100 + seed)
    g = int(rng.choice([1, 2, 3, 4]))
    Cg, Ng = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    C, Co = g * Cg, g * Ng
    KH, KW = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    s = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
    d = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
    p = (int(rng.integers(0, 3)), int(rng.integers(0, 3)))
    H = int(rng.integers(d[0] * (KH - 1) + 1, 10))
    W = int(rng.integers(d[1] * (KW - 1) + 1, 10))
    x, w, b = rnd(rng, 2, C, H, W), rnd(rng, Co, Cg, KH, KW), rnd(rng, Co)
    y = oracle.conv2d(x, w, b, stride=s, padding=p, dilation=d, groups=g)
    ref = F.conv2d(t64(x), t64(w), t64(b), stride=s, padding=p, dilation=d, groups=g).numpy()
    assert y.shape == ref.shape
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_accumulates_in_fp64():
    """1e8 + 1 - 1e8 over three channels of a 1x1 kernel is 1 in fp64 and 0 in
    fp32: the oracle must keep the 1."""
    x = np.array([1e8, 1.0, -1e8]).reshape(1, 3, 1, 1)
    w = np.ones((1, 3, 1, 1))
    assert oracle.conv2d(x, w)[0, 0, 0, 0] == 1.0


# ---------------------------------------------------------------- group mapping

GROUP_CASES = [  # (N, C, Co, H, W, K, groups, pad, stride, dil)
    (2, 4, 6, 5, 6, 3, 2, 1, 1, 1),
    (1, 6, 6, 6, 5, 3, 3, 0, 2, 1),
    (2, 8, 8, 7, 7, 3, 8, 1, 1, 2),
    (1, 4, 8, 4, 4, 1, 4, 0, 1, 1),
    (1, 16, 16, 8, 8, 3, 4, 1, 1, 1),
]


@pytest.mark.parametrize("case", GROUP_CASES)
def test_block_diagonal_dense_equivalence(case):
    """Grouped conv == g=1 conv whose dense weight is zero outside the diagonal
    blocks (input block k x output block k)."""
    N, C, Co, H, W, K, g, p, s, d = case
    rng = np.random.default_rng(sum(case))
    Cg, Ng = C // g, Co // g
    x, w, b = rnd(rng, N, C, H, W), rnd(rng, Co, Cg, K, K), rnd(rng, Co)
    dense = np.zeros((Co, C, K, K))
    for k in range(g):
        dense[k * Ng:(k + 1) * Ng, k * Cg:(k + 1) * Cg] = w[k * Ng:(k + 1) * Ng]
    y = oracle.conv2d(x, w, b, stride=s, padding=p, dilation=d, groups=g)
    ref = oracle.conv2d(x, dense, b, stride=s, padding=p, dilation=d, groups=1)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("case", GROUP_CASES)
def test_per_group_slicing(case):
    """Output block k == g=1 conv of input block k with weight block k."""
    N, C, Co, H, W, K, g, p, s, d = case
    rng = np.random.default_rng(7 + sum(case))
    Cg, Ng = C // g, Co // g
    x, w, b = rnd(rng, N, C, H, W), rnd(rng, Co, Cg, K, K), rnd(rng, Co)
    y = oracle.conv2d(x, w, b, stride=s, padding=p, dilation=d, groups=g)
    for k in range(g):
        yk = oracle.conv2d(x[:, k * Cg:(k + 1) * Cg], w[k * Ng:(k + 1) * Ng], b[k * Ng:(k + 1) * Ng],
                           stride=s, padding=p, dilation=d, groups=1)
        np.testing.assert_array_equal(y[:, k * Ng:(k + 1) * Ng], yk)


@pytest.mark.parametrize("case", GROUP_CASES)
def test_per_group_independence(case):
    """Perturbing the input channels or the filters of group k changes output
    block k and leaves every other output bit-identical."""
    N, C, Co, H, W, K, g, p, s, d = case
    rng = np.random.default_rng(13 + sum(case))
    Cg, Ng = C // g, Co // g
    x, w = rnd(rng, N, C, H, W), rnd(rng, Co, Cg, K, K)
    y0 = oracle.conv2d(x, w, stride=s, padding=p, dilation=d, groups=g)
    for k in range(g):
        for which in ("x", "w"):
            x1, w1 = x.copy(), w.copy()
            if which == "x":
                x1[:, k * Cg:(k + 1) * Cg] += rnd(rng, N, Cg, H, W)
            else:
                w1[k * Ng:(k + 1) * Ng] += rnd(rng, Ng, Cg, K, K)
            y1 = oracle.conv2d(x1, w1, stride=s, padding=p, dilation=d, groups=g)
            mask = np.zeros(Co, bool)
            mask[k * Ng:(k + 1) * Ng] = True
            np.testing.assert_array_equal(y1[:, ~mask], y0[:, ~mask])
            assert np.abs(y1[:, mask] - y0[:, mask]).max() > 0


# ---------------------------------------------------------------- geometry invariants

@pytest.mark.parametrize("s", [2, 3])
def test_stride_is_subsampling(s):
    rng = np.random.default_rng(s)
    x, w = rnd(rng, 1, 4, 11, 10), rnd(rng, 4, 2, 3, 3)
    y1 = oracle.conv2d(x, w, padding=1, groups=2)
    ys = oracle.conv2d(x, w, padding=1, groups=2, stride=s)
    np.testing.assert_array_equal(ys, y1[:, :, ::s, ::s])


@pytest.mark.parametrize("d", [2, 3])
def test_dilation_is_zero_inserted_kernel(d):
    rng = np.random.default_rng(20 + d)
    x, w = rnd(rng, 2, 6, 12, 11), rnd(rng, 6, 3, 3, 2)
    KH, KW = d * 2 + 1, d * 1 + 1
    wz = np.zeros((6, 3, KH, KW))
    wz[:, :, ::d, ::d] = w
    y = oracle.conv2d(x, w, padding=(2, 1), dilation=d, groups=2)
    ref = oracle.conv2d(x, wz, padding=(2, 1), groups=2)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_padding_is_explicit_zero_pad():
    rng = np.random.default_rng(5)
    x, w, b = rnd(rng, 2, 4, 6, 7), rnd(rng, 8, 1, 3, 3), rnd(rng, 8)
    y = oracle.conv2d(x, w, b, padding=(2, 1), groups=4)
    xp = np.pad(x, ((0, 0), (0, 0), (2, 2), (1, 1)))
    np.testing.assert_array_equal(y, oracle.conv2d(xp, w, b, padding=0, groups=4))


def test_linearity_and_bias():
    rng = np.random.default_rng(6)
    x1, x2, w, b = rnd(rng, 1, 6, 5, 5), rnd(rng, 1, 6, 5, 5), rnd(rng, 9, 2, 3, 3), rnd(rng, 9)
    a1, a2 = 0.75, -1.5
    lhs = oracle.conv2d(a1 * x1 + a2 * x2, w, padding=1, groups=3)
    rhs = a1 * oracle.conv2d(x1, w, padding=1, groups=3) + a2 * oracle.conv2d(x2, w, padding=1, groups=3)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    yb = oracle.conv2d(x1, w, b, padding=1, groups=3)
    np.testing.assert_allclose(yb - b[None, :, None, None], oracle.conv2d(x1, w, padding=1, groups=3),
                               rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- closed forms

def test_constant_input_closed_form():
    """x == 1, 3x3, pad 1: interior = b + sum(w[o]); top-left corner = b + the
    sum of the lower-right 2x2 taps; top edge = b + the sum of the lower 2 rows."""
    rng = np.random.default_rng(8)
    C, Co, g = 8, 4, 2
    x = np.ones((1, C, 6, 7))
    w, b = rnd(rng, Co, C // g, 3, 3), rnd(rng, Co)
    y = oracle.conv2d(x, w, b, padding=1, groups=g)
    for o in range(Co):
        np.testing.assert_allclose(y[0, o, 1:-1, 1:-1], b[o] + w[o].sum(), rtol=1e-13)
        np.testing.assert_allclose(y[0, o, 0, 0], b[o] + w[o, :, 1:, 1:].sum(), rtol=1e-13)
        np.testing.assert_allclose(y[0, o, -1, -1], b[o] + w[o, :, :2, :2].sum(), rtol=1e-13)
        np.testing.assert_allclose(y[0, o, 0, 1:-1], b[o] + w[o, :, 1:, :].sum(), rtol=1e-13)
        np.testing.assert_allclose(y[0, o, 1:-1, -1], b[o] + w[o, :, :, :2].sum(), rtol=1e-13)


def test_delta_kernels_identity_and_shift():
    rng = np.random.default_rng(9)
    C = 6
    x = rnd(rng, 2, C, 5, 4)
    w = np.zeros((C, 1, 3, 3))
    w[:, 0, 1, 1] = 1.0                                  # centre tap: identity
    np.testing.assert_array_equal(oracle.conv2d(x, w, padding=1, groups=C), x)
    w = np.zeros((C, 1, 3, 3))
    w[:, 0, 0, 0] = 1.0                                  # top-left tap: y[i,j] = x[i-1,j-1]
    y = oracle.conv2d(x, w, padding=1, groups=C)
    ref = np.zeros_like(x)
    ref[:, :, 1:, 1:] = x[:, :, :-1, :-1]
    np.testing.assert_array_equal(y, ref)


def test_1x1_is_groupwise_matmul():
    rng = np.random.default_rng(10)
    N, C, Co, g, H, W = 2, 12, 9, 3, 4, 5
    x, w, b = rnd(rng, N, C, H, W), rnd(rng, Co, C // g, 1, 1), rnd(rng, Co)
    y = oracle.conv2d(x, w, b, groups=g)
    xs = x.reshape(N, g, C // g, H, W)
    ws = w.reshape(g, Co // g, C // g)
    ref = np.einsum("gok,ngkhw->ngohw", ws, xs).reshape(N, Co, H, W) + b[None, :, None, None]
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- 1-D depthwise, (batch, steps, channels)

def test_dw1d_equals_numpy_correlate():
    rng = np.random.default_rng(30)
    B, T, C, K, p = 2, 40, 5, 31, 15
    x, w, b = rnd(rng, B, T, C), rnd(rng, C, 1, K), rnd(rng, C)
    y = oracle.dwconv1d_btc(x, w, b, padding=p)
    for bb in range(B):
        for c in range(C):
            ref = np.correlate(np.pad(x[bb, :, c], p), w[c, 0], mode="valid") + b[c]
            np.testing.assert_allclose(y[bb, :, c], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("s,p,d,K", [(1, 15, 1, 31), (2, 3, 1, 7), (1, 4, 2, 5), (3, 0, 2, 3), (1, 0, 1, 1)])
def test_dw1d_matches_torch_conv1d(s, p, d, K):
    """Library pin: torch conv1d (batch, channels, steps) with groups=C, fed the
    transposed tensor."""
    rng = np.random.default_rng(31 + K)
    B, T, C = 3, 37, 6
    x, w, b = rnd(rng, B, T, C), rnd(rng, C, 1, K), rnd(rng, C)
    y = oracle.dwconv1d_btc(x, w, b, stride=s, padding=p, dilation=d)
    ref = F.conv1d(t64(x).transpose(1, 2), t64(w), t64(b), stride=s, padding=p, dilation=d,
                   groups=C).transpose(1, 2).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_dw1d_equals_depthwise_conv2d_on_one_row():
    """The two oracle entry points agree: (B,T,C) depthwise == NCHW conv2d with
    H=1, groups=C, on the transposed tensor."""
    rng = np.random.default_rng(32)
    B, T, C, K = 2, 19, 4, 5
    x, w, b = rnd(rng, B, T, C), rnd(rng, C, 1, K), rnd(rng, C)
    y = oracle.dwconv1d_btc(x, w, b, stride=2, padding=2, dilation=1)
    ref = oracle.conv2d(x.transpose(0, 2, 1)[:, :, None, :], w[:, :, None, :], b, stride=(1, 2),
                        padding=(0, 2), groups=C)[:, :, 0, :].transpose(0, 2, 1)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- point evaluation and errors

def test_at_functions_equal_full():
    rng = np.random.default_rng(40)
    x, w, b = rnd(rng, 2, 8, 9, 7), rnd(rng, 6, 4, 3, 3), rnd(rng, 6)
    y = oracle.conv2d(x, w, b, stride=(2, 1), padding=1, dilation=(1, 2), groups=2)
    idx = rng.integers(0, y.size, 200)
    np.testing.assert_array_equal(
        oracle.conv2d_at(x, w, idx, b, stride=(2, 1), padding=1, dilation=(1, 2), groups=2), y.ravel()[idx])
    xd, wd, bd = rnd(rng, 2, 30, 7), rnd(rng, 7, 1, 9), rnd(rng, 7)
    yd = oracle.dwconv1d_btc(xd, wd, bd, padding=4)
    idx = rng.integers(0, yd.size, 100)
    np.testing.assert_array_equal(oracle.dwconv1d_btc_at(xd, wd, idx, bd, padding=4), yd.ravel()[idx])


def test_invalid_arguments_raise():
    x = np.zeros((1, 6, 5, 5))
    with pytest.raises(ValueError):
        oracle.conv2d(x, np.zeros((4, 3, 3, 3)), groups=4)      # 6 % 4 != 0
    with pytest.raises(ValueError):
        oracle.conv2d(x, np.zeros((5, 2, 3, 3)), groups=3)      # 5 % 3 != 0
    with pytest.raises(ValueError):
        oracle.conv2d(x, np.zeros((6, 3, 3, 3)), groups=3)      # w.shape[1] != C/g
    with pytest.raises(ValueError):
        oracle.conv2d(x, np.zeros((6, 2, 7, 7)), groups=3)      # empty output
    assert oracle.conv2d(np.zeros((0, 6, 5, 5)), np.zeros((6, 2, 3, 3)), groups=3).shape == (0, 6, 3, 3)


# ---------------------------------------------------------------- interleaved output order

@pytest.mark.parametrize("N,C,Co,H,W,K,g", [(2, 8, 12, 6, 7, 3, 4), (1, 6, 6, 5, 5, 3, 3), (2, 4, 8, 4, 4, 1, 2)])
def test_interleaved_order_is_the_channel_permutation(N, C, Co, H, W, K, g):
    """Output channel j*g + k holds filter j of group k: the grouped result with its
    channel axis viewed as [g, Cout/g] and transposed to [Cout/g, g]."""
    rng = np.random.default_rng(N * 100 + C)
    x, w, b = rnd(rng, N, C, H, W), rnd(rng, Co, C // g, K, K), rnd(rng, Co)
    yg = oracle.conv2d(x, w, b, 1, K // 2, 1, g)
    yi = oracle.conv2d(x, w, b, 1, K // 2, 1, g, out_order="interleaved")
    OH, OW = yg.shape[2:]
    perm = yg.reshape(N, g, Co // g, OH, OW).transpose(0, 2, 1, 3, 4).reshape(N, Co, OH, OW)
    np.testing.assert_array_equal(yi, perm)


def test_interleaved_order_is_the_identity_for_one_group_or_one_filter_per_group():
    rng = np.random.default_rng(5)
    x = rnd(rng, 2, 6, 5, 5)
    for w, g in ((rnd(rng, 4, 6, 3, 3), 1), (rnd(rng, 6, 1, 3, 3), 6), (rnd(rng, 3, 2, 3, 3), 3)):
        np.testing.assert_array_equal(oracle.conv2d(x, w, None, 1, 1, 1, g, out_order="interleaved"),
                                      oracle.conv2d(x, w, None, 1, 1, 1, g))
