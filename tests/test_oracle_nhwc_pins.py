"""Pins for the oracle's channels-last (NHWC) grouped conv2d (CPU only).

The NHWC function indexes x [N,H,W,C], w [Cout,KH,KW,C/g] and y [N,OH,OW,Cout]
directly.  It is checked against the NCHW oracle on the same tensors permuted (an
independent function, itself pinned), against torch's float64 conv2d on
channels_last tensors, and its point function against the full one.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GEOMS = [  # N, C, Cout, H, W, KH, KW, groups, stride, pad, dil
    (2, 8, 8, 7, 9, 3, 3, 8, 1, 1, 1),        # depthwise
    (1, 6, 12, 9, 8, 3, 3, 6, 2, 1, 1),       # depthwise, 2 filters per channel, stride 2
    (2, 12, 18, 6, 7, 3, 2, 3, (2, 1), (1, 0), (1, 2)),
    (1, 16, 16, 5, 5, 5, 5, 4, 1, 2, 1),
    (2, 9, 6, 6, 6, 1, 1, 3, 1, 0, 1),        # 1x1
    (1, 4, 8, 10, 11, 3, 3, 1, 1, 1, 1),      # dense
    (1, 4, 4, 2, 2, 3, 3, 4, 1, 1, 1),        # image smaller than the filter
]


def _inputs(seed, N, C, Cout, H, W, KH, KW, g):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, H, W, C)), rng.standard_normal((Cout, KH, KW, C // g)),
            rng.standard_normal(Cout))


@pytest.mark.parametrize("gi", range(len(GEOMS)))
def test_nhwc_equals_nchw_on_permuted_tensors(gi):
    N, C, Co, H, W, KH, KW, g, s, p, d = GEOMS[gi]
    x, w, b = _inputs(600 + gi, N, C, Co, H, W, KH, KW, g)
    y = oracle.conv2d_nhwc(x, w, b, s, p, d, g)
    r = oracle.conv2d(x.transpose(0, 3, 1, 2), w.transpose(0, 3, 1, 2), b, s, p, d, g)
    # Same terms, summed in (kh, kw, ci) order instead of (ci, kh, kw): fp64 rounding only.
    np.testing.assert_allclose(y, r.transpose(0, 2, 3, 1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("gi", range(len(GEOMS)))
def test_nhwc_matches_torch_channels_last(gi):
    N, C, Co, H, W, KH, KW, g, s, p, d = GEOMS[gi]
    x, w, b = _inputs(700 + gi, N, C, Co, H, W, KH, KW, g)
    xt = torch.from_numpy(x).permute(0, 3, 1, 2)          # an NCHW view of channels_last memory
    wt = torch.from_numpy(w).permute(0, 3, 1, 2)
    assert xt.is_contiguous(memory_format=torch.channels_last)
    yt = F.conv2d(xt, wt, torch.from_numpy(b), stride=s, padding=p, dilation=d, groups=g)
    np.testing.assert_allclose(oracle.conv2d_nhwc(x, w, b, s, p, d, g), yt.permute(0, 2, 3, 1).numpy(),
                               rtol=0, atol=1e-12)


def test_nhwc_at_equals_full():
    N, C, Co, H, W, KH, KW, g, s, p, d = GEOMS[2]
    x, w, b = _inputs(800, N, C, Co, H, W, KH, KW, g)
    y = oracle.conv2d_nhwc(x, w, b, s, p, d, g)
    idx = np.arange(y.size)
    np.testing.assert_array_equal(oracle.conv2d_nhwc_at(x, w, idx, b, s, p, d, g), y.ravel())
