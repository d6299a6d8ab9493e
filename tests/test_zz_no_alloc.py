"""GPU test of gconv_dw1d_bwd_filter_noalloc, the filter gradient that allocates
nothing (its partial sums go to the library's per-GPU scratch array): called
through the C ABI, its dw and db must equal those of gconv_dw1d_bwd_filter (the
same kernels with a caller workspace) bit for bit, on two calls in a row, the
second with a smaller input, and both must be within the fp32 bar of the fp64
oracle."""
import numpy as np
import pytest
import torch

import depthwise_convolution_gconv_amd as gc
from depthwise_convolution_gconv_amd.workloads import as_f64
import oracle

pytestmark = pytest.mark.gpu


def _case(B, T, C, K, pad, seed, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, T, C, generator=g).to(dtype)
    dy = torch.randn(B, T + 2 * pad - K + 1, C, generator=g).to(dtype)
    return x, dy


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_noalloc_filter_gradient_matches_the_workspace_entry_point(dtype):
    dev = torch.device("cuda:0")
    tol = 1e-4 if dtype == torch.float32 else 1e-2
    # First the Conformer shape (8 x 1024 x 512, K = 31), then a smaller ragged one:
    # the second call must not see the first call's partial sums.
    for (B, T, C, K, pad, seed) in ((8, 1024, 512, 31, 15, 11), (3, 77, 40, 5, 2, 12)):
        print(f"noalloc case B={B} T={T} C={C} K={K} pad={pad} dtype={dtype}", flush=True)
        x, dy = _case(B, T, C, K, pad, seed, dtype)
        xd, dyd = x.to(dev), dy.to(dev)
        dw_ref, db_ref = gc.gconv_dw1d_bwd_filter(xd, dyd, K, 1, pad, 1)
        dw = torch.full((C, 1, K), float("nan"), dtype=dtype, device=dev)
        db = torch.full((C,), float("nan"), dtype=dtype, device=dev)
        gc.gconv_dw1d_bwd_filter_noalloc(xd, dyd, K, 1, pad, 1, dw=dw, db=db)
        assert gc.gconv_last_kernel() == "dw1d_btc_wgrad_partial"
        torch.cuda.synchronize()
        assert torch.equal(dw, dw_ref) and torch.equal(db, db_ref)
        rdw, rdb = oracle.dwconv1d_btc_bwd_filter(as_f64(x), as_f64(dy), K, 1, pad, 1)
        for a, r in ((dw, rdw), (db, rdb)):
            err = float(np.abs(as_f64(a.cpu()) - r).max() / np.abs(r).max())
            assert err <= tol, err


def test_noalloc_filter_gradient_without_bias_and_on_a_side_stream():
    dev = torch.device("cuda:0")
    x, dy = _case(2, 300, 64, 7, 3, 13)
    xd, dyd = x.to(dev), dy.to(dev)
    dw_ref, _ = gc.gconv_dw1d_bwd_filter(xd, dyd, 7, 1, 3, 1, bias=False)
    side = torch.cuda.Stream(dev)
    dw = torch.empty((64, 1, 7), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    gc.gconv_dw1d_bwd_filter_noalloc(xd, dyd, 7, 1, 3, 1, dw=dw, db=None, bias=False, stream=side)
    side.synchronize()
    assert torch.equal(dw, dw_ref)
