"""GPU parity of the run-per-lane implicit GEMM (igemm_rows.hip) against the fp64
oracle, through the C ABI.

That kernel takes the 16-bit 3x3 layers with unit column stride and dilation,
C/g a multiple of 32 and more than 32 filters per group (the headline layer of the
discuss.pytorch.org thread "F.conv2d runs x15 slower in mixed-precision/
half-precision mode" among them).  Besides the accuracy bar (normwise 1e-2 for
16-bit inputs) each case is held to a regression bound near the kernel's own
error: the output rounding alone gives up to 2^-11 (fp16) or 2^-9 (bf16) of
max|r|, so 1e-3 and 4e-3 leave room for that and the fp32 accumulation, while a
dropped product or tap (an error of order 1/sqrt(fan-in) of an output, about
0.03 of max|r| here) still fails.  The elementwise relative error over the
outputs with |r| > 1e-3 max|r| is printed as a diagnostic.
"""
import numpy as np
import pytest
import torch

import depthwise_convolution_gconv_amd as gc
from depthwise_convolution_gconv_amd.workloads import WORKLOADS, as_f64, draw, make_inputs
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f16": 1e-2, "bf16": 1e-2}       # the 16-bit accuracy bar
REG = {"f16": 1e-3, "bf16": 4e-3}       # regression bound of the 16-bit MFMA kernels
KERNEL = "igemm_rows_mfma32x32x16"
DEFER = "igemm_defer_mfma32x32x16"   # 32 channels, 33 to 64 filters per group: deferred stores


def kernel_for(Cg, Ng):
    return DEFER if Cg == 32 and 32 < Ng <= 64 else KERNEL


def errors(y, r):
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert y.shape == r.shape
    assert np.isfinite(y).all()
    den = np.abs(r).max()
    normwise = float(np.abs(y - r).max() / den)
    big = np.abs(r) > 1e-3 * den
    elementwise = float((np.abs(y - r)[big] / np.abs(r)[big]).max()) if big.any() else 0.0
    return normwise, elementwise


def check(name, y, r, dt):
    nw, ew = errors(y, r)
    print(f"{name} {dt}: normwise {nw:.3e}, elementwise over |r| > 1e-3 max|r| {ew:.3e}")
    assert nw <= TOL[dt], nw
    assert nw <= REG[dt], nw


ROWS = [  # N, C, Cout, H, W, groups, stride_h, pad, dilation_h, bias
    (2, 64, 256, 16, 16, 2, 1, 1, 1, True),       # 128 filters per group, 16-byte stores
    (1, 128, 128, 9, 20, 1, 1, 1, 1, False),      # dense, 8 chunks, ragged runs (8-byte stores)
    (3, 64, 160, 7, 12, 2, 1, 1, 1, True),        # 80 filters per group: a partly empty wave
    (2, 64, 384, 17, 24, 2, 2, 1, 1, True),       # row stride 2, two filter tiles per group
    (2, 64, 144, 15, 16, 2, 1, 2, 2, True),       # row dilation 2, pad 2: 18-wide rows (2-byte stores)
    (1, 64, 160, 8, 8, 2, 1, 0, 1, False),        # no padding: 6 x 6 outputs, 80 filters per group
    (5, 32, 96, 5, 8, 1, 1, 1, 1, True),          # tiles spanning several images
    (2, 64, 256, 3, 48, 2, 1, 1, 1, True),        # the whole batch in one tile, 6 runs per row
    # 33 to 64 filters per group, each wave staging a 16-filter half-block; with 32
    # channels per group igemm_defer.hip (runs of 4 columns, each tile's stores
    # issued during the next tile), otherwise igemm_rows.hip with one filter wave
    (2, 64, 128, 16, 16, 2, 1, 1, 1, True),       # 64 filters per group
    (3, 96, 144, 14, 28, 3, 1, 1, 1, True),       # 48: the last half-block empty; 28-wide rows in 4-wide segments
    (2, 64, 80, 10, 16, 2, 1, 1, 1, True),        # 40: a half-block partly empty
    (1, 32, 33, 6, 8, 1, 1, 1, 1, False),         # 33, the fewest on this kernel
    (3, 64, 128, 12, 12, 2, 2, 1, 1, True),       # 64 per group, row stride 2
    (4, 64, 128, 28, 28, 2, 1, 1, 1, False),      # the ensemble layer's 28 x 28 rows, tiles across images
    (2, 128, 128, 12, 20, 2, 1, 1, 1, True),      # 64 channels per group: 4 chunks (igemm_rows)
    (1, 96, 48, 9, 16, 1, 1, 1, 1, True),         # 96 channels, 48 filters: 6 chunks (igemm_rows)
    (2, 64, 128, 10, 12, 2, 1, 0, 1, True),       # no padding: 10-wide rows, a partial last run, 2-byte stores
]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("ci", range(len(ROWS)))
def test_rows_kernel_vs_oracle(ci, dt):
    N, C, Co, H, W, g, sh, p, dh, has_b = ROWS[ci]
    seed = 40 * ci + {"f16": 1, "bf16": 2}[dt]
    x = draw((N, C, H, W), 1.0, 7600 + seed, dt)
    w = draw((Co, C // g, 3, 3), 1.0 / (C // g * 9), 8600 + seed, dt)
    b = draw((Co,), 0.01, 9600 + seed, dt) if has_b else None
    stride, dil = (sh, 1), (dh, 1)
    print(f"rows case {ROWS[ci]} {dt}", flush=True)
    r = oracle.conv2d(as_f64(x), as_f64(w), as_f64(b), stride=stride, padding=p, dilation=dil, groups=g)
    assert gc.gconv_select_route(x.shape, w.shape, stride, p, dil, g, "nchw", dt) == "igemm"
    y = gc.gconv_fwd(x.cuda(), w.cuda(), None if b is None else b.cuda(), stride, p, dil, g, "nchw")
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == kernel_for(C // g, Co // g)
    check(f"rows{ci}", as_f64(y.cpu()), r, dt)


# More tiles than the chip runs workgroups (256), so every workgroup takes several
# tiles in turn; the 128-filter case is the tile walk the headline layer runs.
MANY = [  # N, C, Cout, H, W, groups, bias
    (40, 128, 512, 32, 32, 4, True),      # 128 filters per group, 320 tiles
    (24, 128, 640, 24, 40, 2, False),     # 320 filters per group: 3 filter tiles, the last one partly empty
    (48, 256, 512, 28, 28, 8, True),      # 64 filters per group: 384 tiles, 1 or 2 per workgroup
    (40, 256, 384, 14, 28, 8, False),     # 48 filters per group: 400 tiles
]


@pytest.mark.parametrize("ci", range(len(MANY)))
def test_rows_kernel_many_tiles_vs_oracle(ci):
    N, C, Co, H, W, g, has_b = MANY[ci]
    dt = "f16" if ci % 2 == 0 else "bf16"
    x = draw((N, C, H, W), 1.0, 7700 + ci, dt)
    w = draw((Co, C // g, 3, 3), 1.0 / (C // g * 9), 8700 + ci, dt)
    b = draw((Co,), 0.01, 9700 + ci, dt) if has_b else None
    print(f"rows many-tiles case {MANY[ci]} {dt}", flush=True)
    r = oracle.conv2d(as_f64(x), as_f64(w), as_f64(b), stride=1, padding=1, dilation=1, groups=g)
    y = gc.gconv_fwd(x.cuda(), w.cuda(), None if b is None else b.cuda(), 1, 1, 1, g, "nchw")
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == kernel_for(C // g, Co // g)
    check(f"many{ci}", as_f64(y.cpu()), r, dt)


def test_rows_kernel_interleaved_order_and_unaligned_output():
    N, C, Co, H, W, g = 2, 64, 256, 12, 16, 2
    x = draw((N, C, H, W), 1.0, 7800, "f16")
    w = draw((Co, C // g, 3, 3), 1.0 / (C // g * 9), 8800, "f16")
    b = draw((Co,), 0.01, 9800, "f16")
    xd, wd, bd = x.cuda(), w.cuda(), b.cuda()
    r = oracle.conv2d(as_f64(x), as_f64(w), as_f64(b), 1, 1, 1, g, out_order="interleaved")
    y = gc.gconv_fwd_ex(xd, wd, bd, 1, 1, 1, g, "nchw", route="igemm", out_order="interleaved")
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == KERNEL
    check("interleaved", as_f64(y.cpu()), r, "f16")
    # y two bytes past a 16-byte boundary: the element-wise store path
    r = oracle.conv2d(as_f64(x), as_f64(w), as_f64(b), 1, 1, 1, g)
    n = N * Co * H * W
    buf = torch.full((n + 8,), float("nan"), dtype=torch.float16, device="cuda")
    y = buf[1:1 + n].view(N, Co, H, W)
    gc.gconv_fwd(xd, wd, bd, 1, 1, 1, g, "nchw", y=y)
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == KERNEL
    check("unaligned y", as_f64(y.cpu()), r, "f16")
    assert torch.isnan(buf[0]) and bool(torch.isnan(buf[1 + n:]).all())


def test_defer_kernel_interleaved_order_and_unaligned_output():
    N, C, Co, H, W, g = 2, 64, 128, 12, 16, 2
    x = draw((N, C, H, W), 1.0, 7850, "bf16")
    w = draw((Co, C // g, 3, 3), 1.0 / (C // g * 9), 8850, "bf16")
    b = draw((Co,), 0.01, 9850, "bf16")
    xd, wd, bd = x.cuda(), w.cuda(), b.cuda()
    r = oracle.conv2d(as_f64(x), as_f64(w), as_f64(b), 1, 1, 1, g, out_order="interleaved")
    y = gc.gconv_fwd_ex(xd, wd, bd, 1, 1, 1, g, "nchw", route="igemm", out_order="interleaved")
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == DEFER
    check("defer interleaved", as_f64(y.cpu()), r, "bf16")
    # y two bytes past an 8-byte boundary: the 2-byte store path
    r = oracle.conv2d(as_f64(x), as_f64(w), as_f64(b), 1, 1, 1, g)
    n = N * Co * H * W
    buf = torch.full((n + 8,), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = buf[1:1 + n].view(N, Co, H, W)
    gc.gconv_fwd(xd, wd, bd, 1, 1, 1, g, "nchw", y=y)
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == DEFER
    check("defer unaligned y", as_f64(y.float().cpu()), r, "bf16")
    assert torch.isnan(buf[0]) and bool(torch.isnan(buf[1 + n:]).all())


def test_headline_layer_full_size_vs_oracle_and_direct_route():
    # x [1,512,256,256], w [512,128,3,3], groups 4, fp16: every one of the 33.5 M
    # outputs against the oracle, and against the direct route element by element.
    wl = WORKLOADS["c2_p2layer_f16"]
    x, w, _ = make_inputs(wl)
    xd, wd = x.cuda(), w.cuda()
    y = gc.gconv_fwd(xd, wd, None, 1, 1, 1, 4, "nchw")
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == KERNEL
    yc = as_f64(y.cpu())
    ydir = gc.gconv_fwd_route(xd, wd, None, 1, 1, 1, 4, "nchw", route="direct")
    torch.cuda.synchronize()
    yd = as_f64(ydir.cpu())
    del ydir
    print("headline: oracle over all outputs ...", flush=True)
    r = oracle.conv2d(as_f64(x), as_f64(w), None, 1, 1, 1, 4)
    check("headline vs oracle", yc, r, "f16")
    check("direct route vs oracle", yd, r, "f16")
    nw = float(np.abs(yc - yd).max() / np.abs(r).max())
    print(f"headline: implicit GEMM vs direct route, normwise {nw:.3e}")
    assert nw <= 2 * REG["f16"]
