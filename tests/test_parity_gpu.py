"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar (normwise, fixed in advance): max|y - r| / max|r| <= 1e-4 for fp32 inputs and
<= 1e-2 for fp16/bf16 inputs with fp32 accumulation, where r is the oracle's
fp64 result on the same quantised inputs.  Small cases are compared element by
element in full; the full-size workloads are compared in full where the oracle
finishes in about a second, and on a seeded sample of outputs (each evaluated
one by one by the oracle) otherwise.
"""
import numpy as np
import pytest
import torch

import depthwise_convolution_gconv_amd as gc
from depthwise_convolution_gconv_amd.workloads import NEXT_WORKLOADS, WORKLOADS, as_f64, draw, make_inputs
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "f16": 1e-2, "bf16": 1e-2}
# Regression bound, well inside the bar above, near what the kernels reach: the
# single rounding of a 16-bit output alone is up to 2^-11 (fp16) or 2^-9 (bf16) of
# max|r|, and fp32 accumulation adds little; a dropped product or tap (of order
# 1/sqrt(fan-in) of an output) exceeds it.
REG = {"f32": 1e-4, "f16": 1e-3, "bf16": 4e-3}
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def normwise(y, r):
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert y.shape == r.shape
    assert np.isfinite(y).all()
    den = np.abs(r).max()
    return float(np.abs(y - r).max() / (den if den > 0 else 1.0))


def elementwise(y, r):
    """max |y - r| / |r| over the outputs with |r| > 1e-3 max|r| (a diagnostic)."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    big = np.abs(r) > 1e-3 * np.abs(r).max()
    return float((np.abs(y - r)[big] / np.abs(r)[big]).max()) if big.any() else 0.0


def check(y, r, dt, label=""):
    """The bar and the regression bound, with both error measures printed."""
    nw = normwise(y, r)
    print(f"{label} {dt}: normwise {nw:.3e}, elementwise over |r| > 1e-3 max|r| {elementwise(y, r):.3e}")
    assert nw <= TOL[dt] and nw <= REG[dt], (label, dt, nw)
    return True


def gpu(t):
    return None if t is None else t.cuda()


def run_conv2d(x, w, b, stride, pad, dil, groups, route):
    y = gc.gconv_fwd_route(gpu(x), gpu(w), gpu(b), stride, pad, dil, groups, "nchw", route=route)
    torch.cuda.synchronize()
    return y


# ---------------------------------------------------------------- small sweep

SWEEP = [  # N, C, Cout, H, W, K(h,w), groups, stride, pad, dil, bias
    (2, 8, 8, 9, 9, (3, 3), 8, 1, 1, 1, True),          # depthwise 3x3
    (2, 32, 64, 12, 13, (3, 3), 2, 1, 1, 1, True),      # 16 in / 32 out per group
    (1, 48, 40, 7, 9, (3, 3), 1, 1, 1, 1, False),       # dense, ragged channel counts
    (2, 32, 32, 15, 14, (3, 3), 2, 2, 2, 2, True),      # stride 2 + dilation 2
    (2, 64, 96, 6, 7, (1, 1), 2, 1, 0, 1, True),        # grouped 1x1
    (1, 64, 64, 11, 10, (5, 5), 4, 1, 2, 1, True),      # 5x5
    (3, 16, 16, 2, 2, (3, 3), 1, 1, 1, 1, True),        # image smaller than the kernel
    (5, 32, 64, 5, 5, (3, 3), 2, 1, 1, 1, False),       # tiles spanning several images
    (1, 32, 320, 9, 8, (3, 3), 2, 1, 1, 1, True),       # 160 outputs per group: two n-tiles
    (2, 12, 18, 10, 11, (3, 2), 3, (2, 1), (1, 0), (1, 2), True),  # anisotropic
    (1, 16, 16, 40, 70, (3, 3), 4, 1, 1, 1, True),      # several spatial tiles + ragged edge
    (2, 20, 20, 6, 6, (3, 3), 20, 1, 0, 1, False),      # depthwise, no padding
    (3, 16, 16, 7, 10, (3, 3), 4, 1, 1, 1, True),       # 4 in / 4 out per group, ragged (16-bit: g4 kernel)
    (2, 32, 32, 14, 14, (3, 3), 8, 1, 0, 1, True),      # 4 in / 4 out per group, no padding
    (2, 48, 96, 9, 9, (3, 3), 2, 1, 1, 1, True),        # 24 in per group: a last chunk of 8 channels; 48 filters
    (2, 48, 96, 6, 7, (1, 1), 2, 1, 0, 1, True),        # the same with 1x1 filters
    (2, 24, 32, 9, 9, (3, 3), 2, 1, 1, 1, True),        # 12 in per group: a last fp32 chunk of 4 channels
]


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ci", range(len(SWEEP)))
def test_sweep_vs_oracle(ci, dt):
    N, C, Co, H, W, (KH, KW), g, s, p, d, has_b = SWEEP[ci]
    seed = 50 * ci + {"f32": 0, "f16": 1, "bf16": 2}[dt]
    x = draw((N, C, H, W), 1.0, 7000 + seed, dt)
    w = draw((Co, C // g, KH, KW), 1.0 / (C // g * KH * KW), 8000 + seed, dt)
    b = draw((Co,), 0.01, 9000 + seed, dt) if has_b else None
    r = oracle.conv2d(as_f64(x), as_f64(w), as_f64(b), stride=s, padding=p, dilation=d, groups=g)
    routes = ["direct"]
    if gc.gconv_select_route(x.shape, w.shape, s, p, d, g, "nchw", dt) == "igemm":
        routes.append("igemm")
    else:
        try:
            run_conv2d(x, w, b, s, p, d, g, "igemm")
            routes.append("igemm")
        except gc.GconvError:
            pass
    outs = {}
    for route in routes:
        y = run_conv2d(x, w, b, s, p, d, g, route)
        outs[route] = y
        assert check(as_f64(y.cpu()), r, dt, route)
    if len(outs) == 2:  # the two routes agree with each other to the same bar
        assert normwise(as_f64(outs["igemm"].cpu()), as_f64(outs["direct"].cpu())) <= 2 * REG[dt]


# The 4-in / 4-out kernel (direct2d_g4, 16-bit, 3x3, stride 1): the operands of
# taps kw = 1, 2 come from the neighbouring lanes, 62 output anchors per pass.
G4_CASES = [  # N, C, H, W, pad (h, w), bias, y offset in elements
    (2, 16, 15, 14, (1, 1), True, 0),     # 210 outputs per plane: element stores
    (1, 32, 28, 28, (1, 1), True, 0),     # 30 x 30 padded image, 14 passes
    (2, 16, 10, 6, (1, 0), False, 0),     # padding rows only
    (2, 16, 6, 10, (0, 1), True, 0),      # padding columns only
    (3, 16, 7, 10, (1, 1), True, 1),      # y 2 bytes past alignment: element stores
    (2, 64, 14, 14, (1, 1), True, 0),     # the fully grouped workload's planes
    (1, 8, 2, 2, (1, 1), True, 0),        # 2 x 2 image: one pass, most lanes idle
]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("ci", range(len(G4_CASES)))
def test_g4_kernel_vs_oracle(ci, dt):
    N, C, H, W, pad, has_b, yoff = G4_CASES[ci]
    g = C // 4
    seed = 30 * ci + {"f16": 1, "bf16": 2}[dt]
    x = draw((N, C, H, W), 1.0, 7300 + seed, dt)
    w = draw((C, 4, 3, 3), 1.0 / 36, 8300 + seed, dt)
    b = draw((C,), 0.01, 9300 + seed, dt) if has_b else None
    print(f"g4 case {G4_CASES[ci]} {dt}", flush=True)
    r = oracle.conv2d(as_f64(x), as_f64(w), as_f64(b), stride=1, padding=pad, dilation=1, groups=g)
    n = r.size
    buf = torch.full((n + 8,), float("nan"), dtype=x.dtype, device="cuda")
    y = buf[yoff:yoff + n].view(r.shape)
    gc.gconv_fwd(gpu(x), gpu(w), gpu(b), 1, pad, 1, g, "nchw", y=y)
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == "direct2d_g4"
    yc = as_f64(y.cpu())
    assert normwise(yc, r) <= TOL[dt] and normwise(yc, r) <= REG[dt], normwise(yc, r)
    assert bool(torch.isnan(buf[yoff + n:]).all()) and (yoff == 0 or bool(torch.isnan(buf[:yoff]).all()))


# More tiles than the chip runs workgroups (256), so every workgroup of the implicit
# GEMM takes several tiles in turn; with at most 64 filters per group a tile's outputs
# are stored while the next tile computes.  Compared in full.
MANY_TILES = [  # N, C, Cout, H, W, K, groups, bias
    (4, 128, 128, 56, 56, 3, 16, True),     # 8 filters per group, ragged last tile
    (16, 256, 1024, 24, 24, 1, 16, True),   # 64 filters per group, 1x1
    (15, 128, 1024, 24, 24, 3, 16, False),  # 64 filters per group, 3x3, ragged last tile
]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("ci", range(len(MANY_TILES)))
def test_igemm_many_tiles_per_workgroup(ci, dt):
    N, C, Co, H, W, K, g, has_b = MANY_TILES[ci]
    seed = 30 * ci + {"f16": 1, "bf16": 2}[dt]
    x = draw((N, C, H, W), 1.0, 7300 + seed, dt)
    w = draw((Co, C // g, K, K), 1.0 / (C // g * K * K), 8300 + seed, dt)
    b = draw((Co,), 0.01, 9300 + seed, dt) if has_b else None
    r = oracle.conv2d(as_f64(x), as_f64(w), as_f64(b), stride=1, padding=K // 2, dilation=1, groups=g)
    y = run_conv2d(x, w, b, 1, K // 2, 1, g, "igemm")
    assert gc.gconv_last_kernel().startswith("igemm")
    assert check(as_f64(y.cpu()), r, dt)


DW_SWEEP = [  # B, T, C, K, stride, pad, dil, bias
    (2, 100, 64, 31, 1, 15, 1, True),
    (3, 37, 300, 3, 1, 1, 1, False),
    (1, 257, 40, 9, 1, 4, 1, True),
    (2, 50, 24, 7, 2, 3, 1, True),        # stride 2 (tile kernel)
    (2, 300, 64, 31, 2, 15, 1, True),     # stride 2, K = 31, several tiles and a ragged last one
    (3, 33, 40, 3, 2, 1, 1, False),       # stride 2, odd length
    (1, 97, 20, 9, 2, 0, 1, True),        # stride 2, no padding, C not a multiple of 64
    (2, 45, 16, 5, 1, 4, 2, True),        # dilation 2 (generic kernel)
    (1, 5, 8, 31, 1, 15, 1, True),        # sequence shorter than the kernel
    (2, 64, 33, 6, 1, 0, 1, True),        # even K, no padding (generic kernel)
]


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ci", range(len(DW_SWEEP)))
def test_dw1d_sweep_vs_oracle(ci, dt):
    B_, T, C, K, s, p, d, has_b = DW_SWEEP[ci]
    seed = 40 * ci + {"f32": 0, "f16": 1, "bf16": 2}[dt]
    x = draw((B_, T, C), 1.0, 7500 + seed, dt)
    w = draw((C, 1, K), 1.0 / K, 8500 + seed, dt)
    b = draw((C,), 0.01, 9500 + seed, dt) if has_b else None
    r = oracle.dwconv1d_btc(as_f64(x), as_f64(w), as_f64(b), stride=s, padding=p, dilation=d)
    y = gc.dwconv1d_btc(gpu(x), gpu(w), gpu(b), stride=s, padding=p, dilation=d)
    torch.cuda.synchronize()
    assert check(as_f64(y.cpu()), r, dt)


# Depthwise conv2d (C/g = 1): the dw2d_rows kernel where its plan applies (K in
# {3, 5, 7}, square stride 1 or 2, dilation 1), the tiled kernel otherwise.
DW2D_SWEEP = [  # N, C, M (filters per channel), H, W, K, stride, pad, bias
    (2, 3, 1, 9, 8, 3, 1, 1, True),       # planes smaller than a workgroup's runs
    (2, 3, 1, 9, 8, 3, 2, 1, False),
    (1, 4, 2, 11, 12, 5, 2, 2, True),     # two filters per channel
    (3, 2, 1, 7, 7, 7, 1, 3, True),       # 7x7, odd width (single-element runs and loads)
    (2, 5, 1, 6, 16, 3, 2, 0, True),      # no padding, odd output width
    (1, 3, 3, 13, 24, 3, 1, 1, False),    # three filters per channel
    (1, 2, 1, 64, 40, 3, 2, 1, True),     # several workgroups per plane
    (1, 2, 1, 70, 8, 5, 1, 2, True),
    (4, 8, 1, 4, 4, 3, 1, 1, True),       # many tiny planes per workgroup
    (1, 1, 1, 2, 2, 3, 1, 1, True),       # image smaller than the filter
    (2, 3, 1, 20, 20, 7, 2, 3, True),
    (2, 16, 1, 30, 30, 3, 1, 1, True),    # 30 columns: 8-byte runs in 16-bit
    (1, 8, 1, 33, 35, 3, 2, 1, True),     # odd sizes throughout
    (4, 16, 1, 50, 40, 3, 1, 1, True),    # tens of workgroups, each crossing plane boundaries
    (2, 32, 1, 64, 44, 3, 2, 1, True),
    (3, 24, 2, 30, 28, 5, 1, 2, True),    # two filters per channel over many workgroups
    (2, 4, 1, 16, 32, 7, 2, 3, True),     # 7x7, stride 2, 16-byte staging loads in 16-bit
    (2, 4, 2, 12, 16, 3, 2, 1, False),    # two filters per channel, stride 2, 16-byte runs in 16-bit
    (1, 4, 1, 9, 9, 3, 3, 1, True),       # stride 3: not this kernel (tiled)
    (1, 4, 1, 9, 9, 4, 1, 1, True),       # even filter: not this kernel (tiled)
    # full-width layers (OW * stride == W, W a multiple of 8): dw2d_band in 16-bit
    (2, 3, 1, 70, 8, 3, 1, 1, True),      # one chunk per row: 64 strips side by side in a wave
    (1, 4, 2, 80, 16, 5, 2, 2, True),     # two filters per channel, 5x5 stride 2
    (1, 2, 1, 68, 56, 7, 2, 3, True),     # 7x7 stride 2
    (2, 5, 1, 66, 40, 3, 2, 1, False),    # 33 output rows: a half-empty last strip; 5 chunks per row (4 idle lanes)
    (1, 2, 1, 64, 512, 3, 1, 1, True),    # 64 chunks per row: one strip per wave
    (1, 2, 3, 16, 40, 5, 1, 2, True),     # three filters per channel, stride 1
    (4, 33, 1, 37, 24, 3, 2, 1, True),    # one output row per strip (LDS), many planes per workgroup
    (1, 3, 1, 21, 24, 7, 1, 3, True),     # 7x7 stride 1, odd output rows
    (3, 2, 1, 50, 8, 3, 2, 0, True),      # no padding: output narrower than W/2, dw2d_rows
    (1, 1, 1, 1, 8, 3, 2, 1, True),       # a single output row
    (3, 4, 1, 65, 40, 3, 2, 1, True),     # a plane's last strip reads into the next plane's padded rows
]


def dw2d_kernel(N, C, M, H, W, K, s, p, dt):
    """The depthwise conv2d kernel the dispatcher picks for an aligned NCHW layer
    (every full-width layer here fits the band kernel's LDS)."""
    if K not in (3, 5, 7) or s not in (1, 2):
        return "direct2d_tiled"
    OW = (W + 2 * p - K) // s + 1
    if dt != "f32" and p == (K - 1) // 2 and OW * s == W and W % 8 == 0 and W // 8 <= 64:
        return "dw2d_band"
    return "dw2d_rows"


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ci", range(len(DW2D_SWEEP)))
def test_dw2d_sweep_vs_oracle(ci, dt):
    N, C, M, H, W, K, s, p, has_b = DW2D_SWEEP[ci]
    seed = 60 * ci + {"f32": 0, "f16": 1, "bf16": 2}[dt]
    x = draw((N, C, H, W), 1.0, 7700 + seed, dt)
    w = draw((C * M, 1, K, K), 1.0 / (K * K), 8700 + seed, dt)
    b = draw((C * M,), 0.01, 9700 + seed, dt) if has_b else None
    r = oracle.conv2d(as_f64(x), as_f64(w), as_f64(b), stride=s, padding=p, dilation=1, groups=C)
    y = run_conv2d(x, w, b, s, p, 1, C, "auto")
    assert gc.gconv_last_kernel() == dw2d_kernel(N, C, M, H, W, K, s, p, dt)
    assert check(as_f64(y.cpu()), r, dt)


# Channels-last (NHWC) conv2d: the depthwise tile kernel where it applies, the
# generic kernel for every other geometry.
NHWC_SWEEP = [  # N, C, Cout, H, W, KH, KW, groups, stride, pad, dil, bias
    (2, 64, 64, 9, 8, 3, 3, 64, 1, 1, 1, True),        # depthwise, one channel block
    (1, 100, 100, 13, 11, 3, 3, 100, 2, 1, 1, True),   # depthwise, ragged channel block, stride 2
    (2, 72, 72, 10, 9, 5, 5, 72, 1, 2, 1, False),      # 5x5
    (1, 128, 128, 15, 17, 7, 7, 128, 2, 3, 1, True),   # 7x7, stride 2, two channel blocks
    (3, 12, 12, 6, 7, 3, 3, 12, 1, 0, 1, True),        # C not a multiple of 16 bytes (scalar loads)
    (1, 16, 16, 2, 2, 3, 3, 16, 1, 1, 1, True),        # image smaller than the filter
    (2, 32, 64, 8, 8, 3, 3, 32, 1, 1, 1, True),        # two filters per channel (generic)
    (2, 32, 48, 9, 7, 3, 3, 4, 1, 1, 1, True),         # grouped (generic)
    (1, 24, 24, 11, 10, 3, 2, 3, (2, 1), (1, 0), (1, 2), True),   # anisotropic (generic)
    (2, 16, 16, 7, 7, 3, 3, 16, 1, 2, 2, True),        # depthwise with dilation 2 (generic)
    (2, 64, 64, 9, 10, 3, 3, 16, 1, 1, 1, True),       # 4 in / 4 out per group (g4 kernel)
    (1, 32, 32, 11, 9, 3, 3, 8, 2, 1, 2, False),       # 4 in / 4 out, stride 2, dilation 2
    (1, 16, 16, 7, 8, 5, 3, 4, 1, (2, 1), 1, True),    # 4 in / 4 out with a 5 x 3 filter (g4 kernel)
    (3, 32, 32, 6, 13, 3, 3, 8, 1, 1, 1, True),        # 4 in / 4 out, rows of 13: a ragged 8-output block
    (1, 64, 64, 10, 17, 3, 3, 16, (2, 1), (1, 0), (2, 1), False),   # 4 in / 4 out, row stride and dilation 2
    (2, 16, 16, 5, 8, 3, 3, 4, 1, 0, 1, True),         # 4 in / 4 out, no padding
    # 4 in / 4 out, 16-bit, 3 x 3, unit stride: the whole-image matrix-core kernel
    (4, 128, 128, 14, 14, 3, 3, 32, 1, 1, 1, True),    # the fully grouped layer's image, 4 channel blocks
    (2, 32, 32, 7, 23, 3, 3, 8, 1, 1, 1, True),        # ragged rows, 3 anchor passes per group
    (2, 64, 64, 8, 12, 3, 3, 16, 1, (1, 0), 1, True),  # padding on the rows only
    (1, 48, 48, 10, 10, 3, 3, 12, 1, 1, 1, False),     # 48 channels: blocks of 4 groups
    (1, 32, 32, 40, 40, 3, 3, 8, 1, 1, 1, True),       # an image too large for it: the row kernel
    # depthwise, 16-bit channel pairs (C a multiple of 8)
    (2, 200, 200, 11, 13, 3, 3, 200, 1, 1, 1, True),   # 2 channel blocks, the second partly empty
    (1, 136, 136, 9, 10, 5, 5, 136, 2, 2, 1, False),   # 5x5, stride 2
]


def nhwc_g4_mfma_applies(C, H, W, s, p, d, dt):
    """Whether conv2d_nhwc_g4_mfma takes a 4-in/4-out 3x3 NHWC layer (its host
    conditions: 16-bit, unit stride and dilation, padding at most 1, 4*GPB channels
    per block with GPB = 8 or 4, the image within 8 loads of 16 bytes per thread and
    the planes and outputs within 40 KB of LDS)."""
    two = lambda v: v if isinstance(v, tuple) else (v, v)
    (sh, sw), (ph, pw), (dh, dw) = two(s), two(p), two(d)
    if dt == "f32" or (sh, sw, dh, dw) != (1, 1, 1, 1) or ph > 1 or pw > 1:
        return False
    HP, WP = H + 2 * ph, W + 2 * pw
    if WP > 400 or HP * WP > 1024:
        return False
    OH, OW = HP - 2, WP - 2
    na = (OH - 1) * WP + OW
    npass = -(-na // 62)
    img = max(HP * WP, 62 * (npass - 1) + 64 + 2 * WP + 2) | 1
    for gpb in (8, 4):
        if C % (4 * gpb) or H * W * gpb // 2 > 256 * 8:
            continue
        if (gpb * img + OH * OW * (gpb + 1)) * 8 <= 40 * 1024:
            return True
    return False


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ci", range(len(NHWC_SWEEP)))
def test_nhwc_sweep_vs_oracle(ci, dt):
    N, C, Co, H, W, KH, KW, g, s, p, d, has_b = NHWC_SWEEP[ci]
    seed = 80 * ci + {"f32": 0, "f16": 1, "bf16": 2}[dt]
    x = draw((N, H, W, C), 1.0, 7900 + seed, dt)
    w = draw((Co, KH, KW, C // g), 1.0 / (C // g * KH * KW), 8900 + seed, dt)
    b = draw((Co,), 0.01, 9900 + seed, dt) if has_b else None
    r = oracle.conv2d_nhwc(as_f64(x), as_f64(w), as_f64(b), stride=s, padding=p, dilation=d, groups=g)
    y = gc.conv2d_nhwc(gpu(x), gpu(w), gpu(b), stride=s, padding=p, dilation=d, groups=g)
    torch.cuda.synchronize()
    dw = g == C and Co == C and KH == KW and KH in (3, 5, 7) and s in (1, 2) and d == 1
    g4 = C == 4 * g and Co == C
    sw = s[1] if isinstance(s, tuple) else s
    dw_ = d[1] if isinstance(d, tuple) else d
    row = dt != "f32" and sw == 1 and dw_ == 1
    g4k = ("conv2d_nhwc_g4k3_row" if row else "conv2d_nhwc_g4k3") if (KH, KW) == (3, 3) else "conv2d_nhwc_g4"
    if (KH, KW) == (3, 3) and nhwc_g4_mfma_applies(C, H, W, s, p, d, dt):
        g4k = "conv2d_nhwc_g4_mfma"
    dwk = "dw2d_nhwc_pair" if dt != "f32" and C % 8 == 0 else "dw2d_nhwc_tile"   # 16-bit channel pairs
    assert gc.gconv_last_kernel() == (dwk if dw else g4k if g4 else "conv2d_nhwc_generic")
    assert check(as_f64(y.cpu()), r, dt)


NHWC_IGEMM = [  # N, C, Cout, H, W, KH, KW, groups, stride, pad, dil, bias
    (2, 64, 128, 12, 13, 3, 3, 2, 1, 1, 1, True),     # 32 in / 64 out per group
    (1, 32, 96, 9, 9, 3, 3, 1, 2, 1, 1, False),       # dense, stride 2, 96 filters: a partial filter tile
    (3, 128, 64, 7, 10, 1, 1, 4, 1, 0, 1, True),      # 1x1, ragged positions
    (1, 64, 64, 11, 8, 5, 3, 4, (2, 1), (2, 1), (1, 2), True),   # anisotropic
    (4, 256, 512, 14, 14, 3, 3, 8, 1, 1, 1, True),    # many workgroups
    (2, 32, 24, 8, 9, 3, 3, 2, 1, 1, 1, True),        # 12 filters per group: 8-byte stores, not staged
    (1, 128, 32, 5, 6, 2, 2, 1, 1, 0, 1, False),      # 512 elements per filter: the largest LDS filter block
    (1, 128, 64, 6, 7, 3, 3, 2, 1, 1, 1, True),       # 576 elements per filter: filters from global memory
    (1, 64, 64, 4, 300, 3, 3, 2, 1, 1, 1, True),      # 300-wide rows: input halo too large, filters in LDS
    (3, 64, 64, 5, 7, 3, 3, 2, 2, 1, 1, True),        # stride 2, tiles across several images
    # Strips of several position tiles per workgroup (next tile's halo prefetched):
    (1, 4096, 1024, 32, 32, 3, 3, 256, 1, 1, 1, True),   # 4 filters per group: unstaged stores
    (1, 4096, 2048, 30, 30, 3, 3, 256, 1, 1, 1, True),   # 8 filters per group, ragged last tile
    (2, 64, 384, 96, 96, 3, 3, 4, 1, 1, 1, True),        # 96 filters per group: two filter tiles
]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("ci", range(len(NHWC_IGEMM)))
def test_nhwc_igemm_vs_oracle(ci, dt):
    N, C, Co, H, W, KH, KW, g, s, p, d, has_b = NHWC_IGEMM[ci]
    seed = 85 * ci + {"f16": 1, "bf16": 2}[dt]
    x = draw((N, H, W, C), 1.0, 7920 + seed, dt)
    w = draw((Co, KH, KW, C // g), 1.0 / (C // g * KH * KW), 8920 + seed, dt)
    b = draw((Co,), 0.01, 9920 + seed, dt) if has_b else None
    r = oracle.conv2d_nhwc(as_f64(x), as_f64(w), as_f64(b), stride=s, padding=p, dilation=d, groups=g)
    y = gc.gconv_fwd_route(gpu(x), gpu(w), gpu(b), s, p, d, g, "nhwc", route="igemm")
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == "igemm_nhwc_mfma32x32x16"
    assert check(as_f64(y.cpu()), r, dt)
    yd = gc.gconv_fwd_route(gpu(x), gpu(w), gpu(b), s, p, d, g, "nhwc", route="direct")
    torch.cuda.synchronize()
    assert normwise(as_f64(y.cpu()), as_f64(yd.cpu())) <= 2 * REG[dt]   # the two routes agree


def test_nhwc_implicit_gemm_route_limits():
    # fp32, or 8 input channels per group: not the implicit GEMM; the route says so.
    for dt, cg in ((torch.float32, 16), (torch.float16, 8)):
        x = torch.randn(1, 8, 8, 2 * cg, device="cuda", dtype=dt)
        w = torch.randn(32, 3, 3, cg, device="cuda", dtype=dt)
        with pytest.raises(gc.GconvError) as e:
            gc.gconv_fwd_route(x, w, None, 1, 1, 1, 2, "nhwc", route="igemm")
        assert e.value.status == 3


# The interleaved output-channel order (filter j of group k at channel j*g + k),
# through every kernel family that stores grouped outputs.
ORDER_CASES = [  # N, C, Cout, H, W, K, groups, route, dtypes, kernel prefix
    (2, 32, 64, 12, 13, 3, 2, "igemm", ("f16", "bf16", "f32"), "igemm"),
    (4, 64, 256, 12, 12, 3, 4, "igemm", ("f16",), "igemm"),        # 64 filters per group: deferred stores
    (2, 16, 24, 9, 10, 3, 4, "direct", ("f32", "bf16"), "direct2d_tiled"),
    (3, 16, 16, 7, 10, 3, 4, "direct", ("f16", "bf16"), "direct2d_g4"),
    (2, 8, 16, 9, 9, 3, 8, "direct", ("f32",), "direct2d_tiled"),  # depthwise, 2 filters per channel
]


@pytest.mark.parametrize("ci", range(len(ORDER_CASES)))
def test_interleaved_output_order_vs_oracle(ci):
    N, C, Co, H, W, K, g, route, dts, kern = ORDER_CASES[ci]
    for di, dt in enumerate(dts):
        seed = 90 * ci + di
        x = draw((N, C, H, W), 1.0, 7950 + seed, dt)
        w = draw((Co, C // g, K, K), 1.0 / (C // g * K * K), 8950 + seed, dt)
        b = draw((Co,), 0.01, 9950 + seed, dt)
        r = oracle.conv2d(as_f64(x), as_f64(w), as_f64(b), 1, K // 2, 1, g, out_order="interleaved")
        y = gc.gconv_fwd_ex(gpu(x), gpu(w), gpu(b), 1, K // 2, 1, g, "nchw", route=route, out_order="interleaved")
        torch.cuda.synchronize()
        assert gc.gconv_last_kernel().startswith(kern), gc.gconv_last_kernel()
        assert check(as_f64(y.cpu()), r, dt)


def test_interleaved_output_order_nhwc_and_naive():
    # NHWC generic kernel: against the NCHW interleaved oracle on permuted tensors.
    N, C, Co, H, W, g = 2, 12, 18, 7, 8, 3
    x = draw((N, H, W, C), 1.0, 7990, "f32")
    w = draw((Co, 3, 3, C // g), 1.0 / (C // g * 9), 8990, "f32")
    b = draw((Co,), 0.01, 9990, "f32")
    r = oracle.conv2d(as_f64(x).transpose(0, 3, 1, 2), as_f64(w).transpose(0, 3, 1, 2), as_f64(b), 1, 1, 1, g,
                      out_order="interleaved").transpose(0, 2, 3, 1)
    y = gc.gconv_fwd_ex(gpu(x), gpu(w), gpu(b), 1, 1, 1, g, "nhwc", out_order="interleaved")
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == "conv2d_nhwc_generic"
    assert check(as_f64(y.cpu()), r, "f32")
    # NCHW naive kernel (a dilation whose halo tile does not fit the tiled kernel's LDS).
    x2 = draw((1, 4, 112, 112), 1.0, 7991, "f32")
    w2 = draw((6, 2, 3, 3), 1.0 / 18, 8991, "f32")
    r2 = oracle.conv2d(as_f64(x2), as_f64(w2), None, 1, 0, 55, 2, out_order="interleaved")
    y2 = gc.gconv_fwd_ex(gpu(x2), gpu(w2), None, 1, 0, 55, 2, "nchw", route="direct", out_order="interleaved")
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == "direct2d_naive"
    assert check(as_f64(y2.cpu()), r2, "f32")


def test_autotune_records_a_route_and_auto_calls_follow_it():
    gc.gconv_autotune_clear()
    x = draw((2, 64, 28, 28), 1.0, 7970, "f16")
    w = draw((64, 32, 3, 3), 1.0 / 288, 8970, "f16")
    b = draw((64,), 0.01, 9970, "f16")
    r = oracle.conv2d(as_f64(x), as_f64(w), as_f64(b), 1, 1, 1, 2)
    heur = gc.gconv_select_route(x.shape, w.shape, 1, 1, 1, 2, "nchw", "f16")
    assert heur == "igemm"
    xg, wg, bg = gpu(x), gpu(w), gpu(b)
    y = torch.full((2, 64, 28, 28), float("nan"), dtype=torch.float16, device="cuda")
    best = gc.gconv_autotune(xg, wg, bg, 1, 1, 1, 2, "nchw", reps=3, y=y)
    assert best in ("direct", "igemm")
    assert check(as_f64(y.cpu()), r, "f16")            # y holds the chosen route's result
    assert gc.gconv_select_route(x.shape, w.shape, 1, 1, 1, 2, "nchw", "f16") == best
    y2 = gc.gconv_fwd(xg, wg, bg, 1, 1, 1, 2, "nchw")
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel().startswith("igemm") == (best == "igemm")
    assert check(as_f64(y2.cpu()), r, "f16")
    gc.gconv_autotune_clear()
    assert gc.gconv_select_route(x.shape, w.shape, 1, 1, 1, 2, "nchw", "f16") == heur


def test_autotune_skips_routes_that_cannot_run_the_call():
    gc.gconv_autotune_clear()
    wl = WORKLOADS["c3_dw1d_btc_f32"]
    x, w, b = (gpu(t) for t in make_inputs(wl))
    assert gc.gconv_autotune(x, w, b, wl.stride, wl.pad, wl.dilation, wl.groups, "ntc", reps=2) == "direct"
    gc.gconv_autotune_clear()


# dw2d_band with vertical padding other than the filter's half (the horizontal one
# is fixed by the full-width condition).
BAND_PAD = [  # N, C, M, H, W, K, stride, (ph, pw), bias
    (2, 3, 1, 20, 16, 3, 2, (0, 1), True),     # no vertical padding
    (1, 4, 2, 17, 24, 3, 2, (2, 1), False),    # two padding rows: zero rows inside a strip
    (2, 2, 1, 19, 40, 5, 1, (0, 2), True),
    (1, 3, 1, 23, 8, 7, 2, (1, 3), True),
]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("ci", range(len(BAND_PAD)))
def test_dw2d_band_vertical_padding(ci, dt):
    N, C, M, H, W, K, s, pad, has_b = BAND_PAD[ci]
    seed = 40 * ci + {"f16": 1, "bf16": 2}[dt]
    x = draw((N, C, H, W), 1.0, 7300 + seed, dt)
    w = draw((C * M, 1, K, K), 1.0 / (K * K), 8300 + seed, dt)
    b = draw((C * M,), 0.01, 9300 + seed, dt) if has_b else None
    r = oracle.conv2d(as_f64(x), as_f64(w), as_f64(b), stride=s, padding=pad, dilation=1, groups=C)
    y = run_conv2d(x, w, b, s, pad, 1, C, "auto")
    assert gc.gconv_last_kernel() == "dw2d_band"
    assert check(as_f64(y.cpu()), r, dt)


def test_dw2d_unaligned_output_and_input():
    # y and x that start 4 bytes past a 16-byte boundary: single-element runs and loads.
    N, C, H, W, K = 2, 6, 24, 24, 3
    x = draw((N, C, H, W), 1.0, 7790, "f32")
    w = draw((C, 1, K, K), 1.0 / 9, 8790, "f32")
    b = draw((C,), 0.01, 9790, "f32")
    r = oracle.conv2d(as_f64(x), as_f64(w), as_f64(b), stride=2, padding=1, dilation=1, groups=C)
    xb = torch.empty(x.numel() + 1, device="cuda")
    xu = xb[1:].view(N, C, H, W)
    xu.copy_(x.cuda())
    yb = torch.empty(N * C * 12 * 12 + 1, device="cuda")
    yu = yb[1:].view(N, C, 12, 12)
    gc.gconv_fwd(xu, gpu(w), gpu(b), 2, 1, 1, C, "nchw", y=yu)
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == "dw2d_rows"
    assert check(as_f64(yu.cpu()), r, "f32")


def test_dw1d_unaligned_filters_use_the_window_kernel():
    # The tile kernel reads the filters 16 bytes at a time; filters that start 4 bytes
    # past an aligned address go to the window kernel, with the same result.
    B_, T, C, K = 2, 70, 64, 31
    x = draw((B_, T, C), 1.0, 7600, "f32")
    w = draw((C, 1, K), 1.0 / K, 8600, "f32")
    b = draw((C,), 0.01, 9600, "f32")
    r = oracle.dwconv1d_btc(as_f64(x), as_f64(w), as_f64(b), stride=1, padding=15, dilation=1)
    buf = torch.empty(C * K + 1, device="cuda")
    wu = buf[1:].view(C, 1, K)
    wu.copy_(w.cuda())
    assert wu.data_ptr() % 16 != 0
    y = gc.dwconv1d_btc(gpu(x), wu, gpu(b), stride=1, padding=15, dilation=1)
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == "dw1d_btc_window"
    assert check(as_f64(y.cpu()), r, "f32")
    y2 = gc.dwconv1d_btc(gpu(x), gpu(w), gpu(b), stride=1, padding=15, dilation=1)
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == "dw1d_btc_tile"
    assert check(as_f64(y2.cpu()), r, "f32")
    # x 4 bytes past a 16-byte boundary: the tile kernel with element loads
    xb = torch.empty(B_ * T * C + 1, device="cuda")
    xu = xb[1:].view(B_, T, C)
    xu.copy_(x.cuda())
    y3 = gc.dwconv1d_btc(xu, gpu(w), gpu(b), stride=1, padding=15, dilation=1)
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == "dw1d_btc_tile"
    assert check(as_f64(y3.cpu()), r, "f32")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_dw1d_many_tiles_ragged_steps_and_channels(dt):
    # 13 x 1500 steps x 200 channels, K = 31: 2444 tiles of 32 steps x 64 channels
    # (more than the chip holds at once), a ragged last tile in every sequence
    # (1500 = 46 x 32 + 28) and a last channel block 8 channels wide.
    B_, T, C, K = 13, 1500, 200, 31
    x = draw((B_, T, C), 1.0, 7610, dt)
    w = draw((C, 1, K), 1.0 / K, 8610, dt)
    b = draw((C,), 0.01, 9610, dt)
    print(f"dw1d many tiles {dt}", flush=True)
    r = oracle.dwconv1d_btc(as_f64(x), as_f64(w), as_f64(b), stride=1, padding=15, dilation=1)
    y = gc.dwconv1d_btc(gpu(x), gpu(w), gpu(b), stride=1, padding=15, dilation=1)
    torch.cuda.synchronize()
    assert gc.gconv_last_kernel() == "dw1d_btc_tile"
    assert check(as_f64(y.cpu()), r, dt)


# ---------------------------------------------------------------- backward of the depthwise conv1d

BWD_SWEEP = [  # B, T, C, K, stride, pad, dil
    (2, 100, 64, 31, 1, 15, 1),     # Conformer filter; input gradient on the reversed-filter tile kernel
    (3, 37, 300, 3, 1, 1, 1),       # C not a multiple of 64
    (1, 257, 40, 9, 1, 4, 1),       # ragged last tile
    (2, 50, 24, 7, 2, 3, 1),        # stride 2
    (2, 45, 16, 5, 1, 4, 2),        # dilation 2
    (1, 5, 8, 31, 1, 15, 1),        # sequence shorter than the filter
    (2, 64, 33, 6, 1, 0, 1),        # even K, no padding
    (2, 30, 16, 3, 1, 3, 1),        # padding beyond K - 1
    (1, 70, 20, 40, 3, 20, 1),      # 40 taps, stride 3
]


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("ci", range(len(BWD_SWEEP)))
def test_dw1d_backward_vs_oracle(ci, dt):
    B_, T, C, K, s, p, d = BWD_SWEEP[ci]
    seed = 70 * ci + {"f32": 0, "f16": 1, "bf16": 2}[dt]
    To = oracle.out_len(T, K, s, p, d)
    x = draw((B_, T, C), 1.0, 7800 + seed, dt)
    w = draw((C, 1, K), 1.0 / K, 8800 + seed, dt)
    dy = draw((B_, To, C), 1.0, 9800 + seed, dt)
    dx, dw, db = gc.dwconv1d_btc_backward(gpu(x), gpu(w), gpu(dy), stride=s, padding=p, dilation=d)
    torch.cuda.synchronize()
    rdx = oracle.dwconv1d_btc_bwd_data(as_f64(dy), as_f64(w), T, s, p, d)
    rdw, rdb = oracle.dwconv1d_btc_bwd_filter(as_f64(x), as_f64(dy), K, s, p, d)
    assert check(as_f64(dx.cpu()), rdx, dt)
    assert check(as_f64(dw.cpu()), rdw, dt)
    assert check(as_f64(db.cpu()), rdb, dt)


def test_dw1d_backward_kernels_and_determinism():
    wl = WORKLOADS["c3_dw1d_btc_f32"]
    x, w, _ = make_inputs(wl)
    dy = draw((8, 1024, 512), 1.0, 9900, "f32")
    xg, wg, dyg = gpu(x), gpu(w), gpu(dy)
    dx1 = gc.gconv_dw1d_bwd_data(dyg, wg, 1024, 1, 15, 1)
    assert gc.gconv_last_kernel() == "dw1d_btc_tile_flip"
    dw1, db1 = gc.gconv_dw1d_bwd_filter(xg, dyg, 31, 1, 15, 1)
    assert gc.gconv_last_kernel() == "dw1d_btc_wgrad_partial"
    dx2 = gc.gconv_dw1d_bwd_data(dyg, wg, 1024, 1, 15, 1)
    dw2, db2 = gc.gconv_dw1d_bwd_filter(xg, dyg, 31, 1, 15, 1)
    torch.cuda.synchronize()
    for a, b in ((dx1, dx2), (dw1, dw2), (db1, db2)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    # Full size against the oracle: the filter and bias gradients in full, the input
    # gradient on 20 000 sampled elements.
    rdw, rdb = oracle.dwconv1d_btc_bwd_filter(as_f64(x), as_f64(dy), 31, 1, 15, 1)
    assert normwise(as_f64(dw1.cpu()), rdw) <= 1e-4
    assert normwise(as_f64(db1.cpu()), rdb) <= 1e-4
    idx = _sample_idx(dx1.numel(), 20000, 4545)
    rdx = oracle.dwconv1d_btc_bwd_data_at(as_f64(dy), as_f64(w), 1024, idx, 1, 15, 1)
    assert normwise(as_f64(dx1.cpu()).ravel()[idx], rdx) <= 1e-4


def test_dw1d_bwd_filter_with_a_workspace_4_bytes_off_alignment():
    # The workspace need only be 4-byte aligned; the reduction then reads it 4 bytes at a time.
    B_, T, C, K = 2, 90, 40, 9
    x = draw((B_, T, C), 1.0, 7980, "f32")
    dy = draw((B_, T, C), 1.0, 8980, "f32")
    need = gc.gconv_dw1d_bwd_filter_workspace((B_, T, C), (C, 1, K), 1, 4, 1, "f32")
    buf = torch.empty(need + 16, dtype=torch.uint8, device="cuda")
    ws = buf[4:4 + need]
    assert ws.data_ptr() % 16 == 4
    dw, db = gc.gconv_dw1d_bwd_filter(gpu(x), gpu(dy), K, 1, 4, 1, workspace=ws)
    torch.cuda.synchronize()
    rdw, rdb = oracle.dwconv1d_btc_bwd_filter(as_f64(x), as_f64(dy), K, 1, 4, 1)
    assert normwise(as_f64(dw.cpu()), rdw) <= 1e-4
    assert normwise(as_f64(db.cpu()), rdb) <= 1e-4


def test_dw1d_backward_empty_batch():
    x = torch.empty(0, 16, 8, device="cuda")
    w = torch.randn(8, 1, 3, device="cuda")
    dy = torch.empty(0, 16, 8, device="cuda")
    dx, dw, db = gc.dwconv1d_btc_backward(x, w, dy, stride=1, padding=1)
    torch.cuda.synchronize()
    assert tuple(dx.shape) == (0, 16, 8)
    assert bool((dw == 0).all()) and bool((db == 0).all())


# ---------------------------------------------------------------- the five workloads at full size

def _sample_idx(total, n, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, total, n)
    return np.unique(np.concatenate([idx, [0, total - 1]]))


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workload_full_size(name):
    wl = WORKLOADS[name]
    x, w, b = make_inputs(wl)
    if wl.layout == "ntc":
        y = gc.gconv_fwd(gpu(x), gpu(w), gpu(b), wl.stride, wl.pad, wl.dilation, wl.groups, "ntc")
    else:
        y = gc.gconv_fwd(gpu(x), gpu(w), gpu(b), wl.stride, wl.pad, wl.dilation, wl.groups, "nchw")
    torch.cuda.synchronize()
    yc = as_f64(y.cpu())
    xd, wd, bd = as_f64(x), as_f64(w), as_f64(b)
    macs = int(np.prod(yc.shape)) * int(np.prod(wl.w_shape[1:]))
    # In full where the oracle finishes in seconds, and for the ensemble layer
    # (51.4 M outputs, about 30 G multiply-adds: some 15 s on 16 cores); the two
    # headline layers (38.7 G multiply-adds each) on a sample here, the fp16 one in
    # full in test_igemm_rows_gpu.py.
    if macs <= 3e8 or name == "c5_ensemble_f16":
        if wl.layout == "ntc":
            r = oracle.dwconv1d_btc(xd, wd, bd, wl.stride, wl.pad, wl.dilation)
        else:
            r = oracle.conv2d(xd, wd, bd, wl.stride, wl.pad, wl.dilation, wl.groups)
        err = normwise(yc, r)
        ew = elementwise(yc, r)
    else:
        idx = _sample_idx(yc.size, 20000, 4242 + wl.index)
        r = oracle.conv2d_at(xd, wd, idx, bd, wl.stride, wl.pad, wl.dilation, wl.groups)
        err = normwise(yc.ravel()[idx], r)
        ew = elementwise(yc.ravel()[idx], r)
    print(f"{name}: kernel={gc.gconv_last_kernel()} normwise err={err:.3e} "
          f"elementwise over |r| > 1e-3 max|r| {ew:.3e}")
    assert err <= TOL[wl.dtype] and err <= REG[wl.dtype]


@pytest.mark.parametrize("name", sorted(NEXT_WORKLOADS))
def test_next_workload_full_size(name):
    # The strided depthwise layers at full size, on 20 000 sampled outputs (plus the
    # first and the last), each evaluated one by one by the oracle.
    wl = NEXT_WORKLOADS[name]
    x, w, b = make_inputs(wl)
    y = gc.gconv_fwd(gpu(x), gpu(w), gpu(b), wl.stride, wl.pad, wl.dilation, wl.groups, wl.layout)
    torch.cuda.synchronize()
    yc = as_f64(y.cpu())
    xd, wd, bd = as_f64(x), as_f64(w), as_f64(b)
    idx = _sample_idx(yc.size, 20000, 4343 + wl.index)
    if wl.layout == "ntc":
        r = oracle.dwconv1d_btc_at(xd, wd, idx, bd, wl.stride, wl.pad, wl.dilation)
        assert gc.gconv_last_kernel() == "dw1d_btc_tile"
    elif wl.layout == "nhwc":
        r = oracle.conv2d_nhwc_at(xd, wd, idx, bd, wl.stride, wl.pad, wl.dilation, wl.groups)
        # the 4-in/4-out layers here are 16-bit, 3 x 3, unit stride and dilation, 14 x 14
        dwk = "dw2d_nhwc_pair" if wl.dtype != "f32" else "dw2d_nhwc_tile"
        expect = {1: dwk, 4: "conv2d_nhwc_g4_mfma"}.get(wl.w_shape[3], "igemm_nhwc_mfma32x32x16")
        assert gc.gconv_last_kernel() == expect
    else:
        r = oracle.conv2d_at(xd, wd, idx, bd, wl.stride, wl.pad, wl.dilation, wl.groups)
        N, C, H, W = wl.x_shape
        assert gc.gconv_last_kernel() == dw2d_kernel(N, C, wl.w_shape[0] // C, H, W, wl.w_shape[2],
                                                     wl.stride, wl.pad, wl.dtype)
    err = normwise(yc.ravel()[idx], r)
    print(f"{name}: kernel={gc.gconv_last_kernel()} normwise err={err:.3e} "
          f"elementwise over |r| > 1e-3 max|r| {elementwise(yc.ravel()[idx], r):.3e}")
    assert err <= TOL[wl.dtype] and err <= REG[wl.dtype]


# ---------------------------------------------------------------- properties

@pytest.mark.parametrize("name", ["c2_p2layer_f16", "c4_fullgroup_bf16", "c3_dw1d_btc_f32"])
def test_deterministic(name):
    wl = WORKLOADS[name]
    x, w, b = (gpu(t) for t in make_inputs(wl))
    y1 = gc.gconv_fwd(x, w, b, wl.stride, wl.pad, wl.dilation, wl.groups, wl.layout)
    y2 = gc.gconv_fwd(x, w, b, wl.stride, wl.pad, wl.dilation, wl.groups, wl.layout)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16 if y1.element_size() == 2 else torch.int32),
                       y2.view(torch.int16 if y2.element_size() == 2 else torch.int32))


def test_error_leaves_output_untouched():
    x = torch.randn(1, 6, 5, 5, device="cuda")
    w = torch.randn(6, 3, 3, 3, device="cuda")   # wrong: C/groups = 2
    y = torch.full((1, 6, 5, 5), 7.0, device="cuda")
    with pytest.raises(gc.GconvError):
        gc.gconv_fwd(x, w, None, 1, 1, 1, 3, "nchw", y=y)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())


def test_zero_batch_returns_empty():
    x = torch.randn(0, 8, 5, 5, device="cuda", dtype=torch.float16)
    w = torch.randn(8, 2, 3, 3, device="cuda", dtype=torch.float16)
    y = gc.conv2d(x, w, padding=1, groups=4)
    assert tuple(y.shape) == (0, 8, 5, 5)


def test_runs_on_a_side_stream():
    wl = WORKLOADS["c1_g4_f32"]
    x, w, b = make_inputs(wl)
    r = oracle.conv2d(as_f64(x), as_f64(w), None, 1, 1, 1, 4)
    s = torch.cuda.Stream()
    xg, wg = gpu(x), gpu(w)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y = gc.conv2d(xg, wg, padding=1, groups=4)
    s.synchronize()
    assert normwise(as_f64(y.cpu()), r) <= 1e-4
