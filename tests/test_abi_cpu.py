"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/gconv.h declares, and its host-side validation, output shapes and route
selection behave as documented.  No call here enqueues device work: every
gconv_fwd call below is rejected by host validation before any HIP call."""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

import depthwise_convolution_gconv_amd as gc
from depthwise_convolution_gconv_amd import _binding as B
from depthwise_convolution_gconv_amd.workloads import WORKLOADS
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gconv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gconv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(gc.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {gc.lib_path()}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_status_strings():
    assert gc.gconv_status_string(0) == "ok"
    assert gc.gconv_status_string(3) == "unsupported convolution"
    assert gc.gconv_status_string(99) == "unknown status"


def test_out_shape_of_page_workload_golden():
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "page_workload_shapes.json")))
    for c in g["cases"]:
        assert list(gc.gconv_out_shape(c["x_shape"], c["w_shape"], 1, c["padding"], 1, c["groups"])) == c["y_shape"]


def test_out_shape_matches_oracle_lengths():
    for L, K, s, p, d in itertools.product(range(1, 9), range(1, 4), range(1, 4), range(0, 3), range(1, 3)):
        expect = oracle.out_len(L, K, s, p, d)
        if expect < 1:
            with pytest.raises(gc.GconvError) as e:
                gc.gconv_out_shape((1, 2, L, L), (2, 1, K, K), s, p, d, groups=2)
            assert e.value.status == 2
            continue
        assert gc.gconv_out_shape((1, 2, L, L), (4, 1, K, K), s, p, d, groups=2) == (1, 4, expect, expect)
        assert gc.gconv_out_shape((3, L, 5), (5, 1, K), s, p, d, groups=5, layout="ntc") == (3, expect, 5)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workload_shapes_and_routes(name):
    wl = WORKLOADS[name]
    ys = gc.gconv_out_shape(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dilation, wl.groups, wl.layout)
    if wl.layout == "nchw":
        assert ys == (wl.x_shape[0], wl.w_shape[0], wl.x_shape[2], wl.x_shape[3])
    else:
        assert ys == wl.x_shape
    route = gc.gconv_select_route(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dilation, wl.groups,
                                  wl.layout, wl.dtype)
    expected = {"c1_g4_f32": "direct", "c2_p2layer_f32": "igemm", "c2_p2layer_f16": "igemm",
                "c3_dw1d_btc_f32": "direct", "c4_fullgroup_bf16": "direct", "c5_ensemble_f16": "igemm"}
    assert route == expected[name]


def _raw_fwd(x_shape, w_shape, stride, pad, dil, groups, layout, dtype, x=16, w=4096, b=0, y=1 << 20,
             route=None):
    """Call the C entry point with fake (never dereferenced) device addresses."""
    L = gc.lib()
    arr64 = lambda v: (ctypes.c_int64 * len(v))(*v)
    arr32 = lambda v: (ctypes.c_int32 * len(v))(*v)
    args = [ctypes.c_void_p(x), arr64(x_shape), ctypes.c_void_p(w), arr64(w_shape), ctypes.c_void_p(b),
            ctypes.c_void_p(y), arr32(stride), arr32(pad), arr32(dil), groups, layout, dtype]
    if route is None:
        return L.gconv_fwd(*args, None)
    return L.gconv_fwd_route(*args, route, None)


@pytest.mark.parametrize("case,status", [
    (((1, 6, 5, 5), (4, 3, 3, 3), 4), 2),     # C % groups != 0
    (((1, 6, 5, 5), (5, 2, 3, 3), 3), 2),     # Cout % groups != 0
    (((1, 6, 5, 5), (6, 3, 3, 3), 3), 2),     # w.shape[1] != C/groups
    (((1, 6, 2, 2), (6, 2, 5, 5), 3), 2),     # empty output
    (((1, 6, 5, 5), (6, 2, 3, 3), 0), 1),     # groups < 1
    (((1, 0, 5, 5), (6, 2, 3, 3), 3), 1),     # C < 1
    (((-1, 6, 5, 5), (6, 2, 3, 3), 3), 1),    # N < 0
])
def test_nchw_validation_errors(case, status):
    xs, ws, g = case
    assert _raw_fwd(xs, ws, (1, 1), (0, 0), (1, 1), g, 0, 0) == status
    assert gc.gconv_last_error() != ""


def test_bad_enums_strides_and_pointers():
    ok = ((1, 4, 5, 5), (4, 1, 3, 3), (1, 1), (1, 1), (1, 1), 4)
    assert _raw_fwd(*ok, 0, 7) == 1                           # dtype
    assert _raw_fwd(*ok, 5, 0) == 1                           # layout
    assert _raw_fwd(*ok, 0, 0, route=9) == 1                  # route
    assert _raw_fwd(ok[0], ok[1], (0, 1), ok[3], ok[4], 4, 0, 0) == 1   # stride 0
    assert _raw_fwd(ok[0], ok[1], ok[2], (-1, 0), ok[4], 4, 0, 0) == 1  # negative pad
    assert _raw_fwd(ok[0], ok[1], ok[2], ok[3], (1, 0), 4, 0, 0) == 1   # dilation 0
    assert _raw_fwd(*ok, 0, 0, x=0) == 1                      # NULL x
    assert _raw_fwd(*ok, 0, 0, y=0) == 1                      # NULL y
    assert _raw_fwd(*ok, 0, 0, y=16) == 1                     # y overlaps x


def test_ntc_validation():
    # depthwise only: groups must equal C
    assert _raw_fwd((2, 10, 8), (8, 2, 3), (1,), (1,), (1,), 4, 1, 0) == 3
    # channel multiplier
    assert _raw_fwd((2, 10, 8), (16, 1, 3), (1,), (1,), (1,), 8, 1, 0) == 3
    # forced implicit GEMM on the NTC layout
    assert _raw_fwd((2, 10, 8), (8, 1, 3), (1,), (1,), (1,), 8, 1, 0, route=2) == 3
    # empty output
    assert _raw_fwd((2, 2, 8), (8, 1, 5), (1,), (0,), (1,), 8, 1, 0) == 2


def test_forced_igemm_rejected_outside_its_plan():
    # 5x5 kernels (fp32 and fp16) and fp32 groups of 2 channels are not covered by the
    # implicit-GEMM plans; forcing the route reports UNSUPPORTED before any launch.
    assert _raw_fwd((1, 64, 8, 8), (64, 64, 5, 5), (1, 1), (2, 2), (1, 1), 1, 0, 0, route=2) == 3
    assert _raw_fwd((1, 64, 8, 8), (64, 64, 5, 5), (1, 1), (2, 2), (1, 1), 1, 0, 1, route=2) == 3
    assert _raw_fwd((1, 64, 8, 8), (64, 2, 3, 3), (1, 1), (1, 1), (1, 1), 32, 0, 0, route=2) == 3


def test_zero_batch_enqueues_nothing():
    assert _raw_fwd((0, 4, 5, 5), (4, 1, 3, 3), (1, 1), (1, 1), (1, 1), 4, 0, 0) == 0
    assert gc.gconv_last_kernel() == ""
    assert _raw_fwd((0, 10, 8), (8, 1, 3), (1,), (1,), (1,), 8, 1, 0) == 0


def test_zero_batch_accepts_null_x_and_y():
    assert _raw_fwd((0, 4, 5, 5), (4, 1, 3, 3), (1, 1), (1, 1), (1, 1), 4, 0, 0, x=0, y=0) == 0
    assert _raw_fwd((0, 4, 5, 5), (4, 1, 3, 3), (1, 1), (1, 1), (1, 1), 4, 0, 0, w=0) == 1


# ---------------------------------------------------------------- backward of the depthwise conv1d

def _bwd_filter_call(ws_bytes, K=31, workspace=16):
    L = B.lib()
    s, p, d = B._geom("ntc", 1, 15, 1)
    return L.gconv_dw1d_bwd_filter(B._vp(16), B._arr(B._i64, (8, 1024, 512)), B._vp(1 << 20),
                                   B._arr(B._i64, (512, 1, K)), B._vp(1 << 24), B._vp(0), s, p, d, 0,
                                   B._vp(workspace), ws_bytes, B._vp(0))


def test_bwd_filter_workspace_size_is_per_tile_partials():
    # 8 x 1024 steps in tiles of 64: 128 tiles x (31 taps + the bias row) x 512 channels x 4 bytes.
    assert gc.gconv_dw1d_bwd_filter_workspace((8, 1024, 512), (512, 1, 31), 1, 15, 1, "f32") == 128 * 32 * 512 * 4
    assert gc.gconv_dw1d_bwd_filter_workspace((0, 1024, 512), (512, 1, 31), 1, 15, 1, "f32") == 0
    with pytest.raises(gc.GconvError) as e:
        gc.gconv_dw1d_bwd_filter_workspace((8, 1024, 512), (512, 1, 65), 1, 32, 1, "f32")
    assert e.value.status == B.ERR_UNSUPPORTED


def test_bwd_filter_rejects_a_short_or_misaligned_workspace_before_launch():
    need = gc.gconv_dw1d_bwd_filter_workspace((8, 1024, 512), (512, 1, 31), 1, 15, 1, "f32")
    assert _bwd_filter_call(need - 4) == B.ERR_INVALID_ARG
    assert "needed" in gc.gconv_last_error()
    assert _bwd_filter_call(need, workspace=18) == B.ERR_INVALID_ARG
    assert "aligned" in gc.gconv_last_error()


def test_bwd_data_rejects_bad_shapes_before_launch():
    L = B.lib()
    s, p, d = B._geom("ntc", 1, 1, 1)
    # w for 4 channels against x with 5: the forward's shape check.
    rc = L.gconv_dw1d_bwd_data(B._vp(16), B._arr(B._i64, (2, 10, 5)), B._vp(1 << 20), B._arr(B._i64, (4, 1, 3)),
                               B._vp(1 << 24), s, p, d, 0, B._vp(0))
    assert rc in (B.ERR_SHAPE, B.ERR_UNSUPPORTED)
    # dx overlapping dy.
    rc = L.gconv_dw1d_bwd_data(B._vp(1 << 20), B._arr(B._i64, (2, 10, 4)), B._vp(16), B._arr(B._i64, (4, 1, 3)),
                               B._vp((1 << 20) + 8), s, p, d, 0, B._vp(0))
    assert rc == B.ERR_INVALID_ARG


# ---------------------------------------------------------------- NHWC and output order (host logic)

def test_nhwc_route_selection():
    # The channels-last ensemble layer: the implicit GEMM in 16-bit, the direct route in fp32
    # (no fp32 NHWC implicit GEMM) and for depthwise layers.
    xs, ws = (64, 28, 28, 1024), (2048, 3, 3, 32)
    assert gc.gconv_select_route(xs, ws, 1, 1, 1, 32, "nhwc", "f16") == "igemm"
    assert gc.gconv_select_route(xs, ws, 1, 1, 1, 32, "nhwc", "bf16") == "igemm"
    assert gc.gconv_select_route(xs, ws, 1, 1, 1, 32, "nhwc", "f32") == "direct"
    assert gc.gconv_select_route((8, 512, 40, 256), (256, 3, 3, 1), 2, 1, 1, 256, "nhwc", "f16") == "direct"
    # 8 input channels per group: not the implicit GEMM.
    assert gc.gconv_select_route((2, 8, 8, 64), (64, 3, 3, 8), 1, 1, 1, 8, "nhwc", "f16") == "direct"


def test_nhwc_output_shape_and_weight_check():
    OH, OW = oracle.out_len(9, 3, 2, 1, 1), oracle.out_len(11, 2, 1, 0, 2)
    assert gc.gconv_out_shape((2, 9, 11, 12), (18, 3, 2, 4), (2, 1), (1, 0), (1, 2), 3, "nhwc") == (2, OH, OW, 18)
    with pytest.raises(gc.GconvError) as e:   # w's last axis must be C/groups
        gc.gconv_out_shape((2, 9, 11, 12), (18, 3, 3, 6), 1, 1, 1, 3, "nhwc")
    assert e.value.status == B.ERR_SHAPE


def test_unknown_output_order_is_rejected_before_launch():
    L = B.lib()
    s, p, d = B._geom("nchw", 1, 1, 1)
    rc = L.gconv_fwd_ex(B._vp(16), B._arr(B._i64, (1, 8, 5, 5)), B._vp(1 << 20), B._arr(B._i64, (8, 4, 3, 3)),
                        B._vp(0), B._vp(1 << 24), s, p, d, 2, 0, 0, 0, 7, B._vp(0))
    assert rc == B.ERR_INVALID_ARG
    assert "order" in gc.gconv_last_error()


def test_bwd_filter_noalloc_rejects_a_geometry_beyond_its_scratch_before_launch():
    # 64 x 1024 steps in tiles of 64 need 1024 x 32 x 512 x 4 bytes of partial sums,
    # more than the library's scratch array: rejected on the host (fake pointers).
    L = B.lib()
    need = gc.gconv_dw1d_bwd_filter_workspace((64, 1024, 512), (512, 1, 31), 1, 15, 1, "f32")
    assert need > gc.DW1D_BWD_FILTER_SCRATCH_BYTES
    s, p, d = B._geom("ntc", 1, 15, 1)
    st = L.gconv_dw1d_bwd_filter_noalloc(B._vp(16), B._arr(B._i64, (64, 1024, 512)), B._vp(1 << 30),
                                         B._arr(B._i64, (512, 1, 31)), B._vp(1 << 24), B._vp(0), s, p, d, 0,
                                         B._vp(0))
    assert st == B.ERR_UNSUPPORTED
    assert "scratch" in gc.gconv_last_error()
    # the Conformer shape fits
    assert gc.gconv_dw1d_bwd_filter_workspace((8, 1024, 512), (512, 1, 31), 1, 15, 1, "f32") <= \
        gc.DW1D_BWD_FILTER_SCRATCH_BYTES


def test_header_states_the_noalloc_scratch_size():
    text = open(os.path.join(ROOT, "include", "gconv.h")).read()
    m = re.search(r"#define GCONV_DW1D_BWD_FILTER_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == gc.DW1D_BWD_FILTER_SCRATCH_BYTES
