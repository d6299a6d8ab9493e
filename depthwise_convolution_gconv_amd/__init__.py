"""Grouped-convolution forward engine for AMD Instinct MI355X (gfx950), with the
backward of the (batch, steps, channels) depthwise conv1d.

The compute runs in libgconv.so (hand-written HIP kernels behind the C ABI in
include/gconv.h); this package is its Python binding.  Importing the package
does not load the library; the first call does, and raises if it is missing.
"""
from ._binding import (  # noqa: F401
    DW1D_BWD_FILTER_SCRATCH_BYTES,
    EXPORTS,
    GconvError,
    GconvLaunchError,
    PreparedCall,
    conv2d,
    conv2d_nhwc,
    dwconv1d_btc,
    dwconv1d_btc_backward,
    gconv_autotune,
    gconv_autotune_clear,
    gconv_dw1d_bwd_data,
    gconv_dw1d_bwd_filter,
    gconv_dw1d_bwd_filter_noalloc,
    gconv_dw1d_bwd_filter_workspace,
    gconv_fwd,
    gconv_fwd_ex,
    gconv_fwd_route,
    gconv_last_error,
    gconv_last_kernel,
    gconv_out_shape,
    gconv_select_route,
    gconv_status_string,
    lib,
    lib_path,
)
