"""ctypes binding of libgconv.so: argument marshalling only.

Every function here checks and converts its arguments, then calls the C entry
point of the same name in libgconv.so (declared in include/gconv.h).  No
arithmetic of the convolution happens in Python; torch supplies device memory,
the current device and the current HIP stream.  If libgconv.so is missing the
first call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgconv.so")

OK, ERR_INVALID_ARG, ERR_SHAPE, ERR_UNSUPPORTED, ERR_LAUNCH = 0, 1, 2, 3, 4
LAYOUTS = {"nchw": 0, "ntc": 1, "nhwc": 2}
DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
DTYPE_NAMES = {"f32": 0, "f16": 1, "bf16": 2}
ROUTES = {"auto": 0, "direct": 1, "igemm": 2}
ROUTE_NAMES = {v: k for k, v in ROUTES.items()}
ORDERS = {"grouped": 0, "interleaved": 1}

# Every symbol include/gconv.h declares.
EXPORTS = ("gconv_out_shape", "gconv_select_route", "gconv_fwd", "gconv_fwd_route", "gconv_fwd_ex",
           "gconv_dw1d_bwd_data", "gconv_dw1d_bwd_filter_workspace", "gconv_dw1d_bwd_filter",
           "gconv_dw1d_bwd_filter_noalloc",
           "gconv_autotune", "gconv_autotune_clear",
           "gconv_last_kernel", "gconv_status_string", "gconv_last_error")

_i32, _i64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
_i64p, _i32p = ctypes.POINTER(_i64), ctypes.POINTER(_i32)

_lib = None


class GconvError(ValueError):
    """Argument, shape or coverage error reported by libgconv (status 1-3)."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"gconv status {status}: {detail}")
        self.status = status


class GconvLaunchError(RuntimeError):
    """The HIP runtime failed to launch a libgconv kernel (status 4)."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"gconv status {status}: {detail}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libgconv.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m depthwise_convolution_gconv_amd.build` (no fallback exists)")
        L = ctypes.CDLL(_LIB_PATH)
        conv = [_vp, _i64p, _vp, _i64p, _vp, _vp, _i32p, _i32p, _i32p, _i32, _i32, _i32]
        L.gconv_fwd.argtypes = conv + [_vp]
        L.gconv_fwd.restype = _i32
        L.gconv_fwd_route.argtypes = conv + [_i32, _vp]
        L.gconv_fwd_route.restype = _i32
        L.gconv_fwd_ex.argtypes = conv + [_i32, _i32, _vp]
        L.gconv_fwd_ex.restype = _i32
        L.gconv_out_shape.argtypes = [_i64p, _i64p, _i32p, _i32p, _i32p, _i32, _i32, _i64p]
        L.gconv_out_shape.restype = _i32
        L.gconv_select_route.argtypes = [_i64p, _i64p, _i32p, _i32p, _i32p, _i32, _i32, _i32, _i32p]
        L.gconv_select_route.restype = _i32
        L.gconv_dw1d_bwd_data.argtypes = [_vp, _i64p, _vp, _i64p, _vp, _i32p, _i32p, _i32p, _i32, _vp]
        L.gconv_dw1d_bwd_data.restype = _i32
        L.gconv_dw1d_bwd_filter_workspace.argtypes = [_i64p, _i64p, _i32p, _i32p, _i32p, _i32,
                                                      ctypes.POINTER(ctypes.c_size_t)]
        L.gconv_dw1d_bwd_filter_workspace.restype = _i32
        L.gconv_dw1d_bwd_filter.argtypes = [_vp, _i64p, _vp, _i64p, _vp, _vp, _i32p, _i32p, _i32p, _i32,
                                            _vp, ctypes.c_size_t, _vp]
        L.gconv_dw1d_bwd_filter.restype = _i32
        L.gconv_dw1d_bwd_filter_noalloc.argtypes = [_vp, _i64p, _vp, _i64p, _vp, _vp, _i32p, _i32p, _i32p, _i32,
                                                    _vp]
        L.gconv_dw1d_bwd_filter_noalloc.restype = _i32
        L.gconv_autotune.argtypes = conv + [_i32, _vp, _i32p]
        L.gconv_autotune.restype = _i32
        L.gconv_autotune_clear.argtypes = []
        L.gconv_autotune_clear.restype = None
        L.gconv_last_kernel.argtypes = []
        L.gconv_last_kernel.restype = ctypes.c_char_p
        L.gconv_status_string.argtypes = [_i32]
        L.gconv_status_string.restype = ctypes.c_char_p
        L.gconv_last_error.argtypes = []
        L.gconv_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status == OK:
        return
    L = lib()
    detail = L.gconv_last_error().decode() or L.gconv_status_string(status).decode()
    if status == ERR_LAUNCH:
        raise GconvLaunchError(status, detail)
    raise GconvError(status, detail)


def _arr(ctype, vals):
    vals = list(vals)
    return (ctype * max(len(vals), 1))(*vals)


def _geom(layout: str, stride, pad, dilation):
    n = 1 if layout == "ntc" else 2

    def norm(v):
        if isinstance(v, (tuple, list)):
            if len(v) != n:
                raise GconvError(ERR_INVALID_ARG, f"expected {n} values, got {v}")
            return [int(t) for t in v]
        return [int(v)] * n
    return _arr(_i32, norm(stride)), _arr(_i32, norm(pad)), _arr(_i32, norm(dilation))


def _layout(layout: str) -> int:
    if layout not in LAYOUTS:
        raise GconvError(ERR_INVALID_ARG, f"unknown layout {layout!r}")
    return LAYOUTS[layout]


def gconv_out_shape(x_shape: Sequence[int], w_shape: Sequence[int], stride=1, pad=0, dilation=1,
                    groups: int = 1, layout: str = "nchw") -> Tuple[int, ...]:
    """Output shape from the library's own host validation (no device work)."""
    L = lib()
    s, p, d = _geom(layout, stride, pad, dilation)
    lay = _layout(layout)
    out = (_i64 * 4)()
    _check(L.gconv_out_shape(_arr(_i64, x_shape), _arr(_i64, w_shape), s, p, d, int(groups), lay, out))
    return tuple(int(v) for v in out[: (3 if layout == "ntc" else 4)])


def gconv_select_route(x_shape, w_shape, stride=1, pad=0, dilation=1, groups: int = 1,
                       layout: str = "nchw", dtype: Union[str, torch.dtype] = "f16") -> str:
    """The route ("direct" or "igemm") that route="auto" takes for this geometry."""
    L = lib()
    s, p, d = _geom(layout, stride, pad, dilation)
    dt = DTYPES[dtype] if isinstance(dtype, torch.dtype) else DTYPE_NAMES[dtype]
    r = _i32(-1)
    _check(L.gconv_select_route(_arr(_i64, x_shape), _arr(_i64, w_shape), s, p, d, int(groups),
                                _layout(layout), dt, ctypes.byref(r)))
    return ROUTE_NAMES[r.value]


def _call(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor], y: Optional[torch.Tensor],
          stride, pad, dilation, groups: int, layout: str, route: Optional[str],
          stream: Optional[torch.cuda.Stream], out_order: Optional[str] = None) -> torch.Tensor:
    L = lib()
    for name, t in (("x", x), ("w", w), ("bias", bias), ("y", y)):
        if t is None:
            continue
        if not t.is_cuda:
            raise GconvError(ERR_INVALID_ARG, f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise GconvError(ERR_INVALID_ARG, f"{name} must be contiguous")
        if t.dtype != x.dtype:
            raise GconvError(ERR_INVALID_ARG, f"{name} dtype {t.dtype} differs from x dtype {x.dtype}")
        if t.device != x.device:
            raise GconvError(ERR_INVALID_ARG, f"{name} is on {t.device}, x on {x.device}")
    if x.dtype not in DTYPES:
        raise GconvError(ERR_INVALID_ARG, f"unsupported dtype {x.dtype}")
    expect_dims = 3 if layout == "ntc" else 4
    if x.dim() != expect_dims or w.dim() != expect_dims:
        raise GconvError(ERR_INVALID_ARG, f"{layout} expects {expect_dims}-D x and w")
    if bias is not None and (bias.dim() != 1 or bias.shape[0] != w.shape[0]):
        raise GconvError(ERR_SHAPE, "bias must have shape [w.shape[0]]")
    yshape = gconv_out_shape(tuple(x.shape), tuple(w.shape), stride, pad, dilation, groups, layout)
    if y is None:
        y = torch.empty(yshape, dtype=x.dtype, device=x.device)
    elif tuple(y.shape) != yshape:
        raise GconvError(ERR_SHAPE, f"y has shape {tuple(y.shape)}, expected {yshape}")
    s, p, d = _geom(layout, stride, pad, dilation)
    with torch.cuda.device(x.device):
        st = stream if stream is not None else torch.cuda.current_stream(x.device)
        args = [_vp(x.data_ptr()), _arr(_i64, x.shape), _vp(w.data_ptr()), _arr(_i64, w.shape),
                _vp(bias.data_ptr() if bias is not None else 0), _vp(y.data_ptr()), s, p, d, int(groups),
                _layout(layout), DTYPES[x.dtype]]
        if out_order is not None:
            if out_order not in ORDERS or (route or "auto") not in ROUTES:
                raise GconvError(ERR_INVALID_ARG, f"unknown output order {out_order!r} or route {route!r}")
            _check(L.gconv_fwd_ex(*args, ROUTES[route or "auto"], ORDERS[out_order], _vp(st.cuda_stream)))
        elif route is None:
            _check(L.gconv_fwd(*args, _vp(st.cuda_stream)))
        else:
            if route not in ROUTES:
                raise GconvError(ERR_INVALID_ARG, f"unknown route {route!r}")
            _check(L.gconv_fwd_route(*args, ROUTES[route], _vp(st.cuda_stream)))
    return y


def gconv_fwd(x, w, bias=None, stride=1, pad=0, dilation=1, groups: int = 1, layout: str = "nchw",
              y=None, stream=None) -> torch.Tensor:
    """Grouped convolution forward (route chosen per shape).  Returns y."""
    return _call(x, w, bias, y, stride, pad, dilation, groups, layout, None, stream)


def gconv_fwd_route(x, w, bias=None, stride=1, pad=0, dilation=1, groups: int = 1, layout: str = "nchw",
                    route: str = "auto", y=None, stream=None) -> torch.Tensor:
    """gconv_fwd with the route ("auto", "direct", "igemm") forced."""
    return _call(x, w, bias, y, stride, pad, dilation, groups, layout, route, stream)


def gconv_fwd_ex(x, w, bias=None, stride=1, pad=0, dilation=1, groups: int = 1, layout: str = "nchw",
                 route: str = "auto", out_order: str = "grouped", y=None, stream=None) -> torch.Tensor:
    """gconv_fwd with the route and the output-channel order ("grouped": filter j of
    group k at channel k*Cout/g + j; "interleaved": at channel j*g + k) chosen."""
    return _call(x, w, bias, y, stride, pad, dilation, groups, layout, route, stream, out_order)


def gconv_autotune(x, w, bias=None, stride=1, pad=0, dilation=1, groups: int = 1, layout: str = "nchw",
                   reps: int = 3, y=None, stream=None) -> str:
    """Times every route that can run this call on these tensors (synchronising the
    stream) and records the fastest for the geometry; returns its name.  y (allocated
    when None) is overwritten with the chosen route's result."""
    _check_tensors(x, w=w, bias=bias, y=y)
    yshape = gconv_out_shape(tuple(x.shape), tuple(w.shape), stride, pad, dilation, groups, layout)
    if y is None:
        y = torch.empty(yshape, dtype=x.dtype, device=x.device)
    elif tuple(y.shape) != yshape:
        raise GconvError(ERR_SHAPE, f"y has shape {tuple(y.shape)}, expected {yshape}")
    s, p, d = _geom(layout, stride, pad, dilation)
    best = _i32(-1)
    with torch.cuda.device(x.device):
        st = stream if stream is not None else torch.cuda.current_stream(x.device)
        _check(lib().gconv_autotune(_vp(x.data_ptr()), _arr(_i64, x.shape), _vp(w.data_ptr()), _arr(_i64, w.shape),
                                    _vp(bias.data_ptr() if bias is not None else 0), _vp(y.data_ptr()), s, p, d,
                                    int(groups), _layout(layout), DTYPES[x.dtype], int(reps),
                                    _vp(st.cuda_stream), ctypes.byref(best)))
    return ROUTE_NAMES[best.value]


def gconv_autotune_clear() -> None:
    lib().gconv_autotune_clear()


def gconv_last_kernel() -> str:
    return lib().gconv_last_kernel().decode()


def gconv_status_string(status: int) -> str:
    return lib().gconv_status_string(int(status)).decode()


def gconv_last_error() -> str:
    return lib().gconv_last_error().decode()


# ---- convenience spellings ------------------------------------------------

def conv2d(x, weight, bias=None, stride=1, padding=0, dilation=1, groups: int = 1, route: str = "auto"):
    """F.conv2d-style call: x [N,C,H,W], weight [Cout,C/groups,KH,KW]."""
    return _call(x, weight, bias, None, stride, padding, dilation, groups, "nchw",
                 None if route == "auto" else route, None)


def conv2d_nhwc(x, weight, bias=None, stride=1, padding=0, dilation=1, groups: int = 1):
    """Grouped conv2d over channels-last tensors: x [N,H,W,C], weight [Cout,KH,KW,C/groups];
    returns y [N,OH,OW,Cout]."""
    return _call(x, weight, bias, None, stride, padding, dilation, groups, "nhwc", None, None)


def dwconv1d_btc(x, weight, bias=None, stride=1, padding=0, dilation=1):
    """Depthwise conv1d over x [B,T,C] (batch, steps, channels), weight [C,1,K]."""
    return _call(x, weight, bias, None, stride, padding, dilation, x.shape[-1], "ntc", None, None)


# ---- backward of the depthwise conv1d over (batch, steps, channels) -----------

def _check_tensors(ref: torch.Tensor, **ts):
    for name, t in ts.items():
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise GconvError(ERR_INVALID_ARG, f"{name} must be a contiguous GPU tensor")
        if t.dtype != ref.dtype or t.device != ref.device:
            raise GconvError(ERR_INVALID_ARG, f"{name} must match the dtype and device of the other tensors")
    if ref.dtype not in DTYPES:
        raise GconvError(ERR_INVALID_ARG, f"unsupported dtype {ref.dtype}")


def gconv_dw1d_bwd_data(dy, w, T: int, stride=1, pad=0, dilation=1, dx=None, stream=None) -> torch.Tensor:
    """Input gradient [B,T,C] of the (batch, steps, channels) depthwise conv1d, from
    dy [B,To,C] and w [C,1,K].  Returns dx."""
    _check_tensors(dy, w=w, dx=dx)
    B, _, C = dy.shape
    x_shape = (B, int(T), C)
    if dx is None:
        dx = torch.empty(x_shape, dtype=dy.dtype, device=dy.device)
    elif tuple(dx.shape) != x_shape:
        raise GconvError(ERR_SHAPE, f"dx has shape {tuple(dx.shape)}, expected {x_shape}")
    yshape = gconv_out_shape(x_shape, tuple(w.shape), stride, pad, dilation, C, "ntc")
    if tuple(dy.shape) != yshape:
        raise GconvError(ERR_SHAPE, f"dy has shape {tuple(dy.shape)}, expected {yshape}")
    s, p, d = _geom("ntc", stride, pad, dilation)
    with torch.cuda.device(dy.device):
        st = stream if stream is not None else torch.cuda.current_stream(dy.device)
        _check(lib().gconv_dw1d_bwd_data(_vp(dy.data_ptr()), _arr(_i64, x_shape), _vp(w.data_ptr()),
                                         _arr(_i64, w.shape), _vp(dx.data_ptr()), s, p, d, DTYPES[dy.dtype],
                                         _vp(st.cuda_stream)))
    return dx


def gconv_dw1d_bwd_filter_workspace(x_shape, w_shape, stride=1, pad=0, dilation=1, dtype="f32") -> int:
    """Workspace bytes gconv_dw1d_bwd_filter needs (no device work)."""
    s, p, d = _geom("ntc", stride, pad, dilation)
    dt = DTYPES[dtype] if isinstance(dtype, torch.dtype) else DTYPE_NAMES[dtype]
    n = ctypes.c_size_t(0)
    _check(lib().gconv_dw1d_bwd_filter_workspace(_arr(_i64, x_shape), _arr(_i64, w_shape), s, p, d, dt,
                                                 ctypes.byref(n)))
    return int(n.value)


def gconv_dw1d_bwd_filter(x, dy, K: int, stride=1, pad=0, dilation=1, bias: bool = True, dw=None, db=None,
                          workspace=None, stream=None):
    """Filter gradient [C,1,K] (and bias gradient [C] if `bias`) of the (batch, steps,
    channels) depthwise conv1d, from x [B,T,C] and dy [B,To,C].  The fp32 workspace is
    allocated with torch.empty when not given.  Returns (dw, db or None)."""
    _check_tensors(x, dy=dy, dw=dw, db=db)
    B, T, C = x.shape
    w_shape = (C, 1, int(K))
    yshape = gconv_out_shape(tuple(x.shape), w_shape, stride, pad, dilation, C, "ntc")
    if tuple(dy.shape) != yshape:
        raise GconvError(ERR_SHAPE, f"dy has shape {tuple(dy.shape)}, expected {yshape}")
    if dw is None:
        dw = torch.empty(w_shape, dtype=x.dtype, device=x.device)
    if bias and db is None:
        db = torch.empty((C,), dtype=x.dtype, device=x.device)
    if tuple(dw.shape) != w_shape or (db is not None and tuple(db.shape) != (C,)):
        raise GconvError(ERR_SHAPE, "dw must be [C,1,K] and db [C]")
    need = gconv_dw1d_bwd_filter_workspace(tuple(x.shape), w_shape, stride, pad, dilation, x.dtype)
    own_ws = workspace is None
    if own_ws:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=x.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise GconvError(ERR_INVALID_ARG, "workspace must be a contiguous GPU tensor")
    s, p, d = _geom("ntc", stride, pad, dilation)
    with torch.cuda.device(x.device):
        st = stream if stream is not None else torch.cuda.current_stream(x.device)
        if own_ws and stream is not None:
            # The kernels use the workspace on `stream`: the caching allocator must
            # not hand its memory out again before that stream's work is done.
            workspace.record_stream(st)
        _check(lib().gconv_dw1d_bwd_filter(_vp(x.data_ptr()), _arr(_i64, x.shape), _vp(dy.data_ptr()),
                                           _arr(_i64, w_shape), _vp(dw.data_ptr()),
                                           _vp(db.data_ptr() if db is not None else 0), s, p, d,
                                           DTYPES[x.dtype], _vp(workspace.data_ptr()),
                                           workspace.numel() * workspace.element_size(), _vp(st.cuda_stream)))
    return dw, db


# Bytes of the library's own device scratch behind gconv_dw1d_bwd_filter_noalloc
# (GCONV_DW1D_BWD_FILTER_SCRATCH_BYTES in gconv.h).
DW1D_BWD_FILTER_SCRATCH_BYTES = 16 << 20


def gconv_dw1d_bwd_filter_noalloc(x, dy, K: int, stride=1, pad=0, dilation=1, dw=None, db=None, bias: bool = True,
                                  stream=None):
    """gconv_dw1d_bwd_filter through the entry point that allocates nothing: the
    partial sums go to the library's per-GPU scratch array.  dw (and db when
    `bias`) must be passed in: this call allocates no tensor either.  Calls that
    overlap on one GPU race.  Returns (dw, db or None)."""
    _check_tensors(x, dy=dy, dw=dw, db=db)
    if dw is None or (bias and db is None):
        raise GconvError(ERR_INVALID_ARG, "dw (and db when bias=True) must be given")
    B, T, C = x.shape
    w_shape = (C, 1, int(K))
    if tuple(dw.shape) != w_shape or (db is not None and tuple(db.shape) != (C,)):
        raise GconvError(ERR_SHAPE, "dw must be [C,1,K] and db [C]")
    if tuple(dy.shape[:1]) != (B,) or dy.dim() != 3 or dy.shape[2] != C:
        raise GconvError(ERR_SHAPE, f"dy has shape {tuple(dy.shape)}, expected [{B}, To, {C}]")
    s, p, d = _geom("ntc", stride, pad, dilation)
    with torch.cuda.device(x.device):
        st = stream if stream is not None else torch.cuda.current_stream(x.device)
        _check(lib().gconv_dw1d_bwd_filter_noalloc(_vp(x.data_ptr()), _arr(_i64, x.shape), _vp(dy.data_ptr()),
                                                   _arr(_i64, w_shape), _vp(dw.data_ptr()),
                                                   _vp(db.data_ptr() if db is not None else 0), s, p, d,
                                                   DTYPES[x.dtype], _vp(st.cuda_stream)))
    return dw, db


def dwconv1d_btc_backward(x, weight, dy, stride=1, padding=0, dilation=1, bias: bool = True):
    """(dx, dw, db) of dwconv1d_btc: the input, filter and bias gradients."""
    dx = gconv_dw1d_bwd_data(dy, weight, x.shape[1], stride, padding, dilation)
    dw, db = gconv_dw1d_bwd_filter(x, dy, weight.shape[2], stride, padding, dilation, bias=bias)
    return dx, dw, db


class PreparedCall:
    """gconv_fwd / gconv_fwd_route with its arguments marshalled once.

    For repeated calls on the same tensors (benchmark loops): each __call__ only
    invokes the C entry point with the stored ctypes arguments and checks the
    status.  The tensors must stay alive and unchanged in shape while it is used.
    """

    def __init__(self, x, w, bias, y, stride=1, pad=0, dilation=1, groups: int = 1, layout: str = "nchw",
                 route: Optional[str] = None, stream=None):
        self._keep = (x, w, bias, y)
        yshape = gconv_out_shape(tuple(x.shape), tuple(w.shape), stride, pad, dilation, groups, layout)
        if tuple(y.shape) != yshape or not all(t is None or (t.is_cuda and t.is_contiguous() and
                                                             t.dtype == x.dtype) for t in self._keep):
            raise GconvError(ERR_INVALID_ARG, "tensors must be contiguous GPU tensors of one dtype "
                             "and y must have the output shape")
        s, p, d = _geom(layout, stride, pad, dilation)
        st = stream if stream is not None else torch.cuda.current_stream(x.device)
        self._fn = lib().gconv_fwd if route is None else lib().gconv_fwd_route
        args = [_vp(x.data_ptr()), _arr(_i64, x.shape), _vp(w.data_ptr()), _arr(_i64, w.shape),
                _vp(bias.data_ptr() if bias is not None else 0), _vp(y.data_ptr()), s, p, d, int(groups),
                _layout(layout), DTYPES[x.dtype]]
        if route is not None:
            args.append(ROUTES[route])
        args.append(_vp(st.cuda_stream))
        self._args = tuple(args)

    def __call__(self):
        _check(self._fn(*self._args))
