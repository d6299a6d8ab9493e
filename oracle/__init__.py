"""fp64 CPU oracle for grouped convolution forward -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and it imports nothing from
the product package.

The arithmetic lives in ``gconv_oracle.c`` (plain nested loops, fp64
accumulation); this module only builds that file with gcc and marshals numpy
arrays into it.  Every array passed in is converted to float64 first, so
fp16/bf16/fp32 inputs enter the oracle exactly.

Sources followed (cited by page title and the reply or code block on it):

* neon issue "Grouped convolutions", thestew42's first reply: channels, filters
  and outputs are split into groups with no connections between groups;
  ibmua's reply on output ordering: the usual order is group-contiguous.
* discuss.pytorch.org "F.conv2d runs x15 slower in mixed-precision/half-precision
  mode", the test script: ``F.conv2d(input, weight, padding=3 // 2, groups=4)``
  -- cross-correlation with symmetric zero padding; its later replies turn to the
  NHWC (channels_last) memory format (``conv2d_nhwc``: the same sum over
  x [N,H,W,C], w [Cout,KH,KW,C/g], y [N,OH,OW,Cout]).
* speechbrain issue #2733 "Investigate custom Triton kernels for
  depthwise-separable convolutions in Conformer": depthwise conv with groups equal
  to the channel count, over a (batch, steps, channels) tensor; in its follow-up
  comments the author also writes the backward pass of that conv (the gradients
  with respect to the input, the filters and the bias, ``dwconv1d_btc_bwd_*``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gconv_oracle.c")
_LIB = os.path.join(_HERE, "libgconv_oracle.so")

_i64 = ctypes.c_int64
_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)

_lib = None


def build(force: bool = True) -> str:
    """Compile gconv_oracle.c into libgconv_oracle.so with gcc -O2 -fopenmp."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                        "-Wall", "-Werror", _SRC, "-o", tmp], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.gconv_oracle_out_len.restype = _i64
        lib.gconv_oracle_out_len.argtypes = [_i64] * 5
        lib.gconv_oracle_num_threads.restype = ctypes.c_int
        lib.gconv_oracle_num_threads.argtypes = []
        conv_args = [_dp, _i64, _i64, _i64, _i64, _dp, _i64, _i64, _i64, _i64, _dp, _i64,
                     _i64, _i64, _i64, _i64, _i64, _i64]
        lib.gconv_oracle_conv2d.restype = ctypes.c_int
        lib.gconv_oracle_conv2d.argtypes = conv_args + [_dp]
        lib.gconv_oracle_conv2d_at.restype = ctypes.c_int
        lib.gconv_oracle_conv2d_at.argtypes = conv_args + [_ip, _i64, _dp]
        dw_args = [_dp, _i64, _i64, _i64, _dp, _i64, _dp, _i64, _i64, _i64]
        lib.gconv_oracle_dwconv1d_btc.restype = ctypes.c_int
        lib.gconv_oracle_dwconv1d_btc.argtypes = dw_args + [_dp]
        lib.gconv_oracle_dwconv1d_btc_at.restype = ctypes.c_int
        lib.gconv_oracle_dwconv1d_btc_at.argtypes = dw_args + [_ip, _i64, _dp]
        lib.gconv_oracle_conv2d_interleaved.restype = ctypes.c_int
        lib.gconv_oracle_conv2d_interleaved.argtypes = conv_args + [_dp]
        lib.gconv_oracle_conv2d_nhwc.restype = ctypes.c_int
        lib.gconv_oracle_conv2d_nhwc.argtypes = conv_args + [_dp]
        lib.gconv_oracle_conv2d_nhwc_at.restype = ctypes.c_int
        lib.gconv_oracle_conv2d_nhwc_at.argtypes = conv_args + [_ip, _i64, _dp]
        bwd_args = [_dp, _i64, _i64, _i64, _dp, _i64, _i64, _i64, _i64]
        lib.gconv_oracle_dwconv1d_btc_bwd_data.restype = ctypes.c_int
        lib.gconv_oracle_dwconv1d_btc_bwd_data.argtypes = bwd_args + [_dp]
        lib.gconv_oracle_dwconv1d_btc_bwd_data_at.restype = ctypes.c_int
        lib.gconv_oracle_dwconv1d_btc_bwd_data_at.argtypes = bwd_args + [_ip, _i64, _dp]
        lib.gconv_oracle_dwconv1d_btc_bwd_filter.restype = ctypes.c_int
        lib.gconv_oracle_dwconv1d_btc_bwd_filter.argtypes = [_dp, _dp] + [_i64] * 7 + [_dp, _dp]
        _lib = lib
    return _lib


def _f64(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    return a, a.ctypes.data_as(_dp)


def _pair(v):
    if isinstance(v, (tuple, list)):
        assert len(v) == 2
        return int(v[0]), int(v[1])
    return int(v), int(v)


def num_threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().gconv_oracle_num_threads())


def out_len(L: int, K: int, stride: int = 1, padding: int = 0, dilation: int = 1) -> int:
    """Output length along one axis (-1 for invalid arguments, 0 for empty)."""
    return int(_load().gconv_oracle_out_len(L, K, stride, padding, dilation))


def _rc(rc: int):
    if rc == 1:
        raise ValueError("oracle: invalid argument")
    if rc == 2:
        raise ValueError("oracle: output would be empty")


def conv2d(x, w, bias=None, stride=1, padding=0, dilation=1, groups=1,
           out_order: str = "grouped") -> np.ndarray:
    """Grouped conv2d forward in fp64.  x [N,C,H,W], w [Cout,C/groups,KH,KW].
    out_order "interleaved": filter j of group k goes to output channel j*groups + k
    (the neon issue's 1234... order) instead of k*Cout/groups + j."""
    lib = _load()
    x, xp = _f64(x)
    w, wp = _f64(w)
    N, C, H, W = x.shape
    Cout, Cg_w, KH, KW = w.shape
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    bp = None
    if bias is not None:
        bias, bp = _f64(bias)
        assert bias.shape == (Cout,)
    OH = out_len(H, KH, sh, ph, dh)
    OW = out_len(W, KW, sw, pw, dw)
    y = np.zeros((N, Cout, max(OH, 0), max(OW, 0)), dtype=np.float64)
    if out_order not in ("grouped", "interleaved"):
        raise ValueError("oracle: out_order must be 'grouped' or 'interleaved'")
    fn = lib.gconv_oracle_conv2d if out_order == "grouped" else lib.gconv_oracle_conv2d_interleaved
    _rc(fn(xp, N, C, H, W, wp, Cout, Cg_w, KH, KW, bp, groups, sh, sw, ph, pw, dh, dw,
           y.ctypes.data_as(_dp)))
    return y


def conv2d_at(x, w, flat_idx, bias=None, stride=1, padding=0, dilation=1, groups=1) -> np.ndarray:
    """The elements y.flat[flat_idx] of conv2d(...), evaluated one by one."""
    lib = _load()
    x, xp = _f64(x)
    w, wp = _f64(w)
    N, C, H, W = x.shape
    Cout, Cg_w, KH, KW = w.shape
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    bp = None
    if bias is not None:
        bias, bp = _f64(bias)
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    out = np.zeros(idx.shape, dtype=np.float64)
    _rc(lib.gconv_oracle_conv2d_at(xp, N, C, H, W, wp, Cout, Cg_w, KH, KW, bp, groups,
                                   sh, sw, ph, pw, dh, dw, idx.ctypes.data_as(_ip), idx.size,
                                   out.ctypes.data_as(_dp)))
    return out


def dwconv1d_btc(x, w, bias=None, stride=1, padding=0, dilation=1) -> np.ndarray:
    """Depthwise 1-D conv in fp64.  x [B,T,C], w [C,1,K], bias [C] or None."""
    lib = _load()
    x, xp = _f64(x)
    w, wp = _f64(w)
    B, T, C = x.shape
    assert w.shape[0] == C and w.shape[1] == 1
    K = w.shape[2]
    bp = None
    if bias is not None:
        bias, bp = _f64(bias)
    To = out_len(T, K, stride, padding, dilation)
    y = np.zeros((B, max(To, 0), C), dtype=np.float64)
    _rc(lib.gconv_oracle_dwconv1d_btc(xp, B, T, C, wp, K, bp, int(stride), int(padding),
                                      int(dilation), y.ctypes.data_as(_dp)))
    return y


def dwconv1d_btc_at(x, w, flat_idx, bias=None, stride=1, padding=0, dilation=1) -> np.ndarray:
    """The elements y.flat[flat_idx] of dwconv1d_btc(...), evaluated one by one."""
    lib = _load()
    x, xp = _f64(x)
    w, wp = _f64(w)
    B, T, C = x.shape
    K = w.shape[2]
    bp = None
    if bias is not None:
        bias, bp = _f64(bias)
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    out = np.zeros(idx.shape, dtype=np.float64)
    _rc(lib.gconv_oracle_dwconv1d_btc_at(xp, B, T, C, wp, K, bp, int(stride), int(padding),
                                         int(dilation), idx.ctypes.data_as(_ip), idx.size,
                                         out.ctypes.data_as(_dp)))
    return out


def dwconv1d_btc_bwd_data(dy, w, T: int, stride=1, padding=0, dilation=1) -> np.ndarray:
    """Gradient of dwconv1d_btc with respect to x [B,T,C], given dy [B,To,C] and w [C,1,K]."""
    lib = _load()
    dy, dyp = _f64(dy)
    w, wp = _f64(w)
    B, To, C = dy.shape
    K = w.shape[2]
    if out_len(T, K, stride, padding, dilation) != To:
        raise ValueError("oracle: dy length does not match T")
    dx = np.zeros((B, T, C), dtype=np.float64)
    _rc(lib.gconv_oracle_dwconv1d_btc_bwd_data(dyp, B, int(T), C, wp, K, int(stride), int(padding),
                                               int(dilation), dx.ctypes.data_as(_dp)))
    return dx


def dwconv1d_btc_bwd_data_at(dy, w, T: int, flat_idx, stride=1, padding=0, dilation=1) -> np.ndarray:
    """The elements dx.flat[flat_idx] of dwconv1d_btc_bwd_data(...), evaluated one by one."""
    lib = _load()
    dy, dyp = _f64(dy)
    w, wp = _f64(w)
    B, To, C = dy.shape
    K = w.shape[2]
    if out_len(T, K, stride, padding, dilation) != To:
        raise ValueError("oracle: dy length does not match T")
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    out = np.zeros(idx.shape, dtype=np.float64)
    _rc(lib.gconv_oracle_dwconv1d_btc_bwd_data_at(dyp, B, int(T), C, wp, K, int(stride), int(padding),
                                                  int(dilation), idx.ctypes.data_as(_ip), idx.size,
                                                  out.ctypes.data_as(_dp)))
    return out


def dwconv1d_btc_bwd_filter(x, dy, K: int, stride=1, padding=0, dilation=1):
    """Gradients of dwconv1d_btc with respect to w [C,1,K] and bias [C], given x [B,T,C]
    and dy [B,To,C].  Returns (dw, db)."""
    lib = _load()
    x, xp = _f64(x)
    dy, dyp = _f64(dy)
    B, T, C = x.shape
    if dy.shape != (B, out_len(T, K, stride, padding, dilation), C):
        raise ValueError("oracle: dy shape does not match x and K")
    dw = np.zeros((C, 1, K), dtype=np.float64)
    db = np.zeros((C,), dtype=np.float64)
    _rc(lib.gconv_oracle_dwconv1d_btc_bwd_filter(xp, dyp, B, T, C, int(K), int(stride), int(padding),
                                                 int(dilation), dw.ctypes.data_as(_dp), db.ctypes.data_as(_dp)))
    return dw, db


def conv2d_nhwc(x, w, bias=None, stride=1, padding=0, dilation=1, groups=1) -> np.ndarray:
    """Grouped conv2d forward in fp64 over channels-last tensors: x [N,H,W,C],
    w [Cout,KH,KW,C/groups], bias [Cout] or None; returns y [N,OH,OW,Cout]."""
    lib = _load()
    x, xp = _f64(x)
    w, wp = _f64(w)
    N, H, W, C = x.shape
    Cout, KH, KW, Cg_w = w.shape
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    bp = None
    if bias is not None:
        bias, bp = _f64(bias)
    OH = out_len(H, KH, sh, ph, dh)
    OW = out_len(W, KW, sw, pw, dw)
    y = np.zeros((N, max(OH, 0), max(OW, 0), Cout), dtype=np.float64)
    _rc(lib.gconv_oracle_conv2d_nhwc(xp, N, C, H, W, wp, Cout, Cg_w, KH, KW, bp, groups,
                                     sh, sw, ph, pw, dh, dw, y.ctypes.data_as(_dp)))
    return y


def conv2d_nhwc_at(x, w, flat_idx, bias=None, stride=1, padding=0, dilation=1, groups=1) -> np.ndarray:
    """The elements y.flat[flat_idx] of conv2d_nhwc(...), evaluated one by one."""
    lib = _load()
    x, xp = _f64(x)
    w, wp = _f64(w)
    N, H, W, C = x.shape
    Cout, KH, KW, Cg_w = w.shape
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    bp = None
    if bias is not None:
        bias, bp = _f64(bias)
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    out = np.zeros(idx.shape, dtype=np.float64)
    _rc(lib.gconv_oracle_conv2d_nhwc_at(xp, N, C, H, W, wp, Cout, Cg_w, KH, KW, bp, groups,
                                        sh, sw, ph, pw, dh, dw, idx.ctypes.data_as(_ip), idx.size,
                                        out.ctypes.data_as(_dp)))
    return out
