// api.cpp -- the C ABI of libgconv: validation, output shape, route selection
// and launch.  Everything here runs on the host; the arithmetic is in the HIP
// kernels (direct2d.hip, dw2d.hip, dw1d_ntc.hip, dw1d_wgrad.hip, nhwc.hip,
// igemm.hip, igemm_rows.hip, igemm_nhwc.hip, igemm_f32.hip).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <limits>
#include <map>
#include <mutex>
#include <vector>

#include "common.hpp"
#include "gconv.h"

namespace {

thread_local char g_last_error[512] = "";
thread_local const char *g_last_kernel = "";

gconv_status_t fail(gconv_status_t s, const char *fmt, long long a = 0, long long b = 0, long long c = 0)
{
    std::snprintf(g_last_error, sizeof(g_last_error), fmt, a, b, c);
    return s;
}

constexpr int64_t kDimMax = std::numeric_limits<int32_t>::max();
static_assert(GCONV_DW1D_BWD_FILTER_SCRATCH_BYTES == gconv::kWgradScratchBytes,
              "the header states the scratch size the library holds");

// Length of one output axis; < 1 means the window never fits.
int64_t out_len(int64_t L, int64_t K, int64_t s, int64_t p, int64_t d)
{
    const int64_t last = L + 2 * p - d * (K - 1) - 1;
    if (last < 0) return 0;
    return last / s + 1;
}

struct Geometry {
    gconv_layout_t layout;
    // NCHW
    int64_t N, C, H, W, Cout, Cg_w, KH, KW, OH, OW;
    int32_t sh, sw, ph, pw, dh, dw;
    // NTC
    int64_t B, T, K, To;
    int32_t s, p, d;
    int32_t groups;
};

bool too_big(int64_t a, int64_t b, int64_t c = 1, int64_t d = 1)
{
    // a*b*c*d must stay below 2^62 (element counts and offsets are int64).
    const double v = (double)a * (double)b * (double)c * (double)d;
    return v >= 4.0e18;
}

gconv_status_t validate(const int64_t *x_shape, const int64_t *w_shape, const int32_t *stride,
                        const int32_t *pad, const int32_t *dilation, int32_t groups,
                        gconv_layout_t layout, Geometry *g)
{
    if (!x_shape || !w_shape || !stride || !pad || !dilation)
        return fail(GCONV_ERR_INVALID_ARG, "NULL shape, stride, pad or dilation array");
    if (layout != GCONV_LAYOUT_NCHW && layout != GCONV_LAYOUT_NTC && layout != GCONV_LAYOUT_NHWC)
        return fail(GCONV_ERR_INVALID_ARG, "unknown layout %lld", (long long)layout);
    if (groups < 1) return fail(GCONV_ERR_INVALID_ARG, "groups must be >= 1 (got %lld)", groups);
    g->layout = layout;
    g->groups = groups;
    if (layout == GCONV_LAYOUT_NCHW || layout == GCONV_LAYOUT_NHWC) {
        if (layout == GCONV_LAYOUT_NCHW) {
            g->N = x_shape[0]; g->C = x_shape[1]; g->H = x_shape[2]; g->W = x_shape[3];
            g->Cout = w_shape[0]; g->Cg_w = w_shape[1]; g->KH = w_shape[2]; g->KW = w_shape[3];
        } else {   // x {N,H,W,C}, w {Cout,KH,KW,C/g}
            g->N = x_shape[0]; g->H = x_shape[1]; g->W = x_shape[2]; g->C = x_shape[3];
            g->Cout = w_shape[0]; g->KH = w_shape[1]; g->KW = w_shape[2]; g->Cg_w = w_shape[3];
        }
        g->sh = stride[0]; g->sw = stride[1]; g->ph = pad[0]; g->pw = pad[1];
        g->dh = dilation[0]; g->dw = dilation[1];
        if (g->N < 0 || g->C < 1 || g->H < 1 || g->W < 1)
            return fail(GCONV_ERR_INVALID_ARG, "x shape must have N >= 0 and C, H, W >= 1");
        if (g->Cout < 1 || g->Cg_w < 1 || g->KH < 1 || g->KW < 1)
            return fail(GCONV_ERR_INVALID_ARG, "w shape entries must be >= 1");
        if (g->sh < 1 || g->sw < 1 || g->dh < 1 || g->dw < 1 || g->ph < 0 || g->pw < 0)
            return fail(GCONV_ERR_INVALID_ARG, "stride and dilation must be >= 1, pad >= 0");
        if (g->C % groups != 0)
            return fail(GCONV_ERR_SHAPE, "C=%lld is not divisible by groups=%lld", g->C, groups);
        if (g->Cout % groups != 0)
            return fail(GCONV_ERR_SHAPE, "Cout=%lld is not divisible by groups=%lld", g->Cout, groups);
        if (g->Cg_w != g->C / groups)
            return fail(GCONV_ERR_SHAPE, "w.shape[1]=%lld must equal C/groups=%lld", g->Cg_w, g->C / groups);
        g->OH = out_len(g->H, g->KH, g->sh, g->ph, g->dh);
        g->OW = out_len(g->W, g->KW, g->sw, g->pw, g->dw);
        if (g->OH < 1 || g->OW < 1)
            return fail(GCONV_ERR_SHAPE, "output would be empty (OH=%lld, OW=%lld)", g->OH, g->OW);
        if (g->N > kDimMax || g->C > kDimMax || g->H > kDimMax || g->W > kDimMax || g->Cout > kDimMax ||
            g->KH > kDimMax || g->KW > kDimMax || too_big(g->N, g->C, g->H, g->W) ||
            too_big(g->N, g->Cout, g->OH, g->OW) || too_big(g->Cout, g->Cg_w, g->KH, g->KW) ||
            too_big(g->H + 2 * (int64_t)g->ph, g->W + 2 * (int64_t)g->pw, g->OH, g->OW) ||
            (int64_t)g->dh * (g->KH - 1) > kDimMax || (int64_t)g->dw * (g->KW - 1) > kDimMax ||
            g->H + 2 * (int64_t)g->ph > kDimMax || g->W + 2 * (int64_t)g->pw > kDimMax)
            return fail(GCONV_ERR_UNSUPPORTED, "tensor dimensions exceed the library's index range");
    } else {
        g->B = x_shape[0]; g->T = x_shape[1]; g->C = x_shape[2];
        g->Cout = w_shape[0]; g->Cg_w = w_shape[1]; g->K = w_shape[2];
        g->s = stride[0]; g->p = pad[0]; g->d = dilation[0];
        if (g->B < 0 || g->T < 1 || g->C < 1)
            return fail(GCONV_ERR_INVALID_ARG, "x shape must have B >= 0 and T, C >= 1");
        if (g->Cout < 1 || g->Cg_w < 1 || g->K < 1)
            return fail(GCONV_ERR_INVALID_ARG, "w shape entries must be >= 1");
        if (g->s < 1 || g->d < 1 || g->p < 0)
            return fail(GCONV_ERR_INVALID_ARG, "stride and dilation must be >= 1, pad >= 0");
        if (g->C % groups != 0)
            return fail(GCONV_ERR_SHAPE, "C=%lld is not divisible by groups=%lld", g->C, groups);
        if (g->Cout % groups != 0)
            return fail(GCONV_ERR_SHAPE, "Cout=%lld is not divisible by groups=%lld", g->Cout, groups);
        if (g->Cg_w != g->C / groups)
            return fail(GCONV_ERR_SHAPE, "w.shape[1]=%lld must equal C/groups=%lld", g->Cg_w, g->C / groups);
        if (groups != g->C)
            return fail(GCONV_ERR_UNSUPPORTED, "the (batch, steps, channels) layout is depthwise only: "
                        "groups=%lld must equal C=%lld", groups, g->C);
        if (g->Cout != g->C)
            return fail(GCONV_ERR_UNSUPPORTED, "depthwise channel multiplier (w.shape[0]=%lld != C=%lld) "
                        "is not supported", g->Cout, g->C);
        g->To = out_len(g->T, g->K, g->s, g->p, g->d);
        if (g->To < 1) return fail(GCONV_ERR_SHAPE, "output would be empty (To=%lld)", g->To);
        if (g->B > kDimMax || g->T > kDimMax || g->C > kDimMax || g->K > kDimMax ||
            too_big(g->B, g->T, g->C) || too_big(g->B, g->To, g->C) ||
            (int64_t)g->d * (g->K - 1) > kDimMax || g->T + 2 * (int64_t)g->p > kDimMax)
            return fail(GCONV_ERR_UNSUPPORTED, "tensor dimensions exceed the library's index range");
    }
    return GCONV_OK;
}

size_t elem_size(gconv_dtype_t dt) { return dt == GCONV_F32 ? 4 : 2; }

gconv::Conv2dArgs conv2d_args(const Geometry &g, const void *x, const void *w, const void *bias, void *y,
                              gconv_dtype_t dtype, void *stream)
{
    gconv::Conv2dArgs a;
    a.x = x; a.w = w; a.bias = bias; a.y = y;
    a.N = g.N; a.C = g.C; a.H = g.H; a.W = g.W; a.Cout = g.Cout; a.KH = g.KH; a.KW = g.KW;
    a.groups = g.groups; a.OH = g.OH; a.OW = g.OW;
    a.sh = g.sh; a.sw = g.sw; a.ph = g.ph; a.pw = g.pw; a.dh = g.dh; a.dw = g.dw;
    a.dtype = (int)dtype;
    a.interleaved = 0;
    a.stream = (hipStream_t)stream;
    return a;
}

// Per-shape route cache filled by gconv_autotune (the "time the candidates once,
// keep the fastest" idea: cudnn.benchmark in the discuss.pytorch.org thread, and
// neon compiling kernel variants and keeping the fastest in the grouped-conv
// issue).  Keyed by everything that decides which routes can run a call and how
// fast: layout, dtype, shapes, stride, padding, dilation and groups.
using TuneKey = std::vector<int64_t>;
std::mutex g_tune_mu;
std::map<TuneKey, gconv_route_t> g_tune;

TuneKey tune_key(const Geometry &g, gconv_dtype_t dtype)
{
    if (g.layout == GCONV_LAYOUT_NTC)
        return {g.layout, dtype, g.B, g.T, g.C, g.Cout, g.K, g.s, g.p, g.d, g.groups};
    return {g.layout, dtype, g.N, g.C, g.H, g.W, g.Cout, g.KH, g.KW, g.sh, g.sw, g.ph, g.pw, g.dh, g.dw, g.groups};
}

bool tuned_route(const Geometry &g, gconv_dtype_t dtype, gconv_route_t *r)
{
    std::lock_guard<std::mutex> lk(g_tune_mu);
    if (g_tune.empty()) return false;
    const auto it = g_tune.find(tune_key(g, dtype));
    if (it == g_tune.end()) return false;
    *r = it->second;
    return true;
}

// Route heuristic: the implicit GEMM pays off once the per-group contraction
// (C/g * KH * KW) and the per-group output width (Cout/g) are wide enough to
// fill matrix-core tiles; narrow groups (depthwise, 4-channel groups) stay on
// the direct route, which is bound by memory traffic rather than arithmetic.
gconv_route_t auto_route(const Geometry &g, gconv_dtype_t dtype, bool igemm_ok)
{
    if (g.layout == GCONV_LAYOUT_NTC) return GCONV_ROUTE_DIRECT;
    const int64_t Kg = g.Cg_w * g.KH * g.KW;
    const int64_t Ng = g.Cout / g.groups;
    if (igemm_ok && Kg >= 64 && Ng >= 16) return GCONV_ROUTE_IGEMM;
    return GCONV_ROUTE_DIRECT;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

gconv_status_t run(const void *x, const int64_t *x_shape, const void *w, const int64_t *w_shape,
                   const void *bias, void *y, const int32_t *stride, const int32_t *pad,
                   const int32_t *dilation, int32_t groups, gconv_layout_t layout, gconv_dtype_t dtype,
                   gconv_route_t route, gconv_out_order_t order, void *stream)
{
    g_last_error[0] = '\0';
    if (order != GCONV_ORDER_GROUPED && order != GCONV_ORDER_INTERLEAVED)
        return fail(GCONV_ERR_INVALID_ARG, "unknown output order %lld", (long long)order);
    if (dtype != GCONV_F32 && dtype != GCONV_F16 && dtype != GCONV_BF16)
        return fail(GCONV_ERR_INVALID_ARG, "unknown dtype %lld", (long long)dtype);
    if (route != GCONV_ROUTE_AUTO && route != GCONV_ROUTE_DIRECT && route != GCONV_ROUTE_IGEMM)
        return fail(GCONV_ERR_INVALID_ARG, "unknown route %lld", (long long)route);
    Geometry g;
    gconv_status_t st = validate(x_shape, w_shape, stride, pad, dilation, groups, layout, &g);
    if (st != GCONV_OK) return st;
    const bool nchw = layout != GCONV_LAYOUT_NTC;   // NCHW or NHWC: the 2-D geometry
    if ((nchw && g.N == 0) || (!nchw && g.B == 0)) {
        // An empty batch has no elements: x and y may be NULL and nothing is enqueued.
        if (!w) return fail(GCONV_ERR_INVALID_ARG, "NULL w pointer");
        g_last_kernel = "";
        return GCONV_OK;
    }
    if (!x || !w || !y) return fail(GCONV_ERR_INVALID_ARG, "NULL x, w or y pointer");
    const size_t es = elem_size(dtype);
    const size_t nx = es * (size_t)(nchw ? g.N * g.C * g.H * g.W : g.B * g.T * g.C);
    const size_t nw = es * (size_t)(nchw ? g.Cout * g.Cg_w * g.KH * g.KW : g.C * g.K);
    const size_t nb = bias ? es * (size_t)g.Cout : 0;
    const size_t ny = es * (size_t)(nchw ? g.N * g.Cout * g.OH * g.OW : g.B * g.To * g.C);
    if (overlaps(y, ny, x, nx) || overlaps(y, ny, w, nw) || overlaps(y, ny, bias, nb))
        return fail(GCONV_ERR_INVALID_ARG, "y overlaps x, w or bias");
    hipError_t err;
    const char *kname = "";
    if (layout == GCONV_LAYOUT_NHWC) {
        gconv::Conv2dArgs a = conv2d_args(g, x, w, bias, y, dtype, stream);
        a.interleaved = order == GCONV_ORDER_INTERLEAVED;
        const bool igemm_ok = gconv::igemm_nhwc_supported(a);
        if (route == GCONV_ROUTE_AUTO) {
            gconv_route_t t;
            route = (tuned_route(g, dtype, &t) && (t != GCONV_ROUTE_IGEMM || igemm_ok)) ? t
                                                                                        : auto_route(g, dtype, igemm_ok);
        }
        if (route == GCONV_ROUTE_IGEMM) {
            if (!igemm_ok)
                return fail(GCONV_ERR_UNSUPPORTED, "the NHWC implicit-GEMM route needs fp16/bf16, C/g a multiple "
                            "of 16, Cout/g a multiple of 4, the grouped output order, 16-byte aligned x and w");
            err = gconv::launch_igemm_nhwc(a, &kname);
        } else {
            err = gconv::launch_conv2d_nhwc(a, &kname);
        }
    } else if (nchw) {
        gconv::Conv2dArgs a = conv2d_args(g, x, w, bias, y, dtype, stream);
        a.interleaved = order == GCONV_ORDER_INTERLEAVED;
        const bool rows_ok = dtype != GCONV_F32 && gconv::igemm_rows_supported(a);
        const bool igemm_ok = dtype == GCONV_F32 ? gconv::igemm_f32_supported(a)
                                                 : rows_ok || gconv::igemm_supported(a);
        if (route == GCONV_ROUTE_AUTO) {
            gconv_route_t t;
            route = (tuned_route(g, dtype, &t) && (t != GCONV_ROUTE_IGEMM || igemm_ok)) ? t
                                                                                        : auto_route(g, dtype, igemm_ok);
        }
        if (route == GCONV_ROUTE_IGEMM) {
            if (!igemm_ok)
                return fail(GCONV_ERR_UNSUPPORTED, "the implicit-GEMM route does not cover this geometry "
                            "(3x3 or 1x1 kernels, C/g a multiple of 8 (fp16/bf16) or 4 (fp32), halo tile "
                            "within LDS)");
            err = dtype == GCONV_F32 ? gconv::launch_igemm_f32(a, &kname)
                  : rows_ok          ? gconv::launch_igemm_rows(a, &kname)
                                     : gconv::launch_igemm(a, &kname);
        } else if (gconv::dw2d_supported(a)) {
            err = gconv::launch_dw2d(a, &kname);   // depthwise (C/g = 1), stride 1 or 2
        } else {
            err = gconv::launch_direct2d(a, &kname);
        }
    } else {
        if (route == GCONV_ROUTE_IGEMM)
            return fail(GCONV_ERR_UNSUPPORTED, "the implicit-GEMM route does not run the "
                        "(batch, steps, channels) depthwise layout");
        gconv::Dw1dArgs a;
        a.x = x; a.w = w; a.bias = bias; a.y = y;
        a.B = g.B; a.T = g.T; a.C = g.C; a.K = g.K; a.To = g.To;
        a.s = g.s; a.p = g.p; a.d = g.d;
        a.dtype = (int)dtype;
        a.stream = (hipStream_t)stream;
        err = gconv::launch_dw1d(a, &kname);
    }
    if (err != hipSuccess)
        return fail(GCONV_ERR_LAUNCH, "kernel launch failed: HIP error %lld", (long long)err);
    g_last_kernel = kname;
    return GCONV_OK;
}

// Geometry of a depthwise conv1d over (batch, steps, channels) from the forward
// call's shapes (groups = C).
gconv_status_t dw1d_geometry(const int64_t *x_shape, const int64_t *w_shape, const int32_t *stride,
                             const int32_t *pad, const int32_t *dilation, gconv_dtype_t dtype, Geometry *g)
{
    if (dtype != GCONV_F32 && dtype != GCONV_F16 && dtype != GCONV_BF16)
        return fail(GCONV_ERR_INVALID_ARG, "unknown dtype %lld", (long long)dtype);
    if (!x_shape) return fail(GCONV_ERR_INVALID_ARG, "NULL x_shape");
    if (x_shape[2] < 1 || x_shape[2] > kDimMax)
        return fail(GCONV_ERR_INVALID_ARG, "x_shape[2] (channels) must be in [1, 2^31)");
    return validate(x_shape, w_shape, stride, pad, dilation, (int32_t)x_shape[2], GCONV_LAYOUT_NTC, g);
}

gconv::Dw1dArgs dw1d_args(const Geometry &g, const void *w, gconv_dtype_t dtype, void *stream)
{
    gconv::Dw1dArgs a;
    a.x = nullptr; a.w = w; a.bias = nullptr; a.y = nullptr;
    a.B = g.B; a.T = g.T; a.C = g.C; a.K = g.K; a.To = g.To;
    a.s = g.s; a.p = g.p; a.d = g.d;
    a.dtype = (int)dtype;
    a.stream = (hipStream_t)stream;
    return a;
}

}  // namespace

extern "C" {

gconv_status_t gconv_out_shape(const int64_t *x_shape, const int64_t *w_shape, const int32_t *stride,
                               const int32_t *pad, const int32_t *dilation, int32_t groups,
                               gconv_layout_t layout, int64_t *y_shape)
{
    g_last_error[0] = '\0';
    if (!y_shape) return fail(GCONV_ERR_INVALID_ARG, "NULL y_shape");
    Geometry g;
    const gconv_status_t st = validate(x_shape, w_shape, stride, pad, dilation, groups, layout, &g);
    if (st != GCONV_OK) return st;
    if (layout == GCONV_LAYOUT_NCHW) {
        y_shape[0] = g.N; y_shape[1] = g.Cout; y_shape[2] = g.OH; y_shape[3] = g.OW;
    } else if (layout == GCONV_LAYOUT_NHWC) {
        y_shape[0] = g.N; y_shape[1] = g.OH; y_shape[2] = g.OW; y_shape[3] = g.Cout;
    } else {
        y_shape[0] = g.B; y_shape[1] = g.To; y_shape[2] = g.C;
    }
    return GCONV_OK;
}

gconv_status_t gconv_select_route(const int64_t *x_shape, const int64_t *w_shape, const int32_t *stride,
                                  const int32_t *pad, const int32_t *dilation, int32_t groups,
                                  gconv_layout_t layout, gconv_dtype_t dtype, gconv_route_t *route)
{
    g_last_error[0] = '\0';
    if (!route) return fail(GCONV_ERR_INVALID_ARG, "NULL route");
    if (dtype != GCONV_F32 && dtype != GCONV_F16 && dtype != GCONV_BF16)
        return fail(GCONV_ERR_INVALID_ARG, "unknown dtype %lld", (long long)dtype);
    Geometry g;
    const gconv_status_t st = validate(x_shape, w_shape, stride, pad, dilation, groups, layout, &g);
    if (st != GCONV_OK) return st;
    bool igemm_ok = false;
    // A 16-byte aligned dummy pointer for x and w: the plans only inspect their alignment.
    alignas(16) static const char dummy[16] = {0};
    if (layout == GCONV_LAYOUT_NCHW) {
        const gconv::Conv2dArgs a = conv2d_args(g, dummy, dummy, nullptr, nullptr, dtype, nullptr);
        igemm_ok = dtype == GCONV_F32 ? gconv::igemm_f32_supported(a)
                                      : gconv::igemm_rows_supported(a) || gconv::igemm_supported(a);
    } else if (layout == GCONV_LAYOUT_NHWC) {
        igemm_ok = gconv::igemm_nhwc_supported(conv2d_args(g, dummy, dummy, nullptr, nullptr, dtype, nullptr));
    }
    gconv_route_t t;
    *route = (tuned_route(g, dtype, &t) && (t != GCONV_ROUTE_IGEMM || igemm_ok)) ? t : auto_route(g, dtype, igemm_ok);
    return GCONV_OK;
}

gconv_status_t gconv_autotune(const void *x, const int64_t *x_shape, const void *w, const int64_t *w_shape,
                              const void *bias, void *y, const int32_t *stride, const int32_t *pad,
                              const int32_t *dilation, int32_t groups, gconv_layout_t layout,
                              gconv_dtype_t dtype, int32_t reps, void *hip_stream, gconv_route_t *best)
{
    g_last_error[0] = '\0';
    if (!best) return fail(GCONV_ERR_INVALID_ARG, "NULL best");
    if (reps < 1) return fail(GCONV_ERR_INVALID_ARG, "reps must be >= 1 (got %lld)", reps);
    Geometry g;
    gconv_status_t st = validate(x_shape, w_shape, stride, pad, dilation, groups, layout, &g);
    if (st != GCONV_OK) return st;
    const hipStream_t stream = (hipStream_t)hip_stream;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0) (void)hipEventDestroy(e0);
        return fail(GCONV_ERR_LAUNCH, "hipEventCreate failed");
    }
    gconv_route_t win = GCONV_ROUTE_AUTO;
    float win_ms = 0.0f;
    gconv_status_t first_err = GCONV_OK;
    for (gconv_route_t r : {GCONV_ROUTE_DIRECT, GCONV_ROUTE_IGEMM}) {
        // One untimed call (which also tells whether the route runs this call),
        // then `reps` calls between two events on the caller's stream.
        st = run(x, x_shape, w, w_shape, bias, y, stride, pad, dilation, groups, layout, dtype, r,
                 GCONV_ORDER_GROUPED, hip_stream);
        if (st == GCONV_ERR_UNSUPPORTED) continue;
        if (st != GCONV_OK) { first_err = st; break; }
        float ms = 0.0f;
        bool ok = hipEventRecord(e0, stream) == hipSuccess;
        for (int i = 0; ok && i < reps; ++i)
            ok = run(x, x_shape, w, w_shape, bias, y, stride, pad, dilation, groups, layout, dtype, r,
                     GCONV_ORDER_GROUPED, hip_stream) == GCONV_OK;
        ok = ok && hipEventRecord(e1, stream) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
             hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
        if (!ok) { first_err = GCONV_ERR_LAUNCH; break; }
        if (win == GCONV_ROUTE_AUTO || ms < win_ms) { win = r; win_ms = ms; }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (first_err != GCONV_OK) return first_err == GCONV_ERR_LAUNCH && !g_last_error[0]
                                          ? fail(GCONV_ERR_LAUNCH, "timing a route failed") : first_err;
    if (win == GCONV_ROUTE_AUTO) return fail(GCONV_ERR_UNSUPPORTED, "no route runs this convolution");
    // y ends up holding the chosen route's result.
    st = run(x, x_shape, w, w_shape, bias, y, stride, pad, dilation, groups, layout, dtype, win,
             GCONV_ORDER_GROUPED, hip_stream);
    if (st != GCONV_OK) return st;
    {
        std::lock_guard<std::mutex> lk(g_tune_mu);
        g_tune[tune_key(g, dtype)] = win;
    }
    *best = win;
    return GCONV_OK;
}

void gconv_autotune_clear(void)
{
    std::lock_guard<std::mutex> lk(g_tune_mu);
    g_tune.clear();
}

gconv_status_t gconv_fwd(const void *x, const int64_t *x_shape, const void *w, const int64_t *w_shape,
                         const void *bias, void *y, const int32_t *stride, const int32_t *pad,
                         const int32_t *dilation, int32_t groups, gconv_layout_t layout, gconv_dtype_t dtype,
                         void *hip_stream)
{
    return run(x, x_shape, w, w_shape, bias, y, stride, pad, dilation, groups, layout, dtype,
               GCONV_ROUTE_AUTO, GCONV_ORDER_GROUPED, hip_stream);
}

gconv_status_t gconv_fwd_route(const void *x, const int64_t *x_shape, const void *w, const int64_t *w_shape,
                               const void *bias, void *y, const int32_t *stride, const int32_t *pad,
                               const int32_t *dilation, int32_t groups, gconv_layout_t layout,
                               gconv_dtype_t dtype, gconv_route_t route, void *hip_stream)
{
    return run(x, x_shape, w, w_shape, bias, y, stride, pad, dilation, groups, layout, dtype, route,
               GCONV_ORDER_GROUPED, hip_stream);
}

gconv_status_t gconv_fwd_ex(const void *x, const int64_t *x_shape, const void *w, const int64_t *w_shape,
                            const void *bias, void *y, const int32_t *stride, const int32_t *pad,
                            const int32_t *dilation, int32_t groups, gconv_layout_t layout,
                            gconv_dtype_t dtype, gconv_route_t route, gconv_out_order_t order,
                            void *hip_stream)
{
    return run(x, x_shape, w, w_shape, bias, y, stride, pad, dilation, groups, layout, dtype, route, order,
               hip_stream);
}

gconv_status_t gconv_dw1d_bwd_data(const void *dy, const int64_t *x_shape, const void *w,
                                   const int64_t *w_shape, void *dx, const int32_t *stride,
                                   const int32_t *pad, const int32_t *dilation, gconv_dtype_t dtype,
                                   void *hip_stream)
{
    g_last_error[0] = '\0';
    Geometry g;
    const gconv_status_t st = dw1d_geometry(x_shape, w_shape, stride, pad, dilation, dtype, &g);
    if (st != GCONV_OK) return st;
    if (!w) return fail(GCONV_ERR_INVALID_ARG, "NULL w pointer");
    if (g.B == 0) {
        g_last_kernel = "";
        return GCONV_OK;
    }
    if (!dy || !dx) return fail(GCONV_ERR_INVALID_ARG, "NULL dy or dx pointer");
    const size_t es = elem_size(dtype);
    const size_t ndy = es * (size_t)(g.B * g.To * g.C), ndx = es * (size_t)(g.B * g.T * g.C);
    if (overlaps(dx, ndx, dy, ndy) || overlaps(dx, ndx, w, es * (size_t)(g.C * g.K)))
        return fail(GCONV_ERR_INVALID_ARG, "dx overlaps dy or w");
    const char *kname = "";
    const hipError_t err = gconv::launch_dw1d_bwd_data(dw1d_args(g, w, dtype, hip_stream), dy, dx, &kname);
    if (err != hipSuccess)
        return fail(GCONV_ERR_LAUNCH, "kernel launch failed: HIP error %lld", (long long)err);
    g_last_kernel = kname;
    return GCONV_OK;
}

gconv_status_t gconv_dw1d_bwd_filter_workspace(const int64_t *x_shape, const int64_t *w_shape,
                                               const int32_t *stride, const int32_t *pad,
                                               const int32_t *dilation, gconv_dtype_t dtype, size_t *bytes)
{
    g_last_error[0] = '\0';
    if (!bytes) return fail(GCONV_ERR_INVALID_ARG, "NULL bytes");
    Geometry g;
    const gconv_status_t st = dw1d_geometry(x_shape, w_shape, stride, pad, dilation, dtype, &g);
    if (st != GCONV_OK) return st;
    size_t ws = 0;
    if (!gconv::dw1d_wgrad_plan(dw1d_args(g, nullptr, dtype, nullptr), &ws))
        return fail(GCONV_ERR_UNSUPPORTED, "filter gradient: filter length above 64 or sizes beyond the "
                    "library's index range");
    *bytes = ws;
    return GCONV_OK;
}

gconv_status_t gconv_dw1d_bwd_filter(const void *x, const int64_t *x_shape, const void *dy,
                                     const int64_t *w_shape, void *dw, void *db, const int32_t *stride,
                                     const int32_t *pad, const int32_t *dilation, gconv_dtype_t dtype,
                                     void *workspace, size_t workspace_bytes, void *hip_stream)
{
    g_last_error[0] = '\0';
    Geometry g;
    const gconv_status_t st = dw1d_geometry(x_shape, w_shape, stride, pad, dilation, dtype, &g);
    if (st != GCONV_OK) return st;
    const gconv::Dw1dArgs a = dw1d_args(g, nullptr, dtype, hip_stream);
    size_t need = 0;
    if (!gconv::dw1d_wgrad_plan(a, &need))
        return fail(GCONV_ERR_UNSUPPORTED, "filter gradient: filter length above 64 or sizes beyond the "
                    "library's index range");
    if (!dw) return fail(GCONV_ERR_INVALID_ARG, "NULL dw pointer");
    if (g.B > 0 && (!x || !dy)) return fail(GCONV_ERR_INVALID_ARG, "NULL x or dy pointer");
    if (need > 0 && !workspace) return fail(GCONV_ERR_INVALID_ARG, "NULL workspace");
    if (((uintptr_t)workspace & 3) != 0) return fail(GCONV_ERR_INVALID_ARG, "workspace must be 4-byte aligned");
    if (workspace_bytes < need)
        return fail(GCONV_ERR_INVALID_ARG, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                    (long long)need);
    const size_t es = elem_size(dtype);
    const size_t nx = es * (size_t)(g.B * g.T * g.C), ndy = es * (size_t)(g.B * g.To * g.C);
    const size_t ndw = es * (size_t)(g.C * g.K), ndb = db ? es * (size_t)g.C : 0;
    if (overlaps(dw, ndw, x, nx) || overlaps(dw, ndw, dy, ndy) || overlaps(dw, ndw, workspace, need) ||
        overlaps(dw, ndw, db, ndb) || overlaps(db, ndb, x, nx) || overlaps(db, ndb, dy, ndy) ||
        overlaps(db, ndb, workspace, need) || overlaps(workspace, need, x, nx) ||
        overlaps(workspace, need, dy, ndy))
        return fail(GCONV_ERR_INVALID_ARG, "dw, db, the workspace, x and dy must not overlap");
    const char *kname = "";
    const hipError_t err = gconv::launch_dw1d_bwd_filter(a, x, dy, dw, db, workspace, &kname);
    if (err != hipSuccess)
        return fail(GCONV_ERR_LAUNCH, "kernel launch failed: HIP error %lld", (long long)err);
    g_last_kernel = kname;
    return GCONV_OK;
}

gconv_status_t gconv_dw1d_bwd_filter_noalloc(const void *x, const int64_t *x_shape, const void *dy,
                                             const int64_t *w_shape, void *dw, void *db, const int32_t *stride,
                                             const int32_t *pad, const int32_t *dilation, gconv_dtype_t dtype,
                                             void *hip_stream)
{
    g_last_error[0] = '\0';
    Geometry g;
    const gconv_status_t st = dw1d_geometry(x_shape, w_shape, stride, pad, dilation, dtype, &g);
    if (st != GCONV_OK) return st;
    const gconv::Dw1dArgs a = dw1d_args(g, nullptr, dtype, hip_stream);
    size_t need = 0;
    if (!gconv::dw1d_wgrad_plan(a, &need))
        return fail(GCONV_ERR_UNSUPPORTED, "filter gradient: filter length above 64 or sizes beyond the "
                    "library's index range");
    if (need > gconv::kWgradScratchBytes)
        return fail(GCONV_ERR_UNSUPPORTED, "filter gradient without allocation: this geometry needs %lld bytes "
                    "of scratch, the library holds %lld (use gconv_dw1d_bwd_filter with a workspace)",
                    (long long)need, (long long)gconv::kWgradScratchBytes);
    if (!dw) return fail(GCONV_ERR_INVALID_ARG, "NULL dw pointer");
    if (g.B > 0 && (!x || !dy)) return fail(GCONV_ERR_INVALID_ARG, "NULL x or dy pointer");
    const size_t es = elem_size(dtype);
    const size_t nx = es * (size_t)(g.B * g.T * g.C), ndy = es * (size_t)(g.B * g.To * g.C);
    const size_t ndw = es * (size_t)(g.C * g.K), ndb = db ? es * (size_t)g.C : 0;
    if (overlaps(dw, ndw, x, nx) || overlaps(dw, ndw, dy, ndy) || overlaps(dw, ndw, db, ndb) ||
        overlaps(db, ndb, x, nx) || overlaps(db, ndb, dy, ndy))
        return fail(GCONV_ERR_INVALID_ARG, "dw, db, x and dy must not overlap");
    void *ws = nullptr;
    hipError_t err = gconv::wgrad_scratch(&ws);
    if (err != hipSuccess)
        return fail(GCONV_ERR_LAUNCH, "device address of the scratch array: HIP error %lld", (long long)err);
    const char *kname = "";
    err = gconv::launch_dw1d_bwd_filter(a, x, dy, dw, db, ws, &kname);
    if (err != hipSuccess)
        return fail(GCONV_ERR_LAUNCH, "kernel launch failed: HIP error %lld", (long long)err);
    g_last_kernel = kname;
    return GCONV_OK;
}

const char *gconv_last_kernel(void) { return g_last_kernel; }

const char *gconv_status_string(gconv_status_t status)
{
    switch (status) {
    case GCONV_OK: return "ok";
    case GCONV_ERR_INVALID_ARG: return "invalid argument";
    case GCONV_ERR_SHAPE: return "shape mismatch";
    case GCONV_ERR_UNSUPPORTED: return "unsupported convolution";
    case GCONV_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

const char *gconv_last_error(void) { return g_last_error; }

}  // extern "C"
