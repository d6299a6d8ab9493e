// dw1d_ntc.hip -- depthwise 1-D convolution over a (batch, steps, channels) tensor.
//
// The Conformer convolution module's depthwise conv (speechbrain issue #2733:
// groups set to the channel count, tensor kept in (batch, steps, channels) order
// rather than PyTorch's (batch, channels, steps)).  Channels are the contiguous
// axis, so lanes map to channels and every load and store is coalesced along C.
// Each thread keeps the K filter taps of its channel and a run of R outputs in
// registers and streams the R + K - 1 input steps of that run through them once:
// one load per input step instead of one per tap, the "single load" the issue's
// author wanted in place of a loop over the kernel taps.
//
// dw1d_btc_window<T, K, R>: stride 1, dilation 1, compile-time K.
// dw1d_btc_generic<T>: any K, stride, dilation; one thread per output.
#include <algorithm>

#include "common.hpp"

namespace gconv {
namespace {

constexpr int kThreads = 256;

template <typename T, int K, int R>
__global__ void __launch_bounds__(kThreads)
dw1d_btc_window(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
                T *__restrict__ y, int T_in, int C, int To, int pad, int cblocks, int tblocks)
{
    int64_t b = blockIdx.x;
    const int cb = (int)(b % cblocks); b /= cblocks;
    const int tb = (int)(b % tblocks);
    const int64_t bi = b / tblocks;
    const int c = cb * kThreads + threadIdx.x;
    if (c >= C) return;
    const int t0 = tb * R;

    // The R + K - 1 input steps feeding outputs [t0, t0 + R), zero outside [0, T).
    const T *xb = x + bi * (int64_t)T_in * C + c;
    const int base = t0 - pad;
    float xw[R + K - 1];
#pragma clang loop unroll(full)
    for (int i = 0; i < R + K - 1; ++i) {
        const int ti = base + i;
        xw[i] = (ti >= 0 && ti < T_in) ? to_f32(xb[(int64_t)ti * C]) : 0.0f;
    }
    float wr[K];
#pragma clang loop unroll(full)
    for (int k = 0; k < K; ++k) wr[k] = to_f32(w[(int64_t)c * K + k]);
    const float b0 = bias ? to_f32(bias[c]) : 0.0f;

    T *yb = y + bi * (int64_t)To * C + c;
#pragma clang loop unroll(full)
    for (int r = 0; r < R; ++r) {
        float acc = b0;
#pragma clang loop unroll(full)
        for (int k = 0; k < K; ++k) acc = fmaf(xw[r + k], wr[k], acc);
        if (t0 + r < To) yb[(int64_t)(t0 + r) * C] = from_f32<T>(acc);
    }
}

template <typename T>
__global__ void __launch_bounds__(kThreads)
dw1d_btc_generic(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
                 T *__restrict__ y, int64_t total, int T_in, int C, int To, int K, int s, int p, int d)
{
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
        const int c = (int)(i % C);
        const int t = (int)((i / C) % To);
        const int64_t bi = i / ((int64_t)C * To);
        float acc = bias ? to_f32(bias[c]) : 0.0f;
        for (int k = 0; k < K; ++k) {
            const int ti = t * s - p + k * d;
            if (ti < 0 || ti >= T_in) continue;
            acc = fmaf(to_f32(x[(bi * T_in + ti) * C + c]), to_f32(w[(int64_t)c * K + k]), acc);
        }
        y[i] = from_f32<T>(acc);
    }
}

template <typename T, int K, int R>
hipError_t run_window(const Dw1dArgs &a)
{
    const int cblocks = (int)ceil_div(a.C, kThreads);
    const int tblocks = (int)ceil_div(a.To, R);
    const int64_t blocks = a.B * cblocks * tblocks;
    hipLaunchKernelGGL((dw1d_btc_window<T, K, R>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                       (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, (int)a.T, (int)a.C,
                       (int)a.To, a.p, cblocks, tblocks);
    return hipGetLastError();
}

template <typename T>
hipError_t run_typed(const Dw1dArgs &a, const char **kname)
{
    const int64_t window_blocks = a.B * ceil_div(a.C, kThreads) * ceil_div(a.To, 32);
    if (a.s == 1 && a.d == 1 && window_blocks < (int64_t(1) << 31)) {
        *kname = "dw1d_btc_window";
        switch (a.K) {
        case 3: return run_window<T, 3, 32>(a);
        case 5: return run_window<T, 5, 32>(a);
        case 7: return run_window<T, 7, 32>(a);
        case 9: return run_window<T, 9, 32>(a);
        case 15: return run_window<T, 15, 32>(a);
        case 31: return run_window<T, 31, 32>(a);
        default: break;
        }
    }
    *kname = "dw1d_btc_generic";
    const int64_t total = a.B * a.To * a.C;
    const int64_t blocks = std::min<int64_t>(ceil_div(total, kThreads), 1 << 20);
    hipLaunchKernelGGL((dw1d_btc_generic<T>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                       (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, total, (int)a.T,
                       (int)a.C, (int)a.To, (int)a.K, a.s, a.p, a.d);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dw1d(const Dw1dArgs &a, const char **kname)
{
    switch (a.dtype) {
    case DT_F32: return run_typed<float>(a, kname);
    case DT_F16: return run_typed<_Float16>(a, kname);
    default: return run_typed<__bf16>(a, kname);
    }
}

}  // namespace gconv
