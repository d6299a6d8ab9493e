// dw1d_wgrad.hip -- filter and bias gradients of the depthwise 1-D convolution
// over a (batch, steps, channels) tensor.
//
// The backward pass of the Conformer's depthwise conv is the next step of
// speechbrain issue #2733 (its author's follow-up comments).  For the forward
// y[b,t,c] = bias[c] + sum_k x[b, t*s - p + k*d, c] * w[c,0,k]:
//     dw[c,0,k] = sum over (b, t) of dy[b,t,c] * x[b, t*s - p + k*d, c]   (in range)
//     db[c]     = sum over (b, t) of dy[b,t,c]
// Each gradient is a reduction over B*To terms per (channel, tap), done in two
// deterministic stages (no atomics, so every run gives the same bits):
//  * dw1d_btc_wgrad_partial: one workgroup per tile of TT output steps x 64
//    channels of one batch entry.  The tile's dy rows and the x rows they read
//    ((TT-1)*s + (K-1)*d + 1 of them, zero outside [0, T)) are staged in LDS as
//    fp32 with loads coalesced along C; the 4 waves split the taps (wave g takes
//    taps g, g+4, ...; wave 0 also sums dy for the bias), lane = channel.  The
//    tile's fp32 sums go to part[tile][k][c] (k = K holds the bias sums).
//  * dw1d_btc_wgrad_reduce: one workgroup per (tap, 64 channels); 4 slices of
//    the tiles are summed in order, then combined in a fixed order and rounded
//    once to the tensor dtype.
#include <algorithm>

#include "common.hpp"

namespace gconv {
namespace {

constexpr int kThreads = 256;
constexpr int kCT = 64;                      // channels per tile (lanes)
constexpr int kGroups = kThreads / kCT;      // waves, each taking every 4th tap
constexpr int kMaxTT = 64;                   // output steps per tile
constexpr int kLdsMax = 60 * 1024;

// NT: taps per wave (K <= 4 * NT).
template <typename T, int NT>
__global__ void __launch_bounds__(kThreads)
dw1d_btc_wgrad_partial(const T *__restrict__ x, const T *__restrict__ dy, float *__restrict__ part,
                       int T_in, int C, int To, int K, int s, int p, int d, int TT, int NRW,
                       int tblocks, int cblocks)
{
    extern __shared__ float sm[];
    float *dys = sm;                  // [TT][kCT]
    float *xs = sm + TT * kCT;        // [NRW][kCT]
    const int tid = threadIdx.x, lane = tid % kCT, g = tid / kCT;
    int rest = blockIdx.x;
    const int cb = rest % cblocks;
    rest /= cblocks;
    const int tb = rest % tblocks;
    const int bi = rest / tblocks;
    const int t0 = tb * TT, c0 = cb * kCT, c = c0 + lane;
    const bool cok = c < C;

    // Stage dy[bi, t0 .. t0+TT) and x[bi, t0*s - p .. + NRW), zero outside the
    // tensors (lane = channel: each row is one coalesced read of 64 channels).
    const T *dyb = dy + (int64_t)bi * To * C;
    const T *xb = x + (int64_t)bi * T_in * C;
    for (int r = g; r < TT; r += kGroups) {
        const int t = t0 + r;
        dys[r * kCT + lane] = (cok && t < To) ? to_f32(dyb[(int64_t)t * C + c]) : 0.0f;
    }
    for (int r = g; r < NRW; r += kGroups) {
        const int ti = t0 * s - p + r;
        xs[r * kCT + lane] = (cok && ti >= 0 && ti < T_in) ? to_f32(xb[(int64_t)ti * C + c]) : 0.0f;
    }
    __syncthreads();

    float acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = 0.0f;
    float accb = 0.0f;
    const int tn = min(TT, To - t0);   // output steps of this tile that exist
    for (int t = 0; t < tn; ++t) {
        const float dv = dys[t * kCT + lane];
        accb += dv;
        const float *xr = xs + (t * s) * kCT + lane;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int k = g + kGroups * j;
            if (k < K) acc[j] = fmaf(dv, xr[k * d * kCT], acc[j]);
        }
    }
    if (!cok) return;
    float *pt = part + (int64_t)blockIdx.x / cblocks * (K + 1) * C + c;   // tile (bi, tb)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int k = g + kGroups * j;
        if (k < K) pt[(int64_t)k * C] = acc[j];
    }
    if (g == 0) pt[(int64_t)K * C] = accb;
}

template <typename T>
__global__ void __launch_bounds__(kThreads)
dw1d_btc_wgrad_reduce(const float *__restrict__ part, T *__restrict__ dw, T *__restrict__ db,
                      int C, int K, int ntiles, int cblocks)
{
    __shared__ float red[kGroups][kCT];
    const int tid = threadIdx.x, lane = tid % kCT, q = tid / kCT;
    const int kk = blockIdx.x / cblocks, cb = blockIdx.x % cblocks;   // kk == K: the bias row
    const int c = cb * kCT + lane;
    float acc = 0.0f;
    if (c < C)
        for (int i = q; i < ntiles; i += kGroups) acc += part[((int64_t)i * (K + 1) + kk) * C + c];
    red[q][lane] = acc;
    __syncthreads();
    if (q != 0 || c >= C) return;
    const float v = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
    if (kk < K) dw[(int64_t)c * K + kk] = from_f32<T>(v);
    else if (db) db[c] = from_f32<T>(v);
}

struct Plan {
    int TT, NRW, NT, tblocks, cblocks, ntiles;
    size_t lds, ws_bytes;
    bool ok;
};

Plan make_plan(const Dw1dArgs &a)
{
    Plan pl{};
    pl.ok = false;
    pl.NT = (int)ceil_div(a.K, kGroups);
    if (pl.NT > 16) return pl;                           // K <= 64
    int64_t TT = kMaxTT, NRW = 0;
    for (; TT >= 1; TT /= 2) {
        NRW = (TT - 1) * a.s + (a.K - 1) * a.d + 1;
        if ((TT + NRW) * kCT * (int64_t)sizeof(float) <= kLdsMax) break;
    }
    if (TT < 1) return pl;
    pl.TT = (int)TT;
    pl.NRW = (int)NRW;
    pl.tblocks = (int)ceil_div(a.To, TT);
    pl.cblocks = (int)ceil_div(a.C, kCT);
    const int64_t ntiles = a.B * pl.tblocks;
    if (ntiles * pl.cblocks >= (int64_t(1) << 31) || (a.K + 1) * pl.cblocks >= (int64_t(1) << 31)) return pl;
    pl.ntiles = (int)ntiles;
    pl.lds = (size_t)(TT + NRW) * kCT * sizeof(float);
    pl.ws_bytes = (size_t)ntiles * (size_t)(a.K + 1) * (size_t)a.C * sizeof(float);
    pl.ok = true;
    return pl;
}

template <typename T, int NT>
hipError_t run_partial(const Dw1dArgs &a, const Plan &pl, const void *x, const void *dy, float *part)
{
    hipLaunchKernelGGL((dw1d_btc_wgrad_partial<T, NT>), dim3((unsigned)(pl.ntiles * (int64_t)pl.cblocks)),
                       dim3(kThreads), pl.lds, a.stream, (const T *)x, (const T *)dy, part, (int)a.T,
                       (int)a.C, (int)a.To, (int)a.K, a.s, a.p, a.d, pl.TT, pl.NRW, pl.tblocks, pl.cblocks);
    return hipGetLastError();
}

template <typename T>
hipError_t run_typed(const Dw1dArgs &a, const Plan &pl, const void *x, const void *dy, void *dw, void *db,
                     void *ws)
{
    float *part = static_cast<float *>(ws);
    hipError_t err = hipSuccess;
    if (pl.ntiles == 0) {}   // empty batch: the reduction below writes zeros
    else if (pl.NT <= 1) err = run_partial<T, 1>(a, pl, x, dy, part);
    else if (pl.NT <= 2) err = run_partial<T, 2>(a, pl, x, dy, part);
    else if (pl.NT <= 4) err = run_partial<T, 4>(a, pl, x, dy, part);
    else if (pl.NT <= 8) err = run_partial<T, 8>(a, pl, x, dy, part);
    else err = run_partial<T, 16>(a, pl, x, dy, part);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((dw1d_btc_wgrad_reduce<T>), dim3((unsigned)((a.K + 1) * pl.cblocks)), dim3(kThreads), 0,
                       a.stream, (const float *)part, (T *)dw, (T *)db, (int)a.C, (int)a.K, pl.ntiles,
                       pl.cblocks);
    return hipGetLastError();
}

}  // namespace

bool dw1d_wgrad_plan(const Dw1dArgs &a, size_t *ws_bytes)
{
    const Plan pl = make_plan(a);
    if (pl.ok) *ws_bytes = pl.ws_bytes;
    return pl.ok;
}

hipError_t launch_dw1d_bwd_filter(const Dw1dArgs &a, const void *x, const void *dy, void *dw, void *db,
                                  void *ws, const char **kname)
{
    const Plan pl = make_plan(a);
    if (!pl.ok) return hipErrorInvalidValue;
    *kname = "dw1d_btc_wgrad_partial";
    switch (a.dtype) {
    case DT_F32: return run_typed<float>(a, pl, x, dy, dw, db, ws);
    case DT_F16: return run_typed<_Float16>(a, pl, x, dy, dw, db, ws);
    default: return run_typed<__bf16>(a, pl, x, dy, dw, db, ws);
    }
}

}  // namespace gconv
