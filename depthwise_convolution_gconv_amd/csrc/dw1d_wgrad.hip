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
//    fp32 with 16-byte loads along C, 8 in flight per thread; the 4 waves split
//    the taps (wave g takes taps g, g+4, ...; wave 0 also sums dy for the bias),
//    lane = channel.  The tile's fp32 sums go to part[tile][k][c] (k = K holds
//    the bias sums).
//  * dw1d_btc_wgrad_reduce: one workgroup per (tap, 64 channels); 16 slices of
//    the tiles are summed in order (16-byte loads of 4 channels), then combined
//    in a fixed order and rounded once to the tensor dtype.
#include <algorithm>
#include <mutex>

#include "common.hpp"

namespace gconv {

// Device scratch of gconv_dw1d_bwd_filter_noalloc (the per-tile partial sums),
// for callers that cannot allocate.  Every GPU the library runs on holds its own
// copy until the process ends; host code never passes this name to a kernel (in
// host code it is only a stand-in), it passes the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kWgradScratchBytes];

namespace {

constexpr int kThreads = 256;
constexpr int kCT = 64;                      // channels per tile (lanes)
constexpr int kGroups = kThreads / kCT;      // waves, each taking every 4th tap
constexpr int kMaxTT = 64;                   // output steps per tile
constexpr int kLdsMax = 40 * 1024;           // 4 workgroups per CU

// Element e of VE consecutive values of T held in dwords.
template <typename T> __device__ __forceinline__ float elem(const uint32_t *v, int e);
template <> __device__ __forceinline__ float elem<float>(const uint32_t *v, int e)
{
    return __builtin_bit_cast(float, v[e]);
}
template <> __device__ __forceinline__ float elem<_Float16>(const uint32_t *v, int e)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v[e >> 1] >> (16 * (e & 1))));
}
template <> __device__ __forceinline__ float elem<__bf16>(const uint32_t *v, int e)
{
    return __builtin_bit_cast(float, (v[e >> 1] >> (16 * (e & 1))) << 16);
}

// NT: taps per wave (K <= 4 * NT).  VE: channels per staging load (16 bytes, or one
// element when C or the pointers do not allow that).
// UNIT (stride 1, dilation 1): wave g takes the contiguous taps g*NT .. g*NT+NT-1
// and slides a register window of NT input steps down the tile (one new LDS read
// per step); otherwise wave g takes taps g, g+4, ... and reads each from LDS.
template <typename T, int NT, int VE, bool UNIT>
__global__ void __launch_bounds__(kThreads)
dw1d_btc_wgrad_partial(const T *__restrict__ x, const T *__restrict__ dy, float *__restrict__ part,
                       int T_in, int C, int To, int K, int s, int p, int d, int TT, int NRW,
                       int tblocks, int cblocks)
{
    constexpr int DW = (VE * (int)sizeof(T) + 3) / 4;   // dwords per staging load
    constexpr int CPR = kCT / VE;                       // staging loads per row of 64 channels
    constexpr int NB = 16;                              // staging loads in flight per thread
    extern __shared__ float sm[];
    float *dys = sm;                  // [TT][kCT]
    float *xs = sm + TT * kCT;        // [NRW][kCT], directly after the dy rows
    const int tid = threadIdx.x, lane = tid % kCT, g = tid / kCT;
    int rest = blockIdx.x;
    const int cb = rest % cblocks;
    rest /= cblocks;
    const int tb = rest % tblocks;
    const int bi = rest / tblocks;
    const int t0 = tb * TT, c0 = cb * kCT, c = c0 + lane;
    const bool cok = c < C;

    // Stage the TT rows of dy[bi, t0 ..] and the NRW rows of x[bi, t0*s - p ..] (LDS
    // rows 0 .. TT + NRW, in that order), zero outside the tensors, VE channels per
    // load along C, NB loads in flight per thread.
    const T *dyb = dy + (int64_t)bi * To * C;
    const T *xb = x + (int64_t)bi * T_in * C;
    const int nchunks = (TT + NRW) * CPR;
    for (int base = 0; base < nchunks; base += NB * kThreads) {
        uint32_t v[NB][DW];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int i = base + j * kThreads + tid;
            const int r = i / CPR, cc = c0 + (i - r * CPR) * VE;
            const T *src = nullptr;
            if (i < nchunks && cc < C) {
                if (r < TT) {
                    if (t0 + r < To) src = dyb + (int64_t)(t0 + r) * C + cc;
                } else {
                    const int ti = t0 * s - p + (r - TT);
                    if (ti >= 0 && ti < T_in) src = xb + (int64_t)ti * C + cc;
                }
            }
#pragma unroll
            for (int q = 0; q < DW; ++q) v[j][q] = 0;
            if (src) {
                if constexpr (DW == 4) {
                    const uint4 u = *reinterpret_cast<const uint4 *>(src);
                    v[j][0] = u.x; v[j][1] = u.y; v[j][2] = u.z; v[j][3] = u.w;
                } else if constexpr (sizeof(T) == 4) {
                    v[j][0] = __builtin_bit_cast(uint32_t, *src);
                } else {
                    v[j][0] = __builtin_bit_cast(uint16_t, *src);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int i = base + j * kThreads + tid;
            if (i < nchunks) {
                const int r = i / CPR, cv = (i - r * CPR) * VE;
#pragma unroll
                for (int e = 0; e < VE; ++e) sm[r * kCT + cv + e] = elem<T>(v[j], e);
            }
        }
    }
    __syncthreads();

    float acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = 0.0f;
    float accb = 0.0f;
    const int tn = min(TT, To - t0);   // output steps of this tile that exist
    if constexpr (UNIT) {
        // Before step t + u, slot (j + u) % NT holds x row t + u + k0 + j; after the
        // step, the slot that held j = 0 takes row t + u + k0 + NT (rows up to
        // TT - 1 + 4*NT, all staged).
        const int k0 = g * NT;
        const float *xr = xs + k0 * kCT + lane;
        float win[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) win[j] = xr[j * kCT];
        int t = 0;
        for (; t + NT <= tn; t += NT) {
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                const float dv = dys[(t + u) * kCT + lane];
                accb += dv;
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[j] = fmaf(dv, win[(j + u) % NT], acc[j]);
                win[u] = xr[(t + u + NT) * kCT];
            }
        }
        for (; t < tn; ++t) {
            const float dv = dys[t * kCT + lane];
            accb += dv;
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[j] = fmaf(dv, xr[(t + j) * kCT], acc[j]);
        }
    } else {
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
    }
    if (!cok) return;
    float *pt = part + (int64_t)blockIdx.x / cblocks * (K + 1) * C + c;   // tile (bi, tb)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int k = UNIT ? g * NT + j : g + kGroups * j;
        if (k < K) pt[(int64_t)k * C] = acc[j];
    }
    if (g == 0) pt[(int64_t)K * C] = accb;
}

template <typename T>
__global__ void __launch_bounds__(kThreads)
dw1d_btc_wgrad_reduce(const float *__restrict__ part, T *__restrict__ dw, T *__restrict__ db,
                      int C, int K, int ntiles, int cblocks)
{
    // 16 slices of 16 lanes; lane l of a slice takes channels 4l .. 4l+3 of the block
    // (one 16-byte load per tile when C allows), slice q sums tiles q, q + 16, ...
    // in order, then slice 0 adds the 16 slice sums in order.
    constexpr int kSlices = kThreads / (kCT / 4);
    __shared__ float red[kSlices][kCT];
    const int tid = threadIdx.x, l16 = tid % (kCT / 4), q = tid / (kCT / 4);
    const int kk = blockIdx.x / cblocks, cb = blockIdx.x % cblocks;   // kk == K: the bias row
    const int c4 = cb * kCT + 4 * l16;
    const bool vec = (C & 3) == 0 && (reinterpret_cast<uintptr_t>(part) & 15) == 0;   // 16-byte loads
    constexpr int NB = 8;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const float *src = part + (int64_t)kk * C + c4;
    const int64_t step = (int64_t)(K + 1) * C;
    for (int i0 = q; i0 < ntiles; i0 += NB * kSlices) {
        float4 v[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int i = i0 + j * kSlices;
            v[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (i < ntiles) {
                const float *p = src + i * step;
                if (vec && c4 < C) {
                    v[j] = *reinterpret_cast<const float4 *>(p);
                } else {
                    if (c4 < C) v[j].x = p[0];
                    if (c4 + 1 < C) v[j].y = p[1];
                    if (c4 + 2 < C) v[j].z = p[2];
                    if (c4 + 3 < C) v[j].w = p[3];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            acc[0] += v[j].x; acc[1] += v[j].y; acc[2] += v[j].z; acc[3] += v[j].w;
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) red[q][4 * l16 + e] = acc[e];
    __syncthreads();
    if (tid >= kCT) return;
    const int lane = tid, c = cb * kCT + lane;
    if (c >= C) return;
    float v = 0.0f;
#pragma unroll
    for (int i = 0; i < kSlices; ++i) v += red[i][lane];
    if (kk < K) dw[(int64_t)c * K + kk] = from_f32<T>(v);
    else if (db) db[c] = from_f32<T>(v);
}

struct Plan {
    int TT, NRW, NT, tblocks, cblocks, ntiles;
    bool unit;
    size_t lds, ws_bytes;
    bool ok;
};

Plan make_plan(const Dw1dArgs &a)
{
    Plan pl{};
    pl.ok = false;
    // Taps per wave, as compiled: the next power of two (the window of the unit
    // path spans that many taps per wave).
    const int64_t nt = ceil_div(a.K, kGroups);
    if (nt > 16) return pl;                              // K <= 64
    pl.NT = nt <= 1 ? 1 : nt <= 2 ? 2 : nt <= 4 ? 4 : nt <= 8 ? 8 : 16;
    // Staged x rows: those the tile reads, and with unit stride and dilation the
    // window's reach (TT - 1 + 4*NT: the taps are rounded up to 4 waves of NT).
    pl.unit = a.s == 1 && a.d == 1;
    int64_t TT = kMaxTT, NRW = 0;
    for (; TT >= 1; TT /= 2) {
        NRW = (TT - 1) * a.s + (a.K - 1) * a.d + 1;
        if (pl.unit) NRW = std::max<int64_t>(NRW, TT + kGroups * pl.NT);
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

template <typename T, int NT, int VE, bool UNIT>
hipError_t run_partial_ve(const Dw1dArgs &a, const Plan &pl, const void *x, const void *dy, float *part)
{
    hipLaunchKernelGGL((dw1d_btc_wgrad_partial<T, NT, VE, UNIT>), dim3((unsigned)(pl.ntiles * (int64_t)pl.cblocks)),
                       dim3(kThreads), pl.lds, a.stream, (const T *)x, (const T *)dy, part, (int)a.T,
                       (int)a.C, (int)a.To, (int)a.K, a.s, a.p, a.d, pl.TT, pl.NRW, pl.tblocks, pl.cblocks);
    return hipGetLastError();
}

template <typename T, int NT>
hipError_t run_partial(const Dw1dArgs &a, const Plan &pl, const void *x, const void *dy, float *part)
{
    constexpr int VE = 16 / sizeof(T);
    const bool vec = a.C % VE == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(dy) & 15) == 0;
    if (pl.unit)
        return vec ? run_partial_ve<T, NT, VE, true>(a, pl, x, dy, part)
                   : run_partial_ve<T, NT, 1, true>(a, pl, x, dy, part);
    return vec ? run_partial_ve<T, NT, VE, false>(a, pl, x, dy, part)
               : run_partial_ve<T, NT, 1, false>(a, pl, x, dy, part);
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

// Device address of `scratch` on the current device, looked up once per device
// (each GPU holds the array at its own address).
hipError_t wgrad_scratch(void **out)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
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
