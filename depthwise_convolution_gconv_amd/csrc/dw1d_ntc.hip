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
// dw1d_btc_tile<T, K, S, VE>: stride S (1 or 2), dilation 1, compile-time K.  One
//   workgroup per TT x CT output tile: it stages the tile's filters and its
//   (TT - 1) * S + K input steps
//   in LDS once (16-byte buffer loads, zero outside [0, T)), each thread takes the
//   K taps of its channel into registers and streams the input steps of its RT
//   outputs through them.  Tiles are dealt to the XCDs in contiguous runs, so the
//   halo steps shared by neighbouring tiles come from one L2.
// dw1d_btc_window<T, K, R>: stride 1, dilation 1, compile-time K, no LDS (used
//   when the tile kernel's alignment conditions do not hold).
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

constexpr int kCT = 64;   // channels per tile (one wave's lanes)
constexpr int kRG = kThreads / kCT;   // thread groups per tile, kRT outputs each
// Tile shape, chosen by measurement on the Conformer shape (8 x 1024 x 512, K = 31):
// 8 outputs per thread (32-step tiles).  64-step tiles measured the same; a
// persistent grid with double-buffered tiles measured slower.
constexpr int kRT = 8;                // outputs per thread
constexpr int kTT = kRG * kRT;        // outputs (steps) per tile
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past num_records: the load returns 0

template <int BYTES> struct RawLoad;
template <> struct RawLoad<16> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *d)
    {
        const uint4 u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w;
    }
};
template <> struct RawLoad<8> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *d)
    {
        const uint2 u = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
        d[0] = u.x; d[1] = u.y;
    }
};
template <> struct RawLoad<4> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *d)
    {
        d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
};
template <> struct RawLoad<2> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *d)
    {
        d[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    }
};

template <typename T> __device__ __forceinline__ float elem_f32(const uint32_t *d, int e);
template <> __device__ __forceinline__ float elem_f32<float>(const uint32_t *d, int e)
{
    return __builtin_bit_cast(float, d[e]);
}
template <> __device__ __forceinline__ float elem_f32<_Float16>(const uint32_t *d, int e)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(d[e >> 1] >> (16 * (e & 1))));
}
template <> __device__ __forceinline__ float elem_f32<__bf16>(const uint32_t *d, int e)
{
    return __builtin_bit_cast(float, (d[e >> 1] >> (16 * (e & 1))) << 16);
}

// VE: elements per input staging load (16 bytes, or one element when C or x is not
// aligned for that).  One workgroup per tile, sized so that every workgroup of the
// grid is resident at once on the Conformer shape (at most 64 registers a thread, 8
// workgroups per CU): the loads of all tiles are in flight together and no second
// round of workgroups waits for the first.
// FLIP: the taps are applied in reverse order (the input gradient at stride 1 is
// this convolution of dy with the filter reversed).
template <typename T, int K, int S, int VE, bool FLIP>
__global__ void __launch_bounds__(kThreads, 8)
dw1d_btc_tile(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
              T *__restrict__ y, int T_in, int C, int To, int pad, int tblocks, int cblocks,
              int tiles, int tiles_per_xcd)
{
    constexpr int NRW = (kTT - 1) * S + K;         // staged input steps
    constexpr int NWIN = (kRT - 1) * S + K;        // input steps of one thread's outputs
    constexpr int VPR = kCT / VE;                  // loads per staged step
    constexpr int NL = (NRW * VPR + kThreads - 1) / kThreads;   // input loads per thread
    constexpr int DW = (VE * sizeof(T) + 3) / 4;
    constexpr int WVE = 16 / sizeof(T);            // filter elements per 16-byte load
    constexpr int NWP = (kCT * K + WVE - 1) / WVE; // filter loads per tile
    constexpr int NW = (NWP + kThreads - 1) / kThreads;         // filter loads per thread
    // LDS: the tile's input steps, fp32 [step][channel].  The tile's filters (fp32,
    // [channel][tap]) pass through the same area first.
    __shared__ float xs[NRW][kCT];
    float *const ws = &xs[0][0];
    static_assert(kCT * K <= NRW * kCT, "the filters fit in the input area");

    // Tile of this workgroup: tiles are dealt to the XCDs in contiguous runs
    // (workgroup b runs on XCD b % 8), so neighbouring tiles, which share halo steps,
    // are read through one L2.
    const int xcd = blockIdx.x & 7, rank = blockIdx.x >> 3;
    const int tile = xcd * tiles_per_xcd + rank;
    if (tile >= min((xcd + 1) * tiles_per_xcd, tiles)) return;   // uniform over the workgroup

    const int tid = threadIdx.x;
    const int lane = tid % kCT, rg = tid / kCT;
    const int cb = tile % cblocks, tb = (tile / cblocks) % tblocks, bi = tile / (cblocks * tblocks);
    const int t0 = tb * kTT, c0 = cb * kCT;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T *>(x), (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T *>(w), (short)0, (int)((int64_t)C * K * sizeof(T)), 0x00020000);

    // All loads first: the tile's filters w[c0 .. c0+kCT), one contiguous run of
    // kCT*K elements (zero past the end of w), and input steps [t0 - pad, t0 - pad +
    // NRW) x channels [c0, c0 + kCT) (zero outside the sequence and past channel C).
    uint32_t d[NL][DW], e[NW][4];
    // Filters first: they are waited for (and staged) while the inputs are in flight.
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int i = tid + j * kThreads;
        RawLoad<16>::run(wrs, i < NWP ? (uint32_t)(((int64_t)c0 * K + (int64_t)i * WVE) * sizeof(T)) : kOOB, e[j]);
    }
    // This thread's bias, with the filters: a buffer load of no records when there is
    // no bias (it reads zero), so no branch, which would wait for every load before it.
    const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T *>(bias ? bias : w), (short)0, bias ? (int)((int64_t)C * sizeof(T)) : 0, 0x00020000);
    uint32_t bz[1];
    RawLoad<sizeof(T)>::run(brs, (uint32_t)((c0 + lane) * sizeof(T)), bz);   // zero past channel C
    const int64_t xbase = (int64_t)bi * T_in * C;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int i = tid + j * kThreads;
        const int r = i / VPR, v = i - r * VPR;
        const int ti = t0 * S - pad + r, c = c0 + v * VE;
        const bool ok = i < NRW * VPR && ti >= 0 && ti < T_in && c < C;
        RawLoad<VE * sizeof(T)>::run(xr, ok ? (uint32_t)((xbase + (int64_t)ti * C + c) * sizeof(T)) : kOOB, d[j]);
    }

    // Filters: through LDS into registers (tap k of this thread's channel).
#pragma unroll
    for (int j = 0; j < NW; ++j) {
#pragma unroll
        for (int q = 0; q < WVE; ++q) {
            const int idx = (tid + j * kThreads) * WVE + q;
            if (idx < kCT * K) ws[idx] = elem_f32<T>(e[j], q);
        }
    }
    __syncthreads();
    float wr[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wr[k] = ws[lane * K + (FLIP ? K - 1 - k : k)];
    const int c = c0 + lane;
    const bool cok = c < C;
    const float b0 = elem_f32<T>(bz, 0);
    __syncthreads();   // every thread has its taps; the area now takes the inputs

#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int i = tid + j * kThreads;
        if (i < NRW * VPR) {
            const int r = i / VPR, v = i - r * VPR;
#pragma unroll
            for (int q = 0; q < VE; ++q) xs[r][v * VE + q] = elem_f32<T>(d[j], q);
        }
    }
    __syncthreads();

    // kRT outputs of channel c: input step i of the thread's window feeds output r
    // through tap i - r*S.
    float acc[kRT];
#pragma unroll
    for (int r = 0; r < kRT; ++r) acc[r] = b0;
#pragma unroll
    for (int i = 0; i < NWIN; ++i) {
        // Input steps are read a few at a time (the other resident waves cover the
        // LDS latency), which keeps the thread within its 64 registers.
        const float xv = xs[rg * kRT * S + i][lane];
#pragma unroll
        for (int r = 0; r < kRT; ++r)
            if (i - r * S >= 0 && i - r * S < K) acc[r] = fmaf(xv, wr[i - r * S], acc[r]);
        // Each step's products are taken here (not sunk to the stores, which would
        // keep every input step live at once).
#pragma unroll
        for (int r = 0; r < kRT; ++r) asm volatile("" : "+v"(acc[r]));
    }
    T *yb = y + ((int64_t)bi * To + t0 + rg * kRT) * C + c;
    const int rmax = min(kRT, To - (t0 + rg * kRT));
#pragma unroll
    for (int r = 0; r < kRT; ++r)
        if (cok && r < rmax) store_nt(yb + (int64_t)r * C, from_f32<T>(acc[r]));
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

template <typename T, int K, int S, int VE, bool FLIP = false>
hipError_t run_tile(const Dw1dArgs &a)
{
    const int tblocks = (int)ceil_div(a.To, kTT), cblocks = (int)ceil_div(a.C, kCT);
    const int64_t tiles = a.B * tblocks * cblocks;
    const int64_t per_xcd = ceil_div(tiles, 8);
    const int64_t blocks = 8 * per_xcd;   // one workgroup per tile (the last XCD's run may be short)
    hipLaunchKernelGGL((dw1d_btc_tile<T, K, S, VE, FLIP>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                       (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, (int)a.T, (int)a.C,
                       (int)a.To, a.p, tblocks, cblocks, (int)tiles, (int)per_xcd);
    return hipGetLastError();
}

template <typename T, int K, int S, bool FLIP = false>
hipError_t run_tile_ve(const Dw1dArgs &a)
{
    constexpr int VE = 16 / sizeof(T);
    if (a.C % VE == 0 && (reinterpret_cast<uintptr_t>(a.x) & 15) == 0) return run_tile<T, K, S, VE, FLIP>(a);
    return run_tile<T, K, S, 1, FLIP>(a);
}

template <typename T, int K>
hipError_t run_tile_s(const Dw1dArgs &a)
{
    return a.s == 2 ? run_tile_ve<T, K, 2>(a) : run_tile_ve<T, K, 1>(a);
}

// The tile kernel applies: stride 1 or 2, dilation 1, the input addressable by a
// 31-bit byte offset, tile indices in int, w 16-byte aligned (its filter loads are
// 16 bytes wide), a filter length it is compiled for.
template <typename T>
bool tile_applies(const Dw1dArgs &a)
{
    const int64_t tiles = a.B * ceil_div(a.To, kTT) * ceil_div(a.C, kCT);
    const bool k_ok = a.K == 3 || a.K == 5 || a.K == 7 || a.K == 9 || a.K == 15 || a.K == 31;
    return k_ok && (a.s == 1 || a.s == 2) && a.d == 1 && a.B * a.T * a.C * (int64_t)sizeof(T) < (int64_t(1) << 31) &&
           (reinterpret_cast<uintptr_t>(a.w) & 15) == 0 && a.C * a.K * (int64_t)sizeof(T) < (int64_t(1) << 31) &&
           8 * ceil_div(tiles, 8) < (int64_t(1) << 31) && a.T + a.K < (int64_t(1) << 30);
}

// Input gradient, any stride and dilation: one thread per element of dx.  Output
// step t reads input step t*s - p + k*d, so input step i receives dy[t] * w[k] for
// every tap k with i + p - k*d = t*s, 0 <= t < To.
template <typename T>
__global__ void __launch_bounds__(kThreads)
dw1d_btc_bwd_data_generic(const T *__restrict__ dy, const T *__restrict__ w, T *__restrict__ dx,
                          int64_t total, int T_in, int C, int To, int K, int s, int p, int d)
{
    for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < total;
         j += (int64_t)gridDim.x * kThreads) {
        const int c = (int)(j % C);
        const int i = (int)((j / C) % T_in);
        const int64_t bi = j / ((int64_t)C * T_in);
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) {
            const int ts = i + p - k * d;
            if (ts < 0 || ts % s != 0 || ts / s >= To) continue;
            acc = fmaf(to_f32(dy[(bi * To + ts / s) * C + c]), to_f32(w[(int64_t)c * K + k]), acc);
        }
        dx[j] = from_f32<T>(acc);
    }
}

template <typename T>
hipError_t run_bwd_data(const Dw1dArgs &a, const void *dy, void *dx, const char **kname)
{
    // Stride 1, dilation 1, p <= K - 1: dx is the forward convolution of dy (To
    // steps) with the filter reversed and padding K - 1 - p, which has T outputs.
    Dw1dArgs f = a;
    f.x = dy; f.y = dx; f.bias = nullptr;
    f.T = a.To; f.To = a.T; f.p = (int32_t)(a.K - 1 - a.p);
    if (a.s == 1 && a.d == 1 && a.p <= a.K - 1 && tile_applies<T>(f)) {
        *kname = "dw1d_btc_tile_flip";
        switch (a.K) {
        case 3: return run_tile_ve<T, 3, 1, true>(f);
        case 5: return run_tile_ve<T, 5, 1, true>(f);
        case 7: return run_tile_ve<T, 7, 1, true>(f);
        case 9: return run_tile_ve<T, 9, 1, true>(f);
        case 15: return run_tile_ve<T, 15, 1, true>(f);
        default: return run_tile_ve<T, 31, 1, true>(f);
        }
    }
    *kname = "dw1d_btc_bwd_data_generic";
    const int64_t total = a.B * a.T * a.C;
    const int64_t blocks = std::min<int64_t>(ceil_div(total, kThreads), 1 << 20);
    hipLaunchKernelGGL((dw1d_btc_bwd_data_generic<T>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                       (const T *)dy, (const T *)a.w, (T *)dx, total, (int)a.T, (int)a.C, (int)a.To,
                       (int)a.K, a.s, a.p, a.d);
    return hipGetLastError();
}

template <typename T>
hipError_t run_typed(const Dw1dArgs &a, const char **kname)
{
    if (tile_applies<T>(a)) {
        *kname = "dw1d_btc_tile";
        switch (a.K) {
        case 3: return run_tile_s<T, 3>(a);
        case 5: return run_tile_s<T, 5>(a);
        case 7: return run_tile_s<T, 7>(a);
        case 9: return run_tile_s<T, 9>(a);
        case 15: return run_tile_s<T, 15>(a);
        case 31: return run_tile_s<T, 31>(a);
        default: break;
        }
    }
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

hipError_t launch_dw1d_bwd_data(const Dw1dArgs &a, const void *dy, void *dx, const char **kname)
{
    switch (a.dtype) {
    case DT_F32: return run_bwd_data<float>(a, dy, dx, kname);
    case DT_F16: return run_bwd_data<_Float16>(a, dy, dx, kname);
    default: return run_bwd_data<__bf16>(a, dy, dx, kname);
    }
}

}  // namespace gconv
