// nhwc.hip -- grouped conv2d over channels-last (NHWC) tensors.
//
// The discuss.pytorch.org thread "F.conv2d runs x15 slower in mixed-precision/
// half-precision mode" turns, in its later replies, to the NHWC (channels_last)
// memory format for the fp16 grouped conv.  Tensors: x [N][H][W][C],
// w [Cout][KH][KW][C/g] (the channels_last order of PyTorch's weights),
// y [N][OH][OW][Cout]; the sum is the one of the NCHW route.
//
// dw2d_nhwc_tile<T, K, S, VE>: depthwise layers (C/g = 1, Cout = C), K x K filters,
//   stride S (1 or 2), dilation 1.  Channels are the contiguous axis, so lanes map
//   to channels (as in the (batch, steps, channels) 1-D kernel): one workgroup =
//   64 channels x ROWS output rows (2 per wave at stride 1 where the patch fits
//   in 64 KB of LDS, else 1) x TW = 8/S output columns.  It stages the input patch
//   ((ROWS-1)*S + K rows x (TW-1)*S + K columns x 64 channels, zero outside the
//   image) and the 64 filters in LDS as fp32, with loads of VE channels along C;
//   each thread (one channel, each of its wave's rows) slides a window of (TW-1)*S + K
//   input columns down the K filter rows and stores TW outputs, each store of a
//   wave covering 64 consecutive channels.
// conv2d_nhwc_g4<T>, conv2d_nhwc_g4k3<T>: 4 in / 4 out channels per group (below).
// conv2d_nhwc_generic<T>: any groups, stride, padding and dilation; one thread per
//   output, output channels fastest (coalesced stores, and the group's input
//   channels are contiguous reads).
#include <algorithm>

#include "common.hpp"

namespace gconv {
namespace {

constexpr int kThreads = 256;
constexpr int kCT = 64;                  // channels per tile (lanes)
constexpr int kWaves = kThreads / kCT;

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

// Tile shape: TW output columns per thread, RPW output rows per wave (2 at stride
// 1 when the staged patch and filters fit in 64 KB of LDS, else 1), ROWS = 4 * RPW rows per
// workgroup, an IRH x IRW pixel input patch.
template <int K, int S> struct Tile {
    static constexpr int TW = 8 / S;
    static constexpr int IRW = (TW - 1) * S + K;
    static constexpr int bytes(int rows) { return (((rows - 1) * S + K) * IRW + K * K) * kCT * 4; }
    // Measured on the 8 x 512 x 40 x 256 layers: two rows per wave took the stride-1
    // bf16 layer from 58.9 to 56.4 us and the stride-2 fp32 one from 48.5 to 52.6 us.
    static constexpr int RPW = (S == 1 && bytes(2 * kWaves) <= 64 * 1024) ? 2 : 1;
    static constexpr int ROWS = kWaves * RPW;
    static constexpr int IRH = (ROWS - 1) * S + K;
};

template <typename T, int K, int S, int VE>
__global__ void __launch_bounds__(kThreads)
dw2d_nhwc_tile(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
               T *__restrict__ y, int H, int W, int C, int OH, int OW, int ph, int pw,
               int tiles_w, int tiles_h, int cblocks)
{
    constexpr int TW = Tile<K, S>::TW;
    constexpr int RPW = Tile<K, S>::RPW;
    constexpr int IRH = Tile<K, S>::IRH;              // staged input rows
    constexpr int IRW = Tile<K, S>::IRW;              // staged input columns
    constexpr int KK = K * K;
    constexpr int DW = (VE * (int)sizeof(T) + 3) / 4;
    constexpr int CPP = kCT / VE;                     // staging loads per pixel
    constexpr int NCH = IRH * IRW * CPP;              // staging loads per tile
    constexpr int NB = 8;
    __shared__ float xs[IRH][IRW][kCT];
    __shared__ float ws[KK][kCT];

    int rest = blockIdx.x;
    const int cb = rest % cblocks; rest /= cblocks;
    const int tw = rest % tiles_w; rest /= tiles_w;
    const int th = rest % tiles_h;
    const int n = rest / tiles_h;
    const int tid = threadIdx.x, lane = tid % kCT, rg = tid / kCT;
    const int c0 = cb * kCT, c = c0 + lane;
    const int oh0 = th * Tile<K, S>::ROWS, ow0 = tw * TW;
    const int ih0 = oh0 * S - ph, iw0 = ow0 * S - pw;
    // This channel's bias, loaded ahead of the staging from a valid address either
    // way (a load after the staging would wait for it).
    const float braw = to_f32(bias ? bias[min(c, C - 1)] : w[0]);

    // Filters [tap][channel] (zero past C).
    for (int i = tid; i < KK * kCT; i += kThreads) {
        const int t = i / kCT, cc = c0 + i % kCT;
        ws[t][i % kCT] = cc < C ? to_f32(w[(int64_t)cc * KK + t]) : 0.0f;
    }
    // Input patch, NB loads in flight per thread, zero outside the image and past C.
    const T *xn = x + (int64_t)n * H * W * C;
    for (int base = 0; base < NCH; base += NB * kThreads) {
        uint32_t v[NB][DW];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int i = base + j * kThreads + tid;
            const int pix = i / CPP, cv = (i - pix * CPP) * VE;
            const int r = pix / IRW, q = pix - r * IRW;
            const int ih = ih0 + r, iw = iw0 + q, cc = c0 + cv;
#pragma unroll
            for (int e = 0; e < DW; ++e) v[j][e] = 0;
            if (i < NCH && ih >= 0 && ih < H && iw >= 0 && iw < W && cc < C) {
                const T *src = xn + ((int64_t)ih * W + iw) * C + cc;
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
            if (i < NCH) {
                const int pix = i / CPP, cv = (i - pix * CPP) * VE;
                const int r = pix / IRW, q = pix - r * IRW;
#pragma unroll
                for (int e = 0; e < VE; ++e) xs[r][q][cv + e] = elem<T>(v[j], e);
            }
        }
    }
    __syncthreads();

    if (c >= C) return;
    const float b0 = bias ? braw : 0.0f;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
        const int lr = rg * RPW + rr, oh = oh0 + lr;   // row in the tile, output row
        if (oh >= OH) break;
        float acc[TW];
#pragma unroll
        for (int r = 0; r < TW; ++r) acc[r] = b0;
#pragma unroll
        for (int kh = 0; kh < K; ++kh) {
            float win[IRW];
#pragma unroll
            for (int q = 0; q < IRW; ++q) win[q] = xs[lr * S + kh][q][lane];
#pragma unroll
            for (int kw = 0; kw < K; ++kw) {
                const float wv = ws[kh * K + kw][lane];
#pragma unroll
                for (int r = 0; r < TW; ++r) acc[r] = fmaf(win[r * S + kw], wv, acc[r]);
            }
        }
        T *yp = y + (((int64_t)n * OH + oh) * OW + ow0) * C + c;
#pragma unroll
        for (int r = 0; r < TW; ++r)
            if (ow0 + r < OW) store_nt(yp + (int64_t)r * C, from_f32<T>(acc[r]));
    }
}

template <typename T>
__global__ void __launch_bounds__(kThreads)
conv2d_nhwc_generic(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
                    T *__restrict__ y, int64_t total, int C, int H, int W, int Cout, int KH, int KW,
                    int Cg, int Ng, int OH, int OW, int sh, int sw, int ph, int pw, int dh, int dw,
                    int interleaved)
{
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
        int64_t r = i;
        const int oc = (int)(r % Cout); r /= Cout;   // output channel; o is its filter
        const int ow = (int)(r % OW); r /= OW;
        const int oh = (int)(r % OH);
        const int64_t n = r / OH;
        const int G = Cout / Ng;
        const int o = interleaved ? (oc % G) * Ng + oc / G : oc;
        const int k = o / Ng;
        float acc = bias ? to_f32(bias[o]) : 0.0f;
        for (int kh = 0; kh < KH; ++kh) {
            const int ih = oh * sh - ph + kh * dh;
            if (ih < 0 || ih >= H) continue;
            for (int kw = 0; kw < KW; ++kw) {
                const int iw = ow * sw - pw + kw * dw;
                if (iw < 0 || iw >= W) continue;
                const T *xp = x + ((n * H + ih) * W + iw) * C + (int64_t)k * Cg;
                const T *wp = w + (((int64_t)o * KH + kh) * KW + kw) * Cg;
                for (int ci = 0; ci < Cg; ++ci) acc = fmaf(to_f32(xp[ci]), to_f32(wp[ci]), acc);
            }
        }
        y[i] = from_f32<T>(acc);
    }
}

// conv2d_nhwc_g4<T>: 4 input and 4 output channels per group (the ResNeXt-style
// cardinality of the neon issue), any filter, stride, padding and dilation.  One
// thread per (position, group): the group's 4 channels at each tap are one vector
// load (8 bytes in 16-bit, 16 in fp32), its 4 filters' taps come from L1, and the 4
// outputs are one vector store.  Lanes take consecutive groups of one position, so
// a wave's loads and stores are contiguous runs of 64 groups x 4 channels.
template <typename T> struct Vec4;
template <> struct Vec4<float> { typedef uint4 type; };
template <> struct Vec4<_Float16> { typedef uint2 type; };
template <> struct Vec4<__bf16> { typedef uint2 type; };

template <typename T>
__device__ __forceinline__ void unpack4(typename Vec4<T>::type v, float *f)
{
    const uint32_t *d = reinterpret_cast<const uint32_t *>(&v);
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = elem<T>(d, e);
}

template <typename T>
__global__ void __launch_bounds__(kThreads)
conv2d_nhwc_g4(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
               T *__restrict__ y, int64_t total, int G, int H, int W, int OH, int OW, int KH, int KW,
               int sh, int sw, int ph, int pw, int dh, int dw)
{
    typedef typename Vec4<T>::type V;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
        const int k = (int)(i % G);
        int64_t r = i / G;
        const int ow = (int)(r % OW); r /= OW;
        const int oh = (int)(r % OH);
        const int64_t n = r / OH;
        float acc[4];
#pragma unroll
        for (int o = 0; o < 4; ++o) acc[o] = bias ? to_f32(bias[4 * k + o]) : 0.0f;
        const T *wk = w + (int64_t)(4 * k) * KH * KW * 4;   // [o][kh][kw][ci] of the group's filters
        for (int kh = 0; kh < KH; ++kh) {
            const int ih = oh * sh - ph + kh * dh;
            if (ih < 0 || ih >= H) continue;
            for (int kw = 0; kw < KW; ++kw) {
                const int iw = ow * sw - pw + kw * dw;
                if (iw < 0 || iw >= W) continue;
                float xv[4];
                unpack4<T>(*reinterpret_cast<const V *>(x + ((n * H + ih) * W + iw) * 4 * G + 4 * k), xv);
#pragma unroll
                for (int o = 0; o < 4; ++o) {
                    float wv[4];
                    unpack4<T>(*reinterpret_cast<const V *>(wk + (((int64_t)o * KH + kh) * KW + kw) * 4), wv);
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[o] = fmaf(xv[c], wv[c], acc[o]);
                }
            }
        }
        V out;
        uint32_t *od = reinterpret_cast<uint32_t *>(&out);
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int o = 0; o < 4; ++o) od[o] = __builtin_bit_cast(uint32_t, acc[o]);
        } else {
#pragma unroll
            for (int q = 0; q < 2; ++q)
                od[q] = (uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(acc[2 * q])) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(acc[2 * q + 1])) << 16);
        }
        store_nt(reinterpret_cast<V *>(y + i * 4), out);
    }
}

// The same layer with 3 x 3 filters: each thread keeps its group's 4 x 9 x 4 filter
// values in registers (packed 16-bit, or fp32) and computes kG4Pos consecutive
// positions, so the weights are loaded once per thread instead of once per output.
constexpr int kG4Pos = 8;

template <typename T>
__global__ void __launch_bounds__(kThreads)
conv2d_nhwc_g4k3(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
                 T *__restrict__ y, int npix, int G, int H, int W, int OH, int OW,
                 int sh, int sw, int ph, int pw, int dh, int dw, int wgs, int wgs_per_xcd)
{
    typedef typename Vec4<T>::type V;
    // Workgroups are dealt to the XCDs in contiguous runs (workgroup b runs on XCD
    // b % 8), so the position blocks above and below, which read the same input
    // rows, are read through one L2.
    const int xcd = blockIdx.x & 7, rank = blockIdx.x >> 3;
    const int wg = xcd * wgs_per_xcd + rank;
    if (wg >= min((xcd + 1) * wgs_per_xcd, wgs)) return;   // uniform over the workgroup
    const int64_t t = (int64_t)wg * kThreads + threadIdx.x;
    const int k = (int)(t % G);
    const int64_t pb = t / G;                        // block of kG4Pos positions
    if (pb * kG4Pos >= npix) return;
    V wr[4][9];                                      // [output][tap]: the 4 input channels
#pragma unroll
    for (int o = 0; o < 4; ++o)
#pragma unroll
        for (int tp = 0; tp < 9; ++tp)
            wr[o][tp] = *reinterpret_cast<const V *>(w + ((int64_t)(4 * k + o) * 9 + tp) * 4);
    float b[4];
#pragma unroll
    for (int o = 0; o < 4; ++o) b[o] = bias ? to_f32(bias[4 * k + o]) : 0.0f;
    for (int j = 0; j < kG4Pos; ++j) {
        const int64_t pix = pb * kG4Pos + j;
        if (pix >= npix) break;
        const int ow = (int)(pix % OW);
        const int64_t r = pix / OW;
        const int oh = (int)(r % OH);
        const int64_t n = r / OH;
        float acc[4] = {b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int kh = 0; kh < 3; ++kh) {
            const int ih = oh * sh - ph + kh * dh;
            if (ih < 0 || ih >= H) continue;
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) {
                const int iw = ow * sw - pw + kw * dw;
                if (iw < 0 || iw >= W) continue;
                float xv[4];
                unpack4<T>(*reinterpret_cast<const V *>(x + ((n * H + ih) * W + iw) * 4 * G + 4 * k), xv);
#pragma unroll
                for (int o = 0; o < 4; ++o) {
                    float wv[4];
                    unpack4<T>(wr[o][kh * 3 + kw], wv);
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[o] = fmaf(xv[c], wv[c], acc[o]);
                }
            }
        }
        V out;
        uint32_t *od = reinterpret_cast<uint32_t *>(&out);
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int o = 0; o < 4; ++o) od[o] = __builtin_bit_cast(uint32_t, acc[o]);
        } else {
#pragma unroll
            for (int q = 0; q < 2; ++q)
                od[q] = (uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(acc[2 * q])) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(acc[2 * q + 1])) << 16);
        }
        store_nt(reinterpret_cast<V *>(y + (pix * G + k) * 4), out);
    }
}

// 16-bit 3 x 3 layers with column stride and dilation 1: each thread takes 8
// consecutive outputs of one output row for its group.  It loads its group's
// filters (4 outputs x 9 taps x 4 inputs, packed pairs) and the 3 x 10 input
// vectors the 8 outputs read, all before the first product, and accumulates with
// v_dot2_f32_{f16,bf16} (two products of 16-bit pairs added to an fp32 sum), so no
// operand is converted.  Index math is 32-bit and done once per thread.
template <typename T> __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c);
template <> __device__ __forceinline__ float dot2<_Float16>(uint32_t a, uint32_t b, float c)
{
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}
template <> __device__ __forceinline__ float dot2<__bf16>(uint32_t a, uint32_t b, float c)
{
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), c, false);
}

constexpr int kRowOut = 8;   // outputs per thread along a row

template <typename T>
__global__ void __launch_bounds__(kThreads)
conv2d_nhwc_g4k3_row(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
                     T *__restrict__ y, int G, int H, int W, int OH, int OW, int sh, int ph, int pw, int dh,
                     int nowb, int nrb, int nkb, int wgs, int wgs_per_xcd)
{
    // Workgroups are dealt to the XCDs in contiguous runs (workgroup b runs on XCD
    // b % 8), so neighbouring rows, which read the same input rows, share one L2.
    const int xcd = blockIdx.x & 7, rank = blockIdx.x >> 3;
    const int wg = xcd * wgs_per_xcd + rank;
    if (wg >= min((xcd + 1) * wgs_per_xcd, wgs)) return;   // uniform over the workgroup
    // A wave takes 16 consecutive groups (lanes mod 16) x 4 consecutive row blocks
    // (lanes / 16): each group's filters are read by 4 lanes at once, and each
    // position's 16 groups are one 128-byte run of x or y.  Waves take the group
    // blocks fastest.  Row block rbk = (n*OH + oh)*nowb + owb.
    const int t = wg * kThreads + (int)threadIdx.x;
    const int q = t >> 6, kb = q % nkb;
    const int k = kb * 16 + (t & 15);
    const int rbk = (q / nkb) * 4 + ((t >> 4) & 3);
    if (k >= G || rbk >= nrb) return;
    const int owb = rbk % nowb;
    const int r = rbk / nowb;
    const int oh = r % OH, n = r / OH;
    const int ow0 = owb * kRowOut;
    const int64_t rowstride = (int64_t)W * 4 * G;   // elements between input rows

    uint2 wr[4][9];   // [output][tap]: the 4 input channels as two packed pairs
#pragma unroll
    for (int o = 0; o < 4; ++o)
#pragma unroll
        for (int tp = 0; tp < 9; ++tp)
            wr[o][tp] = *reinterpret_cast<const uint2 *>(w + ((4 * k + o) * 9 + tp) * 4);
    // The bias is read from a valid address either way (the filters when there is
    // none) and issued with the other loads: a load under a branch would wait for
    // every load before it.
    const T *bp = bias ? bias + 4 * k : w + 4 * k;
    uint16_t braw[4];
#pragma unroll
    for (int o = 0; o < 4; ++o) braw[o] = __builtin_bit_cast(uint16_t, bp[o]);
    uint2 xr[3][kRowOut + 2];
#pragma unroll
    for (int kh = 0; kh < 3; ++kh) {
        const int ih = oh * sh - ph + kh * dh;
        const bool rok = ih >= 0 && ih < H;
        const T *xrow = x + ((int64_t)n * H + (rok ? ih : 0)) * rowstride + 4 * k;
#pragma unroll
        for (int c = 0; c < kRowOut + 2; ++c) {
            const int iw = ow0 - pw + c;
            xr[kh][c] = make_uint2(0, 0);
            if (rok && iw >= 0 && iw < W) xr[kh][c] = *reinterpret_cast<const uint2 *>(xrow + (int64_t)iw * 4 * G);
        }
    }
    float b[4];
#pragma unroll
    for (int o = 0; o < 4; ++o) b[o] = bias ? to_f32(__builtin_bit_cast(T, braw[o])) : 0.0f;
    T *yrow = y + (((int64_t)n * OH + oh) * OW) * 4 * G + 4 * k;
#pragma unroll
    for (int j = 0; j < kRowOut; ++j) {
        float acc[4] = {b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int kh = 0; kh < 3; ++kh)
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) {
                const uint2 xv = xr[kh][j + kw];
#pragma unroll
                for (int o = 0; o < 4; ++o) {
                    acc[o] = dot2<T>(xv.x, wr[o][kh * 3 + kw].x, acc[o]);
                    acc[o] = dot2<T>(xv.y, wr[o][kh * 3 + kw].y, acc[o]);
                }
            }
        if (ow0 + j < OW) {
            const uint2 out = make_uint2(
                (uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(acc[0])) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(acc[1])) << 16),
                (uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(acc[2])) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(acc[3])) << 16));
            store_nt(reinterpret_cast<uint2 *>(yrow + (int64_t)(ow0 + j) * 4 * G), out);
        }
    }
}

// conv2d_nhwc_g4_mfma<T, GPB>: 4 in / 4 out channels per group, 3 x 3, unit stride
// and dilation, padding at most 1, 16-bit.  One workgroup per (image, block of GPB
// groups = 4*GPB channels); the whole image of the block goes to LDS once.
//  * Staging: 16-byte loads along C (8 channels = 2 groups of one position) are
//    split into per-group planes of 8-byte entries (the 4 channels of a position),
//    each plane a zero-bordered padded image.  In NHWC a group's 4 channels are
//    already the 8 contiguous bytes of an entry, so no element is moved.
//  * Products: as in direct2d_g4, on v_mfma_f32_4x4x4_16b: a wave takes a group,
//    lanes take 64 consecutive anchors of its padded plane (anchor = the window's
//    top-left entry), each tap is one MFMA with A = the group's 4 x 4 filter matrix
//    at that tap (lane i%4 holds output i's 4 inputs, read straight from w) and
//    B = the anchor's 4 channels; per filter row two LDS reads give the kw = 0 and
//    kw = 2 operands and the kw = 1 operand is the next lane's kw = 0 value (a DPP
//    shift).
//  * Outputs: each anchor's 4 outputs (8 bytes) go to an LDS image of the block's
//    outputs, [position][GPB + 1 entries] (an odd row stride: the 8-byte writes of
//    64 consecutive positions fall on distinct banks), and the workgroup then
//    stores it along C with 16-byte non-temporal stores.
constexpr int kNG4Step = 62;   // anchors per pass (lanes 62, 63 only supply shifted operands)

__host__ __device__ inline int nhwc_g4_img(int HP, int WP, int OH, int OW)
{
    const int na = (OH - 1) * WP + OW;                            // anchors up to the last output
    const int npass = (na + kNG4Step - 1) / kNG4Step;
    const int reach = kNG4Step * (npass - 1) + 64 + 2 * WP + 2;   // entries any lane of any pass reads
    return (HP * WP > reach ? HP * WP : reach) | 1;               // odd: planes start on different banks
}

// q / d for 0 <= q < 2048 and 1 <= d <= 400 as (q * m) >> 20, m = ceil(2^20 / d)
// (the same exact range as the NCHW kernel's division), on the full-rate 24-bit
// multiply: both factors are below 2^24 and the product below 2^31.
__device__ __forceinline__ int ng4_div(int q, uint32_t m) { return (int)(__umul24((uint32_t)q, m) >> 20); }
// a * b for 0 <= a, b < 2^24 with a product below 2^31 (plane positions and sizes).
__device__ __forceinline__ int ng4_mul(int a, int b) { return (int)__umul24((uint32_t)a, (uint32_t)b); }

// The value lane + 1 holds (lane 63 receives zero; its result is not used): a DPP
// move with no old value, so the compiler need not copy the source first.
__device__ __forceinline__ uint2 ng4_next_lane(uint2 v)
{
    return make_uint2((uint32_t)__builtin_amdgcn_mov_dpp((int)v.x, 0x130, 0xf, 0xf, true),
                      (uint32_t)__builtin_amdgcn_mov_dpp((int)v.y, 0x130, 0xf, 0xf, true));
}
constexpr int kNG4NT = 2;   // buffer-store cache policy: non-temporal

typedef _Float16 ng4_f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 ng4_bf16x4 __attribute__((ext_vector_type(4)));
typedef float ng4_f32x4 __attribute__((ext_vector_type(4)));
template <typename T> struct NMfma4;
template <> struct NMfma4<_Float16> {
    static __device__ __forceinline__ ng4_f32x4 run(uint2 a, uint2 b, ng4_f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(ng4_f16x4, a), __builtin_bit_cast(ng4_f16x4, b),
                                                 c, 0, 0, 0);
    }
};
template <> struct NMfma4<__bf16> {
    static __device__ __forceinline__ ng4_f32x4 run(uint2 a, uint2 b, ng4_f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(ng4_bf16x4, a),
                                                     __builtin_bit_cast(ng4_bf16x4, b), c, 0, 0, 0);
    }
};
// Two fp32 values rounded to T and packed (a low), one paired conversion.
typedef _Float16 ng4_f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 ng4_bf16x2 __attribute__((ext_vector_type(2)));
template <typename T> __device__ __forceinline__ uint32_t ng4_pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t ng4_pack2<_Float16>(float a, float b)
{
    return __builtin_bit_cast(uint32_t, ng4_f16x2{(_Float16)a, (_Float16)b});
}
template <> __device__ __forceinline__ uint32_t ng4_pack2<__bf16>(float a, float b)
{
    return __builtin_bit_cast(uint32_t, ng4_bf16x2{(__bf16)a, (__bf16)b});
}

constexpr int kNG4MaxLoads = 8;   // 16-byte input loads per thread (H*W*GPB/2 <= 2048)

template <typename T, int GPB>
__global__ void __launch_bounds__(kThreads)
conv2d_nhwc_g4_mfma(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
                    T *__restrict__ y, int C, int H, int W, int OH, int OW, int ph, int pw, int cblocks, int img,
                    uint32_t mw, uint32_t mwp, int wgs, int wgs_per_xcd)
{
    constexpr int PP = GPB / 2;       // 16-byte pieces of a position's block
    constexpr int GPW = GPB / 4;      // groups per wave
    constexpr int YS = GPB + 1;       // entries per position of the output image
    extern __shared__ __attribute__((aligned(16))) uint2 ng4s[];
    uint2 *xs = ng4s;                 // [GPB][img] padded planes
    uint2 *ys = ng4s + GPB * img;     // [OH*OW][YS] outputs
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Workgroup b runs on XCD b % 8; the XCDs take contiguous runs of (image, channel
    // block) pairs, so the neighbouring blocks of a position, which share its cache
    // lines, are read and written through one L2.
    const int wg = (blockIdx.x & 7) * wgs_per_xcd + (blockIdx.x >> 3);
    if (wg >= wgs) return;   // uniform over the workgroup
    const int cb = wg % cblocks, n = wg / cblocks;
    const int HP = H + 2 * ph, WP = W + 2 * pw, HW = H * W, OHW = OH * OW;
    const int c0 = cb * 4 * GPB;      // first channel of the block
    const int npiece = HW * PP;

    // Every global load is issued before the first is used: the image pieces, then
    // this wave's filters (lane i % 4: output i's 4 inputs at each tap) and biases.
    // The image's block through one buffer: byte offsets (pos * C + 8 * part) * 2,
    // below 2^31, with pos * C on the 24-bit multiply (C < 2^24; both planned).
    const T *xn = x + (int64_t)n * HW * C + c0;
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(xn), (short)0, 0x7fffffff, 0x00020000);
    uint4 xv[kNG4MaxLoads];
#pragma unroll
    for (int j = 0; j < kNG4MaxLoads; ++j) {
        if (kThreads * j < npiece) {   // uniform; the piece index is clamped, not branched on
            const int i = min(tid + kThreads * j, npiece - 1);
            const int pos = i / PP, part = i - pos * PP;
            xv[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, 2 * (ng4_mul(pos, C) + 8 * part), 0, 0));
        }
    }
    uint2 fa[GPW][9], bz[GPW];
#pragma unroll
    for (int s = 0; s < GPW; ++s) {
        const int o = c0 + 4 * (wave + 4 * s);   // first output channel of the group
        const T *wg = w + (int64_t)(o + (lane & 3)) * 36;
#pragma unroll
        for (int t = 0; t < 9; ++t) fa[s][t] = *reinterpret_cast<const uint2 *>(wg + 4 * t);
        bz[s] = bias ? *reinterpret_cast<const uint2 *>(bias + o) : make_uint2(0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep every load ahead of the first use

    // Planes: border entries zero (with padding 0 or 1: the top and bottom rows,
    // 2*ph*WP entries, then the left and right columns of the H image rows, 2*pw*H
    // entries; a lane decodes one and zeroes it in the wave's planes), image entries
    // from the pieces.
    const int nborder = HP * WP - HW;
    for (int b = lane; b < nborder; b += 64) {
        int hp, wp;
        if (b < 2 * ph * WP) {
            const bool bottom = b >= WP;
            hp = bottom ? HP - 1 : 0;
            wp = bottom ? b - WP : b;
        } else {
            const int j = b - 2 * ph * WP;
            hp = ph + (j >> 1);
            wp = (j & 1) ? WP - 1 : 0;
        }
        const int e = ng4_mul(hp, WP) + wp;
#pragma unroll
        for (int sg = 0; sg < GPW; ++sg) xs[ng4_mul(wave + 4 * sg, img) + e] = make_uint2(0, 0);
    }
#pragma unroll
    for (int j = 0; j < kNG4MaxLoads; ++j) {
        const int i = tid + kThreads * j;
        if (kThreads * j < npiece && i < npiece) {
            const int pos = i / PP, part = i - pos * PP;
            const int h = ng4_div(pos, mw), ww = pos - ng4_mul(h, W);
            const int e = ng4_mul(h + ph, WP) + ww + pw;
            xs[ng4_mul(2 * part, img) + e] = make_uint2(xv[j].x, xv[j].y);
            xs[ng4_mul(2 * part + 1, img) + e] = make_uint2(xv[j].z, xv[j].w);
        }
    }
    __syncthreads();

    const int na = (OH - 1) * WP + OW;
#pragma unroll
    for (int s = 0; s < GPW; ++s) {
        const int gl = wave + 4 * s;
        const uint2 *pl = xs + gl * img;
        ng4_f32x4 b0;
        b0[0] = to_f32(__builtin_bit_cast(T, (uint16_t)(bz[s].x & 0xffffu)));
        b0[1] = to_f32(__builtin_bit_cast(T, (uint16_t)(bz[s].x >> 16)));
        b0[2] = to_f32(__builtin_bit_cast(T, (uint16_t)(bz[s].y & 0xffffu)));
        b0[3] = to_f32(__builtin_bit_cast(T, (uint16_t)(bz[s].y >> 16)));
        for (int a0 = 0; a0 < na; a0 += kNG4Step) {
            const int a = a0 + lane;
            ng4_f32x4 acc = b0;
#pragma unroll
            for (int kh = 0; kh < 3; ++kh) {
                const uint2 v0 = pl[a + kh * WP];
                const uint2 v2 = pl[a + kh * WP + 2];   // inside the plane's entries for every lane
                const uint2 v1 = ng4_next_lane(v0);
                acc = NMfma4<T>::run(fa[s][kh * 3 + 0], v0, acc);
                acc = NMfma4<T>::run(fa[s][kh * 3 + 1], v1, acc);
                acc = NMfma4<T>::run(fa[s][kh * 3 + 2], v2, acc);
            }
            const int oh = ng4_div(a, mwp), ow = a - ng4_mul(oh, WP);
            if (lane < kNG4Step && a < na && ow < OW)
                ys[ng4_mul(ng4_mul(oh, OW) + ow, YS) + gl] =
                    make_uint2(ng4_pack2<T>(acc[0], acc[1]), ng4_pack2<T>(acc[2], acc[3]));
        }
    }
    __syncthreads();

    // The block's outputs along C: piece (position, part) is channels c0 + 8*part ..
    // of one position, 16 bytes.
    // Byte offsets (pos * C + 8 * part) * 2 from the block's first output, below 2^31
    // (planned).
    T *yn = y + (int64_t)n * OHW * C + c0;
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(yn, (short)0, 0x7fffffff, 0x00020000);
    for (int i = tid; i < OHW * PP; i += kThreads) {
        const int pos = i / PP, part = i - pos * PP;
        const uint2 lo = ys[ng4_mul(pos, YS) + 2 * part], hi = ys[ng4_mul(pos, YS) + 2 * part + 1];
        __builtin_amdgcn_raw_buffer_store_b128(gconv_u32x4{lo.x, lo.y, hi.x, hi.y}, yr, 2 * (ng4_mul(pos, C) + 8 * part), 0,
                                               kNG4NT);
    }
}

// Groups per workgroup of conv2d_nhwc_g4_mfma, or 0 when it does not apply: 4*GPB
// channels dividing C, the image within the load registers (H*W*GPB/2 pieces of
// 16 bytes over 256 threads, 8 each at most) and the planes and outputs within
// 40 KB of LDS (4 workgroups per CU).
template <typename T>
int nhwc_g4_mfma_gpb(const Conv2dArgs &a, size_t *lds, int *img)
{
    if constexpr (sizeof(T) != 2) {
        return 0;
    } else {
        if (!(a.C == 4 * a.groups && a.Cout == a.C && !a.interleaved && a.KH == 3 && a.KW == 3 && a.sh == 1 &&
              a.sw == 1 && a.dh == 1 && a.dw == 1 && a.ph <= 1 && a.pw <= 1 && a.W + 2 * a.pw <= 400 &&
              (a.H + 2 * a.ph) * (a.W + 2 * a.pw) <= 1024 && a.H * a.W * a.C < (int64_t(1) << 30) &&
              a.OH * a.OW * a.C < (int64_t(1) << 30) && a.C < (int64_t(1) << 24) &&
              ((reinterpret_cast<uintptr_t>(a.x) | reinterpret_cast<uintptr_t>(a.y)) & 15) == 0 &&
              ((reinterpret_cast<uintptr_t>(a.w) | reinterpret_cast<uintptr_t>(a.bias)) & 7) == 0))
            return 0;
        const int HP = (int)(a.H + 2 * a.ph), WP = (int)(a.W + 2 * a.pw), OH = (int)a.OH, OW = (int)a.OW;
        for (int gpb : {8, 4}) {
            if (a.C % (4 * gpb) != 0 || a.H * a.W * (gpb / 2) > kThreads * kNG4MaxLoads) continue;
            const int im = nhwc_g4_img(HP, WP, OH, OW);
            const size_t bytes = ((size_t)gpb * im + (size_t)OH * OW * (gpb + 1)) * sizeof(uint2);
            if (bytes > 40 * 1024) continue;
            if (a.N * (a.C / (4 * gpb)) >= (int64_t(1) << 30)) continue;
            *lds = bytes;
            *img = im;
            return gpb;
        }
        return 0;
    }
}

// dw2d_nhwc_pair<T, K, S>: the depthwise tile kernel for 16-bit tensors with C a
// multiple of 8, each lane taking a pair of adjacent channels.  The patch stays in
// the tensor's 16-bit format in LDS, one dword per (position, channel pair), so a
// 16-byte load along C (8 channels) is one 16-byte LDS write and one window read
// serves two channels: a tile is 128 channels x ROWS output rows x TW columns, with
// the LDS footprint of the fp32 tile of 64 channels.
constexpr int kCP = 2 * kCT;   // channels per tile of the pair kernel

template <typename T> __device__ __forceinline__ float lo16(uint32_t v);
template <typename T> __device__ __forceinline__ float hi16(uint32_t v);
template <> __device__ __forceinline__ float lo16<_Float16>(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)v); }
template <> __device__ __forceinline__ float hi16<_Float16>(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }
template <> __device__ __forceinline__ float lo16<__bf16>(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
template <> __device__ __forceinline__ float hi16<__bf16>(uint32_t v) { return __builtin_bit_cast(float, v & 0xffff0000u); }

template <typename T, int K, int S>
__global__ void __launch_bounds__(kThreads)
dw2d_nhwc_pair(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
               T *__restrict__ y, int H, int W, int C, int OH, int OW, int ph, int pw,
               int tiles_w, int tiles_h, int cblocks)
{
    constexpr int TW = Tile<K, S>::TW;
    constexpr int RPW = Tile<K, S>::RPW;
    constexpr int IRH = Tile<K, S>::IRH;
    constexpr int IRW = Tile<K, S>::IRW;
    constexpr int KK = K * K;
    constexpr int PPP = kCP / 8;                      // 16-byte pieces per position
    constexpr int NCH = IRH * IRW * PPP;              // staging loads per tile
    constexpr int NB = 8;
    __shared__ uint4 xs[IRH][IRW][kCT / 4];           // [row][column][channel pair], 4 pairs a unit
    __shared__ float2 ws[KK][kCT];                    // [tap][channel pair]

    int rest = blockIdx.x;
    const int cb = rest % cblocks; rest /= cblocks;
    const int tw = rest % tiles_w; rest /= tiles_w;
    const int th = rest % tiles_h;
    const int n = rest / tiles_h;
    const int tid = threadIdx.x, lane = tid % kCT, rg = tid / kCT;
    const int c0 = cb * kCP, c = c0 + 2 * lane;       // the lane's channels c, c + 1
    const int oh0 = th * Tile<K, S>::ROWS, ow0 = tw * TW;
    const int ih0 = oh0 * S - ph, iw0 = ow0 * S - pw;
    // The pair's bias, loaded ahead of the staging from a valid address either way.
    const uint32_t braw = *reinterpret_cast<const uint32_t *>((bias ? bias : w) + (c < C ? c : 0));

    // Filters [tap][pair] (zero past C).
    for (int i = tid; i < KK * kCT; i += kThreads) {
        const int t = i / kCT, p = i % kCT, cc = c0 + 2 * p;
        ws[t][p] = cc < C ? make_float2(to_f32(w[(int64_t)cc * KK + t]), to_f32(w[(int64_t)(cc + 1) * KK + t]))
                          : make_float2(0.0f, 0.0f);
    }
    // Input patch, NB 16-byte loads in flight per thread, zero outside the image and
    // past C (C is a multiple of 8: a piece is all in or all out).
    const T *xn = x + (int64_t)n * H * W * C;
    uint4 *xsu = &xs[0][0][0];
    for (int base = 0; base < NCH; base += NB * kThreads) {
        uint4 v[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int i = base + j * kThreads + tid;
            const int pix = i / PPP, part = i - pix * PPP;
            const int r = pix / IRW, q = pix - r * IRW;
            const int ih = ih0 + r, iw = iw0 + q, cc = c0 + 8 * part;
            v[j] = make_uint4(0, 0, 0, 0);
            if (i < NCH && ih >= 0 && ih < H && iw >= 0 && iw < W && cc < C)
                v[j] = *reinterpret_cast<const uint4 *>(xn + ((int64_t)ih * W + iw) * C + cc);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int i = base + j * kThreads + tid;
            if (i < NCH) xsu[i] = v[j];   // unit i = (row, column, part) in row-major order
        }
    }
    __syncthreads();

    if (c >= C) return;
    const uint32_t *xsp = reinterpret_cast<const uint32_t *>(&xs[0][0][0]);
    const float b0 = bias ? lo16<T>(braw) : 0.0f, b1 = bias ? hi16<T>(braw) : 0.0f;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
        const int lr = rg * RPW + rr, oh = oh0 + lr;
        if (oh >= OH) break;
        float a0[TW], a1[TW];
#pragma unroll
        for (int r = 0; r < TW; ++r) { a0[r] = b0; a1[r] = b1; }
#pragma unroll
        for (int kh = 0; kh < K; ++kh) {
            uint32_t win[IRW];
#pragma unroll
            for (int q = 0; q < IRW; ++q) win[q] = xsp[((lr * S + kh) * IRW + q) * kCT + lane];
#pragma unroll
            for (int kw = 0; kw < K; ++kw) {
                const float2 wv = ws[kh * K + kw][lane];
#pragma unroll
                for (int r = 0; r < TW; ++r) {
                    a0[r] = fmaf(lo16<T>(win[r * S + kw]), wv.x, a0[r]);
                    a1[r] = fmaf(hi16<T>(win[r * S + kw]), wv.y, a1[r]);
                }
            }
        }
        T *yp = y + (((int64_t)n * OH + oh) * OW + ow0) * C + c;
#pragma unroll
        for (int r = 0; r < TW; ++r)
            if (ow0 + r < OW)
                store_nt(reinterpret_cast<uint32_t *>(yp + (int64_t)r * C),
                         (uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(a0[r])) |
                             ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(a1[r])) << 16));
    }
}

template <typename T, int K, int S>
hipError_t run_pair(const Conv2dArgs &a)
{
    constexpr int TW = Tile<K, S>::TW;
    const int tiles_w = (int)ceil_div(a.OW, TW), tiles_h = (int)ceil_div(a.OH, Tile<K, S>::ROWS);
    const int cblocks = (int)ceil_div(a.C, kCP);
    const int64_t blocks = a.N * tiles_h * tiles_w * cblocks;
    hipLaunchKernelGGL((dw2d_nhwc_pair<T, K, S>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                       (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, (int)a.H, (int)a.W,
                       (int)a.C, (int)a.OH, (int)a.OW, a.ph, a.pw, tiles_w, tiles_h, cblocks);
    return hipGetLastError();
}

template <typename T, int K, int S, int VE>
hipError_t run_tile(const Conv2dArgs &a)
{
    constexpr int TW = Tile<K, S>::TW;
    const int tiles_w = (int)ceil_div(a.OW, TW), tiles_h = (int)ceil_div(a.OH, Tile<K, S>::ROWS);
    const int cblocks = (int)ceil_div(a.C, kCT);
    const int64_t blocks = a.N * tiles_h * tiles_w * cblocks;
    hipLaunchKernelGGL((dw2d_nhwc_tile<T, K, S, VE>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                       (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, (int)a.H, (int)a.W,
                       (int)a.C, (int)a.OH, (int)a.OW, a.ph, a.pw, tiles_w, tiles_h, cblocks);
    return hipGetLastError();
}

template <typename T, int K, int S>
hipError_t run_tile_ve(const Conv2dArgs &a)
{
    constexpr int VE = 16 / sizeof(T);
    if (a.C % VE == 0 && (reinterpret_cast<uintptr_t>(a.x) & 15) == 0) return run_tile<T, K, S, VE>(a);
    return run_tile<T, K, S, 1>(a);
}

template <typename T, int K>
hipError_t run_tile_s(const Conv2dArgs &a)
{
    return a.sh == 2 ? run_tile_ve<T, K, 2>(a) : run_tile_ve<T, K, 1>(a);
}

template <typename T>
hipError_t run_typed(const Conv2dArgs &a, const char **kname)
{
    // Depthwise tile kernel: C/g = 1 and one filter per channel, square K in {3, 5, 7},
    // square stride 1 or 2, dilation 1, tile indices and one image's offsets in int.
    const bool dw = a.groups == a.C && a.Cout == a.C && a.KH == a.KW &&
                    (a.KH == 3 || a.KH == 5 || a.KH == 7) && a.sh == a.sw && (a.sh == 1 || a.sh == 2) &&
                    a.dh == 1 && a.dw == 1 && a.H * a.W * a.C < (int64_t(1) << 31) &&
                    a.N * a.OH * ceil_div(a.OW, 8 / a.sh) * ceil_div(a.C, kCT) < (int64_t(1) << 31);
    if (dw) {
        if constexpr (sizeof(T) == 2) {
            // 16-bit, C a multiple of 8, x 16-byte and y, w, bias 4-byte aligned: the
            // channel-pair kernel.
            if (a.C % 8 == 0 && (reinterpret_cast<uintptr_t>(a.x) & 15) == 0 &&
                ((reinterpret_cast<uintptr_t>(a.y) | reinterpret_cast<uintptr_t>(a.w) |
                  reinterpret_cast<uintptr_t>(a.bias)) & 3) == 0) {
                *kname = "dw2d_nhwc_pair";
                switch (a.KH) {
                case 3: return a.sh == 2 ? run_pair<T, 3, 2>(a) : run_pair<T, 3, 1>(a);
                case 5: return a.sh == 2 ? run_pair<T, 5, 2>(a) : run_pair<T, 5, 1>(a);
                default: return a.sh == 2 ? run_pair<T, 7, 2>(a) : run_pair<T, 7, 1>(a);
                }
            }
        }
        *kname = "dw2d_nhwc_tile";
        switch (a.KH) {
        case 3: return run_tile_s<T, 3>(a);
        case 5: return run_tile_s<T, 5>(a);
        default: return run_tile_s<T, 7>(a);
        }
    }
    // 4 in / 4 out per group, grouped output order, vector-aligned tensors.
    constexpr uintptr_t kVecAlign = 4 * sizeof(T) - 1;
    if (a.C == 4 * a.groups && a.Cout == a.C && !a.interleaved &&
        ((reinterpret_cast<uintptr_t>(a.x) | reinterpret_cast<uintptr_t>(a.w) |
          reinterpret_cast<uintptr_t>(a.y)) & kVecAlign) == 0) {
        const int64_t npix = a.N * a.OH * a.OW;
        if constexpr (sizeof(T) == 2) {
            size_t lds = 0;
            int img = 0;
            const int gpb = nhwc_g4_mfma_gpb<T>(a, &lds, &img);
            if (gpb) {
                *kname = "conv2d_nhwc_g4_mfma";
                const int cblocks = (int)(a.C / (4 * gpb));
                const int WP = (int)(a.W + 2 * a.pw);
                const uint32_t mw = (uint32_t)(((1u << 20) + a.W - 1) / a.W), mwp = (uint32_t)(((1u << 20) + WP - 1) / WP);
                const int wgs = (int)(a.N * cblocks), per_xcd = (int)ceil_div(wgs, 8);
                auto launch = [&](auto kern) {
                    hipLaunchKernelGGL(kern, dim3((unsigned)(8 * per_xcd)), dim3(kThreads), lds, a.stream,
                                       (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, (int)a.C,
                                       (int)a.H, (int)a.W, (int)a.OH, (int)a.OW, a.ph, a.pw, cblocks, img, mw, mwp,
                                       wgs, per_xcd);
                };
                if (gpb == 16) launch(conv2d_nhwc_g4_mfma<T, 16>);
                else if (gpb == 8) launch(conv2d_nhwc_g4_mfma<T, 8>);
                else launch(conv2d_nhwc_g4_mfma<T, 4>);
                return hipGetLastError();
            }
            const int64_t nowb = ceil_div(a.OW, kRowOut);
            const int64_t nrb = a.N * a.OH * nowb, nkb = ceil_div(a.groups, 16);
            const int64_t total = nkb * ceil_div(nrb, 4) * 64;   // threads, whole waves
            if (a.KH == 3 && a.KW == 3 && a.sw == 1 && a.dw == 1 &&
                8 * ceil_div(ceil_div(total, kThreads), 8) * kThreads < (int64_t(1) << 31) &&
                a.Cout * 9 * 4 < (int64_t(1) << 31)) {
                *kname = "conv2d_nhwc_g4k3_row";
                const int64_t wgs = ceil_div(total, kThreads), per_xcd = ceil_div(wgs, 8);
                hipLaunchKernelGGL((conv2d_nhwc_g4k3_row<T>), dim3((unsigned)(8 * per_xcd)), dim3(kThreads), 0,
                                   a.stream, (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y,
                                   (int)a.groups, (int)a.H, (int)a.W, (int)a.OH, (int)a.OW, a.sh, a.ph, a.pw, a.dh,
                                   (int)nowb, (int)nrb, (int)nkb, (int)wgs, (int)per_xcd);
                return hipGetLastError();
            }
        }
        if (a.KH == 3 && a.KW == 3 && npix < (int64_t(1) << 31) &&
            8 * ceil_div(ceil_div(ceil_div(npix, kG4Pos) * a.groups, kThreads), 8) < (int64_t(1) << 31)) {
            *kname = "conv2d_nhwc_g4k3";
            const int64_t threads = ceil_div(npix, kG4Pos) * a.groups;
            const int64_t wgs = ceil_div(threads, kThreads), per_xcd = ceil_div(wgs, 8);
            hipLaunchKernelGGL((conv2d_nhwc_g4k3<T>), dim3((unsigned)(8 * per_xcd)), dim3(kThreads), 0,
                               a.stream, (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, (int)npix,
                               (int)a.groups, (int)a.H, (int)a.W, (int)a.OH, (int)a.OW, a.sh, a.sw, a.ph, a.pw,
                               a.dh, a.dw, (int)wgs, (int)per_xcd);
            return hipGetLastError();
        }
        *kname = "conv2d_nhwc_g4";
        const int64_t total = a.N * a.OH * a.OW * a.groups;
        const int64_t blocks = std::min<int64_t>(ceil_div(total, kThreads), 1 << 20);
        hipLaunchKernelGGL((conv2d_nhwc_g4<T>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                           (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, total, (int)a.groups,
                           (int)a.H, (int)a.W, (int)a.OH, (int)a.OW, (int)a.KH, (int)a.KW, a.sh, a.sw, a.ph, a.pw,
                           a.dh, a.dw);
        return hipGetLastError();
    }
    *kname = "conv2d_nhwc_generic";
    const int64_t total = a.N * a.OH * a.OW * a.Cout;
    const int64_t blocks = std::min<int64_t>(ceil_div(total, kThreads), 1 << 20);
    hipLaunchKernelGGL((conv2d_nhwc_generic<T>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                       (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, total, (int)a.C, (int)a.H,
                       (int)a.W, (int)a.Cout, (int)a.KH, (int)a.KW, (int)(a.C / a.groups),
                       (int)(a.Cout / a.groups), (int)a.OH, (int)a.OW, a.sh, a.sw, a.ph, a.pw, a.dh, a.dw,
                       a.interleaved);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv2d_nhwc(const Conv2dArgs &a, const char **kname)
{
    switch (a.dtype) {
    case DT_F32: return run_typed<float>(a, kname);
    case DT_F16: return run_typed<_Float16>(a, kname);
    default: return run_typed<__bf16>(a, kname);
    }
}

}  // namespace gconv
