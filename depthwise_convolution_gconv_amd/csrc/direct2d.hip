// direct2d.hip -- direct grouped conv2d (NCHW) on the vector ALUs.
//
// Direct route.  The group index is folded into the launch grid instead of one
// launch per group: the neon issue "Grouped convolutions" proposes offsetting
// the input and output pointers by blockIdx * group stride (ibmua's reply), and
// its replies note that launching one kernel per group costs a fixed overhead
// per launch that swamps small layers.
//
// Two kernels:
//  * direct2d_tiled: one workgroup = (image n, group k, block of NB output
//    channels, TH x TW output tile).  The group's input channels are staged
//    chunk by chunk into LDS as a zero-filled halo tile (coalesced loads along
//    W), the NB x chunk x KH x KW filters next to them, and every thread keeps
//    NB fp32 accumulators for one output position.
//  * direct2d_naive: one thread per output, everything read from global memory.
//    Used only when a halo tile of one channel does not fit in LDS (huge
//    dilation or kernel).
#include <algorithm>

#include "common.hpp"

namespace gconv {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsBudget = 64 * 1024;  // bytes of LDS one tiled workgroup may use

template <typename T>
__global__ void __launch_bounds__(kThreads)
direct2d_naive(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
               T *__restrict__ y, int64_t total, int C, int H, int W, int Cout, int KH, int KW,
               int Cg, int Ng, int OH, int OW, int sh, int sw, int ph, int pw, int dh, int dw)
{
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
        int64_t r = i;
        const int ow = (int)(r % OW); r /= OW;
        const int oh = (int)(r % OH); r /= OH;
        const int o = (int)(r % Cout);
        const int64_t n = r / Cout;
        const int k = o / Ng;
        float acc = bias ? to_f32(bias[o]) : 0.0f;
        const T *xg = x + (n * C + (int64_t)k * Cg) * H * W;
        const T *wo = w + (int64_t)o * Cg * KH * KW;
        for (int ci = 0; ci < Cg; ++ci) {
            for (int kh = 0; kh < KH; ++kh) {
                const int ih = oh * sh - ph + kh * dh;
                if (ih < 0 || ih >= H) continue;
                for (int kw = 0; kw < KW; ++kw) {
                    const int iw = ow * sw - pw + kw * dw;
                    if (iw < 0 || iw >= W) continue;
                    acc = fmaf(to_f32(xg[((int64_t)ci * H + ih) * W + iw]),
                               to_f32(wo[(ci * KH + kh) * KW + kw]), acc);
                }
            }
        }
        y[i] = from_f32<T>(acc);
    }
}

struct TiledGeom {
    int C, H, W, Cout, KH, KW, Cg, Ng, OH, OW;
    int sh, sw, ph, pw, dh, dw;
    int TW, TH;          // output tile (TW * TH == kThreads)
    int IHt, IWt;        // input halo tile
    int CC;              // input channels staged per chunk
    int tiles_w, tiles_h, ochunks, groups;
};

// NB: output channels per workgroup (accumulators per thread).
template <typename T, int NB>
__global__ void __launch_bounds__(kThreads)
direct2d_tiled(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
               T *__restrict__ y, TiledGeom g)
{
    extern __shared__ float lds[];
    float *xs = lds;                                  // [CC][IHt][IWt]
    float *ws = lds + g.CC * g.IHt * g.IWt;           // [NB][CC][KH*KW]
    const int KT = g.KH * g.KW;

    // Unpack the flat block index: (n, group k, output-channel chunk, tile row, tile col).
    int64_t b = blockIdx.x;
    const int tw_i = (int)(b % g.tiles_w); b /= g.tiles_w;
    const int th_i = (int)(b % g.tiles_h); b /= g.tiles_h;
    const int oc_i = (int)(b % g.ochunks); b /= g.ochunks;
    const int k = (int)(b % g.groups);
    const int64_t n = b / g.groups;

    const int tx = threadIdx.x % g.TW, ty = threadIdx.x / g.TW;
    const int oh0 = th_i * g.TH, ow0 = tw_i * g.TW;
    const int oh = oh0 + ty, ow = ow0 + tx;
    const int o0 = k * g.Ng + oc_i * NB;             // first output channel of this block
    const int nb = min(NB, g.Ng - oc_i * NB);        // channels this block really owns
    const int ih0 = oh0 * g.sh - g.ph, iw0 = ow0 * g.sw - g.pw;

    float acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = (bias && j < nb) ? to_f32(bias[o0 + j]) : 0.0f;

    const T *xg = x + ((int64_t)n * g.C + (int64_t)k * g.Cg) * g.H * g.W;
    const int tile_elems = g.IHt * g.IWt;
    for (int c0 = 0; c0 < g.Cg; c0 += g.CC) {
        const int cc = min(g.CC, g.Cg - c0);
        // Stage the halo tile of channels [c0, c0+cc), zero outside the image.
        for (int e = threadIdx.x; e < cc * tile_elems; e += kThreads) {
            const int ci = e / tile_elems, rem = e % tile_elems;
            const int r = rem / g.IWt, c = rem % g.IWt;
            const int ih = ih0 + r, iw = iw0 + c;
            float v = 0.0f;
            if (ih >= 0 && ih < g.H && iw >= 0 && iw < g.W)
                v = to_f32(xg[((int64_t)(c0 + ci) * g.H + ih) * g.W + iw]);
            xs[e] = v;
        }
        // Stage the filters of the block's output channels for these input channels.
        for (int e = threadIdx.x; e < NB * cc * KT; e += kThreads) {
            const int j = e / (cc * KT), rem = e % (cc * KT);
            float v = 0.0f;
            if (j < nb) v = to_f32(w[((int64_t)(o0 + j) * g.Cg + c0) * KT + rem]);
            ws[(j * g.CC) * KT + rem] = v;
        }
        __syncthreads();
        if (ty < g.TH) {
            for (int ci = 0; ci < cc; ++ci) {
                const float *xc = xs + ci * tile_elems + (ty * g.sh) * g.IWt + tx * g.sw;
                const float *wc = ws + ci * KT;
                for (int kh = 0; kh < g.KH; ++kh) {
                    for (int kw = 0; kw < g.KW; ++kw) {
                        const float xv = xc[kh * g.dh * g.IWt + kw * g.dw];
                        const int t = kh * g.KW + kw;
#pragma unroll
                        for (int j = 0; j < NB; ++j) acc[j] = fmaf(xv, wc[j * g.CC * KT + t], acc[j]);
                    }
                }
            }
        }
        __syncthreads();
    }
    if (oh < g.OH && ow < g.OW) {
        T *yp = y + (((int64_t)n * g.Cout + o0) * g.OH + oh) * g.OW + ow;
#pragma unroll
        for (int j = 0; j < NB; ++j)
            if (j < nb) yp[(int64_t)j * g.OH * g.OW] = from_f32<T>(acc[j]);
    }
}

template <typename T, int NB>
hipError_t run_tiled(const Conv2dArgs &a, const TiledGeom &g, size_t lds, int64_t blocks)
{
    hipLaunchKernelGGL((direct2d_tiled<T, NB>), dim3((unsigned)blocks), dim3(kThreads), lds, a.stream,
                       (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, g);
    return hipGetLastError();
}

template <typename T>
hipError_t run_typed(const Conv2dArgs &a, const char **kname)
{
    const int Cg = (int)(a.C / a.groups), Ng = (int)(a.Cout / a.groups);
    TiledGeom g;
    g.C = (int)a.C; g.H = (int)a.H; g.W = (int)a.W; g.Cout = (int)a.Cout;
    g.KH = (int)a.KH; g.KW = (int)a.KW; g.Cg = Cg; g.Ng = Ng; g.OH = (int)a.OH; g.OW = (int)a.OW;
    g.sh = a.sh; g.sw = a.sw; g.ph = a.ph; g.pw = a.pw; g.dh = a.dh; g.dw = a.dw;
    g.TW = a.OW <= 8 ? 8 : a.OW <= 16 ? 16 : a.OW <= 32 ? 32 : 64;
    g.TH = kThreads / g.TW;
    g.IHt = (g.TH - 1) * g.sh + (g.KH - 1) * g.dh + 1;
    g.IWt = (g.TW - 1) * g.sw + (g.KW - 1) * g.dw + 1;
    const int NB = Ng >= 8 ? 8 : Ng >= 4 ? 4 : Ng >= 2 ? 2 : 1;
    const int64_t KT = g.KH * g.KW;
    const int64_t per_chunk = (int64_t)g.IHt * g.IWt + NB * KT;  // floats per staged channel
    int64_t cc = kLdsBudget / (int64_t)sizeof(float) / per_chunk;
    const int64_t tiled_blocks = a.N * a.groups * ceil_div(Ng, NB) * ceil_div(a.OH, g.TH) *
                                 ceil_div(a.OW, g.TW);
    const bool fits = cc >= 1 && tiled_blocks < (int64_t(1) << 31);
    if (!fits) {
        const int64_t total = a.N * a.Cout * a.OH * a.OW;
        const int64_t blocks = std::min<int64_t>(ceil_div(total, kThreads), 1 << 20);
        *kname = "direct2d_naive";
        hipLaunchKernelGGL((direct2d_naive<T>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                           (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, total,
                           (int)a.C, (int)a.H, (int)a.W, (int)a.Cout, (int)a.KH, (int)a.KW, Cg, Ng,
                           (int)a.OH, (int)a.OW, a.sh, a.sw, a.ph, a.pw, a.dh, a.dw);
        return hipGetLastError();
    }
    g.CC = (int)std::min<int64_t>(cc, Cg);
    g.tiles_w = (int)ceil_div(a.OW, g.TW);
    g.tiles_h = (int)ceil_div(a.OH, g.TH);
    g.ochunks = (int)ceil_div(Ng, NB);
    g.groups = (int)a.groups;
    const size_t lds = (size_t)g.CC * per_chunk * sizeof(float);
    const int64_t blocks = a.N * a.groups * g.ochunks * g.tiles_h * g.tiles_w;
    *kname = "direct2d_tiled";
    switch (NB) {
    case 8: return run_tiled<T, 8>(a, g, lds, blocks);
    case 4: return run_tiled<T, 4>(a, g, lds, blocks);
    case 2: return run_tiled<T, 2>(a, g, lds, blocks);
    default: return run_tiled<T, 1>(a, g, lds, blocks);
    }
}

}  // namespace

hipError_t launch_direct2d(const Conv2dArgs &a, const char **kname)
{
    switch (a.dtype) {
    case DT_F32: return run_typed<float>(a, kname);
    case DT_F16: return run_typed<_Float16>(a, kname);
    default: return run_typed<__bf16>(a, kname);
    }
}

}  // namespace gconv
