// direct2d.hip -- direct grouped conv2d (NCHW): two kernels on the vector ALUs and
// one, for 4-in / 4-out groups, on the 4x4x4 matrix-core instructions.
//
// Direct route.  The group index is folded into the launch grid instead of one
// launch per group: the neon issue "Grouped convolutions" proposes offsetting
// the input and output pointers by blockIdx * group stride (ibmua's reply), and
// its replies note that launching one kernel per group costs a fixed overhead
// per launch that swamps small layers.
//
// Three kernels:
//  * direct2d_tiled: one workgroup = (image n, group k, block of NB output
//    channels, TH x TW output tile).  The group's input channels are staged
//    chunk by chunk into LDS as a zero-filled halo tile (coalesced loads along
//    W), the NB x chunk x KH x KW filters next to them, and every thread keeps
//    NB fp32 accumulators for one output position.
//  * direct2d_naive: one thread per output, everything read from global memory.
//    Used only when a halo tile of one channel does not fit in LDS (huge
//    dilation or kernel).
//  * direct2d_g4: fully grouped 3x3 layers with 4 input and 4 output channels
//    per group (the ResNeXt-style cardinality the neon issue discusses), 16-bit
//    types, stride 1, dilation 1, padding 0 or 1.  One wave per (image, group)
//    slab: the slab's 4 channels go to LDS as a zero-bordered [row][col][4]
//    image (one 8-byte entry per position), and each tap is one 4x4x4 MFMA per
//    64 positions (16 blocks of 4 positions: the group's 4x4 filter matrix times
//    the 4 channels of each position), fp32 accumulation.
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
               int Cg, int Ng, int OH, int OW, int sh, int sw, int ph, int pw, int dh, int dw,
               int interleaved)
{
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kThreads) {
        int64_t r = i;
        const int ow = (int)(r % OW); r /= OW;
        const int oh = (int)(r % OH); r /= OH;
        const int oc = (int)(r % Cout);   // output channel; o is its filter
        const int64_t n = r / Cout;
        const int G = Cout / Ng;
        const int o = interleaved ? (oc % G) * Ng + oc / G : oc;
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
    int ocs, okg;        // output channel of filter j of group k: j*ocs + k*okg
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
        T *yp = y + (((int64_t)n * g.Cout + oc_i * NB * g.ocs + k * g.okg) * g.OH + oh) * g.OW + ow;
#pragma unroll
        for (int j = 0; j < NB; ++j)
            if (j < nb) yp[(int64_t)j * g.ocs * g.OH * g.OW] = from_f32<T>(acc[j]);
    }
}

template <typename T, int NB>
hipError_t run_tiled(const Conv2dArgs &a, const TiledGeom &g, size_t lds, int64_t blocks)
{
    hipLaunchKernelGGL((direct2d_tiled<T, NB>), dim3((unsigned)blocks), dim3(kThreads), lds, a.stream,
                       (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, g);
    return hipGetLastError();
}

typedef _Float16 g4_f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 g4_bf16x4 __attribute__((ext_vector_type(4)));
typedef float g4_f32x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_4x4x4_16b_{f16,bf16}: 16 independent 4x4x4 products per wave.  Block b
// is lanes 4b..4b+3; lane m holds row m%4 of its block's A (4 k values), lane l
// holds column l%4 of B (4 k values) and column l%4 of D (4 rows).
template <typename T> struct Mfma4;
template <> struct Mfma4<_Float16> {
    static __device__ __forceinline__ g4_f32x4 run(uint2 a, uint2 b, g4_f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(g4_f16x4, a), __builtin_bit_cast(g4_f16x4, b),
                                                 c, 0, 0, 0);
    }
};
template <> struct Mfma4<__bf16> {
    static __device__ __forceinline__ g4_f32x4 run(uint2 a, uint2 b, g4_f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(g4_bf16x4, a),
                                                     __builtin_bit_cast(g4_bf16x4, b), c, 0, 0, 0);
    }
};
template <typename T> __device__ __forceinline__ uint32_t bits16(T v) { return __builtin_bit_cast(uint16_t, v); }
// Two fp32 values rounded to T and packed (a low), one paired conversion.
typedef _Float16 g4_f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 g4_bf16x2 __attribute__((ext_vector_type(2)));
template <typename T> __device__ __forceinline__ uint32_t g4_pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t g4_pack2<_Float16>(float a, float b)
{
    return __builtin_bit_cast(uint32_t, g4_f16x2{(_Float16)a, (_Float16)b});
}
template <> __device__ __forceinline__ uint32_t g4_pack2<__bf16>(float a, float b)
{
    return __builtin_bit_cast(uint32_t, g4_bf16x2{(__bf16)a, (__bf16)b});
}

constexpr int kG4Waves = kThreads / 64;
constexpr int kG4MaxPos = 1024;   // positions of one padded slab image
constexpr int kG4Filters = 36;    // LDS entries of a group's filters: [tap][output][4 inputs]
constexpr int kG4Step = 62;       // output anchors per pass: lanes 62 and 63 only supply shifted operands

// q / d for 0 <= q < 2048 and 1 <= d <= 400 as (q * m) >> 20 with m = ceil(2^20 / d):
// exact on that range (checked exhaustively on the host side of the tests).  Both
// factors are below 2^24 and the product below 2^31, so the full-rate 24-bit
// multiply gives it exactly.
__device__ __forceinline__ int g4_div(int q, uint32_t m) { return (int)(__umul24((uint32_t)q, m) >> 20); }
// a * b for 0 <= a, b < 2^24 with a product below 2^31 (image positions and sizes).
__device__ __forceinline__ int g4_mul(int a, int b) { return (int)__umul24((uint32_t)a, (uint32_t)b); }

// The value lane + 1 holds (lane 63 receives zero; its result is not used).  A DPP
// move with no old value, so the compiler need not copy the source first.
__device__ __forceinline__ uint2 g4_next_lane(uint2 v)
{
    return make_uint2((uint32_t)__builtin_amdgcn_mov_dpp((int)v.x, 0x130, 0xf, 0xf, true),
                      (uint32_t)__builtin_amdgcn_mov_dpp((int)v.y, 0x130, 0xf, 0xf, true));
}
constexpr int kG4NT = 2;   // buffer-store cache policy: non-temporal

// LDS entries (8 bytes each) of one wave's slab: the padded image and the entries
// past it that the last pass's lanes may read, the filters, and the staged outputs.
struct G4Lds {
    int img, total;
};
__host__ __device__ inline G4Lds g4_lds(int HP, int WP, int OH, int OW)
{
    const int na = (OH - 1) * WP + OW;                           // anchors up to the last output
    const int npass = (na + kG4Step - 1) / kG4Step;
    const int reach = kG4Step * (npass - 1) + 64 + 2 * WP + 2;   // entries any lane of any pass reads
    const int img = ((HP * WP > reach ? HP * WP : reach) + 1) & ~1;   // even: the outputs' entries pair up 16-byte aligned
    return G4Lds{img, img + kG4Filters + OH * OW};
}

// One wave per (image, group) slab.  The slab's 4 channels go to LDS as a
// zero-bordered image of 8-byte entries (4 channels of a position), written in one
// pass: the image positions from the loaded pairs, the border positions as zeros.
// Output positions are anchors a = oh * WP + ow of the padded image (the window's
// top-left entry); tap (kh, kw) of anchor a reads entry a + kh*WP + kw.  Per pass
// and filter row, two 8-byte LDS reads give each lane its kw = 0 and kw = 2
// operands and the kw = 1 operand is the next lane's kw = 0 value (a whole-wave DPP
// shift by one lane), so a pass of 62 anchors takes 6 reads instead of 9.  Each tap is
// one 4x4x4 MFMA for the 16 blocks of 4 anchors: A = the group's 4 x 4 filter
// matrix at that tap, B = the 4 input channels of each anchor, D = the 4 outputs
// of the lane's anchor, fp32 accumulation.
template <typename T>
__global__ void __launch_bounds__(kThreads)
direct2d_g4(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
            T *__restrict__ y, int G, int H, int W, int OH, int OW, int ph, int pw, int slabs,
            uint32_t mw, uint32_t mwp, int ocs, int okg, int ystage)
{
    extern __shared__ __attribute__((aligned(16))) uint2 g4s[];
    const int HP = H + 2 * ph, WP = W + 2 * pw;
    const G4Lds L = g4_lds(HP, WP, OH, OW);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int slab = blockIdx.x * kG4Waves + wave;
    if (slab >= slabs) return;   // whole wave; this kernel has no workgroup barrier
    uint2 *xs = g4s + wave * L.total;
    uint2 *fs = xs + L.img;
    uint2 *ys = fs + kG4Filters;   // [OH*OW][4 outputs] staged outputs
    const int HW = H * W, C = 4 * G, OHW = OH * OW;
    const int n = slab / G, k = slab - n * G;
    auto wave_sync = [&]() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // Every global load of the wave is issued before the first is used: the 4
    // channels of this lane's position pairs (one 32-bit load per channel and
    // pair; H*W is even), its share of the group's 144 filter values, and the 4
    // biases.
    constexpr int kMaxL = kG4MaxPos / 128;
    const T *xg = x + ((int64_t)n * C + 4 * k) * HW;
    const T *wg = w + (int64_t)(4 * k) * 36;   // [output o][input c][tap t]
    const int npair = HW / 2;
    // The slab's 4 channels as one buffer: a lane's pair offset is shared by the 4
    // loads, the channel offset is a scalar.
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(xg), (short)0, 8 * HW, 0x00020000);
    uint32_t xv[kMaxL][4];
#pragma unroll
    for (int j = 0; j < kMaxL; ++j) {
        if (64 * j < npair) {   // uniform; the pair index is clamped, not branched on
            const int q = min(lane + 64 * j, npair - 1);
#pragma unroll
            for (int c = 0; c < 4; ++c) xv[j][c] = __builtin_amdgcn_raw_buffer_load_b32(xr, 4 * q, 2 * c * HW, 0);
        }
    }
    // The group's 144 filter values: lane L < 16 takes output L / 4 and input L % 4,
    // whose 9 taps are the 9 consecutive values at 9 L (the other lanes load lane
    // 15's and write nothing).
    uint16_t wv[9];
    const T *wl = wg + 9 * min(lane, 15);
#pragma unroll
    for (int t = 0; t < 9; ++t) wv[t] = (uint16_t)bits16(wl[t]);
    const T *bp = bias ? bias + 4 * k : wg;   // loaded either way; zero when there is no bias
    T braw[4];
#pragma unroll
    for (int o = 0; o < 4; ++o) braw[o] = bp[o];
    __builtin_amdgcn_sched_barrier(0);   // keep every load ahead of the first use

    // The padded image: border positions zero (with padding 0 or 1: the top and
    // bottom rows, 2*ph*WP entries, then the left and right columns of the H image
    // rows, 2*pw*H entries), image positions from the pairs.
    const int nborder = HP * WP - HW;
    for (int i = lane; i < nborder; i += 64) {
        int hp, wp;
        if (i < 2 * ph * WP) {
            const bool bottom = i >= WP;
            hp = bottom ? HP - 1 : 0;
            wp = bottom ? i - WP : i;
        } else {
            const int j = i - 2 * ph * WP;
            hp = ph + (j >> 1);
            wp = (j & 1) ? WP - 1 : 0;
        }
        xs[g4_mul(hp, WP) + wp] = make_uint2(0, 0);
    }
    // Half e of each channel's pair: channels (0,1) and (2,3) side by side.
    auto entry = [&](int j, int e) {
        const uint32_t sel = e ? 0x07060302u : 0x05040100u;
        return make_uint2(__builtin_amdgcn_perm(xv[j][1], xv[j][0], sel), __builtin_amdgcn_perm(xv[j][3], xv[j][2], sel));
    };
    const bool w_even = (W & 1) == 0;   // a pair's two positions then share a row
#pragma unroll
    for (int j = 0; j < kMaxL; ++j) {
        const int q = lane + 64 * j;
        if (64 * j < npair && q < npair) {
            if (w_even) {
                const int h = g4_div(2 * q, mw), ww = 2 * q - g4_mul(h, W);
                uint2 *d = xs + g4_mul(h + ph, WP) + ww + pw;
                d[0] = entry(j, 0);
                d[1] = entry(j, 1);
            } else {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int p = 2 * q + e;
                    const int h = g4_div(p, mw), ww = p - g4_mul(h, W);
                    xs[g4_mul(h + ph, WP) + ww + pw] = entry(j, e);
                }
            }
        }
    }
    // Filter entry (t, o) holds output o's 4 inputs at tap t: value (o, c, t) at
    // halfword 16 t + 4 o + c, i.e. 16 t + L for lane L.
    uint16_t *fs16 = reinterpret_cast<uint16_t *>(fs);
    if (lane < 16) {
#pragma unroll
        for (int t = 0; t < 9; ++t) fs16[16 * t + lane] = wv[t];
    }
    wave_sync();

    uint2 fa[9];
#pragma unroll
    for (int t = 0; t < 9; ++t) fa[t] = fs[t * 4 + (lane & 3)];

    g4_f32x4 b0;
#pragma unroll
    for (int o = 0; o < 4; ++o) b0[o] = bias ? to_f32(braw[o]) : 0.0f;
    const int na = (OH - 1) * WP + OW;
    T *yg = y + ((int64_t)n * C + k * okg) * OHW;   // filter o of the group: channel o*ocs + k*okg
    for (int a0 = 0; a0 < na; a0 += kG4Step) {
        const int a = a0 + lane;
        g4_f32x4 acc = b0;
#pragma unroll
        for (int kh = 0; kh < 3; ++kh) {
            const uint2 v0 = xs[a + kh * WP];
            const uint2 v2 = xs[a + kh * WP + 2];   // inside the image area for every lane (g4_lds)
            const uint2 v1 = g4_next_lane(v0);
            acc = Mfma4<T>::run(fa[kh * 3 + 0], v0, acc);
            acc = Mfma4<T>::run(fa[kh * 3 + 1], v1, acc);
            acc = Mfma4<T>::run(fa[kh * 3 + 2], v2, acc);
        }
        const int oh = g4_div(a, mwp), ow = a - g4_mul(oh, WP);
        if (lane < kG4Step && a < na && ow < OW) {
            const int p = g4_mul(oh, OW) + ow;
            if (ystage) {
                ys[p] = make_uint2(g4_pack2<T>(acc[0], acc[1]), g4_pack2<T>(acc[2], acc[3]));
            } else {
#pragma unroll
                for (int o = 0; o < 4; ++o) store_nt(yg + (int64_t)o * ocs * OHW + p, from_f32<T>(acc[o]));
            }
        }
    }
    if (ystage) {
        // The group's 4 output planes are one contiguous, 8-byte aligned run of y
        // (OH*OW a multiple of 4): each lane takes 4 consecutive positions (LDS
        // entries of 4 outputs) and writes one 8-byte piece per output plane (2-byte
        // stores would reach HBM as partial lines, the stores being non-temporal).
        wave_sync();
        // The group's 4 output planes as one buffer: the lane's piece offset is shared
        // by the 4 stores, the plane offset is a scalar.
        const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(yg, (short)0, 8 * OHW, 0x00020000);
        for (int i = lane; 4 * i < OHW; i += 64) {
            const uint4 pa = *reinterpret_cast<const uint4 *>(ys + 4 * i);       // positions 4i, 4i+1
            const uint4 pb = *reinterpret_cast<const uint4 *>(ys + 4 * i + 2);   // positions 4i+2, 4i+3
            // output o of a position: the low (o even) or high half of dword o / 2 of its entry
            const uint32_t lo = 0x05040100u, hi = 0x07060302u;
            auto put = [&](int o, uint32_t a, uint32_t b) {
                __builtin_amdgcn_raw_buffer_store_b64(gconv_u32x2{a, b}, yr, 8 * i, 2 * o * OHW, kG4NT);
            };
            put(0, __builtin_amdgcn_perm(pa.z, pa.x, lo), __builtin_amdgcn_perm(pb.z, pb.x, lo));
            put(1, __builtin_amdgcn_perm(pa.z, pa.x, hi), __builtin_amdgcn_perm(pb.z, pb.x, hi));
            put(2, __builtin_amdgcn_perm(pa.w, pa.y, lo), __builtin_amdgcn_perm(pb.w, pb.y, lo));
            put(3, __builtin_amdgcn_perm(pa.w, pa.y, hi), __builtin_amdgcn_perm(pb.w, pb.y, hi));
        }
    }
}

template <typename T>
bool g4_applies(const Conv2dArgs &a)
{
    if constexpr (sizeof(T) != 2) {
        return false;
    } else {
        const int64_t Cg = a.C / a.groups, Ng = a.Cout / a.groups;
        if (!(Cg == 4 && Ng == 4 && a.KH == 3 && a.KW == 3 && a.sh == 1 && a.sw == 1 && a.dh == 1 && a.dw == 1 &&
              a.ph <= 1 && a.pw <= 1 && (a.H + 2 * a.ph) * (a.W + 2 * a.pw) <= kG4MaxPos && a.W <= 339 &&
              (a.H * a.W) % 2 == 0 && (reinterpret_cast<uintptr_t>(a.x) & 3) == 0 &&
              a.N * a.groups < (int64_t(1) << 30)))
            return false;
        // image, filters and staged outputs of 4 waves within 64 KB of LDS
        const G4Lds L = g4_lds((int)(a.H + 2 * a.ph), (int)(a.W + 2 * a.pw), (int)a.OH, (int)a.OW);
        return (int64_t)kG4Waves * L.total * 8 <= 64 * 1024;
    }
}

template <typename T>
hipError_t run_typed(const Conv2dArgs &a, const char **kname)
{
    if constexpr (sizeof(T) == 2) {
        if (!g4_applies<T>(a)) goto tiled;
        const int slabs = (int)(a.N * a.groups);
        const G4Lds L = g4_lds((int)(a.H + 2 * a.ph), (int)(a.W + 2 * a.pw), (int)a.OH, (int)a.OW);
        const size_t lds = (size_t)kG4Waves * L.total * sizeof(uint2);
        const int WP = (int)(a.W + 2 * a.pw);
        *kname = "direct2d_g4";
        hipLaunchKernelGGL((direct2d_g4<T>), dim3((unsigned)ceil_div(slabs, kG4Waves)), dim3(kThreads), lds,
                           a.stream, (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y,
                           (int)a.groups, (int)a.H, (int)a.W, (int)a.OH, (int)a.OW, a.ph, a.pw, slabs,
                           (uint32_t)(((1u << 20) + a.W - 1) / a.W), (uint32_t)(((1u << 20) + WP - 1) / WP),
                           a.interleaved ? (int)a.groups : 1, a.interleaved ? 1 : 4,
                           (!a.interleaved && (reinterpret_cast<uintptr_t>(a.y) & 7) == 0 &&
                            (a.OH * a.OW) % 4 == 0) ? 1 : 0);
        return hipGetLastError();
    }
tiled:
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
                           (int)a.OH, (int)a.OW, a.sh, a.sw, a.ph, a.pw, a.dh, a.dw, a.interleaved);
        return hipGetLastError();
    }
    g.CC = (int)std::min<int64_t>(cc, Cg);
    g.tiles_w = (int)ceil_div(a.OW, g.TW);
    g.tiles_h = (int)ceil_div(a.OH, g.TH);
    g.ochunks = (int)ceil_div(Ng, NB);
    g.groups = (int)a.groups;
    g.ocs = a.interleaved ? (int)a.groups : 1;
    g.okg = a.interleaved ? 1 : Ng;
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
