// igemm.hip -- implicit-GEMM grouped conv2d (NCHW) on the gfx950 matrix cores.
//
// Per group k the convolution is the product
//     Y_k[o][m] = sum_kk W_k[o][kk] * A_k[kk][m],   kk = (tap, input channel),
// where m runs over the output positions (n, oh, ow) and A_k is the im2col
// matrix of the group's input channels.  The neon issue "Grouped convolutions"
// discusses im2col as a lowering and notes that explicit im2col is wasteful; here
// A_k is never written to memory: each input-channel chunk of a tile is staged
// once into LDS as a zero-padded halo of whole input rows, and the MFMA operands
// for every tap are read straight out of that halo.  The discuss.pytorch.org
// thread "F.conv2d runs x15 slower in mixed-precision/half-precision mode"
// traces the slow fp16 grouped conv to grouped convs not reaching the tensor
// cores; this route puts every group's contraction on the matrix cores.
//
// Tile: one workgroup = 4 waves computes BN = WN*32 output channels of one
// group x BM = 4*WM*32 consecutive output positions (flattened over n, oh, ow,
// so a tile may span image boundaries).  Wave w owns positions
// [w*WM*32, (w+1)*WM*32) of the tile and all BN channels: WN x WM blocks of
// v_mfma_f32_32x32x16_{f16,bf16}, the filters as the A operand (rows = output
// channels) and the im2col tile as the B operand (columns = positions), so the
// accumulator columns are positions and stores run along W.
//
// K loop: input channels in chunks of 16, then taps; one MFMA step = one tap x
// 16 channels.  LDS layouts keep the 16 channels of one (row, col) or one
// (tap, filter) contiguous (32 bytes), so an MFMA fragment (8 consecutive
// channels for one lane) is a single 16-byte LDS read; the two 16-byte halves
// are swapped on every other group of 4 slots so that 8 consecutive lanes hit
// distinct banks.
#include <algorithm>

#include "common.hpp"

namespace gconv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kCK = 16;            // input channels per K chunk
constexpr int kMaxSlotsPerThread = 8;
constexpr int kLdsBudget = 72 * 1024;

template <typename T> struct Mfma;
template <> struct Mfma<_Float16> {
    static __device__ __forceinline__ f32x16 run(uint4 a, uint4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <> struct Mfma<__bf16> {
    static __device__ __forceinline__ f32x16 run(uint4 a, uint4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

struct IgemmGeom {
    int N, C, H, W, Cout, Cg, Ng, OH, OW, KH, KW;
    int sh, sw, ph, pw, dh, dw;
    int Hp;              // H + 2*ph: height of one zero-padded image in the virtual row space
    int NR, WL;          // LDS halo: rows, columns (padded coordinates)
    int64_t P;           // N*OH*OW output positions
    int m_tiles, n_tiles, groups;
    int w_vec;           // 1: filter rows can be read with 16-byte loads
};

// Half-swap of the 32-byte slot `s`: selects which 16-byte half holds channels 0-7.
__device__ __forceinline__ int swz(int s, int half) { return half ^ ((s >> 2) & 1); }

template <typename T, int WN, int WM, int KT>
__global__ void __launch_bounds__(kThreads)
igemm_fwd(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
          T *__restrict__ y, IgemmGeom g)
{
    constexpr int BN = WN * 32;
    constexpr int BM = 4 * WM * 32;
    extern __shared__ uint4 lds[];
    uint4 *xs = lds;                          // [NR*WL][2]
    uint4 *ws = lds + g.NR * g.WL * 2;        // [KT][BN][2]

    int bid = blockIdx.x;
    const int mt = bid % g.m_tiles; bid /= g.m_tiles;
    const int nt = bid % g.n_tiles;
    const int k = bid / g.n_tiles;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int OHW = g.OH * g.OW;
    const int64_t HW = (int64_t)g.H * g.W;
    const int kt_rt = KT > 0 ? KT : g.KH * g.KW;

    // First virtual padded input row the tile needs.
    const int64_t p0 = (int64_t)mt * BM;
    const int64_t n_first = p0 / OHW;
    const int oh_first = (int)(p0 % OHW) / g.OW;
    const int64_t R_lo = n_first * g.Hp + (int64_t)oh_first * g.sh;

    // LDS slot of tap (0,0) for each of this lane's output positions.
    int xslot[WM];
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) {
        int64_t p = p0 + wave * WM * 32 + mb * 32 + l32;
        if (p >= g.P) p = g.P - 1;
        const int64_t n = p / OHW;
        const int q = (int)(p % OHW);
        const int oh = q / g.OW, ow = q % g.OW;
        xslot[mb] = (int)(n * g.Hp + (int64_t)oh * g.sh - R_lo) * g.WL + ow * g.sw;
    }

    // Global offsets (channel 0 of the group) of the halo slots this thread stages; -1 = zero.
    const int nslots = g.NR * g.WL;
    int64_t soff[kMaxSlotsPerThread];
#pragma unroll
    for (int i = 0; i < kMaxSlotsPerThread; ++i) {
        const int s = tid + i * kThreads;
        soff[i] = -1;
        if (s < nslots) {
            const int rr = s / g.WL, cc = s % g.WL;
            const int64_t R = R_lo + rr;
            const int64_t n = R / g.Hp;
            const int ih = (int)(R % g.Hp) - g.ph;
            const int iw = cc - g.pw;
            if (n < g.N && ih >= 0 && ih < g.H && iw >= 0 && iw < g.W)
                soff[i] = ((n * g.C + (int64_t)k * g.Cg) * g.H + ih) * g.W + iw;
        }
    }

    const uint16_t *xh = reinterpret_cast<const uint16_t *>(x);
    const uint16_t *wh = reinterpret_cast<const uint16_t *>(w);

    f32x16 acc[WN][WM];
#pragma unroll
    for (int i = 0; i < WN; ++i)
#pragma unroll
        for (int j = 0; j < WM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    for (int ci0 = 0; ci0 < g.Cg; ci0 += kCK) {
        __syncthreads();  // the previous chunk's operands are no longer read
        // ---- stage the input halo: 16 channels per slot, two 16-byte halves
#pragma unroll
        for (int i = 0; i < kMaxSlotsPerThread; ++i) {
            const int s = tid + i * kThreads;
            if (s < nslots) {
                uint32_t v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    uint32_t lo = 0, hi = 0;
                    const int c = ci0 + 2 * j;
                    if (soff[i] >= 0) {
                        if (c < g.Cg) lo = xh[soff[i] + (int64_t)c * HW];
                        if (c + 1 < g.Cg) hi = xh[soff[i] + (int64_t)(c + 1) * HW];
                    }
                    v[j] = lo | (hi << 16);
                }
                xs[s * 2 + swz(s, 0)] = make_uint4(v[0], v[1], v[2], v[3]);
                xs[s * 2 + swz(s, 1)] = make_uint4(v[4], v[5], v[6], v[7]);
            }
        }
        // ---- stage the filters: [tap][filter][16 channels]
        for (int task = tid; task < BN * 2; task += kThreads) {
            const int nn = task >> 1, o = task & 1;
            const int on = nt * BN + nn;
            const int cb = ci0 + 8 * o;
            const bool valid = on < g.Ng;
            const int64_t wrow = ((int64_t)(k * g.Ng + on) * g.Cg + cb) * kt_rt;
            if constexpr (KT > 0) {
                // 8 channels x KT taps of one filter row, as 4*KT packed 16-bit pairs.
                uint32_t d[4 * KT];
                if (valid && g.w_vec && cb + 8 <= g.Cg) {
                    const uint4 *src = reinterpret_cast<const uint4 *>(wh + wrow);
#pragma unroll
                    for (int q = 0; q < KT; ++q) {
                        const uint4 u = src[q];
                        d[4 * q + 0] = u.x; d[4 * q + 1] = u.y; d[4 * q + 2] = u.z; d[4 * q + 3] = u.w;
                    }
                } else {
#pragma unroll
                    for (int e2 = 0; e2 < 4 * KT; ++e2) {
                        uint32_t lo = 0, hi = 0;
                        const int e = 2 * e2;
                        if (valid && cb + e / KT < g.Cg) lo = wh[wrow + e];
                        if (valid && cb + (e + 1) / KT < g.Cg) hi = wh[wrow + e + 1];
                        d[e2] = lo | (hi << 16);
                    }
                }
#pragma unroll
                for (int t = 0; t < KT; ++t) {
                    uint32_t v[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int e0 = (2 * j) * KT + t, e1 = (2 * j + 1) * KT + t;
                        const uint32_t lo = (d[e0 >> 1] >> (16 * (e0 & 1))) & 0xffffu;
                        const uint32_t hi = (d[e1 >> 1] >> (16 * (e1 & 1))) & 0xffffu;
                        v[j] = lo | (hi << 16);
                    }
                    ws[(t * BN + nn) * 2 + swz(nn, o)] = make_uint4(v[0], v[1], v[2], v[3]);
                }
            } else {
                for (int t = 0; t < kt_rt; ++t) {
                    uint32_t v[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        uint32_t lo = 0, hi = 0;
                        if (valid && cb + 2 * j < g.Cg) lo = wh[wrow + (2 * j) * kt_rt + t];
                        if (valid && cb + 2 * j + 1 < g.Cg) hi = wh[wrow + (2 * j + 1) * kt_rt + t];
                        v[j] = lo | (hi << 16);
                    }
                    ws[(t * BN + nn) * 2 + swz(nn, o)] = make_uint4(v[0], v[1], v[2], v[3]);
                }
            }
        }
        __syncthreads();
        // ---- MFMA over the taps of this chunk
        for (int t = 0; t < kt_rt; ++t) {
            const int kh = t / g.KW, kw = t % g.KW;
            const int xoff = kh * g.dh * g.WL + kw * g.dw;
            uint4 bf[WM], af[WN];
#pragma unroll
            for (int mb = 0; mb < WM; ++mb) {
                const int s = xslot[mb] + xoff;
                bf[mb] = xs[s * 2 + swz(s, half)];
            }
#pragma unroll
            for (int nb = 0; nb < WN; ++nb) {
                const int nn = nb * 32 + l32;
                af[nb] = ws[(t * BN + nn) * 2 + swz(nn, half)];
            }
#pragma unroll
            for (int nb = 0; nb < WN; ++nb)
#pragma unroll
                for (int mb = 0; mb < WM; ++mb) acc[nb][mb] = Mfma<T>::run(af[nb], bf[mb], acc[nb][mb]);
        }
    }

    // ---- epilogue: + bias in fp32, one rounding to T, stores along the positions
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) {
        const int64_t p = p0 + wave * WM * 32 + mb * 32 + l32;
        if (p >= g.P) continue;
        const int64_t n = p / OHW;
        const int q = (int)(p % OHW);
        T *yp = y + n * g.Cout * (int64_t)OHW + q;
#pragma unroll
        for (int nb = 0; nb < WN; ++nb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int on = nt * BN + nb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                if (on < g.Ng) {
                    const int co = k * g.Ng + on;
                    float v = acc[nb][mb][r];
                    if (bias) v += to_f32(bias[co]);
                    yp[(int64_t)co * OHW] = from_f32<T>(v);
                }
            }
        }
    }
}

struct Plan {
    IgemmGeom g;
    int WN, WM;
    size_t lds;
    int64_t blocks;
    bool ok;
};

Plan make_plan(const Conv2dArgs &a)
{
    Plan pl{};
    pl.ok = false;
    if (a.dtype != DT_F16 && a.dtype != DT_BF16) return pl;
    IgemmGeom &g = pl.g;
    g.N = (int)a.N; g.C = (int)a.C; g.H = (int)a.H; g.W = (int)a.W; g.Cout = (int)a.Cout;
    g.Cg = (int)(a.C / a.groups); g.Ng = (int)(a.Cout / a.groups);
    g.OH = (int)a.OH; g.OW = (int)a.OW; g.KH = (int)a.KH; g.KW = (int)a.KW;
    g.sh = a.sh; g.sw = a.sw; g.ph = a.ph; g.pw = a.pw; g.dh = a.dh; g.dw = a.dw;
    g.Hp = g.H + 2 * g.ph;
    g.P = a.N * a.OH * a.OW;
    g.groups = (int)a.groups;
    pl.WN = g.Ng > 64 ? 4 : g.Ng > 32 ? 2 : 1;
    pl.WM = 2;
    const int BN = pl.WN * 32, BM = 4 * pl.WM * 32;
    // Virtual output rows one tile can touch, image boundaries inside them, and
    // the resulting bound on the virtual padded input rows of its halo.
    const int64_t V = (BM % g.OW == 0) ? BM / g.OW : (BM - 1) / g.OW + 2;
    const int64_t crossings = (V <= 1) ? 0 : ((BM % g.OW == 0 && g.OH % (BM / g.OW) == 0) ? 0 : (V - 2) / g.OH + 1);
    const int64_t gap = std::max<int64_t>(0, (int64_t)g.Hp - (int64_t)g.OH * g.sh);
    const int64_t NR = (V - 1) * g.sh + crossings * gap + (int64_t)(g.KH - 1) * g.dh + 1;
    const int64_t WL = (int64_t)(g.OW - 1) * g.sw + (int64_t)(g.KW - 1) * g.dw + 1;
    if (NR * WL > (int64_t)kMaxSlotsPerThread * kThreads) return pl;
    g.NR = (int)NR; g.WL = (int)WL;
    const int64_t KT = a.KH * a.KW;
    pl.lds = (size_t)(NR * WL * 2 + KT * BN * 2) * sizeof(uint4);
    if (pl.lds > (size_t)kLdsBudget) return pl;
    g.m_tiles = (int)ceil_div(g.P, BM);
    g.n_tiles = (int)ceil_div(g.Ng, BN);
    pl.blocks = (int64_t)g.m_tiles * g.n_tiles * g.groups;
    if (pl.blocks >= (int64_t(1) << 31) || g.P >= (int64_t(1) << 31)) return pl;
    g.w_vec = ((g.Cg * KT) % 8 == 0) && ((reinterpret_cast<uintptr_t>(a.w) & 15) == 0);
    pl.ok = true;
    return pl;
}

template <typename T, int WN, int KT>
hipError_t run(const Conv2dArgs &a, const Plan &pl)
{
    hipLaunchKernelGGL((igemm_fwd<T, WN, 2, KT>), dim3((unsigned)pl.blocks), dim3(kThreads), pl.lds,
                       a.stream, (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, pl.g);
    return hipGetLastError();
}

template <typename T, int WN>
hipError_t run_kt(const Conv2dArgs &a, const Plan &pl)
{
    const int64_t KT = a.KH * a.KW;
    if (KT == 9) return run<T, WN, 9>(a, pl);
    if (KT == 1) return run<T, WN, 1>(a, pl);
    return run<T, WN, 0>(a, pl);
}

template <typename T>
hipError_t run_typed(const Conv2dArgs &a, const Plan &pl)
{
    switch (pl.WN) {
    case 4: return run_kt<T, 4>(a, pl);
    case 2: return run_kt<T, 2>(a, pl);
    default: return run_kt<T, 1>(a, pl);
    }
}

}  // namespace

bool igemm_supported(const Conv2dArgs &a) { return make_plan(a).ok; }

hipError_t launch_igemm(const Conv2dArgs &a, const char **kname)
{
    const Plan pl = make_plan(a);
    if (!pl.ok) return hipErrorInvalidValue;
    *kname = "igemm_fwd_mfma32x32x16";
    return a.dtype == DT_F16 ? run_typed<_Float16>(a, pl) : run_typed<__bf16>(a, pl);
}

}  // namespace gconv
