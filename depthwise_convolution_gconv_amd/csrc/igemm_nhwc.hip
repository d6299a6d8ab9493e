// igemm_nhwc.hip -- implicit-GEMM grouped conv2d over channels-last (NHWC) tensors
// on the gfx950 matrix cores (fp16 / bf16 in, fp32 accumulate).
//
// The discuss.pytorch.org thread "F.conv2d runs x15 slower in mixed-precision/
// half-precision mode" turns to the NHWC (channels_last) memory format for the fp16
// grouped conv.  In NHWC the operands of v_mfma_f32_32x32x16 are already in their
// register layout in memory: a fragment lane holds 8 consecutive K values (input
// channels) of one row or column, and 8 consecutive channels of one position of x,
// or of one filter tap of w [Cout][KH][KW][C/g], are one contiguous 16-byte run.
// So this kernel loads its fragments straight from global memory (through L1/L2),
// with no LDS staging and no transposes:
//   Y_k[o][m] = sum over (tap, ci) of W_k[o][tap, ci] * X_k[tap, ci][m],
// K steps of one tap x 16 channels; m = (n, oh, ow) output positions.
// Tile: a workgroup = 4 waves = 256 consecutive positions x 64 filters of one
// group; a wave = 64 positions x 64 filters (2 x 2 blocks of 32 x 32, 64 fp32
// accumulators), fragments of 4 K steps in flight.  Output: each lane holds
// 4 consecutive filters of one position per accumulator quad, stored as 8 bytes
// (the two lane halves of a block write 16 contiguous bytes of y's channel run).
#include <algorithm>

#include "common.hpp"
#include "fastdiv.hpp"

namespace gconv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kPosWave = 64;                  // positions per wave (2 blocks of 32)
constexpr int kPosTile = 4 * kPosWave;        // positions per workgroup
constexpr int kFilTile = 64;                  // filters per workgroup (2 blocks of 32)
constexpr int kDepth = 4;                     // K steps of fragments in flight
constexpr int kRowE = kFilTile + 8;           // staged output row (elements): 144 bytes

template <typename T> struct MfmaN;
template <> struct MfmaN<_Float16> {
    static __device__ __forceinline__ f32x16 run(uint4 a, uint4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <> struct MfmaN<__bf16> {
    static __device__ __forceinline__ f32x16 run(uint4 a, uint4 b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(a)) |
           ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(b)) << 16);
}

struct NhwcGeom {
    int N, C, H, W, Cout, Cg, Ng, OH, OW, KH, KW;
    int sh, sw, ph, pw, dh, dw;
    int P;                   // N*OH*OW
    int m_tiles, n_tiles;    // ceil(P / 256), ceil(Ng / 64)
    int tiles, tiles_per_xcd, groups;
    int ksteps;              // KH*KW*Cg/16
    FastDiv fd_ohw, fd_ow, fd_g, fd_nt, fd_cs;   // fd_cs: Cg/16 (channel steps per tap)
};

template <typename T>
__global__ void __launch_bounds__(kThreads)
igemm_nhwc(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
           T *__restrict__ y, NhwcGeom g)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    // Tile: (position tile mt, filter tile nt, group k), groups fastest: the tiles of
    // all groups of one position range run together, so every 128-byte line of x
    // (64 channels, several groups) is used whole while it is in L2.  Tiles are dealt
    // to the XCDs in contiguous runs (workgroup b runs on XCD b % 8), so neighbouring
    // position ranges, which read the same input rows, share one L2.
    const int xcd = blockIdx.x & 7, rank = blockIdx.x >> 3;
    const int tile = xcd * g.tiles_per_xcd + rank;
    if (tile >= min((xcd + 1) * g.tiles_per_xcd, g.tiles)) return;   // uniform over the workgroup
    const int bq = fdiv(tile, g.fd_g);
    const int k = tile - bq * g.groups;
    const int mt = fdiv(bq, g.fd_nt);
    const int nt = bq - mt * g.n_tiles;
    const int f0 = nt * kFilTile;                       // first filter (within the group)
    const int p0 = mt * kPosTile + wave * kPosWave;     // first position of this wave

    // This lane's rows of the A operand (filters f0 + nb*32 + l32) and columns of
    // the B operand (positions p0 + mb*32 + l32); channels c0 + 8*half of a K step.
    const T *wrow[2];
    bool fok[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int f = f0 + nb * 32 + l32;
        fok[nb] = f < g.Ng;
        wrow[nb] = w + (int64_t)(k * g.Ng + (fok[nb] ? f : 0)) * g.KH * g.KW * g.Cg + 8 * half;
    }
    int pn[2], poh[2], pow_[2];
    bool pok[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int p = p0 + mb * 32 + l32;
        pok[mb] = p < g.P;
        const int pc = pok[mb] ? p : 0;
        pn[mb] = fdiv(pc, g.fd_ohw);
        const int q = pc - pn[mb] * g.OH * g.OW;
        poh[mb] = fdiv(q, g.fd_ow);
        pow_[mb] = q - poh[mb] * g.OW;
    }
    const int cbase = k * g.Cg + 8 * half;               // this lane's channel offset in x

    // Fragments of K step s = (tap, channel step): zero for filters past Ng, for
    // positions past P and for taps in the padding.
    auto load_step = [&](int s, uint4 (&a)[2], uint4 (&b)[2]) {
        const int t = fdiv(s, g.fd_cs);
        const int cs = (s - t * (g.Cg / 16)) * 16;
        const int kh = t / g.KW, kw = t - kh * g.KW;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            a[nb] = make_uint4(0, 0, 0, 0);
            if (fok[nb]) a[nb] = *reinterpret_cast<const uint4 *>(wrow[nb] + t * g.Cg + cs);
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int ih = poh[mb] * g.sh - g.ph + kh * g.dh;
            const int iw = pow_[mb] * g.sw - g.pw + kw * g.dw;
            b[mb] = make_uint4(0, 0, 0, 0);
            if (pok[mb] && ih >= 0 && ih < g.H && iw >= 0 && iw < g.W)
                b[mb] = *reinterpret_cast<const uint4 *>(
                    x + (((int64_t)pn[mb] * g.H + ih) * g.W + iw) * g.C + cbase + cs);
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;

    // A ring of kDepth steps of fragments: step s computes from slot s % kDepth,
    // whose next load (step s + kDepth) is issued right after, so each load has
    // kDepth - 1 steps of MFMAs to arrive.
    uint4 fa[kDepth][2], fb[kDepth][2];
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
        if (d < g.ksteps) load_step(d, fa[d], fb[d]);
    for (int s0 = 0; s0 < g.ksteps; s0 += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int s = s0 + d;
            if (s < g.ksteps) {   // uniform
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = MfmaN<T>::run(fa[d][nb], fb[d][mb], acc[nb][mb]);
                if (s + kDepth < g.ksteps) load_step(s + kDepth, fa[d], fb[d]);
            }
        }
    }

    // Epilogue: accumulator r of block (nb, mb) is filter f0 + nb*32 + (r/4)*8 +
    // 4*half + r%4 at position p0 + mb*32 + l32; bias in fp32, one rounding.  When
    // the tile's 64 filters are one 128-byte run of y per position (Cout/g a multiple
    // of 8, y 16-byte aligned), the wave stages its 64 positions x 64 filters in its own LDS area (rows
    // of kRowE elements, padded against bank conflicts) and stores whole 16-byte
    // pieces, 8 lanes per position: the 8-byte pieces of the accumulator layout, from
    // 8 different store instructions, would reach HBM as partial lines.
    __shared__ uint4 ystage[4 * kPosWave * kRowE / 8];
    T *st = reinterpret_cast<T *>(ystage) + wave * kPosWave * kRowE;
    const bool staged = (g.Ng & 7) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int p = p0 + mb * 32 + l32;
        T *yp = y + (int64_t)p * g.Cout + k * g.Ng;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int fl = nb * 32 + q * 8 + 4 * half;   // first of 4 filters, within the tile
                const int f = f0 + fl;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = acc[nb][mb][q * 4 + e];
                    if (bias && f + e < g.Ng) v[e] += to_f32(bias[k * g.Ng + f + e]);
                }
                const uint2 pk = make_uint2(pack2<T>(v[0], v[1]), pack2<T>(v[2], v[3]));
                if (staged)
                    *reinterpret_cast<uint2 *>(st + (mb * 32 + l32) * kRowE + fl) = pk;
                else if (pok[mb] && f < g.Ng)
                    *reinterpret_cast<uint2 *>(yp + f) = pk;
            }
    }
    if (staged) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int nch = min(kFilTile, g.Ng - f0) / 8;   // 16-byte pieces per position
#pragma unroll
        for (int i = 0; i < kPosWave * 8 / 64; ++i) {
            const int c = lane + 64 * i, pos = c >> 3, ch = c & 7;
            const int p = p0 + pos;
            if (p < g.P && ch < nch)
                store_nt(reinterpret_cast<uint4 *>(y + (int64_t)p * g.Cout + k * g.Ng + f0 + ch * 8),
                         *reinterpret_cast<const uint4 *>(st + pos * kRowE + ch * 8));
        }
    }
}

bool make_geom(const Conv2dArgs &a, NhwcGeom &g)
{
    if (a.dtype != DT_F16 && a.dtype != DT_BF16) return false;
    if (a.interleaved) return false;
    const int64_t Cg = a.C / a.groups, Ng = a.Cout / a.groups;
    if (Cg % 16 != 0 || Ng % 4 != 0) return false;
    if ((reinterpret_cast<uintptr_t>(a.x) & 15) || (reinterpret_cast<uintptr_t>(a.w) & 15) ||
        (reinterpret_cast<uintptr_t>(a.y) & 7))
        return false;
    const int64_t P = a.N * a.OH * a.OW;
    const int64_t m_tiles = ceil_div(P, kPosTile), n_tiles = ceil_div(Ng, kFilTile);
    if (P >= (int64_t(1) << 31) || 8 * ceil_div(m_tiles * n_tiles * a.groups, 8) >= (int64_t(1) << 31) ||
        a.Cout * a.KH * a.KW * Cg >= (int64_t(1) << 31))
        return false;
    g.N = (int)a.N; g.C = (int)a.C; g.H = (int)a.H; g.W = (int)a.W; g.Cout = (int)a.Cout;
    g.Cg = (int)Cg; g.Ng = (int)Ng; g.OH = (int)a.OH; g.OW = (int)a.OW; g.KH = (int)a.KH; g.KW = (int)a.KW;
    g.sh = a.sh; g.sw = a.sw; g.ph = a.ph; g.pw = a.pw; g.dh = a.dh; g.dw = a.dw;
    g.P = (int)P;
    g.m_tiles = (int)m_tiles;
    g.n_tiles = (int)n_tiles;
    g.tiles = (int)(m_tiles * n_tiles * a.groups);
    g.tiles_per_xcd = (int)ceil_div(g.tiles, 8);
    g.ksteps = (int)(a.KH * a.KW * Cg / 16);
    g.fd_ohw = make_fastdiv((uint32_t)(a.OH * a.OW));
    g.fd_ow = make_fastdiv((uint32_t)a.OW);
    g.groups = (int)a.groups;
    g.fd_g = make_fastdiv((uint32_t)a.groups);
    g.fd_nt = make_fastdiv((uint32_t)n_tiles);
    g.fd_cs = make_fastdiv((uint32_t)(Cg / 16));
    return true;
}

}  // namespace

bool igemm_nhwc_supported(const Conv2dArgs &a)
{
    NhwcGeom g;
    return make_geom(a, g);
}

hipError_t launch_igemm_nhwc(const Conv2dArgs &a, const char **kname)
{
    NhwcGeom g;
    if (!make_geom(a, g)) return hipErrorInvalidValue;
    *kname = "igemm_nhwc_mfma32x32x16";
    const unsigned blocks = (unsigned)(8 * (int64_t)g.tiles_per_xcd);
    if (a.dtype == DT_F16)
        hipLaunchKernelGGL((igemm_nhwc<_Float16>), dim3(blocks), dim3(kThreads), 0, a.stream,
                           (const _Float16 *)a.x, (const _Float16 *)a.w, (const _Float16 *)a.bias,
                           (_Float16 *)a.y, g);
    else
        hipLaunchKernelGGL((igemm_nhwc<__bf16>), dim3(blocks), dim3(kThreads), 0, a.stream,
                           (const __bf16 *)a.x, (const __bf16 *)a.w, (const __bf16 *)a.bias, (__bf16 *)a.y, g);
    return hipGetLastError();
}

}  // namespace gconv
