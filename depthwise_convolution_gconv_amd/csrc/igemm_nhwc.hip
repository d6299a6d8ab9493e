// igemm_nhwc.hip -- implicit-GEMM grouped conv2d over channels-last (NHWC) tensors
// on the gfx950 matrix cores (fp16 / bf16 in, fp32 accumulate).
//
// The discuss.pytorch.org thread "F.conv2d runs x15 slower in mixed-precision/
// half-precision mode" turns to the NHWC (channels_last) memory format for the fp16
// grouped conv.  In NHWC the operands of v_mfma_f32_32x32x16 are already in their
// register layout in memory: a fragment lane holds 8 consecutive K values (input
// channels) of one row or column, and 8 consecutive channels of one position of x,
// or of one filter tap of w [Cout][KH][KW][C/g], are one contiguous 16-byte run.
// So this kernel needs no transposes.  Three modes, by what fits in LDS:
//  * halo (the usual one): the tile's filter block (64 contiguous rows of w) and
//    a zero-padded halo of the input rows its 256 positions read, the group's C/g
//    channels per position, are copied into LDS once per workgroup with coalesced
//    16-byte loads; every fragment is then an LDS read, and each input element is
//    fetched from memory once per tile instead of once per tap;
//  * filters only: the filter block in LDS, input fragments from global memory;
//  * neither: both fragments from global memory (through L1/L2):
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
constexpr int kMaxKtLds = 512;                // largest KH*KW*C/g whose filter block is staged in LDS
constexpr int kFilPieces = kFilTile * kMaxKtLds / 8 / kThreads;   // 16-byte pieces per thread, at most
constexpr int kYStageBytes = 4 * kPosWave * kRowE * 2;
constexpr int kHaloPieces = 8;                // 16-byte halo pieces per thread, at most
constexpr int kLdsMax = 96 * 1024;            // LDS of one workgroup in halo mode, at most
enum { kModeGlobal = 0, kModeLdsA = 1, kModeHalo = 2 };

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

// Copy of one accumulator, held in an accumulation register, into a VGPR at this
// point: keeps the accumulators in the accumulation registers through the tile loop
// (otherwise the allocator holds them in VGPRs and runs out of them).
__device__ __forceinline__ float acc_read(float v)
{
    float r;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(v));
    return r;
}

struct NhwcGeom {
    int N, C, H, W, Cout, Cg, Ng, OH, OW, KH, KW;
    int sh, sw, ph, pw, dh, dw;
    int P;                   // N*OH*OW
    int m_tiles, n_tiles;    // ceil(P / 256), ceil(Ng / 64)
    int tiles, groups;
    int strips;              // work units per (group, filter tile): position-tile strips
    int wgs, wgs_per_xcd;    // groups*n_tiles*strips; ceil(wgs / 8)
    int ksteps;              // KH*KW*Cg/16
    int ktot;                // KH*KW*Cg: elements of one filter
    FastDiv fd_ohw, fd_ow, fd_g, fd_nt, fd_cs;   // fd_cs: Cg/16 (channel steps per tap)
    FastDiv fd_ppr;          // ktot/8: 16-byte pieces per filter
    // Halo mode: virtual padded input rows R = n*Hp + ih + ph; the tile's halo holds
    // rows R_lo .. R_lo + NR - 1 (R_lo: the first position's first row) and padded
    // columns 0 .. WL - 1, C/g channels per slot plus one spare 16-byte unit.
    int Hp, NR, WL, hpieces;     // hpieces = NR*WL*Cg/8
    int halo_units;              // 16-byte units of the halo area (also the output staging)
    FastDiv fd_hp, fd_wl, fd_c8; // Hp, WL, Cg/8
};

// MODE: kModeGlobal, kModeLdsA (filters in LDS, ktot <= kMaxKtLds) or kModeHalo
// (filters and the input halo in LDS).
template <typename T, int MODE>
__global__ void __launch_bounds__(kThreads)
igemm_nhwc(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
           T *__restrict__ y, NhwcGeom g)
{
    // LDS: the filter block and the input halo during the K loop, then the output
    // staging.
    constexpr bool LDS_A = MODE != kModeGlobal, HALO = MODE == kModeHalo;
    extern __shared__ uint4 smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    // Work unit: a strip of consecutive position tiles [mt_lo, mt_hi) of one filter
    // tile nt of one group k.  Units are ordered groups fastest: the units of all
    // groups of one position range run together, so every 128-byte line of x (64
    // channels, several groups) is used whole while it is in L2.  Units are dealt to
    // the XCDs in contiguous runs (workgroup b runs on XCD b % 8), so neighbouring
    // position ranges, which read the same input rows, share one L2.  In halo mode a
    // strip has several tiles: the filter block and the bias are loaded once, and
    // each tile's input halo is fetched while the tile before it computes.  Other
    // modes take one tile per unit.
    const int xcd = blockIdx.x & 7, rank = blockIdx.x >> 3;
    const int wgi = xcd * g.wgs_per_xcd + rank;
    if (wgi >= min((xcd + 1) * g.wgs_per_xcd, g.wgs)) return;   // uniform over the workgroup
    const int bq = fdiv(wgi, g.fd_g);
    const int k = wgi - bq * g.groups;
    const int strip = fdiv(bq, g.fd_nt);
    const int nt = bq - strip * g.n_tiles;
    const int mt_lo = (int)((int64_t)strip * g.m_tiles / g.strips);
    const int mt_hi = (int)((int64_t)(strip + 1) * g.m_tiles / g.strips);
    const int f0 = nt * kFilTile;                       // first filter (within the group)

    // This lane's rows of the A operand (filters f0 + nb*32 + l32); channels
    // c0 + 8*half of a K step.
    const T *wrow[2];
    bool fok[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int f = f0 + nb * 32 + l32;
        fok[nb] = f < g.Ng;
        wrow[nb] = w + (int64_t)(k * g.Ng + (fok[nb] ? f : 0)) * g.KH * g.KW * g.Cg + 8 * half;
    }
    const int cbase = k * g.Cg + 8 * half;               // this lane's channel offset in x

    // Filter block in LDS: row r (filter f0 + r, zeros past Ng) holds the filter's
    // ktot elements, K order (tap, channel), and one spare unit.  The row stride,
    // ktot/8 + 1 units of 16 bytes, is odd, so the 16-byte A reads of consecutive
    // rows are free of bank conflicts.  All of a thread's loads are issued before
    // the first LDS write.
    const int rowu = g.ktot / 8 + 1;
    if constexpr (LDS_A) {
        const int ppr = g.ktot / 8, nrows = min(kFilTile, g.Ng - f0);
        const uint4 *wsrc = reinterpret_cast<const uint4 *>(w + (int64_t)(k * g.Ng + f0) * g.ktot);
        uint4 pv[kFilPieces];
#pragma unroll
        for (int j = 0; j < kFilPieces; ++j) {
            const int i = tid + j * kThreads;
            pv[j] = make_uint4(0, 0, 0, 0);
            if (i < kFilTile * ppr && fdiv(i, g.fd_ppr) < nrows) pv[j] = wsrc[i];
        }
#pragma unroll
        for (int j = 0; j < kFilPieces; ++j) {
            const int i = tid + j * kThreads;
            if (i < kFilTile * ppr) {
                const int r = fdiv(i, g.fd_ppr);
                smem[r * rowu + (i - r * ppr)] = pv[j];
            }
        }
    }
    // Input halo, after the filter block: slot (rr, col) at units (rr*WL + col)*SU ..,
    // SU = Cg/8 + 1 (odd, so lanes on consecutive slots read distinct banks).  Piece i
    // is 8 channels of one slot; consecutive threads take consecutive pieces, so a
    // load instruction covers whole C/g-channel runs of consecutive input columns.
    // Rows outside the image (padding, or past the last image) and columns in the
    // padding are written as zeros.
    const int SU = g.Cg / 8 + 1, c8n = g.Cg / 8;
    uint4 *halo = smem + kFilTile * rowu;
    auto tile_rlo = [&](int mt) {   // virtual padded input row of the tile's first position
        const int pt = mt * kPosTile;
        const int n_first = fdiv(pt, g.fd_ohw);
        return n_first * g.Hp + fdiv(pt - n_first * g.OH * g.OW, g.fd_ow) * g.sh;
    };
    uint4 hv[HALO ? kHaloPieces : 1];
    auto halo_load = [&](int rlo) {
#pragma unroll
        for (int j = 0; j < kHaloPieces; ++j) {
            const int i = tid + j * kThreads;
            hv[j] = make_uint4(0, 0, 0, 0);
            if (i < g.hpieces) {
                const int slot = fdiv(i, g.fd_c8), c8 = i - slot * c8n;
                const int rr = fdiv(slot, g.fd_wl), col = slot - rr * g.WL;
                const int R = rlo + rr, n = fdiv(R, g.fd_hp);
                const int ih = R - n * g.Hp - g.ph, iw = col - g.pw;
                if (n < g.N && ih >= 0 && ih < g.H && iw >= 0 && iw < g.W)
                    hv[j] = *reinterpret_cast<const uint4 *>(
                        x + (((int64_t)n * g.H + ih) * g.W + iw) * g.C + k * g.Cg + 8 * c8);
            }
        }
    };
    auto halo_store = [&]() {
#pragma unroll
        for (int j = 0; j < kHaloPieces; ++j) {
            const int i = tid + j * kThreads;
            if (i < g.hpieces) {
                const int slot = fdiv(i, g.fd_c8);
                halo[slot * SU + (i - slot * c8n)] = hv[j];
            }
        }
    };
    if constexpr (HALO) {
        halo_load(tile_rlo(mt_lo));
        halo_store();
    }
    if constexpr (LDS_A) __syncthreads();

    // Bias of this lane's accumulator rows, loaded ahead of the K loop: in halo mode
    // once per strip into LDS as fp32 (after the halo area), otherwise into
    // registers as 16-bit values, two per register.
    float *bsm = reinterpret_cast<float *>(halo + g.halo_units);
    uint32_t bv[2][4][2];
    if constexpr (HALO) {
        if (tid < kFilTile) {
            const int f = f0 + tid;
            bsm[tid] = (bias && f < g.Ng) ? to_f32(bias[k * g.Ng + f]) : 0.0f;
        }
        __syncthreads();
    } else {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e2 = 0; e2 < 2; ++e2) {
                    uint32_t lo = 0, hi = 0;
                    const int f = f0 + nb * 32 + q * 8 + 4 * half + 2 * e2;
                    if (bias && f < g.Ng) lo = __builtin_bit_cast(uint16_t, bias[k * g.Ng + f]);
                    if (bias && f + 1 < g.Ng) hi = __builtin_bit_cast(uint16_t, bias[k * g.Ng + f + 1]);
                    bv[nb][q][e2] = lo | (hi << 16);
                }
    }
    int arow[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) arow[nb] = (nb * 32 + l32) * rowu + half;
    // Output staging: in halo mode the halo's area (the filter block stays for the
    // next tile), otherwise the start of the LDS.
    T *st = reinterpret_cast<T *>(HALO ? halo : smem) + wave * kPosWave * kRowE;
    const bool staged = (g.Ng & 7) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;

#pragma unroll 1
    for (int mt = mt_lo; mt < mt_hi; ++mt) {
        const int p0 = mt * kPosTile + wave * kPosWave;     // first position of this wave
        const int R_lo = HALO ? tile_rlo(mt) : 0;
        // Columns of the B operand: positions p0 + mb*32 + l32.
        int pn[2], poh[2], pow_[2], hbase[2];
        bool pok[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int p = p0 + mb * 32 + l32;
            pok[mb] = p < g.P;
            // Positions past P compute on a valid one (P - 1 lies in the tile, so also in its halo).
            const int pc = pok[mb] ? p : (HALO ? g.P - 1 : 0);
            pn[mb] = fdiv(pc, g.fd_ohw);
            const int q = pc - pn[mb] * g.OH * g.OW;
            poh[mb] = fdiv(q, g.fd_ow);
            pow_[mb] = q - poh[mb] * g.OW;
            // halo mode: unit of the position's tap (0, 0) slot, plus this lane's channel octet
            hbase[mb] = ((pn[mb] * g.Hp + poh[mb] * g.sh - R_lo) * g.WL + pow_[mb] * g.sw) * SU + half;
        }
        // The next tile's halo goes to registers now and to LDS after this tile.
        const bool more = mt + 1 < mt_hi;
        if constexpr (HALO)
            if (more) halo_load(tile_rlo(mt + 1));

        // Steps are loaded in order, so the (tap, channel step) of the next load is
        // kept as wave-uniform counters and advanced once per step, with no division.
        struct StepPos {
            int s, cc, kh, kw;   // step; channel step within the tap; tap row and column
            int toff;            // halo mode: units from a position's tap (0,0) slot to its tap (kh,kw) slot
        } ld = {0, 0, 0, 0, 0};
        const int csteps = g.Cg / 16;
        auto advance = [&]() {
            ++ld.s;
            if (++ld.cc == csteps) {
                ld.cc = 0;
                ld.toff += g.dw * SU;
                if (++ld.kw == g.KW) {
                    ld.kw = 0;
                    ++ld.kh;
                    ld.toff += (g.dh * g.WL - g.KW * g.dw) * SU;
                }
            }
        };
        // Fragments of the step at ld: zero for filters past Ng, for positions past P
        // and for taps in the padding.
        auto load_step = [&](uint4 (&a)[2], uint4 (&b)[2]) {
            const int cs = ld.cc * 16;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                if constexpr (LDS_A) {
                    // elements s*16 + 8*half .. +7 of row nb*32 + l32 (K order: tap, channel)
                    a[nb] = smem[arow[nb] + 2 * ld.s];
                } else {
                    a[nb] = make_uint4(0, 0, 0, 0);
                    if (fok[nb])
                        a[nb] = *reinterpret_cast<const uint4 *>(wrow[nb] + (ld.kh * g.KW + ld.kw) * g.Cg + cs);
                }
            }
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                if constexpr (HALO) {
                    // channels cs + 8*half .. +7 at the tap's slot
                    b[mb] = halo[hbase[mb] + ld.toff + 2 * ld.cc];
                } else {
                    const int ih = poh[mb] * g.sh - g.ph + ld.kh * g.dh;
                    const int iw = pow_[mb] * g.sw - g.pw + ld.kw * g.dw;
                    b[mb] = make_uint4(0, 0, 0, 0);
                    if (pok[mb] && ih >= 0 && ih < g.H && iw >= 0 && iw < g.W)
                        b[mb] = *reinterpret_cast<const uint4 *>(
                            x + (((int64_t)pn[mb] * g.H + ih) * g.W + iw) * g.C + cbase + cs);
                }
            }
            advance();
        };

        f32x16 acc[2][2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;

        // A ring of DEPTH steps of fragments: step s computes from slot s % DEPTH,
        // whose next load (step s + DEPTH) is issued right after, so each load has
        // DEPTH - 1 steps of MFMAs to arrive.
        // Halo mode reads every fragment from LDS, where two steps in flight suffice.
        constexpr int DEPTH = HALO ? 2 : kDepth;
        uint4 fa[DEPTH][2], fb[DEPTH][2];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d)
            if (d < g.ksteps) load_step(fa[d], fb[d]);
#pragma unroll 1
        for (int s0 = 0; s0 < g.ksteps; s0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int s = s0 + d;
                if (s < g.ksteps) {   // uniform
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                        for (int mb = 0; mb < 2; ++mb)
                            acc[nb][mb] = MfmaN<T>::run(fa[d][nb], fb[d][mb], acc[nb][mb]);
                    if (s + DEPTH < g.ksteps) load_step(fa[d], fb[d]);
                }
            }
        }

        // Epilogue: accumulator r of block (nb, mb) is filter f0 + nb*32 + (r/4)*8 +
        // 4*half + r%4 at position p0 + mb*32 + l32; bias in fp32, one rounding.  When
        // the tile's 64 filters are one 128-byte run of y per position (Cout/g a
        // multiple of 8, y 16-byte aligned), the wave stages its 64 positions x 64
        // filters in its own LDS area (rows of kRowE elements, padded against bank
        // conflicts) and stores whole 16-byte pieces, 8 lanes per position: the 8-byte
        // pieces of the accumulator layout, from 8 different store instructions, would
        // reach HBM as partial lines.
        if constexpr (LDS_A) __syncthreads();   // every wave's last LDS operand reads are done
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
                        v[e] = acc_read(acc[nb][mb][q * 4 + e]);
                        if (bias) {
                            if constexpr (HALO) {
                                v[e] += bsm[fl + e];
                            } else {
                                const uint16_t h = (uint16_t)(bv[nb][q][e >> 1] >> (16 * (e & 1)));
                                v[e] += to_f32(__builtin_bit_cast(T, h));
                            }
                        }
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
        if constexpr (HALO) {
            if (more) {
                __syncthreads();   // every wave has read its staged outputs
                halo_store();
                __syncthreads();
            }
        }
    }
}

int pick_mode(const NhwcGeom &g);
constexpr int kResidentWgs = 2 * 256;   // halo-mode workgroups the chip holds at once (2 per CU)

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
    g.ksteps = (int)(a.KH * a.KW * Cg / 16);
    g.ktot = (int)(a.KH * a.KW * Cg);
    g.fd_ppr = make_fastdiv((uint32_t)(g.ktot / 8));
    // Halo rows one tile can need: the virtual output rows its kPosTile positions
    // touch (V), the image boundaries among them, each adding the rows between the
    // images' output ranges, and the filter's reach; never more than all N*Hp rows.
    const int64_t Hp = a.H + 2 * (int64_t)a.ph;
    const bool aligned_rows = kPosTile % a.OW == 0;
    const int64_t V = aligned_rows ? kPosTile / a.OW : (kPosTile - 1) / a.OW + 2;
    const int64_t crossings =
        (V <= 1) ? 0 : ((aligned_rows && a.OH % (kPosTile / a.OW) == 0) ? 0 : (V - 2) / a.OH + 1);
    const int64_t gap = std::max<int64_t>(0, Hp - a.OH * (int64_t)a.sh);
    const int64_t NR = std::min<int64_t>((V - 1) * a.sh + crossings * gap + (a.KH - 1) * (int64_t)a.dh + 1,
                                         a.N * Hp);
    const int64_t WL = (a.OW - 1) * (int64_t)a.sw + (a.KW - 1) * (int64_t)a.dw + 1;
    const int64_t hpieces = NR * WL * (Cg / 8);
    g.Hp = (int)std::min<int64_t>(Hp, INT32_MAX);
    g.NR = (int)std::min<int64_t>(NR, INT32_MAX);
    g.WL = (int)std::min<int64_t>(WL, INT32_MAX);
    g.hpieces = (int)std::min<int64_t>(hpieces, INT32_MAX);
    g.fd_hp = make_fastdiv((uint32_t)g.Hp);
    g.fd_wl = make_fastdiv((uint32_t)g.WL);
    g.fd_c8 = make_fastdiv((uint32_t)(Cg / 8));
    g.halo_units = (int)std::min<int64_t>(std::max<int64_t>(NR * WL * (Cg / 8 + 1), kYStageBytes / 16), INT32_MAX);
    // Work units: in halo mode about one per workgroup slot of the chip, each a strip
    // of consecutive position tiles (at least one); otherwise one per tile.
    const int64_t gn = (int64_t)a.groups * n_tiles;
    g.strips = (int)(pick_mode(g) == kModeHalo
                         ? std::min<int64_t>(m_tiles, std::max<int64_t>(1, ceil_div((int64_t)kResidentWgs, gn)))
                         : m_tiles);
    g.wgs = (int)(gn * g.strips);
    g.wgs_per_xcd = (int)ceil_div((int64_t)g.wgs, 8);
    g.fd_ohw = make_fastdiv((uint32_t)(a.OH * a.OW));
    g.fd_ow = make_fastdiv((uint32_t)a.OW);
    g.groups = (int)a.groups;
    g.fd_g = make_fastdiv((uint32_t)a.groups);
    g.fd_nt = make_fastdiv((uint32_t)n_tiles);
    g.fd_cs = make_fastdiv((uint32_t)(Cg / 16));
    return true;
}

// LDS bytes of the filter block and of the input halo.
size_t filter_lds(const NhwcGeom &g) { return (size_t)kFilTile * (g.ktot / 8 + 1) * 16; }
size_t halo_lds(const NhwcGeom &g) { return (size_t)g.NR * g.WL * (g.Cg / 8 + 1) * 16; }

int pick_mode(const NhwcGeom &g)
{
    if (g.ktot > kMaxKtLds) return kModeGlobal;
    if (g.hpieces <= kHaloPieces * kThreads && (int64_t)g.N * g.Hp < (int64_t(1) << 30) &&
        filter_lds(g) + std::max<size_t>(halo_lds(g), kYStageBytes) + kFilTile * 4 <= (size_t)kLdsMax)
        return kModeHalo;
    return kModeLdsA;
}

template <typename T, int MODE>
void launch_mode(const Conv2dArgs &a, const NhwcGeom &g, unsigned blocks, size_t lds)
{
    hipLaunchKernelGGL((igemm_nhwc<T, MODE>), dim3(blocks), dim3(kThreads), lds, a.stream, (const T *)a.x,
                       (const T *)a.w, (const T *)a.bias, (T *)a.y, g);
}

template <typename T>
void launch_typed(const Conv2dArgs &a, const NhwcGeom &g, unsigned blocks)
{
    const int mode = pick_mode(g);
    const size_t lds = std::max<size_t>(
        kYStageBytes, mode == kModeHalo ? filter_lds(g) + (size_t)g.halo_units * 16 + kFilTile * 4
                      : mode == kModeLdsA ? filter_lds(g)
                                          : 0);
    if (mode == kModeHalo)
        launch_mode<T, kModeHalo>(a, g, blocks, lds);
    else if (mode == kModeLdsA)
        launch_mode<T, kModeLdsA>(a, g, blocks, lds);
    else
        launch_mode<T, kModeGlobal>(a, g, blocks, lds);
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
    const unsigned blocks = (unsigned)(8 * (int64_t)g.wgs_per_xcd);
    if (a.dtype == DT_F16)
        launch_typed<_Float16>(a, g, blocks);
    else
        launch_typed<__bf16>(a, g, blocks);
    return hipGetLastError();
}

}  // namespace gconv
