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
// group x BM = 256 consecutive output positions (flattened over n, oh, ow, so a
// tile may span image boundaries).  Every wave computes all BN channels for 64
// of the positions: WN x 2 blocks of v_mfma_f32_32x32x16_{f16,bf16}, filters as
// the A operand (rows = output channels), the im2col tile as the B operand
// (columns = positions).  Column j of block mb of wave w is tile position
// 8j + 2w + mb, which keeps the LDS operand reads free of bank conflicts.
//
// K loop: input channels in chunks of 16, then taps; one MFMA step = one tap x
// 16 channels.  Per chunk:
//  * filters: a small pre-pass (igemm_pack_filters) lays out every (group, filter
//    tile, chunk) as the exact LDS image, [tap][filter][16 channels]; the main
//    kernel copies it with direct global->LDS loads (no registers involved);
//  * input: whole zero-padded input rows of the 16 channels, stored as
//    [row][col][16 channels] so that one MFMA fragment (8 consecutive channels at
//    one position) is a single 16-byte LDS read; loaded 8 positions at a time per
//    channel with buffer loads (out-of-range offsets read as zero, which provides
//    the padding rows), transposed in registers with v_perm.
// Epilogue: bias added in fp32, one rounding to the output dtype, the tile staged
// through LDS and written 16 bytes per lane along W.
#include <algorithm>

#include "common.hpp"

namespace gconv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kCK = 16;            // input channels per K chunk
constexpr int kLdsBudget = 64 * 1024;

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
    int xslots;          // NR*WL rounded up to whole 8-slot rows of lds_unit
    int nseg;            // W / VW: vector segments per input row
    int xtasks;          // 2 channel octets * NR * nseg
    int64_t P;           // N*OH*OW output positions
    int m_tiles, n_tiles, groups, nchunks;
    int xcd_remap;       // 1: spread consecutive tiles over the 8 XCDs in contiguous runs
    int y_vec;           // 1: 8 consecutive positions of a channel are one aligned 16-byte run of y
};

// LDS placement of the 16-byte half `half` (channels 0-7 or 8-15) of 32-byte slot
// `s`, in 16-byte units.  The LDS has 64 banks of 4 bytes, so a 16-byte access by 16
// lanes is conflict-free when the lanes hit 16 distinct units modulo 16.  Each
// 256-byte row (8 slots) XORs its unit column with the row number, so 16 slots that
// lie 8 apart -- in 16 consecutive rows -- land in 16 different columns.  Both hot
// patterns are of that kind: the staging writes (one slot per 8-wide row segment)
// and the MFMA operand reads (lanes own positions 8 apart, see igemm_fwd).  The
// filter image is read 16 consecutive slots at a time: two rows, one per parity.
__device__ __forceinline__ int lds_unit(int s, int half)
{
    const int r = s >> 3;
    return (r << 4) + ((2 * (s & 7) + half) ^ (r & 15));
}

constexpr uint32_t kOOB = 0x80000000u;  // byte offset past num_records: the load returns 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// VW consecutive 16-bit elements, returned as VW/2 (or 1) dwords.
template <int VW> struct VecLoad;
template <> struct VecLoad<8> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so, uint32_t *d)
    {
        const uint4 u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0));
        d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w;
    }
};
template <> struct VecLoad<4> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so, uint32_t *d)
    {
        const uint2 u = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0));
        d[0] = u.x; d[1] = u.y;
    }
};
template <> struct VecLoad<2> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so, uint32_t *d)
    {
        d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0);
    }
};
template <> struct VecLoad<1> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so, uint32_t *d)
    {
        d[0] = __builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0);
    }
};

// Dword made of element v of row ra (low half) and element v of row rb (high half),
// where each row holds VW 16-bit elements packed in dwords.
template <int VW, int v>
__device__ __forceinline__ uint32_t col_pair(const uint32_t *ra, const uint32_t *rb)
{
    if constexpr (VW == 1) {
        return (ra[0] & 0xffffu) | (rb[0] << 16);
    } else {
        constexpr uint32_t b = 2 * (v & 1);
        constexpr uint32_t sel = ((b + 5) << 24) | ((b + 4) << 16) | ((b + 1) << 8) | b;
        return __builtin_amdgcn_perm(rb[v >> 1], ra[v >> 1], sel);
    }
}

// Writes position v of 8 channel rows d[0..7] as one 16-byte channel octet to halo
// slot slot0+v (or to the spare slot when v >= limit).
template <int VW, int DW, int v>
__device__ __forceinline__ void write_octets(uint4 *xs, int slot0, int octet, int limit, int dummy,
                                             const uint32_t (*d)[DW])
{
    const uint4 val = make_uint4(col_pair<VW, v>(d[0], d[1]), col_pair<VW, v>(d[2], d[3]),
                                 col_pair<VW, v>(d[4], d[5]), col_pair<VW, v>(d[6], d[7]));
    const int s = slot0 + v;
    xs[(v < limit) ? lds_unit(s, octet) : dummy] = val;
    if constexpr (v + 1 < VW) write_octets<VW, DW, v + 1>(xs, slot0, octet, limit, dummy, d);
}

constexpr int kMaxXRounds = 2;  // input staging tasks per thread

// Filters of one (group, filter tile, 16-channel chunk), laid out exactly as the
// kernel's LDS image: slot t*BN + filter, two 16-byte channel octets per slot, placed
// by lds_unit.  One thread handles one (filter, 8-channel octet): it reads the
// octet's KT taps of 8 channels (contiguous in w) and writes one 16-byte unit per
// tap.  Filters past Cout/g and channels past C/g are zero.
template <int KT>
__global__ void __launch_bounds__(kThreads)
igemm_pack_filters(const uint16_t *__restrict__ w, uint4 *__restrict__ wp, int64_t tasks, int Ng, int Cg,
                   int BN, int n_tiles, int nchunks)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= tasks) return;
    int64_t r = i;
    const int octet = (int)(r % 2); r /= 2;
    const int nn = (int)(r % BN); r /= BN;
    const int ch = (int)(r % nchunks); r /= nchunks;
    const int nt = (int)(r % n_tiles);
    const int k = (int)(r / n_tiles);
    const int on = nt * BN + nn;
    const int c0 = ch * kCK + octet * 8;
    uint16_t h[8 * KT];
#pragma unroll
    for (int e = 0; e < 8 * KT; ++e) {
        const int c = c0 + e / KT;
        h[e] = (on < Ng && c < Cg) ? w[((int64_t)(k * Ng + on) * Cg + c) * KT + e % KT] : (uint16_t)0;
    }
    uint4 *dst = wp + (((int64_t)k * n_tiles + nt) * nchunks + ch) * (KT * BN * 2);
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            v[e] = (uint32_t)h[(2 * e) * KT + t] | ((uint32_t)h[(2 * e + 1) * KT + t] << 16);
        dst[lds_unit(t * BN + nn, octet)] = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

template <typename T, int WN, int WM, int KT, int VW>
__global__ void __launch_bounds__(kThreads, 2)
igemm_fwd(const T *__restrict__ x, const uint4 *__restrict__ wp, const T *__restrict__ bias,
          T *__restrict__ y, IgemmGeom g)
{
    constexpr int BN = WN * 32;
    constexpr int BM = 4 * WM * 32;
    constexpr int SR = BM / 32;                   // position stride between MFMA columns
    constexpr int DW = VW > 1 ? VW / 2 : 1;       // dwords per staged row segment
    constexpr int WCHUNK = KT * BN * 2;           // 16-byte units of one chunk's filters
    extern __shared__ uint4 lds[];
    uint4 *xs = lds;                              // [xslots][2] x 16 bytes
    uint4 *ws = lds + g.xslots * 2;               // [KT][BN][2] x 16 bytes
    const int dummy = g.xslots * 2 + WCHUNK;      // spare 16 bytes for masked-off writes

    int bid = blockIdx.x;
    if (g.xcd_remap) {
        // Blocks are dealt round-robin to the 8 XCDs; give each XCD a contiguous
        // run of tiles so neighbouring tiles share halo rows in one L2.
        const int per = gridDim.x / 8;
        bid = (bid % 8) * per + bid / 8;
    }
    const int mt = bid % g.m_tiles; bid /= g.m_tiles;
    const int nt = bid % g.n_tiles;
    const int k = bid / g.n_tiles;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int OHW = g.OH * g.OW;
    const int HW = g.H * g.W;

    // First virtual padded input row the tile needs.
    const int64_t p0 = (int64_t)mt * BM;
    const int64_t n_first = p0 / OHW;
    const int oh_first = (int)(p0 % OHW) / g.OW;
    const int64_t R_lo = n_first * g.Hp + (int64_t)oh_first * g.sh;

    // Output positions: column j of MFMA block mb of wave w is tile position
    // SR*j + w*WM + mb (SR = BM/32).  The 16 lanes of a half-block then read halo
    // slots SR apart, which lds_unit spreads over all 16 bank columns; the epilogue
    // restores position order through LDS.
    // LDS slot of tap (0,0) for each of this lane's output positions.
    int xslot[WM];
#pragma unroll
    for (int mb = 0; mb < WM; ++mb) {
        int64_t p = p0 + SR * l32 + wave * WM + mb;
        if (p >= g.P) p = g.P - 1;
        const int64_t n = p / OHW;
        const int q = (int)(p % OHW);
        const int oh = q / g.OW, ow = q % g.OW;
        xslot[mb] = (int)(n * g.Hp + (int64_t)oh * g.sh - R_lo) * g.WL + ow * g.sw;
    }

    // Input staging tasks: (channel octet, halo row rr, segment sg) -> VW positions of 8
    // channels.  Byte offsets are relative to channel 0 of group k in image n_first;
    // rows outside the image get an out-of-range offset and read as zeros.
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + ((int64_t)n_first * g.C + (int64_t)k * g.Cg) * HW,
                                                0x7fffffffu);
    uint32_t xvo[kMaxXRounds];
    int xslot0[kMaxXRounds], xoct[kMaxXRounds], xlim[kMaxXRounds];
#pragma unroll
    for (int i = 0; i < kMaxXRounds; ++i) {
        const int t = tid + i * kThreads;
        xvo[i] = kOOB; xslot0[i] = 0; xoct[i] = 0; xlim[i] = 0;
        if (t < g.xtasks) {
            const int sg = t % g.nseg, rest = t / g.nseg;
            const int rr = rest % g.NR, oc = rest / g.NR;
            const int64_t R = R_lo + rr;
            const int64_t n = R / g.Hp;
            const int ih = (int)(R % g.Hp) - g.ph;
            const int c0 = sg * VW + g.pw;            // LDS column of the segment's first element
            xslot0[i] = rr * g.WL + c0;
            xoct[i] = oc;
            xlim[i] = min(VW, g.WL - c0);             // elements that land inside the halo
            if (n < g.N && ih >= 0 && ih < g.H)
                xvo[i] = (uint32_t)((((n - n_first) * g.C + 8 * oc) * (int64_t)HW + (int64_t)ih * g.W +
                                     sg * VW) * 2);
        }
    }
    const int xrounds = (g.xtasks + kThreads - 1) / kThreads;

    // Packed filters of (k, nt): one contiguous LDS image per chunk.
    const uint4 *wsrc = wp + (int64_t)(k * g.n_tiles + nt) * g.nchunks * WCHUNK;

    // Zero the halo once: padding columns are never written by the staging tasks.
    for (int i = tid; i < g.xslots * 2; i += kThreads) xs[i] = make_uint4(0, 0, 0, 0);

    f32x16 acc[WN][WM];
#pragma unroll
    for (int i = 0; i < WN; ++i)
#pragma unroll
        for (int j = 0; j < WM; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    for (int ch = 0; ch < g.nchunks; ++ch) {
        const int ci0 = ch * kCK;
        __syncthreads();  // the previous chunk's operands (or the zero fill) are done with
        // ---- filters: copy the chunk's LDS image straight from global memory into LDS
        const uint4 *wc = wsrc + (int64_t)ch * WCHUNK;
        for (int u = wave * 64; u < WCHUNK; u += 4 * 64)
            __builtin_amdgcn_global_load_lds((const void *)(wc + u + lane),
                                             (__attribute__((address_space(3))) void *)(ws + u), 16, 0, 0);
        // ---- input halo: load 8 channel rows x VW positions, write VW channel octets
#pragma unroll
        for (int i = 0; i < kMaxXRounds; ++i) {
            if (i < xrounds) {
                uint32_t d[8][DW];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool ok = ci0 + 8 * xoct[i] + e < g.Cg;
                    VecLoad<VW>::run(xr, ok ? xvo[i] : kOOB, (uint32_t)(ci0 + e) * HW * 2, d[e]);
                }
                __builtin_amdgcn_sched_barrier(0);  // issue all loads before the first use
                write_octets<VW, DW, 0>(xs, xslot0[i], xoct[i], xlim[i], dummy, d);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0);  // the filter copy landed in LDS
        __syncthreads();
        // ---- MFMA over the taps of this chunk
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const int kh = t / g.KW, kw = t % g.KW;
            const int xoff = kh * g.dh * g.WL + kw * g.dw;
            uint4 bf[WM], af[WN];
#pragma unroll
            for (int mb = 0; mb < WM; ++mb) {
                const int s = xslot[mb] + xoff;
                bf[mb] = xs[lds_unit(s, half)];
            }
#pragma unroll
            for (int nb = 0; nb < WN; ++nb) {
                const int nn = nb * 32 + l32;
                af[nb] = ws[lds_unit(t * BN + nn, half)];
            }
#pragma unroll
            for (int nb = 0; nb < WN; ++nb)
#pragma unroll
                for (int mb = 0; mb < WM; ++mb) acc[nb][mb] = Mfma<T>::run(af[nb], bf[mb], acc[nb][mb]);
        }
    }

    // ---- epilogue: + bias in fp32, one rounding to T, then through LDS so that each
    // thread stores 8 consecutive positions of one output channel (16 bytes).
    constexpr int EROWS = BN < 64 ? BN : 64;      // output channels per pass
    constexpr int CSTRIDE = BM + 8;               // padded LDS row (elements)
    T *ct = reinterpret_cast<T *>(lds);
    const bool vec_ok = g.y_vec && (p0 + BM <= g.P);
#pragma unroll
    for (int pass = 0; pass < BN / EROWS; ++pass) {
        __syncthreads();
#pragma unroll
        for (int nb = pass * (EROWS / 32); nb < (pass + 1) * (EROWS / 32); ++nb) {
#pragma unroll
            for (int mb = 0; mb < WM; ++mb) {
                const int pl = SR * l32 + wave * WM + mb;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int nl = (nb - pass * (EROWS / 32)) * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                    const int on = nt * BN + pass * EROWS + nl;
                    float v = acc[nb][mb][r];
                    if (bias && on < g.Ng) v += to_f32(bias[k * g.Ng + on]);
                    ct[nl * CSTRIDE + pl] = from_f32<T>(v);
                }
            }
        }
        __syncthreads();
        for (int c = tid; c < EROWS * (BM / 8); c += kThreads) {
            const int row = c / (BM / 8), p8 = c % (BM / 8);
            const int on = nt * BN + pass * EROWS + row;
            const int64_t p = p0 + p8 * 8;
            if (on >= g.Ng || p >= g.P) continue;
            const int co = k * g.Ng + on;
            const T *src = ct + row * CSTRIDE + p8 * 8;
            if (vec_ok) {
                const int64_t n = p / OHW;
                const int q = (int)(p % OHW);
                *reinterpret_cast<uint4 *>(y + (n * g.Cout + co) * (int64_t)OHW + q) =
                    *reinterpret_cast<const uint4 *>(src);
            } else {
                for (int e = 0; e < 8 && p + e < g.P; ++e) {
                    const int64_t n = (p + e) / OHW;
                    const int q = (int)((p + e) % OHW);
                    y[(n * g.Cout + co) * (int64_t)OHW + q] = src[e];
                }
            }
        }
    }
}

struct Plan {
    IgemmGeom g;
    int WN, WM, KT, VW;
    size_t lds;
    int64_t blocks;
    int64_t packed_units;   // 16-byte units of the packed filters
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
    const int64_t KT = a.KH * a.KW;
    if (KT != 1 && KT != 9) return pl;
    pl.KT = (int)KT;
    pl.WN = g.Ng > 32 ? 4 : 1;
    if (g.Ng > 32 && g.Ng <= 64) pl.WN = 2;
    pl.WM = 2;
    const int BN = pl.WN * 32, BM = 4 * pl.WM * 32;
    // Vector width of the input row loads.
    const uintptr_t xa = reinterpret_cast<uintptr_t>(a.x);
    pl.VW = (g.W % 8 == 0 && xa % 16 == 0) ? 8 : (g.W % 4 == 0 && xa % 8 == 0) ? 4
          : (g.W % 2 == 0 && xa % 4 == 0) ? 2 : 1;
    // Virtual output rows one tile can touch, image boundaries inside them, and
    // the resulting bound on the virtual padded input rows of its halo.
    const bool aligned_rows = BM % g.OW == 0;
    const int64_t V = aligned_rows ? BM / g.OW : (BM - 1) / g.OW + 2;
    const int64_t crossings = (V <= 1) ? 0 : ((aligned_rows && g.OH % (BM / g.OW) == 0) ? 0 : (V - 2) / g.OH + 1);
    const int64_t gap = std::max<int64_t>(0, (int64_t)g.Hp - (int64_t)g.OH * g.sh);
    const int64_t NR = (V - 1) * g.sh + crossings * gap + (int64_t)(g.KH - 1) * g.dh + 1;
    const int64_t WL = (int64_t)(g.OW - 1) * g.sw + (int64_t)(g.KW - 1) * g.dw + 1;
    g.NR = (int)NR; g.WL = (int)WL;
    g.xslots = (int)((NR * WL + 7) / 8 * 8);
    g.nseg = (g.W + pl.VW - 1) / pl.VW;
    const int64_t xtasks = 2 * NR * g.nseg;
    if (xtasks > (int64_t)kMaxXRounds * kThreads) return pl;
    g.xtasks = (int)xtasks;
    // Byte offsets of the staged input, relative to one tile's first image, stay below 2^31.
    const int64_t HW = (int64_t)g.H * g.W;
    if ((crossings + 1) * (int64_t)g.C * HW * 2 >= (int64_t(1) << 31)) return pl;
    pl.lds = (size_t)((int64_t)g.xslots * 2 + KT * BN * 2 + 1) * sizeof(uint4);  // + spare unit
    const size_t epi_lds = (size_t)std::min(BN, 64) * (BM + 8) * 2;              // epilogue staging
    pl.lds = std::max(pl.lds, epi_lds);
    if (pl.lds > (size_t)kLdsBudget) return pl;
    g.y_vec = ((int64_t)g.OH * g.OW) % 8 == 0 && (reinterpret_cast<uintptr_t>(a.y) & 15) == 0;
    g.m_tiles = (int)ceil_div(g.P, BM);
    g.n_tiles = (int)ceil_div(g.Ng, BN);
    g.nchunks = (int)ceil_div(g.Cg, kCK);
    pl.blocks = (int64_t)g.m_tiles * g.n_tiles * g.groups;
    if (pl.blocks >= (int64_t(1) << 31) || g.P >= (int64_t(1) << 31)) return pl;
    pl.packed_units = (int64_t)g.groups * g.n_tiles * g.nchunks * KT * BN * 2;
    g.xcd_remap = (pl.blocks % 8 == 0) ? 1 : 0;
    pl.ok = true;
    return pl;
}

template <typename T, int WN, int KT, int VW>
hipError_t run(const Conv2dArgs &a, const Plan &pl, const uint4 *wp)
{
    hipLaunchKernelGGL((igemm_fwd<T, WN, 2, KT, VW>), dim3((unsigned)pl.blocks), dim3(kThreads), pl.lds,
                       a.stream, (const T *)a.x, wp, (const T *)a.bias, (T *)a.y, pl.g);
    return hipGetLastError();
}

template <typename T, int WN, int KT>
hipError_t run_vw(const Conv2dArgs &a, const Plan &pl, const uint4 *wp)
{
    switch (pl.VW) {
    case 8: return run<T, WN, KT, 8>(a, pl, wp);
    case 4: return run<T, WN, KT, 4>(a, pl, wp);
    case 2: return run<T, WN, KT, 2>(a, pl, wp);
    default: return run<T, WN, KT, 1>(a, pl, wp);
    }
}

template <typename T, int WN>
hipError_t run_kt(const Conv2dArgs &a, const Plan &pl, const uint4 *wp)
{
    return pl.KT == 9 ? run_vw<T, WN, 9>(a, pl, wp) : run_vw<T, WN, 1>(a, pl, wp);
}

template <typename T>
hipError_t run_typed(const Conv2dArgs &a, const Plan &pl, const uint4 *wp)
{
    switch (pl.WN) {
    case 4: return run_kt<T, 4>(a, pl, wp);
    case 2: return run_kt<T, 2>(a, pl, wp);
    default: return run_kt<T, 1>(a, pl, wp);
    }
}

}  // namespace

bool igemm_supported(const Conv2dArgs &a) { return make_plan(a).ok; }

hipError_t launch_igemm(const Conv2dArgs &a, const char **kname)
{
    const Plan pl = make_plan(a);
    if (!pl.ok) return hipErrorInvalidValue;
    // Stream-ordered workspace for the packed filters: allocated and released on the
    // caller's stream, so calls on different streams never share it.
    uint4 *wp = nullptr;
    hipError_t err = hipMallocAsync((void **)&wp, (size_t)pl.packed_units * sizeof(uint4), a.stream);
    if (err != hipSuccess) return err;
    const int BN = pl.WN * 32;
    const int64_t tasks = pl.packed_units / pl.KT;   // (filter, octet) pairs
    const int64_t pblocks = ceil_div(tasks, kThreads);
    if (pl.KT == 9)
        hipLaunchKernelGGL(igemm_pack_filters<9>, dim3((unsigned)pblocks), dim3(kThreads), 0, a.stream,
                           (const uint16_t *)a.w, wp, tasks, pl.g.Ng, pl.g.Cg, BN, pl.g.n_tiles, pl.g.nchunks);
    else
        hipLaunchKernelGGL(igemm_pack_filters<1>, dim3((unsigned)pblocks), dim3(kThreads), 0, a.stream,
                           (const uint16_t *)a.w, wp, tasks, pl.g.Ng, pl.g.Cg, BN, pl.g.n_tiles, pl.g.nchunks);
    err = hipGetLastError();
    if (err == hipSuccess) {
        *kname = "igemm_fwd_mfma32x32x16";
        err = a.dtype == DT_F16 ? run_typed<_Float16>(a, pl, wp) : run_typed<__bf16>(a, pl, wp);
    }
    const hipError_t ferr = hipFreeAsync(wp, a.stream);
    return err != hipSuccess ? err : ferr;
}

}  // namespace gconv
