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
// Tile: one workgroup = 4 waves computes BN = WN*32 output channels of one group
// x BM = 512 consecutive output positions (flattened over n, oh, ow, so a tile may
// span image boundaries).  Waves 0-1 take the first 256 positions, waves 2-3 the
// second 256; within its half, wave w owns the positions 8j + 4*(w&1) + mb for
// j < 32 and mb < 4.  Every wave computes all BN channels for its 128 positions:
// WN x 4 blocks of v_mfma_f32_32x32x16_{f16,bf16}, filters as the A operand
// (rows = output channels), the im2col tile as the B operand (columns =
// positions).  Per tap a wave reads WN + 4 operand fragments for 4*WN MFMAs, and
// the lanes of a fragment read halo slots 8 apart, which the LDS map below keeps
// free of bank conflicts.
//
// K loop: input channels in chunks of 16, then taps; one MFMA step = one tap x
// 16 channels.  Chunk c+1 is loaded into registers while chunk c computes:
//  * filters: the chunk's 16 channels x KH*KW taps of one filter are one contiguous
//    run of w; consecutive lanes load consecutive 16-byte pieces of the tile's runs
//    (a wave reads a few whole runs, not one piece of 64 runs), and each element is
//    written with a 2-byte LDS store to its place in the tap-major image, where one
//    16-byte unit is 8 channels of one filter at one tap;
//  * input: whole zero-padded input rows of the 16 channels, stored as
//    [row][col][16 channels] so that one MFMA fragment (8 consecutive channels at
//    one position) is a single 16-byte LDS read; loaded VW positions at a time per
//    channel with buffer loads (out-of-range offsets read as zero, which provides
//    the padding rows), transposed in registers with v_perm.
// Epilogue: the bias is the accumulators' initial value (fp32); one rounding to
// the output dtype; the tile is staged through LDS and written 16 bytes per lane
// along W, while the next tile's first chunk is still in flight.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "fastdiv.hpp"

namespace gconv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kCK = 16;                  // input channels per K chunk
constexpr int kLdsBudget = 160 * 1024;   // one workgroup per CU
constexpr int kWaves = 4;
constexpr int kIgThreads = kWaves * 64;
constexpr int kWM = 4;                   // 32-position MFMA blocks per wave
constexpr int kBM = 512;                 // positions per tile
constexpr int kCStride = kBM + 8;        // epilogue LDS row, in elements

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

// 16-bit storage <-> fp32 bits.
template <typename T> __device__ __forceinline__ float half_bits_to_f32(uint32_t h);
template <> __device__ __forceinline__ float half_bits_to_f32<_Float16>(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
template <> __device__ __forceinline__ float half_bits_to_f32<__bf16>(uint32_t h)
{
    return __builtin_bit_cast(float, h << 16);
}
// Two fp32 values rounded (to nearest even) into one dword of T, a in the low half:
// one v_cvt_pk_{f16,bf16}_f32.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<_Float16>(float a, float b)
{
    return __builtin_bit_cast(uint32_t, f16x2{(_Float16)a, (_Float16)b});
}
template <> __device__ __forceinline__ uint32_t pack2<__bf16>(float a, float b)
{
    return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
}

// Copy of one accumulator (held in an accumulation register) into a VGPR, at this
// point of the program: without it the register allocator moves every accumulator
// into VGPRs at once when the K loop ends, which does not fit.
__device__ __forceinline__ float acc_read(float v)
{
    float r;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(v));
    return r;
}

struct IgemmGeom {
    int N, C, H, W, Cout, Cg, Ng, OH, OW, KH, KW;
    int sh, sw, ph, pw, dh, dw;
    int Hp;              // H + 2*ph: height of one zero-padded image in the virtual row space
    int NR, WL;          // LDS halo: rows, columns (padded coordinates)
    int xslots;          // NR*WL rounded up to a multiple of 8
    int padl, npad;      // halo columns left of the image; all halo columns outside it
    int nseg;            // W / VW: vector segments per input row
    int xtasks;          // 2 channel octets * NR * nseg
    int P;               // N*OH*OW output positions (< 2^31)
    int m_tiles, n_tiles, groups, nchunks;
    int tiles, tiles_per_xcd;   // m_tiles*n_tiles*groups; ceil(tiles/8)
    int y_vec;           // 1: 8 consecutive positions of a channel are one aligned 16-byte run of y
    int defer;           // 1: outputs staged in their own LDS area, stored during the next tile
    int ocs, okg;        // output channel of filter j of group k: j*ocs + k*okg (grouped: 1, Ng;
                         // interleaved: groups, 1)
    uint32_t w_bytes, b_bytes;
    FastDiv fd_ohw, fd_ow, fd_hp, fd_nseg, fd_nr, fd_mt, fd_nt;
};

// LDS placement of the 16-byte half `half` (channels 0-7 or 8-15) of 32-byte slot
// `s`, in 16-byte units: slots in order, with one spare unit after every 8 slots.
// The LDS has 64 banks of 4 bytes, so a 16-byte access by 16 lanes is conflict-free
// when the lanes hit 16 distinct units modulo 16.  Slots 8 apart are 17 units apart,
// so 16 such slots land on 16 different units modulo 16; slots 4 apart alternate
// between +8 and +9.  The hot patterns are of those kinds: the staging writes (one
// slot per row segment of 8 or 4) and the MFMA operand reads (lanes own positions 8
// apart).  Reading a tap's operand costs an add, a shift and a multiply-add.
__device__ __forceinline__ int lds_unit(int s, int half) { return 2 * s + half + (s >> 3); }
// 16-byte units of a halo of `slots` slots (a multiple of 8).
__host__ __device__ inline int halo_units(int slots) { return 2 * slots + slots / 8; }

// Filter image: per tap, two planes (channels 0-7, then 8-15 of the chunk) of one
// unit per filter, so that a tap's operand addresses are the tap-0 addresses plus a
// constant.  The A-operand reads (32 consecutive filters of one plane) are
// conflict-free.  The planes are BN + 4 units apart and the taps 2(BN + 4) + 1: with
// these strides the 2-byte staging writes of a wave (about 3.5 filters x 16 channels
// x 9 taps, each element to its (tap, channel) place) hit each bank at most twice,
// against four times with unpadded planes and one spare unit per tap.
template <int BN> constexpr int kPlaneUnits = BN + 4;
template <int BN> constexpr int kTapUnits = 2 * kPlaneUnits<BN> + 1;

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
// slot slot0+v (or to the spare unit when v >= limit).
template <int VW, int DW, int v>
__device__ __forceinline__ void write_octets(uint4 *xs, int slot0, int octet, int limit, int dummy,
                                             const uint32_t (*d)[DW])  // dummy: unit index relative to xs
{
    const uint4 val = make_uint4(col_pair<VW, v>(d[0], d[1]), col_pair<VW, v>(d[2], d[3]),
                                 col_pair<VW, v>(d[4], d[5]), col_pair<VW, v>(d[6], d[7]));
    const int s = slot0 + v;
    xs[(v < limit) ? lds_unit(s, octet) : dummy] = val;
    if constexpr (v + 1 < VW) write_octets<VW, DW, v + 1>(xs, slot0, octet, limit, dummy, d);
}

// Writes the filter pieces a thread loaded into the chunk's filter image (wimg, in
// bytes).  Piece i belongs to filter ff0 + FPT*i of the tile; wdst[u] is the image
// offset of its element u for filter ff0 (the filter adds 16 bytes per step).  With
// KT = 1 a piece is one whole unit; otherwise its 8 elements go to 8 (tap, channel)
// places, 2 bytes each.
template <int KT, int BN, int NI, int FPT>
__device__ __forceinline__ void write_filter_pieces(char *wimg, const uint32_t *wdst, int ff0,
                                                    const uint32_t *wr)
{
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        if (i + 1 < NI || ff0 + FPT * i < BN) {
            if constexpr (KT == 1) {
                *reinterpret_cast<uint4 *>(wimg + wdst[0] + 16 * FPT * i) =
                    make_uint4(wr[4 * i], wr[4 * i + 1], wr[4 * i + 2], wr[4 * i + 3]);
            } else {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t dw = wr[4 * i + (u >> 1)];
                    *reinterpret_cast<uint16_t *>(wimg + wdst[u] + 16 * FPT * i) =
                        (uint16_t)((u & 1) ? (dw >> 16) : dw);
                }
            }
        }
    }
}

template <typename T, int WN, int KT, int VW>
__global__ void __launch_bounds__(kIgThreads, 1)
igemm_fwd(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
          T *__restrict__ y, IgemmGeom g)
{
    constexpr int BN = WN * 32;                   // filters per tile (all in every wave)
    constexpr int DW = VW > 1 ? VW / 2 : 1;       // dwords per staged row segment
    constexpr int XR = 4 / DW;                    // input staging tasks per thread (<= 32 dwords)
    constexpr int TSU = kTapUnits<BN>;            // 16-byte units per tap of the filter image
    constexpr int BP = kPlaneUnits<BN>;           // 16-byte units between its two channel planes
    constexpr int WCHUNK = KT * TSU;              // 16-byte units of one chunk's filters
    extern __shared__ uint4 lds[];
    // LDS: two pipeline stages [input halo | filter image] and one spare unit for
    // masked-off writes.  Between tiles the epilogue reuses the whole area.
    const int XU = halo_units(g.xslots);
    const int SU = XU + WCHUNK;
    const int dummy = 2 * SU;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    // Tile position of column l32 of this wave's MFMA block 0 (block mb adds mb).
    const int pbase = 256 * (wave >> 1) + 8 * l32 + 4 * (wave & 1);
    const int OHW = g.OH * g.OW;
    const int HW = g.H * g.W;

    // Persistent tile loop.  Workgroups are dealt round-robin to the 8 XCDs, so
    // workgroup b runs on XCD b % 8; that XCD owns a contiguous range of tiles and its
    // workgroups walk it together (tile = start + r + i*nbx), so the tiles in flight
    // on one XCD are neighbours that share halo rows and filters in its L2.
    const int xcd = blockIdx.x & 7, rank = blockIdx.x >> 3;
    const int nbx = ((int)gridDim.x - xcd + 7) >> 3;
    const int t_lo = xcd * g.tiles_per_xcd;
    const int t_hi = min(t_lo + g.tiles_per_xcd, g.tiles);
    int tile = t_lo + rank;
    if (tile >= t_hi) return;  // uniform over the workgroup

    // Tile-independent part of this thread's input staging tasks: (channel octet,
    // halo row rr, segment sg) -> VW positions of 8 channels; task i of the thread is
    // tid + i*kIgThreads.
    int xrr[XR], xsg[XR], xoct[XR], xslot0[XR], xlim[XR];
    bool xtask[XR];
#pragma unroll
    for (int i = 0; i < XR; ++i) {
        const int tk = tid + i * kIgThreads;
        xtask[i] = tk < g.xtasks;
        xrr[i] = xsg[i] = xoct[i] = xslot0[i] = xlim[i] = 0;
        if (xtask[i]) {
            const int rest = fdiv(tk, g.fd_nseg);
            xsg[i] = fmod_q(tk, rest, g.fd_nseg);
            xoct[i] = fdiv(rest, g.fd_nr);
            xrr[i] = fmod_q(rest, xoct[i], g.fd_nr);
            const int c0 = xsg[i] * VW + g.pw;        // LDS column of the segment's first element
            xslot0[i] = xrr[i] * g.WL + c0;
            xlim[i] = min(VW, g.WL - c0);             // elements that land inside the halo
        }
    }
    // Filter staging.  A chunk's filters are BN runs of 16*KT contiguous elements of
    // w (16 channels x KT taps, channel-major), 2*KT pieces of 16 bytes each; piece fj
    // of a run holds elements 8fj .. 8fj+7.  Consecutive lanes load consecutive
    // pieces, so a wave's loads cover a few contiguous runs.  Thread tid takes piece
    // fj = tid % (2KT) of filters ff0 + FPT*i (ff0 = tid / (2KT), i < NI).
    constexpr int PPF = 2 * KT;                   // pieces per filter run
    constexpr int FPT = kIgThreads / PPF;         // filters per step
    constexpr int NI = (BN + FPT - 1) / FPT;      // steps
    const int fj = tid % PPF, ff0 = tid / PPF;
    const bool fact = ff0 < FPT;                  // the last kIgThreads % PPF threads idle
    // Image offset (bytes) of element u of this thread's piece of filter ff0: element
    // e = 8fj + u is channel e / KT at tap e % KT.
    uint32_t wdst[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int e = 8 * fj + u, c = e / KT, t = e - c * KT;
        wdst[u] = (uint32_t)(((t * TSU + (c >> 3) * BP + ff0) * 16) + (c & 7) * 2);
    }
    const __amdgpu_buffer_rsrc_t wr_rsrc = make_rsrc(w, g.w_bytes);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(bias, g.b_bytes);

    // Halo offset of each tap, in slots (wave-uniform).
    int xoff[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        const int kh = t / g.KW, kw = t - kh * g.KW;
        xoff[t] = kh * g.dh * g.WL + kw * g.dw;
    }
    // Filter-image unit of this lane's A fragment of block nb at tap 0.
    int fu[WN];
#pragma unroll
    for (int nb = 0; nb < WN; ++nb) fu[nb] = half * BP + nb * 32 + l32;

    // Per-tile state: coordinates, the input buffer resource, this thread's input
    // offset (out of range for rows outside the image, which then read as zeros),
    // and its filter offset (out of range for filters past Cout/g).
    struct TileState {
        int p0, n_first, R_lo, k, nt;
        int nf;   // filters of the tile that exist (BN, or fewer in the last n-tile)
        __amdgpu_buffer_rsrc_t xr;
        uint32_t xvo[XR];
        uint32_t wvo;
    };
    auto tile_state = [&](int t) {
        TileState ts;
        const int bq = fdiv(t, g.fd_mt);
        const int mt = fmod_q(t, bq, g.fd_mt);
        ts.k = fdiv(bq, g.fd_nt);
        ts.nt = fmod_q(bq, ts.k, g.fd_nt);
        ts.p0 = mt * kBM;
        ts.n_first = fdiv(ts.p0, g.fd_ohw);
        const int oh_first = fdiv(fmod_q(ts.p0, ts.n_first, g.fd_ohw), g.fd_ow);
        ts.R_lo = ts.n_first * g.Hp + oh_first * g.sh;
        ts.xr = make_rsrc(x + ((int64_t)ts.n_first * g.C + (int64_t)ts.k * g.Cg) * HW, 0x7fffffffu);
#pragma unroll
        for (int i = 0; i < XR; ++i) {
            ts.xvo[i] = kOOB;
            if (xtask[i]) {
                const int R = ts.R_lo + xrr[i];
                const int n = fdiv(R, g.fd_hp);
                const int ih = fmod_q(R, n, g.fd_hp) - g.ph;
                if (n < g.N && ih >= 0 && ih < g.H)
                    ts.xvo[i] = (uint32_t)((((int64_t)(n - ts.n_first) * g.C + 8 * xoct[i]) * HW +
                                            (int64_t)ih * g.W + xsg[i] * VW) * 2);
            }
        }
        ts.nf = min(BN, g.Ng - ts.nt * BN);
        ts.wvo = fact ? (uint32_t)(((ts.k * g.Ng + ts.nt * BN + ff0) * g.Cg) * KT * 2 + 16 * fj) : kOOB;
        return ts;
    };
    // Bias of this lane's accumulator rows: rows nb*32 + 8q + 4*half + (0..3) are
    // one 8-byte load (Cout/g is a multiple of 4 when there is a bias).
    auto load_bias = [&](const TileState &ts, uint2 (&bz)[WN][4]) {
#pragma unroll
        for (int nb = 0; nb < WN; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int on = ts.nt * BN + nb * 32 + 8 * q + 4 * half;
                const uint32_t off = on < g.Ng ? (uint32_t)((ts.k * g.Ng + on) * 2) : kOOB;
                bz[nb][q] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(b_rsrc, off, 0, 0));
            }
    };

    // Staging for one pipeline step: 8 channel rows x VW input positions per input
    // task and one filter octet per filter task go to registers, then (after the
    // current step's MFMAs) are transposed into the stage's LDS layout.
    uint32_t d[XR][8][DW];
    uint32_t wr[NI * 4];
    // Staging loads.  In the K loop they are issued one or two at a time between
    // the MFMAs of the taps (all at once, the memory pipeline would stall the wave).
    // Threads without a task load zeros from an out-of-range offset, so there are no
    // branches around the loads.
    constexpr int NXL = XR * 8;                   // input loads per step
    constexpr int LW = KT > 1 ? (KT + 1) / 2 : 1;  // taps over which a step's loads are spread
    auto load_x = [&](const TileState &s, int ch, int j) {   // task j/8, channel j%8
        const int r = j >> 3, e = j & 7;
        const int ci0 = ch * kCK;
        const bool ok = ci0 + 8 * xoct[r] + e < g.Cg;
        VecLoad<VW>::run(s.xr, ok ? s.xvo[r] : kOOB, (uint32_t)(ci0 + e) * HW * 2, d[r][e]);
    };
    auto load_w = [&](const TileState &s, int ch, int i) {   // piece of filter ff0 + FPT*i
        const int ci0 = ch * kCK;
        // The filter exists, and the piece lies in channels < C/g (C/g is a multiple
        // of 8, so a last chunk of 8 channels holds exactly the pieces fj < KT).
        const bool ok = ff0 + FPT * i < s.nf && (fj < KT || ci0 + kCK <= g.Cg);
        const uint4 u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
            wr_rsrc, ok ? s.wvo : kOOB, (uint32_t)((FPT * i * g.Cg + ci0) * KT * 2), 0));
        wr[4 * i] = u.x; wr[4 * i + 1] = u.y; wr[4 * i + 2] = u.z; wr[4 * i + 3] = u.w;
    };
    // The staged registers count as read here in every thread, also where a task is
    // off: otherwise the compiler finds their loads still pending later on and waits
    // for every outstanding memory operation before it reuses those registers.
    auto consume_staging = [&]() {
#pragma unroll
        for (int r = 0; r < XR; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int k = 0; k < DW; ++k) asm volatile("" ::"v"(d[r][e][k]));
#pragma unroll
        for (int i = 0; i < NI * 4; ++i) asm volatile("" ::"v"(wr[i]));
    };
#define GCONV_WRITE_STEP(stage_)                                                             \
    do {                                                                                     \
        _Pragma("unroll") for (int r_ = 0; r_ < XR; ++r_)                                    \
            if (xtask[r_]) write_octets<VW, DW, 0>((stage_), xslot0[r_], xoct[r_], xlim[r_], \
                                                   dummy - (int)((stage_) - lds), d[r_]);     \
        if (fact)                                                                            \
            write_filter_pieces<KT, BN, NI, FPT>(reinterpret_cast<char *>((stage_) + XU),     \
                                                 wdst, ff0, wr);                             \
        consume_staging();                                                                   \
    } while (0)

    // Halo columns outside the image (left/right padding) are never written by the
    // staging tasks; they are zeroed at the start and after every epilogue, which
    // reuses the LDS.
    auto zero_pads = [&](int st) {
        for (int j = tid; j < g.NR * g.npad; j += kIgThreads) {
            const int row = j / g.npad, pc = j - row * g.npad;
            const int col = pc < g.padl ? pc : pc - g.padl + g.pw + g.W;
            const int s = row * g.WL + col;
            lds[st * SU + lds_unit(s, 0)] = make_uint4(0, 0, 0, 0);
            lds[st * SU + lds_unit(s, 1)] = make_uint4(0, 0, 0, 0);
        }
    };

    // Deferred output stores (64-filter tiles whose staged outputs fit in LDS next to
    // the two stages): a tile's outputs wait in their own LDS area and are stored
    // while the next tile computes, a few per tap ahead of that tap's loads, so the
    // output stream overlaps the MFMAs instead of stalling every CU at once.
    constexpr bool kCanDefer = WN == 2;
    constexpr int kDefItems = BN * (kBM / 8) / kIgThreads;   // 16-byte stores per thread per tile
    // 16-byte unit of the staged outputs: their own area after the stages, or the
    // start of the LDS (then the items are read but never stored, as none is pending).
    const int ctu = g.defer ? 2 * SU + 1 : 0;
    int dnext = kDefItems;                                  // nothing pending before the first tile
    int64_t dy = 0;                                         // this thread's output offset, row 0
    int drow0 = 0, dlimit = 0;                              // its first row; rows < dlimit are valid
    // Two items at a time: read from LDS with one tap's operands, stored after that
    // tap's MFMAs, when the reads have long landed.
    auto fetch_deferred = [&](int u) {   // item dnext + u (an in-range row past the end)
        const T *dct = reinterpret_cast<const T *>(lds + ctu);
        const int row = drow0 + 4 * min(dnext + u, kDefItems - 1);
        return *reinterpret_cast<const uint4 *>(dct + row * kCStride + (tid & 63) * 8);
    };
    auto put_deferred = [&](int u, uint4 v) {
        const int row = drow0 + 4 * (dnext + u);
        if (dnext + u < kDefItems && row < dlimit)
            store_nt(reinterpret_cast<uint4 *>(y + dy + (int64_t)row * g.ocs * OHW), v);
    };

    for (int i = tid; i < XU; i += kIgThreads) {
        lds[i] = make_uint4(0, 0, 0, 0);
        lds[SU + i] = make_uint4(0, 0, 0, 0);
    }
    TileState ts = tile_state(tile);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NXL; ++j) load_x(ts, 0, j);
#pragma unroll
    for (int i = 0; i < NI; ++i) load_w(ts, 0, i);
    GCONV_WRITE_STEP(lds);
    __syncthreads();

    int stage = 0;
    for (;;) {
        // LDS slot of tap (0,0) for each of this lane's output positions.
        int xslot[kWM];
#pragma unroll
        for (int mb = 0; mb < kWM; ++mb) {
            const int p = min(ts.p0 + pbase + mb, g.P - 1);
            const int n = fdiv(p, g.fd_ohw);
            const int q = fmod_q(p, n, g.fd_ohw);
            const int oh = fdiv(q, g.fd_ow), ow = fmod_q(q, oh, g.fd_ow);
            xslot[mb] = (n * g.Hp + oh * g.sh - ts.R_lo) * g.WL + ow * g.sw;
        }
        f32x16 acc[WN][kWM];
#pragma unroll
        for (int nb = 0; nb < WN; ++nb)
#pragma unroll
            for (int mb = 0; mb < kWM; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;

        const int next_tile = tile + nbx;
        const bool has_next_tile = next_tile < t_hi;
        TileState nts = ts;
        uint2 bz[WN][4];
        int ch = 0;
        do {  // nchunks >= 1
            const uint4 *cur = lds + stage * SU;
            uint4 *nxt = lds + (stage ^ 1) * SU;
            // Fetch the next pipeline step (next chunk, or chunk 0 of the next tile)
            // into registers while this one computes.
            const bool last = ch + 1 == g.nchunks;
            const bool more = !last || has_next_tile;
            if (last && has_next_tile) nts = tile_state(next_tile);
            // Source of the next pipeline step: (this tile, ch+1) or (next tile, 0);
            // after the last chunk of the last tile the loads fetch nothing.
            TileState src;
            src.xr = last ? nts.xr : ts.xr;
#pragma unroll
            for (int i = 0; i < XR; ++i) src.xvo[i] = !more ? kOOB : last ? nts.xvo[i] : ts.xvo[i];
            src.wvo = !more ? kOOB : last ? nts.wvo : ts.wvo;
            src.nf = last ? nts.nf : ts.nf;
            const int nch = last ? 0 : ch + 1;
            const uint4 *xs = cur;
            const uint4 *ws = cur + XU;
            // Re-derive the tap addresses in every chunk instead of keeping all
            // KT x kWM of them live across the loop.
            int xsl[kWM];
#pragma unroll
            for (int mb = 0; mb < kWM; ++mb) {
                xsl[mb] = xslot[mb];
                asm volatile("" : "+v"(xsl[mb]));
            }
            // Operand registers are double-buffered across taps: the LDS reads of tap
            // t+1 are issued among the MFMAs of tap t (the scheduling groups and fences
            // keep the compiler from folding the two buffers into one and waiting on
            // each read).
            uint4 bf[2][kWM], af[2][WN];
            auto read_tap = [&](int t, int buf) {
#pragma unroll
                for (int mb = 0; mb < kWM; ++mb) bf[buf][mb] = xs[lds_unit(xsl[mb] + xoff[t], half)];
#pragma unroll
                for (int nb = 0; nb < WN; ++nb) af[buf][nb] = ws[t * TSU + fu[nb]];
            };
            read_tap(0, 0);
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const int c = t & 1;
                if (t + 1 < KT) read_tap(t + 1, c ^ 1);
                // The loads go out during the first LW taps, so the last ones have the
                // remaining taps to arrive before they are staged.
                uint4 dv0, dv1;
                if (t < LW) {
                    if (kCanDefer) {
                        dv0 = fetch_deferred(0);
                        dv1 = fetch_deferred(1);
                    }
#pragma unroll
                    for (int j = t * NXL / LW; j < (t + 1) * NXL / LW; ++j) load_x(src, nch, j);
#pragma unroll
                    for (int i = t * NI / LW; i < (t + 1) * NI / LW; ++i) load_w(src, nch, i);
                    // 64-filter tiles: the bias goes out with the last chunk's last loads.
                    if (kCanDefer && t == LW - 1 && last && bias) load_bias(ts, bz);
                }
#pragma unroll
                for (int nb = 0; nb < WN; ++nb)
#pragma unroll
                    for (int mb = 0; mb < kWM; ++mb) acc[nb][mb] = Mfma<T>::run(af[c][nb], bf[c][mb], acc[nb][mb]);
                // Issue order of the tap: each MFMA is followed by one LDS read, a few
                // vector ALU instructions and one global load of the operands to come,
                // which then run while the matrix core works (one wave per SIMD leaves
                // nothing else to fill those cycles).
#pragma unroll
                for (int i = 0; i < WN * kWM; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
                }
                __builtin_amdgcn_sched_barrier(0);
                if (kCanDefer && t < LW) {
                    put_deferred(0, dv0);
                    put_deferred(1, dv1);
                    dnext = min(dnext + 2, kDefItems);
                }
            }
            if (!last) {
                GCONV_WRITE_STEP(nxt);
                __syncthreads();
                stage ^= 1;
            }
        } while (++ch < g.nchunks);

        // ---- epilogue: + bias in fp32, one rounding to T, then through LDS so that
        // each thread stores 8 consecutive positions of one output channel (16 bytes).
        // The next tile's first chunk is still in registers; it is staged afterwards.
        if (kCanDefer && g.defer)   // the rest of the previous tile
            for (; dnext < kDefItems; ++dnext) put_deferred(0, fetch_deferred(0));
        __syncthreads();   // every wave is done with the operands of the last chunk
        if (!kCanDefer && bias) load_bias(ts, bz);
        T *ct = reinterpret_cast<T *>(lds + (kCanDefer ? ctu : 0));
        // Converted 16 accumulators at a time (the fences stop the scheduler from
        // moving every accumulator into VGPRs at once), two per packed conversion;
        // the bias add is compiled only into the loop that has a bias.
        auto write_ct = [&](auto has_bias) {
#pragma unroll
            for (int nb = 0; nb < WN; ++nb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if ((r & 3) == 0) __builtin_amdgcn_sched_barrier(0);
                    const int row = nb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                    float v0 = acc_read(acc[nb][0][r]), v1 = acc_read(acc[nb][1][r]);
                    float v2 = acc_read(acc[nb][2][r]), v3 = acc_read(acc[nb][3][r]);
                    if constexpr (decltype(has_bias)::value) {
                        const uint32_t dw = (r & 2) ? bz[nb][r >> 2].y : bz[nb][r >> 2].x;
                        const float b0 = half_bits_to_f32<T>((r & 1) ? (dw >> 16) : (dw & 0xffffu));
                        v0 += b0; v1 += b0; v2 += b0; v3 += b0;
                    }
                    *reinterpret_cast<uint2 *>(ct + row * kCStride + pbase) =
                        make_uint2(pack2<T>(v0, v1), pack2<T>(v2, v3));
                }
            __builtin_amdgcn_sched_barrier(0);
        };
        if (bias)
            write_ct(std::true_type{});
        else
            write_ct(std::false_type{});
        if (kCanDefer && g.defer && has_next_tile) {
            // Stage the next tile's first chunk (its loads were issued during the last
            // chunk) and leave this tile's outputs for the next tile's taps.
            GCONV_WRITE_STEP(lds + (stage ^ 1) * SU);
            __syncthreads();
            const int p = ts.p0 + (tid & 63) * 8;
            dnext = 0;
            drow0 = tid >> 6;
            dlimit = p < g.P ? min(BN, g.Ng - ts.nt * BN) : 0;
            const int n = fdiv(min(p, g.P - 1), g.fd_ohw);
            const int q = fmod_q(min(p, g.P - 1), n, g.fd_ohw);
            dy = ((int64_t)n * g.Cout + ts.k * g.okg + ts.nt * BN * g.ocs) * OHW + q;
            stage ^= 1;
            tile = next_tile;
            ts = nts;
            continue;
        }
        // The next step's loads (issued during the last chunk) have landed by now.
        // Waiting for them here, before any store is issued, keeps the staging after
        // the stores from waiting for the stores to drain (the counter is in order).
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        __syncthreads();
        if (g.y_vec) {
            // A thread stores the same 8 positions (one 16-byte run of y) of every
            // kRowStep-th filter row, so the position arithmetic is done once.
            constexpr int kRowStep = kIgThreads / (kBM / 8);
            const int p = ts.p0 + (tid % (kBM / 8)) * 8;
            const int nrow = p < g.P ? min(BN, g.Ng - ts.nt * BN) : 0;
            const int n = fdiv(min(p, g.P - 1), g.fd_ohw);
            const int q = fmod_q(min(p, g.P - 1), n, g.fd_ohw);
            T *yp = y + ((int64_t)n * g.Cout + ts.k * g.okg + ts.nt * BN * g.ocs) * OHW + q;
            const int64_t ystep = (int64_t)g.ocs * OHW;   // between consecutive filters
            const T *cp = ct + (tid % (kBM / 8)) * 8;
#pragma unroll 4
            for (int row = tid / (kBM / 8); row < nrow; row += kRowStep)
                store_nt(reinterpret_cast<uint4 *>(yp + row * ystep),
                         *reinterpret_cast<const uint4 *>(cp + row * kCStride));
        } else {
            for (int c = tid; c < BN * (kBM / 8); c += kIgThreads) {
                const int row = c / (kBM / 8), p8 = c % (kBM / 8);
                const int on = ts.nt * BN + row;
                const int p = ts.p0 + p8 * 8;
                if (on >= g.Ng || p >= g.P) continue;
                const int co = on * g.ocs + ts.k * g.okg;
                const T *srcp = ct + row * kCStride + p8 * 8;
                for (int e = 0; e < 8 && p + e < g.P; ++e) {
                    const int n = fdiv(p + e, g.fd_ohw);
                    const int q = fmod_q(p + e, n, g.fd_ohw);
                    y[((int64_t)n * g.Cout + co) * OHW + q] = srcp[e];
                }
            }
        }
        if (!has_next_tile) break;
        __syncthreads();   // the staged outputs have been read
        zero_pads(0);
        zero_pads(1);
        GCONV_WRITE_STEP(lds + (stage ^ 1) * SU);
        __syncthreads();
        stage ^= 1;
        tile = next_tile;
        ts = nts;
    }
}
#undef GCONV_WRITE_STEP

struct Plan {
    IgemmGeom g;
    int WN, KT, VW;
    size_t lds;
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
    const int64_t P = a.N * a.OH * a.OW;
    if (P >= (int64_t(1) << 31) || a.N * (int64_t)g.Hp + a.KH * (int64_t)a.dh + 1024 >= (int64_t(1) << 31)) return pl;
    g.P = (int)P;
    g.groups = (int)a.groups;
    const int64_t KT = a.KH * a.KW;
    if (KT != 1 && KT != 9) return pl;
    pl.KT = (int)KT;
    // Filters: 8-channel octets of one filter are contiguous runs of 16*KT bytes.
    if (g.Cg % 8 != 0 || (reinterpret_cast<uintptr_t>(a.w) & 15) != 0) return pl;
    const int64_t w_bytes = a.Cout * (int64_t)g.Cg * KT * 2;
    if (w_bytes >= (int64_t(1) << 31)) return pl;
    g.w_bytes = (uint32_t)w_bytes;
    // Bias: 4 consecutive filters per 8-byte load.
    g.b_bytes = 0;
    if (a.bias) {
        if (g.Ng % 4 != 0 || (reinterpret_cast<uintptr_t>(a.bias) & 7) != 0) return pl;
        g.b_bytes = (uint32_t)(a.Cout * 2);
    }
    pl.WN = g.Ng > 64 ? 4 : 2;                       // 32-filter blocks per wave (= per tile)
    const int BN = pl.WN * 32;
    // Vector width of the input row loads.
    const uintptr_t xa = reinterpret_cast<uintptr_t>(a.x);
    pl.VW = (g.W % 8 == 0 && xa % 16 == 0) ? 8 : (g.W % 4 == 0 && xa % 8 == 0) ? 4
          : (g.W % 2 == 0 && xa % 4 == 0) ? 2 : 1;
    const int DW = pl.VW > 1 ? pl.VW / 2 : 1;
    const int XR = 4 / DW;
    // Virtual output rows one tile can touch, image boundaries inside them, and
    // the resulting bound on the virtual padded input rows of its halo (never more
    // than all N*Hp of them).
    const bool aligned_rows = kBM % g.OW == 0;
    const int64_t V = aligned_rows ? kBM / g.OW : (kBM - 1) / g.OW + 2;
    const int64_t crossings = (V <= 1) ? 0 : ((aligned_rows && g.OH % (kBM / g.OW) == 0) ? 0 : (V - 2) / g.OH + 1);
    const int64_t gap = std::max<int64_t>(0, (int64_t)g.Hp - (int64_t)g.OH * g.sh);
    int64_t NR = (V - 1) * g.sh + crossings * gap + (int64_t)(g.KH - 1) * g.dh + 1;
    NR = std::min<int64_t>(NR, a.N * (int64_t)g.Hp);
    const int64_t WL = (int64_t)(g.OW - 1) * g.sw + (int64_t)(g.KW - 1) * g.dw + 1;
    if (NR * WL >= (int64_t(1) << 24)) return pl;
    g.NR = (int)NR; g.WL = (int)WL;
    g.xslots = (int)((NR * WL + 7) / 8 * 8);
    g.padl = (int)std::min<int64_t>(g.pw, WL);
    g.npad = g.padl + (int)std::max<int64_t>(0, WL - g.pw - g.W);
    g.nseg = (g.W + pl.VW - 1) / pl.VW;
    const int64_t xtasks = 2 * NR * g.nseg;
    if (xtasks > (int64_t)XR * kIgThreads) return pl;
    g.xtasks = (int)xtasks;
    // Byte offsets of the staged input, relative to one tile's first image, stay below 2^31.
    const int64_t HW = (int64_t)g.H * g.W;
    if ((crossings + 1) * (int64_t)g.C * HW * 2 >= (int64_t(1) << 31)) return pl;
    // Two pipeline stages + spare unit; the epilogue reuses the same area.
    const size_t stage_bytes = (size_t)((int64_t)halo_units(g.xslots) + KT * (2 * (BN + 4) + 1)) * sizeof(uint4);
    pl.lds = 2 * stage_bytes + sizeof(uint4);
    if (pl.lds > (size_t)kLdsBudget) return pl;
    g.ocs = a.interleaved ? g.groups : 1;
    g.okg = a.interleaved ? 1 : g.Ng;
    g.y_vec = ((int64_t)g.OH * g.OW) % 8 == 0 && (reinterpret_cast<uintptr_t>(a.y) & 15) == 0;
    const size_t ct_bytes = (size_t)BN * kCStride * 2;      // staged outputs of one tile
    g.defer = pl.WN == 2 && g.y_vec && pl.lds + ct_bytes <= (size_t)kLdsBudget;
    // Deferred stores: the outputs get their own area after the stages; otherwise
    // the epilogue reuses the whole area.
    pl.lds = g.defer ? pl.lds + ct_bytes : std::max(pl.lds, ct_bytes);
    if (pl.lds > (size_t)kLdsBudget) return pl;
    g.m_tiles = (int)ceil_div(g.P, kBM);
    g.n_tiles = (int)ceil_div(g.Ng, BN);
    g.nchunks = (int)ceil_div(g.Cg, kCK);
    const int64_t tiles = (int64_t)g.m_tiles * g.n_tiles * g.groups;
    if (tiles >= (int64_t(1) << 31)) return pl;
    g.tiles = (int)tiles;
    g.tiles_per_xcd = (int)ceil_div(tiles, 8);
    g.fd_ohw = make_fastdiv((uint32_t)(g.OH * g.OW));
    g.fd_ow = make_fastdiv((uint32_t)g.OW);
    g.fd_hp = make_fastdiv((uint32_t)g.Hp);
    g.fd_nseg = make_fastdiv((uint32_t)g.nseg);
    g.fd_nr = make_fastdiv((uint32_t)g.NR);
    g.fd_mt = make_fastdiv((uint32_t)g.m_tiles);
    g.fd_nt = make_fastdiv((uint32_t)g.n_tiles);
    pl.ok = true;
    return pl;
}

template <typename T, int WN, int KT, int VW>
hipError_t run(const Conv2dArgs &a, const Plan &pl)
{
    // Dynamic LDS beyond 64 KB must be allowed explicitly, once per kernel.
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&igemm_fwd<T, WN, KT, VW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget);
    if (attr != hipSuccess) return attr;
    // Persistent grid: one workgroup per CU (the LDS footprint allows no more).
    int dev = 0, cus = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    const int64_t blocks = std::min<int64_t>(pl.g.tiles, std::max(cus, 8));
    hipLaunchKernelGGL((igemm_fwd<T, WN, KT, VW>), dim3((unsigned)blocks), dim3(kIgThreads), pl.lds,
                       a.stream, (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, pl.g);
    return hipGetLastError();
}

template <typename T, int WN, int KT>
hipError_t run_vw(const Conv2dArgs &a, const Plan &pl)
{
    switch (pl.VW) {
    case 8: return run<T, WN, KT, 8>(a, pl);
    case 4: return run<T, WN, KT, 4>(a, pl);
    case 2: return run<T, WN, KT, 2>(a, pl);
    default: return run<T, WN, KT, 1>(a, pl);
    }
}

template <typename T, int WN>
hipError_t run_kt(const Conv2dArgs &a, const Plan &pl)
{
    return pl.KT == 9 ? run_vw<T, WN, 9>(a, pl) : run_vw<T, WN, 1>(a, pl);
}

template <typename T>
hipError_t run_typed(const Conv2dArgs &a, const Plan &pl)
{
    return pl.WN == 4 ? run_kt<T, 4>(a, pl) : run_kt<T, 2>(a, pl);
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
