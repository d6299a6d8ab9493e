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
//    kernel copies it with plain 16-byte loads and stores;
//  * input: whole zero-padded input rows of the 16 channels, stored as
//    [row][col][16 channels] so that one MFMA fragment (8 consecutive channels at
//    one position) is a single 16-byte LDS read; loaded 8 positions at a time per
//    channel with buffer loads (out-of-range offsets read as zero, which provides
//    the padding rows), transposed in registers with v_perm.
// Epilogue: bias added in fp32, one rounding to the output dtype, the tile staged
// through LDS and written 16 bytes per lane along W.
#include <algorithm>
#include <mutex>
#include <vector>

#include "common.hpp"
#include "fastdiv.hpp"

namespace gconv {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kCK = 16;            // input channels per K chunk
constexpr int kLdsBudget = 160 * 1024;  // one workgroup per CU

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
    int P;               // N*OH*OW output positions (< 2^31)
    int m_tiles, n_tiles, groups, nchunks;
    int tiles, tiles_per_xcd;   // m_tiles*n_tiles*groups; ceil(tiles/8)
    int y_vec;           // 1: 8 consecutive positions of a channel are one aligned 16-byte run of y
    FastDiv fd_ohw, fd_ow, fd_hp, fd_nseg, fd_nr, fd_mt, fd_nt;
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

// Filter image: one block of 2*BN units per tap, each laid out by lds_unit over
// the filter index, so a tap's operand addresses are the tap-0 addresses plus a
// constant.
__device__ __forceinline__ int wimg_unit(int t, int BN, int n, int half) { return t * BN * 2 + lds_unit(n, half); }

constexpr uint32_t kOOB = 0x80000000u;  // byte offset past num_records: the load returns 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from global memory straight into LDS: lane l writes the LDS
// bytes [lds_byte + 16*l, +16).  Written as inline assembly so that the compiler
// does not treat it as an LDS store it must wait for before every later LDS read;
// the caller waits (vmcnt(0)) before the barrier that publishes the data.  lds_byte
// must be uniform over the wave.
__device__ __forceinline__ void dma16(const void *gbase, uint32_t voff, uint32_t lds_byte)
{
    // The global base and the LDS address are wave-uniform by construction; make
    // that explicit so both live in scalar registers as the instruction requires.
    // readfirstlane works on (signed) int: widen through uint32_t, never sign-extend.
    const uint64_t b = reinterpret_cast<uint64_t>(gbase);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const uint64_t bu = ((uint64_t)hi << 32) | (uint64_t)lo;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds_byte)), "v"(voff), "s"(bu)
                 : "memory");
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
                                             const uint32_t (*d)[DW])  // dummy: unit index relative to xs
{
    const uint4 val = make_uint4(col_pair<VW, v>(d[0], d[1]), col_pair<VW, v>(d[2], d[3]),
                                 col_pair<VW, v>(d[4], d[5]), col_pair<VW, v>(d[6], d[7]));
    const int s = slot0 + v;
    xs[(v < limit) ? lds_unit(s, octet) : dummy] = val;
    if constexpr (v + 1 < VW) write_octets<VW, DW, v + 1>(xs, slot0, octet, limit, dummy, d);
}


// Filters of one (group, filter tile, 16-channel chunk), laid out exactly as the
// kernel's LDS image (wimg_unit: per tap, two 16-byte channel octets per filter).
// One thread writes one 16-byte unit (consecutive threads, consecutive units): it
// inverts wimg_unit to find its (tap, filter, octet) and gathers the 8 channels of
// that octet.  Filters past Cout/g and channels past C/g are zero.
__global__ void __launch_bounds__(kThreads)
igemm_pack_filters(const uint16_t *__restrict__ w, uint4 *__restrict__ wp, int64_t units, int Ng, int Cg,
                   int KT, int BN, int n_tiles, int nchunks)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= units) return;
    const int per_chunk = KT * BN * 2;
    const int u = (int)(i % per_chunk);
    int64_t r = i / per_chunk;
    const int ch = (int)(r % nchunks); r /= nchunks;
    const int nt = (int)(r % n_tiles);
    const int k = (int)(r / n_tiles);
    // invert wimg_unit: unit u -> (tap t, filter nn, half)
    const int t = u / (BN * 2), ut = u % (BN * 2);
    const int row = ut >> 4;
    const int col = (ut & 15) ^ (row & 15);
    const int nn = row * 8 + (col >> 1), octet = col & 1;
    const int on = nt * BN + nn;
    uint32_t v[4] = {0, 0, 0, 0};
    if (on < Ng) {
        const uint16_t *src = w + ((int64_t)(k * Ng + on) * Cg) * KT + t;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = ch * kCK + octet * 8 + e;
            const uint32_t h = (c < Cg) ? src[(int64_t)c * KT] : 0u;
            v[e >> 1] |= h << (16 * (e & 1));
        }
    }
    wp[i] = make_uint4(v[0], v[1], v[2], v[3]);
}

// Workgroup: 4 waves, one per SIMD (the accumulators live in the matrix-core
// accumulator registers).  Wave w computes every filter of the tile for the
// positions SR*j + 2*w + mb.
constexpr int kWaves = 4;
constexpr int kIgThreads = kWaves * 64;
constexpr int kMaxXRounds = 1;   // input staging tasks per thread

template <typename T, int WN, int KT, int VW>
__global__ void __launch_bounds__(kIgThreads, 1)
igemm_fwd(const T *__restrict__ x, const uint4 *__restrict__ wp, const T *__restrict__ bias,
          T *__restrict__ y, IgemmGeom g)
{
    constexpr int WM = 2;                         // 32-position MFMA blocks per wave
    constexpr int BN = WN * 32;                   // filters per tile (all in every wave)
    constexpr int BM = 4 * WM * 32;               // positions per tile (256)
    constexpr int SR = BM / 32;                   // position stride between MFMA columns
    constexpr int DW = VW > 1 ? VW / 2 : 1;       // dwords per staged row segment
    constexpr int WCHUNK = KT * BN * 2;           // 16-byte units of one chunk's filters
    constexpr int EROWS = 64;                     // output channels per epilogue pass
    constexpr int CSTRIDE = BM + 8;               // padded epilogue LDS row (elements)
    extern __shared__ uint4 lds[];
    // LDS: two pipeline stages [input halo | filter image], one spare unit for
    // masked-off writes, then the epilogue staging area.
    const int XU = g.xslots * 2;
    const int SU = XU + WCHUNK;
    const int dummy = 2 * SU;
    T *ct = reinterpret_cast<T *>(lds + 2 * SU + 1);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave;
    const int half = lane >> 5, l32 = lane & 31;
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
    int xrr[kMaxXRounds], xsg[kMaxXRounds], xoct[kMaxXRounds], xslot0[kMaxXRounds], xlim[kMaxXRounds];
    bool xtask[kMaxXRounds];
#pragma unroll
    for (int i = 0; i < kMaxXRounds; ++i) {
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

    // Per-tile state: coordinates, the input buffer resource, this thread's input
    // offset (out of range for rows outside the image, which then read as zeros),
    // and the packed filters.
    struct TileState {
        int p0, n_first, R_lo, k, nt;
        __amdgpu_buffer_rsrc_t xr;
        uint32_t xvo[kMaxXRounds];
        const uint4 *wsrc;
    };
    auto tile_state = [&](int t) {
        TileState ts;
        const int bq = fdiv(t, g.fd_mt);
        const int mt = fmod_q(t, bq, g.fd_mt);
        ts.k = fdiv(bq, g.fd_nt);
        ts.nt = fmod_q(bq, ts.k, g.fd_nt);
        ts.p0 = mt * BM;
        ts.n_first = fdiv(ts.p0, g.fd_ohw);
        const int oh_first = fdiv(fmod_q(ts.p0, ts.n_first, g.fd_ohw), g.fd_ow);
        ts.R_lo = ts.n_first * g.Hp + oh_first * g.sh;
        ts.xr = make_rsrc(x + ((int64_t)ts.n_first * g.C + (int64_t)ts.k * g.Cg) * HW, 0x7fffffffu);
#pragma unroll
        for (int i = 0; i < kMaxXRounds; ++i) {
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
        ts.wsrc = wp + (int64_t)(ts.k * g.n_tiles + ts.nt) * g.nchunks * WCHUNK;
        return ts;
    };

    // Staging for one pipeline step: the filter image goes straight from global
    // memory into the stage buffer (dma16); 8 channel rows x VW input positions go
    // through registers, where they are transposed into channel octets.
    uint32_t d[kMaxXRounds][8][DW];
#define GCONV_LOAD_STEP(ts_, ch_, stage_)                                                    \
    do {                                                                                     \
        const uint4 *wc_ = (ts_).wsrc + (int64_t)(ch_) * WCHUNK;                             \
        const uint32_t wl_ = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint4 *)((stage_) + XU); \
        for (int u_ = wave * 64; u_ < WCHUNK; u_ += kIgThreads)                              \
            dma16(wc_ + u_, (uint32_t)lane * 16u, wl_ + (uint32_t)u_ * 16u);                  \
        const int ci0_ = (ch_) * kCK;                                                        \
        _Pragma("unroll") for (int r_ = 0; r_ < kMaxXRounds; ++r_) {                          \
            if (xtask[r_]) {                                                                 \
                _Pragma("unroll") for (int e_ = 0; e_ < 8; ++e_) {                           \
                    const bool ok_ = ci0_ + 8 * xoct[r_] + e_ < g.Cg;                        \
                    VecLoad<VW>::run((ts_).xr, ok_ ? (ts_).xvo[r_] : kOOB, (uint32_t)(ci0_ + e_) * HW * 2, \
                                     d[r_][e_]);                                              \
                }                                                                            \
            }                                                                                \
        }                                                                                    \
    } while (0)
#define GCONV_WRITE_STEP(stage_)                                                             \
    do {                                                                                     \
        _Pragma("unroll") for (int r_ = 0; r_ < kMaxXRounds; ++r_)                           \
            if (xtask[r_]) write_octets<VW, DW, 0>((stage_), xslot0[r_], xoct[r_], xlim[r_], \
                                                   dummy - (int)((stage_) - lds), d[r_]);     \
    } while (0)

    // Zero both halos once: padding columns are never written by the staging tasks.
    for (int i = tid; i < XU; i += kIgThreads) {
        lds[i] = make_uint4(0, 0, 0, 0);
        lds[SU + i] = make_uint4(0, 0, 0, 0);
    }
    TileState ts = tile_state(tile);
    __syncthreads();
    GCONV_LOAD_STEP(ts, 0, lds);
    GCONV_WRITE_STEP(lds);
    wait_vmem_all();
    __syncthreads();

    int stage = 0;
    for (;;) {
        // LDS slot of tap (0,0) for each of this lane's output positions.  Column j
        // of MFMA block mb of wave column wm is tile position SR*j + WM*wm + mb, so
        // the 16 lanes of a half-block read halo slots SR apart, which lds_unit
        // spreads over all 16 bank columns; the epilogue restores position order.
        int xslot[WM];
#pragma unroll
        for (int mb = 0; mb < WM; ++mb) {
            const int p = min(ts.p0 + SR * l32 + wm * WM + mb, g.P - 1);
            const int n = fdiv(p, g.fd_ohw);
            const int q = fmod_q(p, n, g.fd_ohw);
            const int oh = fdiv(q, g.fd_ow), ow = fmod_q(q, oh, g.fd_ow);
            xslot[mb] = (n * g.Hp + oh * g.sh - ts.R_lo) * g.WL + ow * g.sw;
        }
        f32x16 acc[WN][WM];
#pragma unroll
        for (int i = 0; i < WN; ++i)
#pragma unroll
            for (int j = 0; j < WM; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        const int next_tile = tile + nbx;
        const bool has_next_tile = next_tile < t_hi;
        TileState nts = ts;
        for (int ch = 0; ch < g.nchunks; ++ch) {
            uint4 *cur = lds + stage * SU;
            uint4 *nxt = lds + (stage ^ 1) * SU;
            // Fetch the next pipeline step (next chunk, or chunk 0 of the next tile)
            // into registers while this one computes.
            const bool last = ch + 1 == g.nchunks;
            const bool more = !last || has_next_tile;
            if (last && has_next_tile) nts = tile_state(next_tile);
            if (more) {
                // One load path: the source is (this tile, ch+1) or (next tile, 0).
                TileState src;
                src.xr = last ? nts.xr : ts.xr;
#pragma unroll
                for (int i = 0; i < kMaxXRounds; ++i) src.xvo[i] = last ? nts.xvo[i] : ts.xvo[i];
                src.wsrc = last ? nts.wsrc : ts.wsrc;
                GCONV_LOAD_STEP(src, last ? 0 : ch + 1, nxt);
            }
            const uint4 *xs = cur;
            const uint4 *ws = cur + XU;
            // Operand registers are double-buffered across taps: every LDS read of tap
            // t+1 is issued before the MFMAs of tap t (the scheduling fences keep the
            // compiler from folding the two buffers into one and waiting on each read).
            uint4 bf[2][WM], af[2][WN];
            auto read_tap = [&](int t, int buf) {
                const int kh = t / g.KW, kw = t - kh * g.KW;
                const int xoff = kh * g.dh * g.WL + kw * g.dw;
#pragma unroll
                for (int mb = 0; mb < WM; ++mb) bf[buf][mb] = xs[lds_unit(xslot[mb] + xoff, half)];
#pragma unroll
                for (int nb = 0; nb < WN; ++nb) af[buf][nb] = ws[wimg_unit(t, BN, nb * 32 + l32, half)];
            };
            read_tap(0, 0);
#pragma unroll
            for (int t = 0; t < KT; ++t) {
                const int c = t & 1;
                if (t + 1 < KT) read_tap(t + 1, c ^ 1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int nb = 0; nb < WN; ++nb)
#pragma unroll
                    for (int mb = 0; mb < WM; ++mb) acc[nb][mb] = Mfma<T>::run(af[c][nb], bf[c][mb], acc[nb][mb]);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (more) GCONV_WRITE_STEP(nxt);
            wait_vmem_all();  // the filter image of the next step has landed in LDS
            __syncthreads();
            stage ^= 1;
        }

        // ---- epilogue: + bias in fp32, one rounding to T, then through the LDS
        // staging area so that each thread stores 8 consecutive positions of one
        // output channel (16 bytes).  These stores drain while the next tile computes.
        const bool vec_ok = g.y_vec && (ts.p0 <= g.P - BM);
#pragma unroll
        for (int pass = 0; pass < BN / EROWS; ++pass) {
            if (pass > 0) __syncthreads();
#pragma unroll
            for (int nb = 0; nb < WN; ++nb) {
                const int nrow = nb * 32;             // tile row of this 32-filter block
                if (nrow / EROWS != pass) continue;
#pragma unroll
                for (int mb = 0; mb < WM; ++mb) {
                    const int pl = SR * l32 + wm * WM + mb;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int nl = nrow % EROWS + (r >> 2) * 8 + half * 4 + (r & 3);
                        const int on = ts.nt * BN + pass * EROWS + nl;
                        float v = acc[nb][mb][r];
                        if (bias && on < g.Ng) v += to_f32(bias[ts.k * g.Ng + on]);
                        ct[nl * CSTRIDE + pl] = from_f32<T>(v);
                    }
                }
            }
            __syncthreads();
            for (int c = tid; c < EROWS * (BM / 8); c += kIgThreads) {
                const int row = c / (BM / 8), p8 = c % (BM / 8);
                const int on = ts.nt * BN + pass * EROWS + row;
                const int p = ts.p0 + p8 * 8;
                if (on >= g.Ng || p >= g.P) continue;
                const int co = ts.k * g.Ng + on;
                const T *src = ct + row * CSTRIDE + p8 * 8;
                if (vec_ok) {
                    const int n = fdiv(p, g.fd_ohw);
                    const int q = fmod_q(p, n, g.fd_ohw);
                    *reinterpret_cast<uint4 *>(y + ((int64_t)n * g.Cout + co) * OHW + q) =
                        *reinterpret_cast<const uint4 *>(src);
                } else {
                    for (int e = 0; e < 8 && p + e < g.P; ++e) {
                        const int n = fdiv(p + e, g.fd_ohw);
                        const int q = fmod_q(p + e, n, g.fd_ohw);
                        y[((int64_t)n * g.Cout + co) * OHW + q] = src[e];
                    }
                }
            }
        }
        if (!has_next_tile) break;
        tile = next_tile;
        ts = nts;
    }
}
#undef GCONV_LOAD_STEP
#undef GCONV_WRITE_STEP

struct Plan {
    IgemmGeom g;
    int WN, WM, KT, VW;
    size_t lds;
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
    const int64_t P = a.N * a.OH * a.OW;
    if (P >= (int64_t(1) << 31) || a.N * (int64_t)g.Hp + a.KH * (int64_t)a.dh + 512 >= (int64_t(1) << 31)) return pl;
    g.P = (int)P;
    g.groups = (int)a.groups;
    const int64_t KT = a.KH * a.KW;
    if (KT != 1 && KT != 9) return pl;
    pl.KT = (int)KT;
    pl.WN = g.Ng > 64 ? 4 : 2;                       // 32-filter blocks per wave (= per tile)
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
    if (xtasks > (int64_t)kMaxXRounds * kIgThreads) return pl;
    g.xtasks = (int)xtasks;
    // Byte offsets of the staged input, relative to one tile's first image, stay below 2^31.
    const int64_t HW = (int64_t)g.H * g.W;
    if ((crossings + 1) * (int64_t)g.C * HW * 2 >= (int64_t(1) << 31)) return pl;
    // Two pipeline stages + spare unit + epilogue staging area (64 rows of BM+8 16-bit).
    pl.lds = (size_t)(2 * ((int64_t)g.xslots * 2 + KT * BN * 2) + 1) * sizeof(uint4) + (size_t)64 * (BM + 8) * 2;
    if (pl.lds > (size_t)kLdsBudget) return pl;
    g.y_vec = ((int64_t)g.OH * g.OW) % 8 == 0 && (reinterpret_cast<uintptr_t>(a.y) & 15) == 0;
    g.m_tiles = (int)ceil_div(g.P, BM);
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
    pl.packed_units = (int64_t)g.groups * g.n_tiles * g.nchunks * KT * BN * 2;
    pl.ok = true;
    return pl;
}

template <typename T, int WN, int KT, int VW>
hipError_t run(const Conv2dArgs &a, const Plan &pl, const uint4 *wp)
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
    return pl.WN == 4 ? run_kt<T, 4>(a, pl, wp) : run_kt<T, 2>(a, pl, wp);
}

}  // namespace

bool igemm_supported(const Conv2dArgs &a) { return make_plan(a).ok; }

namespace {

// Packed-filter workspace, one buffer per (device, stream): calls on one stream are
// ordered, so they can share a buffer; calls on different streams never do.  A
// buffer only grows, after the stream has drained the work that used it.
struct Workspace {
    int device;
    hipStream_t stream;
    void *ptr;
    size_t bytes;
};
std::mutex g_ws_mutex;
std::vector<Workspace> g_ws;

hipError_t workspace(hipStream_t stream, size_t bytes, void **out)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    for (Workspace &w : g_ws) {
        if (w.device != dev || w.stream != stream) continue;
        if (w.bytes >= bytes) {
            *out = w.ptr;
            return hipSuccess;
        }
        err = hipStreamSynchronize(stream);
        if (err != hipSuccess) return err;
        err = hipFree(w.ptr);
        if (err != hipSuccess) return err;
        w.ptr = nullptr;
        w.bytes = 0;
        err = hipMalloc(&w.ptr, bytes);
        if (err != hipSuccess) return err;
        w.bytes = bytes;
        *out = w.ptr;
        return hipSuccess;
    }
    Workspace w{dev, stream, nullptr, 0};
    err = hipMalloc(&w.ptr, bytes);
    if (err != hipSuccess) return err;
    w.bytes = bytes;
    g_ws.push_back(w);
    *out = w.ptr;
    return hipSuccess;
}

}  // namespace

hipError_t launch_igemm(const Conv2dArgs &a, const char **kname)
{
    const Plan pl = make_plan(a);
    if (!pl.ok) return hipErrorInvalidValue;
    void *wsp = nullptr;
    hipError_t err = workspace(a.stream, (size_t)pl.packed_units * sizeof(uint4), &wsp);
    if (err != hipSuccess) return err;
    uint4 *wp = static_cast<uint4 *>(wsp);
    const int BN = pl.WN * 32;
    hipLaunchKernelGGL(igemm_pack_filters, dim3((unsigned)ceil_div(pl.packed_units, kThreads)), dim3(kThreads), 0,
                       a.stream, (const uint16_t *)a.w, wp, pl.packed_units, pl.g.Ng, pl.g.Cg, pl.KT, BN,
                       pl.g.n_tiles, pl.g.nchunks);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    *kname = "igemm_fwd_mfma32x32x16";
    return a.dtype == DT_F16 ? run_typed<_Float16>(a, pl, wp) : run_typed<__bf16>(a, pl, wp);
}

}  // namespace gconv
