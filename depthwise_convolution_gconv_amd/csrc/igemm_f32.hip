// igemm_f32.hip -- implicit-GEMM grouped conv2d (NCHW) for fp32 tensors on the
// gfx950 matrix cores: v_mfma_f32_32x32x2_f32, fp32 products and fp32
// accumulation.  The discuss.pytorch.org thread "F.conv2d runs x15 slower in
// mixed-precision/half-precision mode" times the same layer in fp32 (O0) and in
// fp16; this is the fp32 half of that pair on the matrix cores.
//
// The tiling is the one of igemm.hip (workgroup = 4 waves, BN = WN*32 filters of one
// group x 512 consecutive output positions, each wave all BN filters x 128
// positions in 4 x WN accumulator blocks, persistent XCD-aware tile walk, two LDS
// stages with the next step's loads spread over the first taps).  What differs:
//  * a K chunk is 8 input channels, so one 32-byte LDS slot holds the 8 fp32
//    channels of one position as two 16-byte units, unit h = channels 4h..4h+3;
//  * one MFMA consumes 2 channels.  Its k-step s (0..3) pairs channel s (lanes
//    0-31) with channel 4+s (lanes 32-63), so a lane's operand for all four
//    k-steps of a tap is element s of one 16-byte LDS read;
//  * filters: the chunk's 8 channels x KH*KW taps of one filter are one contiguous
//    run of w; consecutive lanes load consecutive 16-byte pieces of the tile's runs,
//    and each float is written with a 4-byte LDS store to its (tap, channel) place
//    in the image of quad units;
//  * the epilogue stages 64 output channels at a time in fp32.
#include <algorithm>

#include "common.hpp"
#include "fastdiv.hpp"

namespace gconv {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kCK = 8;                   // input channels per K chunk
constexpr int kLdsBudget = 160 * 1024;   // one workgroup per CU
constexpr int kThreads = 256;            // 4 waves
constexpr int kWM = 4;                   // 32-position MFMA blocks per wave
constexpr int kBM = 512;                 // positions per tile
constexpr int kERows = 64;               // output channels per epilogue pass
constexpr int kCStride = kBM + 4;        // epilogue LDS row, in floats
constexpr uint32_t kOOB = 0x80000000u;   // byte offset past num_records: the load returns 0

struct GeomF32 {
    int N, C, H, W, Cout, Cg, Ng, OH, OW, KH, KW;
    int sh, sw, ph, pw, dh, dw;
    int Hp;              // H + 2*ph: height of one zero-padded image in the virtual row space
    int NR, WL;          // LDS halo: rows, columns (padded coordinates)
    int xslots;          // NR*WL rounded up to a multiple of 8
    int padl, npad;      // halo columns left of the image; all halo columns outside it
    int nseg;            // W / VW: vector segments per input row
    int xtasks;          // NR * nseg
    int P;               // N*OH*OW output positions (< 2^31)
    int m_tiles, n_tiles, groups, nchunks;
    int tiles, tiles_per_xcd;
    int y_vec;           // 1: 4 consecutive positions of a channel are one aligned 16-byte run of y
    int ocs, okg;        // output channel of filter j of group k: j*ocs + k*okg (grouped: 1, Ng;
                         // interleaved: groups, 1)
    uint32_t w_bytes, b_bytes;
    FastDiv fd_ohw, fd_ow, fd_hp, fd_nseg, fd_mt, fd_nt;
};

// Same LDS map as the 16-bit kernel: 16-byte unit `half` of 32-byte slot `s`, slots
// in order with one spare unit after every 8 slots, so that 16 slots 8 apart (or 4
// apart) hit 16 different bank groups.
__device__ __forceinline__ int lds_unit(int s, int half) { return 2 * s + half + (s >> 3); }
// 16-byte units of a halo of `slots` slots (a multiple of 8).
__host__ __device__ inline int halo_units_f32(int slots) { return 2 * slots + slots / 8; }

// Filter image: per tap, two planes of BN units (channels 0-3, then 4-7 of the
// chunk), one unit per filter, and one spare unit that staggers the taps across the
// banks for the 4-byte staging writes.  The A-operand reads (32 consecutive filters)
// are conflict-free.
template <int BN> constexpr int kTapUnitsF32 = 2 * BN + 1;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// One accumulator copied out of the accumulation registers at this point of the
// program (otherwise all of them are copied into VGPRs when the K loop ends).
__device__ __forceinline__ float acc_read(float v)
{
    float r;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(v));
    return r;
}

// VW consecutive floats.
template <int VW> struct VecLoadF32;
template <> struct VecLoadF32<4> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so, float *d)
    {
        const f32x4 u = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0));
        d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w;
    }
};
template <> struct VecLoadF32<2> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so, float *d)
    {
        const uint2 u = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0));
        d[0] = __builtin_bit_cast(float, u.x); d[1] = __builtin_bit_cast(float, u.y);
    }
};
template <> struct VecLoadF32<1> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so, float *d)
    {
        d[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0));
    }
};

template <int WN, int KT, int VW>
__global__ void __launch_bounds__(kThreads, 1)
igemm_fwd_f32(const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
              float *__restrict__ y, GeomF32 g)
{
    constexpr int BN = WN * 32;                   // filters per tile (all in every wave)
    constexpr int XR = 4 / VW;                    // input staging tasks per thread (<= 32 floats)
    constexpr int TSU = kTapUnitsF32<BN>;         // 16-byte units per tap of the filter image
    constexpr int WCHUNK = KT * TSU;              // 16-byte units of one chunk's filters
    extern __shared__ uint4 lds[];
    const int XU = halo_units_f32(g.xslots);
    const int SU = XU + WCHUNK;
    const int dummy = 2 * SU;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    // Tile position of column l32 of this wave's MFMA block 0 (block mb adds mb).
    const int pbase = 256 * (wave >> 1) + 8 * l32 + 4 * (wave & 1);
    const int OHW = g.OH * g.OW;
    const int HW = g.H * g.W;

    // Persistent, XCD-aware tile walk (see igemm.hip).
    const int xcd = blockIdx.x & 7, rank = blockIdx.x >> 3;
    const int nbx = ((int)gridDim.x - xcd + 7) >> 3;
    const int t_lo = xcd * g.tiles_per_xcd;
    const int t_hi = min(t_lo + g.tiles_per_xcd, g.tiles);
    int tile = t_lo + rank;
    if (tile >= t_hi) return;  // uniform over the workgroup

    // Input staging tasks: (halo row rr, segment sg) -> VW positions x 8 channels.
    int xrr[XR], xsg[XR], xslot0[XR], xlim[XR];
    bool xtask[XR];
#pragma unroll
    for (int i = 0; i < XR; ++i) {
        const int tk = tid + i * kThreads;
        xtask[i] = tk < g.xtasks;
        xrr[i] = xsg[i] = xslot0[i] = xlim[i] = 0;
        if (xtask[i]) {
            xrr[i] = fdiv(tk, g.fd_nseg);
            xsg[i] = fmod_q(tk, xrr[i], g.fd_nseg);
            const int c0 = xsg[i] * VW + g.pw;
            xslot0[i] = xrr[i] * g.WL + c0;
            xlim[i] = min(VW, g.WL - c0);
        }
    }
    // Filter staging.  A chunk's filters are BN runs of 8*KT contiguous floats of w
    // (8 channels x KT taps, channel-major), 2*KT pieces of 16 bytes each; piece fj of
    // a run holds elements 4fj .. 4fj+3.  Consecutive lanes load consecutive pieces,
    // so a wave's loads cover a few contiguous runs.  Thread tid takes piece
    // fj = tid % (2KT) of filters ff0 + FPT*i (ff0 = tid / (2KT), i < NI).
    constexpr int PPF = 2 * KT;                   // pieces per filter run
    constexpr int FPT = kThreads / PPF;           // filters per step
    constexpr int NI = (BN + FPT - 1) / FPT;      // steps
    const int fj = tid % PPF, ff0 = tid / PPF;
    const bool fact = ff0 < FPT;                  // the last kThreads % PPF threads idle
    // Image offset (bytes) of element u of this thread's piece of filter ff0: element
    // e = 4fj + u is channel e / KT at tap e % KT.
    uint32_t wdst[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = 4 * fj + u, c = e / KT, t = e - c * KT;
        wdst[u] = (uint32_t)(((t * TSU + (c >> 2) * BN + ff0) * 16) + (c & 3) * 4);
    }
    const __amdgpu_buffer_rsrc_t wr_rsrc = make_rsrc(w, g.w_bytes);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(bias, g.b_bytes);

    int xoff[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        const int kh = t / g.KW, kw = t - kh * g.KW;
        xoff[t] = kh * g.dh * g.WL + kw * g.dw;
    }
    int fu[WN];
#pragma unroll
    for (int nb = 0; nb < WN; ++nb) fu[nb] = half * BN + nb * 32 + l32;

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
                    ts.xvo[i] = (uint32_t)((((int64_t)(n - ts.n_first) * g.C) * HW + (int64_t)ih * g.W +
                                            xsg[i] * VW) * 4);
            }
        }
        ts.nf = min(BN, g.Ng - ts.nt * BN);
        ts.wvo = fact ? (uint32_t)(((ts.k * g.Ng + ts.nt * BN + ff0) * g.Cg) * KT * 4 + 16 * fj) : kOOB;
        return ts;
    };

    // Staging registers: 8 channel rows x VW positions per input task, and NI
    // filter pieces of 4 floats.
    float d[XR][8][VW];
    float wr[4 * NI];
    constexpr int NXL = XR * 8;
    constexpr int LW = KT > 1 ? (KT + 1) / 2 : 1;
    auto load_x = [&](const TileState &s, int ch, int j) {   // task j/8, channel j%8
        const int r = j >> 3, e = j & 7;
        const int ci0 = ch * kCK;
        const bool ok = ci0 + e < g.Cg;
        VecLoadF32<VW>::run(s.xr, ok ? s.xvo[r] : kOOB, (uint32_t)(ci0 + e) * HW * 4, d[r][e]);
    };
    auto load_w = [&](const TileState &s, int ch, int i) {   // piece of filter ff0 + FPT*i
        const int ci0 = ch * kCK;
        // The filter exists, and the piece lies in channels < C/g (C/g is a multiple
        // of 4, so a last chunk of 4 channels holds exactly the pieces fj < KT).
        const bool ok = ff0 + FPT * i < s.nf && (fj < KT || ci0 + kCK <= g.Cg);
        const f32x4 u = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
            wr_rsrc, ok ? s.wvo : kOOB, (uint32_t)((FPT * i * g.Cg + ci0) * KT * 4), 0));
        wr[4 * i] = u.x; wr[4 * i + 1] = u.y; wr[4 * i + 2] = u.z; wr[4 * i + 3] = u.w;
    };
    auto write_step = [&](uint4 *st) {
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            if (!xtask[r]) continue;
#pragma unroll
            for (int v = 0; v < VW; ++v) {
                const int s = xslot0[r] + v;
                const bool in = v < xlim[r];
                st[in ? lds_unit(s, 0) : dummy - (int)(st - lds)] =
                    __builtin_bit_cast(uint4, f32x4{d[r][0][v], d[r][1][v], d[r][2][v], d[r][3][v]});
                st[in ? lds_unit(s, 1) : dummy - (int)(st - lds)] =
                    __builtin_bit_cast(uint4, f32x4{d[r][4][v], d[r][5][v], d[r][6][v], d[r][7][v]});
            }
        }
        if (fact) {
            // Piece i goes to filter ff0 + FPT*i (16 bytes further per step); with
            // KT = 1 it is one whole unit, otherwise 4 (tap, channel) places.
            char *wimg = reinterpret_cast<char *>(st + XU);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                if (i + 1 < NI || ff0 + FPT * i < BN) {
                    if constexpr (KT == 1) {
                        *reinterpret_cast<f32x4 *>(wimg + wdst[0] + 16 * FPT * i) =
                            f32x4{wr[4 * i], wr[4 * i + 1], wr[4 * i + 2], wr[4 * i + 3]};
                    } else {
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            *reinterpret_cast<float *>(wimg + wdst[u] + 16 * FPT * i) = wr[4 * i + u];
                    }
                }
            }
        }
        // The staged registers count as read here in every thread, also where a task
        // is off: otherwise the compiler finds their loads still pending later on and
        // waits for every outstanding memory operation before it reuses them.
#pragma unroll
        for (int r = 0; r < XR; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int v = 0; v < VW; ++v) asm volatile("" ::"v"(d[r][e][v]));
#pragma unroll
        for (int i = 0; i < 4 * NI; ++i) asm volatile("" ::"v"(wr[i]));
    };
    auto zero_pads = [&](int st) {
        for (int j = tid; j < g.NR * g.npad; j += kThreads) {
            const int row = j / g.npad, pc = j - row * g.npad;
            const int col = pc < g.padl ? pc : pc - g.padl + g.pw + g.W;
            const int s = row * g.WL + col;
            lds[st * SU + lds_unit(s, 0)] = make_uint4(0, 0, 0, 0);
            lds[st * SU + lds_unit(s, 1)] = make_uint4(0, 0, 0, 0);
        }
    };

    for (int i = tid; i < XU; i += kThreads) {
        lds[i] = make_uint4(0, 0, 0, 0);
        lds[SU + i] = make_uint4(0, 0, 0, 0);
    }
    TileState ts = tile_state(tile);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NXL; ++j) load_x(ts, 0, j);
#pragma unroll
    for (int i = 0; i < NI; ++i) load_w(ts, 0, i);
    write_step(lds);
    __syncthreads();

    int stage = 0;
    for (;;) {
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
        int ch = 0;
        do {  // nchunks >= 1
            const uint4 *cur = lds + stage * SU;
            uint4 *nxt = lds + (stage ^ 1) * SU;
            const bool last = ch + 1 == g.nchunks;
            const bool more = !last || has_next_tile;
            if (last && has_next_tile) nts = tile_state(next_tile);
            TileState src;
            src.xr = last ? nts.xr : ts.xr;
#pragma unroll
            for (int i = 0; i < XR; ++i) src.xvo[i] = !more ? kOOB : last ? nts.xvo[i] : ts.xvo[i];
            src.wvo = !more ? kOOB : last ? nts.wvo : ts.wvo;
            src.nf = last ? nts.nf : ts.nf;
            const int nch = last ? 0 : ch + 1;
            const uint4 *xs = cur;
            const uint4 *ws = cur + XU;
            int xsl[kWM];
#pragma unroll
            for (int mb = 0; mb < kWM; ++mb) {
                xsl[mb] = xslot[mb];
                asm volatile("" : "+v"(xsl[mb]));
            }
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
                if (t < LW) {
#pragma unroll
                    for (int j = t * NXL / LW; j < (t + 1) * NXL / LW; ++j) load_x(src, nch, j);
#pragma unroll
                    for (int i = t * NI / LW; i < (t + 1) * NI / LW; ++i) load_w(src, nch, i);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int nb = 0; nb < WN; ++nb)
#pragma unroll
                        for (int mb = 0; mb < kWM; ++mb)
                            acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                __builtin_bit_cast(f32x4, af[c][nb])[s], __builtin_bit_cast(f32x4, bf[c][mb])[s],
                                acc[nb][mb], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (!last) {
                write_step(nxt);
                __syncthreads();
                stage ^= 1;
            }
        } while (++ch < g.nchunks);

        // ---- epilogue: + bias, then through LDS, kERows output channels per pass,
        // so that each thread stores 4 consecutive positions of one output channel.
        __syncthreads();   // every wave is done with the operands of the last chunk
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): the next step's loads, before any store
        float *ct = reinterpret_cast<float *>(lds);
        for (int pass = 0; pass < (BN + kERows - 1) / kERows; ++pass) {
            if (pass > 0) __syncthreads();   // the previous pass has been read
#pragma unroll
            for (int nb = 0; nb < WN; ++nb) {
                if ((nb * 32) / kERows != pass) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    __builtin_amdgcn_sched_barrier(0);
                    const int row0 = nb * 32 + q * 8 + half * 4;   // rows row0 .. row0+3
                    f32x4 bv = {0.0f, 0.0f, 0.0f, 0.0f};
                    if (bias) {
                        const int on = ts.nt * BN + row0;
                        const uint32_t off = on < g.Ng ? (uint32_t)((ts.k * g.Ng + on) * 4) : kOOB;
                        bv = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, off, 0, 0));
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = q * 4 + e;
                        const f32x4 v = {acc_read(acc[nb][0][r]) + bv[e], acc_read(acc[nb][1][r]) + bv[e],
                                         acc_read(acc[nb][2][r]) + bv[e], acc_read(acc[nb][3][r]) + bv[e]};
                        *reinterpret_cast<f32x4 *>(ct + (row0 + e - pass * kERows) * kCStride + pbase) = v;
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            const int rows = min(kERows, BN - pass * kERows);
            for (int c = tid; c < rows * (kBM / 4); c += kThreads) {
                const int row = c / (kBM / 4), p4 = c % (kBM / 4);
                const int on = ts.nt * BN + pass * kERows + row;
                const int p = ts.p0 + p4 * 4;
                if (on >= g.Ng || p >= g.P) continue;
                const int co = on * g.ocs + ts.k * g.okg;
                const float *srcp = ct + row * kCStride + p4 * 4;
                if (g.y_vec) {
                    const int n = fdiv(p, g.fd_ohw);
                    const int q = fmod_q(p, n, g.fd_ohw);
                    store_nt(reinterpret_cast<uint4 *>(y + ((int64_t)n * g.Cout + co) * OHW + q),
                             *reinterpret_cast<const uint4 *>(srcp));
                } else {
                    for (int e = 0; e < 4 && p + e < g.P; ++e) {
                        const int n = fdiv(p + e, g.fd_ohw);
                        const int q = fmod_q(p + e, n, g.fd_ohw);
                        y[((int64_t)n * g.Cout + co) * OHW + q] = srcp[e];
                    }
                }
            }
        }
        if (!has_next_tile) break;
        __syncthreads();   // the staged outputs have been read
        zero_pads(0);
        zero_pads(1);
        write_step(lds + (stage ^ 1) * SU);
        __syncthreads();
        stage ^= 1;
        tile = next_tile;
        ts = nts;
    }
}

struct PlanF32 {
    GeomF32 g;
    int WN, KT, VW;
    size_t lds;
    bool ok;
};

PlanF32 make_plan_f32(const Conv2dArgs &a)
{
    PlanF32 pl{};
    pl.ok = false;
    if (a.dtype != DT_F32) return pl;
    GeomF32 &g = pl.g;
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
    // Filters: 4-channel quads of one filter are contiguous 16-byte aligned runs.
    if (g.Cg % 4 != 0 || (reinterpret_cast<uintptr_t>(a.w) & 15) != 0) return pl;
    const int64_t w_bytes = a.Cout * (int64_t)g.Cg * KT * 4;
    if (w_bytes >= (int64_t(1) << 31)) return pl;
    g.w_bytes = (uint32_t)w_bytes;
    g.b_bytes = 0;
    if (a.bias) {
        if (g.Ng % 4 != 0 || (reinterpret_cast<uintptr_t>(a.bias) & 15) != 0) return pl;
        g.b_bytes = (uint32_t)(a.Cout * 4);
    }
    pl.WN = g.Ng > 64 ? 4 : 2;
    const int BN = pl.WN * 32;
    const uintptr_t xa = reinterpret_cast<uintptr_t>(a.x);
    pl.VW = (g.W % 4 == 0 && xa % 16 == 0) ? 4 : (g.W % 2 == 0 && xa % 8 == 0) ? 2 : 1;
    const int XR = 4 / pl.VW;
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
    const int64_t xtasks = NR * g.nseg;
    if (xtasks > (int64_t)XR * kThreads) return pl;
    g.xtasks = (int)xtasks;
    const int64_t HW = (int64_t)g.H * g.W;
    if ((crossings + 1) * (int64_t)g.C * HW * 4 >= (int64_t(1) << 31)) return pl;
    const size_t stage_bytes = (size_t)((int64_t)halo_units_f32(g.xslots) + KT * (2 * BN + 1)) * sizeof(uint4);
    pl.lds = std::max(2 * stage_bytes + sizeof(uint4), (size_t)kERows * kCStride * sizeof(float));
    if (pl.lds > (size_t)kLdsBudget) return pl;
    g.y_vec = ((int64_t)g.OH * g.OW) % 4 == 0 && (reinterpret_cast<uintptr_t>(a.y) & 15) == 0;
    g.ocs = a.interleaved ? (int)a.groups : 1;
    g.okg = a.interleaved ? 1 : g.Ng;
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
    g.fd_mt = make_fastdiv((uint32_t)g.m_tiles);
    g.fd_nt = make_fastdiv((uint32_t)g.n_tiles);
    pl.ok = true;
    return pl;
}

template <int WN, int KT, int VW>
hipError_t run_f32(const Conv2dArgs &a, const PlanF32 &pl)
{
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&igemm_fwd_f32<WN, KT, VW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget);
    if (attr != hipSuccess) return attr;
    int dev = 0, cus = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    const int64_t blocks = std::min<int64_t>(pl.g.tiles, std::max(cus, 8));
    hipLaunchKernelGGL((igemm_fwd_f32<WN, KT, VW>), dim3((unsigned)blocks), dim3(kThreads), pl.lds, a.stream,
                       (const float *)a.x, (const float *)a.w, (const float *)a.bias, (float *)a.y, pl.g);
    return hipGetLastError();
}

template <int WN, int KT>
hipError_t run_f32_vw(const Conv2dArgs &a, const PlanF32 &pl)
{
    switch (pl.VW) {
    case 4: return run_f32<WN, KT, 4>(a, pl);
    case 2: return run_f32<WN, KT, 2>(a, pl);
    default: return run_f32<WN, KT, 1>(a, pl);
    }
}

template <int WN>
hipError_t run_f32_kt(const Conv2dArgs &a, const PlanF32 &pl)
{
    return pl.KT == 9 ? run_f32_vw<WN, 9>(a, pl) : run_f32_vw<WN, 1>(a, pl);
}

}  // namespace

bool igemm_f32_supported(const Conv2dArgs &a) { return make_plan_f32(a).ok; }

hipError_t launch_igemm_f32(const Conv2dArgs &a, const char **kname)
{
    const PlanF32 pl = make_plan_f32(a);
    if (!pl.ok) return hipErrorInvalidValue;
    *kname = "igemm_fwd_f32_mfma32x32x2";
    return pl.WN == 4 ? run_f32_kt<4>(a, pl) : run_f32_kt<2>(a, pl);
}

}  // namespace gconv
