// igemm_defer.hip -- implicit-GEMM grouped conv2d (NCHW, 3x3 filters, unit column
// stride and dilation, 16-bit) for 33 to 64 filters per group, on the gfx950
// matrix cores, with each tile's output stores deferred into the next tile.
//
// The product is the one of igemm_rows.hip (per group k, Y_k = W_k * A_k over
// kk = (input channel, tap), A_k the group's im2col matrix, never written out; the
// discuss.pytorch.org thread "F.conv2d runs x15 slower in mixed-precision/
// half-precision mode" on grouped fp16 convs missing the tensor cores, and the
// functorch issue "Batching rules for ensembles" whose model ensembles folded into
// groups have few filters per group).  What differs:
//
// Runs of 4 columns.  A lane owns a run of 4 consecutive output columns and MFMA
// block mb < 4 computes column mb of the 32 runs of a wave; a filter row's 12 B
// operands come from a window of 6 positions.  Rows of 28 columns are then 7 whole
// runs.
//
// Tile: 64 filters (2 blocks of 32, all in every wave) x 128 runs (4 waves of 32),
// 128 fp32 accumulators per lane, and two accumulator sets.  Tile t accumulates in
// set t % 2 while the 32 output stores per lane of tile t-1 (set (t-1) % 2, one
// rounding; the bias seeds the accumulators) are issued between the MFMAs of tile
// t's first chunk.  With 32 channels per group a tile is 2 chunks of 16 channels,
// and its stores (as many bytes as a whole chunk of MFMA time can write) would
// otherwise run with the matrix cores idle.
//
// Vector memory counts loads and stores in one in-order counter, so every wait for
// a load also waits for the stores issued before it.  All the global loads of the
// first chunk (the next tile's filters, both chunks, and input rows) are issued
// before its stores, and what later waits for them does not wait for the stores:
// the filters are copied raw into LDS buffers of their own (chunk 0's, and chunk
// 1's in one of two by tile parity) and transposed into the filter images during
// the chunks: the next tile's chunk 0 during this tile's chunk 1, a tile's chunk 1
// during its chunk 0.
//
// Input staging as in igemm_rows.hip (two halo stages, the rows of step c+2 loaded
// into registers during chunk c and written during chunk c+1).  The halo keeps 9
// units per 4 columns (8 channel pairs and a spare), so consecutive runs are 9 units
// apart and 16 runs read by a half-wave hit 16 different units modulo 16.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "fastdiv.hpp"

namespace gconv {
namespace {

#include "rows_common.hpp"

constexpr int kThreads = 256;
constexpr int kRun = 4;                          // output columns per run
constexpr int kWin = kRun + 2;                   // window positions of one filter row
constexpr int kSub = 320;                        // units of a 16-filter half-block (288 + padding)
constexpr int kBlk = 2 * kSub;                   // a 32-filter block
constexpr int kFU = 2 * kBlk;                    // filter units per image: 64 filters
constexpr int kHU = (kLdsUnits - 5 * kFU) / 2;   // halo units per stage (2 images, 3 raw buffers)
constexpr int kRT = 128;                         // runs per tile: 4 waves x 32
constexpr int kNFC = 5;                          // filter copy instructions per wave and chunk
constexpr int kStores = 32;                      // output stores per lane and tile

// Halo unit of half hf of column col in halo row `row` (row stride rsu units).
__device__ __forceinline__ int dhalo_unit(int row, int col, int hf, int rsu)
{
    return row * rsu + 2 * col + (col >> 2) + hf;
}

struct DeferGeom {
    int N, C, H, W, Cout, Cg, Ng, OH, OW;
    int sh, ph, pw, dh;
    int Hp;                  // H + 2*ph
    int RPR, NRUN;           // runs per output row; N*OH*RPR runs in all
    int RTU;                 // runs a tile covers (at most 128): whole images or rows
    int NR, SROW, RSU;       // halo rows; columns per halo row (a multiple of 4); units per row
    int kh_units;            // unit step of one filter row: dh * RSU
    int nseg, xtasks;        // VW-wide segments per input row; staging tasks = 2*NR*nseg
    int npad;                // halo columns of a row outside the image
    int m_tiles, groups, tiles, tiles_per_xcd;
    int ocs, okg;            // channel of filter j of group k: j*ocs + k*okg
    uint32_t w_bytes, b_bytes;
    FastDiv fd_oh, fd_rpr, fd_hp, fd_nseg, fd_nr, fd_mt;
};

// W4: every run lies inside its output row (OW a multiple of 4) and y is 8-byte
// aligned, so a run's 4 outputs of a filter are one 8-byte store; otherwise 2-byte
// stores.
// FN: the group has 64 filters, so every filter row a lane stores exists and no store
// tests its row (a lane without a run still stores past the end: its base is past
// the end and 59 filter steps from there stay below 2^32, planned).
template <typename T, int XR, int VW, bool W4, bool FN>
__global__ void __launch_bounds__(kThreads, 1)
igemm_defer_fwd(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
                T *__restrict__ y, DeferGeom g)
{
    constexpr int DW = VW / 2;
    __shared__ uint4 hal0[kHU], hal1[kHU];
    __shared__ uint4 fim0[kFU], fim1[kFU];   // filter images of chunks 0 and 1
    // The filter runs as copied: chunk 0's (raw0), and chunk 1's in one of two
    // buffers by tile parity (raw1a for even tiles of the walk, raw1b for odd ones).
    __shared__ uint4 raw0[kFU], raw1a[kFU], raw1b[kFU];
    auto hal = [&](auto st) -> uint4 * {
        if constexpr (decltype(st)::value == 0) return hal0; else return hal1;
    };
    auto fim = [&](auto st) -> uint4 * {
        if constexpr (decltype(st)::value == 0) return fim0; else return fim1;
    };
    auto raw = [&](auto b) -> uint4 * {   // 0: raw0, 1: raw1a, 2: raw1b
        if constexpr (decltype(b)::value == 0) return raw0;
        else if constexpr (decltype(b)::value == 1) return raw1a;
        else return raw1b;
    };
    using B0 = std::integral_constant<int, 0>;
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // = the wave's 32 runs
    const int hf = lane >> 5, l32 = lane & 31;
    const int OHW = g.OH * g.OW;
    const int HW = g.H * g.W;

    // Persistent tile walk over XCD-contiguous tile ranges (as in igemm_rows.hip).
    const int xcd = blockIdx.x & 7, rank = blockIdx.x >> 3;
    const int nbx = ((int)gridDim.x - xcd + 7) >> 3;
    const int t_lo = xcd * g.tiles_per_xcd;
    const int t_hi = min(t_lo + g.tiles_per_xcd, g.tiles);
    int tile = t_lo + rank;
    if (tile >= t_hi) return;   // uniform over the workgroup

    // Input staging tasks (channel octet, halo row, VW-wide segment): tid + i*256.
    int xrr[XR], xoct[XR], xcol[XR];
    bool xtask[XR];
#pragma unroll
    for (int i = 0; i < XR; ++i) {
        const int tk = tid + i * kThreads;
        xtask[i] = tk < g.xtasks;
        xrr[i] = xoct[i] = xcol[i] = 0;
        if (xtask[i]) {
            const int rest = fdiv(tk, g.fd_nseg);
            const int sgm = fmod_q(tk, rest, g.fd_nseg);
            xoct[i] = fdiv(rest, g.fd_nr);
            xrr[i] = fmod_q(rest, xoct[i], g.fd_nr);
            xcol[i] = sgm * VW;
        }
    }
    // Transpose: lane = (filter tf, channel half th) of the wave's half-block (lanes
    // 32-63 repeat 0-31).  A operand: filter nb*32 + l32, channel half hf, tap t at
    // aub + nb*kBlk + t*32.
    const int tf = (lane >> 1) & 15, th = lane & 1;
    const int traw = 18 * tf + 9 * th;
    const int tdst = fimg_unit(tf, th);
    const int aub = (l32 >> 4) * kSub + fimg_unit(l32 & 15, hf);

    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, g.w_bytes);
    const __amdgpu_buffer_rsrc_t br = make_rsrc(bias, g.b_bytes);   // 0 bytes without bias: loads give 0

    struct TileState {
        int k, run0, R_lo, n_first;
        int fbase;   // w row of this wave's first staged filter: k*Ng + 16*wave
        int nfw;     // filters of this wave's half-block that exist
        __amdgpu_buffer_rsrc_t xr;
        uint32_t xvo[XR];
    };
    auto tile_state = [&](int t) {
        TileState s;
        s.k = fdiv(t, g.fd_mt);
        const int mt = fmod_q(t, s.k, g.fd_mt);
        s.run0 = mt * g.RTU;
        const int Rf = fdiv(s.run0, g.fd_rpr);
        s.n_first = fdiv(Rf, g.fd_oh);
        const int oh_first = fmod_q(Rf, s.n_first, g.fd_oh);
        s.R_lo = s.n_first * g.Hp + oh_first * g.sh;
        s.fbase = s.k * g.Ng + 16 * wave;
        s.nfw = min(16, max(0, g.Ng - 16 * wave));
        s.xr = make_rsrc(x + ((int64_t)s.n_first * g.C + (int64_t)s.k * g.Cg) * HW, 0x7fffffffu);
#pragma unroll
        for (int i = 0; i < XR; ++i) {
            s.xvo[i] = kOOB;
            if (xtask[i]) {
                const int R = s.R_lo + xrr[i];
                const int n = fdiv(R, g.fd_hp);
                const int ih = fmod_q(R, n, g.fd_hp) - g.ph;
                if (n < g.N && ih >= 0 && ih < g.H)
                    s.xvo[i] = (uint32_t)((((int64_t)(n - s.n_first) * g.C + 8 * xoct[i]) * HW +
                                           (int64_t)ih * g.W + xcol[i]) * 2);
            }
        }
        return s;
    };

    uint32_t d[2][XR][8][DW];   // staged input rows, two sets
    uint32_t E[36];             // a filter run being transposed: 8 channels x 9 taps
    // Filter copy instruction i (< 5) of chunk ch of tile s into raw buffer rb: pieces
    // 64i + lane of the wave's half-block,
    // piece q being bytes 16*(q % 18) of filter q / 18's 288-byte run; pieces past the
    // 16 filters (and filters past Ng) read zeros into the padding.
    auto filter_copy = [&](const TileState &s, int ch, auto rb, int i) {
        const int q = 64 * i + lane;
        const int pf = (q * 3641) >> 16;    // q / 18 for q < 576
        const uint32_t off = pf < s.nfw ? (uint32_t)(pf * g.Cg * 18 + 16 * (q - 18 * pf)) : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, GCONV_LDS(raw(rb) + kSub * wave + 64 * i), 16, off,
                                                 (uint32_t)(s.fbase * g.Cg + ch * 16) * 18, 0, 0);
    };
    auto input_load = [&](auto set, const TileState &s, int ch, int j) {
        const int r = j >> 3, e = j & 7;
        VecLoad<VW>::run(s.xr, xtask[r] ? s.xvo[r] : kOOB, (uint32_t)(ch * 16 + e) * HW * 2,
                         d[decltype(set)::value][r][e]);
    };
    auto transpose_read = [&](auto rb, int u) {
        const uint4 v = raw(rb)[kSub * wave + traw + u];
        E[4 * u] = v.x; E[4 * u + 1] = v.y; E[4 * u + 2] = v.z; E[4 * u + 3] = v.w;
    };
    auto transpose_write = [&](auto stg, int t) {
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e0 = 18 * q + t, e1 = e0 + 9;
            const uint32_t a = 2 * (e0 & 1), b = 4 + 2 * (e1 & 1);
            const uint32_t sel = ((b + 1) << 24) | (b << 16) | ((a + 1) << 8) | a;
            o[q] = __builtin_amdgcn_perm(E[e1 >> 1], E[e0 >> 1], sel);
        }
        fim(stg)[kSub * wave + tdst + 32 * t] = make_uint4(o[0], o[1], o[2], o[3]);
    };
    // Transpose of the wave's half-block: raw buffer rb -> filter image stg.
    auto transpose_all = [&](auto rb, auto stg) {
#pragma unroll
        for (int u = 0; u < 9; ++u) transpose_read(rb, u);
#pragma unroll
        for (int q = 0; q < 36; ++q) asm volatile("" : "+v"(E[q]));
#pragma unroll
        for (int t = 0; t < 9; ++t) transpose_write(stg, t);
    };
    auto input_write = [&](auto set, auto stg, int o) {
        constexpr int SET = decltype(set)::value;
        const int r = o / VW, v = o % VW;
        const uint32_t *ra = d[SET][r][0], *rb = d[SET][r][1], *rc = d[SET][r][2], *rd = d[SET][r][3];
        const uint32_t *re = d[SET][r][4], *rf = d[SET][r][5], *rg = d[SET][r][6], *rh = d[SET][r][7];
        const uint32_t bsel = 2 * (v & 1);
        const uint32_t sel = ((bsel + 5) << 24) | ((bsel + 4) << 16) | ((bsel + 1) << 8) | bsel;
        const int w2 = v >> 1;
        const uint4 val = make_uint4(__builtin_amdgcn_perm(rb[w2], ra[w2], sel), __builtin_amdgcn_perm(rd[w2], rc[w2], sel),
                                     __builtin_amdgcn_perm(rf[w2], re[w2], sel), __builtin_amdgcn_perm(rh[w2], rg[w2], sel));
        const int unit = xtask[r] ? dhalo_unit(xrr[r], g.pw + xcol[r] + v, xoct[r], g.RSU) : kHU - 1;
        hal(stg)[unit] = val;
    };

    // Halo columns outside the image are zero in both stages for the whole kernel.
    for (int j = tid; j < g.NR * g.npad; j += kThreads) {
        const int row = j / g.npad, pc = j - row * g.npad;
        const int col = pc < g.pw ? pc : pc - g.pw + g.pw + g.W;
        const int u = dhalo_unit(row, col, 0, g.RSU);
        hal0[u] = make_uint4(0, 0, 0, 0);
        hal0[u + 1] = make_uint4(0, 0, 0, 0);
        hal1[u] = make_uint4(0, 0, 0, 0);
        hal1[u + 1] = make_uint4(0, 0, 0, 0);
    }

    // Bias of a tile's filters (seeding its accumulators): lane's filter rows
    // nb*32 + 8q + 4hf .. +3 as 4 packed 16-bit values (zeros without bias).
    uint2 bz[2][4];
    auto bias_load = [&](const TileState &s) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int on = nb * 32 + 8 * q + 4 * hf;
                const uint32_t off = on < g.Ng ? (uint32_t)((s.k * g.Ng + on) * 2) : kOOB;
                bz[nb][q] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(br, off, 0, 0));
            }
    };

    f32x16 acc[2][2][kRun];   // [set][filter block][column]
    // The bias seeds a tile's accumulators: row (r/4)*8 + hf*4 + r%4 of block nb is
    // element r%4 of bz[nb][r/4].  Item q (< 32) seeds the 4 columns of (nb, r) =
    // (q / 16, q % 16).
    auto seed = [&](auto set, int q) {
        constexpr int PS = decltype(set)::value;
        const int nb = q >> 4, r = q & 15;
        const uint32_t dwd = (r & 2) ? bz[nb][r >> 2].y : bz[nb][r >> 2].x;
        const float b0 = half_to_f32<T>((r & 1) ? (dwd >> 16) : (dwd & 0xffffu));
#pragma unroll
        for (int mb = 0; mb < kRun; ++mb) acc[PS][nb][mb][r] = b0;
    };

    // Prologue: the first tile's filters (chunk 0 raw then transposed; chunk 1 raw,
    // transposed during chunk 0), bias, and input rows of both chunks.
    TileState ts = tile_state(tile);
#pragma unroll
    for (int i = 0; i < kNFC; ++i) filter_copy(ts, 0, B0{}, i);
#pragma unroll
    for (int i = 0; i < kNFC; ++i) filter_copy(ts, 1, std::integral_constant<int, 1>{}, i);
    bias_load(ts);
#pragma unroll
    for (int j = 0; j < 8 * XR; ++j) input_load(S0{}, ts, 0, j);
#pragma unroll
    for (int j = 0; j < 8 * XR; ++j) input_load(S1{}, ts, 1, j);
    transpose_all(B0{}, S0{});
#pragma unroll
    for (int o = 0; o < XR * VW; ++o) input_write(S0{}, S0{}, o);
    __syncthreads();

    // The stores of the previous tile: its output base (a buffer resource at its
    // first image), the lane's byte offset from there for its first filter row
    // (4*hf: the lane's half of each group of 8 rows), or past the end when the lane
    // has no run, its first column and the rows below Ng from there.
    __amdgpu_buffer_rsrc_t pyr = make_rsrc(y, 0);
    uint32_t pyh = kOOB;
    int pow0 = 0, plim = 0;
    const int fs2 = 2 * g.ocs * OHW;   // bytes between consecutive filters of y

    // Store j (< 32) of the previous tile, from accumulator set PS: filter row
    // nb*32 + (r/4)*8 + hf*4 + r%4 of the lane's run, one rounding.
    auto store_item = [&](auto ps, int j) {
        constexpr int PS = decltype(ps)::value;
        const int nb = j >> 4, r = j & 15;
        const int rowc = nb * 32 + (r >> 2) * 8 + (r & 3);   // the row less 4*hf
        // The offsets are formed here, from opaque copies of the base, not hoisted
        // ahead of the chunk where all 32 would hold registers.  (A lane without a run
        // has its base past the end, and so every offset from it.)
        uint32_t pb = pyh;
        int lim = plim;
        asm volatile("" : "+v"(pb), "+v"(lim));
        const uint32_t yo = (FN || rowc < lim) ? pb + (uint32_t)(rowc * fs2) : kOOB;
        float v[kRun];
#pragma unroll
        for (int mb = 0; mb < kRun; ++mb) v[mb] = acc_read(acc[PS][nb][mb][r]);
        if constexpr (W4) {
            const uint2 o = make_uint2(pack2<T>(v[0], v[1]), pack2<T>(v[2], v[3]));
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(gconv_u32x2, o), pyr, yo, 0, kNT);
        } else {
#pragma unroll
            for (int mb = 0; mb < kRun; ++mb)
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, from_f32<T>(v[mb])), pyr,
                                                      pow0 + mb < g.OW ? yo + 2u * mb : kOOB, 0, kNT);
        }
    };

    // One tile in accumulator set P: chunk 0 (stage 0), chunk 1 (stage 1), then the
    // filter images of the next tile.
    auto tile_body = [&](auto par) __attribute__((always_inline)) -> bool {
        constexpr int P = decltype(par)::value;
        using PP = std::integral_constant<int, 1 - P>;
        // (Lanes past the tile's runs or the last run redo the tile's last run, inside
        // its halo, and store nothing.)
        const int run = ts.run0 + wave * 32 + l32;
        const bool run_ok = wave * 32 + l32 < g.RTU && run < g.NRUN;
        const int rc = min(run, min(ts.run0 + g.RTU, g.NRUN) - 1);
        const int R = fdiv(rc, g.fd_rpr);
        const int jr = fmod_q(rc, R, g.fd_rpr);
        const int n = fdiv(R, g.fd_oh);
        const int oh = fmod_q(R, n, g.fd_oh);
        const int ow0 = kRun * jr;
        const int ub = dhalo_unit(n * g.Hp + oh * g.sh - ts.R_lo, ow0, hf, g.RSU);
        // Seed this tile's accumulators with its bias (loaded during the previous
        // tile's first chunk, or the prologue).
#pragma unroll
        for (int q = 0; q < 32; ++q) seed(par, q);


        const int next_tile = tile + nbx;
        const bool has_next = next_tile < t_hi;
        const TileState nts = has_next ? tile_state(next_tile) : ts;

        // One chunk of 16 channels from stage CUR (0 or 1).  9 taps x 8 slots; slot
        // s = 8t + i is MFMA i (block mb = i / 2, nb = i % 2) followed by its share of
        // the other work, in this order:
        //  * slots 0-1 of a tap: the next tap's A operands;
        //  * window positions of the next filter row, each read right after the MFMA
        //    that last uses it in this row;
        //  * chunk 0, slots 1-26, one per slot: the next tile's filter copies (both
        //    chunks, into raw0 and the raw buffer of its parity) and its bias, then the
        //    input rows two steps ahead (the next tile's chunk 0); slots 27-58, one per
        //    slot: the previous tile's 32 stores;
        //  * chunk 1, slots 1-16: the input rows two steps ahead (the next tile's
        //    chunk 1);
        //  * slots 46-54 and 56-64: the transpose into the other filter image (chunk
        //    0: this tile's chunk 1, from the raw buffer of this tile's parity; chunk 1:
        //    the next tile's chunk 0, from raw0);
        //  * odd slots 57-71: the input staging writes into the other stage.
        using RT = std::integral_constant<int, 1 + P>;   // this tile's chunk-1 raw buffer
        using RN = std::integral_constant<int, 2 - P>;   // the next tile's
        auto chunk = [&](auto cur) {
            using CUR = decltype(cur);
            constexpr int C0 = CUR::value == 0;
            using NXT = std::integral_constant<int, 1 - CUR::value>;
            const NXT nst{};
            const uint4 *hs = hal(cur);
            const uint4 *fs = fim(cur);
            uint4 win[kWin], af[2][2];
            af[0][0] = fs[aub];
            win[0] = hs[ub];
            af[0][1] = fs[aub + kBlk];
#pragma unroll
            for (int e = 1; e < kWin; ++e) win[e] = hs[ub + 2 * e + (e >> 2)];
            __builtin_amdgcn_sched_barrier(0);
            constexpr int NFIL = C0 ? 2 * kNFC + 1 : 0;   // filter copies and the bias (8 loads, one slot)
            constexpr int NVM = NFIL + 8 * XR;
#pragma unroll
            for (int t = 0; t < 9; ++t) {
                const int kh = t / 3, kw = t % 3;
#pragma unroll
                for (int i = 0; i < 2 * kRun; ++i) {
                    const int mb = i >> 1, nb = i & 1;
                    const int s = 2 * kRun * t + i;
                    acc[P][nb][mb] = Mfma<T>::run(af[t & 1][nb], win[mb + kw], acc[P][nb][mb]);
                    if (i < 2 && t < 8) af[(t + 1) & 1][i] = fs[aub + i * kBlk + 32 * (t + 1)];
                    if (kh < 2 && nb == 1 && (kw == 2 || mb == 0)) {
                        const int e = mb + kw;
                        win[e] = hs[ub + (kh + 1) * g.kh_units + 2 * e + (e >> 2)];
                    }
                    if (s >= 1 && s - 1 < NVM) {
                        const int o = s - 1;
                        if (C0 && o < kNFC) filter_copy(nts, 0, B0{}, o);
                        else if (C0 && o < 2 * kNFC) filter_copy(nts, 1, RN{}, o - kNFC);
                        else if (C0 && o == 2 * kNFC) bias_load(nts);
                        else input_load(cur, nts, CUR::value, o - NFIL);
                    }
                    if constexpr (C0) {
                        if (s >= 27 && s - 27 < kStores) store_item(PP{}, s - 27);
                    }
                    if (s >= 46 && s <= 54) {
                        if constexpr (C0) transpose_read(RT{}, s - 46);
                        else transpose_read(B0{}, s - 46);
                    }
                    if (s == 55) {
#pragma unroll
                        for (int q = 0; q < 36; ++q) asm volatile("" : "+v"(E[q]));
                    }
                    if (s >= 56 && s <= 64) transpose_write(nst, s - 56);
                    if (s >= 57 && (s & 1) == 1 && (s - 57) / 2 < XR * VW) input_write(nst, nst, (s - 57) / 2);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __syncthreads();
        };
        chunk(S0{});
        chunk(S1{});

        // This tile's outputs become the previous tile's.
        pyr = make_rsrc(y + (int64_t)ts.n_first * g.Cout * OHW, 0x7fffffffu);
        pyh = run_ok ? (uint32_t)(((n - ts.n_first) * g.Cout + ts.k * g.okg) * OHW + oh * g.OW + ow0) * 2u +
                           (uint32_t)(4 * hf * fs2)
                     : kOOB;
        plim = g.Ng - 4 * hf;
        pow0 = ow0;
        if (!has_next) return false;
        tile = next_tile;
        ts = nts;
        return true;
    };
    // The last tile's stores, after the walk.  (The filter copies of its chunk 0,
    // of no next tile, are waited for here: no copy into LDS may be in flight when
    // the workgroup ends.)
    auto flush = [&](auto ps) {
#pragma unroll
        for (int j = 0; j < kStores; ++j) store_item(ps, j);
        __builtin_amdgcn_s_waitcnt(0);
    };

    // (Before the first tile there is nothing to store: the base is past the end, so
    // its first chunk's stores are all dropped.)
    for (;;) {
        if (!tile_body(P0{})) {
            flush(P0{});
            return;
        }
        if (!tile_body(P1{})) {
            flush(P1{});
            return;
        }
    }
}

struct DeferPlan {
    DeferGeom g;
    int XR, VW;
    bool W4;
    bool ok;
};

DeferPlan make_defer_plan(const Conv2dArgs &a)
{
    DeferPlan pl{};
    pl.ok = false;
    if (a.dtype != DT_F16 && a.dtype != DT_BF16) return pl;
    if (a.KH != 3 || a.KW != 3 || a.sw != 1 || a.dw != 1) return pl;
    DeferGeom &g = pl.g;
    g.N = (int)a.N; g.C = (int)a.C; g.H = (int)a.H; g.W = (int)a.W; g.Cout = (int)a.Cout;
    g.Cg = (int)(a.C / a.groups); g.Ng = (int)(a.Cout / a.groups);
    g.OH = (int)a.OH; g.OW = (int)a.OW;
    g.sh = a.sh; g.ph = a.ph; g.pw = a.pw; g.dh = a.dh;
    g.groups = (int)a.groups;
    // 33 to 64 filters per group: one filter tile of 64.  C/g = 32: two chunks of 16
    // channels per tile.
    if (g.Ng <= 32 || g.Ng > 64) return pl;
    if (g.Cg != 32 || (reinterpret_cast<uintptr_t>(a.w) & 15) != 0) return pl;
    const int64_t w_bytes = a.Cout * (int64_t)g.Cg * 18;
    if (w_bytes >= (int64_t(1) << 31)) return pl;
    g.w_bytes = (uint32_t)w_bytes;
    g.b_bytes = 0;
    if (a.bias) {
        if (g.Ng % 4 != 0 || (reinterpret_cast<uintptr_t>(a.bias) & 7) != 0) return pl;
        g.b_bytes = (uint32_t)(a.Cout * 2);
    }
    g.Hp = (int)(a.H + 2 * a.ph);
    g.RPR = (int)ceil_div(a.OW, kRun);
    const int64_t NRUN = a.N * a.OH * (int64_t)g.RPR;
    if (NRUN >= (int64_t(1) << 31) - 2 * kRT || a.N * (int64_t)g.Hp + 3 * (int64_t)a.dh + 1024 >= (int64_t(1) << 31))
        return pl;
    g.NRUN = (int)NRUN;
    // Runs per tile: whole images when they fill at least 7/8 of the 128 lanes, else
    // whole rows when they do, else 128.
    const int64_t img = (int64_t)g.OH * g.RPR;
    int64_t RTU = kRT;
    if (img <= kRT && 8 * (kRT / img * img) >= 7 * kRT) RTU = kRT / img * img;
    else if (g.RPR <= kRT && 8 * (kRT / g.RPR * g.RPR) >= 7 * kRT) RTU = kRT / g.RPR * g.RPR;
    g.RTU = (int)RTU;
    // Output rows a tile touches, image boundaries among them, and the padded input
    // rows of its halo (the bound igemm_rows.hip uses).
    const bool aligned = RTU % g.RPR == 0;
    const int64_t V = aligned ? RTU / g.RPR : (RTU - 1) / g.RPR + 2;
    const int64_t crossings = V <= 1                           ? 0
                              : aligned && g.OH % V == 0       ? 0
                              : aligned && V % g.OH == 0       ? V / g.OH - 1
                                                               : (V - 2) / g.OH + 1;
    const int64_t gap = std::max<int64_t>(0, (int64_t)g.Hp - (int64_t)g.OH * g.sh);
    int64_t NR = (V - 1) * g.sh + crossings * gap + 2 * (int64_t)g.dh + 1;
    NR = std::min<int64_t>(NR, a.N * (int64_t)g.Hp);
    const int64_t WL = kRun * (int64_t)g.RPR + 2;   // padded columns the windows read
    const int64_t SROW = (WL + 3) / 4 * 4;
    if (NR * SROW >= (int64_t(1) << 24)) return pl;
    // Row stride in units: 9 per 4 columns, plus a padding making it congruent to
    // 9*RPR modulo 16 when a row has fewer than 16 runs (and the padded rows fit), so
    // that the 16 consecutive runs of a half-wave read 16 different units modulo 16.
    int64_t RSU = 9 * (SROW / 4) + (g.RPR < 16 ? ((9 * g.RPR - 9 * (SROW / 4)) % 16 + 16) % 16 : 0);
    if (NR * RSU > kHU - 1) RSU = 9 * (SROW / 4);
    if (NR * RSU > kHU - 1) return pl;   // the last unit is the spare one
    g.NR = (int)NR; g.SROW = (int)SROW; g.RSU = (int)RSU;
    g.kh_units = g.dh * g.RSU;
    g.npad = g.pw + (int)(SROW - g.pw - g.W);
    // Input rows in VW-wide segments.
    const uintptr_t xa = reinterpret_cast<uintptr_t>(a.x);
    pl.VW = (g.W % 8 == 0 && xa % 16 == 0) ? 8 : (g.W % 4 == 0 && xa % 8 == 0) ? 4 : 0;
    if (pl.VW == 0) return pl;
    g.nseg = g.W / pl.VW;
    int64_t xtasks = 2 * NR * g.nseg;
    if (pl.VW == 8 && xtasks > kThreads && (xa % 8) == 0) {
        pl.VW = 4;
        g.nseg = g.W / 4;
        xtasks = 2 * NR * g.nseg;
    }
    pl.XR = (int)ceil_div(xtasks, kThreads);
    if (pl.XR * pl.VW > 8) return pl;
    g.xtasks = (int)xtasks;
    const int64_t HW = (int64_t)g.H * g.W;
    if ((crossings + 1) * (int64_t)g.C * HW * 2 >= (int64_t(1) << 31) || (int64_t)(g.Cg + 16) * HW * 2 >= (int64_t(1) << 31))
        return pl;
    if ((crossings + 1) * (int64_t)g.Cout * g.OH * g.OW * 2 >= (int64_t(1) << 31)) return pl;   // output offsets
    pl.W4 = g.OW % 4 == 0 && (reinterpret_cast<uintptr_t>(a.y) & 7) == 0;
    g.ocs = a.interleaved ? g.groups : 1;
    g.okg = a.interleaved ? 1 : g.Ng;
    g.m_tiles = (int)ceil_div(NRUN, RTU);
    const int64_t tiles = (int64_t)g.m_tiles * g.groups;
    if (tiles >= (int64_t(1) << 31)) return pl;
    g.tiles = (int)tiles;
    g.tiles_per_xcd = (int)ceil_div(tiles, 8);
    g.fd_oh = make_fastdiv((uint32_t)g.OH);
    g.fd_rpr = make_fastdiv((uint32_t)g.RPR);
    g.fd_hp = make_fastdiv((uint32_t)g.Hp);
    g.fd_nseg = make_fastdiv((uint32_t)g.nseg);
    g.fd_nr = make_fastdiv((uint32_t)g.NR);
    g.fd_mt = make_fastdiv((uint32_t)g.m_tiles);
    pl.ok = true;
    return pl;
}

template <typename T, int XR, int VW, bool W4, bool FN>
hipError_t run(const Conv2dArgs &a, const DeferPlan &pl)
{
    int dev = 0, cus = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    const int64_t blocks = std::min<int64_t>(pl.g.tiles, std::max(cus, 8));
    hipLaunchKernelGGL((igemm_defer_fwd<T, XR, VW, W4, FN>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                       (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, pl.g);
    return hipGetLastError();
}

template <typename T>
hipError_t run_typed(const Conv2dArgs &a, const DeferPlan &pl)
{
    // (XR, VW) = (1, 8) or (at most 2, 4).  FN: 64 filters per group, and a base
    // past the end plus 59 filter steps (2 * ocs * OH * OW bytes each) below 2^32.
    const bool fn = pl.g.Ng == 64 && 59 * 2 * (int64_t)pl.g.ocs * pl.g.OH * pl.g.OW < (int64_t(1) << 31);
    if (fn) {
        if (pl.W4) return pl.VW == 8 ? run<T, 1, 8, true, true>(a, pl) : run<T, 2, 4, true, true>(a, pl);
        return pl.VW == 8 ? run<T, 1, 8, false, true>(a, pl) : run<T, 2, 4, false, true>(a, pl);
    }
    if (pl.W4) return pl.VW == 8 ? run<T, 1, 8, true, false>(a, pl) : run<T, 2, 4, true, false>(a, pl);
    return pl.VW == 8 ? run<T, 1, 8, false, false>(a, pl) : run<T, 2, 4, false, false>(a, pl);
}

}  // namespace

bool igemm_defer_supported(const Conv2dArgs &a) { return make_defer_plan(a).ok; }

hipError_t launch_igemm_defer(const Conv2dArgs &a, const char **kname)
{
    const DeferPlan pl = make_defer_plan(a);
    if (!pl.ok) return hipErrorInvalidValue;
    *kname = "igemm_defer_mfma32x32x16";
    return a.dtype == DT_F16 ? run_typed<_Float16>(a, pl) : run_typed<__bf16>(a, pl);
}

}  // namespace gconv
