// igemm_rows.hip -- implicit-GEMM grouped conv2d (NCHW, 3x3 filters, unit column
// stride and dilation) on the gfx950 matrix cores, each lane owning a run of 8
// consecutive output columns.
//
// Per group k the convolution is the product
//     Y_k[o][m] = sum_kk W_k[o][kk] * A_k[kk][m],   kk = (input channel, tap),
// over the output positions m of the group's Cout/g filters, A_k being the im2col
// matrix of the group's input channels.  The discuss.pytorch.org thread "F.conv2d
// runs x15 slower in mixed-precision/half-precision mode" traces the slow fp16
// grouped conv to grouped convs not reaching the tensor cores; here every group's
// contraction runs on v_mfma_f32_32x32x16_{f16,bf16} and A_k is never written out
// (the neon issue "Grouped convolutions" on explicit im2col being wasteful).
//
// Runs.  Each output row is cut into runs of 8 consecutive columns (the last run
// of a row may be partial).  In a wave, lane l32 (and its partner l32 + 32, which
// holds the other 8 channels of each K step) owns one run, and MFMA block mb
// (mb < 8) computes column mb of every run.  v_mfma_f32_32x32x16 leaves lane l32
// with column l32 of the 32 filter rows of a block, so after the K loop a lane
// holds 8 consecutive outputs of each of its filters: one 16-byte store per filter
// straight from the accumulators, 512 contiguous bytes per half-wave.  For filter
// row kh the B operands of the taps kw = 0, 1, 2 of block mb are the input columns
// ow0 + mb + kw of one halo row: a window of 10 positions x 8 channels (10 16-byte
// LDS reads) feeds all 24 B operands of the filter row.
//
// Tile: 4 waves.  FW (1 or 2) waves across the filters, 64 each (2 blocks of 32),
// and 4/FW across the runs, 32 each: 128 runs x 64 filters, or 64 runs x 128
// filters of one group.  Every wave issues 16 MFMAs per K step.
//
// K loop: chunks of 16 input channels, then the 9 taps; one MFMA step = one tap x
// 16 channels.  While chunk c computes, chunk c+1 is staged into the other LDS
// stage:
//  * input: a zero-padded halo of whole input rows, [row][column][16 channels], so
//    that one B fragment (8 channels of one position) is one 16-byte read; loaded 8
//    channel rows x VW columns per task and transposed in registers with v_perm;
//  * filters: the chunk of a 32-filter block is 32 runs of 16 channels x 9 taps (288
//    contiguous bytes of w each).  One wave copies them straight into LDS (buffer
//    loads with an LDS destination, 16 bytes per lane) and transposes them in place:
//    each lane reads one filter's 8 channels x 9 taps (9 16-byte reads at a 144-byte
//    lane stride, free of bank conflicts), forms the 9 units of 8 channels at one tap
//    with v_perm, and writes them back where the A operand reads expect them.  Each
//    wave only touches its own block's bytes, so no barrier is needed between the
//    copy and the transpose.
// The halo and filter images live in separate LDS arrays, so the compiler waits for
// the LDS-destination loads only before the filter reads, not before every read.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "fastdiv.hpp"

namespace gconv {
namespace {

#include "rows_common.hpp"

constexpr int kThreads = 256;
constexpr int kBlockUnits = 576;             // one 32-filter block's chunk: 32 x 16 ch x 9 taps x 2 B
constexpr int kSubUnits = 288;               // one 16-filter half of it
// LDS stride of a 16-filter half-block in the filter image: 288 units with 128
// filters per tile; 320 with 64, where each wave stages one half-block with 5
// copy instructions of 64 units (the last one's extra lanes write zeros into the
// 32 padding units, not into the next half-block).
template <int FW> constexpr int kSub = FW == 1 ? 320 : kSubUnits;
template <int FW> constexpr int kBlk = 2 * kSub<FW>;                    // a 32-filter block
constexpr int kRun = 8;                      // output columns per run
constexpr int kWin = kRun + 2;               // window positions of one filter row (3 taps)

template <int FW> constexpr int kFU = 2 * FW * kBlk<FW>;                 // filter units per stage
template <int FW> constexpr int kHU = (kLdsUnits - 2 * kFU<FW>) / 2;     // halo units per stage

// Halo map: 16-byte half `hf` (channels 0-7 or 8-15) of the 32-byte slot of column
// col in halo row `row`, with one spare unit after every 8 columns and a row stride
// of rsu units.  Columns 8 apart are 17 units apart, so the 16 lanes of a half-wave
// reading the same window position of 16 consecutive runs of one row hit 16
// different units modulo 16; rsu is chosen congruent to the runs per row modulo 16
// when a row has fewer than 16 runs, so that runs spanning several rows do too.
__device__ __forceinline__ int halo_unit(int row, int col, int hf, int rsu)
{
    return row * rsu + 2 * col + (col >> 3) + hf;
}




struct RowsGeom {
    int N, C, H, W, Cout, Cg, Ng, OH, OW;
    int sh, ph, pw, dh;
    int Hp;                  // H + 2*ph: rows of one zero-padded image in the virtual row space
    int RPR, NRUN;           // runs per output row; N*OH*RPR runs in all (< 2^31)
    int RTU;                 // runs a tile covers (at most its 32*PW lanes): whole rows or images
    int NR, SROW;            // halo rows; slots per halo row (a multiple of 8)
    int RSU;                 // units per halo row: 17 * SROW / 8 plus a padding below 16
    int kh_units;            // unit step of one filter row in the halo: dh * RSU
    int nseg, xtasks;        // VW-wide segments per input row; staging tasks = 2*NR*nseg
    int npad;                // halo columns of a row outside the image: [0, pw) and [pw + W, SROW)
    int m_tiles, n_tiles, groups, nchunks, tiles, tiles_per_xcd;
    int sg;                  // output store width in elements: 8 (16 bytes), 4 (8 bytes) or 1
    int ocs, okg;            // channel of filter j of group k: j*ocs + k*okg
    uint32_t w_bytes, b_bytes;
    FastDiv fd_oh, fd_rpr, fd_hp, fd_nseg, fd_nr, fd_mt, fd_nt;
};

template <typename T, int FW, int XR, int VW, bool SG8>
__global__ void __launch_bounds__(kThreads, 1)
igemm_rows_fwd(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
               T *__restrict__ y, RowsGeom g)
{
    constexpr int BN = 64 * FW;              // filters per tile
    constexpr int PW = 4 / FW;               // waves across the runs
    constexpr int RT = 32 * PW;              // runs per tile
    constexpr int DW = VW / 2;               // dwords per staged row segment
    // Each wave stages a 32-filter block (128 filters per tile) or a 16-filter
    // half-block (64): FPW filters, NFC copy instructions, SW units of the image.
    constexpr int FPW = 32 * FW / 2;
    constexpr int NFC = FW == 1 ? 5 : 9;
    constexpr int SW = FW == 1 ? kSub<1> : kBlk<2>;
    constexpr int SUB = kSub<FW>, BLK = kBlk<FW>;
    constexpr int FU = kFU<FW>;
    constexpr int HU = kHU<FW>;
    // Input halo and filter image, two pipeline stages each, as four LDS arrays: the
    // compiler tracks LDS-destination loads per array, and with the stage known at
    // compile time in each copy of the chunk body, reads of the current stage never
    // wait for the copies into the next one.
    __shared__ uint4 hal0[HU], hal1[HU];
    __shared__ uint4 fim0[FU], fim1[FU];
    auto hal = [&](auto st) -> uint4 * {
        if constexpr (decltype(st)::value == 0) return hal0; else return hal1;
    };
    auto fim = [&](auto st) -> uint4 * {
        if constexpr (decltype(st)::value == 0) return fim0; else return fim1;
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in a scalar register
    const int hf = lane >> 5, l32 = lane & 31;
    const int pwv = wave / FW, fwv = wave % FW;
    const int OHW = g.OH * g.OW;
    const int HW = g.H * g.W;

    // Persistent tile walk: workgroup b runs on XCD b % 8, which owns a contiguous
    // range of tiles; its workgroups walk the range together, so the tiles in flight
    // on one XCD are neighbours sharing halo rows and filters in its L2.
    const int xcd = blockIdx.x & 7, rank = blockIdx.x >> 3;
    const int nbx = ((int)gridDim.x - xcd + 7) >> 3;
    const int t_lo = xcd * g.tiles_per_xcd;
    const int t_hi = min(t_lo + g.tiles_per_xcd, g.tiles);
    int tile = t_lo + rank;
    if (tile >= t_hi) return;   // uniform over the workgroup

    // Input staging tasks (channel octet, halo row, VW-wide segment); task i of this
    // thread is tid + i*256.
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
    // Transpose: lane = (filter tf, channel half th) of the wave's block.
    // (With 16-filter half-blocks, lanes 32-63 repeat lanes 0-31: the same reads and
    // the same values written to the same units.)
    const int tf = (lane >> 1) & (FPW - 1), th = lane & 1;
    const int traw = 18 * tf + 9 * th;                                    // first raw unit
    const int tdst = (tf >> 4) * SUB + fimg_unit(tf & 15, th);            // tap-0 unit
    // A operand: filter fwv*64 + nb*32 + l32, channel half hf, tap t at
    // aub + nb*BLK + t*32.
    const int aub = (fwv * 4 + (l32 >> 4)) * SUB + fimg_unit(l32 & 15, hf);

    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, g.w_bytes);
    const __amdgpu_buffer_rsrc_t br = make_rsrc(bias, g.b_bytes);

    struct TileState {
        int k, nt, run0, R_lo, n_first;
        int fbase;   // w row of this wave's first staged filter (k*Ng + nt*BN + FPW*wave)
        int nfw;     // filters of this wave's staged block that exist
        __amdgpu_buffer_rsrc_t xr;
        uint32_t xvo[XR];
    };
    auto tile_state = [&](int t) {
        TileState s;
        const int bq = fdiv(t, g.fd_mt);
        const int mt = fmod_q(t, bq, g.fd_mt);
        s.k = fdiv(bq, g.fd_nt);
        s.nt = fmod_q(bq, s.k, g.fd_nt);
        s.run0 = mt * g.RTU;
        const int Rf = fdiv(s.run0, g.fd_rpr);          // first output row (n*OH + oh)
        s.n_first = fdiv(Rf, g.fd_oh);
        const int oh_first = fmod_q(Rf, s.n_first, g.fd_oh);
        s.R_lo = s.n_first * g.Hp + oh_first * g.sh;
        s.fbase = s.k * g.Ng + s.nt * BN + FPW * wave;
        s.nfw = min(FPW, max(0, g.Ng - s.nt * BN - FPW * wave));
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

    // Staged input rows, two sets: while chunk c writes step c+1's rows (loaded
    // during chunk c-1) into LDS, step c+2's rows arrive in the other set, a whole
    // chunk ahead of their use.
    uint32_t d[2][XR][8][DW];
    uint32_t E[36];          // a filter run being transposed: 8 channels x 9 taps
    // Filter copy instruction i (< 9) of one pipeline step (tile s, chunk ch) into
    // stage stg, by a staging wave: pieces 64i + lane of the wave's block, piece q
    // being bytes 16*(q % 18) of filter q / 18's 288-byte run.
    // (Every chunk holds 16 channels: C/g is a multiple of 32 here.)  The lane's piece
    // of copy instruction i is filter pf[i] of the block, bytes 16*pj[i] of its run:
    // a byte offset pf*18*C/g + 16*pj from the block's first filter, the same in every
    // tile and chunk; the tile and chunk add a uniform offset.
    auto filter_copy = [&](const TileState &s, int ch, auto stg, int i) {
        const int q = 64 * i + lane;
        const int pf = (q * 3641) >> 16;    // q / 18 for q < 576
        const uint32_t off = pf < s.nfw ? (uint32_t)(pf * g.Cg * 18 + 16 * (q - 18 * pf)) : kOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, GCONV_LDS(fim(stg) + SW * wave + 64 * i), 16, off,
                                                 (uint32_t)(s.fbase * g.Cg + ch * 16) * 18, 0, 0);
    };
    // Input load j (< 8*XR) of one pipeline step into registers: task j/8, channel row j%8.
    auto input_load = [&](auto set, const TileState &s, int ch, int j) {
        const int r = j >> 3, e = j & 7;
        VecLoad<VW>::run(s.xr, xtask[r] ? s.xvo[r] : kOOB, (uint32_t)(ch * 16 + e) * HW * 2,
                         d[decltype(set)::value][r][e]);
    };
    // Transpose of this wave's block in stage stg, in place: read u (< 9) brings raw
    // unit u of the lane's run (8 channels x 9 taps); write t (< 9) forms the unit of
    // the 8 channels at tap t.  Every read of the wave comes before its first write
    // (the writes land on units other lanes read).
    auto transpose_read = [&](auto stg, int u) {
        const uint4 v = fim(stg)[SW * wave + traw + u];
        E[4 * u] = v.x; E[4 * u + 1] = v.y; E[4 * u + 2] = v.z; E[4 * u + 3] = v.w;
    };
    auto transpose_write = [&](auto stg, int t) {
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // channels 2q, 2q+1 at tap t: elements 18q + t and 18q + 9 + t of the run
            const int e0 = 18 * q + t, e1 = e0 + 9;
            const uint32_t a = 2 * (e0 & 1), b = 4 + 2 * (e1 & 1);
            const uint32_t sel = ((b + 1) << 24) | (b << 16) | ((a + 1) << 8) | a;
            o[q] = __builtin_amdgcn_perm(E[e1 >> 1], E[e0 >> 1], sel);
        }
        fim(stg)[SW * wave + tdst + 32 * t] = make_uint4(o[0], o[1], o[2], o[3]);
    };
    // Staging write o (< XR*VW) into stage stg: column o % VW of task o / VW as one
    // unit of 8 channels; a thread without that task writes the spare unit.
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
        const int unit = xtask[r] ? halo_unit(xrr[r], g.pw + xcol[r] + v, xoct[r], g.RSU) : HU - 1;
        hal(stg)[unit] = val;
    };

    // Halo columns outside the image are zero in both stages for the whole kernel
    // (staging writes only columns [pw, pw + W)).
    for (int j = tid; j < g.NR * g.npad; j += kThreads) {
        const int row = j / g.npad, pc = j - row * g.npad;
        const int col = pc < g.pw ? pc : pc - g.pw + g.pw + g.W;
        const int u = halo_unit(row, col, 0, g.RSU);
        hal0[u] = make_uint4(0, 0, 0, 0);
        hal0[u + 1] = make_uint4(0, 0, 0, 0);
        hal1[u] = make_uint4(0, 0, 0, 0);
        hal1[u + 1] = make_uint4(0, 0, 0, 0);
    }

    TileState ts = tile_state(tile);
#pragma unroll
    for (int i = 0; i < NFC; ++i) filter_copy(ts, 1, S1{}, i);   // chunk 1's (issued first: see below)
#pragma unroll
    for (int i = 0; i < NFC; ++i) filter_copy(ts, 0, S0{}, i);
#pragma unroll
    for (int j = 0; j < 8 * XR; ++j) input_load(S0{}, ts, 0, j);
#pragma unroll
    for (int j = 0; j < 8 * XR; ++j) input_load(S1{}, ts, 1, j);   // step 1, written during chunk 0
#pragma unroll
    for (int u = 0; u < 9; ++u) transpose_read(S0{}, u);
#pragma unroll
    for (int q = 0; q < 36; ++q) asm volatile("" : "+v"(E[q]));
#pragma unroll
    for (int t = 0; t < 9; ++t) transpose_write(S0{}, t);
#pragma unroll
    for (int o = 0; o < XR * VW; ++o) input_write(S0{}, S0{}, o);
    __syncthreads();

    // One tile: its chunks, then its output stores.
    //
    // Vector memory counts loads and stores in one in-order counter, so a wait for a
    // load also waits for every store issued before it.  The filter copies that the
    // transposes of a tile's first chunk wait for (chunk 1's filters) are therefore
    // issued before the previous tile's output stores, not during the first chunk:
    // that chunk then waits for its copies but for at most the oldest of the stores,
    // and computes while the rest drain.  The first tile runs as a copy of its own, so
    // that the wait counts the compiler derives at the loop's entry are those of a
    // tile that follows another (an entry straight from the prologue, where no stores
    // follow the copies, would set them for every tile).
    auto tile_body = [&]() __attribute__((always_inline)) -> bool {
        // This lane's run and its halo and output addresses.
        // (Lanes past the tile's runs or the last run redo the tile's last run, inside
        // its halo, and store nothing.)
        const int run = ts.run0 + pwv * 32 + l32;
        const bool run_ok = pwv * 32 + l32 < g.RTU && run < g.NRUN;
        const int rc = min(run, min(ts.run0 + g.RTU, g.NRUN) - 1);
        const int R = fdiv(rc, g.fd_rpr);
        const int jr = fmod_q(rc, R, g.fd_rpr);
        const int n = fdiv(R, g.fd_oh);
        const int oh = fmod_q(R, n, g.fd_oh);
        const int ow0 = kRun * jr;
        const int ub = halo_unit(n * g.Hp + oh * g.sh - ts.R_lo, ow0, hf, g.RSU);

        f32x16 acc[2][8];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[nb][mb][r] = 0.0f;

        const int next_tile = tile + nbx;
        const bool has_next = next_tile < t_hi;
        const TileState nts = has_next ? tile_state(next_tile) : ts;
        // One chunk: computes from stage CUR and stages the next pipeline step into
        // the other one (instantiated once per stage, so every LDS array is named
        // statically).
        auto chunk = [&](auto cur, int ch, auto first) {
            using CUR = decltype(cur);
            constexpr bool FIRST = decltype(first)::value;   // copies no filters
            using NXT = std::integral_constant<int, 1 - CUR::value>;
            const NXT nst{};
            const bool last = ch + 1 == g.nchunks;
            // Next pipeline step: chunk ch+1 of this tile, or chunk 0 of the next tile
            // (its filters are copied now); the input rows two steps ahead.
            const TileState src = last ? nts : ts;
            const int nch = last ? 0 : ch + 1;
            const TileState src2 = ch + 2 < g.nchunks ? ts : nts;
            const int nch2 = ch + 2 < g.nchunks ? ch + 2 : ch + 2 - g.nchunks;

            const uint4 *hs = hal(cur);
            const uint4 *fs = fim(cur);
            uint4 win[kWin], af[2][2];
            // First the operands of the first MFMAs, then the rest of the window.
            af[0][0] = fs[aub];
            win[0] = hs[ub];
            af[0][1] = fs[aub + BLK];
#pragma unroll
            for (int e = 1; e < kWin; ++e) win[e] = hs[ub + 2 * e + (e >> 3)];
            __builtin_amdgcn_sched_barrier(0);
            // The chunk as 9 taps x 16 slots; slot i of tap t is MFMA i (block mb =
            // i / 2, nb = i % 2) followed by its share of the staging work, in this
            // order (the scheduling barriers keep it):
            //  * slots 0-1: the next tap's A operands;
            //  * the window of the next filter row, each position read into its register
            //    right after the MFMA that last uses it in this row (position 0 after
            //    tap kw = 0, position 1 after kw = 1, position 2 + mb after block mb of
            //    kw = 2), at least 16 MFMAs before its first use;
            //  * from slot 3 of tap 0 on, every second slot: the global loads of the
            //    next pipeline step, the input rows (from memory, first touch) before
            //    the filter copies (from L2);
            //  * taps 6-8, odd slots: the input staging writes; tap 6: the transpose
            //    reads; taps 7-8: its 9 unit writes.
            constexpr int NVM = (FIRST ? 0 : NFC) + 8 * XR;   // global loads per step
#pragma unroll
            for (int t = 0; t < 9; ++t) {
                const int kh = t / 3, kw = t % 3;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int mb = i >> 1, nb = i & 1;
                    acc[nb][mb] = Mfma<T>::run(af[t & 1][nb], win[mb + kw], acc[nb][mb]);
                    if (i < 2 && t < 8) af[(t + 1) & 1][i] = fs[aub + i * BLK + 32 * (t + 1)];
                    if (kh < 2 && nb == 1 && (kw == 2 || mb == 0)) {
                        const int e = mb + kw;   // its last use in this row was this MFMA
                        win[e] = hs[ub + (kh + 1) * g.kh_units + 2 * e + (e >> 3)];
                    }
                    // Global loads: the input rows, then the filter copies, one every
                    // second slot from slot 3 of tap 0 on.
                    const int sl = 16 * t + i - 3;
                    if (sl >= 0 && (sl & 1) == 0 && sl / 2 < NVM) {
                        const int o = sl / 2;
                        if (o < 8 * XR) input_load(cur, src2, nch2, o);
                        else if (!FIRST) filter_copy(src, nch, nst, o - 8 * XR);
                    }
                    if (t == 6 && i >= 2 && i <= 10) transpose_read(nst, i - 2);
                    if (t == 7 && i == 0) {
                        // every transpose read has returned before the first write
#pragma unroll
                        for (int q = 0; q < 36; ++q) asm volatile("" : "+v"(E[q]));
                    }
                    if ((t == 7 && i % 4 == 0) || (t == 8 && i % 3 == 0 && i < 15))
                        transpose_write(nst, t == 7 ? i / 4 : 4 + i / 3);
                    if (t >= 6 && (i & 1) == 1) {
                        const int ow = (t - 6) * 8 + i / 2;
                        if (ow < XR * VW) input_write(nst, nst, ow);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __syncthreads();
        };
        // An even number of chunks (planned), so every tile starts on stage 0.
        chunk(S0{}, 0, std::true_type{});
        chunk(S1{}, 1, std::false_type{});
        for (int ch = 2; ch < g.nchunks; ch += 2) {
            chunk(S0{}, ch, std::false_type{});
            chunk(S1{}, ch + 1, std::false_type{});
        }
        // The next tile's chunk-1 filters into stage 1, free since the barrier above.
        // (None after the last tile: no copy into LDS may be in flight at the end.)
        if (has_next) {
#pragma unroll
            for (int i = 0; i < NFC; ++i) filter_copy(nts, 1, S1{}, i);
        }

        // Epilogue: + bias in fp32, one rounding to T, stored straight from the
        // accumulators: 8 consecutive outputs of one filter per lane and row.  The
        // stores go through a buffer resource based at the tile's first image, and a
        // lane or row with nothing to store gives an offset past its end, which the
        // hardware drops: every lane issues the same stores and no branch skips them,
        // so the wait counts derived after the epilogue hold on every path.
        {
            // Filters this lane's rows cover: the wave's 64 from fb0, those below Ng.
            const int fb0 = ts.nt * BN + fwv * 64;
            const __amdgpu_buffer_rsrc_t yr = make_rsrc(y + (int64_t)ts.n_first * g.Cout * OHW, 0x7fffffffu);
            // Element offset of the lane's first output of filter fb0 from that image
            // (below 2^30, planned), or -1.  Formed here, not hoisted to the tile start
            // where it would hold registers through the K loop.
            int ybase = run_ok ? ((n - ts.n_first) * g.Cout + fb0 * g.ocs + ts.k * g.okg) * OHW + oh * g.OW + ow0 : -1;
            int fstep = g.ocs * OHW;   // between consecutive filters
            asm volatile("" : "+v"(ybase), "+s"(fstep));
            auto store_rows = [&](auto has_bias) {
                uint2 bz[2][4];
                if constexpr (decltype(has_bias)::value) {
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int on = fb0 + nb * 32 + 8 * q + 4 * hf;
                            const uint32_t off = on < g.Ng ? (uint32_t)((ts.k * g.Ng + on) * 2) : kOOB;
                            bz[nb][q] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(br, off, 0, 0));
                        }
                }
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = nb * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
                        const bool ok = ybase >= 0 && fb0 + row < g.Ng;
                        const uint32_t yo = ok ? (uint32_t)(ybase + row * fstep) * 2u : kOOB;
                        float v[8];
#pragma unroll
                        for (int mb = 0; mb < 8; ++mb) v[mb] = acc_read(acc[nb][mb][r]);
                        if constexpr (decltype(has_bias)::value) {
                            const uint32_t dwd = (r & 2) ? bz[nb][r >> 2].y : bz[nb][r >> 2].x;
                            const float b0 = half_to_f32<T>((r & 1) ? (dwd >> 16) : (dwd & 0xffffu));
#pragma unroll
                            for (int mb = 0; mb < 8; ++mb) v[mb] += b0;
                        }
                        if constexpr (SG8) {
                            const uint4 o = make_uint4(pack2<T>(v[0], v[1]), pack2<T>(v[2], v[3]),
                                                       pack2<T>(v[4], v[5]), pack2<T>(v[6], v[7]));
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(gconv_u32x4, o), yr, yo, 0, kNT);
                        } else if (g.sg == 4) {
                            const uint2 o0 = make_uint2(pack2<T>(v[0], v[1]), pack2<T>(v[2], v[3]));
                            const uint2 o1 = make_uint2(pack2<T>(v[4], v[5]), pack2<T>(v[6], v[7]));
                            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(gconv_u32x2, o0), yr, yo, 0, kNT);
                            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(gconv_u32x2, o1), yr,
                                                                  ow0 + 4 < g.OW ? yo + 8u : kOOB, 0, kNT);
                        } else {
#pragma unroll
                            for (int mb = 0; mb < 8; ++mb)
                                __builtin_amdgcn_raw_buffer_store_b16(
                                    __builtin_bit_cast(unsigned short, from_f32<T>(v[mb])), yr,
                                    ow0 + mb < g.OW ? yo + 2u * mb : kOOB, 0, kNT);
                        }
                    }
            };
            if (bias)
                store_rows(std::true_type{});
            else
                store_rows(std::false_type{});
        }
        if (!has_next) return false;
        tile = next_tile;
        ts = nts;
        return true;
    };
    if (tile_body())
        while (tile_body()) {
        }
}

struct RowsPlan {
    RowsGeom g;
    int FW, XR, VW;
    bool ok;
};

RowsPlan make_rows_plan(const Conv2dArgs &a)
{
    RowsPlan pl{};
    pl.ok = false;
    if (a.dtype != DT_F16 && a.dtype != DT_BF16) return pl;
    if (a.KH != 3 || a.KW != 3 || a.sw != 1 || a.dw != 1) return pl;
    RowsGeom &g = pl.g;
    g.N = (int)a.N; g.C = (int)a.C; g.H = (int)a.H; g.W = (int)a.W; g.Cout = (int)a.Cout;
    g.Cg = (int)(a.C / a.groups); g.Ng = (int)(a.Cout / a.groups);
    g.OH = (int)a.OH; g.OW = (int)a.OW;
    g.sh = a.sh; g.ph = a.ph; g.pw = a.pw; g.dh = a.dh;
    g.groups = (int)a.groups;
    // Filters: a chunk of one filter is 16 channels x 9 taps = 288 contiguous bytes,
    // copied in 16-byte pieces.
    // C/g a multiple of 32: every chunk holds 16 channels and the chunk loop, unrolled
    // over the two stages, takes an even number of them.
    if (g.Cg % 32 != 0 || (reinterpret_cast<uintptr_t>(a.w) & 15) != 0) return pl;
    const int64_t w_bytes = a.Cout * (int64_t)g.Cg * 18;
    if (w_bytes >= (int64_t(1) << 31)) return pl;
    g.w_bytes = (uint32_t)w_bytes;
    g.b_bytes = 0;
    if (a.bias) {
        if (g.Ng % 4 != 0 || (reinterpret_cast<uintptr_t>(a.bias) & 7) != 0) return pl;
        g.b_bytes = (uint32_t)(a.Cout * 2);
    }
    // 64 filters per wave: two waves across the filters for more than 64 filters per
    // group, one for 33 to 64 (fewer filters per group stay on the implicit GEMM of
    // igemm.hip, whose tiles are narrower).
    if (g.Ng <= 32) return pl;
    pl.FW = g.Ng > 64 ? 2 : 1;
    const int RT = 32 * (4 / pl.FW);
    g.Hp = (int)(a.H + 2 * a.ph);
    g.RPR = (int)ceil_div(a.OW, 8);
    const int64_t NRUN = a.N * a.OH * (int64_t)g.RPR;
    if (NRUN >= (int64_t(1) << 31) - 2 * RT || a.N * (int64_t)g.Hp + 3 * (int64_t)a.dh + 1024 >= (int64_t(1) << 31))
        return pl;
    g.NRUN = (int)NRUN;
    // Runs per tile: whole images when they fill at least 7/8 of the RT lanes, else
    // whole rows when they do, else all RT.  (Whole images need no halo rows beyond
    // their own, and no output line is shared by two tiles.)
    const int64_t img = (int64_t)g.OH * g.RPR;
    int64_t RTU = RT;
    if (img <= RT && 8 * (RT / img * img) >= 7 * RT) RTU = RT / img * img;
    else if (g.RPR <= RT && 8 * (RT / g.RPR * g.RPR) >= 7 * RT) RTU = RT / g.RPR * g.RPR;
    g.RTU = (int)RTU;
    // Output rows a tile's RTU runs can touch, image boundaries among them, and the
    // resulting bound on the padded input rows of its halo.
    const bool aligned = RTU % g.RPR == 0;
    const int64_t V = aligned ? RTU / g.RPR : (RTU - 1) / g.RPR + 2;
    const int64_t crossings = V <= 1                           ? 0
                              : aligned && g.OH % V == 0       ? 0
                              : aligned && V % g.OH == 0       ? V / g.OH - 1   // whole images
                                                               : (V - 2) / g.OH + 1;
    const int64_t gap = std::max<int64_t>(0, (int64_t)g.Hp - (int64_t)g.OH * g.sh);
    int64_t NR = (V - 1) * g.sh + crossings * gap + 2 * (int64_t)g.dh + 1;
    NR = std::min<int64_t>(NR, a.N * (int64_t)g.Hp);
    const int64_t WL = 8 * (int64_t)g.RPR + 2;   // padded columns the runs' windows read
    const int64_t SROW = (WL + 7) / 8 * 8;
    if (NR * SROW >= (int64_t(1) << 24)) return pl;
    // Row stride in units: 17 per 8 columns, plus (RPR - SROW/8) mod 16 when a row
    // has fewer than 16 runs (then the 16 runs a half-wave reads span several rows)
    // and the padded rows fit.
    const int HU = pl.FW == 2 ? kHU<2> : kHU<1>;
    int64_t RSU = 17 * (SROW / 8) + (g.RPR < 16 ? ((g.RPR - SROW / 8) % 16 + 16) % 16 : 0);
    if (NR * RSU > HU - 1) RSU = 17 * (SROW / 8);
    if (NR * RSU > HU - 1) return pl;   // the last unit is the spare one
    g.NR = (int)NR; g.SROW = (int)SROW; g.RSU = (int)RSU;
    g.kh_units = g.dh * g.RSU;
    g.npad = g.pw + (int)(SROW - g.pw - g.W);
    // Input rows in VW-wide segments (whole rows: W a multiple of VW).
    const uintptr_t xa = reinterpret_cast<uintptr_t>(a.x);
    pl.VW = (g.W % 8 == 0 && xa % 16 == 0) ? 8 : (g.W % 4 == 0 && xa % 8 == 0) ? 4 : 0;
    if (pl.VW == 0) return pl;
    g.nseg = g.W / pl.VW;
    int64_t xtasks = 2 * NR * g.nseg;
    if (pl.VW == 8 && xtasks > kThreads && (xa % 8) == 0) {   // 16 dwords of staging registers at most
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
    const uintptr_t ya = reinterpret_cast<uintptr_t>(a.y);
    g.sg = (g.OW % 8 == 0 && ya % 16 == 0) ? 8 : (g.OW % 4 == 0 && ya % 8 == 0) ? 4 : 1;
    g.ocs = a.interleaved ? g.groups : 1;
    g.okg = a.interleaved ? 1 : g.Ng;
    g.m_tiles = (int)ceil_div(NRUN, RTU);
    g.n_tiles = (int)ceil_div(g.Ng, 64 * pl.FW);
    g.nchunks = g.Cg / 16;
    const int64_t tiles = (int64_t)g.m_tiles * g.n_tiles * g.groups;
    if (tiles >= (int64_t(1) << 31)) return pl;
    g.tiles = (int)tiles;
    g.tiles_per_xcd = (int)ceil_div(tiles, 8);
    g.fd_oh = make_fastdiv((uint32_t)g.OH);
    g.fd_rpr = make_fastdiv((uint32_t)g.RPR);
    g.fd_hp = make_fastdiv((uint32_t)g.Hp);
    g.fd_nseg = make_fastdiv((uint32_t)g.nseg);
    g.fd_nr = make_fastdiv((uint32_t)g.NR);
    g.fd_mt = make_fastdiv((uint32_t)g.m_tiles);
    g.fd_nt = make_fastdiv((uint32_t)g.n_tiles);
    pl.ok = true;
    return pl;
}

template <typename T, int FW, int XR, int VW, bool SG8>
hipError_t run(const Conv2dArgs &a, const RowsPlan &pl)
{
    int dev = 0, cus = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    // Persistent grid: one workgroup per CU (the LDS footprint allows no more).
    const int64_t blocks = std::min<int64_t>(pl.g.tiles, std::max(cus, 8));
    hipLaunchKernelGGL((igemm_rows_fwd<T, FW, XR, VW, SG8>), dim3((unsigned)blocks), dim3(kThreads), 0, a.stream,
                       (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, pl.g);
    return hipGetLastError();
}

template <typename T>
hipError_t run_typed(const Conv2dArgs &a, const RowsPlan &pl)
{
    // (XR, VW) = (1, 8) or (at most 2, 4): 8 channel rows x 16 bytes of staged input
    // per thread, at most.
    auto pick = [&](auto fw) -> hipError_t {
        constexpr int FW = decltype(fw)::value;
        if (pl.g.sg == 8) return pl.VW == 8 ? run<T, FW, 1, 8, true>(a, pl) : run<T, FW, 2, 4, true>(a, pl);
        return pl.VW == 8 ? run<T, FW, 1, 8, false>(a, pl) : run<T, FW, 2, 4, false>(a, pl);
    };
    return pl.FW == 2 ? pick(std::integral_constant<int, 2>{}) : pick(std::integral_constant<int, 1>{});
}

}  // namespace

bool igemm_rows_supported(const Conv2dArgs &a) { return make_rows_plan(a).ok || igemm_defer_supported(a); }

hipError_t launch_igemm_rows(const Conv2dArgs &a, const char **kname)
{
    // 33 to 64 filters per group: the kernel with runs of 4 columns and deferred
    // output stores (igemm_defer.hip) where it applies.
    if (igemm_defer_supported(a)) return launch_igemm_defer(a, kname);
    const RowsPlan pl = make_rows_plan(a);
    if (!pl.ok) return hipErrorInvalidValue;
    *kname = "igemm_rows_mfma32x32x16";
    return a.dtype == DT_F16 ? run_typed<_Float16>(a, pl) : run_typed<__bf16>(a, pl);
}

}  // namespace gconv
