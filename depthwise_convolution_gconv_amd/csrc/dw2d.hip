// dw2d.hip -- depthwise conv2d (NCHW, groups = C) on the vector ALUs, stride 1 or 2.
//
// The depthwise extreme of grouped convolution: every output channel reads one
// input channel (C/g = 1; Cout/g = M filters per channel, M = 1 being the plain
// depthwise layer).  The work per output is K*K multiply-adds, so the layer is
// bound by HBM traffic, not arithmetic: the kernel's job is to read x once and
// write y once, both coalesced.  Stride 2 is the depthwise-separable downsampling
// layer that speechbrain issue #2733 names as the next candidate after the
// Conformer's 1-D depthwise conv (Fast Conformer's subsampling CNN, which needs
// stride).
//
// Two kernels: dw2d_band (below dw2d_rows) for 16-bit layers whose output rows
// cover the input rows exactly (OW * S == W), dw2d_rows for the rest.
//
// dw2d_rows<T, K, S, R, VI>: K x K filters, stride S, dilation 1.
//  * Work unit: a run of R consecutive outputs of one output row (R*sizeof(T) =
//    16 or 8 bytes, or R = 1).  Runs are numbered over (output plane, row, run),
//    i.e. in the memory order of y, and workgroup b takes runs_per_wg consecutive
//    ones, so a workgroup's stores cover one contiguous stretch of y.
//  * Staging: the zero-padded input rows those runs read (virtual rows of the
//    padded planes, so a workgroup may span plane boundaries) go to LDS (fp32,
//    or the raw 16 bits of 16-bit tensors), one row every WP elements, with
//    16-byte buffer loads along W (out-of-range offsets read as zero, which
//    supplies the padding rows).  The filters and biases of the
//    planes the workgroup touches go next to them.
//  * Compute: each thread slides its run's window ((R-1)*S + K input columns,
//    16-byte LDS reads) down the K filter rows, R fp32 accumulators, bias added
//    in fp32, one rounding to T, one R-element vector store.
//  * Workgroups are dealt to the XCDs in contiguous runs (workgroup b runs on XCD
//    b % 8), so the halo rows that neighbouring workgroups share come from one L2.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "fastdiv.hpp"

namespace gconv {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsTarget = 20 * 1024;     // LDS per workgroup that keeps 8 resident per CU
constexpr int kLdsBudget = 40 * 1024;     // most LDS per workgroup (>= 4 resident per CU)
constexpr uint32_t kOOB = 0x80000000u;    // buffer offset past num_records: the load returns 0

struct Dw2dGeom {
    int C, H, W, Cout, OH, OW;
    int ph, pw;
    int Hp;            // H + 2*ph: rows of one padded plane in the virtual row space
    int planes;        // N * Cout output planes
    int WP;            // LDS row stride (floats, multiple of 4)
    int RPR;           // runs per output row (OW / R)
    int CPR;           // staging loads per input row (W / VI)
    int npad;          // LDS columns of a row outside the image (WP - W)
    int runs_per_wg, total_runs, wgs, wgs_per_xcd;
    int NRmax;         // LDS rows reserved for the input (bound on any workgroup's rows)
    // A thread's staging chunks are 256 apart: (st_r rows, st_c chunks) of the staged
    // rows, st_r = st_rq padded planes + st_rm rows; with one filter per channel the
    // input offset advances by st_off elements (plus W for a carried row, plus
    // st_wrap when the padded row wraps into the next plane).
    int st_c, st_r, st_rq, st_rm, st_off, st_wrap;
    FastDiv fd_rpr, fd_oh, fd_hp, fd_cpr, fd_cout, fd_m, fd_npad;
};

template <int BYTES> struct Load;
template <> struct Load<16> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *d)
    {
        const uint4 u = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w;
    }
};
template <> struct Load<4> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *d)
    {
        d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
};
template <> struct Load<2> {
    static __device__ __forceinline__ void run(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t *d)
    {
        d[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    }
};

// LDS element of the staged input: fp32 for fp32 tensors, the raw 16 bits for
// 16-bit ones (widened when read, which halves the LDS a workgroup's rows take).
template <typename T> using LdsT = std::conditional_t<sizeof(T) == 4, float, uint16_t>;
template <typename T> __device__ __forceinline__ LdsT<T> lds_elem(const uint32_t *d, int e)
{
    if constexpr (sizeof(T) == 4) return __builtin_bit_cast(float, d[e]);
    else return (uint16_t)(d[e >> 1] >> (16 * (e & 1)));
}
template <typename T> __device__ __forceinline__ float widen(LdsT<T> v)
{
    if constexpr (sizeof(T) == 4) return v;
    else if constexpr (std::is_same_v<T, _Float16>) return (float)__builtin_bit_cast(_Float16, v);
    else return __builtin_bit_cast(float, (uint32_t)v << 16);
}

// Bits of one rounded T value (round to nearest even), in the low bits of a dword.
template <typename T> __device__ __forceinline__ uint32_t bits_of(float v)
{
    if constexpr (sizeof(T) == 4) return __builtin_bit_cast(uint32_t, v);
    else return (uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(v));
}

// Stores R values of T (R * sizeof(T) bytes, aligned to that size) at p.
template <typename T, int R>
__device__ __forceinline__ void store_run(T *p, const float *v)
{
    constexpr int NDW = (R * (int)sizeof(T) + 3) / 4;
    if constexpr (R * sizeof(T) < 4) {
        store_nt(p, from_f32<T>(v[0]));
    } else {
        uint32_t d[NDW];
#pragma unroll
        for (int i = 0; i < NDW; ++i) {
            if constexpr (sizeof(T) == 4) d[i] = bits_of<T>(v[i]);
            else d[i] = bits_of<T>(v[2 * i]) | (bits_of<T>(v[2 * i + 1]) << 16);
        }
        if constexpr (NDW == 4) store_nt(reinterpret_cast<uint4 *>(p), make_uint4(d[0], d[1], d[2], d[3]));
        else if constexpr (NDW == 2) store_nt(reinterpret_cast<uint2 *>(p), make_uint2(d[0], d[1]));
        else store_nt(reinterpret_cast<uint32_t *>(p), d[0]);
    }
}

template <typename T, int K, int S, int R, int VI>
__global__ void __launch_bounds__(kThreads)
dw2d_rows(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
          T *__restrict__ y, Dw2dGeom g)
{
    using LT = LdsT<T>;
    constexpr int KK = K * K;
    constexpr int G = 16 / (int)sizeof(LT);               // LDS elements per 16-byte read
    constexpr bool kVecRead = (R * S) % G == 0;           // window starts are 16-byte aligned
    constexpr int NWIN = (R - 1) * S + K;                 // input columns of one run
    constexpr int NWR = kVecRead ? (NWIN + G - 1) / G * G : NWIN;
    constexpr int DW = (VI * (int)sizeof(T) + 3) / 4;     // dwords per staging load
    constexpr int NB = 8;                                 // staging loads in flight per thread
    extern __shared__ uint4 lds[];

    const int xcd = blockIdx.x & 7, rank = blockIdx.x >> 3;
    const int wg = xcd * g.wgs_per_xcd + rank;
    if (wg >= min((xcd + 1) * g.wgs_per_xcd, g.wgs)) return;   // uniform over the workgroup
    const int tid = threadIdx.x;

    // Runs [u0, u1) of this workgroup; the output rows (virtual: plane * OH + oh) and
    // the padded input rows (virtual: plane * Hp + hp) they cover.
    const int u0 = wg * g.runs_per_wg;
    const int u1 = min(u0 + g.runs_per_wg, g.total_runs);
    const int vr_a = fdiv(u0, g.fd_rpr), vr_b = fdiv(u1 - 1, g.fd_rpr);
    const int pa = fdiv(vr_a, g.fd_oh), pb = fdiv(vr_b, g.fd_oh);
    const int R_lo = pa * g.Hp + (vr_a - pa * g.OH) * S;
    const int NR = pb * g.Hp + (vr_b - pb * g.OH) * S + K - R_lo;
    LT *xs = reinterpret_cast<LT *>(lds);                 // [NR][WP]
    float *ws = reinterpret_cast<float *>(xs + g.NRmax * g.WP);   // [pb - pa + 1][K*K + 1] (16-byte aligned)

    // Input plane read by output plane p: image n = p / Cout, channel (p % Cout) / M.
    auto in_plane = [&](int p) {
        const int n = fdiv(p, g.fd_cout);
        return n * g.C + fdiv(p - n * g.Cout, g.fd_m);
    };
    const int pia = in_plane(pa);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T *>(x + (int64_t)pia * g.H * g.W), (short)0, 0x7fffffff, 0x00020000);

    // Stage the rows, NB loads per thread in flight at a time.  A thread's chunks are
    // i = tid + 256 k: row r = i / CPR and column chunk ch advance by fixed steps, and
    // so do the row's plane and row within it (and with one filter per channel, ONE,
    // its input offset), with no division per chunk.
    const int nchunks = NR * g.CPR;
    auto stage = [&](auto one) {
        constexpr bool ONE = decltype(one)::value;
        int r = fdiv(tid, g.fd_cpr), ch = tid - r * g.CPR;
        int sp = fdiv(R_lo + r, g.fd_hp), shp = R_lo + r - sp * g.Hp;
        int rowoff = (sp - pa) * g.H * g.W + (shp - g.ph) * g.W;   // ONE: the row's first input element
        for (int base = 0; base < nchunks; base += NB * kThreads) {
            uint32_t d[NB][DW];
            int dst[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                uint32_t off = kOOB;
                dst[j] = -1;
                if (r < NR) {
                    const int ih = shp - g.ph;
                    if (sp < g.planes && ih >= 0 && ih < g.H) {
                        if constexpr (ONE)
                            off = (uint32_t)((rowoff + ch * VI) * (int)sizeof(T));
                        else
                            off = (uint32_t)((((int64_t)(in_plane(sp) - pia) * g.H + ih) * g.W + ch * VI) * sizeof(T));
                    }
                    dst[j] = r * g.WP + g.pw + ch * VI;
                }
                Load<VI * sizeof(T) >= 4 ? 4 * DW : 2>::run(xr, off, d[j]);
                ch += g.st_c;
                r += g.st_r;
                shp += g.st_rm;
                sp += g.st_rq;
                rowoff += g.st_off;
                if (ch >= g.CPR) { ch -= g.CPR; ++r; ++shp; rowoff += g.W; }
                if (shp >= g.Hp) { shp -= g.Hp; ++sp; rowoff += g.st_wrap; }
            }
#pragma unroll
            for (int j = 0; j < NB; ++j)
                if (dst[j] >= 0) {
#pragma unroll
                    for (int q = 0; q < VI; ++q) xs[dst[j] + q] = lds_elem<T>(d[j], q);
                }
        }
    };
    if (g.Cout == g.C)
        stage(std::true_type{});
    else
        stage(std::false_type{});
    // Columns outside the image: zero.
    for (int i = tid; i < NR * g.npad; i += kThreads) {
        const int r = fdiv(i, g.fd_npad), c = i - r * g.npad;
        xs[r * g.WP + (c < g.pw ? c : c + g.W)] = LT(0);   // +0.0 in every storage type
    }
    // Filters of output planes pa .. pb, each followed by the plane's bias (zero
    // without one): read here from LDS, the bias costs no global load in the run
    // loop, where a load would wait for the previous runs' stores.
    for (int i = tid; i < (pb - pa + 1) * (KK + 1); i += kThreads) {
        const int p = pa + i / (KK + 1), t = i - (i / (KK + 1)) * (KK + 1);
        const int o = p - fdiv(p, g.fd_cout) * g.Cout;
        ws[i] = t < KK ? to_f32(w[(int64_t)o * KK + t]) : (bias ? to_f32(bias[o]) : 0.0f);
    }
    __syncthreads();

    for (int u = u0 + tid; u < u1; u += kThreads) {
        const int vr = fdiv(u, g.fd_rpr), rc = u - vr * g.RPR;
        const int p = fdiv(vr, g.fd_oh), oh = vr - p * g.OH;
        const float *wt = ws + (p - pa) * (KK + 1);
        const float b0 = wt[KK];
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = b0;
        const LT *xrow = xs + (p * g.Hp + oh * S - R_lo) * g.WP + rc * (R * S);
#pragma unroll
        for (int kh = 0; kh < K; ++kh) {
            float win[NWR];
            if constexpr (kVecRead) {
#pragma unroll
                for (int v = 0; v < NWR / G; ++v) {
                    LT q[G];
                    *reinterpret_cast<uint4 *>(q) = *reinterpret_cast<const uint4 *>(xrow + kh * g.WP + G * v);
#pragma unroll
                    for (int e = 0; e < G; ++e) win[G * v + e] = widen<T>(q[e]);
                }
            } else {
#pragma unroll
                for (int v = 0; v < NWR; ++v) win[v] = widen<T>(xrow[kh * g.WP + v]);
            }
#pragma unroll
            for (int kw = 0; kw < K; ++kw) {
                const float wv = wt[kh * K + kw];
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = fmaf(win[r * S + kw], wv, acc[r]);
            }
        }
        store_run<T, R>(y + (int64_t)vr * g.OW + rc * R, acc);
    }
}

// ---------------------------------------------------------------------------
// dw2d_band<T, K, S, KR>: 16-bit layers at full width, OW * S == W (for odd K
// that is pw = (K - 1) / 2), with W a multiple of 8 and at most 512 columns.
//  * Chunk: 8 input columns, 16 bytes.  Run: the R = 8 / S outputs of one output
//    row whose windows start in one chunk; the window is PW columns before the
//    chunk, the chunk, and NWIN - 8 - PW columns after it.
//  * Strip: KR runs stacked in one chunk column, output rows oh0 .. oh0+KR-1 of
//    one plane (rows past OH are computed and not stored).  A wave takes G =
//    64 / CPR strips side by side (CPR = W / 8 chunks per row), lane = slot * CPR
//    + chunk column, so a row's chunks sit in adjacent lanes of one wave; a
//    workgroup takes 4 G consecutive strips.
//  * Staging: the padded input rows of the workgroup's strips (virtual rows of
//    the padded planes, as in dw2d_rows) go to LDS chunk by chunk, coalesced
//    16-byte buffer loads (zero outside the image), each written as one aligned
//    16-byte LDS store.  Chunk c of staged row r sits at 16-byte unit
//    r * CPR + c + (r / (KR * S)) * GAP with GAP = CPR * (1 - KR * S) mod 8: the
//    strips of a wave then start CPR units apart modulo 8 units, so the chunks
//    its lanes read together fall on distinct bank groups in every 8 lanes.
//  * Compute: per input row of its strip a lane reads its own chunk (one 16-byte
//    LDS read) and takes the window columns outside it from the lanes beside it
//    by DPP wave shifts (zero at the row ends).  dw2d_rows reads the whole
//    window per row (two 16-byte reads at 3 x 3, stride 2) and stages each row
//    at the padding offset, 2 bytes past 16-byte alignment.  Products and sums
//    are fp32 in the order of dw2d_rows (kh, then kw): both give the same bits.

// Lane i gets lane i - 1's value (DPP wave_shr:1); lane 0 gets 0.
__device__ __forceinline__ uint32_t from_lane_before(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x138, 0xf, 0xf, false);
}
// Lane i gets lane i + 1's value (DPP wave_shl:1); lane 63 gets 0.
__device__ __forceinline__ uint32_t from_lane_after(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x130, 0xf, 0xf, false);
}

// Element e of a chunk of 16-bit values held as dwords, widened to fp32.
template <typename T> __device__ __forceinline__ float chunk_elem(const uint32_t *d, int e)
{
    const uint32_t v = d[e >> 1];
    if constexpr (std::is_same_v<T, _Float16>)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> (16 * (e & 1))));
    else
        return __builtin_bit_cast(float, (e & 1) ? (v & 0xffff0000u) : (v << 16));
}

struct BandGeom {
    int C, H, W, Cout, OH, OW, ph;
    int Hp;            // H + 2*ph: rows of one padded plane in the virtual row space
    int planes;        // N * Cout output planes
    int CPR;           // chunks per row (W / 8), at most 64
    int G;             // strips side by side in one wave (64 / CPR)
    int SPP;           // strips per output plane (ceil(OH / KR))
    int strips;        // planes * SPP
    int spw;           // strips per workgroup (4 G)
    int GAP;           // 16-byte units left free after every KR * S staged rows
    int units;         // 16-byte LDS units reserved for the staged rows (the filters follow)
    int sp_p, sp_hp;   // 4G staged rows as (planes, rows) of the padded row space
    int step_off;      // with one filter per channel: input elements between rows 4G apart
    int wrap_off;      // and the correction when the padded row wraps into the next plane
    int wgs, wgs_per_xcd;
    FastDiv fd_cpr, fd_spp, fd_hp, fd_cout, fd_m;
};

template <typename T, int K, int S, int KR>
__global__ void __launch_bounds__(kThreads)
dw2d_band(const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ bias,
          T *__restrict__ y, BandGeom g)
{
    static_assert(sizeof(T) == 2, "16-bit tensors");
    constexpr int R = 8 / S;                    // outputs per run
    constexpr int PW = (K - 1) / 2;             // window columns before the chunk
    constexpr int NWIN = (R - 1) * S + K;       // window columns of a run
    constexpr int NAFT = NWIN - 8 - PW;         // window columns after the chunk (<= 0: none)
    constexpr int NRW = (KR - 1) * S + K;       // input rows of a strip
    constexpr int BAND = KR * S;                // staged rows per gap
    constexpr int KK = K * K;
    constexpr int DB = (8 - PW) / 2;            // first dword of the lane before that the window uses
    constexpr int DA = NAFT > 0 ? (NAFT + 1) / 2 : 0;   // dwords of the lane after that it uses
    constexpr int NB = 8;                       // staging loads in flight per thread
    constexpr int RB = R * 2;                   // bytes of one run of outputs
    extern __shared__ uint4 lds[];              // [units] staged rows, then [planes][K*K + 1] fp32
    float *ws = reinterpret_cast<float *>(lds + g.units);

    const int xcd = blockIdx.x & 7, rank = blockIdx.x >> 3;
    const int wg = xcd * g.wgs_per_xcd + rank;
    if (wg >= min((xcd + 1) * g.wgs_per_xcd, g.wgs)) return;   // uniform over the workgroup
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slot = fdiv(lane, g.fd_cpr), rc = lane - slot * g.CPR;
    const int s_first = wg * g.spw, s_last = min(s_first + g.spw, g.strips) - 1;
    const int pa = fdiv(s_first, g.fd_spp), pb = fdiv(s_last, g.fd_spp);
    // Staged rows: from the first strip's first padded row to the last strip's last.
    const int R_lo = pa * g.Hp + (s_first - pa * g.SPP) * BAND;
    const int NR = pb * g.Hp + (s_last - pb * g.SPP) * BAND + NRW - R_lo;

    // Input plane read by output plane q: image n = q / Cout, channel (q % Cout) / M.
    auto in_plane = [&](int q) {
        const int n = fdiv(q, g.fd_cout);
        return n * g.C + fdiv(q - n * g.Cout, g.fd_m);
    };
    // Offsets relative to the workgroup's first input and output planes (the host
    // bounds both spans to 31 bits); kOOB reads 0 and drops stores.
    const int pia = in_plane(pa);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T *>(x + (int64_t)pia * g.H * g.W), (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
        y + (int64_t)pa * g.OH * g.OW, (short)0, 0x7fffffff, 0x00020000);

    // Stage the rows, NB loads per thread in flight at a time.  A thread takes chunk
    // rc of staged rows r = wave * G + slot + k * 4G (the compute lanes' mapping: a
    // load instruction covers G consecutive rows, contiguous in x within a plane).
    // The row advances by 4G, a multiple of BAND, so the plane and row within it
    // advance by a fixed step and the LDS unit by a fixed stride: no division per row.
    // With one filter per channel the input plane is the output plane, and the row's
    // input offset advances by a fixed step too (ONE); otherwise each row maps its
    // plane to the input plane it reads.
    auto stage = [&](auto one) {
        constexpr bool ONE = decltype(one)::value;
        const int rstep = 4 * g.G;
        const int r0 = wave * g.G + slot;
        int vr = R_lo + r0;
        int sp = fdiv(vr, g.fd_hp);
        int shp = vr - sp * g.Hp;                     // row within the padded plane
        int rowoff = (sp - pa) * g.H * g.W + (shp - g.ph) * g.W;   // ONE: the row's first input element
        int su = r0 * g.CPR + rc + (r0 / BAND) * g.GAP;
        const int ustep = rstep * g.CPR + (rstep / BAND) * g.GAP;
        const bool lane_ok = slot < g.G;
        for (int kb = r0; kb < NR; kb += NB * rstep) {
            uint32_t d[NB][4];
            int dst[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int r = kb + j * rstep;
                const int ih = shp - g.ph;
                const bool ok = lane_ok && r < NR && sp < g.planes && ih >= 0 && ih < g.H;
                uint32_t off;
                if constexpr (ONE)
                    off = ok ? (uint32_t)((rowoff + 8 * rc) * 2) : kOOB;
                else
                    off = ok ? (uint32_t)((((in_plane(sp) - pia) * g.H + ih) * g.W + 8 * rc) * 2) : kOOB;
                dst[j] = lane_ok && r < NR ? su : -1;
                Load<16>::run(xr, off, d[j]);
                su += ustep;
                shp += g.sp_hp;
                sp += g.sp_p;
                rowoff += g.step_off;
                if (shp >= g.Hp) { shp -= g.Hp; ++sp; rowoff += g.wrap_off; }
            }
#pragma unroll
            for (int j = 0; j < NB; ++j)
                if (dst[j] >= 0) lds[dst[j]] = make_uint4(d[j][0], d[j][1], d[j][2], d[j][3]);
        }
    };
    if (g.Cout == g.C)
        stage(std::true_type{});
    else
        stage(std::false_type{});
    // Filters of output planes pa .. pb, each followed by the plane's bias (zero
    // without one), from addresses that are always valid.
    for (int i = tid; i < (pb - pa + 1) * (KK + 1); i += kThreads) {
        const int q = pa + i / (KK + 1), t = i - (i / (KK + 1)) * (KK + 1);
        const int o = q - fdiv(q, g.fd_cout) * g.Cout;
        const bool has = t < KK || bias != nullptr;
        const T *src = t < KK ? w + (int64_t)o * KK + t : (has ? bias + o : w);
        const float v = to_f32(*src);
        ws[i] = has ? v : 0.0f;
    }
    __syncthreads();

    // This lane's strip (lanes past the wave's strips, and strips past the
    // workgroup's, are idle: they take the first strip and store nothing).
    const int s = s_first + wave * g.G + slot;
    const bool act = slot < g.G && s <= s_last;
    const int sc = act ? s : s_first;
    const int p = fdiv(sc, g.fd_spp), oh0 = (sc - p * g.SPP) * KR;
    const int lr0 = p * g.Hp + oh0 * S - R_lo;   // staged row of the strip's first input row
    const float *wt = ws + (p - pa) * (KK + 1);
    float wk[KK + 1];
#pragma unroll
    for (int t = 0; t <= KK; ++t) wk[t] = wt[t];
    // The DPP moves run on the whole wave (a lane reads its neighbour's register, so
    // no lane may be masked off); the row ends are cleared afterwards with masks.
    const uint32_t keep_before = rc == 0 ? 0u : ~0u, keep_after = rc == g.CPR - 1 ? 0u : ~0u;
    float acc[KR][R];
#pragma unroll
    for (int i = 0; i < KR; ++i)
#pragma unroll
        for (int j = 0; j < R; ++j) acc[i][j] = wk[KK];
#pragma unroll
    for (int r = 0; r < NRW; ++r) {
        const int lr = lr0 + r;
        const uint4 q = lds[lr * g.CPR + rc + (lr / BAND) * g.GAP];
        const uint32_t own[4] = {q.x, q.y, q.z, q.w};
        uint32_t bef[4], aft[4];
#pragma unroll
        for (int e = DB; e < 4; ++e) bef[e] = from_lane_before(own[e]) & keep_before;
#pragma unroll
        for (int e = 0; e < DA; ++e) aft[e] = from_lane_after(own[e]) & keep_after;
        float win[NWIN];
#pragma unroll
        for (int t = 0; t < NWIN; ++t) {
            const int c = t - PW;
            win[t] = c < 0 ? chunk_elem<T>(bef, 8 + c) : c < 8 ? chunk_elem<T>(own, c) : chunk_elem<T>(aft, c - 8);
        }
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            const int kh = r - i * S;
            if (kh >= 0 && kh < K) {
#pragma unroll
                for (int kw = 0; kw < K; ++kw)
#pragma unroll
                    for (int j = 0; j < R; ++j) acc[i][j] = fmaf(win[j * S + kw], wk[kh * K + kw], acc[i][j]);
            }
        }
    }
    // Branch-free stores: rows past OH and idle lanes get the dropped offset.  Store
    // i writes row i of every strip, so it covers every other output row of the
    // wave and a line is completed by the next store.  Write-back stores let L2
    // join the two halves; non-temporal ones reached HBM as partial lines (1.5x
    // the output bytes on the 8 x 256 x 512 x 40 layer).
    const int row0 = (p - pa) * g.OH + oh0;
#pragma unroll
    for (int i = 0; i < KR; ++i) {
        const uint32_t off = act && oh0 + i < g.OH ? (uint32_t)((row0 + i) * g.OW * 2 + rc * RB) : kOOB;
        uint32_t d[RB / 4];
#pragma unroll
        for (int e = 0; e < RB / 4; ++e) d[e] = bits_of<T>(acc[i][2 * e]) | (bits_of<T>(acc[i][2 * e + 1]) << 16);
        if constexpr (RB == 8)
            __builtin_amdgcn_raw_buffer_store_b64(gconv_u32x2{d[0], d[1]}, yr, off, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b128(gconv_u32x4{d[0], d[1], d[2], d[3]}, yr, off, 0, 0);
    }
}

struct Plan {
    Dw2dGeom g;
    int K, S, R, VI;
    size_t lds;
    bool ok;
};

Plan make_plan(const Conv2dArgs &a)
{
    Plan pl{};
    pl.ok = false;
    const int es = a.dtype == DT_F32 ? 4 : 2;
    if (a.groups != a.C || a.KH != a.KW || (a.KH != 3 && a.KH != 5 && a.KH != 7)) return pl;
    if (a.sh != a.sw || (a.sh != 1 && a.sh != 2) || a.dh != 1 || a.dw != 1) return pl;
    if (a.ph > a.KH || a.pw > a.KW) return pl;
    if (a.interleaved && a.Cout != a.C) return pl;   // the order differs only with several filters per channel
    const int K = (int)a.KH, S = a.sh;
    Dw2dGeom &g = pl.g;
    // Run length: 16 or 8 bytes of y when the output rows split into such runs and y
    // is aligned for them, else single elements.
    const uintptr_t ya = reinterpret_cast<uintptr_t>(a.y);
    pl.R = 1;
    for (int R : {16 / es, 8 / es}) {
        if (R >= 2 && a.OW % R == 0 && ya % (uintptr_t)(R * es) == 0 && (R * S) % 4 == 0) {
            pl.R = R;
            break;
        }
    }
    const int VI16 = 16 / es;
    pl.VI = (a.W % VI16 == 0 && reinterpret_cast<uintptr_t>(a.x) % 16 == 0) ? VI16 : 1;
    const int64_t planes = a.N * a.Cout;
    const int64_t Hp = a.H + 2 * (int64_t)a.ph;
    const int64_t RPR = a.OW / pl.R;
    const int64_t total_runs = planes * a.OH * RPR;
    if (planes * Hp + 2 * K >= (int64_t(1) << 31) || total_runs >= (int64_t(1) << 31)) return pl;
    const int R = pl.R;
    const int NWIN = (R - 1) * S + K;
    const int les = es;                                   // LDS bytes per staged element
    const int G = 16 / les;
    const int NWR = (R * S) % G == 0 ? (NWIN + G - 1) / G * G : NWIN;
    const int64_t WP = (std::max<int64_t>(a.W + 2 * a.pw, (RPR - 1) * R * S + NWR) + G - 1) / G * G;
    // Runs per workgroup: as many as keep the workgroup's LDS within kLdsTarget, so
    // that 8 workgroups stay resident per CU with the most input bytes in flight
    // (measured on the 8 x 256 x 512 x 40 layers: stride 1 took 114 us with 256 runs
    // per workgroup and 76 us with 1024; stride 2 is fastest with 256, at 19 KB); a
    // single pass may use up to kLdsBudget.
    const int64_t gap = Hp - a.OH * S;   // >= K - S > 0: rows between two planes' windows
    auto lds_for = [&](int64_t runs, int64_t *nr_out) {
        const int64_t V = (runs + RPR - 1) / RPR + 1;            // output rows touched (bound)
        const int64_t crossings = V <= 1 ? 0 : (V - 2) / a.OH + 1;
        int64_t NR = (V - 1) * S + K + crossings * gap;
        NR = std::min<int64_t>(NR, planes * Hp);
        const int64_t NP = std::min<int64_t>(crossings + 1, planes);
        *nr_out = NR;
        return NR * WP * les + NP * (K * K + 1) * (int64_t)sizeof(float);
    };
    int64_t passes = 8, nr = 0;
    while (passes > 1 && lds_for(passes * kThreads, &nr) > kLdsTarget) --passes;
    const int64_t bytes = lds_for(passes * kThreads, &nr);
    if (bytes > kLdsBudget) return pl;
    // Staging offsets (relative to the workgroup's first input plane) fit 31 bits.
    const int64_t V = (passes * kThreads + RPR - 1) / RPR + 1;
    const int64_t np_in = std::min<int64_t>(V <= 1 ? 1 : (V - 2) / a.OH + 2, planes);
    if ((np_in + 1) * a.H * a.W * es >= (int64_t(1) << 31)) return pl;
    g.C = (int)a.C; g.H = (int)a.H; g.W = (int)a.W; g.Cout = (int)a.Cout;
    g.OH = (int)a.OH; g.OW = (int)a.OW; g.ph = a.ph; g.pw = a.pw;
    g.Hp = (int)Hp;
    g.planes = (int)planes;
    g.WP = (int)WP;
    g.RPR = (int)RPR;
    g.CPR = (int)(a.W / pl.VI);
    g.npad = (int)(WP - a.W);
    g.runs_per_wg = (int)(passes * kThreads);
    g.total_runs = (int)total_runs;
    g.wgs = (int)ceil_div(total_runs, g.runs_per_wg);
    g.wgs_per_xcd = (int)ceil_div(g.wgs, 8);
    g.NRmax = (int)nr;
    g.st_c = kThreads % g.CPR;
    g.st_r = kThreads / g.CPR;
    g.st_rq = (int)(g.st_r / Hp);
    g.st_rm = (int)(g.st_r % Hp);
    g.st_off = (int)(g.st_rq * a.H * a.W + g.st_rm * a.W);
    g.st_wrap = (int)(a.H * a.W - Hp * a.W);
    g.fd_rpr = make_fastdiv((uint32_t)RPR);
    g.fd_oh = make_fastdiv((uint32_t)a.OH);
    g.fd_hp = make_fastdiv((uint32_t)Hp);
    g.fd_cpr = make_fastdiv((uint32_t)g.CPR);
    g.fd_cout = make_fastdiv((uint32_t)a.Cout);
    g.fd_m = make_fastdiv((uint32_t)(a.Cout / a.C));
    g.fd_npad = make_fastdiv((uint32_t)std::max(g.npad, 1));   // npad = 0: the pad loop is empty
    pl.K = K;
    pl.S = S;
    pl.lds = (size_t)bytes;
    pl.ok = true;
    return pl;
}

template <typename T, int K, int S, int R, int VI>
hipError_t run(const Conv2dArgs &a, const Plan &pl)
{
    const unsigned blocks = (unsigned)(8 * (int64_t)pl.g.wgs_per_xcd);
    hipLaunchKernelGGL((dw2d_rows<T, K, S, R, VI>), dim3(blocks), dim3(kThreads), pl.lds, a.stream,
                       (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, pl.g);
    return hipGetLastError();
}

template <typename T, int K, int S, int R>
hipError_t run_vi(const Conv2dArgs &a, const Plan &pl)
{
    return pl.VI > 1 ? run<T, K, S, R, 16 / sizeof(T)>(a, pl) : run<T, K, S, R, 1>(a, pl);
}

template <typename T, int K, int S>
hipError_t run_r(const Conv2dArgs &a, const Plan &pl)
{
    if constexpr (sizeof(T) == 2) {
        if (pl.R == 8) return run_vi<T, K, S, 8>(a, pl);
    }
    if (pl.R == 4) return run_vi<T, K, S, 4>(a, pl);
    if constexpr (S == 2) {
        if (pl.R == 2) return run_vi<T, K, S, 2>(a, pl);
    }
    return run_vi<T, K, S, 1>(a, pl);
}

template <typename T, int K>
hipError_t run_s(const Conv2dArgs &a, const Plan &pl)
{
    return pl.S == 2 ? run_r<T, K, 2>(a, pl) : run_r<T, K, 1>(a, pl);
}

template <typename T>
hipError_t run_typed(const Conv2dArgs &a, const Plan &pl)
{
    switch (pl.K) {
    case 3: return run_s<T, 3>(a, pl);
    case 5: return run_s<T, 5>(a, pl);
    default: return run_s<T, 7>(a, pl);
    }
}

struct BandPlan {
    BandGeom g;
    int K, S, KR;
    size_t lds;
    bool ok;
};

// Staged rows of a workgroup of spw strips at most (bound over all workgroups), and
// the LDS they and the filter table take.
int64_t band_rows(int64_t spw, int64_t SPP, int64_t Hp, int64_t planes, int KR, int S, int K)
{
    const int64_t NRW = (int64_t)(KR - 1) * S + K;
    const int64_t band = (int64_t)KR * S;
    // c plane boundaries crossed add c * (Hp - SPP * band) rows to (spw - 1) * band + NRW.
    const int64_t cmax = std::min<int64_t>(spw <= 1 ? 0 : (spw - 2) / SPP + 1, planes - 1);
    return (spw - 1) * band + NRW + std::max<int64_t>(0, cmax * (Hp - SPP * band));
}

BandPlan make_band_plan(const Conv2dArgs &a)
{
    BandPlan pl{};
    pl.ok = false;
    if (a.dtype == DT_F32) return pl;
    if (a.groups != a.C || a.KH != a.KW || (a.KH != 3 && a.KH != 5 && a.KH != 7)) return pl;
    if (a.sh != a.sw || (a.sh != 1 && a.sh != 2) || a.dh != 1 || a.dw != 1) return pl;
    if (a.ph > a.KH) return pl;
    if (a.interleaved && a.Cout != a.C) return pl;
    const int K = (int)a.KH, S = a.sh, R = 8 / S;
    // Full width: every chunk of a row starts one run (OW * S == W), and a row's
    // chunks fit in one wave.
    if (a.pw != (K - 1) / 2 || a.OW * S != a.W || a.W % 8 != 0 || a.W / 8 > 64) return pl;
    if (reinterpret_cast<uintptr_t>(a.x) % 16 != 0) return pl;
    if (reinterpret_cast<uintptr_t>(a.y) % (uintptr_t)(R * 2) != 0) return pl;
    const int64_t planes = a.N * a.Cout;
    const int64_t Hp = a.H + 2 * (int64_t)a.ph;
    const int CPR = (int)(a.W / 8), G = 64 / CPR, spw = 4 * G;
    const int KK1 = K * K + 1;
    // Two output rows per strip where the staged rows fit kLdsTarget (8 workgroups
    // per CU), else one; planes shorter than a strip would leave most of it empty.
    auto lds_for = [&](int KR, int64_t *units) {
        const int64_t SPP = ceil_div(a.OH, (int64_t)KR);
        const int64_t NR = std::min<int64_t>(band_rows(spw, SPP, Hp, planes, KR, S, K),
                                             planes * Hp + (int64_t)(KR - 1) * S + K);
        const int GAP = (int)(((int64_t)CPR * (1 - KR * S) % 8 + 8) % 8);
        *units = NR * CPR + (NR / (KR * S) + 1) * GAP;
        const int64_t NP = std::min<int64_t>(planes, (spw - 1) / SPP + 2);
        return *units * 16 + NP * KK1 * (int64_t)sizeof(float);
    };
    int64_t units = 0;
    int KR = 2;
    if (a.OH < 2 || lds_for(2, &units) > kLdsTarget) KR = 1;
    const int64_t bytes = lds_for(KR, &units);
    if (bytes > kLdsBudget) return pl;
    const int64_t SPP = ceil_div(a.OH, (int64_t)KR);
    const int64_t strips = planes * SPP;
    if (strips + spw >= (int64_t(1) << 31) || planes * Hp + 2 * K >= (int64_t(1) << 31)) return pl;
    // Offsets relative to a workgroup's first input / output plane fit 31 bits.
    const int64_t NP = std::min<int64_t>(planes, (spw - 1) / SPP + 2);
    if ((NP + 1) * a.H * a.W * 2 >= (int64_t(1) << 31) || (NP + 1) * a.OH * a.OW * 2 >= (int64_t(1) << 31)) return pl;
    BandGeom &g = pl.g;
    g.C = (int)a.C; g.H = (int)a.H; g.W = (int)a.W; g.Cout = (int)a.Cout;
    g.OH = (int)a.OH; g.OW = (int)a.OW; g.ph = a.ph;
    g.Hp = (int)Hp;
    g.planes = (int)planes;
    g.CPR = CPR;
    g.G = G;
    g.SPP = (int)SPP;
    g.strips = (int)strips;
    g.spw = spw;
    g.GAP = (int)(((int64_t)CPR * (1 - KR * S) % 8 + 8) % 8);
    g.units = (int)units;
    g.sp_p = (int)(4 * G / Hp);
    g.sp_hp = (int)(4 * G % Hp);
    g.step_off = (int)(g.sp_hp * a.W + (int64_t)g.sp_p * a.H * a.W);
    g.wrap_off = (int)(a.H * a.W - Hp * a.W);
    g.wgs = (int)ceil_div(strips, (int64_t)spw);
    g.wgs_per_xcd = (int)ceil_div(g.wgs, 8);
    g.fd_cpr = make_fastdiv((uint32_t)CPR);
    g.fd_spp = make_fastdiv((uint32_t)SPP);
    g.fd_hp = make_fastdiv((uint32_t)Hp);
    g.fd_cout = make_fastdiv((uint32_t)a.Cout);
    g.fd_m = make_fastdiv((uint32_t)(a.Cout / a.C));
    pl.K = K;
    pl.S = S;
    pl.KR = KR;
    pl.lds = (size_t)bytes;
    pl.ok = true;
    return pl;
}

template <typename T, int K, int S, int KR>
hipError_t run_band(const Conv2dArgs &a, const BandPlan &pl)
{
    const unsigned blocks = (unsigned)(8 * (int64_t)pl.g.wgs_per_xcd);
    hipLaunchKernelGGL((dw2d_band<T, K, S, KR>), dim3(blocks), dim3(kThreads), pl.lds, a.stream,
                       (const T *)a.x, (const T *)a.w, (const T *)a.bias, (T *)a.y, pl.g);
    return hipGetLastError();
}

template <typename T, int K, int S>
hipError_t run_band_kr(const Conv2dArgs &a, const BandPlan &pl)
{
    return pl.KR == 2 ? run_band<T, K, S, 2>(a, pl) : run_band<T, K, S, 1>(a, pl);
}

template <typename T>
hipError_t run_band_typed(const Conv2dArgs &a, const BandPlan &pl)
{
    switch (pl.K * 4 + pl.S) {
    case 13: return run_band_kr<T, 3, 1>(a, pl);
    case 14: return run_band_kr<T, 3, 2>(a, pl);
    case 21: return run_band_kr<T, 5, 1>(a, pl);
    case 22: return run_band_kr<T, 5, 2>(a, pl);
    case 29: return run_band_kr<T, 7, 1>(a, pl);
    default: return run_band_kr<T, 7, 2>(a, pl);
    }
}

}  // namespace

bool dw2d_supported(const Conv2dArgs &a) { return make_band_plan(a).ok || make_plan(a).ok; }

hipError_t launch_dw2d(const Conv2dArgs &a, const char **kname)
{
    const BandPlan bp = make_band_plan(a);
    if (bp.ok) {
        *kname = "dw2d_band";
        return a.dtype == DT_F16 ? run_band_typed<_Float16>(a, bp) : run_band_typed<__bf16>(a, bp);
    }
    const Plan pl = make_plan(a);
    if (!pl.ok) return hipErrorInvalidValue;
    *kname = "dw2d_rows";
    switch (a.dtype) {
    case DT_F32: return run_typed<float>(a, pl);
    case DT_F16: return run_typed<_Float16>(a, pl);
    default: return run_typed<__bf16>(a, pl);
    }
}

}  // namespace gconv
