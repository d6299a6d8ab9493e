// peaks.hip -- measurement kernels for the roofline figures of bench.py (built
// into libgconv_peaks.so, apart from the convolution library).
//
//  * mfma loops: every wave issues back-to-back independent matrix-core
//    instructions on register operands (8 or 16 accumulators in turn, each
//    started from its own values so that no two chains are the same), no memory
//    traffic: the rate the chip sustains for v_mfma_f32_32x32x16_f16,
//    v_mfma_f32_32x32x2_f32 and the 16-block v_mfma_f32_4x4x4_f16 /
//    v_mfma_f32_4x4x4_bf16 (the instructions of the implicit-GEMM and the
//    fully grouped direct kernels).  Wave 0 of workgroup 0 also reads the shader
//    clock counter (s_memtime) and the 100 MHz real-time counter (s_memrealtime)
//    at its start and end, which gives the core clock during the loop.
//  * valu_fma_loop / valu_dot2_loop: the same for plain (non-packed) fp32 FMA
//    and for v_dot2_f32_f16 (two 16-bit products added to an fp32 sum) on the
//    vector ALUs, the arithmetic of the direct kernels.
//  * stream_copy: one non-temporal 16-byte load and store per thread
//    over the whole buffer (of the layouts tried -- grid-stride loops with 4 pieces
//    in flight, 2 to 8 pieces per thread, plain or non-temporal loads and stores --
//    the fastest for a 1 GiB copy): the HBM bandwidth a plain streaming kernel
//    reaches (read + write bytes).
//  * tile_copy: the copy of a (rows, channels) fp32 tensor in tiles of 32 rows x
//    64 channels, one workgroup of 256 threads per tile, each thread 2 x 16 bytes
//    (plain loads, which measured faster here than non-temporal ones; non-temporal
//    stores):
//    the grid and access pattern of the (batch, steps, channels) depthwise kernel's
//    tiles without the halo and the arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void stamp_clocks(unsigned long long *clk, int slot)
{
    const unsigned long long t = __builtin_amdgcn_s_memtime();
    const unsigned long long r = __builtin_amdgcn_s_memrealtime();
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        clk[2 * slot] = t;
        clk[2 * slot + 1] = r;
    }
}

__global__ void __launch_bounds__(256) mfma_f16_loop(float *out, int iters, unsigned long long *clk)
{
    // Operands from the thread index, so nothing folds at compile time.
    const float s = (float)(threadIdx.x & 7) * 1e-3f;
    f16x8 a, b;
    for (int i = 0; i < 8; ++i) { a[i] = (_Float16)(s + i); b[i] = (_Float16)(s - i); }
    f32x16 acc[8];
    for (int j = 0; j < 8; ++j)
        for (int r = 0; r < 16; ++r) acc[j][r] = s + (float)(j * 16 + r);
    stamp_clocks(clk, 0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j & 7] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j & 7], 0, 0, 0);
    }
    stamp_clocks(clk, 1);
    float v = 0.0f;
    for (int j = 0; j < 8; ++j)
        for (int r = 0; r < 16; ++r) v += acc[j][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = v;
}

__global__ void __launch_bounds__(256) mfma_f32_loop(float *out, int iters, unsigned long long *clk)
{
    const float s = (float)(threadIdx.x & 7) * 1e-3f;
    const float a = s + 1.0f, b = s - 1.0f;
    f32x16 acc[8];
    for (int j = 0; j < 8; ++j)
        for (int r = 0; r < 16; ++r) acc[j][r] = s + (float)(j * 16 + r);
    stamp_clocks(clk, 0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j & 7] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[j & 7], 0, 0, 0);
    }
    stamp_clocks(clk, 1);
    float v = 0.0f;
    for (int j = 0; j < 8; ++j)
        for (int r = 0; r < 16; ++r) v += acc[j][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = v;
}

__global__ void __launch_bounds__(256) mfma_4x4_loop(float *out, int iters, unsigned long long *clk, int bf16)
{
    const float s = (float)(threadIdx.x & 7) * 1e-3f;
    f16x4 a, b;
    s16x4 ab, bb;
    for (int i = 0; i < 4; ++i) {
        a[i] = (_Float16)(s + i);
        b[i] = (_Float16)(s - i);
        ab[i] = (short)(0x3f80 + (threadIdx.x & 7) + i);
        bb[i] = (short)(0x3f00 + (threadIdx.x & 7) - i);
    }
    f32x4 acc[16];
    for (int j = 0; j < 16; ++j)
        for (int r = 0; r < 4; ++r) acc[j][r] = s + (float)(j * 4 + r);
    stamp_clocks(clk, 0);
    if (bf16) {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ab, bb, acc[j], 0, 0, 0);
        }
    } else {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, acc[j], 0, 0, 0);
        }
    }
    stamp_clocks(clk, 1);
    float v = 0.0f;
    for (int j = 0; j < 16; ++j)
        for (int r = 0; r < 4; ++r) v += acc[j][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = v;
}

__global__ void __launch_bounds__(256) valu_fma_loop(float *out, int iters, unsigned long long *clk)
{
    const float s = (float)(threadIdx.x & 7) * 1e-3f;
    const float a = 1.0f + s * 1e-3f, b = s;
    float acc[16];
    for (int j = 0; j < 16; ++j) acc[j] = s + j;
    stamp_clocks(clk, 0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = __builtin_fmaf(acc[j], a, b);
    }
    stamp_clocks(clk, 1);
    float v = 0.0f;
    for (int j = 0; j < 16; ++j) v += acc[j];
    out[blockIdx.x * blockDim.x + threadIdx.x] = v;
}

__global__ void __launch_bounds__(256) valu_dot2_loop(float *out, int iters, unsigned long long *clk)
{
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const float s = (float)(threadIdx.x & 7) * 1e-3f;
    h2 a, b;
    a[0] = (_Float16)(1.0f + s);
    a[1] = (_Float16)(s);
    b[0] = (_Float16)(1e-3f);
    b[1] = (_Float16)(-1e-3f);
    float acc[16];
    for (int j = 0; j < 16; ++j) acc[j] = s + j;
    stamp_clocks(clk, 0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_fdot2(a, b, acc[j], false);
    }
    stamp_clocks(clk, 1);
    float v = 0.0f;
    for (int j = 0; j < 16; ++j) v += acc[j];
    out[blockIdx.x * blockDim.x + threadIdx.x] = v;
}

// One 16-byte piece per thread, non-temporal load and store; the grid covers the
// buffer once.
__global__ void __launch_bounds__(256) stream_copy(const uint4 *__restrict__ src, uint4 *__restrict__ dst, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + i)),
                                    reinterpret_cast<u32x4 *>(dst + i));
}

// rows x C fp32, C a multiple of 64 and rows a multiple of 32 (checked by the launcher).
__global__ void __launch_bounds__(256) tile_copy(const float *__restrict__ src, float *__restrict__ dst, int C,
                                                 int cblocks)
{
    const int cb = blockIdx.x % cblocks, tb = blockIdx.x / cblocks;
    const int t = threadIdx.x;
    // 32 rows x 64 channels = 512 pieces of 16 bytes; thread t takes pieces t and t + 256.
    int64_t off[2];
    uint4 v[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int p = t + 256 * k, row = p >> 4, c4 = (p & 15) * 4;
        off[k] = ((int64_t)tb * 32 + row) * C + cb * 64 + c4;
        v[k] = *reinterpret_cast<const uint4 *>(src + off[k]);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v[k]), reinterpret_cast<u32x4 *>(dst + off[k]));
}

}  // namespace

extern "C" {

// Loop kinds: 0 fp16 32x32x16 MFMA, 1 fp32 32x32x2 MFMA, 2 fp16 4x4x4 (16 blocks)
// MFMA, 3 bf16 4x4x4 (16 blocks) MFMA, 4 fp32 FMA on the vector ALUs, 5 v_dot2_f32_f16
// on the vector ALUs.
// FLOP of one workgroup of loop `kind` with `iters` iterations (-1 for an unknown kind).
double gconv_peak_mfma_flop(int kind, int iters)
{
    double per;
    switch (kind) {
    case 0: per = 2.0 * 32 * 32 * 16; break;
    case 1: per = 2.0 * 32 * 32 * 2; break;
    case 2:
    case 3: per = 2.0 * 16 * 4 * 4 * 4; break;
    case 4: per = 2.0 * 64; break;
    case 5: per = 4.0 * 64; break;
    default: return -1.0;
    }
    return per * 16.0 * iters * 4.0;   // 16 instructions per iteration, 4 waves
}

// out: blocks*256 floats; clk: 4 uint64 (memtime, realtime at start and end).
int gconv_peak_mfma(int kind, float *out, int blocks, int iters, unsigned long long *clk, void *stream)
{
    if (blocks < 1 || iters < 1 || !out || !clk || kind < 0 || kind > 5) return 1;
    const hipStream_t st = (hipStream_t)stream;
    switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_f16_loop, dim3(blocks), dim3(256), 0, st, out, iters, clk); break;
    case 1: hipLaunchKernelGGL(mfma_f32_loop, dim3(blocks), dim3(256), 0, st, out, iters, clk); break;
    case 2:
    case 3: hipLaunchKernelGGL(mfma_4x4_loop, dim3(blocks), dim3(256), 0, st, out, iters, clk, kind == 3); break;
    case 4: hipLaunchKernelGGL(valu_fma_loop, dim3(blocks), dim3(256), 0, st, out, iters, clk); break;
    default: hipLaunchKernelGGL(valu_dot2_loop, dim3(blocks), dim3(256), 0, st, out, iters, clk); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// Copies n16 16-byte pieces (src, dst 16-byte aligned, not overlapping).
int gconv_peak_stream_copy(const void *src, void *dst, int64_t n16, void *stream)
{
    if (n16 < 1 || !src || !dst) return 1;
    const int64_t blocks = (n16 + 255) / 256;
    if (blocks >= (int64_t(1) << 31)) return 1;
    hipLaunchKernelGGL(stream_copy, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, (const uint4 *)src,
                       (uint4 *)dst, n16);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// Copies a rows x C fp32 tensor in 32 x 64 tiles (rows % 32 == 0, C % 64 == 0, 16-byte aligned).
int gconv_peak_tile_copy(const float *src, float *dst, int64_t rows, int C, void *stream)
{
    if (!src || !dst || rows < 32 || rows % 32 != 0 || C < 64 || C % 64 != 0) return 1;
    const int64_t blocks = rows / 32 * (C / 64);
    if (blocks >= (int64_t(1) << 31)) return 1;
    hipLaunchKernelGGL(tile_copy, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, src, dst, C, C / 64);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
