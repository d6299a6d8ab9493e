// peaks.hip -- measurement kernels for the roofline figures of bench.py (built
// into libgconv_peaks.so, apart from the convolution library).
//
//  * mfma_loop: every wave issues back-to-back independent matrix-core
//    instructions on register operands (16 accumulators in turn), no memory
//    traffic: the MFMA rate the chip sustains, for v_mfma_f32_32x32x16_f16 and
//    v_mfma_f32_32x32x2_f32.  Wave 0 of workgroup 0 also reads the shader clock
//    counter (s_memtime) and the 100 MHz real-time counter (s_memrealtime) at its
//    start and end, which gives the core clock during the loop.
//  * stream_copy: a grid-stride copy with 16-byte loads (4 in flight per thread)
//    and non-temporal 16-byte stores: the HBM bandwidth a plain streaming kernel
//    reaches (read + write bytes).
//  * tile_copy: the copy of a (rows, channels) fp32 tensor in tiles of 32 rows x
//    64 channels, one workgroup of 256 threads per tile, each thread 2 x 16 bytes:
//    the grid and access pattern of the (batch, steps, channels) depthwise kernel's
//    tiles without the halo and the arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
    f32x16 acc[16];
    for (int j = 0; j < 16; ++j)
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    stamp_clocks(clk, 0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
    }
    stamp_clocks(clk, 1);
    float v = 0.0f;
    for (int j = 0; j < 16; ++j)
        for (int r = 0; r < 16; ++r) v += acc[j][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = v;
}

__global__ void __launch_bounds__(256) mfma_f32_loop(float *out, int iters, unsigned long long *clk)
{
    const float s = (float)(threadIdx.x & 7) * 1e-3f;
    const float a = s + 1.0f, b = s - 1.0f;
    f32x16 acc[16];
    for (int j = 0; j < 16; ++j)
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    stamp_clocks(clk, 0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[j], 0, 0, 0);
    }
    stamp_clocks(clk, 1);
    float v = 0.0f;
    for (int j = 0; j < 16; ++j)
        for (int r = 0; r < 16; ++r) v += acc[j][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = v;
}

__global__ void __launch_bounds__(256) stream_copy(const uint4 *__restrict__ src, uint4 *__restrict__ dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
        uint4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = src[i + k * stride];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v[k]), reinterpret_cast<u32x4 *>(dst + i + k * stride));
    }
    for (; i < n; i += stride)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, src[i]), reinterpret_cast<u32x4 *>(dst + i));
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

// FLOP of one workgroup of mfma loop `kind` (0: f16 32x32x16, 1: f32 32x32x2) with `iters` iterations.
double gconv_peak_mfma_flop(int kind, int iters)
{
    const double per = kind == 0 ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 2;
    return per * 16.0 * iters * 4.0;   // 16 instructions per iteration, 4 waves
}

// kind 0: fp16, 1: fp32.  out: blocks*256 floats; clk: 4 uint64 (memtime, realtime at start and end).
int gconv_peak_mfma(int kind, float *out, int blocks, int iters, unsigned long long *clk, void *stream)
{
    if (blocks < 1 || iters < 1 || !out || !clk) return 1;
    if (kind == 0)
        hipLaunchKernelGGL(mfma_f16_loop, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, clk);
    else
        hipLaunchKernelGGL(mfma_f32_loop, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters, clk);
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

// Copies n16 16-byte pieces (src, dst 16-byte aligned, not overlapping).
int gconv_peak_stream_copy(const void *src, void *dst, int64_t n16, int blocks, void *stream)
{
    if (blocks < 1 || n16 < 0 || !src || !dst) return 1;
    hipLaunchKernelGGL(stream_copy, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const uint4 *)src,
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
