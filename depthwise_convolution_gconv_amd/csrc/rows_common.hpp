// rows_common.hpp -- device helpers shared by the run-per-lane implicit-GEMM
// kernels (igemm_rows.hip, igemm_defer.hip): MFMA wrappers, 16-bit packing, buffer
// resources, the filter-image map and the input row loads.  Included inside each
// kernel file's unnamed namespace.
#pragma once

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#define GCONV_LDS(p) ((__attribute__((address_space(3))) void *)(p))

constexpr int kLdsUnits = 160 * 1024 / 16;   // 16-byte units of LDS per workgroup (one per CU)

constexpr uint32_t kOOB = 0x80000000u;       // byte offset past num_records: loads return 0, stores drop
constexpr int kNT = 2;                       // cache policy of the output stores: non-temporal

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

template <typename T> __device__ __forceinline__ float half_to_f32(uint32_t hbits);
template <> __device__ __forceinline__ float half_to_f32<_Float16>(uint32_t hbits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)hbits);
}
template <> __device__ __forceinline__ float half_to_f32<__bf16>(uint32_t hbits)
{
    return __builtin_bit_cast(float, hbits << 16);
}
// Two fp32 values rounded to nearest even into one dword of T (a in the low half).
template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<_Float16>(float a, float b)
{
    return __builtin_bit_cast(uint32_t, f16x2{(_Float16)a, (_Float16)b});
}
template <> __device__ __forceinline__ uint32_t pack2<__bf16>(float a, float b)
{
    return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
}

// One accumulator copied out of its accumulation register at this point of the
// program (otherwise the allocator moves all of them into VGPRs at once).
__device__ __forceinline__ float acc_read(float v)
{
    float r;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(v));
    return r;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Filter image: per 16-filter half-block, per tap, 32 units; filter f (< 16) and
// channel half hh at unit 2f + (hh ^ bit 3 of f).  The A-operand read (16 lanes on
// 16 consecutive filters, one channel half) and the transposing write (16 lanes on
// 8 filters x 2 halves) both hit 16 different units modulo 16.
__device__ __forceinline__ int fimg_unit(int f, int hh) { return 2 * f + (hh ^ ((f >> 3) & 1)); }

// VW consecutive 16-bit elements of one input row, as VW/2 dwords.
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
