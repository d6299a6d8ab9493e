// common.hpp -- shared definitions of the HIP side of libgconv (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gconv {

// Geometry of one NCHW grouped conv2d call, validated on the host.
struct Conv2dArgs {
    const void *x;
    const void *w;
    const void *bias;  // nullptr: no bias
    void *y;
    int64_t N, C, H, W;
    int64_t Cout, KH, KW;
    int64_t groups;
    int64_t OH, OW;
    int32_t sh, sw, ph, pw, dh, dw;
    int dtype;  // gconv_dtype_t
    int interleaved;  // 1: filter j of group k is stored at output channel j*groups + k
    hipStream_t stream;
};

// Geometry of one depthwise conv1d call over (batch, steps, channels).
struct Dw1dArgs {
    const void *x;
    const void *w;
    const void *bias;
    void *y;
    int64_t B, T, C, K, To;
    int32_t s, p, d;
    int dtype;
    hipStream_t stream;
};

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// Storage <-> fp32.  Widening is exact for every storage type; narrowing
// rounds to nearest, ties to even (v_cvt_f16_f32 / v_cvt_pk_bf16_f32).
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(_Float16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(__bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float v) { return (_Float16)v; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float v) { return (__bf16)v; }

// Output stores that do not keep the written lines in L2 (non-temporal): outputs are
// written once and not read again by the kernel, while the inputs a tile shares with
// its neighbours (halo rows, filters) are.  Measured on the Conformer depthwise
// conv1d: 12.1 -> 9.3 us.
typedef uint32_t gconv_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t gconv_u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_nt(uint4 *p, uint4 v)
{
    __builtin_nontemporal_store(__builtin_bit_cast(gconv_u32x4, v), reinterpret_cast<gconv_u32x4 *>(p));
}
__device__ __forceinline__ void store_nt(uint2 *p, uint2 v)
{
    __builtin_nontemporal_store(__builtin_bit_cast(gconv_u32x2, v), reinterpret_cast<gconv_u32x2 *>(p));
}
__device__ __forceinline__ void store_nt(uint32_t *p, uint32_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_nt(float *p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_nt(_Float16 *p, _Float16 v)
{
    __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, v), reinterpret_cast<uint16_t *>(p));
}
__device__ __forceinline__ void store_nt(__bf16 *p, __bf16 v)
{
    __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, v), reinterpret_cast<uint16_t *>(p));
}

// Launchers (each returns the launch status and the kernel name it picked).
hipError_t launch_direct2d(const Conv2dArgs &a, const char **kname);
bool dw2d_supported(const Conv2dArgs &a);
hipError_t launch_conv2d_nhwc(const Conv2dArgs &a, const char **kname);   // x, w, y channels-last
bool igemm_nhwc_supported(const Conv2dArgs &a);       // channels-last, fp16 / bf16
hipError_t launch_igemm_nhwc(const Conv2dArgs &a, const char **kname);             // depthwise K x K, stride 1 or 2
hipError_t launch_dw2d(const Conv2dArgs &a, const char **kname);
bool igemm_supported(const Conv2dArgs &a);            // fp16 / bf16
hipError_t launch_igemm(const Conv2dArgs &a, const char **kname);
bool igemm_rows_supported(const Conv2dArgs &a);       // fp16 / bf16, 3x3, unit column stride and dilation
hipError_t launch_igemm_rows(const Conv2dArgs &a, const char **kname);
bool igemm_defer_supported(const Conv2dArgs &a);      // fp16 / bf16, 3x3, 33-64 filters per group
hipError_t launch_igemm_defer(const Conv2dArgs &a, const char **kname);
bool igemm_f32_supported(const Conv2dArgs &a);        // fp32
hipError_t launch_igemm_f32(const Conv2dArgs &a, const char **kname);
hipError_t launch_dw1d(const Dw1dArgs &a, const char **kname);
// Backward of the depthwise conv1d (a: the forward geometry; a.x, a.y, a.bias unused).
hipError_t launch_dw1d_bwd_data(const Dw1dArgs &a, const void *dy, void *dx, const char **kname);
bool dw1d_wgrad_plan(const Dw1dArgs &a, size_t *ws_bytes);
hipError_t launch_dw1d_bwd_filter(const Dw1dArgs &a, const void *x, const void *dy, void *dw, void *db,
                                  void *ws, const char **kname);
// Size of the library's own device scratch for the filter gradient (one copy per
// GPU), and its device address on the current device (looked up once per device;
// no allocation).
constexpr size_t kWgradScratchBytes = size_t(16) << 20;
hipError_t wgrad_scratch(void **addr);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace gconv
