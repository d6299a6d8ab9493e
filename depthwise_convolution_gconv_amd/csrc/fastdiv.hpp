// fastdiv.hpp -- exact division of 31-bit non-negative integers by a runtime
// divisor, by multiplication with a precomputed reciprocal (the round-up method of
// Granlund and Montgomery, "Division by invariant integers using multiplication",
// PLDI 1994).  The neon issue "Grouped convolutions" describes the same device for
// unpacking grid indices (blockIdx.z * magic >> shift).
//
// For a divisor 1 <= d < 2^31 let l = ceil(log2 d) and m = floor(2^(31+l) / d) + 1
// (m < 2^33).  For every 0 <= n < 2^31:  floor(n / d) == (n * m) >> (31 + l).
// Proof sketch: n*m / 2^(31+l) = n/d + e with 0 < e <= n / 2^(31+l) < 2^-l <= 1/d,
// and n/d = q + r/d with r <= d-1, so q <= n/d + e < q + 1.
#pragma once

#include <stdint.h>

namespace gconv {

struct FastDiv {
    uint64_t mul;
    uint32_t shift;
    uint32_t d;
};

#if defined(__HIPCC__) || defined(__HIP__)
#define GCONV_HD __host__ __device__
#else
#define GCONV_HD
#endif

inline FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f;
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    f.d = d;
    f.shift = 31 + l;
    f.mul = ((uint64_t(1) << f.shift) / d) + 1;
    return f;
}

// floor(n / f.d) for 0 <= n < 2^31.
GCONV_HD inline int fdiv(int n, const FastDiv &f)
{
    return (int)(((uint64_t)(uint32_t)n * f.mul) >> f.shift);
}

// n % f.d given q = fdiv(n, f).
GCONV_HD inline int fmod_q(int n, int q, const FastDiv &f) { return n - q * (int)f.d; }

}  // namespace gconv
