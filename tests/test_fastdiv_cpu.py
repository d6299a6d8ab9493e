"""Host check of the multiply-and-shift division the kernels use for index
unpacking (csrc/fastdiv.hpp): exact floor division for every numerator below 2^31,
checked against the C++ '/' operator on edge values and random samples."""
import os
import subprocess
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "depthwise_convolution_gconv_amd", "csrc")

PROG = r'''
#include <cstdio>
#include <cstdint>
#include <random>
#include "fastdiv.hpp"
int main() {
    std::mt19937_64 rng(12345);
    const int64_t top = (int64_t(1) << 31) - 1;
    uint32_t ds[] = {1, 2, 3, 5, 7, 28, 30, 49, 196, 256, 258, 784, 1000, 65535, 65536, 65537,
                     (1u << 30) - 1, 1u << 30, (1u << 30) + 1, (1u << 31) - 1};
    long bad = 0, n_checked = 0;
    auto check = [&](int64_t n, uint32_t d, const gconv::FastDiv &f) {
        ++n_checked;
        const int q = gconv::fdiv((int)n, f);
        if (q != (int)(n / d) || gconv::fmod_q((int)n, q, f) != (int)(n % d)) ++bad;
    };
    for (int rep = 0; rep < 2000; ++rep) {
        uint32_t d = rep < 20 ? ds[rep] : (uint32_t)(rng() % top) + 1;
        if (rep >= 20 && rep % 3 == 0) d = (uint32_t)(rng() % 4096) + 1;
        const gconv::FastDiv f = gconv::make_fastdiv(d);
        for (int64_t n : {int64_t(0), int64_t(1), int64_t(d) - 1, int64_t(d), int64_t(d) + 1,
                          top, top - 1, top - int64_t(top % d), top - int64_t(top % d) - 1})
            if (n >= 0 && n <= top) check(n, d, f);
        for (int i = 0; i < 2000; ++i) check((int64_t)(rng() % (top + 1)), d, f);
        for (int64_t m = 1; m < 64 && m * d <= top; ++m) { check(m * d - 1, d, f); check(m * d, d, f); }
    }
    std::printf("%ld %ld\n", n_checked, bad);
    return bad != 0;
}
'''


def test_fastdiv_is_exact_below_2_pow_31():
    with tempfile.TemporaryDirectory() as td:
        src = os.path.join(td, "t.cpp")
        exe = os.path.join(td, "t")
        open(src, "w").write(PROG)
        subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True)
        checked, bad = map(int, out.stdout.split())
        assert checked > 4_000_000 and bad == 0, out.stdout


def test_small_multiply_shift_division_is_exact():
    # The fully grouped 3x3 kernel divides positions q < 2048 by an image row width
    # d <= 400 as (q * ceil(2^20 / d)) >> 20; every pair of that range is checked.
    import numpy as np
    q = np.arange(2048, dtype=np.uint64)
    for d in range(1, 401):
        m = np.uint64(((1 << 20) + d - 1) // d)
        assert np.array_equal((q * m) >> np.uint64(20), q // np.uint64(d)), d
