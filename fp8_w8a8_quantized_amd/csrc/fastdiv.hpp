// fastdiv.hpp -- exact division of 31-bit indices by a runtime divisor.
//
// Plain C++ (host and device), so the same code compiles for the host check
// in tests/native/fastdiv_check.cpp and for the kernels.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define FP8_FD_HD __host__ __device__
#else
#define FP8_FD_HD
#endif

namespace fp8k {

// Division by a runtime divisor d >= 1 of any n in [0, 2^31): with
// l = ceil(log2 d) and m = ceil(2^(31+l) / d), which fits in 32 bits,
// floor(n / d) = (n * m) >> (31 + l) exactly.  (m d = 2^(31+l) + e with
// 0 <= e < d, so n m / 2^(31+l) = n / d + n e / (d 2^(31+l)), and the second
// term is below 2^31 d / (d 2^(31+l)) = 2^-l <= 1 / d: it never reaches the
// next integer.)  One 32 x 32 -> 64-bit multiply and a shift instead of the
// ~15 instructions of an integer division.
struct FastDiv {
    uint32_t m;
    int sh;
};

inline FastDiv fast_div(int64_t d) {  // host side, d in [1, 2^31); d < 1 is taken as 1
    if (d < 1) d = 1;
    int l = 0;
    while ((int64_t(1) << l) < d) ++l;
    const unsigned __int128 num = (unsigned __int128)1 << (31 + l);
    const uint64_t m = (uint64_t)((num + (unsigned __int128)(d - 1)) / (unsigned __int128)d);
    return FastDiv{(uint32_t)m, 31 + l};
}

FP8_FD_HD inline uint32_t fdiv(uint32_t n, const FastDiv& f) {
    return (uint32_t)(((uint64_t)n * f.m) >> f.sh);
}

}  // namespace fp8k
