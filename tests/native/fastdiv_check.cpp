// Host check of fastdiv.hpp: floor(n / d) for n in [0, 2^31) by the kernels'
// multiply and shift, against the integer division, over every divisor up to
// 4096 (boundary and random dividends) and random divisors up to 2^31 - 1.
#include <cstdint>
#include <cstdio>
#include <random>

#include "../../fp8_w8a8_quantized_amd/csrc/fastdiv.hpp"

using fp8k::fast_div;
using fp8k::fdiv;

int main() {
    std::mt19937_64 rng(12345);
    long bad = 0, tests = 0;
    auto chk = [&](int64_t d, uint32_t n) {
        ++tests;
        if (fdiv(n, fast_div(d)) != n / (uint64_t)d && bad++ < 5)
            std::printf("d=%lld n=%u: %u, expected %llu\n", (long long)d, n, fdiv(n, fast_div(d)),
                        (unsigned long long)(n / (uint64_t)d));
    };
    auto around_multiples = [&](int64_t d) {
        for (int k = 0; k < 64; ++k) {
            const uint64_t q = rng() % (0x7FFFFFFFull / (uint64_t)d + 1), n = q * (uint64_t)d;
            if (n < 0x80000000ull) {
                chk(d, (uint32_t)n);
                if (n) chk(d, (uint32_t)(n - 1));
            }
        }
    };
    for (int64_t d = 1; d <= 4096; ++d) {
        for (uint32_t n : {0u, 1u, (uint32_t)d - 1, (uint32_t)d, (uint32_t)d + 1, 0x7FFFFFFEu,
                           0x7FFFFFFFu})
            chk(d, n);
        for (int k = 0; k < 256; ++k) chk(d, (uint32_t)(rng() & 0x7FFFFFFF));
        around_multiples(d);
    }
    for (int k = 0; k < 100000; ++k) {
        const int64_t d = 1 + (int64_t)(rng() % 0x7FFFFFFEull);
        chk(d, (uint32_t)(rng() & 0x7FFFFFFF));
        chk(d, 0x7FFFFFFFu);
        around_multiples(d);
    }
    std::printf("%ld cases, %ld wrong\n", tests, bad);
    return bad != 0;
}
