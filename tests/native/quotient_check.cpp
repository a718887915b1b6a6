// Exhaustive host check of the quantizers' element quotient.
//
// For every positive finite bf16 amax, s = amax / 448 (IEEE fp32) and every
// finite bf16 x with |x| <= amax, the reciprocal-corrected quotient used by
// the GPU kernels must equal the IEEE quotient x / s bit for bit, or both
// quotients must be below 2^-11 in magnitude with the same sign (there every
// E4M3 code is a signed zero).  Groups whose scale is below the corrected
// path's bound do not use it and are skipped.  Prints the number of pairs checked and the
// number of mismatches, and exits non-zero on any mismatch.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../fp8_w8a8_quantized_amd/csrc/quotient.hpp"

static float from_bits(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

int main() {
    unsigned long long checked = 0, bad = 0, tiny = 0;
    volatile float d448 = 448.0f;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : checked, bad, tiny)
    for (int ai = 1; ai < 0x7F80; ++ai) {
        float amax = from_bits((uint32_t)ai << 16);
        float s = amax / d448;
        if (!fp8q::scale_has_fast_path(s)) continue;
        volatile float one = 1.0f;
        float r = one / s;
        for (int xi = 0; xi <= ai; ++xi) {
            for (int sg = 0; sg < 2; ++sg) {
                float x = from_bits(((uint32_t)xi << 16) | (sg ? 0x80000000u : 0u));
                float ref = x / s;
                float got = fp8q::quotient(x, s, r);
                ++checked;
                if (to_bits(ref) == to_bits(got)) continue;
                if (std::fabs(ref) < 0x1p-11f && std::fabs(got) < 0x1p-11f &&
                    std::signbit(ref) == std::signbit(got)) { ++tiny; continue; }
                ++bad;
            }
        }
    }
    std::printf("checked %llu pairs, tiny-equivalent %llu, mismatches %llu\n", checked, tiny, bad);
    return bad == 0 ? 0 : 1;
}
