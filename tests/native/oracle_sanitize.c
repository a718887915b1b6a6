/*
 * oracle_sanitize.c -- drives every function of the CPU oracle
 * (oracle/fp8_oracle.c) on small inputs held in buffers of exactly the sizes
 * the functions may touch, so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer turns any out-of-bounds access, overflow or
 * other undefined behaviour into a failure.  It also checks results that the
 * number formats fix on their own (landmark codes and values, exact scales,
 * closed-form RMSNorm), so a sanitized build that computes something else
 * fails as well.  Exit status 0: every check passed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/fp8_oracle.h"

static int failures = 0;
#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

static uint16_t bf16_of(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16); /* exact for the values used here */
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}

/* deterministic bf16 values in about [-8, 8], with a few zeros */
static void fill(uint16_t* x, int64_t n, uint32_t seed) {
    uint32_t s = seed * 2654435761u + 1u;
    for (int64_t i = 0; i < n; ++i) {
        s = s * 1664525u + 1013904223u;
        float v = ((float)(s >> 8) / 16777216.0f - 0.5f) * 16.0f;
        x[i] = (s & 63) == 0 ? 0 : bf16_of(v);
    }
}

static void codec(void) {
    CHECK(orc_e4m3_decode(0x7E) == 448.0);
    CHECK(orc_e4m3_decode(0x08) == ldexp(1.0, -6));
    CHECK(orc_e4m3_decode(0x01) == ldexp(1.0, -9));
    CHECK(orc_e4m3_decode(0x80) == 0.0 && signbit(orc_e4m3_decode(0x80)));
    CHECK(isnan(orc_e4m3_decode(0x7F)) && isnan(orc_e4m3_decode(0xFF)));
    for (int c = 0; c < 256; ++c) {
        if ((c & 0x7F) == 0x7F) continue;
        const float v = (float)orc_e4m3_decode((uint8_t)c);
        CHECK(orc_e4m3_encode(v) == c);
        CHECK(orc_e4m3_encode_bits(v) == c);
    }
    CHECK(orc_e4m3_encode(1e30f) == 0x7E && orc_e4m3_encode(-1e30f) == 0xFE);
    /* the two encoders agree on a strided slice of all fp32 patterns */
    CHECK(orc_e4m3_encoders_disagree(0x3F000000ull, 0x3F000000ull + (1u << 20)) == 0);
    CHECK(orc_e4m3_encoders_disagree(0xC3000000ull, 0xC3000000ull + (1u << 20)) == 0);
    float v[5] = {0.0f, -0.0f, 448.0f, 1e-9f, -300.0f};
    uint8_t* out = xmalloc(5);
    orc_e4m3_encode_array(v, 5, out);
    CHECK(out[0] == 0x00 && out[1] == 0x80 && out[2] == 0x7E && out[3] == 0x00);
    free(out);
}

static void bf16_and_scales(void) {
    CHECK(orc_bf16_to_f32(0x3F80) == 1.0f);
    CHECK(orc_f32_to_bf16_rne(1.0f + ldexpf(1.0f, -8)) == 0x3F80);     /* tie to even */
    CHECK(orc_f32_to_bf16_rne(1.0f + 3 * ldexpf(1.0f, -8)) == 0x3F82); /* tie to even */
    float f[3] = {1.0f, -2.5f, 0.0f};
    uint16_t* b = xmalloc(3 * sizeof(uint16_t));
    orc_bf16_rne_array(f, 3, b);
    CHECK(b[0] == 0x3F80 && b[1] == 0xC020 && b[2] == 0);
    free(b);
    CHECK(orc_scale_f32(448.0f) == 1.0f);
    CHECK(orc_scale_f32(0.0f) == 0.0f);
    CHECK(orc_e8m0_exponent(1.0f) == 0 && orc_e8m0_exponent(1.5f) == 1);
    CHECK(orc_e8m0_exponent(0.0f) == -127 && orc_e8m0_exponent(0.25f) == -2);
    float* p2 = xmalloc(255 * sizeof(float));
    uint8_t* codes = xmalloc(255);
    for (int e = -127; e <= 127; ++e) p2[e + 127] = ldexpf(1.0f, e);
    CHECK(orc_e8m0_lossless(p2, 255, codes) == 1);
    for (int e = -127; e <= 127; ++e) CHECK(codes[e + 127] == e + 127);
    p2[3] = 3.0f;
    CHECK(orc_e8m0_lossless(p2, 255, codes) == 0);
    free(p2);
    free(codes);
}

static void quantizers(void) {
    const int64_t M = 3, K = 384, N = 256;
    uint16_t* x = xmalloc(M * K * 2);
    fill(x, M * K, 1);
    for (int64_t k = 128; k < 256; ++k) x[k] = 0;  /* an all-zero group */
    x[1] = bf16_of(448.0f);                        /* group 0 has amax 448: scale 1 */
    uint8_t* q = xmalloc(M * K);
    float* s = xmalloc(M * (K / 128) * sizeof(float));
    orc_quantize_block(x, M, K, q, s);
    CHECK(s[0] == 1.0f && s[1] == 0.0f);
    for (int64_t k = 0; k < 128; ++k) CHECK(q[k] == orc_e4m3_encode(orc_bf16_to_f32(x[k])));
    for (int64_t k = 128; k < 256; ++k) CHECK(q[k] == 0);
    uint8_t* s8 = xmalloc(M * (K / 128));
    orc_quantize_block_e8m0(x, M, K, q, s8);
    CHECK(s8[0] == 127 && s8[1] == 0);
    float* st = xmalloc(M * sizeof(float));
    orc_quantize_token(x, M, K, q, st);
    CHECK(st[0] == 1.0f);
    float one;
    orc_quantize_tensor(x, M * K, q, &one);
    CHECK(one >= 1.0f);
    free(s8);
    free(st);

    uint16_t* w = xmalloc(N * K * 2);
    fill(w, N * K, 2);
    uint8_t* qw = xmalloc(N * K);
    float* sw = xmalloc((N / 128) * (K / 128) * sizeof(float));
    uint8_t* sw8 = xmalloc((N / 128) * (K / 128));
    orc_quantize_weight_block(w, N, K, 0, qw, sw);
    orc_quantize_weight_block(w, N, K, 1, qw, sw8);
    for (int64_t i = 0; i < (N / 128) * (K / 128); ++i)
        CHECK(sw[i] > 0.0f && ldexpf(1.0f, sw8[i] - 127) >= sw[i]);
    free(w);
    free(qw);
    free(sw);
    free(sw8);
    free(x);
    free(q);
    free(s);
}

static void rmsnorm(void) {
    const int64_t M = 2, K = 520; /* K % 8 == 0, not a multiple of 512 */
    uint16_t* x = xmalloc(M * K * 2);
    uint16_t* g = xmalloc(K * 2);
    uint16_t* y = xmalloc(M * K * 2);
    for (int64_t i = 0; i < M * K; ++i) x[i] = 0x3F80; /* 1.0 */
    for (int64_t i = 0; i < K; ++i) g[i] = 0x3F80;
    CHECK(orc_rms_sumsq(x, K) == (float)K);
    orc_rmsnorm_bf16(x, g, 1e-6f, M, K, y);
    CHECK(y[0] == 0x3F80 && y[M * K - 1] == 0x3F80); /* 1 / sqrt(1 + 1e-6) rounds to 1 */
    uint8_t* q = xmalloc(M * K);
    float* s = xmalloc(M * sizeof(float));
    orc_rmsnorm_quant(x, g, 1e-6f, M, K, q, s);
    for (int64_t i = 0; i < M * K; ++i) CHECK(q[i] == 0x7E);
    free(q);
    free(s);
    free(x);
    free(g);
    free(y);
}

static void elementwise(void) {
    const int64_t n = 1 << 16;
    uint16_t* g = xmalloc(n * 2);
    float* sl = xmalloc(n * sizeof(float));
    for (int64_t i = 0; i < n; ++i) g[i] = (uint16_t)i;
    orc_silu_array(g, n, sl);
    CHECK(sl[0] == 0.0f && sl[0x4120] == orc_silu_f32(0x4120));
    CHECK(orc_silu_f32(bf16_of(300.0f)) == 300.0f);
    free(sl);
    uint16_t* h = xmalloc(n * 2);
    orc_add_bf16(g, g, n, h);
    CHECK(h[0x3F80] == 0x4000); /* 1 + 1 = 2 */
    free(h);
    free(g);

    const int64_t T = 3, I = 128;
    uint16_t* gu = xmalloc(T * 2 * I * 2);
    uint16_t* y = xmalloc(T * I * 2);
    fill(gu, T * 2 * I, 3);
    for (int64_t i = 0; i < I; ++i) gu[I + i] = 0x3F80; /* up = 1: y = bf16(silu(gate)) */
    orc_swiglu_bf16(gu, T, I, y);
    for (int64_t i = 0; i < I; ++i)
        CHECK(y[i] == orc_f32_to_bf16_rne(orc_silu_f32(gu[i])));
    free(gu);
    free(y);

    const int64_t Tr = 3, H = 2, D = 16, R = 8, P = 4;
    uint16_t* o = xmalloc(Tr * H * D * 2);
    uint16_t* z = xmalloc(Tr * H * D * 2);
    int64_t pos[3] = {0, 3, 9}; /* the last is outside the cache: zero row */
    float* c = xmalloc(P * (R / 2) * sizeof(float));
    float* sn = xmalloc(P * (R / 2) * sizeof(float));
    for (int64_t i = 0; i < P * (R / 2); ++i) {
        c[i] = 1.0f;
        sn[i] = 0.0f;
    }
    fill(o, Tr * H * D, 4);
    orc_inverse_rope_bf16(o, pos, c, sn, Tr, H, D, R, P, z);
    for (int64_t i = 0; i < 2 * H * D; ++i) CHECK(z[i] == o[i]); /* angle 0: identity */
    for (int64_t i = 2 * H * D; i < 3 * H * D; ++i) CHECK(z[i] == 0);
    free(o);
    free(z);
    free(c);
    free(sn);
}

int main(void) {
    codec();
    bf16_and_scales();
    quantizers();
    rmsnorm();
    elementwise();
    printf("oracle sanitize checks: %d failures\n", failures);
    return failures == 0 ? 0 : 1;
}
