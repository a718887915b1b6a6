/*
 * fp8_oracle.c -- plain CPU oracle for FP8 (OCP E4M3FN) W8A8 quantization.
 *
 * TEST INFRASTRUCTURE ONLY (see fp8_oracle.h): used by tests, the smoke check
 * and the benchmark's CPU-baseline leg; never by the product path.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 * (no FMA contraction and no fast-math, so every float operation below is one
 * IEEE binary32 operation with round-to-nearest-even, subnormals kept).
 *
 * Readings where the pages are silent:
 *   rounding to E4M3 is round-to-nearest-even; overflow saturates to +-448;
 *   the element quotient is one correctly rounded fp32 division x / s by the
 *   stored scale; an all-zero group has scale 0 and signed-zero codes; the
 *   E8M0 exponent is the ceiling of log2 of the fp32 scale; the RMSNorm sum of
 *   squares uses the fixed order documented at orc_rms_sumsq.
 */
#include "fp8_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* E4M3FN codec                                                             */
/* ------------------------------------------------------------------------ */

/* Format (OCP 8-bit FP spec, E4M3 variant without infinities): 1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0 holds
 * subnormals m * 2^-9; otherwise the value is (1 + m/8) * 2^(E-7).  The
 * pattern S.1111.111 is NaN; the largest finite magnitude is S.1111.110 = 448. */
double orc_e4m3_decode(uint8_t code) {
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(8.0 + (double)m, e - 10);
    return sign ? -mag : mag;
}

/* Non-negative finite magnitudes in code order: codes 0..126 ascend.  The
 * table is filled from orc_e4m3_decode once, when the library is loaded. */
static double POS[127];
__attribute__((constructor)) static void fill_pos(void) {
    int c;
    for (c = 0; c < 127; ++c) POS[c] = orc_e4m3_decode((uint8_t)c);
}
static double pos_value(int code) { return POS[code]; }

uint8_t orc_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a;
    int lo, hi, c;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E); /* saturate */
    /* largest code whose value is <= a */
    lo = 0;
    hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (pos_value(mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    if (pos_value(lo) == a) return (uint8_t)(sign | lo);
    {
        /* a lies strictly between the values of codes lo and lo+1; both
         * distances are exact in double (Sterbenz, or trivially when lo = 0). */
        double dlo = a - pos_value(lo);
        double dhi = pos_value(lo + 1) - a;
        if (dlo < dhi)
            c = lo;
        else if (dhi < dlo)
            c = lo + 1;
        else
            c = (lo & 1) ? lo + 1 : lo; /* tie: the even code */
    }
    return (uint8_t)(sign | c);
}

uint8_t orc_e4m3_encode_bits(float v) {
    uint32_t u, a, mant;
    int ebits, e;
    uint8_t sign;
    memcpy(&u, &v, 4);
    sign = (uint8_t)((u >> 31) << 7);
    a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return (uint8_t)(sign | 0x7F); /* NaN */
    if (a >= 0x43E00000u) return (uint8_t)(sign | 0x7E); /* >= 448 (incl. inf) */
    ebits = (int)(a >> 23);
    mant = a & 0x7FFFFFu;
    e = ebits - 127;
    if (ebits != 0 && e >= -6) {
        /* E4M3 normal range: keep 3 of the 23 fraction bits, RNE on the rest. */
        uint32_t keep = mant >> 20;
        uint32_t rest = mant & 0xFFFFFu;
        uint32_t code = ((uint32_t)(e + 7) << 3) | keep;
        if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) code += 1u;
        return (uint8_t)(sign | code);
    } else {
        /* E4M3 subnormal range: the code is round(|v| * 2^9) with RNE.
         * |v| = S * 2^(p) with S the integer significand. */
        uint64_t S = (ebits == 0) ? (uint64_t)mant : (uint64_t)(mant | 0x800000u);
        int p = (ebits == 0) ? -149 : (ebits - 150);
        int shift = -(p + 9); /* |v| * 2^9 = S * 2^(p+9) = S >> shift */
        uint64_t q, rem, half;
        if (shift >= 64) return sign; /* far below half of 2^-9 */
        q = S >> shift;
        rem = S & ((1ull << shift) - 1ull);
        half = 1ull << (shift - 1);
        if (rem > half || (rem == half && (q & 1ull))) q += 1ull;
        return (uint8_t)(sign | (uint8_t)q); /* q <= 8; 8 is the least normal */
    }
}

uint64_t orc_e4m3_encoders_disagree(uint64_t lo, uint64_t hi) {
    uint64_t bad = 0;
    int64_t i;
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (i = (int64_t)lo; i < (int64_t)hi; ++i) {
        uint32_t u = (uint32_t)i;
        float f;
        memcpy(&f, &u, 4);
        if (orc_e4m3_encode(f) != orc_e4m3_encode_bits(f)) bad += 1;
    }
    return bad;
}

void orc_e4m3_encode_array(const float* v, int64_t n, uint8_t* out) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

/* ------------------------------------------------------------------------ */
/* bf16                                                                     */
/* ------------------------------------------------------------------------ */

float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Nearest bf16 (8-bit significand), ties to even.  Finite inputs only. */
uint16_t orc_f32_to_bf16_rne(float f) {
    uint32_t u, low, hi;
    memcpy(&u, &f, 4);
    hi = u >> 16;
    low = u & 0xFFFFu;
    if (low > 0x8000u || (low == 0x8000u && (hi & 1u))) hi += 1u;
    return (uint16_t)hi;
}

void orc_bf16_rne_array(const float* v, int64_t n, uint16_t* out) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) out[i] = orc_f32_to_bf16_rne(v[i]);
}

/* Nearest bf16 to a finite double, ties to even; below the smallest normal
 * the bf16 quantum is 2^-133.  Magnitudes past the largest finite bf16 do not
 * occur for the sums formed here and are not handled. */
static uint16_t f64_to_bf16_rne(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v), r;
    int e, qe;
    float f;
    uint32_t u;
    if (a == 0.0) return sign;
    (void)frexp(a, &e); /* a = m * 2^e with 0.5 <= m < 1 */
    qe = e - 8;         /* 8 significant bits: quantum 2^(e-8) */
    if (qe < -133) qe = -133;
    r = rint(ldexp(a, -qe)); /* count of quanta, ties to even (default mode) */
    f = (float)ldexp(r, qe); /* exact: every bf16 value is an fp32 value */
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

/* Residual add of the fused add + RMSNorm (the add_rmsnorm_quant entry named
 * on the SGLang RMSNorm + per-token fusion page, section 1): the new residual
 * stream is the bf16 value nearest to the exact sum x + r.  The fp64 sum of
 * two bf16 values is exact unless their exponents differ by 45 or more; then
 * the smaller one is far below half a bf16 ulp of the larger and both the
 * exact and the fp64 sum round to the larger one. */
void orc_add_bf16(const uint16_t* x, const uint16_t* r, int64_t n, uint16_t* h) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        h[i] = f64_to_bf16_rne((double)orc_bf16_to_f32(x[i]) + (double)orc_bf16_to_f32(r[i]));
}

/* SiLU of a bf16 value, correctly rounded to fp32: the nearest fp32 to
 * g * sigmoid(g) = g / (1 + e^-g) (ties cannot occur: the value is
 * transcendental for g != 0).  Evaluated in fp64 and rounded once; the fp64
 * error (a few 2^-53 relative) decides the rounding only within that distance
 * of an fp32 midpoint, and an exhaustive test over every bf16 input against
 * high-precision decimal arithmetic shows no such case.  Large |g|: e^-g
 * overflows to +inf for g < -709 and the quotient is -0; for g > 745 it is 0
 * and the quotient is g. */
float orc_silu_f32(uint16_t gb) {
    double g = (double)orc_bf16_to_f32(gb);
    return (float)(g / (1.0 + exp(-g)));
}

void orc_silu_array(const uint16_t* g, int64_t n, float* out) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) out[i] = orc_silu_f32(g[i]);
}

/* SwiGLU of the gate_up projection's bf16 output (the MoE chain between the
 * gate_up and down grouped GEMMs): gu [T, 2I], gate = columns [0, I), up =
 * columns [I, 2I); y[t][i] = bf16_rne(silu(gate) * up), one fp32 multiply of
 * the correctly rounded silu and the up value. */
void orc_swiglu_bf16(const uint16_t* gu, int64_t T, int64_t I, uint16_t* y) {
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        int64_t i;
        for (i = 0; i < I; ++i) {
            float sg = orc_silu_f32(gu[t * 2 * I + i]);
            float u = orc_bf16_to_f32(gu[t * 2 * I + I + i]);
            y[t * I + i] = orc_f32_to_bf16_rne(sg * u);
        }
    }
}

/* Inverse RoPE ahead of the output projection (the vLLM DeepSeek V4 page,
 * section 3: inverse_rope_group_quant(o, positions, cos, sin, ...)).  o is
 * bf16 [T][H][D]; the last R dims of each head carry the rotary part, as
 * interleaved pairs (y0, y1) = dims (D-R+2i, D-R+2i+1) with angle index i;
 * cos/sin are fp32 [P][R/2] rows indexed by the token's position.  The
 * inverse rotation by that angle is
 *     x0 = y0*c + y1*s,   x1 = y1*c - y0*s,
 * each product and the sum one fp32 operation, then rounded to bf16.  Other
 * dims pass through.  A position outside [0, P) gives a zero row. */
void orc_inverse_rope_bf16(const uint16_t* o, const int64_t* pos, const float* cosc,
                           const float* sinc, int64_t T, int64_t H, int64_t D, int64_t R,
                           int64_t P, uint16_t* z) {
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        int64_t h, d, p = pos[t];
        for (h = 0; h < H; ++h) {
            const uint16_t* yr = o + (t * H + h) * D;
            uint16_t* zr = z + (t * H + h) * D;
            for (d = 0; d < D; ++d) {
                if (p < 0 || p >= P) {
                    zr[d] = 0;
                } else if (d < D - R) {
                    zr[d] = yr[d];
                } else {
                    int64_t r = d - (D - R), i = r / 2;
                    float c = cosc[p * (R / 2) + i], s = sinc[p * (R / 2) + i];
                    float v;
                    if (r % 2 == 0) {
                        float y0 = orc_bf16_to_f32(yr[d]), y1 = orc_bf16_to_f32(yr[d + 1]);
                        float a = y0 * c, b = y1 * s;
                        v = a + b;
                    } else {
                        float y0 = orc_bf16_to_f32(yr[d - 1]), y1 = orc_bf16_to_f32(yr[d]);
                        float a = y1 * c, b = y0 * s;
                        v = a - b;
                    }
                    zr[d] = orc_f32_to_bf16_rne(v);
                }
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Scales                                                                   */
/* ------------------------------------------------------------------------ */

float orc_scale_f32(float amax) {
    volatile float d = 448.0f; /* keep it one runtime IEEE division */
    return amax / d;
}

int orc_e8m0_exponent(float s) {
    uint32_t u, mant;
    int ebits, e;
    memcpy(&u, &s, 4);
    u &= 0x7FFFFFFFu;
    if (u == 0) return -127;
    ebits = (int)(u >> 23);
    mant = u & 0x7FFFFFu;
    if (ebits == 0) {
        /* subnormal: s = mant * 2^-149, ceil(log2 s) = ceil(log2 mant) - 149 */
        int c = 0;
        while ((1u << c) < mant) ++c;
        e = c - 149;
    } else {
        e = ebits - 127 + (mant != 0 ? 1 : 0);
    }
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

int orc_e8m0_lossless(const float* s, int64_t n, uint8_t* codes) {
    int64_t i;
    for (i = 0; i < n; ++i) {
        double sf = (double)s[i];
        double ex = round(log2(sf));
        if (!(exp2(ex) == sf)) return 0;
        codes[i] = (uint8_t)((int)ex + 127);
    }
    return 1;
}

/* ------------------------------------------------------------------------ */
/* Quantizers                                                               */
/* ------------------------------------------------------------------------ */

/* One element of a group with fp32 scale s ([FP8-RL] blockwise W8A8; scale
 * amax/448 in fp32).  An all-zero group (s == 0) yields signed zeros. */
static uint8_t quant_elem(float x, float s) {
    if (s == 0.0f) return signbit(x) ? 0x80 : 0x00;
    return orc_e4m3_encode(x / s);
}

static float group_amax(const uint16_t* x, int64_t n, int64_t stride, int64_t rows) {
    /* max |x| over `rows` rows of n elements, row stride `stride` (exact) */
    float amax = 0.0f;
    int64_t r, k;
    for (r = 0; r < rows; ++r)
        for (k = 0; k < n; ++k) {
            float a = fabsf(orc_bf16_to_f32(x[r * stride + k]));
            if (a > amax) amax = a;
        }
    return amax;
}

void orc_quantize_block(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s) {
    int64_t G = K / 128, m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        int64_t g, k;
        for (g = 0; g < G; ++g) {
            const uint16_t* xg = x + m * K + g * 128;
            float sc = orc_scale_f32(group_amax(xg, 128, 0, 1));
            s[m * G + g] = sc;
            for (k = 0; k < 128; ++k)
                q[m * K + g * 128 + k] = quant_elem(orc_bf16_to_f32(xg[k]), sc);
        }
    }
}

/* 1x128 groups with E8M0 scales ([vllm-54894] §1 scale format, §3 group size
 * 128): per group e = ceil(log2(amax / 448)) (amax / 448 the fp32 scale),
 * clamped to [-127, 127]; byte e + 127; each element encoded from x / 2^e,
 * an exact division. */
void orc_quantize_block_e8m0(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, uint8_t* s) {
    int64_t G = K / 128, m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        int64_t g, k;
        for (g = 0; g < G; ++g) {
            const uint16_t* xg = x + m * K + g * 128;
            int e = orc_e8m0_exponent(orc_scale_f32(group_amax(xg, 128, 0, 1)));
            float p2 = ldexpf(1.0f, e); /* exact, subnormal for e = -127 */
            s[m * G + g] = (uint8_t)(e + 127);
            for (k = 0; k < 128; ++k)
                q[m * K + g * 128 + k] = orc_e4m3_encode(orc_bf16_to_f32(xg[k]) / p2);
        }
    }
}

/* One scale for a whole tensor ([FP8-RL] abstract (ii): FP8 KV cache with
 * per-step scale recalibration; [E2E-FP8] per-tensor dynamic scaling;
 * [verl-3084] "Docs" tensorwise option): s = amax over all n elements / 448,
 * q = E4M3(x / s). */
void orc_quantize_tensor(const uint16_t* x, int64_t n, uint8_t* q, float* s) {
    int64_t k;
    float amax = 0.0f, sc;
    for (k = 0; k < n; ++k) {
        float a = fabsf(orc_bf16_to_f32(x[k]));
        if (a > amax) amax = a;
    }
    sc = orc_scale_f32(amax);
    *s = sc;
#pragma omp parallel for schedule(static)
    for (k = 0; k < n; ++k) q[k] = quant_elem(orc_bf16_to_f32(x[k]), sc);
}

void orc_quantize_token(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, float* s) {
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        int64_t k;
        const uint16_t* xr = x + m * K;
        float sc = orc_scale_f32(group_amax(xr, K, 0, 1));
        s[m] = sc;
        for (k = 0; k < K; ++k) q[m * K + k] = quant_elem(orc_bf16_to_f32(xr[k]), sc);
    }
}

void orc_quantize_weight_block(const uint16_t* w, int64_t N, int64_t K, int fmt,
                               uint8_t* q, void* s) {
    int64_t NB = N / 128, KB = K / 128, bi;
#pragma omp parallel for schedule(static)
    for (bi = 0; bi < NB; ++bi) {
        int64_t bj, r, k;
        for (bj = 0; bj < KB; ++bj) {
            const uint16_t* wb = w + bi * 128 * K + bj * 128;
            float amax = group_amax(wb, 128, K, 128);
            float sc = orc_scale_f32(amax);
            if (fmt == 0) {
                ((float*)s)[bi * KB + bj] = sc;
                for (r = 0; r < 128; ++r)
                    for (k = 0; k < 128; ++k)
                        q[(bi * 128 + r) * K + bj * 128 + k] =
                            quant_elem(orc_bf16_to_f32(wb[r * K + k]), sc);
            } else {
                int e = orc_e8m0_exponent(sc);
                float p2 = ldexpf(1.0f, e); /* exact, subnormal for e = -127 */
                ((uint8_t*)s)[bi * KB + bj] = (uint8_t)(e + 127);
                for (r = 0; r < 128; ++r)
                    for (k = 0; k < 128; ++k)
                        q[(bi * 128 + r) * K + bj * 128 + k] =
                            orc_e4m3_encode(orc_bf16_to_f32(wb[r * K + k]) / p2);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* RMSNorm ([sglang-21403] §1; definition of torch.nn.RMSNorm: y = x / sqrt(  */
/* mean(x^2) + eps) * gamma), computed in fp32 with this fixed order:        */
/*   squares sq[k] = x[k]^2 (exact in fp32 for bf16 x);                      */
/*   64 partial sums P[l], l = 0..63: P[l] starts at +0 and adds, in order,  */
/*     the 8 squares of each 8-element vector v = l, l+64, l+128, ... (v <   */
/*     K/8), elements 8v+0 .. 8v+7 in ascending order;                       */
/*   the total is the halving tree T(0..63) = T(0..31) + T(32..63), applied  */
/*     recursively down to single partials.                                  */
/* The pages fix no order; an unfixed order would leave the FP8 bytes of the */
/* fused operator undetermined, so this one is part of the definition.      */
/* ------------------------------------------------------------------------ */

static float tree_sum(const float* p, int n) {
    if (n == 1) return p[0];
    return tree_sum(p, n / 2) + tree_sum(p + n / 2, n / 2);
}

float orc_rms_sumsq(const uint16_t* xrow, int64_t K) {
    float P[64];
    int64_t V = K / 8, v;
    int l, j;
    for (l = 0; l < 64; ++l) {
        P[l] = 0.0f;
        for (v = l; v < V; v += 64)
            for (j = 0; j < 8; ++j) {
                float xv = orc_bf16_to_f32(xrow[8 * v + j]);
                P[l] = P[l] + xv * xv;
            }
    }
    return tree_sum(P, 64);
}

static void rmsnorm_row(const uint16_t* xr, const uint16_t* gamma, float eps, int64_t K,
                        uint16_t* yr) {
    volatile float kf = (float)K;
    float S = orc_rms_sumsq(xr, K);
    float ms = S / kf;
    float inv = 1.0f / sqrtf(ms + eps);
    int64_t k;
    for (k = 0; k < K; ++k) {
        float t = orc_bf16_to_f32(xr[k]) * inv;
        float u = t * orc_bf16_to_f32(gamma[k]);
        yr[k] = orc_f32_to_bf16_rne(u);
    }
}

void orc_rmsnorm_bf16(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M,
                      int64_t K, uint16_t* y) {
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) rmsnorm_row(x + m * K, gamma, eps, K, y + m * K);
}

void orc_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M,
                       int64_t K, uint8_t* q, float* s) {
    /* the normalized row is rounded to bf16 first, then quantized per token */
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        uint16_t* yr = (uint16_t*)malloc((size_t)K * sizeof(uint16_t));
        int64_t k;
        float sc;
        rmsnorm_row(x + m * K, gamma, eps, K, yr);
        sc = orc_scale_f32(group_amax(yr, K, 0, 1));
        s[m] = sc;
        for (k = 0; k < K; ++k) q[m * K + k] = quant_elem(orc_bf16_to_f32(yr[k]), sc);
        free(yr);
    }
}
