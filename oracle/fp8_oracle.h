/*
 * fp8_oracle.h -- plain CPU oracle for FP8 (OCP E4M3FN) W8A8 quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library under fp8_w8a8_quantized_amd/) never calls, links or includes
 * anything here, and this code includes nothing from it.
 *
 * Every function is the plain definition of one step, written for a reader to
 * check by eye: no blocking, no vector tricks, no reordering of floating-point
 * work beyond what the definition states.  Loops over independent rows or
 * groups may run under OpenMP; that never changes a result.
 *
 * Pages cited (short tag -> page title, section):
 *   [FP8-RL]     "FP8-RL: A Practical and Stable Low-Precision Stack for LLM RL",
 *                abstract, contribution (i) blockwise W8A8 linears and the
 *                per-step weight re-quantization.
 *   [verl-3084]  "[vllm] feat: Support online quant for rollout with torchao",
 *                section "Test" (torchao PerRow config: e4m3fn on both operands,
 *                activation_value_lb/ub null).
 *   [vllm-54894] "[vllm] [ROCm] DeepSeek V4 ... FP8 WO_A 출력 프로젝션 최적화 분석",
 *                §1 (E8M0 scale normalization), §2 (group-128 shape check),
 *                §3 (group-128 quant feeding an a8w8 GEMM); its references name
 *                the OCP MX v1.0 spec and the HIP low-precision types page,
 *                which define the E4M3FN and E8M0 encodings used here.
 *   [sglang-21403] "[sglang] SGLang의 AMD GPU 최적화: RMSNorm과 FP8 Per-token
 *                Quantization 커널 융합", §1 (fused RMSNorm + per-token quant,
 *                group_size 0), §3 ((q, scale) tuple fed to the a8w8 GEMM);
 *                its reference is the torch.nn.RMSNorm definition.
 */
#ifndef FP8_ORACLE_H
#define FP8_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- OCP E4M3FN codec (format defined by the OCP 8-bit FP spec cited by
 *      [vllm-54894] references; dtype float8_e4m3fn named by [verl-3084]) ---- */

/* Exact value of an E4M3FN code; NaN for 0x7F / 0xFF. */
double orc_e4m3_decode(uint8_t code);

/* The defining encoder: nearest finite E4M3FN value, ties to the even code,
 * |v| >= 448 saturates to +-448, sign of zero kept.  NaN maps to 0x7F|sign. */
uint8_t orc_e4m3_encode(float v);

/* A second, independent encoder by integer bit arithmetic.  Used only to pin
 * orc_e4m3_encode (the two must agree on all 2^32 fp32 patterns). */
uint8_t orc_e4m3_encode_bits(float v);

/* Count fp32 bit patterns in [lo, hi) (64-bit bounds, hi <= 2^32) on which the
 * two encoders disagree. */
uint64_t orc_e4m3_encoders_disagree(uint64_t lo, uint64_t hi);

/* Encode n fp32 values with the defining encoder (bulk helper for tests). */
void orc_e4m3_encode_array(const float* v, int64_t n, uint8_t* out);

/* ---- bf16 helpers ---- */
float    orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16_rne(float f);
void     orc_bf16_rne_array(const float* v, int64_t n, uint16_t* out);

/* Residual add (SGLang RMSNorm + per-token fusion page, section 1, the
 * add_rmsnorm_quant entry): h = bf16 nearest (ties to even) to the exact
 * x + r, elementwise over n values. */
void     orc_add_bf16(const uint16_t* x, const uint16_t* r, int64_t n, uint16_t* h);

/* SiLU of a bf16 value, correctly rounded to fp32 (nearest fp32 to
 * g / (1 + e^-g)); the array form is for pinning. */
float    orc_silu_f32(uint16_t g);
void     orc_silu_array(const uint16_t* g, int64_t n, float* out);

/* SwiGLU between the MoE gate_up and down GEMMs: gu bf16 [T, 2I], gate =
 * columns [0, I), up = [I, 2I); y bf16 [T, I] = bf16_rne(silu(gate) * up). */
void     orc_swiglu_bf16(const uint16_t* gu, int64_t T, int64_t I, uint16_t* y);

/* Inverse RoPE (vLLM DeepSeek V4 page §3): o bf16 [T][H][D], rotary part =
 * last R dims of each head as interleaved pairs; cos/sin fp32 [P][R/2];
 * x0 = y0*c + y1*s, x1 = y1*c - y0*s in fp32, rounded to bf16; a position
 * outside [0, P) gives a zero row. */
void     orc_inverse_rope_bf16(const uint16_t* o, const int64_t* pos, const float* cosc,
                               const float* sinc, int64_t T, int64_t H, int64_t D, int64_t R,
                               int64_t P, uint16_t* z);

/* ---- scales ---- */

/* fp32 scale of a group whose largest magnitude is amax: amax / 448 as one
 * IEEE fp32 division (no clamp, no epsilon: activation_value_lb/ub are null in
 * [verl-3084] "Test"). */
float orc_scale_f32(float amax);

/* E8M0 exponent of a positive-or-zero fp32 scale s: e = ceil(log2(s)) taken
 * exactly from the bits of s, clamped to [-127, 127]; s == 0 gives -127. */
int orc_e8m0_exponent(float s);

/* [vllm-54894] §1: lossless fp32 -> E8M0 conversion.  For each scale,
 * e = round(log2(s)); the conversion is accepted only if 2^e == s exactly; the
 * byte is e + 127.  Returns 1 if every element converted, 0 otherwise. */
int orc_e8m0_lossless(const float* s, int64_t n, uint8_t* codes);

/* ---- quantizers (all inputs bf16 bit patterns, row-major, K innermost) ---- */

/* 1x128 groups: s[m][g] over x[m][128g : 128g+128].  K % 128 == 0. */
void orc_quantize_block(const uint16_t* x, int64_t M, int64_t K,
                        uint8_t* q, float* s);

/* One group per row: s[m] over x[m][0:K]. */
/* 1x128 groups with E8M0 scale bytes s[M][K/128] (e + 127). */
void orc_quantize_block_e8m0(const uint16_t* x, int64_t M, int64_t K, uint8_t* q, uint8_t* s);
/* One fp32 scale for all n elements (per-tensor): *s = amax / 448. */
void orc_quantize_tensor(const uint16_t* x, int64_t n, uint8_t* q, float* s);
void orc_quantize_token(const uint16_t* x, int64_t M, int64_t K,
                        uint8_t* q, float* s);

/* 128x128 weight blocks: s[i][j] over w[128i:+128][128j:+128].
 * fmt 0: fp32 scale (float* s, [N/128][K/128]).
 * fmt 1: E8M0 scale byte (uint8_t* s), element divided by 2^e.
 * N % 128 == 0 and K % 128 == 0. */
void orc_quantize_weight_block(const uint16_t* w, int64_t N, int64_t K, int fmt,
                               uint8_t* q, void* s);

/* RMSNorm of one bf16 matrix to bf16, with the fixed fp32 reduction order
 * described in fp8_oracle.c.  K % 8 == 0. */
void orc_rmsnorm_bf16(const uint16_t* x, const uint16_t* gamma, float eps,
                      int64_t M, int64_t K, uint16_t* y);

/* Per-row sum of squares in the fixed order (exposed for pinning). */
float orc_rms_sumsq(const uint16_t* xrow, int64_t K);

/* Fused RMSNorm + per-token quantization ([sglang-21403] §1, group_size 0):
 * equal by definition to orc_rmsnorm_bf16 followed by orc_quantize_token. */
void orc_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, float eps,
                       int64_t M, int64_t K, uint8_t* q, float* s);

#ifdef __cplusplus
}
#endif
#endif /* FP8_ORACLE_H */
