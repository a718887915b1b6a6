/*
 * fp8w8a8.h -- C ABI of the MI355X (gfx950) FP8 W8A8 quantization and scaled
 * GEMM library (libfp8w8a8.so).
 *
 * What it computes (pages cited by title and section):
 *   "FP8-RL: A Practical and Stable Low-Precision Stack for LLM RL", abstract,
 *     contribution (i): rollout with FP8 W8A8 linear layers using blockwise FP8
 *     quantization, for dense and MoE models; policy weights change every RL
 *     step, so they are re-quantized before each sync into the engine.
 *   "[vllm] feat: Support online quant for rollout with torchao", section
 *     "Test": dynamic FP8 with per-row granularity, float8_e4m3fn for both
 *     activations and weights, no activation value bounds.
 *   "[vllm] [ROCm] DeepSeek V4 ... FP8 WO_A 출력 프로젝션 최적화 분석":
 *     §1 E8M0 power-of-two scales (exponent byte, bias 127, accepted only when
 *     lossless); §2 weights viewed (groups, out, in) with block scales
 *     (groups, out/128, in/128), and refusal of shapes not divisible by 128;
 *     §3 group-128 activation quantization feeding an a8w8 GEMM.
 *   "[sglang] SGLang의 AMD GPU 최적화: RMSNorm과 FP8 Per-token Quantization 커널
 *     융합": §1 fused RMSNorm + per-token FP8 quantization called output-first
 *     (out_fp8, hidden_states, scale, weight, epsilon, group_size = 0);
 *     §3 the (q, scale) pair passed to a per-token x per-channel a8w8 GEMM
 *     whose arguments are (A, B, A-scale, B-scale, bias = None, bf16 out).
 *
 * Number formats:
 *   E4M3FN (OCP 8-bit FP): 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
 *   infinities, max finite 448.  Encoding is round-to-nearest-even and
 *   saturating (|v| >= 448 -> +-448, never NaN); the sign of zero is kept.
 *   Scale of a group = amax / 448, one IEEE fp32 division (no clamp); each
 *   element is the E4M3 encoding of the correctly rounded fp32 quotient x / s.
 *   An all-zero group has scale 0 and signed-zero codes.
 *   E8M0: one byte e + 127 meaning 2^e, e = ceil(log2(amax / 448)) clamped to
 *   [-127, 127]; elements are encoded from x / 2^e (exact).
 *
 * Conventions for every call:
 *   * Tensors are row-major and contiguous, innermost dimension last.  bf16
 *     and E4M3 data pointers must be 16-byte aligned; fp32 scale pointers
 *     4-byte aligned; everything except host descriptor tables is device
 *     memory on the current HIP device.
 *   * `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     on it; the call returns before the kernels finish.
 *   * The caller owns and allocates every input and output buffer, and the
 *     library keeps no pointer to them after the call returns (the kernels
 *     use the buffers until the stream reaches them).  The library allocates
 *     no memory: the GEMMs' partial-tile workspace is the caller's too (see
 *     fp8_gemm_workspace_size).
 *   * Errors: argument, shape and device checks run on the host before any
 *     launch; on error nothing is written and a negative fp8_status returns.
 *     Launch failures return FP8_ERR_LAUNCH.  Faults inside kernels surface
 *     at the caller's next synchronization of the stream.
 *   * Empty inputs (M == 0, n == 0, T == 0) are valid and launch nothing.
 *   * The device must be gfx950 (MI355X); other devices get FP8_ERR_DEVICE so
 *     the caller can keep its bf16 path (the capability check + fallback of
 *     the DeepSeek V4 page, §2).
 */
#ifndef FP8W8A8_H
#define FP8W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8W8A8_ABI_VERSION 3

typedef enum {
    FP8_OK = 0,
    FP8_ERR_ARG = -1,    /* null/invalid pointer or argument, non-NULL bias   */
    FP8_ERR_SHAPE = -2,  /* a dimension breaks the divisibility rules below   */
    FP8_ERR_ALIGN = -3,  /* a pointer breaks the alignment rules above        */
    FP8_ERR_DEVICE = -4, /* no HIP device, or the device is not gfx950        */
    FP8_ERR_LAUNCH = -5  /* the kernel launch itself failed                   */
} fp8_status;

typedef enum {
    FP8_GRAN_BLOCK = 0, /* activations 1x128 groups, weights 128x128 blocks */
    FP8_GRAN_ROW = 1    /* activations one scale per row (token), weights one
                           scale per output row (channel)                    */
} fp8_gran;

typedef enum {
    FP8_SCALE_F32 = 0, /* fp32 scale amax / 448                           */
    FP8_SCALE_E8M0 = 1 /* one byte: power-of-two scale 2^(byte - 127)      */
} fp8_scale_fmt;

/* Version of this header's ABI (FP8W8A8_ABI_VERSION). */
int fp8_abi_version(void);

/* SHA-256 (hex) of the sources this library was built from (csrc/ and this
 * header), or "unknown"; lets a test session check that the binary it loads
 * matches the source tree. */
const char* fp8_build_source_hash(void);

/* Static, human-readable name of a status code. */
const char* fp8_status_string(int status);

/*
 * 1x128 group quantization of activations ("FP8-RL" abstract (i) blockwise;
 * DeepSeek V4 page §3 quant_group_size = 128).
 *   x  : bf16 [M, K]            q : E4M3 [M, K]            s : fp32 [M, K/128]
 *   s[m][g] = amax(x[m][128g : 128g+128]) / 448.
 *   K % 128 != 0 -> FP8_ERR_SHAPE.  M may be any value >= 0.
 */
int fp8_quantize_block(const void* x_bf16, int64_t M, int64_t K, void* q_e4m3, float* s,
                       void* stream);

/*
 * 1x128 group quantization with E8M0 scale bytes (DeepSeek V4 page §1 E8M0
 * format, §3 group size 128; the activation side of the MX-scaled GEMM).
 *   x : bf16 [M, K]            q : E4M3 [M, K]            s : uint8 [M, K/128]
 *   s[m][g] = e + 127, e = ceil(log2(amax / 448)) of the fp32 scale amax / 448,
 *   clamped to [-127, 127] (0 for an all-zero group); q = E4M3(x / 2^e), an
 *   exact division.  K % 128 != 0 -> FP8_ERR_SHAPE.  s needs no alignment.
 */
int fp8_quantize_block_e8m0(const void* x_bf16, int64_t M, int64_t K, void* q_e4m3, void* s_e8m0,
                            void* stream);

/*
 * Per-row quantization: per-token activations, or per-output-channel weights
 * (torchao PerRow of the verl "Test" section; CHANNEL strategy of the SGLang
 * page §2).
 *   x  : bf16 [M, K]            q : E4M3 [M, K]            s : fp32 [M]
 *   K % 8 != 0 or K == 0 -> FP8_ERR_SHAPE.
 */
int fp8_quantize_token(const void* x_bf16, int64_t M, int64_t K, void* q_e4m3, float* s,
                       void* stream);

/*
 * Fused RMSNorm + FP8 quantization, output-first as in the SGLang page §1.
 *   q     : E4M3 [M, K] (out)     x : bf16 [M, K]
 *   s     : fp32 [M] (group_size 0, per token) or [M, K/128] (group_size 128)
 *   gamma : bf16 [K]              eps : added to mean(x^2) in fp32
 *   y = bf16_rne((x * inv) * gamma), inv = 1 / sqrt(S / K + eps), S the fp32
 *   sum of x^2 in a fixed order: 64 partial sums, partial l adding the squares
 *   of 8-element vectors l, l+64, l+128, ... in order, combined by a halving
 *   tree; then y is quantized per token (or per 1x128 group).  Equal to
 *   RMSNorm -> bf16 -> fp8_quantize_token (or fp8_quantize_block).
 *   K % 8 != 0 (group_size 0) or K % 128 != 0 (group_size 128) ->
 *   FP8_ERR_SHAPE; another group_size -> FP8_ERR_ARG.
 */
int fp8_rmsnorm_quant(void* q_e4m3, const void* x_bf16, float* s, const void* gamma_bf16,
                      float eps, int64_t M, int64_t K, int group_size, void* stream);

/*
 * Fused residual add + RMSNorm + FP8 quantization (the add_rmsnorm_quant
 * entry named in the SGLang page §1; the page shows only the call without a
 * residual, so the add is read as the usual pre-norm residual update).
 *   residual : bf16 [M, K], in/out.  On return it holds h = bf16_rne(x +
 *              residual), the nearest bf16 to the exact elementwise sum.
 *   Then h takes x's place in fp8_rmsnorm_quant: q, s, gamma, eps, M, K and
 *   group_size mean the same and are validated the same way.
 *   x and residual must not overlap (FP8_ERR_ARG); q, s may not alias either.
 *   M * K * 2 beyond INT64_MAX -> FP8_ERR_SHAPE.  On an error nothing is
 *   launched and residual is left unchanged.
 */
int fp8_add_rmsnorm_quant(void* q_e4m3, const void* x_bf16, void* residual_bf16, float* s,
                          const void* gamma_bf16, float eps, int64_t M, int64_t K,
                          int group_size, void* stream);

/*
 * Fused SwiGLU + 1x128 FP8 quantization: the MoE chain between the gate_up
 * and down grouped GEMMs (the "FP8-RL" abstract (i): W8A8 linears of MoE
 * models, whose down projection consumes this activation; the 1x128 groups of
 * the vLLM DeepSeek V4 page §3).  The pages show no SwiGLU, so it is read as
 * the usual silu_and_mul:
 *   gu : bf16 [T, 2I], the gate_up GEMM output; gate = columns [0, I),
 *        up = columns [I, 2I).
 *   y  = bf16_rne(silu(gate) * up): silu(g) is the fp32 value nearest to
 *        g / (1 + e^-g) (correctly rounded), times up in one fp32 multiply.
 *   q  : E4M3 [T, I] (out)       s : fp32 [T, I/128] (out), y's 1x128 groups
 *        quantized exactly as fp8_quantize_block would quantize y.
 *   T < 0 -> FP8_ERR_ARG; I <= 0 or I % 128 != 0 -> FP8_ERR_SHAPE.
 */
int fp8_swiglu_quant(const void* gu_bf16, int64_t T, int64_t I, void* q_e4m3, float* s,
                     void* stream);

/*
 * Token gather + 1x128 FP8 quantization: the MoE dispatch that lays the
 * routed copies of each token out in expert order before the grouped gate_up
 * GEMM ("FP8-RL" abstract (i): W8A8 linears of MoE models; 1x128 groups as in
 * fp8_quantize_block).
 *   x         : bf16 [n_src, K], one row per token   (K % 128 == 0)
 *   row_token : int32 [T], device; output row t takes token row_token[t]
 *   q         : E4M3 [T, K] (out)     s : fp32 [T, K/128] (out)
 *   q[t], s[t] are exactly fp8_quantize_block of the row x[row_token[t]].
 *   An index outside [0, n_src) gives a zero row (codes 0, scales 0) and reads
 *   nothing.  T < 0, n_src < 0 or n_src > INT32_MAX -> FP8_ERR_ARG.
 */
int fp8_quantize_block_gather(const void* x_bf16, int64_t n_src, int64_t K,
                              const int32_t* row_token, int64_t T, void* q_e4m3, float* s,
                              void* stream);

/*
 * Inverse RoPE + 1x128 E8M0 quantization: the pre-op of the DeepSeek V4
 * output projection in the vLLM page §3 (inverse_rope_group_quant(o,
 * positions, cos, sin, num_groups, quant_group_size=128) feeding
 * batched_gemm_a8w8_mxscale).  The page shows only the call; the readings:
 *   o          : bf16 [T, H, D] (D % 8 == 0); the last rope_dim dims of each
 *                head are the rotary part, as interleaved pairs (y0, y1) =
 *                dims (D - rope_dim + 2i, D - rope_dim + 2i + 1), angle index i
 *   positions  : int64 [T]; cos_cache, sin_cache : fp32 [max_pos, rope_dim/2]
 *   x0 = y0*c + y1*s, x1 = y1*c - y0*s (fp32, each operation rounded, no
 *   fused multiply-add), rounded to bf16; other dims pass through.
 *   q : E4M3 [T, H*D] (out), read as [T, num_groups, H*D/num_groups] by
 *   fp8_batched_gemm_a8w8_mxscale;  s : E8M0 bytes [T, H*D/128] (out), each
 *   1x128 group of the flattened row quantized as fp8_quantize_block_e8m0.
 *   A position outside [0, max_pos) gives a zero row (codes 0, bytes 0).
 *   Errors: T < 0, odd or negative rope_dim, rope_dim > 0 with max_pos 0,
 *   num_groups <= 0 -> FP8_ERR_ARG; H or D <= 0, D % 8, rope_dim > D,
 *   H % num_groups, (H/num_groups)*D % 128, H*D >= 2^31 -> FP8_ERR_SHAPE.
 */
int fp8_inverse_rope_group_quant(const void* o_bf16, const int64_t* positions,
                                 const float* cos_cache, const float* sin_cache, int64_t T,
                                 int64_t H, int64_t D, int64_t rope_dim, int64_t max_pos,
                                 int64_t num_groups, void* q_e4m3, uint8_t* s_e8m0,
                                 void* stream);

/*
 * Diagnostic (test support): out[i] = silu of the bf16 bit pattern
 * first_bits + i, as computed inside fp8_swiglu_quant (fp32).  The patterns
 * must lie in [0, 0x10000); out holds n floats (device, 4-byte aligned).
 */
int fp8_silu_f32_of_bf16(uint32_t first_bits, int64_t n, float* out, void* stream);

/* One weight of a re-quantization batch (all pointers device memory). */
typedef struct {
    const void* w_bf16; /* [N, K] bf16                                          */
    void* q_e4m3;       /* [N, K] E4M3 (out)                                    */
    void* s;            /* [N/128, K/128] fp32, or uint8 E8M0 bytes (out)      */
    int64_t N;          /* multiple of 128 (a stacked expert tensor [E, N', K]  */
    int64_t K;          /* with N' % 128 == 0 is passed as N = E * N')          */
} fp8_weight_desc;

/* One tensor of a per-tensor quantization batch (all pointers device memory). */
typedef struct {
    const void* x_bf16; /* bf16, n elements (any shape, contiguous)             */
    void* q_e4m3;       /* E4M3, n elements (out)                                */
    float* s;           /* one fp32 scale (out): amax over the tensor / 448     */
    int64_t n;          /* element count, a multiple of 8                        */
} fp8_tensor_desc;

/*
 * Per-tensor dynamic quantization ("FP8-RL" abstract (ii): FP8 KV cache with
 * per-step scale recalibration; "LLM FP8 ..." page: per-tensor dynamic
 * scaling; verl "Docs": tensorwise option): each descriptor's tensor gets one
 * scale s = amax / 448 over all its elements and codes E4M3(x / s), exactly as
 * fp8_quantize_token would give the tensor flattened to one row.  Meant for
 * recalibrating the K and V caches of every layer in one call.  `descs` is a
 * host array of n entries, read during the call only; each 64 descriptors
 * take four small kernels.  While those kernels run, *s holds the amax's
 * bits; the last one writes the scale.
 *   n % 8 != 0 -> FP8_ERR_SHAPE; n < 0 (count or element count) -> FP8_ERR_ARG;
 *   x and q 16-byte aligned, s 4-byte aligned; tensors with n == 0 are skipped
 *   (their s is not written).
 */
int fp8_quantize_tensors(const fp8_tensor_desc* descs, int n, void* stream);

/*
 * Workspace of fp8_requantize_weights for n descriptors: 0.  The descriptors
 * travel in the kernels' arguments (64 per launch), so no device copy of the
 * table is made; the size query and the workspace arguments keep the call's
 * shape stable should a layout ever need one.  n < 0 also gives 0.
 */
size_t fp8_requantize_workspace_size(int n);

/*
 * Per-RL-step policy weight re-quantization ("FP8-RL" abstract: weights change
 * every step and are re-quantized before each sync into the engine): every
 * descriptor's weight is quantized in 128x128 blocks, with fp32 scales or E8M0
 * bytes (DeepSeek V4 page §1/§2).  `descs` is a host array of n entries, read
 * during the call only.  The library enqueues one kernel per 64 descriptors.
 * `workspace` (device memory, caller-owned, 16-byte aligned) holds at least
 * fp8_requantize_workspace_size(n) bytes; with a size of 0 it may be NULL
 * (workspace_bytes then 0).
 *   N % 128 or K % 128 != 0 -> FP8_ERR_SHAPE; n < 0 -> FP8_ERR_ARG;
 *   workspace NULL with workspace_bytes > 0, or too small -> FP8_ERR_ARG;
 *   workspace misaligned -> FP8_ERR_ALIGN.
 */
int fp8_requantize_weights(const fp8_weight_desc* descs, int n, int scale_fmt, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Workspace of fp8_gemm_a8w8_scaled: the bytes of device memory its split-tile
 * path needs for this shape and granularity (0 when the path splits no tile;
 * also 0 for arguments the GEMM would refuse).  At most 64 MiB (256
 * workgroups x 2 partial tiles of 256 x 128 fp32).
 */
size_t fp8_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int gran);

/*
 * Scaled W8A8 GEMM, Y = X W^T with bf16 output (SGLang page §3 argument order:
 * A, B, A-scale, B-scale, bias, out; DeepSeek V4 page §3 for block scales).
 *   a : E4M3 [M, K]    w : E4M3 [N, K]    y : bf16 [M, N] (out)
 *   FP8_GRAN_BLOCK: a_s fp32 [M, K/128], w_s fp32 [N/128, K/128],
 *     Y[m,n] = sum_kb a_s[m,kb] * w_s[n/128,kb] * sum_{k in kb} a[m,k] w[n,k]
 *   FP8_GRAN_ROW: a_s fp32 [M], w_s fp32 [N],
 *     Y[m,n] = a_s[m] * w_s[n] * sum_k a[m,k] w[n,k]
 *   Products are exact, sums fp32 (matrix-core accumulate, block results
 *   scaled and added in fp32), output rounded to bf16 (nearest even).
 *   bias must be NULL (FP8_ERR_ARG otherwise).  K % 128 != 0 or
 *   N % 128 != 0 -> FP8_ERR_SHAPE.  M is any value >= 0.
 *   Small M (below 1024 with fewer than 192 tiles of 256 x 256; also
 *   N % 256 != 0 or K > 2^22): when whole tiles fill at least 3/4 of the CUs
 *   evenly, each workgroup takes whole tiles; otherwise, given a workspace,
 *   the K steps of all tiles are split evenly over the CUs (stream-K) and a
 *   second kernel sums each split tile's fp32 partials in a fixed order, so
 *   repeated calls give identical bytes.  Above 128 rows the tiles are
 *   256 x 128 (each weight block read once per 256 rows), else 128 x 128.
 *   workspace, workspace_bytes : device memory the split path writes its
 *     partial tiles to (16-byte aligned, at least
 *     fp8_gemm_workspace_size(M, N, K, gran) bytes; FP8_ERR_ARG if smaller,
 *     FP8_ERR_ALIGN if misaligned).  It must not overlap the other buffers,
 *     and it is in use until the stream reaches the end of the call: calls
 *     that may run at the same time (other streams, overlapping graph
 *     replays) need distinct workspaces.  NULL with 0 bytes is allowed: then
 *     no tile is split (one tile per workgroup at a time where whole tiles do
 *     not fill the chip), with results within the GEMM tolerance but not the
 *     same bytes as the split path.  A graph captured with a workspace
 *     records its address.
 */
int fp8_gemm_a8w8_scaled(const void* a_e4m3, const void* w_e4m3, const float* a_s,
                         const float* w_s, const void* bias, void* y_bf16, int64_t M,
                         int64_t N, int64_t K, int gran, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * fp8_gemm_a8w8_scaled for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without the workspace pair, the same
 * kernels and the same result bytes as fp8_gemm_a8w8_scaled given a workspace
 * of fp8_gemm_workspace_size bytes.  The partial tiles go to a library array
 * of 64 MiB in each GPU's memory (the largest workspace any shape needs), set
 * aside when the library's code is loaded on that GPU and held until the
 * process ends; no call allocates.  Every call on one GPU shares that array
 * and it keeps the last call's contents; nothing in it needs clearing, since a
 * call reads only the partial slots it has written.  Calls that may overlap on
 * one GPU (other streams, other threads, graph replays) race on it and must be
 * serialized by the caller.  A shape whose
 * workspace would exceed the array gets FP8_ERR_SHAPE (none does today);
 * FP8_ERR_DEVICE if the array's address cannot be found on this device.
 */
int fp8_gemm_a8w8_scaled_noalloc(const void* a_e4m3, const void* w_e4m3, const float* a_s,
                                 const float* w_s, const void* bias, void* y_bf16, int64_t M,
                                 int64_t N, int64_t K, int gran, void* stream);

/*
 * Grouped (MoE) block-scaled W8A8 GEMM ("FP8-RL" abstract: MoE models; DeepSeek
 * V4 page §2 weight view (groups, out, in) and scale view (groups, out/128,
 * in/128)).  Rows of A are grouped by expert: rows offsets[e] .. offsets[e+1]-1
 * use expert e's weight.
 *   a   : E4M3 [T, K]          a_s : fp32 [T, K/128]
 *   w   : E4M3 [E, N, K]       w_s : fp32 [E, N/128, K/128]
 *   offsets : int32 [E+1], DEVICE memory, non-decreasing, offsets[0] = 0,
 *             offsets[E] = T (empty experts allowed).  The kernel reads and
 *             writes only rows in [0, T) whatever the offsets hold.
 *   y   : bf16 [T, N] (out); rows covered by no expert are left untouched.
 *   When the experts average at least 192 rows the work runs on 256 x 256
 *   tiles, otherwise on 128 x 128 tiles (results within the GEMM tolerance).
 *   K % 128 != 0 or N % 128 != 0 -> FP8_ERR_SHAPE; E < 1, E > 1024 or
 *   T > 2^31 - 1 -> FP8_ERR_ARG.
 */
int fp8_grouped_gemm_a8w8_scaled(const void* a_e4m3, const void* w_e4m3, const float* a_s,
                                 const float* w_s, const int32_t* offsets, void* y_bf16,
                                 int64_t T, int64_t E, int64_t N, int64_t K, void* stream);

/*
 * Workspace of fp8_batched_gemm_a8w8_mxscale for this shape, as
 * fp8_gemm_workspace_size (0 unless B == 1 takes the small-M path and splits
 * tiles; 0 for arguments the GEMM would refuse).
 */
size_t fp8_batched_gemm_mxscale_workspace_size(int64_t B, int64_t M, int64_t N, int64_t K);

/*
 * Batched W8A8 GEMM with E8M0 block scales (DeepSeek V4 page §3
 * batched_gemm_a8w8_mxscale(A, W, A-scale, W-scale, bf16); §2 weight view
 * (groups, out, in) and scale view (groups, out/128, in/128)), on the gfx950
 * MX-scaled matrix instruction.  B batches (groups), token-major:
 *   a   : E4M3 [M, B, K]          a_s : uint8 [M, B, K/128]  (E8M0 bytes)
 *   w   : E4M3 [B, N, K]          w_s : uint8 [B, N/128, K/128]
 *   y   : bf16 [M, B, N] (out)
 *   Y[m,b,n] = sum_kb 2^(a_s[m,b,kb] - 127) * 2^(w_s[b,n/128,kb] - 127)
 *              * sum_{k in kb} a[m,b,k] w[b,n,k]
 *   Products exact; sums fp32 in the matrix core, which applies the power-of-
 *   two scales; bf16 out, round to nearest even.  B = 1 is the dense GEMM
 *   (a [M, K], y [M, N]).
 *   N % 128 != 0, K % 128 != 0 or B * K > 2^22 -> FP8_ERR_SHAPE; M, B < 0 ->
 *   FP8_ERR_ARG; M == 0 or B == 0 launch nothing.  Scale pointers need no
 *   alignment.
 *   Dense small M (B = 1, M below 1024 with fewer than 192 tiles of 256 x 256)
 *   takes the small-M kernels of fp8_gemm_a8w8_scaled; workspace and
 *   workspace_bytes follow that call's rules, sized by
 *   fp8_batched_gemm_mxscale_workspace_size.
 */
int fp8_batched_gemm_a8w8_mxscale(const void* a_e4m3, const void* w_e4m3, const void* a_s,
                                  const void* w_s, void* y_bf16, int64_t B, int64_t M, int64_t N,
                                  int64_t K, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Diagnostic: the device E4M3 encoder alone.  q[i] = E4M3(float with bit
 * pattern first_bits + i) for 0 <= i < n (n <= 2^32 - first_bits), so that a
 * test can compare the encoder used by every quantizer above on all 2^32 fp32
 * patterns.
 *   q : uint8 [n] device memory, 16-byte aligned.
 */
int fp8_encode_f32_bits(uint64_t first_bits, int64_t n, void* q, void* stream);

/*
 * Diagnostic (measurement support): the matrix-core rate with operands in
 * registers.  Launches 1024 workgroups of 4 waves; each wave runs `iters`
 * rounds of 8 independent 16 x 16 x 128 E4M3 MFMAs (2 * 16 * 16 * 128 flops
 * each), so the work is 4096 * iters * 8 * 65536 flops.  The caller times it
 * (events on `stream`).  out : float [4096] device memory (one value per
 * wave, kept so the work is not optimized away).  iters in [0, 2^32].
 */
int fp8_mfma_rate_probe(int64_t iters, float* out, void* stream);

/*
 * Diagnostic: the device bf16 rounding alone.  out[i] = bf16 bit pattern of
 * the float with bit pattern first_bits + i, round to nearest even (the
 * rounding of the RMSNorm output y and of every bf16 GEMM output), for
 * 0 <= i < n (n <= 2^32 - first_bits).
 *   out : uint16 [n] device memory, 16-byte aligned.
 */
int fp8_bf16_round_f32_bits(uint64_t first_bits, int64_t n, void* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FP8W8A8_H */
