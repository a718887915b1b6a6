// Launch interface of the per-tensor, SwiGLU, token-gather and inverse-RoPE
// quantizers.
// Per-tensor dynamic quantization: one fp32 scale per tensor (amax / 448); up
// to kTensMaxDescs tensors per launch sequence, with descriptors passed in
// kernel arguments.  A tensor of nvec 16-byte vectors covers
// ceil(nvec / kTensChunk) workgroup chunks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8k {

constexpr int kTensMaxDescs = 64;
constexpr int64_t kTensChunk = 2048;  // vectors (32 KiB of bf16) per workgroup
struct TensDesc {
    const void* x;        // bf16 [nvec * 8]
    void* q;              // E4M3 [nvec * 8]
    float* s;             // holds the amax bits during the sequence, then the scale
    int64_t nvec;
    int64_t chunk_begin;  // first chunk of this tensor in the launch
};
struct TensBatch {
    TensDesc d[kTensMaxDescs];
    int n;
};
hipError_t launch_tensor_batch(const TensBatch& batch, int64_t chunks, hipStream_t st);

// SwiGLU + 1x128 quantization of gu bf16 [T, 2I] (I % 128 == 0, T > 0), and
// the diagnostic silu of bf16 bit patterns.
hipError_t launch_swiglu_quant(const void* gu, int64_t T, int64_t I, void* q, float* s,
                               hipStream_t st);
hipError_t launch_silu_bits(uint32_t first, int64_t n, float* out, hipStream_t st);

// Token gather + 1x128 quantization: q[t] = quant(x[row_token[t]]), x bf16
// [n_src, K] (K % 128 == 0, T > 0).
// Inverse RoPE + 1x128 E8M0 quantization of o bf16 [T][H][D] (D % 8 == 0,
// even R <= D, H * D % 128 == 0, T > 0; P >= 1 when R > 0).
hipError_t launch_inv_rope_quant(const void* o, const int64_t* pos, const float* cosc,
                                 const float* sinc, int64_t T, int64_t H, int64_t D, int64_t R,
                                 int64_t P, void* q, uint8_t* s, hipStream_t st);

hipError_t launch_quant_gather(const void* x, int64_t n_src, int64_t K, const int32_t* row_token,
                               int64_t T, void* q, float* s, hipStream_t st);

}  // namespace fp8k
