// launch.hpp -- internal launchers behind the C ABI (shapes already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8k {

// Descriptor of one weight inside a re-quantization launch.
struct ReqDesc {
    const uint16_t* w;
    uint8_t* q;
    void* s;
    int64_t K;
    int64_t block_begin;  // first block index of this weight within the launch
    int32_t kblocks;      // K / 128
    int32_t pad;
};

constexpr int kReqMaxDescs = 64;

struct ReqBatch {
    ReqDesc d[kReqMaxDescs];
    int32_t n;
    int32_t pad;
};

hipError_t launch_quantize_block(const void* x, int64_t M, int64_t K, void* q, void* s, int fmt,
                                 hipStream_t st);
hipError_t launch_quantize_token(const void* x, int64_t M, int64_t K, void* q, float* s,
                                 hipStream_t st);
// res null: RMSNorm of x; else res := bf16(x + res) first, and that is normalized
hipError_t launch_rmsnorm_quant(void* q, const void* x, void* res, float* s, const void* gamma,
                                float eps, int64_t M, int64_t K, int group_size,
                                hipStream_t st);
hipError_t launch_requant(const ReqBatch& batch, int64_t total_blocks, int fmt, hipStream_t st);

hipError_t launch_encode_bits(uint64_t first, int64_t n, void* q, hipStream_t st);
hipError_t launch_bf16_bits(uint64_t first, int64_t n, void* out, hipStream_t st);

// Workspace of the stream-K small-M GEMM (caller-provided device memory):
// partial tiles of up to 256 workgroups x 2 slots of up to 256 x 128 fp32.
// Tile counts above kGemmWsMaxTiles run without a split.
constexpr int64_t kGemmWsMaxBytes = int64_t(256) * 2 * 256 * 128 * 4;
constexpr int64_t kGemmWsMaxTiles = int64_t(1) << 16;
struct GemmWorkspace {
    void* part;
    int64_t bytes;
};
// Workspace bytes launch_gemm / launch_batched_gemm_mx use for a shape (0 when
// the shape's path splits no tile); a smaller workspace runs the plan without
// a split.
int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int64_t mx_workspace_bytes(int64_t B, int64_t M, int64_t N, int64_t K);
// true when launch_gemm takes the small-M (128 x 128 tile) path for this shape
bool gemm_small_path(int64_t M, int64_t N, int64_t K);
// ws null or smaller than gemm_workspace_bytes: no tile is split
hipError_t launch_gemm(const void* a, const void* w, const float* a_s, const float* w_s,
                       void* y, int64_t M, int64_t N, int64_t K, int gran,
                       const GemmWorkspace* ws, hipStream_t st);
hipError_t launch_grouped_gemm(const void* a, const void* w, const float* a_s, const float* w_s,
                               const int32_t* offsets, void* y, int64_t T, int64_t E,
                               int64_t N, int64_t K, hipStream_t st);
// true when launch_batched_gemm_mx takes the small-M (128 x 128 tile) path
bool mx_small_path(int64_t B, int64_t M, int64_t N);
// B batches: A [M, B, K], W [B, N, K], E8M0 scales [M, B, K/128] and
// [B, N/128, K/128], Y [M, B, N].  Requires B * K <= 2^22 and int tile counts.
// ws as for launch_gemm (used by the small-M path, B == 1).
hipError_t launch_batched_gemm_mx(const void* a, const void* w, const uint8_t* a_s,
                                  const uint8_t* w_s, void* y, int64_t B, int64_t M, int64_t N,
                                  int64_t K, const GemmWorkspace* ws, hipStream_t st);

// Diagnostic: matrix-core rate probe (register operands), 1024 workgroups of
// 4 waves, out [4096] floats.
constexpr int kMfmaProbeWorkgroups = 1024;
hipError_t launch_mfma_probe(int64_t iters, float* out, hipStream_t st);

}  // namespace fp8k
