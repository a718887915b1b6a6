// abi_sanitize.cpp -- the C ABI's host-side validation under AddressSanitizer
// and UndefinedBehaviorSanitizer.  Built host-only (no device code) together
// with the library's sources, it calls every entry point with the invalid
// arguments that must be refused before any device work, and with valid ones
// that must reach the device check (no HIP device is needed: without one the
// calls return FP8_ERR_DEVICE).  Exit status 0: every status was as expected
// and the sanitizers saw nothing.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../include/fp8w8a8.h"

static int failures = 0;
#define EXPECT(call, want)                                                          \
    do {                                                                            \
        const int got_ = (call);                                                    \
        if (got_ != (want)) {                                                       \
            std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, \
                         #call, got_, (int)(want));                                 \
            ++failures;                                                             \
        }                                                                           \
    } while (0)

int main() {
    // a non-null, 64 KiB-aligned address that the refused calls never touch
    void* f = reinterpret_cast<void*>(uintptr_t(0x10000));
    char* fc = static_cast<char*>(f);
    float* ff = static_cast<float*>(f);
    const int ARG = FP8_ERR_ARG, SHAPE = FP8_ERR_SHAPE, ALIGN = FP8_ERR_ALIGN;
    const int DEVICE = FP8_ERR_DEVICE;

    EXPECT(fp8_abi_version(), FP8W8A8_ABI_VERSION);
    for (int st = -6; st <= 1; ++st) EXPECT(fp8_status_string(st) != nullptr, 1);
    EXPECT(fp8_build_source_hash() != nullptr, 1);

    EXPECT(fp8_quantize_block(f, 4, 200, f, ff, nullptr), SHAPE);
    EXPECT(fp8_quantize_block(f, -1, 128, f, ff, nullptr), ARG);
    EXPECT(fp8_quantize_block(fc + 2, 4, 128, f, ff, nullptr), ALIGN);
    EXPECT(fp8_quantize_block(f, 0, 128, nullptr, nullptr, nullptr), FP8_OK);
    EXPECT(fp8_quantize_block_e8m0(f, 4, 128, f, nullptr, nullptr), ARG);
    EXPECT(fp8_quantize_token(f, 4, 12, f, ff, nullptr), SHAPE);
    EXPECT(fp8_rmsnorm_quant(f, f, ff, f, 1e-6f, 4, 16, 64, nullptr), ARG);
    EXPECT(fp8_add_rmsnorm_quant(f, f, fc + 64, ff, f, 1e-6f, 4, 16, 0, nullptr), ARG);
    EXPECT(fp8_add_rmsnorm_quant(f, f, fc + (1 << 20), ff, f, 1e-6f, int64_t(1) << 60, 16, 0,
                                 nullptr),
           SHAPE);
    EXPECT(fp8_swiglu_quant(f, 4, 100, f, ff, nullptr), SHAPE);
    EXPECT(fp8_silu_f32_of_bf16(0xFFFF, 2, ff, nullptr), ARG);
    EXPECT(fp8_quantize_block_gather(f, int64_t(1) << 31, 128, static_cast<int32_t*>(f), 4, f, ff,
                                     nullptr),
           ARG);
    EXPECT(fp8_inverse_rope_group_quant(f, static_cast<int64_t*>(f), ff, ff, 4, 4, 128, 63, 16, 1,
                                        f, static_cast<uint8_t*>(f), nullptr),
           ARG);
    EXPECT(fp8_inverse_rope_group_quant(f, static_cast<int64_t*>(f), ff, ff, 4, INT64_MAX, 128,
                                        64, 16, 1, f, static_cast<uint8_t*>(f), nullptr),
           SHAPE);
    // element counts whose byte sizes would overflow
    EXPECT(fp8_quantize_block(f, INT64_MAX / 128, 256, f, ff, nullptr), SHAPE);
    EXPECT(fp8_quantize_token(f, INT64_MAX / 8, 16, f, ff, nullptr), SHAPE);
    EXPECT(fp8_rmsnorm_quant(f, f, ff, f, 1e-6f, INT64_MAX / 8, 16, 0, nullptr), SHAPE);
    EXPECT(fp8_swiglu_quant(f, 4, INT64_MAX - 127, f, ff, nullptr), SHAPE);
    EXPECT(fp8_swiglu_quant(f, INT64_MAX / 256, 128, f, ff, nullptr), SHAPE);
    EXPECT(fp8_gemm_a8w8_scaled(f, f, ff, ff, nullptr, f, INT64_MAX, 256, 256, 0, nullptr, 0,
                                nullptr),
           SHAPE);
    EXPECT(fp8_grouped_gemm_a8w8_scaled(f, f, ff, ff, static_cast<int32_t*>(f), f, 64, 4,
                                        INT64_MAX - 127, 256, nullptr),
           SHAPE);
    EXPECT(fp8_encode_f32_bits(0xFFFFFFFFull, 2, f, nullptr), ARG);
    EXPECT(fp8_bf16_round_f32_bits(uint64_t(1) << 32, 1, f, nullptr), ARG);

    // requantization: a descriptor table of several entries, one bad
    std::vector<fp8_weight_desc> d(70, fp8_weight_desc{f, f, f, 256, 256});
    EXPECT(fp8_requantize_workspace_size(70), 0u);
    EXPECT(fp8_requantize_weights(d.data(), 70, FP8_SCALE_F32, nullptr, 0, nullptr), DEVICE);
    EXPECT(fp8_requantize_weights(d.data(), 70, FP8_SCALE_F32, nullptr, 64, nullptr), ARG);
    d[69].N = 200;
    EXPECT(fp8_requantize_weights(d.data(), 70, FP8_SCALE_F32, nullptr, 0, nullptr), SHAPE);
    EXPECT(fp8_requantize_weights(d.data(), 70, 5, nullptr, 0, nullptr), ARG);
    std::vector<fp8_tensor_desc> t(3, fp8_tensor_desc{f, f, ff, 64});
    t[1].n = 12;
    EXPECT(fp8_quantize_tensors(t.data(), 3, nullptr), SHAPE);
    t[1].n = INT64_MAX - 7;  // a multiple of 8 whose chunk count must not overflow
    EXPECT(fp8_quantize_tensors(t.data(), 3, nullptr), DEVICE);

    // GEMMs, their workspace queries and checks
    EXPECT(fp8_gemm_a8w8_scaled(f, f, ff, ff, f, f, 16, 256, 256, 0, nullptr, 0, nullptr), ARG);
    EXPECT(fp8_gemm_a8w8_scaled(f, f, ff, ff, nullptr, f, 16, 200, 256, 0, nullptr, 0, nullptr),
           SHAPE);
    const size_t need = fp8_gemm_workspace_size(256, 4096, 12288, FP8_GRAN_BLOCK);
    EXPECT(need == size_t(256) * 2 * 256 * 128 * 4, 1);
    EXPECT(fp8_gemm_workspace_size(INT64_MAX, 256, 256, 0) == 0, 1);
    EXPECT(fp8_gemm_workspace_size(1, INT64_MAX - 127, 128, 0) == 0, 1);
    EXPECT(fp8_gemm_a8w8_scaled(f, f, ff, ff, nullptr, f, 256, 4096, 12288, 0, f, need - 16,
                                nullptr),
           ARG);
    EXPECT(fp8_gemm_a8w8_scaled(f, f, ff, ff, nullptr, f, 256, 4096, 12288, 0, f, need, nullptr),
           DEVICE);
    EXPECT(fp8_gemm_a8w8_scaled_noalloc(f, f, ff, ff, nullptr, f, 256, 4096, 12288, 0, nullptr),
           DEVICE);
    EXPECT(fp8_grouped_gemm_a8w8_scaled(f, f, ff, ff, static_cast<int32_t*>(f), f, 64, 1025, 256,
                                        256, nullptr),
           ARG);
    EXPECT(fp8_batched_gemm_a8w8_mxscale(f, f, f, f, f, 4, 16, 256, int64_t(1) << 21, nullptr, 0,
                                         nullptr),
           SHAPE);
    EXPECT(fp8_batched_gemm_a8w8_mxscale(f, f, f, f, f, INT64_MAX, INT64_MAX, 256, 256, nullptr,
                                         0, nullptr),
           SHAPE);
    EXPECT(fp8_batched_gemm_mxscale_workspace_size(1, 256, 4096, 12288) == need, 1);

    std::printf("abi sanitize checks: %d failures\n", failures);
    return failures == 0 ? 0 : 1;
}
