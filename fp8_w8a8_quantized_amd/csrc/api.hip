// api.hip -- the C ABI of libfp8w8a8.so (declared in include/fp8w8a8.h).
//
// Each entry point validates its arguments on the host (null pointers,
// alignment, the divisibility rules), then checks that the current device is
// gfx950, then enqueues its kernels.  On any error nothing is launched and
// nothing is written.  The refusal of shapes that are not multiples of 128 and
// the device capability check mirror the FP8 path preparation of the page
// "[vllm] [ROCm] DeepSeek V4 ... FP8 WO_A ...", §2, where the caller keeps its
// bf16 path when either fails.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/fp8w8a8.h"
#include "launch.hpp"
#include "tensor.hpp"

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_arch_once[kMaxDevices];
bool g_arch_ok[kMaxDevices];

// gfx950 check of the current device, cached per device.  The environment
// variable FP8W8A8_FORCE_ARCH replaces the reported architecture name (used
// to exercise the refusal path on a gfx950 machine).
int device_check() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return FP8_ERR_DEVICE;
    }
    const char* forced = std::getenv("FP8W8A8_FORCE_ARCH");
    if (forced) return std::strncmp(forced, "gfx950", 6) == 0 ? FP8_OK : FP8_ERR_DEVICE;
    std::call_once(g_arch_once[dev], [dev] {
        hipDeviceProp_t prop;
        g_arch_ok[dev] = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                         std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        (void)hipGetLastError();
    });
    return g_arch_ok[dev] ? FP8_OK : FP8_ERR_DEVICE;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int launched(hipError_t e) { return e == hipSuccess ? FP8_OK : FP8_ERR_LAUNCH; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Element counts whose byte sizes (up to 4 bytes per element) fit in int64.
bool count_ok(int64_t rows, int64_t cols) { return rows <= INT64_MAX / 4 / cols; }

// GEMM dimensions the kernels' index arithmetic covers: each below 2^31 and
// every operand below 2^48 bytes (far past any device memory), so no tile or
// step count overflows.
bool gemm_dims_ok(int64_t M, int64_t N, int64_t K) {
    const int64_t lim = int64_t(1) << 48;
    return M <= INT32_MAX && N <= INT32_MAX && K <= INT32_MAX && M * K < lim && N * K < lim &&
           M * N < lim / 2;
}

// The workspace argument pair of the GEMMs: NULL with 0 bytes runs the plan
// without a split; otherwise the pointer must be 16-byte aligned and hold at
// least `need` bytes.
int workspace_check(const void* ws, size_t bytes, int64_t need) {
    if (ws == nullptr) return bytes == 0 ? FP8_OK : FP8_ERR_ARG;
    if (!aligned(ws, 16)) return FP8_ERR_ALIGN;
    return bytes >= (size_t)need ? FP8_OK : FP8_ERR_ARG;
}

// Scratch of fp8_gemm_a8w8_scaled_noalloc: the stream-K partial tiles of the
// largest plan (256 workgroups x 2 slots of 256 x 128 fp32), one array per
// GPU, held until the process ends.  Host code never uses the array's name as
// an address: each device's address comes from hipGetSymbolAddress, taken on
// the first call on that device.
constexpr int64_t kScratchBytes = fp8k::kGemmWsMaxBytes;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch address (looked up once per device, with that
// device current), or null when the lookup failed.
void* scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            p = nullptr;
        }
        g_scratch_ptr[dev] = p;
    });
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int fp8_abi_version(void) { return FP8W8A8_ABI_VERSION; }

#ifndef FP8W8A8_SOURCE_SHA256
#define FP8W8A8_SOURCE_SHA256 "unknown"
#endif
// The tag makes the hash findable in the file without loading it.
static const char kSourceHash[] = "FP8W8A8_SOURCE_SHA256=" FP8W8A8_SOURCE_SHA256;

const char* fp8_build_source_hash(void) { return kSourceHash + 22; }

const char* fp8_status_string(int status) {
    switch (status) {
        case FP8_OK: return "ok";
        case FP8_ERR_ARG: return "invalid argument";
        case FP8_ERR_SHAPE: return "unsupported shape (a dimension is not a required multiple)";
        case FP8_ERR_ALIGN: return "misaligned pointer";
        case FP8_ERR_DEVICE: return "no gfx950 (MI355X) HIP device";
        case FP8_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

int fp8_quantize_block(const void* x, int64_t M, int64_t K, void* q, float* s, void* stream) {
    if (M < 0 || K <= 0) return K <= 0 ? FP8_ERR_SHAPE : FP8_ERR_ARG;
    if (K % 128 != 0 || !count_ok(M, K)) return FP8_ERR_SHAPE;
    if (M == 0) return FP8_OK;
    if (!x || !q || !s) return FP8_ERR_ARG;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return FP8_ERR_ALIGN;
    if (int st = device_check()) return st;
    return launched(fp8k::launch_quantize_block(x, M, K, q, s, 0, as_stream(stream)));
}

int fp8_quantize_block_e8m0(const void* x, int64_t M, int64_t K, void* q, void* s,
                            void* stream) {
    if (M < 0 || K <= 0) return K <= 0 ? FP8_ERR_SHAPE : FP8_ERR_ARG;
    if (K % 128 != 0 || !count_ok(M, K)) return FP8_ERR_SHAPE;
    if (M == 0) return FP8_OK;
    if (!x || !q || !s) return FP8_ERR_ARG;
    if (!aligned(x, 16) || !aligned(q, 16)) return FP8_ERR_ALIGN;
    if (int st = device_check()) return st;
    return launched(fp8k::launch_quantize_block(x, M, K, q, s, 1, as_stream(stream)));
}

int fp8_quantize_token(const void* x, int64_t M, int64_t K, void* q, float* s, void* stream) {
    if (M < 0) return FP8_ERR_ARG;
    if (K <= 0 || K % 8 != 0 || !count_ok(M, K)) return FP8_ERR_SHAPE;
    if (M == 0) return FP8_OK;
    if (!x || !q || !s) return FP8_ERR_ARG;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return FP8_ERR_ALIGN;
    if (int st = device_check()) return st;
    return launched(fp8k::launch_quantize_token(x, M, K, q, s, as_stream(stream)));
}

int fp8_rmsnorm_quant(void* q, const void* x, float* s, const void* gamma, float eps, int64_t M,
                      int64_t K, int group_size, void* stream) {
    if (M < 0 || (group_size != 0 && group_size != 128)) return FP8_ERR_ARG;
    if (K <= 0 || K % (group_size == 0 ? 8 : 128) != 0 || !count_ok(M, K)) return FP8_ERR_SHAPE;
    if (M == 0) return FP8_OK;
    if (!x || !q || !s || !gamma) return FP8_ERR_ARG;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(gamma, 16) || !aligned(s, 4))
        return FP8_ERR_ALIGN;
    if (int st = device_check()) return st;
    return launched(fp8k::launch_rmsnorm_quant(q, x, nullptr, s, gamma, eps, M, K, group_size,
                                               as_stream(stream)));
}

int fp8_add_rmsnorm_quant(void* q, const void* x, void* residual, float* s, const void* gamma,
                          float eps, int64_t M, int64_t K, int group_size, void* stream) {
    if (M < 0 || (group_size != 0 && group_size != 128)) return FP8_ERR_ARG;
    if (K <= 0 || K % (group_size == 0 ? 8 : 128) != 0) return FP8_ERR_SHAPE;
    if (M == 0) return FP8_OK;
    if (!x || !residual || !q || !s || !gamma) return FP8_ERR_ARG;
    if (!aligned(x, 16) || !aligned(residual, 16) || !aligned(q, 16) || !aligned(gamma, 16) ||
        !aligned(s, 4))
        return FP8_ERR_ALIGN;
    if (M > INT64_MAX / 2 / K) return FP8_ERR_SHAPE;  // byte size must fit
    const int64_t bytes = M * K * 2;
    const char* xb = static_cast<const char*>(x);
    const char* rb = static_cast<const char*>(residual);
    if (xb < rb + bytes && rb < xb + bytes) return FP8_ERR_ARG;  // x and residual overlap
    if (int st = device_check()) return st;
    return launched(fp8k::launch_rmsnorm_quant(q, x, residual, s, gamma, eps, M, K, group_size,
                                               as_stream(stream)));
}

size_t fp8_requantize_workspace_size(int n) {
    (void)n;
    return 0;
}

int fp8_requantize_weights(const fp8_weight_desc* descs, int n, int scale_fmt, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (n < 0 || (scale_fmt != FP8_SCALE_F32 && scale_fmt != FP8_SCALE_E8M0)) return FP8_ERR_ARG;
    if (int st = workspace_check(workspace, workspace_bytes, (int64_t)fp8_requantize_workspace_size(n)))
        return st;
    if (n == 0) return FP8_OK;
    if (!descs) return FP8_ERR_ARG;
    int work = 0;
    for (int i = 0; i < n; ++i) {
        const fp8_weight_desc& d = descs[i];
        if (d.N < 0 || d.K < 0) return FP8_ERR_ARG;
        if (d.N % 128 != 0 || d.K % 128 != 0) return FP8_ERR_SHAPE;
        if (d.N == 0 || d.K == 0) continue;
        if (!d.w_bf16 || !d.q_e4m3 || !d.s) return FP8_ERR_ARG;
        if (!aligned(d.w_bf16, 16) || !aligned(d.q_e4m3, 16) ||
            !aligned(d.s, scale_fmt == FP8_SCALE_F32 ? 4 : 1))
            return FP8_ERR_ALIGN;
        ++work;
    }
    if (work == 0) return FP8_OK;  // only empty weights: nothing to launch
    if (int st = device_check()) return st;
    fp8k::ReqBatch batch;
    std::memset(&batch, 0, sizeof(batch));
    int64_t blocks = 0;
    auto flush = [&]() -> int {
        if (batch.n == 0) return FP8_OK;
        const int r = launched(fp8k::launch_requant(batch, blocks, scale_fmt, as_stream(stream)));
        std::memset(&batch, 0, sizeof(batch));
        blocks = 0;
        return r;
    };
    for (int i = 0; i < n; ++i) {
        const fp8_weight_desc& d = descs[i];
        if (d.N == 0 || d.K == 0) continue;
        fp8k::ReqDesc& r = batch.d[batch.n++];
        r.w = static_cast<const uint16_t*>(d.w_bf16);
        r.q = static_cast<uint8_t*>(d.q_e4m3);
        r.s = d.s;
        r.K = d.K;
        r.kblocks = (int32_t)(d.K / 128);
        r.block_begin = blocks;
        blocks += (d.N / 128) * (d.K / 128);
        if (batch.n == fp8k::kReqMaxDescs)
            if (int st = flush()) return st;
    }
    return flush();
}

int fp8_quantize_tensors(const fp8_tensor_desc* descs, int n, void* stream) {
    if (n < 0) return FP8_ERR_ARG;
    if (n == 0) return FP8_OK;
    if (!descs) return FP8_ERR_ARG;
    int work = 0;
    for (int i = 0; i < n; ++i) {
        const fp8_tensor_desc& d = descs[i];
        if (d.n < 0) return FP8_ERR_ARG;
        if (d.n % 8 != 0) return FP8_ERR_SHAPE;
        if (d.n == 0) continue;
        if (!d.x_bf16 || !d.q_e4m3 || !d.s) return FP8_ERR_ARG;
        if (!aligned(d.x_bf16, 16) || !aligned(d.q_e4m3, 16) || !aligned(d.s, 4))
            return FP8_ERR_ALIGN;
        ++work;
    }
    if (work == 0) return FP8_OK;  // only empty tensors: nothing to launch
    if (int st = device_check()) return st;
    fp8k::TensBatch batch;
    std::memset(&batch, 0, sizeof(batch));
    int64_t chunks = 0;
    auto flush = [&]() -> int {
        if (batch.n == 0) return FP8_OK;
        const int r = launched(fp8k::launch_tensor_batch(batch, chunks, as_stream(stream)));
        std::memset(&batch, 0, sizeof(batch));
        chunks = 0;
        return r;
    };
    for (int i = 0; i < n; ++i) {
        const fp8_tensor_desc& d = descs[i];
        if (d.n == 0) continue;
        fp8k::TensDesc& t = batch.d[batch.n++];
        t.x = d.x_bf16;
        t.q = d.q_e4m3;
        t.s = d.s;
        t.nvec = d.n / 8;
        t.chunk_begin = chunks;
        chunks += (t.nvec + fp8k::kTensChunk - 1) / fp8k::kTensChunk;
        if (batch.n == fp8k::kTensMaxDescs || chunks > (int64_t(1) << 30))
            if (int st = flush()) return st;
    }
    return flush();
}

size_t fp8_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int gran) {
    if (gran != FP8_GRAN_BLOCK && gran != FP8_GRAN_ROW) return 0;
    if (M <= 0 || N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0) return 0;
    if (!gemm_dims_ok(M, N, K)) return 0;
    return (size_t)fp8k::gemm_workspace_bytes(M, N, K);
}

int fp8_gemm_a8w8_scaled(const void* a, const void* w, const float* a_s, const float* w_s,
                         const void* bias, void* y, int64_t M, int64_t N, int64_t K, int gran,
                         void* workspace, size_t workspace_bytes, void* stream) {
    if (bias != nullptr) return FP8_ERR_ARG;
    if (gran != FP8_GRAN_BLOCK && gran != FP8_GRAN_ROW) return FP8_ERR_ARG;
    if (M < 0) return FP8_ERR_ARG;
    if (N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0) return FP8_ERR_SHAPE;
    if (!gemm_dims_ok(M, N, K)) return FP8_ERR_SHAPE;
    if (M == 0) return FP8_OK;
    if (!a || !w || !a_s || !w_s || !y) return FP8_ERR_ARG;
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(y, 16) || !aligned(a_s, 4) ||
        !aligned(w_s, 4))
        return FP8_ERR_ALIGN;
    if (int st = workspace_check(workspace, workspace_bytes, fp8k::gemm_workspace_bytes(M, N, K)))
        return st;
    if (int st = device_check()) return st;
    const fp8k::GemmWorkspace ws{workspace, (int64_t)workspace_bytes};
    return launched(fp8k::launch_gemm(a, w, a_s, w_s, y, M, N, K, gran, &ws, as_stream(stream)));
}

int fp8_gemm_a8w8_scaled_noalloc(const void* a, const void* w, const float* a_s,
                                 const float* w_s, const void* bias, void* y, int64_t M, int64_t N,
                                 int64_t K, int gran, void* stream) {
    if (bias != nullptr) return FP8_ERR_ARG;
    if (gran != FP8_GRAN_BLOCK && gran != FP8_GRAN_ROW) return FP8_ERR_ARG;
    if (M < 0) return FP8_ERR_ARG;
    if (N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0) return FP8_ERR_SHAPE;
    if (!gemm_dims_ok(M, N, K)) return FP8_ERR_SHAPE;
    if (M == 0) return FP8_OK;
    if (!a || !w || !a_s || !w_s || !y) return FP8_ERR_ARG;
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(y, 16) || !aligned(a_s, 4) ||
        !aligned(w_s, 4))
        return FP8_ERR_ALIGN;
    if (fp8k::gemm_workspace_bytes(M, N, K) > kScratchBytes) return FP8_ERR_SHAPE;
    if (int st = device_check()) return st;
    void* ptr = scratch_address();
    if (ptr == nullptr) return FP8_ERR_DEVICE;
    const fp8k::GemmWorkspace ws{ptr, kScratchBytes};
    return launched(fp8k::launch_gemm(a, w, a_s, w_s, y, M, N, K, gran, &ws, as_stream(stream)));
}

int fp8_grouped_gemm_a8w8_scaled(const void* a, const void* w, const float* a_s,
                                 const float* w_s, const int32_t* offsets, void* y, int64_t T,
                                 int64_t E, int64_t N, int64_t K, void* stream) {
    if (T < 0 || E < 1 || E > 1024 || T > INT32_MAX) return FP8_ERR_ARG;
    if (N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0) return FP8_ERR_SHAPE;
    if (!gemm_dims_ok(T, N, K) || E * N > INT32_MAX || !gemm_dims_ok(T, E * N, K))
        return FP8_ERR_SHAPE;
    if (T == 0) return FP8_OK;
    if (!a || !w || !a_s || !w_s || !offsets || !y) return FP8_ERR_ARG;
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(y, 16) || !aligned(a_s, 4) ||
        !aligned(w_s, 4) || !aligned(offsets, 4))
        return FP8_ERR_ALIGN;
    if (int st = device_check()) return st;
    return launched(fp8k::launch_grouped_gemm(a, w, a_s, w_s, offsets, y, T, E, N, K,
                                              as_stream(stream)));
}

// Shape limits of the batched MX GEMM: 32-bit tile offsets (256 rows of B * K
// bytes), tile and step counts in int.
static int mx_shape_check(int64_t B, int64_t M, int64_t N, int64_t K) {
    if (N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0) return FP8_ERR_SHAPE;
    if (B <= 0 || M <= 0) return FP8_OK;
    if (B > (int64_t(1) << 22) / K) return FP8_ERR_SHAPE;  // B * K > 2^22
    if (N > INT32_MAX || !gemm_dims_ok(M, B * N, B * K)) return FP8_ERR_SHAPE;
    const int64_t tiles = B * ((M + 255) / 256) * ((N + 255) / 256);
    if (tiles > INT32_MAX || (tiles / 256 + 1) * (K / 128) > INT32_MAX) return FP8_ERR_SHAPE;
    return FP8_OK;
}

size_t fp8_batched_gemm_mxscale_workspace_size(int64_t B, int64_t M, int64_t N, int64_t K) {
    if (B <= 0 || M <= 0 || mx_shape_check(B, M, N, K) != FP8_OK) return 0;
    return (size_t)fp8k::mx_workspace_bytes(B, M, N, K);
}

int fp8_batched_gemm_a8w8_mxscale(const void* a, const void* w, const void* a_s, const void* w_s,
                                  void* y, int64_t B, int64_t M, int64_t N, int64_t K,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (M < 0 || B < 0) return FP8_ERR_ARG;
    if (int st = mx_shape_check(B, M, N, K)) return st;
    if (M == 0 || B == 0) return FP8_OK;
    if (!a || !w || !a_s || !w_s || !y) return FP8_ERR_ARG;
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(y, 16)) return FP8_ERR_ALIGN;
    if (int st = workspace_check(workspace, workspace_bytes,
                                 fp8k::mx_workspace_bytes(B, M, N, K)))
        return st;
    if (int st = device_check()) return st;
    const fp8k::GemmWorkspace ws{workspace, (int64_t)workspace_bytes};
    return launched(fp8k::launch_batched_gemm_mx(a, w, static_cast<const uint8_t*>(a_s),
                                                 static_cast<const uint8_t*>(w_s), y, B, M, N, K,
                                                 &ws, as_stream(stream)));
}

int fp8_encode_f32_bits(uint64_t first_bits, int64_t n, void* q, void* stream) {
    if (n < 0 || first_bits > 0xFFFFFFFFull || (uint64_t)n > 0x100000000ull - first_bits)
        return FP8_ERR_ARG;
    if (n == 0) return FP8_OK;
    if (!q) return FP8_ERR_ARG;
    if (!aligned(q, 16)) return FP8_ERR_ALIGN;
    if (int st = device_check()) return st;
    return launched(fp8k::launch_encode_bits(first_bits, n, q, as_stream(stream)));
}

int fp8_bf16_round_f32_bits(uint64_t first_bits, int64_t n, void* out, void* stream) {
    if (n < 0 || first_bits > 0xFFFFFFFFull || (uint64_t)n > 0x100000000ull - first_bits)
        return FP8_ERR_ARG;
    if (n == 0) return FP8_OK;
    if (!out) return FP8_ERR_ARG;
    if (!aligned(out, 16)) return FP8_ERR_ALIGN;
    if (int st = device_check()) return st;
    return launched(fp8k::launch_bf16_bits(first_bits, n, out, as_stream(stream)));
}

int fp8_swiglu_quant(const void* gu, int64_t T, int64_t I, void* q, float* s, void* stream) {
    if (T < 0) return FP8_ERR_ARG;
    if (I <= 0 || I % 128 != 0 || I > INT64_MAX / 8 || !count_ok(T, 2 * I)) return FP8_ERR_SHAPE;
    if (T == 0) return FP8_OK;
    if (!gu || !q || !s) return FP8_ERR_ARG;
    if (!aligned(gu, 16) || !aligned(q, 16) || !aligned(s, 4)) return FP8_ERR_ALIGN;
    if (int st = device_check()) return st;
    return launched(fp8k::launch_swiglu_quant(gu, T, I, q, s, as_stream(stream)));
}

int fp8_quantize_block_gather(const void* x, int64_t n_src, int64_t K, const int32_t* row_token,
                              int64_t T, void* q, float* s, void* stream) {
    if (T < 0 || n_src < 0 || n_src > INT32_MAX) return FP8_ERR_ARG;
    if (K <= 0 || K % 128 != 0 || !count_ok(T, K) || !count_ok(n_src, K)) return FP8_ERR_SHAPE;
    if (T == 0) return FP8_OK;
    if (!row_token || !q || !s || (n_src > 0 && !x)) return FP8_ERR_ARG;
    if (!aligned(x, 16) || !aligned(row_token, 4) || !aligned(q, 16) || !aligned(s, 4))
        return FP8_ERR_ALIGN;
    if (int st = device_check()) return st;
    return launched(
        fp8k::launch_quant_gather(x, n_src, K, row_token, T, q, s, as_stream(stream)));
}

int fp8_inverse_rope_group_quant(const void* o, const int64_t* positions, const float* cos_cache,
                                 const float* sin_cache, int64_t T, int64_t H, int64_t D,
                                 int64_t rope_dim, int64_t max_pos, int64_t num_groups, void* q,
                                 uint8_t* s, void* stream) {
    if (T < 0 || rope_dim < 0 || rope_dim % 2 != 0 || max_pos < 0 || num_groups <= 0)
        return FP8_ERR_ARG;
    if (H <= 0 || D <= 0 || D % 8 != 0 || rope_dim > D || H % num_groups != 0 ||
        D > INT32_MAX || H > (INT32_MAX - 1) / D)  // a row's offsets fit in int
        return FP8_ERR_SHAPE;
    if ((H / num_groups) * D % 128 != 0 || !count_ok(T, H * D)) return FP8_ERR_SHAPE;
    if (rope_dim > 0 && max_pos == 0) return FP8_ERR_ARG;
    if (max_pos > INT64_MAX / (rope_dim / 2 + 1)) return FP8_ERR_ARG;
    if (T == 0) return FP8_OK;
    if (!o || !positions || !q || !s || (rope_dim > 0 && (!cos_cache || !sin_cache)))
        return FP8_ERR_ARG;
    if (!aligned(o, 16) || !aligned(q, 16) || !aligned(positions, 8) || !aligned(cos_cache, 4) ||
        !aligned(sin_cache, 4))
        return FP8_ERR_ALIGN;
    if (int st = device_check()) return st;
    return launched(fp8k::launch_inv_rope_quant(o, positions, cos_cache, sin_cache, T, H, D,
                                                rope_dim, max_pos, q, s, as_stream(stream)));
}

int fp8_mfma_rate_probe(int64_t iters, float* out, void* stream) {
    if (iters < 0 || iters > (int64_t(1) << 32)) return FP8_ERR_ARG;
    if (!out) return FP8_ERR_ARG;
    if (!aligned(out, 4)) return FP8_ERR_ALIGN;
    if (int st = device_check()) return st;
    return launched(fp8k::launch_mfma_probe(iters, out, as_stream(stream)));
}

int fp8_silu_f32_of_bf16(uint32_t first_bits, int64_t n, float* out, void* stream) {
    if (n < 0 || first_bits > 0xFFFFu || (uint64_t)n > 0x10000u - first_bits) return FP8_ERR_ARG;
    if (n == 0) return FP8_OK;
    if (!out) return FP8_ERR_ARG;
    if (!aligned(out, 4)) return FP8_ERR_ALIGN;
    if (int st = device_check()) return st;
    return launched(fp8k::launch_silu_bits(first_bits, n, out, as_stream(stream)));
}

}  // extern "C"
