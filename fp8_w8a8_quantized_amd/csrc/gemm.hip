// gemm.hip -- FP8 W8A8 scaled GEMMs for gfx950 (dense and MoE-grouped).
//
// Pages (title, section):
//   "FP8-RL: A Practical and Stable Low-Precision Stack for LLM RL", abstract
//     (i): W8A8 linear layers with blockwise scales, dense and MoE models.
//   "[vllm] [ROCm] DeepSeek V4 ... FP8 WO_A ...", §2 weights (groups, out, in)
//     with block scales (groups, out/128, in/128); §3 the a8w8 GEMM fed by
//     group-128 activations, bf16 output.
//   "[sglang] SGLang의 AMD GPU 최적화: RMSNorm과 FP8 Per-token Quantization 커널
//     융합", §3 the per-token x per-channel a8w8 GEMM (A, B, A-scale, B-scale,
//     bias None, bf16 out).
//
// Y = X W^T, X [M, K] and W [N, K] both K-contiguous E4M3.
//   BLOCK: Y[m,n] = sum_kb sA[m,kb] sW[n/128,kb] P_kb[m,n], P_kb the exact-product
//          fp32 sum over the 128-wide K block kb.
//   ROW:   Y[m,n] = sA[m] sW[n] sum_k X[m,k] W[n,k].
//
// Design (CDNA4):
//   * Workgroup tile 128 x 128, K step 128 = one scale block; 256 threads as
//     2 x 2 waves, each wave a 64 x 64 sub-tile of 4 x 4 MFMA tiles.
//   * v_mfma_f32_16x16x128_f8f6f4 (both operands E4M3): one instruction is a
//     16 x 16 tile over a whole 128-wide K block, so BLOCK mode gets P_kb from
//     one MFMA with a zero accumulator and promotes it with one fp32 FMA per
//     output element: acc += P_kb * (sA * sW).  ROW mode accumulates in the
//     MFMA and scales once in the epilogue.
//   * A and W tiles are staged in LDS, double buffered: the next K block is
//     loaded into registers (16-byte loads, one 128-byte row segment per 8
//     threads) while the current one is multiplied, then written to the other
//     buffer; one barrier per K block.  16-byte chunks of each 128-byte tile
//     row are XOR-swizzled by the row index so the MFMA operand reads of 8
//     consecutive rows hit distinct banks.
//   * MFMA operand layout (16x16x128, 8-bit): lane l supplies row l % 16 of
//     its operand and 32 consecutive K bytes starting at 32 * (l / 16); A and
//     W use the same K assignment, so every product pairs matching k.  The
//     result holds D[4 * (l / 16) + i][l % 16] in element i of lane l.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "launch.hpp"

namespace fp8k {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int GRAN_BLOCK = 0, GRAN_ROW = 1;

__device__ __forceinline__ v4f mfma_f8(const v8i& a, const v8i& b, const v4f& c) {
    // cbsz = blgp = 0: both operands E4M3; scale operands 0 -> unscaled form
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// byte offset of 16-byte chunk `c` of tile row `r` (128 bytes per row)
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ (r & 7)) << 4); }

// One output tile's work description.
struct Tile {
    const uint8_t* A;   // first row of the tile's rows (row0)
    const float* sA;    // scales of row0 (BLOCK: [.., KB] per row; ROW: one per row)
    const uint8_t* W;   // first row of the tile's columns (n0)
    const float* sW;    // BLOCK: scale row of weight block n0/128; ROW: sW + n0
    uint16_t* Y;        // &Y[row0][n0]
    int rows;           // valid rows in this tile (1..128)
};

template <int GRAN>
__device__ __forceinline__ void stage_load(const Tile& t, int64_t K, int64_t KB, int64_t kb,
                                           int gr, int gc, int tid, v4i (&ra)[4],
                                           v4i (&rb)[4], float& rsa) {
    // Rows past the tile's end (ragged M) re-read the last valid row: a row of
    // A only reaches its own output row, and those rows are never stored.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = gr + 32 * i;
        const int ra_row = r < t.rows ? r : t.rows - 1;
        ra[i] = *reinterpret_cast<const v4i*>(t.A + ra_row * K + kb * BK + gc * 16);
        rb[i] = *reinterpret_cast<const v4i*>(t.W + r * K + kb * BK + gc * 16);
    }
    if constexpr (GRAN == GRAN_BLOCK) {
        if (tid < BM) rsa = t.sA[(tid < t.rows ? tid : t.rows - 1) * KB + kb];
    }
}

template <int GRAN>
__device__ __forceinline__ void stage_store(uint8_t* lds_a, uint8_t* lds_b, float* lds_sa,
                                            int buf, int gr, int gc, int tid,
                                            const v4i (&ra)[4], const v4i (&rb)[4],
                                            float rsa) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = gr + 32 * i;
        *reinterpret_cast<v4i*>(lds_a + buf * BM * BK + swz(r, gc)) = ra[i];
        *reinterpret_cast<v4i*>(lds_b + buf * BN * BK + swz(r, gc)) = rb[i];
    }
    if constexpr (GRAN == GRAN_BLOCK) {
        if (tid < BM) lds_sa[buf * BM + tid] = rsa;
    }
}

template <int GRAN>
__device__ __forceinline__ void gemm_tile(const Tile& t, int64_t K, int64_t ldy, uint8_t* lds) {
    uint8_t* lds_a = lds;                       // [2][BM * BK]
    uint8_t* lds_b = lds + 2 * BM * BK;         // [2][BN * BK]
    float* lds_sa = reinterpret_cast<float*>(lds + 2 * (BM + BN) * BK);  // [2][BM]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lk = lane >> 4;
    const int64_t KB = K / BK;

    // global -> register staging: thread loads chunk (tid & 7) of rows tid/8 + 32 i
    const int gc = tid & 7, gr = tid >> 3;
    v4i ra[4], rb[4];
    float rsa = 0.0f;
    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    stage_load<GRAN>(t, K, KB, 0, gr, gc, tid, ra, rb, rsa);
    stage_store<GRAN>(lds_a, lds_b, lds_sa, 0, gr, gc, tid, ra, rb, rsa);
    __syncthreads();

    for (int64_t kb = 0; kb < KB; ++kb) {
        const int cur = (int)(kb & 1);
        if (kb + 1 < KB) stage_load<GRAN>(t, K, KB, kb + 1, gr, gc, tid, ra, rb, rsa);

        const uint8_t* la = lds_a + cur * BM * BK;
        const uint8_t* lb = lds_b + cur * BN * BK;
        v8i a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 64 + i * 16 + lr;
            const v4i lo = *reinterpret_cast<const v4i*>(la + swz(r, 2 * lk));
            const v4i hi = *reinterpret_cast<const v4i*>(la + swz(r, 2 * lk + 1));
            a[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = wn * 64 + j * 16 + lr;
            const v4i lo = *reinterpret_cast<const v4i*>(lb + swz(r, 2 * lk));
            const v4i hi = *reinterpret_cast<const v4i*>(lb + swz(r, 2 * lk + 1));
            b[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        if constexpr (GRAN == GRAN_BLOCK) {
            const float sw = t.sW[kb];
            v4f sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const v4f s4 = *reinterpret_cast<const v4f*>(lds_sa + cur * BM + wm * 64 +
                                                             i * 16 + 4 * lk);
                sc[i] = s4 * sw;
            }
            const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const v4f p = mfma_f8(a[i], b[j], zero);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i][j][e] = __builtin_fmaf(p[e], sc[i][e], acc[i][j][e]);
                }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i][j] = mfma_f8(a[i], b[j], acc[i][j]);
        }

        if (kb + 1 < KB) stage_store<GRAN>(lds_a, lds_b, lds_sa, cur ^ 1, gr, gc, tid, ra, rb, rsa);
        __syncthreads();
    }

    // epilogue: bf16 (nearest even) stores; ROW mode applies sA[m] * sW[n]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = wm * 64 + i * 16 + 4 * lk + e;
            if (r >= t.rows) continue;
            float sa = 1.0f;
            if constexpr (GRAN == GRAN_ROW) sa = t.sA[r];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = wn * 64 + j * 16 + lr;
                float v = acc[i][j][e];
                if constexpr (GRAN == GRAN_ROW) v = v * (sa * t.sW[c]);
                t.Y[(int64_t)r * ldy + c] = (uint16_t)bf16_rne_bits(v);
            }
        }
    }
}

constexpr int kLdsBytes = 2 * (BM + BN) * BK + 2 * BM * 4;

// Dense: tiles ordered in bands of 8 row-tiles so consecutive workgroups share
// weight tiles.
template <int GRAN>
__global__ __launch_bounds__(kThreads, 2) void k_gemm(const uint8_t* __restrict__ A,
                                                   const uint8_t* __restrict__ W,
                                                   const float* __restrict__ sA,
                                                   const float* __restrict__ sW,
                                                   uint16_t* __restrict__ Y, int64_t M,
                                                   int64_t N, int64_t K) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    const int64_t tm_count = (M + BM - 1) / BM, tn_count = N / BN;
    const int64_t bid = blockIdx.x;
    constexpr int64_t GROUP = 8;
    const int64_t band = bid / (GROUP * tn_count);
    const int64_t first_m = band * GROUP;
    const int64_t band_m = (tm_count - first_m) < GROUP ? (tm_count - first_m) : GROUP;
    const int64_t in_band = bid - band * GROUP * tn_count;
    const int64_t tm = first_m + in_band % band_m;
    const int64_t tn = in_band / band_m;

    const int64_t KB = K / BK;
    const int64_t row0 = tm * BM, n0 = tn * BN;
    Tile t;
    t.A = A + row0 * K;
    t.W = W + n0 * K;
    t.Y = Y + row0 * N + n0;
    t.rows = (int)((M - row0) < BM ? (M - row0) : BM);
    if constexpr (GRAN == GRAN_BLOCK) {
        t.sA = sA + row0 * KB;
        t.sW = sW + tn * KB;
    } else {
        t.sA = sA + row0;
        t.sW = sW + n0;
    }
    gemm_tile<GRAN>(t, K, N, lds);
}

// Grouped (MoE): blockIdx.x enumerates row tiles of all experts in expert
// order (an upper bound of them; surplus workgroups exit), blockIdx.y the
// column tile.  Wave 0 locates the expert of its row tile with a prefix sum of
// ceil(rows_e / 128) over the experts.
__global__ __launch_bounds__(kThreads, 2) void k_grouped_gemm(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ W,
    const float* __restrict__ sA, const float* __restrict__ sW,
    const int32_t* __restrict__ offsets, uint16_t* __restrict__ Y, int64_t T, int64_t E,
    int64_t N, int64_t K) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    __shared__ int64_t s_task[3];  // expert (-1: none), first row, rows
    const int64_t tile = blockIdx.x;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int64_t base = 0, found = -1, frow = 0, nrows = 0;
        for (int64_t e0 = 0; e0 < E && found < 0; e0 += 64) {
            const int64_t e = e0 + lane;
            int64_t lo = 0, hi = 0;
            if (e < E) {
                lo = offsets[e];
                hi = offsets[e + 1];
                lo = lo < 0 ? 0 : (lo > T ? T : lo);
                hi = hi < lo ? lo : (hi > T ? T : hi);
            }
            const int64_t cnt = (hi - lo + BM - 1) / BM;
            int64_t incl = cnt;  // inclusive prefix over the 64 lanes
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int64_t up = __shfl_up(incl, o);
                if (lane >= o) incl += up;
            }
            const int64_t excl = incl - cnt;
            const bool mine = cnt > 0 && tile >= base + excl && tile < base + incl;
            const unsigned long long bal = __ballot(mine);
            if (bal) {
                const int src = __ffsll((long long)bal) - 1;
                const int64_t lt = tile - base - excl;  // meaningful in lane src
                const int64_t r0 = lo + lt * BM;
                const int64_t rn = (hi - r0) < BM ? (hi - r0) : BM;
                found = __shfl(e, src);
                frow = __shfl(r0, src);
                nrows = __shfl(rn, src);
            }
            base += __shfl(incl, 63);
        }
        if (lane == 0) {
            s_task[0] = found;
            s_task[1] = frow;
            s_task[2] = nrows;
        }
    }
    __syncthreads();
    const int64_t e = s_task[0];
    if (e < 0) return;  // whole workgroup leaves together
    const int64_t row0 = s_task[1];
    const int64_t KB = K / BK, tn = blockIdx.y, n0 = tn * BN;
    Tile t;
    t.A = A + row0 * K;
    t.sA = sA + row0 * KB;
    t.W = W + (e * N + n0) * K;
    t.sW = sW + (e * (N / BN) + tn) * KB;
    t.Y = Y + row0 * N + n0;
    t.rows = (int)s_task[2];
    gemm_tile<GRAN_BLOCK>(t, K, N, lds);
}

}  // namespace

hipError_t launch_gemm(const void* a, const void* w, const float* a_s, const float* w_s,
                       void* y, int64_t M, int64_t N, int64_t K, int gran, hipStream_t st) {
    const int64_t tiles = ((M + BM - 1) / BM) * (N / BN);
    if (tiles == 0) return hipSuccess;
    const auto* A = static_cast<const uint8_t*>(a);
    const auto* Wp = static_cast<const uint8_t*>(w);
    auto* Yp = static_cast<uint16_t*>(y);
    if (gran == GRAN_BLOCK)
        hipLaunchKernelGGL(k_gemm<GRAN_BLOCK>, dim3((unsigned)tiles), dim3(kThreads), 0, st, A,
                           Wp, a_s, w_s, Yp, M, N, K);
    else
        hipLaunchKernelGGL(k_gemm<GRAN_ROW>, dim3((unsigned)tiles), dim3(kThreads), 0, st, A,
                           Wp, a_s, w_s, Yp, M, N, K);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(const void* a, const void* w, const float* a_s, const float* w_s,
                               const int32_t* offsets, void* y, int64_t T, int64_t E,
                               int64_t N, int64_t K, hipStream_t st) {
    const int64_t mt = (T + BM - 1) / BM + E;  // >= sum_e ceil(rows_e / 128)
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(k_grouped_gemm, dim3((unsigned)mt, (unsigned)(N / BN)), dim3(kThreads), 0,
                       st, static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(w), a_s,
                       w_s, offsets, static_cast<uint16_t*>(y), T, E, N, K);
    return hipGetLastError();
}

}  // namespace fp8k
