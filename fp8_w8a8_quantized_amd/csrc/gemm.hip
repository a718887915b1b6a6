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
//     row are XOR-swizzled by the row index (swz) so the MFMA operand reads
//     of 16 consecutive rows hit distinct banks.
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

// Byte offset of 16-byte chunk `c` of tile row `r` (128 bytes per row).  The
// gfx950 LDS serves a 16-byte-per-lane read 16 lanes (256 bytes, 64 banks) at
// a time; the MFMA operand reads put 16 consecutive rows, same chunk, in one
// such group.  Row parity already selects the bank half (rows are 128 bytes),
// so XOR-ing the chunk with (r >> 1) & 7 spreads the 8 rows of each parity
// over 8 distinct 16-byte bank groups: conflict-free.
__device__ __forceinline__ int swz_pos(int r, int c) { return c ^ ((r >> 1) & 7); }
__device__ __forceinline__ int swz(int r, int c) { return r * BK + (swz_pos(r, c) << 4); }

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

// ---------------------------------------------------------------------------
// Large-M kernel: workgroup tile 256 x 256, K step 128, 512 threads as 4 x 2
// waves, each wave 64 rows x 128 columns of Y (its 128 columns are one weight
// scale block).
//   * The MFMA computes the transposed tile: operand A is a 16-row W
//     fragment (16 output columns), operand B a 16-row X fragment (16 output
//     rows), so element e of lane l is Y[row 16i + l % 16][col 16j + 4 (l/16)
//     + e].  A lane then holds 4 consecutive columns of one row: the block
//     promotion is acc += P * s with one activation scale per lane and row
//     tile, and the epilogue stores 8 bytes of bf16 straight to HBM.
//   * A and W tiles move HBM -> LDS with direct-to-LDS 16-byte loads
//     (global_load_lds_dwordx4: the 16 bytes of lane i land at the wave's LDS
//     base + 16 i), so no registers stage them; the lane -> global address
//     map applies the chunk swizzle.  Two LDS stages: the next K block streams
//     into one while the current one is multiplied.
//   * Per K block a wave keeps its 4 X fragments in registers and streams the
//     8 W fragments (double-buffered); the FMAs that promote one MFMA's result
//     are issued after the next MFMA, so they never wait on the matrix core.
//   * Tiles are assigned so that each XCD (blockIdx % 8) owns a contiguous
//     range of tiles, ordered in bands of 4 row-tiles, so the workgroups
//     resident on one XCD share A rows and W columns in its L2.
// ---------------------------------------------------------------------------
constexpr int BM2 = 256, BN2 = 256, kThreads2 = 512;
constexpr int kStage2 = (BM2 + BN2) * BK;             // 64 KiB per stage
constexpr int kLds2 = 2 * kStage2 + 2 * BM2 * 4;       // two stages + two sA slices
static_assert(kLds2 <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

__device__ __forceinline__ void g2l_16(const void* g, uint8_t* l) {
    __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)l, 16, 0, 0);
}
__device__ __forceinline__ void g2l_4(const void* g, uint8_t* l) {
    __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)l, 4, 0, 0);
}

// Stage K block kb of the A and W tiles (and the A scales) into LDS stage st.
template <int GRAN>
__device__ __forceinline__ void stage_big(uint8_t* lds, int st, const uint8_t* A, const uint8_t* W,
                                          const float* sA, int rows, int64_t K, int64_t KB,
                                          int64_t kb, int wave, int lane) {
    uint8_t* la = lds + st * kStage2;
    uint8_t* lb = la + BM2 * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int pbase = (i * 8 + wave) * 64;  // LDS chunk of lane 0 (8 rows per wave load)
        const int p = pbase + lane;
        const int r = p >> 3;
        const int c = swz_pos(r, p & 7);  // the global chunk whose LDS slot is p
        const int ra = r < rows ? r : rows - 1;
        g2l_16(A + ra * K + kb * BK + c * 16, la + pbase * 16);
        g2l_16(W + r * K + kb * BK + c * 16, lb + pbase * 16);
    }
    if constexpr (GRAN == GRAN_BLOCK) {
        if (wave < 4) {
            const int r = wave * 64 + lane;
            const int rr = r < rows ? r : rows - 1;
            g2l_4(sA + rr * KB + kb, lds + 2 * kStage2 + st * BM2 * 4 + wave * 256);
        }
    }
}

__device__ __forceinline__ v8i frag(const uint8_t* base, int r, int lk) {
    const v4i lo = *reinterpret_cast<const v4i*>(base + swz(r, 2 * lk));
    const v4i hi = *reinterpret_cast<const v4i*>(base + swz(r, 2 * lk + 1));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int GRAN>
__global__ __launch_bounds__(kThreads2) void k_gemm_big(const uint8_t* __restrict__ A,
                                                        const uint8_t* __restrict__ W,
                                                        const float* __restrict__ sA,
                                                        const float* __restrict__ sW,
                                                        uint16_t* __restrict__ Y, int64_t M,
                                                        int64_t N, int64_t K) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLds2];
    const int64_t tm_count = (M + BM2 - 1) / BM2, tn_count = N / BN2;
    const int64_t T = tm_count * tn_count;
    // XCD-contiguous tile order: XCD x = blockIdx % 8 gets logical tiles
    // [x * q + min(x, r), ...) where T = 8 q + r.
    const int64_t bid = blockIdx.x, xcd = bid & 7, idx = bid >> 3;
    const int64_t q = T >> 3, rem = T & 7;
    const int64_t logical = xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
    constexpr int64_t GROUP = 4;
    const int64_t band = logical / (GROUP * tn_count);
    const int64_t first_m = band * GROUP;
    const int64_t band_m = (tm_count - first_m) < GROUP ? (tm_count - first_m) : GROUP;
    const int64_t in_band = logical - band * GROUP * tn_count;
    const int64_t tm = first_m + in_band % band_m, tn = in_band / band_m;

    const int64_t KB = K / BK;
    const int64_t row0 = tm * BM2, n0 = tn * BN2;
    const int rows = (int)((M - row0) < BM2 ? (M - row0) : BM2);
    const uint8_t* At = A + row0 * K;
    const uint8_t* Wt = W + n0 * K;
    const float* sAt = GRAN == GRAN_BLOCK ? sA + row0 * KB : sA + row0;
    const float* sWt = GRAN == GRAN_BLOCK ? sW + (n0 / BK) * KB : sW + n0;

    const int tid = threadIdx.x, lane = tid & 63;
    // wave index made provably wave-uniform, so per-wave scale reads become
    // scalar loads (a vector load would make the loop's vmcnt waits also wait
    // for the next stage's direct-to-LDS loads)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 3, wn = wave >> 2;
    const int lr = lane & 15, lk = lane >> 4;

    v4f acc[4][8];  // [row tile i][column tile j]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    stage_big<GRAN>(lds, 0, At, Wt, sAt, rows, K, KB, 0, wave, lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's LDS-bound loads landed
    __syncthreads();

    for (int64_t kb = 0; kb < KB; ++kb) {
        const int cur = (int)(kb & 1);
        if (kb + 1 < KB) stage_big<GRAN>(lds, cur ^ 1, At, Wt, sAt, rows, K, KB, kb + 1, wave, lane);

        const uint8_t* la = lds + cur * kStage2;
        const uint8_t* lb = la + BM2 * BK;
        v8i x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = frag(la, wm * 64 + i * 16 + lr, lk);
        if constexpr (GRAN == GRAN_BLOCK) {
            const float sw = sWt[wn * KB + kb];
            const float* lsa = reinterpret_cast<const float*>(lds + 2 * kStage2 + cur * BM2 * 4);
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] = lsa[wm * 64 + i * 16 + lr] * sw;
            const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
            v8i wcur = frag(lb, wn * 128 + lr, lk);
            v4f prev;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v8i wnext = wcur;
                if (j < 7) wnext = frag(lb, wn * 128 + (j + 1) * 16 + lr, lk);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const v4f p = mfma_f8(wcur, x[i], zero);
                    // promote the previous MFMA's result (tile (i-1, j) or (3, j-1))
                    if (i > 0 || j > 0) {
                        const int pi = i > 0 ? i - 1 : 3, pj = i > 0 ? j : j - 1;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[pi][pj][e] = __builtin_fmaf(prev[e], sc[pi], acc[pi][pj][e]);
                    }
                    prev = p;
                }
                wcur = wnext;
                // keep each column tile's MFMAs in their step: hoisting them
                // further only raises register pressure past 256 VGPRs
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[3][7][e] = __builtin_fmaf(prev[e], sc[3], acc[3][7][e]);
        } else {
            v8i wcur = frag(lb, wn * 128 + lr, lk);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v8i wnext = wcur;
                if (j < 7) wnext = frag(lb, wn * 128 + (j + 1) * 16 + lr, lk);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i][j] = mfma_f8(wcur, x[i], acc[i][j]);
                wcur = wnext;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // next stage's loads landed
        __syncthreads();
    }

    // epilogue: lane holds Y[row][col .. col+3] per tile -> one 8-byte bf16 store
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + lr;
        if (r >= rows) continue;
        float sa = 1.0f;
        if constexpr (GRAN == GRAN_ROW) sa = sAt[r];
        uint16_t* yrow = Y + (row0 + r) * N + n0 + wn * 128 + 4 * lk;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v4f v = acc[i][j];
            if constexpr (GRAN == GRAN_ROW) {
                const v4f s4 = *reinterpret_cast<const v4f*>(sWt + wn * 128 + j * 16 + 4 * lk);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = v[e] * (sa * s4[e]);
            }
            uint2 o;
            o.x = bf16_rne_bits(v[0]) | (bf16_rne_bits(v[1]) << 16);
            o.y = bf16_rne_bits(v[2]) | (bf16_rne_bits(v[3]) << 16);
            *reinterpret_cast<uint2*>(yrow + j * 16) = o;
        }
    }
}

}  // namespace

hipError_t launch_gemm(const void* a, const void* w, const float* a_s, const float* w_s,
                       void* y, int64_t M, int64_t N, int64_t K, int gran, hipStream_t st) {
    const int64_t tiles = ((M + BM - 1) / BM) * (N / BN);
    if (tiles == 0) return hipSuccess;
    const auto* A = static_cast<const uint8_t*>(a);
    const auto* Wp = static_cast<const uint8_t*>(w);
    auto* Yp = static_cast<uint16_t*>(y);
    if (M >= 1024 && N % BN2 == 0) {
        const int64_t tiles2 = ((M + BM2 - 1) / BM2) * (N / BN2);
        if (gran == GRAN_BLOCK)
            hipLaunchKernelGGL(k_gemm_big<GRAN_BLOCK>, dim3((unsigned)tiles2), dim3(kThreads2), 0,
                               st, A, Wp, a_s, w_s, Yp, M, N, K);
        else
            hipLaunchKernelGGL(k_gemm_big<GRAN_ROW>, dim3((unsigned)tiles2), dim3(kThreads2), 0,
                               st, A, Wp, a_s, w_s, Yp, M, N, K);
        return hipGetLastError();
    }
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
