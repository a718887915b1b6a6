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
// Two kernels share one tile recipe (CDNA4):
//   * v_mfma_f32_16x16x128_f8f6f4 with both operands E4M3: one instruction is a
//     16 x 16 tile over a whole 128-wide K block, so BLOCK mode gets P_kb from
//     one MFMA with a zero accumulator and promotes it with one fp32 FMA per
//     output element, acc += P_kb * (sA * sW); ROW mode accumulates in the
//     MFMA and scales once in the epilogue.
//   * MFMA operand layout (16x16x128, 8-bit): lane l supplies row l % 16 of
//     its operand and 32 consecutive K bytes starting at 32 * (l / 16); both
//     operands use the same K assignment, so every product pairs matching k.
//     The result holds D[4 * (l / 16) + i][l % 16] in element i of lane l.
//     The kernels put the W fragment in operand A and the X fragment in
//     operand B (they compute the transposed tile), so a lane holds four
//     consecutive output columns of one row.
//   * Operand tiles are staged in LDS by direct-to-LDS 16-byte loads, with
//     16-byte chunks of each 128-byte tile row XOR-swizzled (swz) so the
//     operand reads are free of bank conflicts.
//   k_gemm_pp   (M >= 1024 or >= 192 tiles; block, row or dense E8M0
//     scales; the MoE grouped GEMM when experts average >= 192 rows):
//     persistent, 256 x 256 tile, two LDS stages, 8 waves in two groups one
//     phase apart (one group reads fragments while the other multiplies).
//   k_gemm_big  (batched E8M0, N % 256 == 128, N >= 2^22): the same tile and
//     stages, all 8 waves in step.
//   k_gemm_pipe / k_gemm_sk (small M, sparser MoE routing): persistent,
//     128 x 128 tile, 8 waves, a ring of four LDS stages with three in
//     flight; k_gemm_sk splits the K steps of all tiles evenly (stream-K).
//   k_gemm_dk (small M above 128 rows with >= 8 K steps per workgroup):
//     stream-K on 256 x 128 tiles, so each weight block is read once per
//     256 rows; three LDS stages, scales of 4 K blocks loaded together.
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "launch.hpp"

namespace fp8k {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BK = 128;  // K step: one scale block
// s_waitcnt immediate for vmcnt(n), expcnt and lgkmcnt left unconstrained (gfx9),
// and for lgkmcnt(0) with the others unconstrained
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kLgkm0 = 0xC07F;
constexpr int GRAN_BLOCK = 0, GRAN_ROW = 1, GRAN_MX = 2;  // MX: E8M0 block scales

__device__ __forceinline__ v4f mfma_f8(const v8i& a, const v8i& b, const v4f& c) {
    // cbsz = blgp = 0: both operands E4M3; scale operands 0 -> unscaled form
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Byte offset of 16-byte chunk `c` of tile row `r` (128 bytes per row).  The
// gfx950 LDS serves a 16-byte-per-lane read in four cycles of 16 lanes, 256
// bytes over 64 banks each: lanes {0-3, 12-15, 20-27}, {4-11, 16-19, 28-31}
// and the same sets + 32 (measured with a two-lane conflict probe).  An MFMA
// operand read puts row base + (l & 15), chunk 2 (l >> 4) + h in lane l; the
// row's parity picks the bank half, and XOR-ing the chunk with
// (r & 4) | ((r >> 1) & 1) gives the 16 lanes of every cycle 16 distinct
// 16-byte bank slots: conflict-free.
__device__ __forceinline__ int swz_pos(int r, int c) { return c ^ ((r & 4) | ((r >> 1) & 1)); }
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
//   * A and W tiles move HBM -> LDS with direct-to-LDS 16-byte buffer loads
//     (buffer_load_dwordx4 ... lds: the 16 bytes of lane i land at the wave's
//     LDS base + 16 i), so no registers stage them; the lane -> offset map
//     applies the chunk swizzle.  Two LDS stages: the next K block streams
//     into one while the current one is multiplied.
//   * Per K block a wave keeps its 4 X fragments in registers and streams the
//     8 W fragments (double-buffered); the FMAs that promote one MFMA's result
//     are issued after the next MFMA, so they never wait on the matrix core.
//   * Persistent: one workgroup per CU walks its tiles; each XCD
//     (blockIdx % 8) owns a contiguous range of tiles, ordered in bands of 4
//     row tiles, so the workgroups resident on one XCD share A rows and W
//     columns in its L2.
// ---------------------------------------------------------------------------
constexpr int BM2 = 256, BN2 = 256, kThreads2 = 512;
constexpr int kStage2 = (BM2 + BN2) * BK;             // 64 KiB per stage
constexpr int kSw2 = 2 * kStage2 + 2 * BM2 * 4;        // after two stages + two sA slices
constexpr int kLds2 = kSw2 + 2 * 256;                  // + two 256-byte sW slices
static_assert(kLds2 <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

__device__ __forceinline__ void g2l_16(const void* g, uint8_t* l) {
    __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)l, 16, 0, 0);
}
__device__ __forceinline__ void g2l_4(const void* g, uint8_t* l) {
    __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)l, 4, 0, 0);
}

// Buffer resource over `bytes` bytes at p (gfx9 raw buffer: stride 0, 32-bit
// data format word).  Loads through it take 32-bit offsets.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

// Direct-to-LDS load through a buffer resource: lane i's `size` bytes from
// byte voff + soff land at l + size * i.  Unlike the global form, the buffer
// form is not a FLAT instruction, so the compiler keeps counted lgkmcnt waits
// for the LDS reads that run while it is in flight.
__device__ __forceinline__ void b2l(__amdgpu_buffer_rsrc_t r, uint8_t* l, int size, int voff,
                                    int soff) {
    if (size == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)l, 16, voff, soff, 0, 0);
    else if (size == 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)l, 4, voff, soff, 0, 0);
    else  // one byte, written zero-extended as the lane's 32-bit word
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)l, 1, voff, soff, 0, 0);
}

// Shape of a large-M GEMM: B batches of A [M, B, K] x W [B, N, K] -> Y [M, B,
// N]; batch b of A is every B-th K-row (the token-major layout of the page's
// batched MX GEMM).  B = 1 is the dense GEMM (A [M, K], Y [M, N]).
struct BigGeom {
    int64_t M, N, K;
    int B;
};

// Per-tile load sources of the large-M kernel: buffer resources over the
// tile's A rows, W rows and scales, and each lane's loop-invariant offsets.
struct BigSrc {
    __amdgpu_buffer_rsrc_t a, w, sa, sw;
    int offa[4], offw[4];  // byte offsets of this lane's 16-byte chunks at kb = 0
    int offsa, offsw;      // byte offsets of this lane's scale at kb = 0
};

// Tile coordinates of logical tile `logical`: batch-major; inside a batch,
// bands of 4 row tiles, column-major inside a band, so consecutive logical
// tiles share A rows and W columns.  The last column tile may hold 128 valid
// columns (N % 256 == 128).
struct BigTile {
    int b, tm, tn, rows, cols;
    int64_t row0;  // first row of A and Y (per batch)
    int e;         // weight batch: the batch b, or the expert of a grouped tile
};

__device__ __forceinline__ BigTile big_tile(int logical, int tm_count, int tn_count,
                                            const BigGeom& G) {
    constexpr int GROUP = 4;
    BigTile t;
    const int per_batch = tm_count * tn_count;
    t.b = logical / per_batch;
    logical -= t.b * per_batch;
    const int band = logical / (GROUP * tn_count);
    const int first_m = band * GROUP;
    const int band_m = (tm_count - first_m) < GROUP ? (tm_count - first_m) : GROUP;
    const int in_band = logical - band * GROUP * tn_count;
    t.tm = first_m + in_band % band_m;
    t.tn = in_band / band_m;
    const int64_t left = G.M - (int64_t)t.tm * BM2, cleft = G.N - (int64_t)t.tn * BN2;
    t.rows = left < BM2 ? (int)left : BM2;
    t.cols = cleft < BN2 ? (int)cleft : BN2;
    t.row0 = 0;  // read only for grouped tiles
    t.e = 0;
    return t;
}

// Grouped (MoE) tiles: expert by expert, then column tile by column tile with
// the expert's row tiles adjacent (they share the W tile).  pre[e] (LDS) is
// the prefix over experts of ceil(rows_e / 256) * tn_count; expert e's rows
// are [rlo[e], rhi[e]) of A and Y.
struct BigGroups {
    const int32_t* pre;
    const int32_t* rlo;
    const int32_t* rhi;
    int E;
};

__device__ __forceinline__ BigTile big_tile_grouped(int logical, int tn_count, const BigGeom& G,
                                                    const BigGroups& g) {
    int lo = 0, hi = g.E - 1;  // last expert whose prefix start <= logical
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (g.pre[mid] <= logical) lo = mid; else hi = mid - 1;
    }
    BigTile t;
    const int r_lo = g.rlo[lo], r_hi = g.rhi[lo];
    const int mt = (r_hi - r_lo + BM2 - 1) / BM2;
    const int lt = logical - g.pre[lo];
    t.b = 0;
    t.e = lo;
    t.tn = lt / mt;
    t.tm = lt - t.tn * mt;
    t.row0 = (int64_t)r_lo + (int64_t)t.tm * BM2;
    const int64_t left = r_hi - t.row0, cleft = G.N - (int64_t)t.tn * BN2;
    t.rows = left < BM2 ? (int)left : BM2;
    t.cols = cleft < BN2 ? (int)cleft : BN2;
    return t;
}

// Load sources of tile t.  Rows past M (and columns past N) read the last
// valid row (column): their results are never stored.
template <int GRAN, bool GROUPED>
__device__ __forceinline__ BigSrc big_tile_src(const BigTile& t, const uint8_t* A, const uint8_t* W,
                                               const void* sA, const void* sW, const BigGeom& G,
                                               int wave, int lane) {
    const int K = (int)G.K, KB = K / BK, B = G.B;
    // grouped tiles carry their first row and expert; dense and batched ones
    // are at row tm * 256 of batch b
    const int64_t row0 = GROUPED ? t.row0 : (int64_t)t.tm * BM2, n0 = (int64_t)t.tn * BN2;
    const int64_t wb = GROUPED ? t.e : t.b;
    const int lda = B * K;  // bytes between consecutive rows of one batch of A
    BigSrc S;
    S.a = buffer_rsrc(A + (row0 * B + t.b) * (int64_t)K, (t.rows - 1) * lda + K);
    S.w = buffer_rsrc(W + (wb * G.N + n0) * K, t.cols * K);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = (i * 8 + wave) * 64 + lane;  // LDS chunk this lane fills
        const int r = p >> 3;
        const int c = swz_pos(r, p & 7);           // the tile chunk whose LDS slot is p
        const int ra = r < t.rows ? r : t.rows - 1;
        const int rw = r < t.cols ? r : t.cols - 1;
        S.offa[i] = ra * lda + c * 16;
        S.offw[i] = rw * K + c * 16;
    }
    const int r = (wave & 3) * 64 + lane;
    const int rr = r < t.rows ? r : t.rows - 1;
    const int nb = t.cols / BK;                              // weight blocks in the tile
    const int wbl = (lane & 1) < nb ? (lane & 1) : nb - 1;  // lane l: weight block l & 1
    if constexpr (GRAN == GRAN_BLOCK) {  // fp32 scales (B == 1)
        const float* sa = static_cast<const float*>(sA) + row0 * KB;
        const float* sw = static_cast<const float*>(sW) + (wb * (G.N / BK) + n0 / BK) * KB;
        S.sa = buffer_rsrc(sa, t.rows * KB * 4);
        S.sw = buffer_rsrc(sw, nb * KB * 4);
        S.offsa = rr * KB * 4;
        S.offsw = wbl * KB * 4;
    } else if constexpr (GRAN == GRAN_MX) {  // E8M0 bytes [M, B, KB] and [B, N/128, KB]
        const uint8_t* sa = static_cast<const uint8_t*>(sA) + (row0 * B + t.b) * KB;
        const uint8_t* sw =
            static_cast<const uint8_t*>(sW) + (wb * (G.N / BK) + n0 / BK) * KB;
        S.sa = buffer_rsrc(sa, (t.rows - 1) * B * KB + KB);
        S.sw = buffer_rsrc(sw, nb * KB);
        S.offsa = rr * B * KB;
        S.offsw = wbl * KB;
    } else {
        S.sa = S.sw = S.a;
        S.offsa = S.offsw = 0;
    }
    return S;
}

// Stage K block kb of the A and W tiles (and, for block scales, the A and W
// scales of kb) into LDS stage st.  Scales land one 32-bit word per row (an
// E8M0 byte zero-extended) and one word per weight block.
template <int GRAN>
__device__ __forceinline__ void stage_big(uint8_t* lds, int st, const BigSrc& S, int kb, int wave) {
    uint8_t* la = lds + st * kStage2;
    uint8_t* lb = la + BM2 * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int pbase = (i * 8 + wave) * 64;  // LDS chunk of lane 0 (8 rows per wave load)
        b2l(S.a, la + pbase * 16, 16, S.offa[i], kb * BK);
        b2l(S.w, lb + pbase * 16, 16, S.offw[i], kb * BK);
    }
    if constexpr (GRAN == GRAN_BLOCK || GRAN == GRAN_MX) {
        constexpr int size = GRAN == GRAN_BLOCK ? 4 : 1;
        if (wave < 4)
            b2l(S.sa, lds + 2 * kStage2 + st * BM2 * 4 + wave * 256, size, S.offsa, kb * size);
        else if (wave == 4)
            b2l(S.sw, lds + kSw2 + st * 256, size, S.offsw, kb * size);
    }
}

// The MFMA fragment of tile row r for lane group lk: K bytes 32 lk .. +31, the
// two 16-byte chunks 2 lk and 2 lk + 1 of the (swizzled) row.
__device__ __forceinline__ v8i frag(const uint8_t* base, int r, int lk) {
    const v4i lo = *reinterpret_cast<const v4i*>(base + swz(r, 2 * lk));
    const v4i hi = *reinterpret_cast<const v4i*>(base + swz(r, 2 * lk + 1));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A K block runs in two parts.  Column steps 6 and 7 of each K block are
// deferred past the barrier that ends the block: their eight MFMAs read only
// registers (those steps' W fragments and the block's X fragments).  The
// head runs them X-fragment by X-fragment, so each X register is free after
// its second MFMA and the next block's fragment is read into it right away:
// the matrix core stays busy while the next block's X fragments arrive from
// LDS.  The body then runs column steps 0..5.  Promotions (BLOCK) run one
// MFMA behind their product throughout, so the last product of a part is
// promoted at the start of the next one.
struct BigCarry {
    v8i w6, w7;  // W fragments of column steps 6 and 7 of the previous K block
    float sc[4]; // the previous block's promotion scales (BLOCK)
    v4f p;       // last product not yet promoted (BLOCK)
    float psc;   // its scale
    int sa[4];   // the previous block's E8M0 row scales (MX)
    int sw;      // and its E8M0 weight-block scale
};

// The scales of the current K block: BLOCK uses sc (sA * sW per X
// fragment), MX the E8M0 words sa (per X fragment) and sw (the wave's weight
// block).
struct BigScales {
    float sc[4];
    int sa[4];
    int sw;
};

// sched_group_barrier masks
constexpr int kSgValu = 0x002, kSgMfma = 0x008, kSgVmem = 0x010, kSgDsRead = 0x100;

__device__ __forceinline__ void promote(v4f& acc, const v4f& p, float s) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(p[e], s, acc[e]);
}

// MX-scaled MFMA: W fragment (operand A) scaled by 2^(sw - 127), X fragment
// (operand B) by 2^(sa - 127); every lane of a row or column gives the same
// byte, so the scale covers the whole 128-wide K block.
__device__ __forceinline__ v4f mfma_mx(const v8i& w, const v8i& x, const v4f& c, int sw, int sa) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, c, 0, 0, 0, sw, 0, sa);
}

// Head of K block `cur`: the previous block's deferred steps 6 and 7, and
// this block's scales, first W fragment (returned in w0) and X fragments.
// BLOCK: c.p enters as the previous block's product of tile (3, 5) and leaves
// as its product of tile (3, 7).
template <int GRAN>
__device__ __forceinline__ void big_head(const uint8_t* lds, int cur, v4f (&acc)[4][8],
                                         v8i (&x)[4], v8i& w0, BigScales& bs, BigCarry& c,
                                         int wm, int wn, int lr, int lk) {
    const uint8_t* la = lds + cur * kStage2;
    const uint8_t* lb = la + BM2 * BK;
    if constexpr (GRAN == GRAN_BLOCK) {
        // All operands and scales come from LDS, so each wait is a counted
        // lgkmcnt on in-order LDS reads (a scalar load in flight would force
        // lgkmcnt(0) on every wait).
        const float* lsa = reinterpret_cast<const float*>(lds + 2 * kStage2 + cur * BM2 * 4);
        const float sw = reinterpret_cast<const float*>(lds + kSw2 + cur * 256)[wn];
        // scales and w0 first (the body's first MFMA needs w0), then per X
        // fragment its two deferred MFMAs, each followed by the promotion of
        // the product before it, then the read of the next block's fragment
        // into the freed registers; the fences keep exactly this order, so
        // the body's waits are counted (w0 and x0 landed, x1..x3 may not)
        float sa4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sa4[i] = lsa[wm * 64 + i * 16 + lr];
        w0 = frag(lb, wn * 128 + lr, lk);
        __builtin_amdgcn_sched_barrier(0);
        const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
        int pi = 3, pj = 5;  // tile of c.p
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 6; j < 8; ++j) {
                const v4f d = mfma_f8(j == 6 ? c.w6 : c.w7, x[i], zero);
                promote(acc[pi][pj], c.p, c.psc);
                c.p = d;
                c.psc = c.sc[i];
                pi = i;
                pj = j;
            }
            x[i] = frag(la, wm * 64 + i * 16 + lr, lk);
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgValu, 4, 0);
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgValu, 4, 0);
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) bs.sc[i] = sa4[i] * sw;
    } else {
        if constexpr (GRAN == GRAN_MX) {
            const int* lsa = reinterpret_cast<const int*>(lds + 2 * kStage2 + cur * BM2 * 4);
            bs.sw = reinterpret_cast<const int*>(lds + kSw2 + cur * 256)[wn];
#pragma unroll
            for (int i = 0; i < 4; ++i) bs.sa[i] = lsa[wm * 64 + i * 16 + lr];
        }
        w0 = frag(lb, wn * 128 + lr, lk);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (GRAN == GRAN_MX) {
                acc[i][6] = mfma_mx(c.w6, x[i], acc[i][6], c.sw, c.sa[i]);
                acc[i][7] = mfma_mx(c.w7, x[i], acc[i][7], c.sw, c.sa[i]);
            } else {
                acc[i][6] = mfma_f8(c.w6, x[i], acc[i][6]);
                acc[i][7] = mfma_f8(c.w7, x[i], acc[i][7]);
            }
            x[i] = frag(la, wm * 64 + i * 16 + lr, lk);
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Body of K block `cur`: column steps 0..5; steps 6 and 7's W fragments go to
// c.w6 and c.w7, this block's scales to the carry.  BLOCK: c.p enters as the
// previous block's product of tile (3, 7) and leaves as this block's product
// of tile (3, 5).
template <int GRAN>
__device__ __forceinline__ void big_body(const uint8_t* lds, int cur, v4f (&acc)[4][8],
                                         const v8i (&x)[4], v8i w0, const BigScales& bs,
                                         BigCarry& c, int wn, int lr, int lk) {
    const uint8_t* lb = lds + cur * kStage2 + BM2 * BK;
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    v8i wcur = w0;
    int pi = 3, pj = 7;  // tile of c.p (the previous block's last product)
#pragma unroll
    for (int j = 0; j < 6; ++j) {
        const v8i wnext = frag(lb, wn * 128 + (j + 1) * 16 + lr, lk);
        if (j == 5) c.w7 = frag(lb, wn * 128 + 7 * 16 + lr, lk);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (GRAN == GRAN_BLOCK) {
                const v4f p = mfma_f8(wcur, x[i], zero);
                promote(acc[pi][pj], c.p, c.psc);
                c.p = p;
                c.psc = bs.sc[i];
                pi = i;
                pj = j;
            } else if constexpr (GRAN == GRAN_MX) {
                acc[i][j] = mfma_mx(wcur, x[i], acc[i][j], bs.sw, bs.sa[i]);
            } else {
                acc[i][j] = mfma_f8(wcur, x[i], acc[i][j]);
            }
        }
        wcur = wnext;
        // per column step: MFMA, the next W fragment's LDS reads, then after
        // every further MFMA the 4 FMAs promoting the MFMA before it
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        if (j == 5)
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 4, 0);
        else
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if constexpr (GRAN == GRAN_BLOCK) __builtin_amdgcn_sched_group_barrier(kSgValu, 4, 0);
            if (t < 3) __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    c.w6 = wcur;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (GRAN == GRAN_BLOCK) c.sc[i] = bs.sc[i];
        if constexpr (GRAN == GRAN_MX) c.sa[i] = bs.sa[i];
    }
    if constexpr (GRAN == GRAN_MX) c.sw = bs.sw;
}

// The last block's deferred steps 6 and 7 (no next block to read).
template <int GRAN>
__device__ __forceinline__ void big_tail(v4f (&acc)[4][8], const v8i (&x)[4], BigCarry& c) {
    if constexpr (GRAN == GRAN_BLOCK) {
        const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
        promote(acc[3][5], c.p, c.psc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            promote(acc[i][6], mfma_f8(c.w6, x[i], zero), c.sc[i]);
            promote(acc[i][7], mfma_f8(c.w7, x[i], zero), c.sc[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (GRAN == GRAN_MX) {
                acc[i][6] = mfma_mx(c.w6, x[i], acc[i][6], c.sw, c.sa[i]);
                acc[i][7] = mfma_mx(c.w7, x[i], acc[i][7], c.sw, c.sa[i]);
            } else {
                acc[i][6] = mfma_f8(c.w6, x[i], acc[i][6]);
                acc[i][7] = mfma_f8(c.w7, x[i], acc[i][7]);
            }
        }
    }
}

// Store a wave's 64 x 128 block of tile t (bf16, 8 bytes per lane and column
// tile) and clear the accumulators for the next tile.  ROW applies the per-row
// and per-column fp32 scales here (B == 1).
template <int GRAN, bool GROUPED>
__device__ __forceinline__ void big_store(v4f (&acc)[4][8], const BigTile& t, uint16_t* Y,
                                          const void* sA, const void* sW, const BigGeom& G,
                                          int wm, int wn, int lr, int lk) {
    const int64_t row0 = GROUPED ? t.row0 : (int64_t)t.tm * BM2, n0 = (int64_t)t.tn * BN2;
    const int64_t ldy = (int64_t)G.B * G.N;
    if (wn * 128 < t.cols) {  // the wave's 128 columns exist
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 64 + i * 16 + lr;
            if (r < t.rows) {
                float sa = 1.0f;
                if constexpr (GRAN == GRAN_ROW) sa = static_cast<const float*>(sA)[row0 + r];
                uint16_t* yrow = Y + (row0 + r) * ldy + (int64_t)t.b * G.N + n0 + wn * 128 + 4 * lk;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    v4f v = acc[i][j];
                    if constexpr (GRAN == GRAN_ROW) {
                        const v4f s4 = *reinterpret_cast<const v4f*>(
                            static_cast<const float*>(sW) + n0 + wn * 128 + j * 16 + 4 * lk);
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = v[e] * (sa * s4[e]);
                    }
                    uint2 o;
                    o.x = bf16x2_rne(v[0], v[1]);
                    o.y = bf16x2_rne(v[2], v[3]);
                    *reinterpret_cast<uint2*>(yrow + j * 16) = o;
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
}

constexpr int kMaxExpertsBig = 1024;  // expert table size of the grouped form

// The expert tables of a grouped large-M launch, built by wave 0 into tab (LDS):
// pre[e] (e <= E) the prefix over experts of ceil(rows_e / 256) * tn_count,
// then rlo[e] and rhi[e], expert e's rows [offsets[e], offsets[e + 1])
// clamped to [0, M].  The caller synchronizes the workgroup before use.
__device__ __forceinline__ void big_groups(uint8_t* tab, const int32_t* offsets, int E, int64_t M,
                                           int tn_count) {
    int32_t* s_pre = reinterpret_cast<int32_t*>(tab);
    int32_t* s_rlo = s_pre + kMaxExpertsBig + 1;
    int32_t* s_rhi = s_rlo + kMaxExpertsBig;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int base = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            int cnt = 0;
            if (e < E) {
                int64_t lo = offsets[e], hi = offsets[e + 1];
                lo = lo < 0 ? 0 : (lo > M ? M : lo);
                hi = hi < lo ? lo : (hi > M ? M : hi);
                cnt = (int)((hi - lo + BM2 - 1) / BM2) * tn_count;
                s_rlo[e] = (int32_t)lo;
                s_rhi[e] = (int32_t)hi;
            }
            int incl = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int up = __shfl_up(incl, o);
                if (lane >= o) incl += up;
            }
            if (e < E) s_pre[e] = base + incl - cnt;
            base += __shfl(incl, 63);
        }
        if (lane == 0) s_pre[E] = base;
    }
}

// Persistent: workgroup b runs on XCD b % 8; the XCD's workgroups share a
// contiguous range of logical tiles and take them round-robin.  The steps
// (tile, K block) of one workgroup form one stream through the two LDS
// stages, so the first K block of the next tile loads while the last K block
// of the current one is multiplied and its output stored.
template <int GRAN, bool GROUPED>
__global__ __launch_bounds__(kThreads2) void k_gemm_big(const uint8_t* __restrict__ A,
                                                        const uint8_t* __restrict__ W,
                                                        const void* __restrict__ sA,
                                                        const void* __restrict__ sW,
                                                        uint16_t* __restrict__ Y, BigGeom G,
                                                        const int32_t* __restrict__ offsets,
                                                        int E) {
    // one LDS object for the stage ring and (grouped) the expert tables, so the
    // compiler keeps telling the direct-to-LDS stage writes from operand reads
    constexpr int kTab = GROUPED ? (3 * kMaxExpertsBig + 1) * 4 : 0;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLds2 + kTab];
    const int tm_count = (int)((G.M + BM2 - 1) / BM2), tn_count = (int)((G.N + BN2 - 1) / BN2);
    int T = G.B * tm_count * tn_count;
    BigGroups grp{};
    if constexpr (GROUPED) {
        // prefix over experts of their tile counts, and their row ranges (wave 0)
        big_groups(lds + kLds2, offsets, E, G.M, tn_count);
        __syncthreads();
        const int32_t* s_pre = reinterpret_cast<const int32_t*>(lds + kLds2);
        grp = BigGroups{s_pre, s_pre + kMaxExpertsBig + 1, s_pre + 2 * kMaxExpertsBig + 1, E};
        T = s_pre[E];
    }
    auto tile_of = [&](int logical) {
        if constexpr (GROUPED)
            return big_tile_grouped(logical, tn_count, G, grp);
        else
            return big_tile(logical, tm_count, tn_count, G);
    };
    const int KB = (int)(G.K / BK);
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int nwg = ((int)gridDim.x - xcd + 7) >> 3;  // workgroups on this XCD
    const int q = T >> 3, rem = T & 7;
    const int xbeg = xcd * q + (xcd < rem ? xcd : rem), tx = q + (xcd < rem ? 1 : 0);
    if (idx >= tx) return;
    const int nt = (tx - idx + nwg - 1) / nwg;  // tiles of this workgroup
    const int first = xbeg + idx;               // its k-th tile: first + k * nwg

    const int tid = threadIdx.x, lane = tid & 63;
    // wave index made provably wave-uniform, so per-wave LDS bases are scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 3, wn = wave >> 2;
    const int lr = lane & 15, lk = lane >> 4;

    v4f acc[4][8];  // [row tile i][column tile j]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // The wave's X fragments of the current K block, and what a block hands
    // to the next (zero operands at the start, so the first head's deferred
    // steps add exact zeros).
    v8i x[4];
    BigCarry c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        c.sc[i] = 0.0f;
        c.sa[i] = 127;
    }
    c.sw = 127;
    c.w6 = c.w7 = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    c.p = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    c.psc = 0.0f;

    int lt = 0, lkb = 0;  // load cursor: tile, K block
    BigSrc S = big_tile_src<GRAN, GROUPED>(tile_of(first), A, W, sA, sW, G, wave, lane);
    stage_big<GRAN>(lds, 0, S, 0, wave);
    // Materialize the output pointer now: a scalar load still in flight
    // during the loop would turn every LDS wait into lgkmcnt(0).
    asm volatile("" ::"s"(Y));

    int ct = 0, ckb = 0;  // compute cursor: tile, K block
    const int NS = nt * KB;
    for (int g = 0; g < NS; ++g) {
        const int cur = g & 1;
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's loads of stage g landed
        __syncthreads();                     // ... and everyone's; stage g - 1 is free
        if (g + 1 < NS) {
            if (++lkb == KB) {
                lkb = 0;
                ++lt;
                S = big_tile_src<GRAN, GROUPED>(tile_of(first + lt * nwg), A, W, sA, sW, G, wave,
                                                lane);
            }
            stage_big<GRAN>(lds, cur ^ 1, S, lkb, wave);
        }
        v8i w0;
        BigScales bs;
        big_head<GRAN>(lds, cur, acc, x, w0, bs, c, wm, wn, lr, lk);
        if (ckb == 0 && g > 0) {
            // the head finished the previous tile's last block: store it
            if constexpr (GRAN == GRAN_BLOCK) {
                promote(acc[3][7], c.p, c.psc);
                c.p = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            }
            big_store<GRAN, GROUPED>(acc, tile_of(first + (ct - 1) * nwg), Y, sA, sW, G, wm, wn,
                                     lr, lk);
        }
        big_body<GRAN>(lds, cur, acc, x, w0, bs, c, wn, lr, lk);
        if (++ckb == KB) {
            ckb = 0;
            ++ct;
        }
    }
    big_tail<GRAN>(acc, x, c);
    big_store<GRAN, GROUPED>(acc, tile_of(first + (ct - 1) * nwg), Y, sA, sW, G, wm, wn, lr, lk);
}

// ---------------------------------------------------------------------------
// Ping-pong large-M kernel (block scales, dense B = 1): the 256 x 256 tile,
// the two LDS stages and the direct-to-LDS loads of k_gemm_big, with the 8
// waves split into two groups of 4 (waves 0-3 and 4-7, one of each per SIMD)
// that run one phase apart.  A wave alternates a memory phase (read the K
// block's 4 X and 8 W fragments and its scales from LDS into registers) and
// a compute phase (32 MFMAs from registers, each product promoted by 4 fp32
// FMAs while the next MFMA runs).  Every phase ends at a workgroup barrier,
// so while one group of a SIMD multiplies, the other reads: the matrix core
// never waits on LDS, and the compute phase runs at the rate of an
// all-register MFMA loop.
//
// Stage s % 2 holds K block s from the barrier before group 0 reads it
// (phase 2s) until group 1 has read it (phase 2s + 1).  Group 0 issues its
// share of block s + 1 at the start of its memory phase of block s (phase
// 2s) and waits for it at the end of the following compute phase; group 1
// issues its share of block s + 2 at the start of its compute phase of block
// s (phase 2s + 2) and waits for it at the end of its next memory phase.
// Both shares land before the barrier that opens phase 2s + 4.
//
// The output of a tile is stored in the memory phase of the next tile's
// first block.  Lanes l and l + 16 swap packed columns (v_permlane16_swap),
// so each lane writes 8 consecutive bf16 (16 bytes) and a store covers 64
// contiguous bytes of each of 16 rows.
// ---------------------------------------------------------------------------

// Workgroup barrier without a memory fence: the waits that order LDS and
// global traffic around it are explicit.
__device__ __forceinline__ void pp_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Store a wave's 64 x 128 block (tile rows wm * 64 .., columns col0 ..)
// through Yr, a buffer resource over the tile's valid rows of Y [.., ldy]:
// rows past M fall outside it and the hardware drops their writes, so every
// wave issues exactly kPPStores store instructions.  Clears the accumulators.
constexpr int kPPStores = 16;
typedef unsigned v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void pp_store(v4f (&acc)[4][8], __amdgpu_buffer_rsrc_t Yr, int ldy,
                                         int col0, int wm, int lr, int lk) {
    const int cq = 16 * (lk & 1) + 8 * (lk >> 1);  // lane's column inside a 32-column pair
    // the lane's byte offset of row wm * 64 + lr, recomputed here: kept across
    // the whole loop, its four row offsets would take registers it lacks
    int off0 = ((wm * 64 + lr) * ldy + col0 + cq) * 2;
    asm volatile("" : "+v"(off0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int off = off0 + i * 16 * ldy * 2;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const v4f& a = acc[i][2 * p];
            const v4f& b = acc[i][2 * p + 1];
            // lane (lr, lk) holds columns 16 j + 4 lk .. + 3 of fragment j;
            // the swap of rows 1, 3 of the first operand with rows 0, 2 of
            // the second gives lane (lr, lk) the 8 columns starting at
            // 32 p + cq
            const auto s0 = __builtin_amdgcn_permlane16_swap(bf16x2_rne(a[0], a[1]),
                                                             bf16x2_rne(b[0], b[1]), false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(bf16x2_rne(a[2], a[3]),
                                                             bf16x2_rne(b[2], b[3]), false, false);
            const v4u o = {s0[0], s1[0], s0[1], s1[1]};
            __builtin_amdgcn_raw_buffer_store_b128(o, Yr, off + 64 * p, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
}

// Store tile k's block of this wave.
// Y is [M, B, N]: batch b's rows are B N apart.
__device__ __forceinline__ void pp_store_tile(v4f (&acc)[4][8], const BigTile& t, uint16_t* Y,
                                              int N, int B, int wn, int wm, int lr, int lk) {
    const int ldy = B * N;
    const __amdgpu_buffer_rsrc_t Yr =
        buffer_rsrc(Y + (t.row0 * B + t.b) * N, ((t.rows - 1) * ldy + N) * 2);
    pp_store(acc, Yr, ldy, t.tn * BN2 + wn * 128, wm, lr, lk);
}

// Everything a ping-pong wave needs besides its registers.
struct PPCtx {
    const uint8_t* A;
    const uint8_t* W;
    const uint8_t* sA;  // fp32 (block scales) or E8M0 bytes (MX), per row and K block
    const uint8_t* sW;  // per 128-row weight block and K block, same type
    uint16_t* Y;
    BigGeom G;
    int tm_count, tn_count, first, nwg, NS, KB, K;
    int lda;          // bytes between consecutive rows of one batch of A (B K)
    bool grouped;     // MoE: tiles over the expert tables in grp
    BigGroups grp;
    int wave, wm, wn, lr, lk;
    int off0;  // group 0: lane's byte offset of its first W chunk of a block
    int offA;  // group 1: the same for its first A chunk (rows lda apart)
    int offa;  // group 1: lane's byte offset of its sA scale at kb = 0
    int offw;  // group 1: lane's byte offset of its sW scale at kb = 0
};

// Tile k of this workgroup (its fields made provably wave-uniform, so the
// buffer resources built from them stay in scalar registers).
// row0 is the first row of A and Y, e the weight batch (the expert).
__device__ __forceinline__ BigTile pp_tile(const PPCtx& c, int k) {
    BigTile t = c.grouped ? big_tile_grouped(c.first + k * c.nwg, c.tn_count, c.G, c.grp)
                          : big_tile(c.first + k * c.nwg, c.tm_count, c.tn_count, c.G);
    if (!c.grouped) t.row0 = (int64_t)t.tm * BM2;
    t.tn = __builtin_amdgcn_readfirstlane(t.tn);
    t.rows = __builtin_amdgcn_readfirstlane(t.rows);
    t.e = __builtin_amdgcn_readfirstlane(c.grouped ? t.e : t.b);  // the weight batch
    t.b = __builtin_amdgcn_readfirstlane(t.b);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)t.row0);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)t.row0 >> 32));
    t.row0 = (int64_t)(((uint64_t)hi << 32) | lo);
    return t;
}

// Sources of the blocks one wave loads: group 0 the W tile (r0), group 1 the
// A tile (r0), its sA rows (r1) and sW blocks (r2).  Rows past M lie past the
// A and sA resources, so their loads return zeros (never stored).  SB: bytes
// per scale (4: fp32 block scales, 1: E8M0).
struct PPSrc {
    __amdgpu_buffer_rsrc_t r0, r1, r2;
};

template <int GRP, int SB>
__device__ __forceinline__ PPSrc pp_src(const PPCtx& c, int tile) {
    const BigTile t = pp_tile(c, tile);
    const int K = c.K, KB = c.KB;
    const int64_t row0 = t.row0, n0 = (int64_t)t.e * c.G.N + (int64_t)t.tn * BN2;
    PPSrc S;
    if (GRP == 0) {
        S.r0 = buffer_rsrc(c.W + n0 * K, BN2 * K);
        S.r1 = S.r2 = S.r0;
    } else {
        // batch b of A is every B-th K-row ([M, B, K]); its scales [M, B, KB]
        const int B = c.G.B;
        const int64_t arow = row0 * B + t.b;
        S.r0 = buffer_rsrc(c.A + arow * K, (t.rows - 1) * c.lda + K);
        S.r1 = buffer_rsrc(c.sA + arow * KB * SB, ((t.rows - 1) * B * KB + KB) * SB);
        S.r2 = buffer_rsrc(c.sW + (n0 / BK) * KB * SB, 2 * KB * SB);
    }
    return S;
}

// Cursor over the blocks a wave loads: block b, its tile and K block, and the
// sources of that tile.  Blocks past the last one reload the last block into
// their (free) stage, so the loads of a phase never depend on a branch.
template <int GRP, int SB>
struct PPCur {
    int b, t, kb;
    PPSrc S;
    __device__ __forceinline__ void start(const PPCtx& c, int b0) {
        b = b0;
        const int bc = b0 < c.NS ? b0 : c.NS - 1;
        t = bc / c.KB;
        kb = bc - t * c.KB;
        S = pp_src<GRP, SB>(c, t);
    }
    __device__ __forceinline__ void next(const PPCtx& c) {
        ++b;
        if (b < c.NS && ++kb == c.KB) {
            kb = 0;
            ++t;
            S = pp_src<GRP, SB>(c, t);
        }
    }
};

// Loads of one phase.  A stage holds the A slice (256 rows x 128 bytes) and
// the W slice (W half h = rows 128 h ..), each as 16-byte chunks p (tile row
// p / 8, swizzled 16-byte column swz_pos of p % 8), and the scale words.
// The wave with index q in its group covers chunks (i * 4 + q) * 64 + lane.
// Group 1, load n of 10: n < 8 the A chunks with i = n, n = 8 its 64 sA rows,
// n = 9 the two sW words (every wave of the group writes the same words); an
// E8M0 scale lands zero-extended in its 32-bit word.  Group 0, load n of 8:
// W half 1 of block cur (n < 4, i = n) or W half 0 of block nxt (i = n - 4).
template <int SB>
__device__ __forceinline__ void pp_load1(uint8_t* lds, const PPCtx& c, const PPCur<1, SB>& L,
                                         int o, int n) {
    const int q = c.wave & 3, st = L.b & 1;
    uint8_t* la = lds + st * kStage2;
    if (n < 8)
        b2l(L.S.r0, la + (n * 4 + q) * 64 * 16, 16, o + n * 32 * c.lda, L.kb * BK);
    else if (n == 8)
        b2l(L.S.r1, lds + 2 * kStage2 + st * BM2 * 4 + q * 256, SB, c.offa, L.kb * SB);
    else
        b2l(L.S.r2, lds + kSw2 + st * 256, SB, c.offw, L.kb * SB);
}

template <int SB>
__device__ __forceinline__ void pp_load0(uint8_t* lds, const PPCtx& c, const PPCur<0, SB>& cur,
                                         const PPCur<0, SB>& nxt, int o, int n) {
    const int q = c.wave & 3, h = n < 4 ? 1 : 0, i = n & 3;
    const PPCur<0, SB>& L = h ? cur : nxt;
    uint8_t* lb = lds + (L.b & 1) * kStage2 + BM2 * BK;
    b2l(L.S.r0, lb + (h * 1024 + (i * 4 + q) * 64) * 16, 16, o + (h * 128 + i * 32) * c.K,
        L.kb * BK);
}

// The scales of a wave's K block: BLOCK, sA * sW per X fragment (sc); MX,
// the E8M0 words of its X fragments' rows (sa) and of its weight block (sw).
struct PPScales {
    float sc[4];
    int sa[4];
    int sw;
};

// Memory phase of block s: the wave's X and W fragments and scales into
// registers.
template <int GRAN>
__device__ __forceinline__ void pp_read(const uint8_t* lds, const PPCtx& c, int s, v8i (&x)[4],
                                        v8i (&w)[8], PPScales& ps) {
    const int slot = s & 1;
    const uint8_t* la = lds + slot * kStage2;
    const uint8_t* lbw = la + BM2 * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = frag(la, c.wm * 64 + i * 16 + c.lr, c.lk);
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = frag(lbw, c.wn * 128 + j * 16 + c.lr, c.lk);
    if constexpr (GRAN == GRAN_BLOCK) {
        const float* lsa = reinterpret_cast<const float*>(lds + 2 * kStage2 + slot * BM2 * 4);
        const float sw = reinterpret_cast<const float*>(lds + kSw2 + slot * 256)[c.wn];
#pragma unroll
        for (int i = 0; i < 4; ++i) ps.sc[i] = lsa[c.wm * 64 + i * 16 + c.lr] * sw;
    } else if constexpr (GRAN == GRAN_MX) {
        const int* lsa = reinterpret_cast<const int*>(lds + 2 * kStage2 + slot * BM2 * 4);
        ps.sw = reinterpret_cast<const int*>(lds + kSw2 + slot * 256)[c.wn];
#pragma unroll
        for (int i = 0; i < 4; ++i) ps.sa[i] = lsa[c.wm * 64 + i * 16 + c.lr];
    }
}

// Row scales (GRAN_ROW): the tile's accumulators times sA[row] * sW[col],
// once, before the store (the MFMA accumulated the unscaled products).
__device__ __forceinline__ void pp_row_scale(v4f (&acc)[4][8], const PPCtx& c, const BigTile& t,
                                             int wn, int wm, int lr, int lk) {
    const float* sa = reinterpret_cast<const float*>(c.sA);
    const float* sw = reinterpret_cast<const float*>(c.sW) + (int64_t)t.tn * BN2 + wn * 128 + 4 * lk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + lr;
        const float a = sa[t.row0 + (r < t.rows ? r : t.rows - 1)];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const v4f b = *reinterpret_cast<const v4f*>(sw + j * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = acc[i][j][e] * (a * b[e]);
        }
    }
}

// The phase loop of group GRP (0: waves 0-3, 1: waves 4-7; group 1 enters
// one barrier later, so group 0 reads block s in global phase 2s and group 1
// in 2s + 1).  Group 0 reads only W half 0 and group 1 only W half 1, so
// the halves and the A slice of a stage free up at different phases, and
// every load of the loop is issued in a compute phase, spread over its
// MFMAs, at least one phase before it is read:
//   group 1, compute phase of block s (global 2s + 2): A slice and scales of
//     block s + 2; waits at the end of its next memory phase (2s + 3);
//   group 0, compute phase of block s (global 2s + 1): W half 1 of block
//     s + 1 and W half 0 of block s + 2; waits at the end of its next memory
//     phase (2s + 2).
// Each group has its own copy of the loop, so every wait is unconditional
// and the compute phase is one straight block.
template <int GRAN, int GRP>
__device__ __forceinline__ void pp_loop(uint8_t* lds, const PPCtx& c,
                                        PPCur<GRP, GRAN == GRAN_MX ? 1 : 4>& cur) {
    v4f acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    v8i x[4], w[8];
    PPScales ps;
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const int NS = c.NS, KB = c.KB, wm = c.wm, wn = c.wn, lr = c.lr, lk = c.lk;
    PPCur<GRP, GRAN == GRAN_MX ? 1 : 4> nxt = cur;  // group 0: the block after cur

    // the last two products of a compute phase, promoted after its barrier so
    // the other group's first MFMA queues right behind them
    v4f carry = zero, carry2 = zero;
    float carry_sc = 0.0f, carry2_sc = 0.0f;
    int ct = 0, ckb = 0;  // compute cursor: tile, K block
    for (int s = 0; s < NS; ++s) {
        // ---- memory phase of block s ----
        promote(acc[2][7], carry2, carry2_sc);
        promote(acc[3][7], carry, carry_sc);
        const bool stored = ckb == 0 && s > 0;
        if (stored) {  // the previous tile is complete: store it
            const BigTile t = pp_tile(c, ct - 1);
            if constexpr (GRAN == GRAN_ROW) pp_row_scale(acc, c, t, wn, wm, lr, lk);
            pp_store_tile(acc, t, c.Y, (int)c.G.N, c.G.B, wn, wm, lr, lk);
        }
        pp_read<GRAN>(lds, c, s, x, w, ps);
        __builtin_amdgcn_s_waitcnt(kLgkm0);  // fragments and scales in registers
        // the previous compute phase's loads; vector memory operations complete
        // in issue order, so the stores just issued need not be waited for
        if (stored)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPPStores));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        pp_barrier();
        // ---- compute phase of block s ----
        // advance the load cursor here, before the MFMAs: a branch after them
        // would let the compiler sink their promotions past it
        if (GRP == 0) {
            nxt = cur;
            nxt.next(c);  // cur: block s + 1, nxt: block s + 2
        } else {
            cur.next(c);  // block s + 2
        }
        int o = GRP == 0 ? c.off0 : c.offA;
        asm volatile("" : "+v"(o));  // recomputed per phase, not held across the loop
        __builtin_amdgcn_sched_barrier(0);
        v4f pr[3];
#pragma unroll
        for (int n = 0; n < 32; ++n) {
            if constexpr (GRAN == GRAN_BLOCK) {
                pr[n % 3] = mfma_f8(w[n >> 2], x[n & 3], zero);
                if (n > 1) {
                    const int m = n - 2;
                    promote(acc[m & 3][m >> 2], pr[m % 3], ps.sc[m & 3]);
                }
            } else if constexpr (GRAN == GRAN_MX) {
                acc[n & 3][n >> 2] =
                    mfma_mx(w[n >> 2], x[n & 3], acc[n & 3][n >> 2], ps.sw, ps.sa[n & 3]);
            } else {
                acc[n & 3][n >> 2] = mfma_f8(w[n >> 2], x[n & 3], acc[n & 3][n >> 2]);
            }
            // group 0: 8 loads, one per 4 MFMAs; group 1: 10 (8 without
            // per-block scales), one per 3 (4)
            const bool ld = GRP == 0 || GRAN == GRAN_ROW ? (n & 3) == 0 : (n % 3 == 0 && n <= 27);
            if (ld) {
                if constexpr (GRP == 0)
                    pp_load0(lds, c, cur, nxt, o, n >> 2);
                else
                    pp_load1(lds, c, cur, o, GRAN == GRAN_ROW ? n >> 2 : n / 3);
            }
            // MFMA; the 4 FMAs promoting the MFMA before it, plus the address
            // add of a chunk load; then the load
            const bool add = ld && (GRP == 0 || GRAN == GRAN_ROW || n / 3 < 8);
            const bool fma = GRAN == GRAN_BLOCK && n > 1;
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            if (fma && add)
                __builtin_amdgcn_sched_group_barrier(kSgValu, 5, 0);
            else if (fma)
                __builtin_amdgcn_sched_group_barrier(kSgValu, 4, 0);
            else if (add)
                __builtin_amdgcn_sched_group_barrier(kSgValu, 1, 0);
            if (ld) __builtin_amdgcn_sched_group_barrier(kSgVmem, 1, 0);
        }
        if constexpr (GRAN == GRAN_BLOCK) {
            carry2 = pr[30 % 3];
            carry2_sc = ps.sc[2];
            carry = pr[31 % 3];
            carry_sc = ps.sc[3];
        }
        __builtin_amdgcn_sched_barrier(0);
        if (GRP == 0) cur = nxt;
        pp_barrier();
        if (++ckb == KB) {
            ckb = 0;
            ++ct;
        }
    }
    if (GRP == 0) pp_barrier();  // the barrier count of group 1's offset
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the last compute phase's loads
    promote(acc[2][7], carry2, carry2_sc);
    promote(acc[3][7], carry, carry_sc);
    const BigTile t = pp_tile(c, ct - 1);
    if constexpr (GRAN == GRAN_ROW) pp_row_scale(acc, c, t, wn, wm, lr, lk);
    pp_store_tile(acc, t, c.Y, (int)c.G.N, c.G.B, wn, wm, lr, lk);
}

// GRAN_BLOCK (fp32 scales, promotion FMAs), GRAN_MX (E8M0 scales applied by
// the MX-scaled MFMA, which accumulates) or GRAN_ROW (the MFMA accumulates,
// per-row x per-column scales at the store); dense (B = 1), N % 256 == 0.
// GROUPED (block scales): the MoE form over E experts, expert e's rows
// [offsets[e], offsets[e + 1]) of A and Y against W[e] (G.M = total rows).
template <int GRAN, bool GROUPED = false>
__global__ __launch_bounds__(kThreads2) void k_gemm_pp(const uint8_t* __restrict__ A,
                                                       const uint8_t* __restrict__ W,
                                                       const void* __restrict__ sA,
                                                       const void* __restrict__ sW,
                                                       uint16_t* __restrict__ Y, BigGeom G,
                                                       const int32_t* __restrict__ offsets,
                                                       int E) {
    constexpr int SB = GRAN == GRAN_MX ? 1 : 4;  // bytes per scale
    constexpr int NL1 = GRAN == GRAN_ROW ? 8 : 10;  // group 1's loads per block
    // one LDS object for the stage ring and (grouped) the expert tables
    constexpr int kTab = GROUPED ? (3 * kMaxExpertsBig + 1) * 4 : 0;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLds2 + kTab];
    PPCtx c;
    c.A = A; c.W = W; c.Y = Y; c.G = G;
    c.sA = static_cast<const uint8_t*>(sA);
    c.sW = static_cast<const uint8_t*>(sW);
    c.tm_count = (int)((G.M + BM2 - 1) / BM2);
    c.tn_count = (int)(G.N / BN2);
    c.grouped = GROUPED;
    c.grp = BigGroups{};
    int T = c.tm_count * c.tn_count * G.B;  // batch-major (B = 1 but for the batched MX GEMM)
    if constexpr (GROUPED) {
        big_groups(lds + kLds2, offsets, E, G.M, c.tn_count);
        __syncthreads();
        const int32_t* s_pre = reinterpret_cast<const int32_t*>(lds + kLds2);
        c.grp = BigGroups{s_pre, s_pre + kMaxExpertsBig + 1, s_pre + 2 * kMaxExpertsBig + 1, E};
        T = s_pre[E];
    }
    c.K = (int)G.K;
    c.KB = c.K / BK;
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    c.nwg = ((int)gridDim.x - xcd + 7) >> 3;
    const int q = T >> 3, rem = T & 7;
    const int xbeg = xcd * q + (xcd < rem ? xcd : rem), tx = q + (xcd < rem ? 1 : 0);
    if (idx >= tx) return;
    const int nt = (tx - idx + c.nwg - 1) / c.nwg;
    c.first = xbeg + idx;
    c.NS = nt * c.KB;

    const int tid = threadIdx.x, lane = tid & 63;
    c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = c.wave >> 2, wq = c.wave & 3;
    c.wm = wq;
    c.wn = grp;
    c.lr = lane & 15;
    c.lk = lane >> 4;
    c.lda = G.B * c.K;
    c.off0 = (wq * 8 + (lane >> 3)) * c.K + swz_pos(lane >> 3, lane & 7) * 16;
    c.offA = (wq * 8 + (lane >> 3)) * c.lda + swz_pos(lane >> 3, lane & 7) * 16;
    c.offa = (wq * 64 + lane) * G.B * c.KB * SB;
    c.offw = (lane & 1) * c.KB * SB;
    asm volatile("" ::"s"(Y));
    // prologue: all of block 0 and, of block 1, everything but W half 1
    // (group 0 loads it in its first compute phase)
    if (grp == 0) {
        PPCur<0, SB> cur, nxt;
        cur.start(c, 0);
        nxt.start(c, 0);
        const int o = c.off0;
#pragma unroll
        for (int n = 0; n < 8; ++n) pp_load0(lds, c, cur, nxt, o, n);  // W halves 1, 0 of block 0
        nxt.next(c);
#pragma unroll
        for (int n = 4; n < 8; ++n) pp_load0(lds, c, cur, nxt, o, n);  // W half 0 of block 1
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        pp_barrier();
        pp_loop<GRAN, 0>(lds, c, nxt);  // cur = block 1
    } else {
        PPCur<1, SB> cur;
        cur.start(c, 0);
        const int o = c.offA;
#pragma unroll
        for (int n = 0; n < NL1; ++n) pp_load1(lds, c, cur, o, n);  // block 0
        cur.next(c);
#pragma unroll
        for (int n = 0; n < NL1; ++n) pp_load1(lds, c, cur, o, n);  // block 1
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        pp_barrier();
        pp_barrier();  // group 1 runs one phase behind
        pp_loop<GRAN, 1>(lds, c, cur);
    }
}

// ---------------------------------------------------------------------------
// Small-M and grouped kernel: tile 128 x 128, K step 128, 512 threads as 2 x 4
// waves of 64 x 32 (two waves per SIMD), the same transposed MFMA, promotion
// and 8-byte stores as
// k_gemm_big, and a ring of 4 LDS stages filled by direct-to-LDS loads with 3
// stages in flight.  At small M (decode, MoE experts) a tile's loads come
// mostly from HBM, so the latency of one stage is far longer than its
// multiply; three stages of lookahead keep ~96 KiB in flight per CU.
// Every wave issues the same number of loads per stage (4 tile chunks plus,
// in BLOCK mode, one scale: the eight waves load the 128 row scales in four
// copies), so the waits are immediates: before multiplying stage kb a wave
// waits until only the stages issued after kb may be outstanding, then a bare
// s_barrier publishes everyone's loads.  (A barrier with a fence would wait for
// every outstanding direct-to-LDS load and collapse the ring to one stage.)
// ---------------------------------------------------------------------------
constexpr int BMP = 128, BNP = 128, kThreadsP = 512, NSTP = 4;
constexpr int64_t kPersistentGrid = 256;  // one workgroup per CU (LDS bound)
constexpr int64_t kMaxExperts = 1024;     // prefix array size of the grouped kernel
constexpr int kStageTileP = (BMP + BNP) * BK;            // 32 KiB of operands
constexpr int kSwP = kStageTileP + 4 * BMP * 4;           // after four copies of sA:
constexpr int kStageP = kSwP + 8 * 256;                   // each wave's copy of sW (BUF)
constexpr int kLdsP = NSTP * kStageP;
static_assert(kLdsP + (3 * 1024 + 1) * 4 <= 160 * 1024,
              "gfx950 has 160 KiB of LDS per workgroup (stage ring + expert tables)");


// Where a stage's loads come from.  BUF (K <= 2^22): buffer resources over
// the tile's rows and scales, with each lane's 32-bit offsets computed once
// per tile; the loads are buffer_load ... lds, which keep the compiler's LDS
// waits counted, and each wave also stages its own copy of the weight-block
// scale.  Otherwise (longer K): the global form from the tile's pointers, and
// the weight-block scale read with a scalar load.
struct PipeSrc {
    __amdgpu_buffer_rsrc_t a, w, sa, sw;
    int offa[2], offw[2], offsa;
};

template <int GRAN, bool BUF>
struct PipeLoad {
    Tile t;
    PipeSrc s;
    __device__ __forceinline__ void set(const Tile& tile, int64_t K, int64_t KB, int wave,
                                        int lane) {
        t = tile;
        if constexpr (BUF) {
            const int k = (int)K, kbn = (int)KB;
            s.a = buffer_rsrc(t.A, t.rows * k);
            s.w = buffer_rsrc(t.W, BNP * k);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int p = (i * 8 + wave) * 64 + lane;
                const int r = p >> 3;
                const int c = swz_pos(r, p & 7);
                const int ra = r < t.rows ? r : t.rows - 1;
                s.offa[i] = ra * k + c * 16;
                s.offw[i] = r * k + c * 16;
            }
            if constexpr (GRAN == GRAN_BLOCK || GRAN == GRAN_MX) {
                constexpr int sb = GRAN == GRAN_MX ? 1 : 4;  // bytes per scale
                const int r = (wave & 1) * 64 + lane;
                const int rr = r < t.rows ? r : t.rows - 1;
                s.sa = buffer_rsrc(t.sA, t.rows * kbn * sb);
                s.sw = buffer_rsrc(t.sW, kbn * sb);
                s.offsa = rr * kbn * sb;
            }
        }
    }
};

template <int GRAN, bool BUF>
__device__ __forceinline__ void stage_pipe(uint8_t* lds, int st, const PipeLoad<GRAN, BUF>& L,
                                           int64_t K, int64_t KB, int kb, int wave, int lane) {
    uint8_t* la = lds + st * kStageP;
    uint8_t* lb = la + BMP * BK;
    if constexpr (BUF) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int pbase = (i * 8 + wave) * 64;  // LDS chunk of lane 0 (8 rows per wave load)
            b2l(L.s.a, la + pbase * 16, 16, L.s.offa[i], kb * BK);
            b2l(L.s.w, lb + pbase * 16, 16, L.s.offw[i], kb * BK);
        }
        if constexpr (GRAN == GRAN_BLOCK || GRAN == GRAN_MX) {
            // an E8M0 byte lands zero-extended in its lane's 32-bit word
            constexpr int sb = GRAN == GRAN_MX ? 1 : 4;
            b2l(L.s.sa, la + kStageTileP + (wave >> 1) * (BMP * 4) + (wave & 1) * 256, sb,
                L.s.offsa, kb * sb);
            b2l(L.s.sw, la + kSwP + wave * 256, sb, 0, kb * sb);  // every lane the same word
        }
    } else {
        const Tile& t = L.t;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int pbase = (i * 8 + wave) * 64;
            const int p = pbase + lane;
            const int r = p >> 3;
            const int c = swz_pos(r, p & 7);
            const int ra = r < t.rows ? r : t.rows - 1;
            g2l_16(t.A + ra * K + kb * BK + c * 16, la + pbase * 16);
            g2l_16(t.W + r * K + kb * BK + c * 16, lb + pbase * 16);
        }
        if constexpr (GRAN == GRAN_BLOCK) {
            const int r = (wave & 1) * 64 + lane;
            const int rr = r < t.rows ? r : t.rows - 1;
            g2l_4(t.sA + rr * KB + kb,
                  la + kStageTileP + (wave >> 1) * (BMP * 4) + (wave & 1) * 256);
        }
    }
}

template <int GRAN, bool BUF>
__device__ __forceinline__ void wait_stage(int kb, int KB) {
    // loads per stage per thread
    constexpr int per = GRAN == GRAN_BLOCK || GRAN == GRAN_MX ? (BUF ? 6 : 5) : 4;
    if (kb + 2 < KB)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * per));
    else if (kb + 1 < KB)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(per));
    else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// Scalar load of a wave-uniform element of a read-only device array: the
// pointer and index go through readfirstlane (provably uniform) and the load
// goes through the constant address space, which the backend lowers to
// s_load.  A vector or flat load here would count in vmcnt, and its wait
// would drain the whole stage ring.
__device__ __forceinline__ float uniform_load(const float* p, int idx) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    typedef const __attribute__((address_space(4))) float cfloat;
    cfloat* c = (cfloat*)(((uint64_t)hi << 32) | lo);
    return c[__builtin_amdgcn_readfirstlane(idx)];
}

// Where a persistent workgroup's tiles come from.  Dense: a tm_count x
// tn_count grid, row tiles of one column tile adjacent.  Grouped (MoE): expert
// by expert, then column tile by column tile with that expert's row tiles
// adjacent; pre[] (in LDS) is the prefix over experts of ceil(rows_e/128) * NT.
struct TileSpace {
    const uint8_t* A;
    const uint8_t* W;
    const float* sA;
    const float* sW;
    uint16_t* Y;
    const int32_t* offsets;  // grouped only (device)
    const int32_t* pre;      // grouped only (LDS), E + 1 entries
    const int32_t* rlo;      // grouped only (LDS): expert e's rows [rlo[e], rhi[e])
    const int32_t* rhi;
    int64_t M, N, K, E;
    int64_t tm_count;        // dense only
};

// Every kernel argument the small-M kernels read, wanted in SGPRs at once:
// the compiler then issues all the argument loads together and waits for
// them once, instead of one round trip per group of first uses spread over
// the index arithmetic (three to four at these kernels' starts).
template <class T0, class T1, class T2>
__device__ __forceinline__ void args_ready(const TileSpace& S, T0 a, T1 b, T2 c) {
    asm volatile("" ::"s"(S.A), "s"(S.W), "s"(S.sA), "s"(S.sW), "s"(S.Y), "s"(S.M), "s"(S.N),
                 "s"(S.K), "s"(S.tm_count), "s"(a), "s"(b), "s"(c));
}

template <int GRAN, bool GROUPED>
__device__ __forceinline__ Tile tile_at(const TileSpace& S, int64_t logical) {
    const int64_t KB = S.K / BK, NT = S.N / BNP;
    Tile t;
    int64_t row0, n0, e = 0, rows;
    if constexpr (GROUPED) {
        int lo = 0, hi = (int)S.E - 1;  // last expert whose prefix start <= logical
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (S.pre[mid] <= logical) lo = mid; else hi = mid - 1;
        }
        e = lo;
        const int64_t r_lo = S.rlo[e], r_hi = S.rhi[e];
        const int64_t mt = (r_hi - r_lo + BMP - 1) / BMP;
        const int64_t lt = logical - S.pre[e];
        const int64_t tn = lt / mt, tm = lt % mt;
        row0 = r_lo + tm * BMP;
        n0 = tn * BNP;
        rows = (r_hi - row0) < BMP ? (r_hi - row0) : BMP;
        t.W = S.W + (e * S.N + n0) * S.K;
        t.sW = S.sW + (e * NT + tn) * KB;
    } else {
        const int64_t tm = logical % S.tm_count, tn = logical / S.tm_count;
        row0 = tm * BMP;
        n0 = tn * BNP;
        rows = (S.M - row0) < BMP ? (S.M - row0) : BMP;
        t.W = S.W + n0 * S.K;
        t.sW = GRAN == GRAN_BLOCK ? S.sW + tn * KB : S.sW + n0;
    }
    t.A = S.A + row0 * S.K;
    t.sA = GRAN == GRAN_BLOCK ? S.sA + row0 * KB : S.sA + row0;
    if constexpr (GRAN == GRAN_MX) {  // E8M0 bytes [M, KB] and [N/128, KB] (dense)
        t.sA = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(S.sA) + row0 * KB);
        t.sW = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(S.sW) +
                                              (n0 / BNP) * KB);
    }
    t.Y = S.Y + row0 * S.N + n0;
    t.rows = (int)rows;
    return t;
}

// One K step of a 128 x 128 tile from LDS stage `la`: BLOCK promotes each
// 16 x 16 product by its row scale x the weight block scale into acc (the FMA
// of a product trails its MFMA by one); ROW accumulates in the MFMA; MX
// accumulates in the MX-scaled MFMA, which applies the E8M0 scales.
template <int GRAN, bool BUF>
__device__ __forceinline__ void pipe_mma(const uint8_t* la, const float* sW, int kb,
                                         v4f (&acc)[4][2], int wm, int wn, int lr, int lk) {
    const uint8_t* lb = la + BMP * BK;
    v8i x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = frag(la, wm * 64 + i * 16 + lr, lk);
    if constexpr (GRAN == GRAN_BLOCK) {
        float sw;
        if constexpr (BUF)
            sw = *reinterpret_cast<const float*>(la + kSwP + (wm | (wn << 1)) * 256);
        else
            sw = uniform_load(sW, kb);
        const float* lsa = reinterpret_cast<const float*>(la + kStageTileP);
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = lsa[wm * 64 + i * 16 + lr] * sw;
        const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
        v8i wcur = frag(lb, wn * 32 + lr, lk);
        v4f prev;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            v8i wnext = wcur;
            if (jj < 1) wnext = frag(lb, wn * 32 + (jj + 1) * 16 + lr, lk);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const v4f pk = mfma_f8(wcur, x[i], zero);
                if (i > 0 || jj > 0) {
                    const int pi = i > 0 ? i - 1 : 3, pj = i > 0 ? jj : jj - 1;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[pi][pj][e] = __builtin_fmaf(prev[e], sc[pi], acc[pi][pj][e]);
                }
                prev = pk;
            }
            wcur = wnext;
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[3][1][e] = __builtin_fmaf(prev[e], sc[3], acc[3][1][e]);
    } else if constexpr (GRAN == GRAN_MX) {  // BUF: scales staged with the stage
        const int sw = *reinterpret_cast<const int*>(la + kSwP + (wm | (wn << 1)) * 256);
        const int* lsa = reinterpret_cast<const int*>(la + kStageTileP);
        int sa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] = lsa[wm * 64 + i * 16 + lr];
        v8i wcur = frag(lb, wn * 32 + lr, lk);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            v8i wnext = wcur;
            if (jj < 1) wnext = frag(lb, wn * 32 + (jj + 1) * 16 + lr, lk);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i][jj] = mfma_mx(wcur, x[i], acc[i][jj], sw, sa[i]);
            wcur = wnext;
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        v8i wcur = frag(lb, wn * 32 + lr, lk);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            v8i wnext = wcur;
            if (jj < 1) wnext = frag(lb, wn * 32 + (jj + 1) * 16 + lr, lk);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i][jj] = mfma_f8(wcur, x[i], acc[i][jj]);
            wcur = wnext;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// bf16 stores of a finished 128 x 128 tile (ROW: scaled by the row and column
// scales first); acc is left zeroed for the next tile.
template <int GRAN>
__device__ __forceinline__ void pipe_store(const Tile& ct, v4f (&acc)[4][2], int64_t N, int wm,
                                           int wn, int lr, int lk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + lr;
        float sa = 1.0f;
        if constexpr (GRAN == GRAN_ROW) sa = ct.sA[r < ct.rows ? r : ct.rows - 1];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            v4f v = acc[i][jj];
            acc[i][jj] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (GRAN == GRAN_ROW) {
                const v4f s4 =
                    *reinterpret_cast<const v4f*>(ct.sW + wn * 32 + jj * 16 + 4 * lk);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = v[e] * (sa * s4[e]);
            }
            if (r < ct.rows) {
                uint2 o;
                o.x = bf16x2_rne(v[0], v[1]);
                o.y = bf16x2_rne(v[2], v[3]);
                *reinterpret_cast<uint2*>(ct.Y + (int64_t)r * N + wn * 32 + jj * 16 +
                                          4 * lk) = o;
            }
        }
    }
}

// Persistent small-M / grouped kernel.  The grid holds one workgroup per CU
// (at most); XCD x = blockIdx % 8 owns the x-th eighth of the tile order and
// its workgroups take every nx-th tile of it, so the workgroups of one XCD
// work on adjacent tiles together.  A workgroup's K steps over all of its
// tiles form one sequence g = (tile i, k block) that the 4-stage ring walks
// without a break: the next tile's first stages load while the current tile
// finishes.
template <int GRAN, bool GROUPED, bool BUF>
__global__ __launch_bounds__(kThreadsP) void k_gemm_pipe(TileSpace S, int64_t dense_tiles) {
    // one LDS object for the stage ring and (grouped) the expert tables: with
    // separate __shared__ arrays the compiler can no longer tell the
    // direct-to-LDS stage writes from the operand reads and waits for every
    // outstanding load before each read
    constexpr int kTab = GROUPED ? (3 * kMaxExperts + 1) * 4 : 0;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsP + kTab];
    int32_t* s_pre = reinterpret_cast<int32_t*>(lds + kLdsP);
    int32_t* s_rlo = s_pre + kMaxExperts + 1;
    int32_t* s_rhi = s_rlo + kMaxExperts;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;  // wn in 0..3: 32 columns each
    const int lr = lane & 15, lk = lane >> 4;
    const int64_t KB = S.K / BK;

    int64_t T = dense_tiles;
    if constexpr (GROUPED) {
        // prefix over experts of their tile counts, into LDS (wave 0)
        const int64_t NT = S.N / BNP;
        if (wave == 0) {
            int64_t base = 0;
            for (int64_t e0 = 0; e0 < S.E; e0 += 64) {
                const int64_t e = e0 + lane;
                int64_t cnt = 0;
                if (e < S.E) {
                    int64_t lo = S.offsets[e], hi = S.offsets[e + 1];
                    lo = lo < 0 ? 0 : (lo > S.M ? S.M : lo);
                    hi = hi < lo ? lo : (hi > S.M ? S.M : hi);
                    cnt = (hi - lo + BMP - 1) / BMP * NT;
                    s_rlo[e] = (int32_t)lo;
                    s_rhi[e] = (int32_t)hi;
                }
                int64_t incl = cnt;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int64_t up = __shfl_up(incl, o);
                    if (lane >= o) incl += up;
                }
                if (e < S.E) s_pre[e] = (int32_t)(base + incl - cnt);
                base += __shfl(incl, 63);
            }
            if (lane == 0) s_pre[S.E] = (int32_t)base;
        }
        __syncthreads();
        S.pre = s_pre;
        S.rlo = s_rlo;
        S.rhi = s_rhi;
        T = s_pre[S.E];
    }
    // this workgroup's tiles: first, first + nx, ... (< last)
    const int64_t G = gridDim.x, bid = blockIdx.x, xcd = bid & 7, j = bid >> 3;
    const int64_t nx = (G - xcd + 7) >> 3;  // workgroups on this XCD
    const int64_t q = T >> 3, rem = T & 7;
    const int64_t first_x = xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q;
    const int64_t last_x = first_x + (xcd < rem ? q + 1 : q);
    const int64_t first = first_x + j;
    const int64_t ntiles = first < last_x ? (last_x - first + nx - 1) / nx : 0;
    const int64_t NG = ntiles * KB;  // K steps of all this workgroup's tiles
    if (NG == 0) return;  // whole workgroup leaves together

    v4f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) acc[i][jj] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // Loop counters are 32-bit and advanced incrementally: a 64-bit division
    // in the loop is expanded on the vector ALU, its result (and any address
    // built from it) lands in VGPRs, and a weight-scale read then becomes a
    // vector load whose wait drains the whole stage ring.
    const int kbn = (int)KB, ng = (int)NG;
    PipeLoad<GRAN, BUF> lt;  // tile being loaded
    lt.set(tile_at<GRAN, GROUPED>(S, first), S.K, KB, wave, lane);
    int l_ti = 0, l_kb = 0;                      // (tile, k block) of the next stage to load
#pragma unroll
    for (int st = 0; st < NSTP - 1; ++st) {
        if (st < ng) {
            stage_pipe<GRAN, BUF>(lds, st, lt, S.K, KB, l_kb, wave, lane);
            if (++l_kb == kbn) {
                l_kb = 0;
                ++l_ti;
                if (l_ti < ntiles)
                    lt.set(tile_at<GRAN, GROUPED>(S, first + l_ti * nx), S.K, KB, wave, lane);
            }
        }
    }
    Tile ct = tile_at<GRAN, GROUPED>(S, first);  // tile being multiplied
    int c_ti = 0, kb = 0;

    for (int g = 0; g < ng; ++g) {
        asm volatile("" ::: "memory");
        wait_stage<GRAN, BUF>(g, ng);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (g + NSTP - 1 < ng) {  // refill the stage consumed at g - 1
            stage_pipe<GRAN, BUF>(lds, (g + NSTP - 1) % NSTP, lt, S.K, KB, l_kb, wave, lane);
            if (++l_kb == kbn) {
                l_kb = 0;
                ++l_ti;
                if (l_ti < ntiles)
                    lt.set(tile_at<GRAN, GROUPED>(S, first + l_ti * nx), S.K, KB, wave, lane);
            }
        }

        pipe_mma<GRAN, BUF>(lds + (g % NSTP) * kStageP, ct.sW, kb, acc, wm, wn, lr, lk);
        if (kb == kbn - 1) pipe_store<GRAN>(ct, acc, S.N, wm, wn, lr, lk);  // tile done
        if (++kb == kbn) {
            kb = 0;
            ++c_ti;
            if (c_ti < ntiles) ct = tile_at<GRAN, GROUPED>(S, first + c_ti * nx);
        }
    }
}

// ---------------------------------------------------------------------------
// Stream-K small-M kernel (dense only).  The tiles' K steps, tile after tile
// (u = tile * KB + kb, tiles in the k_gemm_pipe order), are cut into G equal
// contiguous ranges, one per workgroup, so every CU gets the same number of
// steps whatever the tile count (at decode M a linear has fewer 128 x 128
// tiles than there are CUs, and a long K would leave most CUs idle).  A
// workgroup whose range covers a whole tile stores it directly.  For a tile
// cut between workgroups each contributor stores its fp32 accumulators in its
// partial slot and moves on; k_sk_reduce, launched next on the same stream,
// sums each such tile's partials in contributor order (so the bytes do not
// depend on timing) and stores it.  The kernel boundary orders the partial
// stores before the reads on every XCD, so neither kernel waits on another
// workgroup or needs a counter.
//   Workspace: part = G x 2 slots of 128 x 128 fp32 (slot 0: the first tile
//   of a workgroup's range, slot 1: its last), in register order (v4f index
//   (slot * 8 + i * 2 + jj) * 512 + tid).
// ---------------------------------------------------------------------------
static_assert(kGemmWsMaxBytes >= kPersistentGrid * 2 * BMP * BNP * 4, "partial slots");

struct SkWork {
    v4f* part;
};

// one v4f of a partial tile (plain 16-byte accesses: the kernel boundary
// between the stream-K kernel and the reduce orders them)
__device__ __forceinline__ void sk_put(v4f* p, const v4f& v) { *p = v; }
__device__ __forceinline__ v4f sk_get(const v4f* p) { return *p; }

// A thread's 4 x 2 accumulator fragments (rows wm * 64 + i * 16 + lr of its
// wave) to a partial slot; CHECK skips rows at or past `wrows` (rows of the
// wave that exist), which only the wave holding row M - 1 needs.
template <bool CHECK>
__device__ __forceinline__ void sk_write(v4f* mine, const v4f (&acc)[4][2], int wrows, int lr) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (!CHECK || i * 16 + lr < wrows)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) sk_put(mine + (i * 2 + jj) * kThreadsP, acc[i][jj]);
}
// first K step of rank c's range, and the rank owning step u
__device__ __forceinline__ int64_t sk_start(int64_t c, int64_t Wt, int64_t G) {
    return c * Wt / G;
}
__device__ __forceinline__ int64_t sk_owner(int64_t u, int64_t Wt, int64_t G) {
    return ((u + 1) * G + Wt - 1) / Wt - 1;
}

template <int GRAN, bool BUF>
__global__ __launch_bounds__(kThreadsP) void k_gemm_sk(TileSpace S, int64_t tiles, SkWork ws) {
    args_ready(S, tiles, ws.part, gridDim.x);
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsP];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int lr = lane & 15, lk = lane >> 4;
    const int64_t KB = S.K / BK, Wt = tiles * KB, G = gridDim.x;
    // XCD-contiguous rank: the workgroups of XCD x (blockIdx % 8 == x) hold
    // consecutive ranks, so one XCD's ranges are adjacent steps and tiles
    const int64_t bid = blockIdx.x, xcd = bid & 7;
    const int64_t q8 = G >> 3, r8 = G & 7;
    const int64_t c = xcd * q8 + (xcd < r8 ? xcd : r8) + (bid >> 3);
    const int64_t u0 = sk_start(c, Wt, G), u1 = sk_start(c + 1, Wt, G);
    const int ng = (int)(u1 - u0);
    if (ng <= 0) return;  // whole workgroup leaves together
    const int64_t t_first = u0 / KB;

    v4f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) acc[i][jj] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int kbn = (int)KB;
    int64_t l_t = t_first;  // tile and k block of the next stage to load
    int l_kb = (int)(u0 - t_first * KB);
    PipeLoad<GRAN, BUF> lt;
    lt.set(tile_at<GRAN, false>(S, l_t), S.K, KB, wave, lane);
#pragma unroll
    for (int st = 0; st < NSTP - 1; ++st) {
        if (st < ng) {
            stage_pipe<GRAN, BUF>(lds, st, lt, S.K, KB, l_kb, wave, lane);
            if (++l_kb == kbn) {
                l_kb = 0;
                ++l_t;
                if (l_t < tiles) lt.set(tile_at<GRAN, false>(S, l_t), S.K, KB, wave, lane);
            }
        }
    }
    int64_t c_t = t_first;  // tile being multiplied, its k block, where this range entered it
    int kb = (int)(u0 - t_first * KB);
    int kb_in = kb;
    Tile ct = tile_at<GRAN, false>(S, c_t);

    for (int g = 0; g < ng; ++g) {
        asm volatile("" ::: "memory");
        wait_stage<GRAN, BUF>(g, ng);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (g + NSTP - 1 < ng) {
            stage_pipe<GRAN, BUF>(lds, (g + NSTP - 1) % NSTP, lt, S.K, KB, l_kb, wave, lane);
            if (++l_kb == kbn) {
                l_kb = 0;
                ++l_t;
                if (l_t < tiles) lt.set(tile_at<GRAN, false>(S, l_t), S.K, KB, wave, lane);
            }
        }
        pipe_mma<GRAN, BUF>(lds + (g % NSTP) * kStageP, ct.sW, kb, acc, wm, wn, lr, lk);

        if (kb == kbn - 1 || g == ng - 1) {  // this range's part of tile c_t is done
            if (kb_in == 0 && kb == kbn - 1) {
                pipe_store<GRAN>(ct, acc, S.N, wm, wn, lr, lk);
            } else {
                const int slot = (c_t == t_first) ? 0 : 1;
                // rows past M carry nothing: a wave whose 64 rows are all
                // valid (the common case) moves its partial without checks
                const int wrows = ct.rows - wm * 64;
                v4f* mine = ws.part + (c * 2 + slot) * 8 * kThreadsP + tid;
                if (wrows >= 64)
                    sk_write<false>(mine, acc, wrows, lr);
                else if (wrows > 0)
                    sk_write<true>(mine, acc, wrows, lr);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) acc[i][jj] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
        if (++kb == kbn) {
            kb = 0;
            kb_in = 0;
            ++c_t;
            if (c_t < tiles) ct = tile_at<GRAN, false>(S, c_t);
        }
    }
}

// Sum of the partials of each tile that the stream-K kernel split, in
// contributor order (so the bytes do not depend on timing), then the bf16
// store.  kSkRedSplit workgroups per tile, workgroup r of a tile taking row
// fragment i = r of every wave (rows wm * 64 + 16 r + lr): one workgroup per
// tile left three quarters of the chip idle at decode shapes and read 64 KiB
// per partial through one CU.  A tile one workgroup covered whole exits at
// once.  Threads map to accumulator fragments exactly as in the stream-K
// kernel.
constexpr int kSkRedSplit = 4;

template <int GRAN>
__global__ __launch_bounds__(kThreadsP) void k_sk_reduce(TileSpace S, int64_t tiles, int64_t G,
                                                        const v4f* __restrict__ part) {
    args_ready(S, tiles, G, part);
    const int64_t t = blockIdx.x / kSkRedSplit, KB = S.K / BK, Wt = tiles * KB;
    const int i = (int)(blockIdx.x % kSkRedSplit);
    const int64_t c_lo = sk_owner(t * KB, Wt, G), c_hi = sk_owner(t * KB + KB - 1, Wt, G);
    if (c_lo == c_hi) return;  // stored whole by its workgroup
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1, lr = lane & 15, lk = lane >> 4;
    const Tile ct = tile_at<GRAN, false>(S, t);
    const int r = wm * 64 + i * 16 + lr;  // this thread's row of the tile
    v4f sum[2] = {v4f{0.0f, 0.0f, 0.0f, 0.0f}, v4f{0.0f, 0.0f, 0.0f, 0.0f}};
    if (r < ct.rows) {
        for (int64_t cc = c_lo; cc <= c_hi; ++cc) {
            const int sl = (sk_start(cc, Wt, G) / KB == t) ? 0 : 1;
            const v4f* pp = part + (cc * 2 + sl) * 8 * kThreadsP + tid;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const v4f p = sk_get(pp + (i * 2 + jj) * kThreadsP);
#pragma unroll
                for (int e = 0; e < 4; ++e) sum[jj][e] = sum[jj][e] + p[e];
            }
        }
        float sa = 1.0f;
        if constexpr (GRAN == GRAN_ROW) sa = ct.sA[r];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            v4f v = sum[jj];
            if constexpr (GRAN == GRAN_ROW) {
                const v4f s4 = *reinterpret_cast<const v4f*>(ct.sW + wn * 32 + jj * 16 + 4 * lk);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = v[e] * (sa * s4[e]);
            }
            uint2 o;
            o.x = bf16x2_rne(v[0], v[1]);
            o.y = bf16x2_rne(v[2], v[3]);
            *reinterpret_cast<uint2*>(ct.Y + (int64_t)r * S.N + wn * 32 + jj * 16 + 4 * lk) = o;
        }
    }
}

// k_sk_reduce for tiles with many contributors: SPLIT workgroups per tile
// (8 or more), each taking NF = 8 / SPLIT of the eight
// accumulator fragments (i * 2 + jj: rows wm * 64 + 16 i + lr, columns
// wn * 32 + 16 jj + 4 lk) of every wave; one workgroup per tile left most of
// the chip idle at decode shapes.  A thread sums one 16-byte value per
// contributor and fragment, four such loads issued together (over 4 / NF
// contributors) and added in contributor order.  A tile one workgroup covered whole exits
// at once.  Threads map to accumulator fragments exactly as in the stream-K
// kernel.
template <int GRAN, int SPLIT>
__global__ __launch_bounds__(kThreadsP) void k_sk_reduce_wide(TileSpace S, int64_t tiles, int64_t G,
                                                        const v4f* __restrict__ part) {
    args_ready(S, tiles, G, part);
    constexpr int NF = 8 / SPLIT;
    const int64_t t = blockIdx.x / SPLIT, KB = S.K / BK, Wt = tiles * KB;
    const int f0 = (int)(blockIdx.x % SPLIT) * NF;
    const int64_t c_lo = sk_owner(t * KB, Wt, G), c_hi = sk_owner(t * KB + KB - 1, Wt, G);
    if (c_lo == c_hi) return;  // stored whole by its workgroup
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1, lr = lane & 15, lk = lane >> 4;
    const Tile ct = tile_at<GRAN, false>(S, t);
    const int r = wm * 64 + (f0 >> 1) * 16 + lr;  // the NF fragments share a row
    if (r >= ct.rows) return;
    // contributor cc's partial slot (0 if its range starts in tile t), at this
    // thread's first fragment
    auto base = [&](int64_t cc) {
        const int sl = (sk_start(cc, Wt, G) / KB == t) ? 0 : 1;
        return part + (cc * 2 + sl) * 8 * kThreadsP + f0 * kThreadsP + tid;
    };
    v4f sum[NF];
#pragma unroll
    for (int n = 0; n < NF; ++n) sum[n] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int QB = NF >= 4 ? 1 : 4 / NF;  // contributors per batch: 4 loads in flight
    int64_t cc = c_lo;
    for (; cc + QB - 1 <= c_hi; cc += QB) {
        v4f p[QB][NF];
#pragma unroll
        for (int q = 0; q < QB; ++q) {
            const v4f* b = base(cc + q);
#pragma unroll
            for (int n = 0; n < NF; ++n) p[q][n] = sk_get(b + n * kThreadsP);
        }
#pragma unroll
        for (int q = 0; q < QB; ++q)
#pragma unroll
            for (int n = 0; n < NF; ++n)
#pragma unroll
                for (int e = 0; e < 4; ++e) sum[n][e] = sum[n][e] + p[q][n][e];
    }
    for (; cc <= c_hi; ++cc) {
        const v4f* b = base(cc);
#pragma unroll
        for (int n = 0; n < NF; ++n) {
            const v4f p = sk_get(b + n * kThreadsP);
#pragma unroll
            for (int e = 0; e < 4; ++e) sum[n][e] = sum[n][e] + p[e];
        }
    }
#pragma unroll
    for (int n = 0; n < NF; ++n) {
        const int col = wn * 32 + ((f0 + n) & 1) * 16 + 4 * lk;
        v4f v = sum[n];
        if constexpr (GRAN == GRAN_ROW) {
            const float sa = ct.sA[r];
            const v4f s4 = *reinterpret_cast<const v4f*>(ct.sW + col);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = v[e] * (sa * s4[e]);
        }
        uint2 o;
        o.x = bf16x2_rne(v[0], v[1]);
        o.y = bf16x2_rne(v[2], v[3]);
        *reinterpret_cast<uint2*>(ct.Y + (int64_t)r * S.N + col) = o;
    }
}

// Grid that deals whole tiles out evenly (n = ceil(tiles / 256) per
// workgroup) when that keeps at least 3/4 of the CUs busy, else 0 (stream-K).
// A split tile costs its partial stores and a second kernel that reads them
// back; at decode shapes the chip's bandwidth, not each CU's, bounds the
// GEMM, so idle CUs cost less (gate_up at M=256: 192 tiles on 192 CUs 46.7 µs,
// stream-K over 256 CUs with its reduce 52.4 µs).
__host__ inline int64_t whole_tile_grid(int64_t tiles) {
    const int64_t n = (tiles + kPersistentGrid - 1) / kPersistentGrid;
    return tiles % n == 0 && 4 * tiles >= 3 * kPersistentGrid * n ? tiles / n : 0;
}

// The wide reduce (one fragment per workgroup, four contributors' loads in
// flight) when each split tile has many contributors (ranges shorter than a
// quarter of a tile); with up to four contributors a tile's reduce is short
// and the narrow form, with fewer workgroups to start, is faster.
__host__ inline bool reduce_wide(int64_t steps, int64_t grid, int64_t KB) {
    return 4 * (steps / grid) < KB;
}

// ---------------------------------------------------------------------------
// Stream-K small-M kernel on 256 x 128 tiles (128 < M on the small-M path).
// A 128-row tile reads a weight block once per row tile, so at M = 256 every
// weight byte is fetched twice (the second time from the Infinity Cache at
// best); the 256-row tile fetches it once and halves the K steps.  512
// threads as 4 x 2 waves of 64 x 64 (wave w: rows 64 (w & 3), columns
// 64 (w >> 2)); a ring of 3 stages (two in flight, 96 KiB) of 48 KiB operands
// plus scales, filled by direct-to-LDS buffer loads (K <= 2^22).  Ranges,
// partial slots and the fixed-order reduce work as in k_gemm_sk, with
// 256 x 128 fp32 slots (v4f index (slot * 16 + i * 4 + jj) * 512 + tid).
// ---------------------------------------------------------------------------
constexpr int BMD = 256, NSD = 3;
constexpr int kSaD = (BMD + BNP) * BK;        // 48 KiB of operands, then the 256 row scales
constexpr int kSwD = kSaD + BMD * 4;          // the block scale (64 copies of one word)
constexpr int kStageD = kSwD + 256;
// SG (K / 128 % 4 == 0): the scales of 4 K blocks are loaded together, once
// per 4 steps, into a ring of two group slots after the stages: 256 rows x 16
// bytes (fp32; E8M0: 4 bytes per row) and 64 copies of the block scales.
constexpr int kGrpD = NSD * kStageD, kGrpSlotD = BMD * 16 + 1024;
constexpr int kLdsD = kGrpD + 2 * kGrpSlotD;
static_assert(kLdsD <= 160 * 1024, "gfx950 has 160 KiB of LDS per workgroup");
static_assert(kGemmWsMaxBytes >= kPersistentGrid * 2 * BMD * BNP * 4, "partial slots");

struct DkSrc {
    __amdgpu_buffer_rsrc_t a, w, sa, sw;
    int offa[4], offw[2], offsa;
};

// Tile `logical` of a dense space of ceil(M / 256) x N / 128 tiles, row tiles
// of one column tile adjacent.
template <int GRAN>
__device__ __forceinline__ Tile dk_tile(const TileSpace& S, int64_t logical) {
    const int64_t KB = S.K / BK;
    const int64_t tm = logical % S.tm_count, tn = logical / S.tm_count;
    const int64_t row0 = tm * BMD, n0 = tn * BNP;
    Tile t;
    t.rows = (int)((S.M - row0) < BMD ? (S.M - row0) : BMD);
    t.A = S.A + row0 * S.K;
    t.W = S.W + n0 * S.K;
    if constexpr (GRAN == GRAN_MX) {  // E8M0 bytes [M, KB] and [N/128, KB]
        t.sA = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(S.sA) + row0 * KB);
        t.sW = reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(S.sW) + tn * KB);
    } else {
        t.sA = GRAN == GRAN_BLOCK ? S.sA + row0 * KB : S.sA + row0;
        t.sW = GRAN == GRAN_BLOCK ? S.sW + tn * KB : S.sW + n0;
    }
    t.Y = S.Y + row0 * S.N + n0;
    return t;
}

template <int GRAN>
__device__ __forceinline__ void dk_src(DkSrc& s, const Tile& t, int K, int KB, int wave,
                                       int lane) {
    s.a = buffer_rsrc(t.A, t.rows * K);
    s.w = buffer_rsrc(t.W, BNP * K);
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // LDS chunk p holds chunk swz_pos(r, p % 8) of row r = p / 8
        const int p = (i * 8 + wave) * 64 + lane;
        const int r = p >> 3;
        const int ra = r < t.rows ? r : t.rows - 1;
        s.offa[i] = ra * K + swz_pos(r, p & 7) * 16;
        if (i < 2) s.offw[i] = r * K + swz_pos(r, p & 7) * 16;
    }
    if constexpr (GRAN == GRAN_BLOCK || GRAN == GRAN_MX) {
        constexpr int sb = GRAN == GRAN_MX ? 1 : 4;  // bytes per scale
        const int r = (wave & 3) * 64 + lane;
        const int rr = r < t.rows ? r : t.rows - 1;
        s.sa = buffer_rsrc(t.sA, t.rows * KB * sb);
        s.sw = buffer_rsrc(t.sW, KB * sb);
        s.offsa = rr * KB * sb;
    }
}

// Loads per stage per thread: 4 A chunks and 2 W chunks; with block or E8M0
// scales waves 0-3 also load the row scales (one gather of 64 rows each) and
// wave 4 the block scale.  A scale gather touches 64 cache lines, so it is
// issued once per row, not once per wave.
template <int GRAN>
__device__ __forceinline__ bool dk_scale_wave(int wave) {
    return (GRAN == GRAN_BLOCK || GRAN == GRAN_MX) && wave < 5;
}

// Stage st of K block kb; with SG, grp is the group slot to fill when this
// stage starts a scale group (null otherwise).
template <int GRAN, bool SG>
__device__ __forceinline__ void dk_stage(uint8_t* lds, int st, const DkSrc& s, int kb, int wave,
                                         uint8_t* grp) {
    uint8_t* la = lds + st * kStageD;
    uint8_t* lb = la + BMD * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) b2l(s.a, la + (i * 8 + wave) * 1024, 16, s.offa[i], kb * BK);
#pragma unroll
    for (int i = 0; i < 2; ++i) b2l(s.w, lb + (i * 8 + wave) * 1024, 16, s.offw[i], kb * BK);
    if constexpr (SG) {
        // fp32: 16 bytes (4 scales) per row; E8M0: 4 bytes, one 32-bit word
        constexpr int gb = GRAN == GRAN_MX ? 4 : 16;
        const int k0 = (kb & ~3) * (gb / 4);
        if (grp != nullptr) {
            if (wave < 4)
                b2l(s.sa, grp + wave * 64 * gb, gb, s.offsa, k0);
            else if (wave == 4)
                b2l(s.sw, grp + BMD * 16, gb, 0, k0);  // every lane the same bytes
        }
    } else if constexpr (GRAN == GRAN_BLOCK || GRAN == GRAN_MX) {
        // an E8M0 byte lands zero-extended in its lane's 32-bit word
        constexpr int sb = GRAN == GRAN_MX ? 1 : 4;
        if (wave < 4)
            b2l(s.sa, la + kSaD + wave * 256, sb, s.offsa, kb * sb);
        else if (wave == 4)
            b2l(s.sw, la + kSwD, sb, 0, kb * sb);  // every lane the same word
    }
}

// Wait for stage g: only stage g + 1 may stay in flight.  next_scale: stage
// g + 1 carries a scale load for this wave.
__device__ __forceinline__ void dk_wait(int g, int ng, bool next_scale) {
    if (g + 1 >= ng)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    else if (next_scale)  // wave-uniform
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(7));
    else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(6));
}

// This lane's scales for K block kb: BLOCK sc[i] = row scale x block scale,
// MX the E8M0 bytes (sa[i], sw); from the stage (SG false) or the group slot.
template <int GRAN, bool SG>
__device__ __forceinline__ void dk_scales(const uint8_t* la, const uint8_t* gp, int kb, int wm,
                                          int lr, float (&sc)[4], int (&sa)[4], int& sw) {
    if constexpr (GRAN == GRAN_BLOCK) {
        float w;
        if constexpr (SG) {
            w = *reinterpret_cast<const float*>(gp + BMD * 16 + (kb & 3) * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sc[i] = *reinterpret_cast<const float*>(gp + (wm * 64 + i * 16 + lr) * 16 +
                                                        (kb & 3) * 4) * w;
        } else {
            w = *reinterpret_cast<const float*>(la + kSwD);
            const float* lsa = reinterpret_cast<const float*>(la + kSaD);
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] = lsa[wm * 64 + i * 16 + lr] * w;
        }
    } else if constexpr (GRAN == GRAN_MX) {
        if constexpr (SG) {
            const int sh = (kb & 3) * 8;
            sw = (*reinterpret_cast<const int*>(gp + BMD * 16) >> sh) & 0xFF;
            const int* lsa = reinterpret_cast<const int*>(gp);
#pragma unroll
            for (int i = 0; i < 4; ++i) sa[i] = (lsa[wm * 64 + i * 16 + lr] >> sh) & 0xFF;
        } else {
            sw = *reinterpret_cast<const int*>(la + kSwD);
            const int* lsa = reinterpret_cast<const int*>(la + kSaD);
#pragma unroll
            for (int i = 0; i < 4; ++i) sa[i] = lsa[wm * 64 + i * 16 + lr];
        }
    }
}

// One K step of a wave's 64 x 64 block from stage `la` (promotion as in
// pipe_mma: each product's FMAs trail its MFMA by one).
template <int GRAN, bool SG>
__device__ __forceinline__ void dk_mma(const uint8_t* la, const uint8_t* gp, int kb,
                                       v4f (&acc)[4][4], int wm, int wn, int lr, int lk) {
    const uint8_t* lb = la + BMD * BK;
    v8i x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = frag(la, wm * 64 + i * 16 + lr, lk);
    float sc[4];
    int sa[4] = {0, 0, 0, 0}, sw = 0;
    dk_scales<GRAN, SG>(la, gp, kb, wm, lr, sc, sa, sw);
    if constexpr (GRAN == GRAN_BLOCK) {
        const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
        v8i wcur = frag(lb, wn * 64 + lr, lk);
        v4f prev;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            v8i wnext = wcur;
            if (jj < 3) wnext = frag(lb, wn * 64 + (jj + 1) * 16 + lr, lk);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const v4f pk = mfma_f8(wcur, x[i], zero);
                if (i > 0 || jj > 0) {
                    const int pi = i > 0 ? i - 1 : 3, pj = i > 0 ? jj : jj - 1;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[pi][pj][e] = __builtin_fmaf(prev[e], sc[pi], acc[pi][pj][e]);
                }
                prev = pk;
            }
            wcur = wnext;
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[3][3][e] = __builtin_fmaf(prev[e], sc[3], acc[3][3][e]);
    } else {
        v8i wcur = frag(lb, wn * 64 + lr, lk);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            v8i wnext = wcur;
            if (jj < 3) wnext = frag(lb, wn * 64 + (jj + 1) * 16 + lr, lk);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (GRAN == GRAN_MX)
                    acc[i][jj] = mfma_mx(wcur, x[i], acc[i][jj], sw, sa[i]);
                else
                    acc[i][jj] = mfma_f8(wcur, x[i], acc[i][jj]);
            }
            wcur = wnext;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// bf16 store of a wave's row fragment i (rows wm * 64 + 16 i + lr, 64
// columns); ROW scales by the row and column scales first.
template <int GRAN>
__device__ __forceinline__ void dk_store_frag(const Tile& ct, const v4f (&v4)[4], int64_t N,
                                              int r, int wn, int lk) {
    if (r >= ct.rows) return;
    float sa = 1.0f;
    if constexpr (GRAN == GRAN_ROW) sa = ct.sA[r];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        v4f v = v4[jj];
        if constexpr (GRAN == GRAN_ROW) {
            const v4f s4 = *reinterpret_cast<const v4f*>(ct.sW + wn * 64 + jj * 16 + 4 * lk);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = v[e] * (sa * s4[e]);
        }
        uint2 o;
        o.x = bf16x2_rne(v[0], v[1]);
        o.y = bf16x2_rne(v[2], v[3]);
        *reinterpret_cast<uint2*>(ct.Y + (int64_t)r * N + wn * 64 + jj * 16 + 4 * lk) = o;
    }
}

template <int GRAN, bool SG>
__global__ __launch_bounds__(kThreadsP) void k_gemm_dk(TileSpace S, int64_t tiles, SkWork ws) {
    args_ready(S, tiles, ws.part, gridDim.x);
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsD];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 3, wn = wave >> 2;
    const int lr = lane & 15, lk = lane >> 4;
    const int64_t KB = S.K / BK, Wt = tiles * KB, G = gridDim.x;
    // XCD-contiguous rank, as in k_gemm_sk
    const int64_t bid = blockIdx.x, xcd = bid & 7;
    const int64_t q8 = G >> 3, r8 = G & 7;
    const int64_t c = xcd * q8 + (xcd < r8 ? xcd : r8) + (bid >> 3);
    const int64_t u0 = sk_start(c, Wt, G), u1 = sk_start(c + 1, Wt, G);
    const int ng = (int)(u1 - u0);
    if (ng <= 0) return;  // whole workgroup leaves together
    const int64_t t_first = u0 / KB;
    const int K = (int)S.K, kbn = (int)KB;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    int64_t l_t = t_first;  // tile and k block of the next stage to load
    int l_kb = (int)(u0 - t_first * KB);
    DkSrc src;
    dk_src<GRAN>(src, dk_tile<GRAN>(S, l_t), K, kbn, wave, lane);
    // SG: scale groups loaded (gl) and in use (gc); a group starts at a K block
    // that is a multiple of 4 or at the first step of the range
    int gl = 0, gc = -1;
    auto group_slot = [&](bool starts) -> uint8_t* {
        if (!SG || !starts) return nullptr;
        return lds + kGrpD + ((gl++) & 1) * kGrpSlotD;
    };
#pragma unroll
    for (int st = 0; st < NSD - 1; ++st) {
        if (st < ng) {
            dk_stage<GRAN, SG>(lds, st, src, l_kb, wave, group_slot(st == 0 || (l_kb & 3) == 0));
            if (++l_kb == kbn) {
                l_kb = 0;
                ++l_t;
                if (l_t < tiles) dk_src<GRAN>(src, dk_tile<GRAN>(S, l_t), K, kbn, wave, lane);
            }
        }
    }
    int64_t c_t = t_first;  // tile being multiplied, its k block, where this range entered it
    int kb = (int)(u0 - t_first * KB);
    int kb_in = kb;
    Tile ct = dk_tile<GRAN>(S, c_t);

    for (int g = 0; g < ng; ++g) {
        asm volatile("" ::: "memory");
        {
            const int kb1 = kb + 1 == kbn ? 0 : kb + 1;  // K block of stage g + 1
            dk_wait(g, ng, dk_scale_wave<GRAN>(wave) && (!SG || (kb1 & 3) == 0));
        }
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (g + NSD - 1 < ng) {  // refill the stage consumed at g - 1
            dk_stage<GRAN, SG>(lds, (g + NSD - 1) % NSD, src, l_kb, wave,
                               group_slot((l_kb & 3) == 0));
            if (++l_kb == kbn) {
                l_kb = 0;
                ++l_t;
                if (l_t < tiles) dk_src<GRAN>(src, dk_tile<GRAN>(S, l_t), K, kbn, wave, lane);
            }
        }
        if (g == 0 || (kb & 3) == 0) ++gc;
        dk_mma<GRAN, SG>(lds + (g % NSD) * kStageD, lds + kGrpD + (gc & 1) * kGrpSlotD, kb, acc,
                         wm, wn, lr, lk);

        if (kb == kbn - 1 || g == ng - 1) {  // this range's part of tile c_t is done
            if (kb_in == 0 && kb == kbn - 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dk_store_frag<GRAN>(ct, acc[i], S.N, wm * 64 + i * 16 + lr, wn, lk);
            } else {
                const int slot = (c_t == t_first) ? 0 : 1;
                v4f* mine = ws.part + (c * 2 + slot) * 16 * kThreadsP + tid;
                const int wrows = ct.rows - wm * 64;  // rows of this wave that exist
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (i * 16 + lr < wrows)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            sk_put(mine + (i * 4 + jj) * kThreadsP, acc[i][jj]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc[i][jj] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        }
        if (++kb == kbn) {
            kb = 0;
            kb_in = 0;
            ++c_t;
            if (c_t < tiles) ct = dk_tile<GRAN>(S, c_t);
        }
    }
}

// Sum of the partials of each split 256 x 128 tile in contributor order, then
// the bf16 store; 4 workgroups per tile, workgroup i taking row fragment i of
// every wave.
template <int GRAN>
__global__ __launch_bounds__(kThreadsP) void k_dk_reduce(TileSpace S, int64_t tiles, int64_t G,
                                                        const v4f* __restrict__ part) {
    args_ready(S, tiles, G, part);
    const int64_t t = blockIdx.x >> 2, KB = S.K / BK, Wt = tiles * KB;
    const int i = (int)(blockIdx.x & 3);
    const int64_t c_lo = sk_owner(t * KB, Wt, G), c_hi = sk_owner(t * KB + KB - 1, Wt, G);
    if (c_lo == c_hi) return;  // stored whole by its workgroup
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 3, wn = wave >> 2, lr = lane & 15, lk = lane >> 4;
    const Tile ct = dk_tile<GRAN>(S, t);
    const int r = wm * 64 + i * 16 + lr;
    if (r >= ct.rows) return;
    v4f sum[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) sum[jj] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t cc = c_lo; cc <= c_hi; ++cc) {
        const int sl = (sk_start(cc, Wt, G) / KB == t) ? 0 : 1;
        const v4f* pp = part + (cc * 2 + sl) * 16 * kThreadsP + tid;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const v4f p = sk_get(pp + (i * 4 + jj) * kThreadsP);
#pragma unroll
            for (int e = 0; e < 4; ++e) sum[jj][e] = sum[jj][e] + p[e];
        }
    }
    dk_store_frag<GRAN>(ct, sum, S.N, r, wn, lk);
}

// k_dk_reduce for tiles with many contributors: SPLIT workgroups per tile,
// each taking NF = 16 / SPLIT of the sixteen fragments (i * 4 + jj) of every
// wave, as k_sk_reduce_wide does.
template <int GRAN, int SPLIT>
__global__ __launch_bounds__(kThreadsP) void k_dk_reduce_wide(TileSpace S, int64_t tiles, int64_t G,
                                                        const v4f* __restrict__ part) {
    args_ready(S, tiles, G, part);
    constexpr int NF = 16 / SPLIT;
    const int64_t t = blockIdx.x / SPLIT, KB = S.K / BK, Wt = tiles * KB;
    const int f0 = (int)(blockIdx.x % SPLIT) * NF;
    const int64_t c_lo = sk_owner(t * KB, Wt, G), c_hi = sk_owner(t * KB + KB - 1, Wt, G);
    if (c_lo == c_hi) return;  // stored whole by its workgroup
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 3, wn = wave >> 2, lr = lane & 15, lk = lane >> 4;
    const Tile ct = dk_tile<GRAN>(S, t);
    const int r = wm * 64 + (f0 >> 2) * 16 + lr;  // the NF fragments share a row
    if (r >= ct.rows) return;
    // contributor cc's partial slot (0 if its range starts in tile t), at this
    // thread's first fragment
    auto base = [&](int64_t cc) {
        const int sl = (sk_start(cc, Wt, G) / KB == t) ? 0 : 1;
        return part + (cc * 2 + sl) * 16 * kThreadsP + f0 * kThreadsP + tid;
    };
    v4f sum[NF];
#pragma unroll
    for (int n = 0; n < NF; ++n) sum[n] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int QB = NF >= 4 ? 1 : 4 / NF;  // contributors per batch: 4 loads in flight
    int64_t cc = c_lo;
    for (; cc + QB - 1 <= c_hi; cc += QB) {
        v4f p[QB][NF];
#pragma unroll
        for (int q = 0; q < QB; ++q) {
            const v4f* b = base(cc + q);
#pragma unroll
            for (int n = 0; n < NF; ++n) p[q][n] = sk_get(b + n * kThreadsP);
        }
#pragma unroll
        for (int q = 0; q < QB; ++q)
#pragma unroll
            for (int n = 0; n < NF; ++n)
#pragma unroll
                for (int e = 0; e < 4; ++e) sum[n][e] = sum[n][e] + p[q][n][e];
    }
    for (; cc <= c_hi; ++cc) {
        const v4f* b = base(cc);
#pragma unroll
        for (int n = 0; n < NF; ++n) {
            const v4f p = sk_get(b + n * kThreadsP);
#pragma unroll
            for (int e = 0; e < 4; ++e) sum[n][e] = sum[n][e] + p[e];
        }
    }
#pragma unroll
    for (int n = 0; n < NF; ++n) {
        const int col = wn * 64 + ((f0 + n) & 3) * 16 + 4 * lk;
        v4f v = sum[n];
        if constexpr (GRAN == GRAN_ROW) {
            const float sa = ct.sA[r];
            const v4f s4 = *reinterpret_cast<const v4f*>(ct.sW + col);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = v[e] * (sa * s4[e]);
        }
        uint2 o;
        o.x = bf16x2_rne(v[0], v[1]);
        o.y = bf16x2_rne(v[2], v[3]);
        *reinterpret_cast<uint2*>(ct.Y + (int64_t)r * S.N + col) = o;
    }
}

// ---------------------------------------------------------------------------
// Diagnostic: the matrix-core rate with operands in registers.  Every wave
// runs `iters` rounds of 8 independent 16 x 16 x 128 E4M3 MFMAs (8
// accumulator chains), so with 4 waves per SIMD the matrix cores never wait
// on a dependency; the operands are fixed finite E4M3 patterns that vary by
// lane.  out[wave] receives a sum of the accumulators (keeps the work live).
// 2 * 16 * 16 * 128 flops per MFMA.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_mfma_probe(int64_t iters, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // bytes below 0x78 in magnitude: finite E4M3 values, never NaN
        const uint32_t h = (uint32_t)(lane * 2654435761u + i * 40503u);
        a[i] = (int)(h & 0x37373737u);
        b[i] = (int)((h >> 3) & 0x37373737u);
    }
    v4f acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = mfma_f8(a, b, acc[j]);
    }
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) t += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (lane == 0) out[wave] = t;
}

}  // namespace

// The large-M kernel addresses a tile with 32-bit buffer offsets (256 rows x
// K bytes, so K <= 2^22) and counts tiles and steps in int.  It takes M >=
// 1024, and smaller M when the 256 x 256 tiles alone fill most of the chip
// (>= 192 of them: e.g. the gate_up projection at M = 512 runs 30% faster
// than on the small-M kernel).
bool gemm_small_path(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles2 = ((M + BM2 - 1) / BM2) * (N / BN2);
    return !((M >= 1024 || tiles2 >= 192) && N % BN2 == 0 && K <= (int64_t(1) << 22) &&
             (tiles2 / 256 + 1) * (K / BK) < (int64_t(1) << 31));
}

// Launch plan of the small-M GEMM of a dense tile space.  Without a split
// there are no partials: the 256 x 128 kernel when the tiles' whole grid fills
// the chip, else the 128 x 128 one, else one tile per workgroup at a time.
// With a workspace of at least ws_bytes, tiles are split between workgroups
// (stream-K) and a second kernel sums the partials.
enum { SP_PIPE = 0, SP_SK = 1, SP_DK = 2 };
struct SmallPlan {
    int kind;
    int64_t tm_count;  // row tiles (128 or 256 rows)
    int64_t tiles, steps, grid;
    bool split;        // some tile is cut between workgroups
    int64_t ws_bytes;  // workspace the split needs (0 without a split)
};

static SmallPlan plan_small(int64_t M, int64_t N, int64_t K, bool with_ws) {
    SmallPlan p{};
    const int64_t KB = K / BK;
    const bool buf = K <= (int64_t(1) << 22);  // 256 rows x K bytes fit 32-bit buffer offsets
    if (M > BMP && buf) {  // 256-row tiles: each weight block read once
        const int64_t tm = (M + BMD - 1) / BMD, tiles = tm * (N / BNP), steps = tiles * KB;
        // with fewer than 8 K steps per workgroup the larger stages' fill and
        // partials cost more than the second weight read saves
        if (steps >= 8 * kPersistentGrid && tiles <= kGemmWsMaxTiles &&
            steps < (int64_t(1) << 31)) {
            const int64_t whole = whole_tile_grid(tiles);
            if (whole > 0 || with_ws) {
                p.kind = SP_DK;
                p.tm_count = tm; p.tiles = tiles; p.steps = steps;
                p.grid = whole > 0 ? whole : (steps < kPersistentGrid ? steps : kPersistentGrid);
                p.split = steps % p.grid != 0 || (steps / p.grid) % KB != 0;
                p.ws_bytes = p.split ? p.grid * 2 * BMD * BNP * 4 : 0;
                return p;
            }
        }
    }
    const int64_t tm = (M + BMP - 1) / BMP, tiles = tm * (N / BNP), steps = tiles * KB;
    p.tm_count = tm; p.tiles = tiles; p.steps = steps;
    if (tiles <= kGemmWsMaxTiles && steps < (int64_t(1) << 31)) {
        // stream-K: every workgroup gets at least one K step (grid <= steps),
        // or whole tiles when they fill the chip evenly
        const int64_t whole = whole_tile_grid(tiles);
        if (whole > 0 || with_ws) {
            p.kind = SP_SK;
            p.grid = whole > 0 ? whole : (steps < kPersistentGrid ? steps : kPersistentGrid);
            p.split = steps % p.grid != 0 || (steps / p.grid) % KB != 0;
            p.ws_bytes = p.split ? p.grid * 2 * BMP * BNP * 4 : 0;
            return p;
        }
    }
    p.kind = SP_PIPE;
    p.grid = tiles < kPersistentGrid ? tiles : kPersistentGrid;
    return p;
}

// The plan a call runs: the split plan when the workspace holds its partials,
// else the plan without a split.
static SmallPlan plan_small_ws(int64_t M, int64_t N, int64_t K, const GemmWorkspace* ws) {
    const SmallPlan p = plan_small(M, N, K, true);
    if (!p.split || (ws != nullptr && ws->part != nullptr && ws->bytes >= p.ws_bytes)) return p;
    return plan_small(M, N, K, false);
}

// The small-M GEMM of a dense tile space (see plan_small).  MX shapes always
// take buffer loads (B K <= 2^22).
template <int G>
static hipError_t launch_small(TileSpace S, const GemmWorkspace* ws, hipStream_t st) {
    const int64_t K = S.K;
    const SmallPlan p = plan_small_ws(S.M, S.N, K, ws);
    const bool buf = K <= (int64_t(1) << 22);  // 128 rows x K bytes fit 32-bit buffer offsets
    S.tm_count = p.tm_count;
    const SkWork sk{p.split ? static_cast<v4f*>(ws->part) : nullptr};
    if (p.kind == SP_DK) {
        // scale groups of 4 K blocks: whole groups per row, aligned group loads
        const int64_t salign = G == GRAN_MX ? 4 : 16;
        const bool sg = G != GRAN_ROW && (K / BK) % 4 == 0 &&
                        reinterpret_cast<uintptr_t>(S.sA) % salign == 0 &&
                        reinterpret_cast<uintptr_t>(S.sW) % salign == 0;
        if constexpr (G != GRAN_ROW)
            if (sg)
                hipLaunchKernelGGL((k_gemm_dk<G, true>), dim3((unsigned)p.grid), dim3(kThreadsP),
                                   0, st, S, p.tiles, sk);
        if (!sg)
            hipLaunchKernelGGL((k_gemm_dk<G, false>), dim3((unsigned)p.grid), dim3(kThreadsP), 0,
                               st, S, p.tiles, sk);
        if (hipError_t e = hipGetLastError()) return e;
        if (p.split) {
            if (reduce_wide(p.steps, p.grid, K / BK))
                hipLaunchKernelGGL((k_dk_reduce_wide<G, 16>), dim3((unsigned)(p.tiles * 16)),
                                   dim3(kThreadsP), 0, st, S, p.tiles, p.grid,
                                   static_cast<const v4f*>(sk.part));
            else
                hipLaunchKernelGGL(k_dk_reduce<G>, dim3((unsigned)(p.tiles * 4)), dim3(kThreadsP),
                                   0, st, S, p.tiles, p.grid, static_cast<const v4f*>(sk.part));
        }
        return hipGetLastError();
    }
    if (p.kind == SP_SK) {
        if (G == GRAN_MX || buf)
            hipLaunchKernelGGL((k_gemm_sk<G, true>), dim3((unsigned)p.grid), dim3(kThreadsP), 0,
                               st, S, p.tiles, sk);
        else if constexpr (G != GRAN_MX)
            hipLaunchKernelGGL((k_gemm_sk<G, false>), dim3((unsigned)p.grid), dim3(kThreadsP), 0,
                               st, S, p.tiles, sk);
        if (hipError_t e = hipGetLastError()) return e;
        if (p.split) {
            if (reduce_wide(p.steps, p.grid, K / BK))
                hipLaunchKernelGGL((k_sk_reduce_wide<G, 8>), dim3((unsigned)(p.tiles * 8)),
                                   dim3(kThreadsP), 0, st, S, p.tiles, p.grid,
                                   static_cast<const v4f*>(sk.part));
            else
                hipLaunchKernelGGL(k_sk_reduce<G>, dim3((unsigned)(p.tiles * kSkRedSplit)),
                                   dim3(kThreadsP), 0, st, S, p.tiles, p.grid,
                                   static_cast<const v4f*>(sk.part));
        }
        return hipGetLastError();
    }
    if (G == GRAN_MX || buf)
        hipLaunchKernelGGL((k_gemm_pipe<G, false, true>), dim3((unsigned)p.grid), dim3(kThreadsP),
                           0, st, S, p.tiles);
    else if constexpr (G != GRAN_MX)
        hipLaunchKernelGGL((k_gemm_pipe<G, false, false>), dim3((unsigned)p.grid),
                           dim3(kThreadsP), 0, st, S, p.tiles);
    return hipGetLastError();
}

int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || !gemm_small_path(M, N, K)) return 0;
    return plan_small(M, N, K, true).ws_bytes;
}

int64_t mx_workspace_bytes(int64_t B, int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || !mx_small_path(B, M, N)) return 0;
    return plan_small(M, N, K, true).ws_bytes;
}

hipError_t launch_gemm(const void* a, const void* w, const float* a_s, const float* w_s,
                       void* y, int64_t M, int64_t N, int64_t K, int gran,
                       const GemmWorkspace* ws, hipStream_t st) {
    if (M == 0) return hipSuccess;
    const auto* A = static_cast<const uint8_t*>(a);
    const auto* Wp = static_cast<const uint8_t*>(w);
    auto* Yp = static_cast<uint16_t*>(y);
    if (!gemm_small_path(M, N, K)) {
        const int64_t tiles2 = ((M + BM2 - 1) / BM2) * (N / BN2);
        const unsigned grid = (unsigned)(tiles2 < 256 ? tiles2 : 256);  // one per CU
        const BigGeom G{M, N, K, 1};
        // the ping-pong kernel addresses a tile's output rows with 32-bit
        // buffer offsets (256 rows x N bf16 < 2^31 bytes)
        if (gran == GRAN_BLOCK && N < (int64_t(1) << 22))
            hipLaunchKernelGGL(k_gemm_pp<GRAN_BLOCK>, dim3(grid), dim3(kThreads2), 0, st, A, Wp,
                               static_cast<const void*>(a_s), static_cast<const void*>(w_s), Yp,
                               G, nullptr, 0);
        else if (gran == GRAN_BLOCK)
            hipLaunchKernelGGL((k_gemm_big<GRAN_BLOCK, false>), dim3(grid), dim3(kThreads2), 0,
                               st, A, Wp, static_cast<const void*>(a_s),
                               static_cast<const void*>(w_s), Yp, G, nullptr, 0);
        else if (N < (int64_t(1) << 22))
            hipLaunchKernelGGL(k_gemm_pp<GRAN_ROW>, dim3(grid), dim3(kThreads2), 0, st, A, Wp,
                               static_cast<const void*>(a_s), static_cast<const void*>(w_s), Yp,
                               G, nullptr, 0);
        else
            hipLaunchKernelGGL((k_gemm_big<GRAN_ROW, false>), dim3(grid), dim3(kThreads2), 0,
                               st, A, Wp, static_cast<const void*>(a_s),
                               static_cast<const void*>(w_s), Yp, G, nullptr, 0);
        return hipGetLastError();
    }
    TileSpace S{};
    S.A = A; S.W = Wp; S.sA = a_s; S.sW = w_s; S.Y = Yp;
    S.M = M; S.N = N; S.K = K; S.E = 0;
    S.tm_count = (M + BMP - 1) / BMP;
    if (gran == GRAN_BLOCK) return launch_small<GRAN_BLOCK>(S, ws, st);
    return launch_small<GRAN_ROW>(S, ws, st);
}

hipError_t launch_grouped_gemm(const void* a, const void* w, const float* a_s, const float* w_s,
                               const int32_t* offsets, void* y, int64_t T, int64_t E,
                               int64_t N, int64_t K, hipStream_t st) {
    if (T == 0) return hipSuccess;
    TileSpace S{};
    S.A = static_cast<const uint8_t*>(a);
    S.W = static_cast<const uint8_t*>(w);
    S.sA = a_s; S.sW = w_s;
    S.Y = static_cast<uint16_t*>(y);
    S.offsets = offsets;
    S.M = T; S.N = N; S.K = K; S.E = E;
    // Experts with a few hundred rows each fill 256-row tiles: the large-M
    // kernel then reads each operand byte from LDS half as often as the
    // 128 x 128 tiles do.  Its buffer offsets need K <= 2^22, and the tile and
    // step counts (at most ceil(T/256) + E row tiles) must fit in int.
    const int64_t max_tiles = (T / BM2 + E) * ((N + BN2 - 1) / BN2);
    if (T >= 192 * E && K <= (int64_t(1) << 22) && max_tiles < (int64_t(1) << 31) &&
        (max_tiles / 256 + 1) * (K / BK) < (int64_t(1) << 31)) {
        const BigGeom G{T, N, K, 1};
        if (N % BN2 == 0 && N < (int64_t(1) << 22)) {  // full tiles: the ping-pong kernel
            hipLaunchKernelGGL((k_gemm_pp<GRAN_BLOCK, true>), dim3((unsigned)kPersistentGrid),
                               dim3(kThreads2), 0, st, S.A, S.W, static_cast<const void*>(a_s),
                               static_cast<const void*>(w_s), S.Y, G, offsets, (int)E);
            return hipGetLastError();
        }
        hipLaunchKernelGGL((k_gemm_big<GRAN_BLOCK, true>), dim3((unsigned)kPersistentGrid),
                           dim3(kThreads2), 0, st, S.A, S.W, static_cast<const void*>(a_s),
                           static_cast<const void*>(w_s), S.Y, G, offsets, (int)E);
        return hipGetLastError();
    }
    if (K <= (int64_t(1) << 22))
        hipLaunchKernelGGL((k_gemm_pipe<GRAN_BLOCK, true, true>), dim3((unsigned)kPersistentGrid),
                           dim3(kThreadsP), 0, st, S, (int64_t)0);
    else
        hipLaunchKernelGGL((k_gemm_pipe<GRAN_BLOCK, true, false>), dim3((unsigned)kPersistentGrid),
                           dim3(kThreadsP), 0, st, S, (int64_t)0);
    return hipGetLastError();
}

bool mx_small_path(int64_t B, int64_t M, int64_t N) {
    const int64_t tiles2 = ((M + BM2 - 1) / BM2) * ((N + BN2 - 1) / BN2);
    return B == 1 && M < 1024 && tiles2 < 192;
}

hipError_t launch_batched_gemm_mx(const void* a, const void* w, const uint8_t* a_s,
                                  const uint8_t* w_s, void* y, int64_t B, int64_t M, int64_t N,
                                  int64_t K, const GemmWorkspace* ws, hipStream_t st) {
    if (M == 0 || B == 0) return hipSuccess;
    if (mx_small_path(B, M, N)) {  // dense small M: the 128 x 128 kernels
        TileSpace S{};
        S.A = static_cast<const uint8_t*>(a);
        S.W = static_cast<const uint8_t*>(w);
        S.sA = reinterpret_cast<const float*>(a_s);  // E8M0 bytes, addressed as bytes
        S.sW = reinterpret_cast<const float*>(w_s);
        S.Y = static_cast<uint16_t*>(y);
        S.M = M; S.N = N; S.K = K; S.E = 0;
        S.tm_count = (M + BMP - 1) / BMP;
        return launch_small<GRAN_MX>(S, ws, st);
    }
    const int64_t tiles = B * ((M + BM2 - 1) / BM2) * ((N + BN2 - 1) / BN2);
    const unsigned grid = (unsigned)(tiles < 256 ? tiles : 256);  // one per CU
    const BigGeom G{M, N, K, (int)B};
    // full 256-column tiles: the ping-pong kernel (32-bit offsets into 256
    // output rows of B N bf16, batch-major tiles)
    if (N % BN2 == 0 && B * N < (int64_t(1) << 22)) {
        hipLaunchKernelGGL(k_gemm_pp<GRAN_MX>, dim3(grid), dim3(kThreads2), 0, st,
                           static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(w),
                           static_cast<const void*>(a_s), static_cast<const void*>(w_s),
                           static_cast<uint16_t*>(y), G, nullptr, 0);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_gemm_big<GRAN_MX, false>), dim3(grid), dim3(kThreads2), 0, st,
                       static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(w),
                       static_cast<const void*>(a_s), static_cast<const void*>(w_s),
                       static_cast<uint16_t*>(y), G, nullptr, 0);
    return hipGetLastError();
}

// 1024 workgroups of 4 waves: 4 waves per SIMD on 256 CUs.
hipError_t launch_mfma_probe(int64_t iters, float* out, hipStream_t st) {
    hipLaunchKernelGGL(k_mfma_probe, dim3(kMfmaProbeWorkgroups), dim3(256), 0, st, iters, out);
    return hipGetLastError();
}

}  // namespace fp8k
