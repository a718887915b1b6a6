// quant.hip -- memory-bound FP8 quantizers for gfx950.
//
// Pages (title, section):
//   "FP8-RL: A Practical and Stable Low-Precision Stack for LLM RL", abstract
//     (i): blockwise FP8 quantization of linear-layer inputs and weights, and
//     per-RL-step re-quantization of the policy weights.
//   "[vllm] feat: Support online quant for rollout with torchao", "Test":
//     per-row dynamic scales, e4m3fn operands, no activation value bounds.
//   "[vllm] [ROCm] DeepSeek V4 ... FP8 WO_A ...", §1 E8M0 scales, §2 the
//     (groups, out/128, in/128) block-scale view, §3 group-128 quantization.
//   "[sglang] SGLang의 AMD GPU 최적화: RMSNorm과 FP8 Per-token Quantization 커널
//     융합", §1 RMSNorm fused with per-token quantization in registers, so the
//     normalized tensor never makes an HBM round trip.
//
// Every kernel streams bf16 through 16-byte loads (8 elements per lane), keeps
// a group in registers, reduces |x| with cross-lane max, computes the group
// scale s = amax / 448 with one IEEE division, and encodes each element from
// the correctly rounded quotient x / s (quotient.hpp) with the hardware E4M3
// conversion (device.hpp).
#include <hip/hip_runtime.h>

#include "device.hpp"
#include "launch.hpp"
#include "tensor.hpp"
#include "quotient.hpp"

namespace fp8k {
namespace {

// Encoder state of one group: its scale and how to divide by it.
struct GroupDiv {
    float s;     // stored scale amax / 448 (0 for an all-zero group)
    float r;     // RN(1 / s) when the reciprocal path applies
    float d;     // IEEE divisor otherwise (1 for an all-zero group: codes are +-0)
    bool fast;
};

__device__ __forceinline__ GroupDiv group_div(float amax) {
    GroupDiv g;
    g.s = amax / 448.0f;
    g.fast = fp8q::scale_has_fast_path(g.s);
    g.r = g.fast ? 1.0f / g.s : 0.0f;
    g.d = (g.s == 0.0f) ? 1.0f : g.s;
    return g;
}

// Load vector idx of an n-vector array, or zeros when idx >= n, without a
// branch: the address is clamped to the last vector (always in bounds) and the
// value selected afterwards.  A branch around each load makes the compiler
// wait for every load before issuing the next one.
__device__ __forceinline__ uint4 load_or_zero(const uint4* __restrict__ p, int64_t idx, int64_t n) {
    const uint4 t = p[idx < n ? idx : n - 1];
    const bool in = idx < n;
    return make_uint4(in ? t.x : 0u, in ? t.y : 0u, in ? t.z : 0u, in ? t.w : 0u);
}

// Non-temporal 16-byte load and 8-byte store (streamed data: no cache
// allocation).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(static_cast<const u4*>(p)));
}
__device__ __forceinline__ void store_nt8(void* p, uint2 v) {
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(__builtin_bit_cast(u2, v), static_cast<u2*>(p));
}
// load_or_zero with a non-temporal load
__device__ __forceinline__ uint4 load_or_zero_nt(const uint4* __restrict__ p, int64_t idx,
                                                 int64_t n) {
    const uint4 t = load_nt16(p + (idx < n ? idx : n - 1));
    const bool in = idx < n;
    return make_uint4(in ? t.x : 0u, in ? t.y : 0u, in ? t.z : 0u, in ? t.w : 0u);
}

__device__ __forceinline__ uint2 encode8(const float (&f)[8], const GroupDiv& g) {
    float t[8];
    if (g.fast) {
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = fp8q::quotient(f[i], g.s, g.r);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = f[i] / g.d;
    }
    return e4m3x8(t);
}

// E8M0 exponent of an fp32 scale: ceil(log2 s) from its bits, clamped to
// [-127, 127] (-127 for s == 0).
__device__ __forceinline__ int e8m0_exponent(float s) {
    const uint32_t u = __float_as_uint(s) & 0x7FFFFFFFu;
    int e;
    if (u == 0) return -127;
    const int eb = (int)(u >> 23);
    const uint32_t m = u & 0x7FFFFFu;
    if (eb == 0)  // subnormal: s = m * 2^-149; ceil(log2 m) - 149
        e = (m == 1u ? 0 : 32 - __clz((int)(m - 1u))) - 149;
    else
        e = eb - 127 + (m != 0u ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^-e as a float for the exponents bf16 data can produce (e <= 120, so
// 127 - e >= 7 and 2^-e is a normal number): x * 2^-e == x / 2^e exactly.
__device__ __forceinline__ float e8m0_inv(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// ---------------------------------------------------------------------------
// 1x128 groups.  The M x K/128 groups are contiguous 256-byte runs in memory,
// so the kernel treats x as a flat array of groups: a wave covers 4 groups
// (16 lanes x 16 bytes each) per step and takes U steps, all loads issued
// before any compute.  x is read and the codes written non-temporally (a
// stream: 4.5 -> 4.9 TB/s at K = 4096, 5.5 -> 6.1 at K = 12288).
// ---------------------------------------------------------------------------
// FMT 0: fp32 scale amax / 448; FMT 1: E8M0 byte e + 127, e the ceiling
// exponent of that scale, elements encoded from x * 2^-e.
template <int U, int FMT>
__global__ __launch_bounds__(256) void k_quant_block(const uint4* __restrict__ x,
                                                     uint2* __restrict__ q,
                                                     void* __restrict__ s, int64_t G) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t chunk0 = wave * U;
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        v[u] = load_or_zero_nt(x, (chunk0 + u) * 64 + lane, G * 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t gid = (chunk0 + u) * 4 + (lane >> 4);
        float f[8];
        unpack8(v[u], f);
        const float amax = max_16lanes(amax8(f));
        if constexpr (FMT == 0) {
            const GroupDiv g = group_div(amax);
            if (gid < G) {
                store_nt8(q + (chunk0 + u) * 64 + lane, encode8(f, g));
                if ((lane & 15) == 0) static_cast<float*>(s)[gid] = g.s;
            }
        } else {
            const int e = e8m0_exponent(amax / 448.0f);
            const float inv = e8m0_inv(e);
            float t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) t[j] = f[j] * inv;
            if (gid < G) {
                store_nt8(q + (chunk0 + u) * 64 + lane, e4m3x8(t));
                if ((lane & 15) == 0) static_cast<uint8_t*>(s)[gid] = (uint8_t)(e + 127);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// One scale per row.  One wave per row; lane l holds the row's 8-element
// vectors l, l+64, l+128, ... in registers (VPL of them), so the row is read
// from HBM once (non-temporally).  VPL == 0 streams the row twice (rows
// longer than 32 * 512; those reads stay cached for the second pass).  Codes
// are stored non-temporally.
// ---------------------------------------------------------------------------
template <int VPL>
__global__ __launch_bounds__(256) void k_quant_token(const uint4* __restrict__ x,
                                                     uint2* __restrict__ q,
                                                     float* __restrict__ s, int64_t M,
                                                     int64_t V) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;  // whole wave leaves together
    const uint4* xr = x + row * V;
    uint2* qr = q + row * V;
    if constexpr (VPL > 0) {
        uint4 v[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) v[i] = load_or_zero_nt(xr, lane + 64 * i, V);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            float f[8];
            unpack8(v[i], f);
            m = fmaxf(m, amax8(f));
        }
        const GroupDiv g = group_div(max_wave(m));
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int64_t idx = lane + 64 * i;
            if (idx < V) {
                float f[8];
                unpack8(v[i], f);
                store_nt8(qr + idx, encode8(f, g));
            }
        }
        if (lane == 0) s[row] = g.s;
    } else {
        float m = 0.0f;
        for (int64_t idx = lane; idx < V; idx += 64) {
            float f[8];
            unpack8(xr[idx], f);
            m = fmaxf(m, amax8(f));
        }
        const GroupDiv g = group_div(max_wave(m));
        for (int64_t idx = lane; idx < V; idx += 64) {
            float f[8];
            unpack8(xr[idx], f);
            store_nt8(qr + idx, encode8(f, g));
        }
        if (lane == 0) s[row] = g.s;
    }
}

// ---------------------------------------------------------------------------
// One scale per row, one row per workgroup of 4 waves (rows of more than 128
// vectors): thread t holds vectors t, t + 256, ...; the row's amax is the max
// of the 4 waves' maxima (order-free).  Shorter chains per wave than one wave
// per row, so a CU's workgroups drift out of phase and loads overlap stores.
// ---------------------------------------------------------------------------
template <int VPL4>
__global__ __launch_bounds__(256) void k_token_row(const uint4* __restrict__ x,
                                                   uint2* __restrict__ q,
                                                   float* __restrict__ s, int64_t V) {
    __shared__ float red[4];
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;
    const uint4* xr = x + row * V;
    uint2* qr = q + row * V;
    uint4 v[VPL4];
#pragma unroll
    for (int k = 0; k < VPL4; ++k) v[k] = load_or_zero_nt(xr, t + 256 * k, V);
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL4; ++k) {
        float f[8];
        unpack8(v[k], f);
        m = fmaxf(m, amax8(f));
    }
    m = max_wave(m);
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    const GroupDiv g = group_div(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
#pragma unroll
    for (int k = 0; k < VPL4; ++k) {
        const int64_t idx = t + 256 * k;
        if (idx < V) {
            float f[8];
            unpack8(v[k], f);
            store_nt8(qr + idx, encode8(f, g));
        }
    }
    if (t == 0) s[row] = g.s;
}

// ---------------------------------------------------------------------------
// Fused RMSNorm + quantization, one wave per row.
//   sum of squares: lane l adds, in order, the squares of its vectors
//   l, l+64, ... (elements 8v .. 8v+7 in order), then the 64 lane partials are
//   combined by the halving tree; mean = S / K; inv = 1 / sqrt(mean + eps);
//   y = bf16_rne((x * inv) * gamma), all single fp32 operations (the library is
//   built without FMA contraction).  y stays in registers and is quantized per
//   row (GROUP == 0) or per 1x128 group (GROUP == 128): with vector v held by
//   lane v % 64, a 128-element group is 16 adjacent lanes of one step.
//   RES: a residual add comes first.  h = bf16_rne(x + r) (one fp32 add of
//   two bf16 values, whose bf16 rounding equals that of the exact sum) is
//   written back over r as the new residual stream and takes x's place in
//   everything after it.  x (read once) and the codes go non-temporally; r,
//   its write-back and gamma through the caches.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 add_bf16x8(const uint4& a, const uint4& b) {
    float fa[8], fb[8];
    unpack8(a, fa);
    unpack8(b, fb);
    uint4 o;
    o.x = bf16x2_rne(fa[0] + fb[0], fa[1] + fb[1]);
    o.y = bf16x2_rne(fa[2] + fb[2], fa[3] + fb[3]);
    o.z = bf16x2_rne(fa[4] + fb[4], fa[5] + fb[5]);
    o.w = bf16x2_rne(fa[6] + fb[6], fa[7] + fb[7]);
    return o;
}

__device__ __forceinline__ void rms_y8(const uint4& xv, const uint4& gv, float inv,
                                       float (&y)[8]) {
    float f[8], g[8];
    unpack8(xv, f);
    unpack8(gv, g);
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
        const uint32_t p = bf16x2_rne((f[j] * inv) * g[j], (f[j + 1] * inv) * g[j + 1]);
        y[j] = bf16_lo(p);
        y[j + 1] = bf16_hi(p);
    }
}

__device__ __forceinline__ uint4 pack_bf16x8(const float (&y)[8]) {
    // y already holds bf16 values; keep their upper halves
    uint4 o;
    o.x = (__float_as_uint(y[0]) >> 16) | (__float_as_uint(y[1]) & 0xFFFF0000u);
    o.y = (__float_as_uint(y[2]) >> 16) | (__float_as_uint(y[3]) & 0xFFFF0000u);
    o.z = (__float_as_uint(y[4]) >> 16) | (__float_as_uint(y[5]) & 0xFFFF0000u);
    o.w = (__float_as_uint(y[6]) >> 16) | (__float_as_uint(y[7]) & 0xFFFF0000u);
    return o;
}

__device__ __forceinline__ float sumsq8(float p, const uint4& xv) {
    float f[8];
    unpack8(xv, f);
#pragma unroll
    for (int j = 0; j < 8; ++j) p = p + f[j] * f[j];
    return p;
}

// Waves per SIMD asked of the register allocator: rows held in registers
// (VPL vectors per lane, twice that while x and the residual are both live)
// need room, and 4 waves per SIMD keep enough loads in flight.
constexpr int rms_waves(int vpl, bool res) {
    return vpl > 10 ? 1 : (res && vpl >= 8) ? 3 : 4;
}

template <int VPL, int GROUP, bool RES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(rms_waves(VPL, RES)))) void k_rmsnorm_quant(uint2* __restrict__ q,
                                                       const uint4* __restrict__ x,
                                                       uint4* __restrict__ res,
                                                       float* __restrict__ s,
                                                       const uint4* __restrict__ gamma,
                                                       float eps, int64_t M, int64_t V) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    const uint4* xr = x + row * V;
    uint4* rr = RES ? res + row * V : nullptr;
    uint2* qr = q + row * V;
    const float kf = (float)(V * 8);
    if constexpr (VPL > 0) {
        uint4 v[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) v[i] = load_or_zero_nt(xr, lane + 64 * i, V);
        if constexpr (RES) {
            uint4 r[VPL];
#pragma unroll
            for (int i = 0; i < VPL; ++i) r[i] = load_or_zero(rr, lane + 64 * i, V);
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                v[i] = add_bf16x8(v[i], r[i]);
                if (lane + 64 * i < V) rr[lane + 64 * i] = v[i];
            }
        }
        float p = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (lane + 64 * i < V) p = sumsq8(p, v[i]);
        const float S = tree_sum_wave(p);
        const float inv = 1.0f / sqrtf(S / kf + eps);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int64_t idx = lane + 64 * i;
            float y[8];
            rms_y8(v[i], load_or_zero(gamma, idx, V), inv, y);
            v[i] = pack_bf16x8(y);  // keep y (bf16) in place of x
            if constexpr (GROUP == 0) m = fmaxf(m, amax8(y));
        }
        if constexpr (GROUP == 0) {
            const GroupDiv g = group_div(max_wave(m));
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int64_t idx = lane + 64 * i;
                if (idx < V) {
                    float y[8];
                    unpack8(v[i], y);
                    store_nt8(qr + idx, encode8(y, g));
                }
            }
            if (lane == 0) s[row] = g.s;
        } else {
            const int64_t groups = V / 16;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int64_t idx = lane + 64 * i;
                float y[8];
                unpack8(v[i], y);
                const GroupDiv g = group_div(max_16lanes(amax8(y)));
                if (idx < V) {
                    store_nt8(qr + idx, encode8(y, g));
                    if ((lane & 15) == 0) s[row * groups + (idx >> 4)] = g.s;
                }
            }
        }
    } else {
        // long rows: sum pass, then y recomputed (bit-identically) per pass;
        // with RES the sum pass stores h over r and later passes read h back
        // (each lane reads only what it wrote itself)
        float p = 0.0f;
        if constexpr (RES) {
            for (int64_t idx = lane; idx < V; idx += 64) {
                const uint4 h = add_bf16x8(xr[idx], rr[idx]);
                rr[idx] = h;
                p = sumsq8(p, h);
            }
            xr = rr;
        } else {
            for (int64_t idx = lane; idx < V; idx += 64) p = sumsq8(p, xr[idx]);
        }
        const float S = tree_sum_wave(p);
        const float inv = 1.0f / sqrtf(S / kf + eps);
        if constexpr (GROUP == 0) {
            float m = 0.0f;
            for (int64_t idx = lane; idx < V; idx += 64) {
                float y[8];
                rms_y8(xr[idx], gamma[idx], inv, y);
                m = fmaxf(m, amax8(y));
            }
            const GroupDiv g = group_div(max_wave(m));
            for (int64_t idx = lane; idx < V; idx += 64) {
                float y[8];
                rms_y8(xr[idx], gamma[idx], inv, y);
                store_nt8(qr + idx, encode8(y, g));
            }
            if (lane == 0) s[row] = g.s;
        } else {
            const int64_t groups = V / 16;
            // V % 16 == 0 here, so every step covers whole groups
            for (int64_t base = 0; base < V; base += 64) {
                const int64_t idx = base + lane;
                float y[8];
                rms_y8(load_or_zero(xr, idx, V), load_or_zero(gamma, idx, V), inv, y);
                const GroupDiv g = group_div(max_16lanes(amax8(y)));
                if (idx < V) {
                    store_nt8(qr + idx, encode8(y, g));
                    if ((lane & 15) == 0) s[row * groups + (idx >> 4)] = g.s;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Fused RMSNorm + quantization, one row per workgroup of 4 waves (rows of
// more than 128 vectors).  The same fixed order as above, spread over 256
// lanes: partial l (vectors l, l + 64, l + 128, ... in order) belongs to wave
// l / 16; lane j of wave w holds partial l = 16 w + (j & 15) and its vectors
// i = (j >> 4), (j >> 4) + 4, ... (vector v = l + 64 i).  The ordered sum of a
// partial passes through its 4 lanes in turn: the lane holding vector i adds
// that vector's 8 squares in order, then a shuffle hands the running sum to
// the lanes of vector i + 1.  The halving tree ends inside each wave over its
// 16 partials (xor 1, 2, 4, 8) and through LDS across the waves:
// S = (T0 + T1) + (T2 + T3).  With the row's work on 4 waves, each wave's
// chain of loads, sums and stores is a quarter as long, and a CU holds
// workgroups at different phases, so loads of some rows overlap the stores
// of others.  A 1x128 group (vectors 16 g .. 16 g + 15) is 16 adjacent lanes
// of wave g % 4 (vector slot g / 16, lane group (g / 4) % 4).
// ---------------------------------------------------------------------------
template <int VPL4, int GROUP, bool RES>
__global__ __launch_bounds__(256) void k_rms_row(uint2* __restrict__ q,
                                                 const uint4* __restrict__ x,
                                                 uint4* __restrict__ res,
                                                 float* __restrict__ s,
                                                 const uint4* __restrict__ gamma, float eps,
                                                 int64_t V) {
    __shared__ float red[8];
    const int t = threadIdx.x, j = t & 63, w = t >> 6;
    const int64_t row = blockIdx.x;
    const int l = 16 * w + (j & 15), qg = j >> 4;
    const uint4* xr = x + row * V;
    uint4* rr = RES ? res + row * V : nullptr;
    uint2* qr = q + row * V;
    uint4 v[VPL4];
#pragma unroll
    for (int k = 0; k < VPL4; ++k) v[k] = load_or_zero_nt(xr, l + 64 * (qg + 4 * k), V);
    if constexpr (RES) {
        uint4 r[VPL4];
#pragma unroll
        for (int k = 0; k < VPL4; ++k) r[k] = load_or_zero(rr, l + 64 * (qg + 4 * k), V);
#pragma unroll
        for (int k = 0; k < VPL4; ++k) {
            const int64_t idx = l + 64 * (qg + 4 * k);
            v[k] = add_bf16x8(v[k], r[k]);
            if (idx < V) rr[idx] = v[k];
        }
    }
    // ordered partial sums, handed from lane group to lane group
    float P = 0.0f;
#pragma unroll
    for (int i = 0; i < 4 * VPL4; ++i) {
        const int owner = i & 3;
        if (qg == owner && l + 64 * i < V) P = sumsq8(P, v[i >> 2]);
        P = __shfl(P, (j & 15) + 16 * owner);
    }
    float T = P;
    T = T + __shfl_xor(T, 1);
    T = T + __shfl_xor(T, 2);
    T = T + __shfl_xor(T, 4);
    T = T + __shfl_xor(T, 8);
    if (j == 0) red[w] = T;
    __syncthreads();
    const float S = (red[0] + red[1]) + (red[2] + red[3]);
    const float kf = (float)(V * 8);
    const float inv = 1.0f / sqrtf(S / kf + eps);
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL4; ++k) {
        const int64_t idx = l + 64 * (qg + 4 * k);
        float y[8];
        rms_y8(v[k], load_or_zero(gamma, idx, V), inv, y);
        v[k] = pack_bf16x8(y);
        if constexpr (GROUP == 0) m = fmaxf(m, amax8(y));
    }
    if constexpr (GROUP == 0) {
        m = max_wave(m);
        if (j == 0) red[4 + w] = m;
        __syncthreads();
        const GroupDiv g = group_div(fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7])));
#pragma unroll
        for (int k = 0; k < VPL4; ++k) {
            const int64_t idx = l + 64 * (qg + 4 * k);
            if (idx < V) {
                float y[8];
                unpack8(v[k], y);
                store_nt8(qr + idx, encode8(y, g));
            }
        }
        if (t == 0) s[row] = g.s;
    } else {
        const int64_t groups = V / 16;
#pragma unroll
        for (int k = 0; k < VPL4; ++k) {
            const int64_t idx = l + 64 * (qg + 4 * k);
            float y[8];
            unpack8(v[k], y);
            const GroupDiv g = group_div(max_16lanes(amax8(y)));
            if (idx < V) {
                store_nt8(qr + idx, encode8(y, g));
                if ((j & 15) == 0) s[row * groups + (idx >> 4)] = g.s;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 128x128 weight blocks, many weights per launch.  One 256-thread workgroup
// per block: thread t reads 16 bytes of rows t/16 + 16 i (i = 0..7) at column
// chunk t % 16, so each wave reads four whole 256-byte row segments per step.
// FMT 0: fp32 scale; FMT 1: E8M0 byte e + 127 with e = ceil(log2(amax / 448)).
// ---------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(256) void k_requant(ReqBatch batch) {
    __shared__ float red[4];
    const int64_t b = blockIdx.x;
    // which weight: last descriptor whose first block is <= b (uniform search)
    int lo = 0, hi = batch.n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (batch.d[mid].block_begin <= b) lo = mid; else hi = mid - 1;
    }
    const ReqDesc& d = batch.d[lo];
    const int64_t local = b - d.block_begin;
    const int64_t bi = local / d.kblocks, bj = local % d.kblocks;
    const int64_t K = d.K;
    const int t = threadIdx.x;
    const int c = t & 15, r0 = t >> 4;
    const uint16_t* wb = d.w + (bi * 128) * K + bj * 128 + c * 8;
    uint8_t* qb = d.q + (bi * 128) * K + bj * 128 + c * 8;
    // the weights are read once and the codes written once: non-temporal
    // accesses keep the stream from filling L2 and the Infinity Cache
    // (5.50 -> 5.85 TB/s over the 144 policy weights)
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = load_nt16(wb + (int64_t)(r0 + 16 * i) * K);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float f[8];
        unpack8(v[i], f);
        m = fmaxf(m, amax8(f));
    }
    m = max_wave(m);
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if constexpr (FMT == 0) {
        const GroupDiv g = group_div(amax);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float f[8];
            unpack8(v[i], f);
            store_nt8(qb + (int64_t)(r0 + 16 * i) * K, encode8(f, g));
        }
        if (t == 0) static_cast<float*>(d.s)[local] = g.s;
    } else {
        const int e = e8m0_exponent(amax / 448.0f);
        const float inv = e8m0_inv(e);  // x * 2^-e == x / 2^e exactly
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float f[8], tq[8];
            unpack8(v[i], f);
#pragma unroll
            for (int j = 0; j < 8; ++j) tq[j] = f[j] * inv;
            store_nt8(qb + (int64_t)(r0 + 16 * i) * K, e4m3x8(tq));
        }
        if (t == 0) static_cast<uint8_t*>(d.s)[local] = (uint8_t)(e + 127);
    }
}

// ---------------------------------------------------------------------------
// Diagnostic: encode the fp32 bit patterns first .. first + n - 1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_encode_bits(uint64_t first, int64_t n,
                                                     uint32_t* __restrict__ q) {
    const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i4 >= n) return;
    float f[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = __uint_as_float((uint32_t)(first + i4 + j));
    const uint32_t packed = e4m3x4(f[0], f[1], f[2], f[3]);
    if (i4 + 4 <= n) {
        q[i4 >> 2] = packed;
    } else {
        uint8_t* qb = reinterpret_cast<uint8_t*>(q);
        for (int j = 0; i4 + j < n; ++j) qb[i4 + j] = (uint8_t)(packed >> (8 * j));
    }
}

template <typename Kern, typename... Args>
hipError_t launch(Kern k, int64_t blocks, hipStream_t st, Args... args) {
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(256), 0, st, args...);
    return hipGetLastError();
}

template <typename Kern, typename... Args>
hipError_t launch_threads(Kern k, int64_t blocks, int threads, hipStream_t st, Args... args) {
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3((unsigned)threads), 0, st, args...);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Diagnostic: bf16 rounding (the device helper every bf16 output uses) of the
// fp32 bit patterns first .. first + n - 1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bf16_bits(uint64_t first, int64_t n,
                                                   uint32_t* __restrict__ out) {
    const int64_t i2 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 2;
    if (i2 >= n) return;
    const uint32_t p = bf16x2_rne(__uint_as_float((uint32_t)(first + i2)),
                                  __uint_as_float((uint32_t)(first + i2 + 1)));
    if (i2 + 2 <= n)
        out[i2 >> 1] = p;
    else
        reinterpret_cast<uint16_t*>(out)[i2] = (uint16_t)p;
}

// ---------------------------------------------------------------------------
// SwiGLU + 1x128 quantization (the MoE chain between the gate_up and down
// GEMMs).  gu bf16 [T, 2I]: gate = columns [0, I), up = [I, 2I).
//   silu(g): the fp32 value nearest to g / (1 + e^-g), from closed forms and
//   a small table built in binary128 (silu_f32 below; a test over all 65536
//   bf16 inputs compares every value with the correctly rounded one);
//   y = bf16_rne(silu(g) * u), one fp32 multiply;
//   then y's 1x128 groups are quantized as k_quant_block does.
// Layout as k_quant_block: a 1x128 group is 16 lanes x 8 elements, a wave
// covers 4 groups per step; group gid = t * (I/128) + j reads 16 bytes of gate
// and 16 of up per lane and writes 8 bytes of codes.
// ---------------------------------------------------------------------------
// silu(g) of a bf16 gate, correctly rounded to fp32.  The build step
// gen_silu_table.c computes silu in binary128 for every bf16 pattern, checks
// that the closed forms below hold outside a middle band, and tabulates the
// band, which each workgroup stages in LDS (7522 words, 29.4 KiB):
//   [0, 3589]     silu of the positive gates 0x3380..0x4185 (2^-24 .. 16.625)
//   3590          unused (read by lanes whose value is selected elsewhere)
//   [3591, 7520]  silu of the negative gates 0xB380..0xC2D9 (-2^-24 .. -108.5)
//   7521          -0, silu of every finite gate below -108.5
// A gate's word is h - 0x3380 (h >= 0) or h - 0xA579 (h < 0), h its bf16
// bits, clamped to [0, 7521]; two gates' words come from 16-bit packed
// integer operations on the pair as loaded.  Outside the table:
//   |g| < 2^-24: g / 2 (exact; the next term, g^2/4, is below half an ulp);
//   g > 16.625 (and +inf): g;
//   -inf: the quiet NaN 0xFFC00000 (the quotient -inf / inf an fp64
//   evaluation of g / (1 + e^-g) returns), which is g's bits with the quiet
//   bit set; a NaN gate gives a NaN of its sign the same way;
//   finite g < -108.5: the table's -0.
// A test over all 65536 bf16 inputs compares every non-NaN value with the
// correctly rounded one.
constexpr int kSiluBandN = 7522;
constexpr int kSiluBandPad = 7524;  // 16-byte multiple, for the staging copy
__device__ const uint32_t kSiluBand[kSiluBandPad] = {
#include "silu_table.inc"
};

__device__ __forceinline__ void silu_band_to_lds(uint32_t* band) {
    const uint4* src = reinterpret_cast<const uint4*>(kSiluBand);
    uint4* dst = reinterpret_cast<uint4*>(band);
    for (int i = threadIdx.x; i < kSiluBandPad / 4; i += blockDim.x) dst[i] = src[i];
    __syncthreads();
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

// Byte offsets into the table of the two bf16 gates in w (low half, then
// high half), each computed in its own 16-bit lane.
__device__ __forceinline__ void silu_offsets(uint32_t w, uint32_t& lo, uint32_t& hi) {
    const u16x2 h = __builtin_bit_cast(u16x2, w);
    const u16x2 neg = __builtin_bit_cast(u16x2, __builtin_bit_cast(s16x2, h) >> (s16x2)15);
    const u16x2 d = h - (u16x2)0x3380u - (neg & (u16x2)(0xA579u - 0x3380u));
    s16x2 c = __builtin_elementwise_max(__builtin_bit_cast(s16x2, d), (s16x2)0);
    c = __builtin_elementwise_min(c, (s16x2)(kSiluBandN - 1));
    const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, c) << (u16x2)2);
    lo = b & 0xFFFFu;
    hi = b >> 16;
}

// silu of gate g from its table word t, for any g.
__device__ __forceinline__ float silu_select(float g, float t) {
    // -inf and NaN first, so each select takes cheap operands (the compiler
    // keeps the sequence branch-free); later selects never fire for them
    float r = !(g >= -3.40282346638528859812e+38f)
                  ? __uint_as_float(__float_as_uint(g) | 0x00400000u) : t;
    r = fabsf(g) < 0x1p-24f ? g * 0.5f : r;
    r = g > 16.625f ? g : r;
    return r;
}

__device__ __forceinline__ float band_word(const uint32_t* band, uint32_t byte_off) {
    return __uint_as_float(*reinterpret_cast<const uint32_t*>(
        reinterpret_cast<const uint8_t*>(band) + byte_off));
}

__device__ __forceinline__ float silu_f32(float g, const uint32_t* band) {  // g a bf16 value
    uint32_t lo, hi;
    silu_offsets(__float_as_uint(g) >> 16, lo, hi);
    return silu_select(g, band_word(band, lo));
}

// y = bf16_rne(silu(g) * u) for a lane's 8 gate and 8 up values; the 8 table
// reads are issued before any of them is used.  When every gate of the wave
// is in the table's domain (2^-24 <= |g| <= 16.625, or g negative and
// finite: 16-bit min / max of the patterns decide it), the table word is
// silu(g) and the selects are skipped.
__device__ __forceinline__ void swiglu8(const uint4& gv, const uint4& uv, const uint32_t* band,
                                        float (&y)[8]) {
    float g[8], u[8], t[8];
    unpack8(gv, g);
    unpack8(uv, u);
    const uint32_t w[4] = {gv.x, gv.y, gv.z, gv.w};
    u16x2 amin = (u16x2)0xFFFFu, amax = (u16x2)0u;
    s16x2 hmax = (s16x2)-32768;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t lo, hi;
        silu_offsets(w[k], lo, hi);
        t[2 * k] = band_word(band, lo);
        t[2 * k + 1] = band_word(band, hi);
        const u16x2 a = __builtin_bit_cast(u16x2, w[k]) & (u16x2)0x7FFFu;
        amin = __builtin_elementwise_min(amin, a);
        amax = __builtin_elementwise_max(amax, a);
        hmax = __builtin_elementwise_max(hmax, __builtin_bit_cast(s16x2, w[k]));
    }
    // every |g| >= 2^-24, no gate above 16.625, no infinity or NaN
    const bool in = amin.x >= 0x3380u && amin.y >= 0x3380u && hmax.x <= 0x4185 &&
                    hmax.y <= 0x4185 && amax.x < 0x7F80u && amax.y < 0x7F80u;
    if (__builtin_expect(__all(in), 1)) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            const uint32_t p = bf16x2_rne(t[j] * u[j], t[j + 1] * u[j + 1]);
            y[j] = bf16_lo(p);
            y[j + 1] = bf16_hi(p);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            const uint32_t p = bf16x2_rne(silu_select(g[j], t[j]) * u[j],
                                          silu_select(g[j + 1], t[j + 1]) * u[j + 1]);
            y[j] = bf16_lo(p);
            y[j + 1] = bf16_hi(p);
        }
    }
}

// Persistent: 512-thread workgroups, each staging the table once and striding
// over the groups.  A lane keeps, for each of its U groups, the group index
// and the uint4 offset of its gate chunk in gu, and advances both by the
// grid stride (the row and the column block as a carry, no division per
// step).  The loads of a pass are issued before the previous pass is
// computed (the first pass's before the table is staged), so every wave has
// a pass of gate and up values in flight while it computes.
constexpr int kSwigluWaves = 8;
template <int U>
__global__ __launch_bounds__(64 * kSwigluWaves) void k_swiglu_quant(const uint4* __restrict__ gu,
                                                                   uint2* __restrict__ q,
                                                                   float* __restrict__ s,
                                                                   int64_t G, int64_t GI) {
    __shared__ __align__(16) uint32_t band[kSiluBandPad];
    const int lane = threadIdx.x & 63, li = lane & 15;
    const int64_t step = (int64_t)gridDim.x * kSwigluWaves * 4 * U;  // groups per grid pass
    const int64_t dt = step / GI, dj = step - dt * GI;
    const int64_t row_u4 = GI * 32;  // uint4 per row of gu (2I bf16)
    const int64_t doff = dt * row_u4 + dj * 16;
    const int64_t first = ((int64_t)blockIdx.x * kSwigluWaves + (threadIdx.x >> 6)) * U * 4;
    int64_t gid[U], j[U], off[U];  // of the pass being loaded
#pragma unroll
    for (int u = 0; u < U; ++u) {
        gid[u] = first + u * 4 + (lane >> 4);
        const int64_t t = gid[u] / GI;
        j[u] = gid[u] - t * GI;
        off[u] = t * row_u4 + j[u] * 16;
    }
    const int64_t tl = (G - 1) / GI;  // lanes past the end re-read the last group
    const int64_t off_last = tl * row_u4 + (G - 1 - tl * GI) * 16;
    uint4 gv[U], uv[U];
    int64_t gc[U];  // group index of the pass in gv, uv
    auto load_pass = [&](uint4 (&a)[U], uint4 (&b)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t o = (gid[u] < G ? off[u] : off_last) + li;
            a[u] = load_nt16(gu + o);
            b[u] = load_nt16(gu + o + GI * 16);
            gc[u] = gid[u];
            gid[u] += step;
            j[u] += dj;
            off[u] += doff;
            if (j[u] >= GI) {  // carry into the next row
                j[u] -= GI;
                off[u] += GI * 16;
            }
        }
    };
    if (first < G) load_pass(gv, uv);
    silu_band_to_lds(band);
    for (int64_t g0 = first; g0 < G; g0 += step) {
        int64_t gcur[U];
#pragma unroll
        for (int u = 0; u < U; ++u) gcur[u] = gc[u];
        uint4 gn[U], un[U];
        if (g0 + step < G) load_pass(gn, un);  // wave-uniform
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float y[8];
            swiglu8(gv[u], uv[u], band, y);
            const GroupDiv g = group_div(max_16lanes(amax8(y)));
            if (gcur[u] < G) {
                store_nt8(q + gcur[u] * 16 + li, encode8(y, g));
                if (li == 0) s[gcur[u]] = g.s;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            gv[u] = gn[u];
            uv[u] = un[u];
        }
    }
}

// ---------------------------------------------------------------------------
// Token gather + 1x128 quantization (the MoE dispatch before the gate_up
// GEMM): output row t is the 1x128 quantization of x[row_token[t]].  The
// layout is k_quant_block's (16 lanes x 8 elements per group, 4 groups per
// wave step); each group looks up its source row first.  An index outside
// [0, n_src) yields a zero row (codes 0, scale 0) and reads nothing.
// ---------------------------------------------------------------------------
// IDX: the index type of groups (32-bit when every group index fits, which
// lets the row of a group come from a multiply and shift).
template <int U, typename IDX>
__global__ __launch_bounds__(256) void k_quant_gather(const uint4* __restrict__ x,
                                                      const int32_t* __restrict__ row_token,
                                                      uint2* __restrict__ q,
                                                      float* __restrict__ s, int64_t G,
                                                      int64_t GK, int64_t n_src, FastDiv fgk) {
    const int lane = threadIdx.x & 63, li = lane & 15;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t chunk0 = wave * U;
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t gid = (chunk0 + u) * 4 + (lane >> 4);
        v[u] = uint4{0u, 0u, 0u, 0u};
        if (gid < G) {
            int64_t t;
            if constexpr (sizeof(IDX) == 4) t = fdiv((uint32_t)gid, fgk);
            else t = gid / GK;
            const int64_t j = gid - t * GK;
            const int64_t src = row_token[t];
            if (src >= 0 && src < n_src) v[u] = x[src * GK * 16 + j * 16 + li];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t gid = (chunk0 + u) * 4 + (lane >> 4);
        float f[8];
        unpack8(v[u], f);
        const GroupDiv g = group_div(max_16lanes(amax8(f)));
        if (gid < G) {
            store_nt8(q + gid * 16 + li, encode8(f, g));
            if (li == 0) s[gid] = g.s;
        }
    }
}

// ---------------------------------------------------------------------------
// Inverse RoPE + 1x128 E8M0 quantization (the DeepSeek V4 output projection's
// pre-op, feeding the batched MX GEMM).  o bf16 [T][H][D] (D % 8 == 0): the
// last R dims of each head are interleaved pairs (y0, y1) with angle index i;
// cos/sin fp32 [P][R/2].  x0 = y0*c + y1*s and x1 = y1*c - y0*s as single
// fp32 operations (the library is built without FMA contraction), rounded to
// bf16; other dims pass through.  Each token's flattened [H*D] row is then
// quantized in 1x128 groups with E8M0 scales, as k_quant_block<U, 1> does.
// A lane's 8 elements lie in one head; a position outside [0, P) gives a
// zero row and reads nothing from the caches.
// ---------------------------------------------------------------------------
// IDX: the index type of groups (32-bit when the group count fits).  VEC:
// R % 8 == 0 and (D - R) % 8 == 0, so a lane's 8 elements are either all
// rotary (4 consecutive angles, one 16-byte cos and sin load each) or all
// pass-through.
template <int U, typename IDX, bool VEC>
__global__ __launch_bounds__(256) void k_inv_rope_quant(
    const uint4* __restrict__ o, const int64_t* __restrict__ pos, const float* __restrict__ cosc,
    const float* __restrict__ sinc, uint2* __restrict__ q, uint8_t* __restrict__ s, int64_t G64,
    int64_t GK64, int D, int R, int64_t P, FastDiv fgk, FastDiv fd) {
    const int lane = threadIdx.x & 63, li = lane & 15;
    const IDX G = (IDX)G64, GK = (IDX)GK64;
    const IDX wave = (IDX)blockIdx.x * 4 + (IDX)(threadIdx.x >> 6);
    const IDX chunk0 = wave * U;
    const int half = R >> 1, rope0 = D - R;
    // 32-bit indices divide by multiply and shift (every dividend < 2^31)
    auto div_gk = [&](IDX n) -> IDX {
        if constexpr (sizeof(IDX) == 4) return (IDX)fdiv((uint32_t)n, fgk);
        else return n / GK;
    };
    auto mod_d = [&](int e) -> int {
        if constexpr (sizeof(IDX) == 4) return e - (int)fdiv((uint32_t)e, fd) * D;
        else return e - (e / D) * D;
    };
    uint4 v[U];
    int64_t p[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const IDX gid = (chunk0 + u) * 4 + (IDX)(lane >> 4);
        v[u] = uint4{0u, 0u, 0u, 0u};
        p[u] = -1;
        if (gid < G) {  // both loads in bounds; an invalid position zeroes the row after
            p[u] = pos[div_gk(gid)];
            v[u] = load_nt16(o + (int64_t)gid * 16 + li);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const IDX gid = (chunk0 + u) * 4 + (IDX)(lane >> 4);
        if (p[u] < 0 || p[u] >= P) {
            p[u] = -1;
            v[u] = uint4{0u, 0u, 0u, 0u};
        }
        float f[8];
        unpack8(v[u], f);
        if (p[u] >= 0) {
            const IDX j = gid - div_gk(gid) * GK;
            const int e0 = (int)(j * 128) + li * 8;    // element offset in the row
            const int d0 = mod_d(e0);                  // its dim within the head
            const float* cr = cosc + p[u] * half;
            const float* sr = sinc + p[u] * half;
            float x[8];
            if constexpr (VEC) {
                if (d0 >= rope0) {
                    const int i0 = (d0 - rope0) >> 1;  // a multiple of 4
                    const float4 c4 = *reinterpret_cast<const float4*>(cr + i0);
                    const float4 s4 = *reinterpret_cast<const float4*>(sr + i0);
                    const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
                    const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                    for (int k = 0; k < 8; k += 2) {
                        const float c = cv[k >> 1], sn = sv[k >> 1];
                        const float a = f[k] * c, b = f[k + 1] * sn;
                        const float a1 = f[k + 1] * c, b1 = f[k] * sn;
                        x[k] = a + b;
                        x[k + 1] = a1 - b1;
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < 8; ++k) x[k] = f[k];
                }
            } else {
#pragma unroll
            for (int k = 0; k < 8; k += 2) {
                const int d = d0 + k;
                if (d >= rope0) {
                    const int i = (d - rope0) >> 1;
                    const float c = cr[i], sn = sr[i];
                    const float a = f[k] * c, b = f[k + 1] * sn;
                    const float a1 = f[k + 1] * c, b1 = f[k] * sn;
                    x[k] = a + b;
                    x[k + 1] = a1 - b1;
                } else {
                    x[k] = f[k];
                    x[k + 1] = f[k + 1];
                }
            }
            }
#pragma unroll
            for (int k = 0; k < 8; k += 2) {
                const uint32_t pr = bf16x2_rne(x[k], x[k + 1]);
                f[k] = bf16_lo(pr);
                f[k + 1] = bf16_hi(pr);
            }
        }
        const float amax = max_16lanes(amax8(f));
        const int e = e8m0_exponent(amax / 448.0f);
        const float inv = e8m0_inv(e);
        float t8[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) t8[k] = f[k] * inv;
        if (gid < G) {
            store_nt8(q + (int64_t)gid * 16 + li, e4m3x8(t8));
            if (li == 0) s[gid] = (uint8_t)(e + 127);
        }
    }
}

// Diagnostic: silu of the bf16 bit patterns first .. first + n - 1, as fp32.
__global__ __launch_bounds__(256) void k_silu_bits(uint32_t first, int64_t n,
                                                   float* __restrict__ out) {
    __shared__ __align__(16) uint32_t band[kSiluBandPad];
    silu_band_to_lds(band);
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = silu_f32(__uint_as_float((first + (uint32_t)i) << 16), band);
}

// ---------------------------------------------------------------------------
// Per-tensor quantization (one scale per tensor), four kernels per batch:
// clear each tensor's scale slot, reduce |x| into it (the amax's fp32 bits:
// for non-negative floats the unsigned integer order is the numeric order, so
// an unsigned atomic max of the bits is the max), quantize with s = amax / 448,
// then write s itself.  The kernel boundaries order the steps.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_tens_clear(TensBatch b) {
    if ((int)threadIdx.x < b.n) *reinterpret_cast<uint32_t*>(b.d[threadIdx.x].s) = 0u;
}

__device__ __forceinline__ int tens_find(const TensBatch& b, int64_t chunk) {
    int lo = 0, hi = b.n - 1;  // last descriptor whose first chunk is <= chunk
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (b.d[mid].chunk_begin <= chunk) lo = mid; else hi = mid - 1;
    }
    return lo;
}

constexpr int kTensVpt = (int)(kTensChunk / 256);  // vectors per thread

__global__ __launch_bounds__(256) void k_tens_amax(TensBatch b) {
    __shared__ float red[4];
    const TensDesc& d = b.d[tens_find(b, blockIdx.x)];
    const int64_t base = ((int64_t)blockIdx.x - d.chunk_begin) * kTensChunk + threadIdx.x;
    const uint4* x = static_cast<const uint4*>(d.x);
    uint4 v[kTensVpt];
#pragma unroll
    for (int i = 0; i < kTensVpt; ++i) v[i] = load_or_zero_nt(x, base + 256 * i, d.nvec);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kTensVpt; ++i) {
        float f[8];
        unpack8(v[i], f);
        m = fmaxf(m, amax8(f));
    }
    m = max_wave(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        atomicMax(reinterpret_cast<unsigned int*>(d.s), __float_as_uint(m));
    }
}

__global__ __launch_bounds__(256) void k_tens_quant(TensBatch b) {
    const TensDesc& d = b.d[tens_find(b, blockIdx.x)];
    const int64_t base = ((int64_t)blockIdx.x - d.chunk_begin) * kTensChunk + threadIdx.x;
    const uint4* x = static_cast<const uint4*>(d.x);
    uint2* q = static_cast<uint2*>(d.q);
    const GroupDiv g = group_div(__uint_as_float(*reinterpret_cast<const uint32_t*>(d.s)));
    uint4 v[kTensVpt];
#pragma unroll
    for (int i = 0; i < kTensVpt; ++i) v[i] = load_or_zero_nt(x, base + 256 * i, d.nvec);
#pragma unroll
    for (int i = 0; i < kTensVpt; ++i) {
        const int64_t idx = base + 256 * i;
        if (idx < d.nvec) {
            float f[8];
            unpack8(v[i], f);
            store_nt8(q + idx, encode8(f, g));
        }
    }
}

__global__ __launch_bounds__(64) void k_tens_final(TensBatch b) {
    if ((int)threadIdx.x < b.n) {
        float* s = b.d[threadIdx.x].s;
        *s = __uint_as_float(*reinterpret_cast<const uint32_t*>(s)) / 448.0f;
    }
}

}  // namespace

hipError_t launch_quantize_block(const void* x, int64_t M, int64_t K, void* q, void* s, int fmt,
                                 hipStream_t st) {
    // 4 groups per wave and step; U steps per wave.  Between 2^14 and 2^18
    // groups (4 to 32 MiB of bf16) a launch is mostly fill and drain, and one
    // step per wave (four times the waves, each with one load in flight) is
    // faster: 256 x 12288 4.6 -> 3.8 us, 1024 x 4096 4.9 -> 4.1 us.  Smaller
    // launches pay more for the extra workgroups than they gain (256 x 4096:
    // 3.2 -> 3.7 us), larger ones lose (8192 x 12288: 13% slower).
    constexpr int U = 4;
    const int64_t G = M * (K / 128);
    const int64_t waves = (G + 4 * U - 1) / (4 * U);
    if (G >= (int64_t(1) << 14) && G < (int64_t(1) << 18)) {
        const int64_t w1 = (G + 3) / 4;
        if (fmt == 0)
            return launch(k_quant_block<1, 0>, (w1 + 3) / 4, st, static_cast<const uint4*>(x),
                          static_cast<uint2*>(q), s, G);
        return launch(k_quant_block<1, 1>, (w1 + 3) / 4, st, static_cast<const uint4*>(x),
                      static_cast<uint2*>(q), s, G);
    }
    if (fmt == 0)
        return launch(k_quant_block<U, 0>, (waves + 3) / 4, st, static_cast<const uint4*>(x),
                      static_cast<uint2*>(q), s, G);
    return launch(k_quant_block<U, 1>, (waves + 3) / 4, st, static_cast<const uint4*>(x),
                  static_cast<uint2*>(q), s, G);
}

hipError_t launch_swiglu_quant(const void* gu, int64_t T, int64_t I, void* q, float* s,
                               hipStream_t st) {
    // persistent: at most 4 workgroups of 8 waves per CU (the LDS holds four
    // copies of the table), striding over the groups; one group per lane and
    // pass keeps the kernel at 55 VGPRs, so all 8 waves per SIMD fit
    constexpr int U = 1;
    const int64_t GI = I / 128, G = T * GI;
    const int64_t waves = (G + 4 * U - 1) / (4 * U);
    const int64_t blocks = (waves + kSwigluWaves - 1) / kSwigluWaves;
    return launch_threads(k_swiglu_quant<U>, blocks < 1024 ? blocks : 1024, 64 * kSwigluWaves, st,
                  static_cast<const uint4*>(gu), static_cast<uint2*>(q), s, G, GI);
}

hipError_t launch_quant_gather(const void* x, int64_t n_src, int64_t K, const int32_t* row_token,
                               int64_t T, void* q, float* s, hipStream_t st) {
    constexpr int U = 4;
    const int64_t GK = K / 128, G = T * GK;
    const int64_t waves = (G + 4 * U - 1) / (4 * U);
    const int64_t blocks = (waves + 3) / 4;
    if (blocks * 16 * U < (int64_t(1) << 31))  // every group index fits in 31 bits
        return launch(k_quant_gather<U, int32_t>, blocks, st, static_cast<const uint4*>(x),
                      row_token, static_cast<uint2*>(q), s, G, GK, n_src, fast_div(GK));
    return launch(k_quant_gather<U, int64_t>, blocks, st, static_cast<const uint4*>(x), row_token,
                  static_cast<uint2*>(q), s, G, GK, n_src, FastDiv{1u, 0});
}

hipError_t launch_inv_rope_quant(const void* o, const int64_t* pos, const float* cosc,
                                 const float* sinc, int64_t T, int64_t H, int64_t D, int64_t R,
                                 int64_t P, void* q, uint8_t* s, hipStream_t st) {
    constexpr int U = 4;
    const int64_t GK = H * D / 128, G = T * GK;
    const int64_t waves = (G + 4 * U - 1) / (4 * U);
    const int64_t blocks = (waves + 3) / 4;
    const bool small = blocks * 16 * U < (int64_t(1) << 31);  // every gid fits in int32
    const bool vec = R % 8 == 0 && (D - R) % 8 == 0 &&
                     reinterpret_cast<uintptr_t>(cosc) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(sinc) % 16 == 0;
    const auto* ov = static_cast<const uint4*>(o);
    auto* qv = static_cast<uint2*>(q);
    const FastDiv fgk = fast_div(GK), fd = fast_div(D);
#define FP8_ROPE(IDX, VEC) \
    launch(k_inv_rope_quant<U, IDX, VEC>, blocks, st, ov, pos, cosc, sinc, qv, s, G, GK, (int)D, \
           (int)R, P, fgk, fd)
    if (small) return vec ? FP8_ROPE(int32_t, true) : FP8_ROPE(int32_t, false);
    return vec ? FP8_ROPE(int64_t, true) : FP8_ROPE(int64_t, false);
#undef FP8_ROPE
}

hipError_t launch_silu_bits(uint32_t first, int64_t n, float* out, hipStream_t st) {
    return launch(k_silu_bits, (n + 255) / 256, st, first, n, out);
}

hipError_t launch_quantize_token(const void* x, int64_t M, int64_t K, void* q, float* s,
                                 hipStream_t st) {
    const int64_t V = K / 8, blocks = (M + 3) / 4;
    const uint4* xv = static_cast<const uint4*>(x);
    uint2* qv = static_cast<uint2*>(q);
    // rows of 129 .. 2048 vectors: one row per 4-wave workgroup (W [12288,
    // 5120]: 33.3 -> 31.1 us on rotated inputs)
#define FP8_TOKEN_ROW_CASE(VPL4) \
    if (V <= 256 * VPL4) return launch(k_token_row<VPL4>, M, st, xv, qv, s, V);
    if (V > 128 && M <= INT32_MAX) {
        FP8_TOKEN_ROW_CASE(1)
        FP8_TOKEN_ROW_CASE(2)
        FP8_TOKEN_ROW_CASE(3)
        FP8_TOKEN_ROW_CASE(4)
        FP8_TOKEN_ROW_CASE(6)
        FP8_TOKEN_ROW_CASE(8)
    }
#undef FP8_TOKEN_ROW_CASE
    // vectors per lane: the smallest instantiation that holds the row, so short
    // rows keep few registers and many waves per SIMD
#define FP8_TOKEN_CASE(VPL) \
    if (V <= 64 * VPL) return launch(k_quant_token<VPL>, blocks, st, xv, qv, s, M, V);
    FP8_TOKEN_CASE(2)
    FP8_TOKEN_CASE(4)
    FP8_TOKEN_CASE(6)
    FP8_TOKEN_CASE(8)
    FP8_TOKEN_CASE(10)
    FP8_TOKEN_CASE(12)
    FP8_TOKEN_CASE(16)
    FP8_TOKEN_CASE(24)
    FP8_TOKEN_CASE(32)
#undef FP8_TOKEN_CASE
    return launch(k_quant_token<0>, blocks, st, xv, qv, s, M, V);
}

hipError_t launch_rmsnorm_quant(void* q, const void* x, void* res, float* s, const void* gamma,
                                float eps, int64_t M, int64_t K, int group_size,
                                hipStream_t st) {
    const int64_t V = K / 8, blocks = (M + 3) / 4;
    uint2* qv = static_cast<uint2*>(q);
    const uint4* xv = static_cast<const uint4*>(x);
    uint4* rv = static_cast<uint4*>(res);
    const uint4* gv = static_cast<const uint4*>(gamma);
    // with a residual, rows of 129 .. 2048 vectors take one row per 4-wave
    // workgroup ([4096, 5120]: 32.3 -> 30.4 us on rotated inputs); without one
    // the one-wave rows are faster (16.3 against 18.2 us)
#define FP8_RMS_ROW(VPL4, G, R) \
    launch(k_rms_row<VPL4, G, R>, M, st, qv, xv, rv, s, gv, eps, V)
#define FP8_RMS_ROW_CASE(VPL4)                                                   \
    if (V <= 256 * VPL4) {                                                       \
        if (group_size == 0)                                                     \
            return rv ? FP8_RMS_ROW(VPL4, 0, true) : FP8_RMS_ROW(VPL4, 0, false);  \
        return rv ? FP8_RMS_ROW(VPL4, 128, true) : FP8_RMS_ROW(VPL4, 128, false);  \
    }
    if (rv != nullptr && V > 128 && M <= INT32_MAX) {
        FP8_RMS_ROW_CASE(1)
        FP8_RMS_ROW_CASE(2)
        FP8_RMS_ROW_CASE(3)
        FP8_RMS_ROW_CASE(4)
        FP8_RMS_ROW_CASE(6)
        FP8_RMS_ROW_CASE(8)
    }
#undef FP8_RMS_ROW_CASE
#undef FP8_RMS_ROW
#define FP8_RMS_LAUNCH(VPL, G, R) \
    launch(k_rmsnorm_quant<VPL, G, R>, blocks, st, qv, xv, rv, s, gv, eps, M, V)
#define FP8_RMS_CASE(VPL)                                                            \
    if (VPL == 0 || V <= 64 * VPL) {                                                 \
        if (group_size == 0)                                                         \
            return rv ? FP8_RMS_LAUNCH(VPL, 0, true) : FP8_RMS_LAUNCH(VPL, 0, false);  \
        return rv ? FP8_RMS_LAUNCH(VPL, 128, true) : FP8_RMS_LAUNCH(VPL, 128, false);  \
    }
    FP8_RMS_CASE(2)
    FP8_RMS_CASE(4)
    FP8_RMS_CASE(6)
    FP8_RMS_CASE(8)
    FP8_RMS_CASE(10)
    FP8_RMS_CASE(12)
    FP8_RMS_CASE(16)
    FP8_RMS_CASE(24)
    FP8_RMS_CASE(32)
    FP8_RMS_CASE(0)
#undef FP8_RMS_CASE
#undef FP8_RMS_LAUNCH
    return hipErrorInvalidValue;
}

hipError_t launch_requant(const ReqBatch& batch, int64_t total_blocks, int fmt,
                          hipStream_t st) {
    if (fmt == 0) return launch(k_requant<0>, total_blocks, st, batch);
    return launch(k_requant<1>, total_blocks, st, batch);
}

hipError_t launch_tensor_batch(const TensBatch& batch, int64_t chunks, hipStream_t st) {
    if (batch.n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_tens_clear, dim3(1), dim3(64), 0, st, batch);
    if (chunks > 0) {
        hipLaunchKernelGGL(k_tens_amax, dim3((unsigned)chunks), dim3(256), 0, st, batch);
        hipLaunchKernelGGL(k_tens_quant, dim3((unsigned)chunks), dim3(256), 0, st, batch);
    }
    hipLaunchKernelGGL(k_tens_final, dim3(1), dim3(64), 0, st, batch);
    return hipGetLastError();
}

hipError_t launch_bf16_bits(uint64_t first, int64_t n, void* out, hipStream_t st) {
    const int64_t blocks = (n + 511) / 512;
    return launch(k_bf16_bits, blocks, st, first, n, static_cast<uint32_t*>(out));
}

hipError_t launch_encode_bits(uint64_t first, int64_t n, void* q, hipStream_t st) {
    const int64_t blocks = (n + 1023) / 1024;
    return launch(k_encode_bits, blocks, st, first, n, static_cast<uint32_t*>(q));
}

}  // namespace fp8k
