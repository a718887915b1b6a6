// device.hpp -- gfx950 device helpers shared by the quantizer and GEMM kernels:
// bf16 unpacking and rounding, the E4M3FN encoder, wave reductions.
//
// E4M3FN (OCP 8-bit FP, E4M3 without infinities, max 448; the float8_e4m3fn
// dtype of the verl "Test" section) is produced by the gfx950 conversion
// instruction v_cvt_pk_fp8_f32, which rounds to nearest even into the OCP
// format.  The input is first clamped to [-448, 448] with v_med3_f32, which
// makes the conversion saturating: it never produces the NaN pattern.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.hpp"

namespace fp8k {



__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// 8 bf16 values packed in 16 bytes -> 8 floats (element i = i-th bf16 in memory)
__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (a in the low half), round to nearest even, by the
// gfx950 conversion v_cvt_pk_bf16_f32.  It matches the bit-level definition
// (add 0x7FFF plus the kept LSB, truncate) on every non-NaN fp32 pattern,
// subnormals included; fp8_bf16_round_f32_bits exposes it to that test.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2_t));
}

// fp32 -> bf16 bit pattern, round to nearest even.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) { return bf16x2_rne(f, 0.0f) & 0xFFFFu; }

// Four floats -> four E4M3FN bytes (byte i encodes element i).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    uint32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
}

__device__ __forceinline__ uint2 e4m3x8(const float (&t)[8]) {
    return make_uint2(e4m3x4(t[0], t[1], t[2], t[3]), e4m3x4(t[4], t[5], t[6], t[7]));
}

__device__ __forceinline__ float amax8(const float (&f)[8]) {
    float m = fabsf(f[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
    return m;
}

// Max over aligned groups of 16 lanes (order-free, so exact).
// max with the value of another lane of the same 16-lane row, by a DPP
// move (no LDS round trip)
template <int CTRL>
__device__ __forceinline__ float max_dpp(float v) {
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF,
                                                               0xF, false)));
}

// Max over each aligned group of 16 lanes, in every lane of the group: lane
// i ^ 1, then i ^ 2 (quad permutes), then 7 - i within 8 lanes and 15 - i
// within 16 (half-row and row mirrors); fmax is order-free, so the result is
// the group's max whatever the pairing.
__device__ __forceinline__ float max_16lanes(float v) {
    v = max_dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v = max_dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v = max_dpp<0x141>(v);  // row_half_mirror
    v = max_dpp<0x140>(v);  // row_mirror
    return v;
}

__device__ __forceinline__ float max_wave(float v) {
    v = max_16lanes(v);
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// Sum over the 64 lanes as the halving tree T(0..63) = T(0..31) + T(32..63),
// recursively: the xor partner at distance 1, 2, 4, ... 32 holds the sibling
// subtree, and IEEE addition is commutative, so every lane ends with the same
// tree sum.
__device__ __forceinline__ float tree_sum_wave(float v) {
    v = v + __shfl_xor(v, 1);
    v = v + __shfl_xor(v, 2);
    v = v + __shfl_xor(v, 4);
    v = v + __shfl_xor(v, 8);
    v = v + __shfl_xor(v, 16);
    v = v + __shfl_xor(v, 32);
    return v;
}

}  // namespace fp8k
