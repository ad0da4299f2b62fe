// Tile layer for gfx950 (CDNA4): bf16 MFMA fragments, wave64 row reductions,
// bf16 packing, and the global/LDS moves the attention kernel is built from.
//
// The pages treat a small matrix tile as the primitive type and name the two
// contractions attention needs, A·Bᵀ for Q·Kᵀ and A·B for P·V with V read in
// transposed form ("Distilling a 4.5 hour CUDA talk", section 10, register
// tiles). On gfx950 the native shape is the 32x32x16 bf16 MFMA with fp32
// accumulation, so that is the tile here; the operands live in VGPRs.
//
// Fragment layout of v_mfma_f32_32x32x16_bf16 (wave64), for C = A·B with A
// 32xK16, B K16x32, lane l, half g = l / 32:
//   A operand: 8 bf16 of row (l % 32), k = 8g .. 8g+7 (the same k numbering
//              as B, so any consistent in-lane k order contracts correctly);
//   B operand: 8 bf16 of column (l % 32), the same k range;
//   C (16 fp32): column (l % 32), rows 8*(r/4) + 4g + (r%4) for r = 0..15.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// C += A·B on one 32x32x16 bf16 tile, fp32 accumulate.
__device__ __forceinline__ f32x16 mfma_32x32x16(const bf16x8 a, const bf16x8 b, const f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator held in register r by a lane of half g.
__device__ __forceinline__ constexpr int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// Combine a value with the one held by lane l ^ 32 (the other half of the
// wave): one v_permlane32_swap, no LDS traffic.
__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x on the transcendental unit (v_exp_f32). exp2(-inf) = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    __bf16 a = (__bf16)lo, b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ bf16x8 u32x4_as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight consecutive elements starting at p, as bf16 (16 bytes). fp32 inputs
// are rounded to bf16 here, once, on their way on chip.
__device__ __forceinline__ u32x4 load8_bf16(const __bf16 *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ u32x4 load8_bf16(const float *p) {
    const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
    return u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                 pack_bf16x2(b[2], b[3])};
}

// Select the low (hi = false) or high 16-bit halves of two dwords into one
// dword: result = half(lo_src) | half(hi_src) << 16 (one v_perm_b32).
__device__ __forceinline__ uint32_t pick_halves(uint32_t lo_src, uint32_t hi_src, bool hi) {
    return __builtin_amdgcn_perm(hi_src, lo_src, hi ? 0x07060302u : 0x05040100u);
}

// Stores of four consecutive output values.
__device__ __forceinline__ void store4(__bf16 *p, float a, float b, float c, float d) {
    *(u32x2 *)p = u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
    *(f32x4 *)p = f32x4{a, b, c, d};
}

}  // namespace attn
