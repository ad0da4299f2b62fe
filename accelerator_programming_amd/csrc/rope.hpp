// Rotary position embedding (RoPE) on gfx950: the step that precedes
// attention in the decoder chain ("CS149 L11: Programming Specialized
// Hardware", section 6), and the pages' example of a kernel in the
// load-compute-store-finish form ("Distilling a 4.5 hour CUDA talk", section
// 12: rope loads, computes and stores every iteration).
//
// Reading (the pages do not write the formula out): the rotation of the
// original RoPE paper (Su et al., RoFormer) on interleaved pairs. Element
// pair k of a row at position t, (x[2k], x[2k + 1]), is rotated by the angle
//   theta = t * base^(-2k / d):
//   y[2k]     = x[2k] cos theta - x[2k + 1] sin theta
//   y[2k + 1] = x[2k] sin theta + x[2k + 1] cos theta.
// A 16-byte chunk of a row holds four whole pairs, so one lane rotates a
// chunk in registers. The angle is formed and reduced to [-pi, pi] in fp64
// (t up to 2^31 and theta up to t radians need more than fp32's 24 bits),
// then cos and sin are taken in fp32 and the rotation runs in fp32; the
// result is rounded to bf16 (round to nearest even).
#pragma once
#include "tile.hpp"

namespace attn {

// cos and sin of t * base^(-2k / d), with log2_base = log2(base)
__device__ __forceinline__ void rope_angle(int64_t t, int k, int d, double log2_base, float &c,
                                           float &s) {
    const double inv_freq = exp2(-(double)(2 * k) / (double)d * log2_base);
    const double theta = (double)t * inv_freq;
    constexpr double kTwoPi = 6.283185307179586476925;
    const double red = theta - kTwoPi * rint(theta * (1.0 / kTwoPi));
    __sincosf((float)red, &s, &c);
}

// rotate the four pairs of a 16-byte bf16 chunk whose first element is
// element 2 * k0 of its row (k0 = index of its first pair)
__device__ __forceinline__ u32x4 rope_chunk(u32x4 v, int64_t t, int k0, int d, double log2_base) {
    u32x4 out;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        // the element is copied out first: a bit cast of a vector element
        // subscript read element 0 in every iteration
        const uint32_t word = v[p];
        const bf16x2 xy = __builtin_bit_cast(bf16x2, word);
        const float x = (float)xy[0], y = (float)xy[1];
        float c, s;
        rope_angle(t, k0 + p, d, log2_base, c, s);
        out[p] = pack_bf16x2(x * c - y * s, x * s + y * c);
    }
    return out;
}

struct RopeArgs {
    const __bf16 *x;
    __bf16 *y;
    int64_t x_sb, x_sh, x_sn, y_sb, y_sh, y_sn;  // (b, h, n) strides in elements
    int32_t H, N, d;
    int64_t chunks;  // B * H * N * d / 8
    double log2_base;
};

// One lane per 16-byte chunk: load, rotate, store. Memory-bound: every byte
// of X is read once and every byte of Y written once, in row order.
__global__ void __launch_bounds__(256) rope_bf16_kernel(const RopeArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.chunks) return;
    const int cpr = a.d / 8;
    const int c = (int)(i % cpr);
    const int64_t r = i / cpr;
    const int64_t n = r % a.N;
    const int64_t bh = r / a.N;
    const int64_t h = bh % a.H, b = bh / a.H;
    const __bf16 *src = a.x + b * a.x_sb + h * a.x_sh + n * a.x_sn + 8 * c;
    __bf16 *dst = a.y + b * a.y_sb + h * a.y_sh + n * a.y_sn + 8 * c;
    const u32x4 v = *(const u32x4 *)src;
    *(u32x4 *)dst = rope_chunk(v, n, 4 * c, a.d, a.log2_base);
}

}  // namespace attn
