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

// base^(-2k / d), with log2_base = log2(base)
__device__ __forceinline__ double rope_inv_freq(int k, int d, double log2_base) {
    return exp2(-(double)(2 * k) / (double)d * log2_base);
}

// cos and sin of t * inv_freq: the angle formed and reduced to [-pi, pi] in
// fp64, then cos and sin in fp32
__device__ __forceinline__ void rope_cos_sin(int64_t t, double inv_freq, float &c, float &s) {
    const double theta = (double)t * inv_freq;
    constexpr double kTwoPi = 6.283185307179586476925;
    const double red = theta - kTwoPi * rint(theta * (1.0 / kTwoPi));
    __sincosf((float)red, &s, &c);
}

// rotate the four pairs of a 16-byte bf16 chunk of the row at position t;
// inv_freq[p] is the frequency of the chunk's pair p
__device__ __forceinline__ u32x4 rope_chunk_f(u32x4 v, int64_t t, const double (&inv_freq)[4]) {
    u32x4 out;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        // the element is copied out first: a bit cast of a vector element
        // subscript read element 0 in every iteration
        const uint32_t word = v[p];
        const bf16x2 xy = __builtin_bit_cast(bf16x2, word);
        const float x = (float)xy[0], y = (float)xy[1];
        float c, s;
        rope_cos_sin(t, inv_freq[p], c, s);
        out[p] = pack_bf16x2(x * c - y * s, x * s + y * c);
    }
    return out;
}

// the same, with the frequencies of pairs k0 .. k0 + 3 formed here
__device__ __forceinline__ u32x4 rope_chunk(u32x4 v, int64_t t, int k0, int d, double log2_base) {
    double f[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) f[p] = rope_inv_freq(k0 + p, d, log2_base);
    return rope_chunk_f(v, t, f);
}

struct RopeArgs {
    const __bf16 *x;
    __bf16 *y;
    int64_t x_sb, x_sh, x_sn, y_sb, y_sh, y_sn;  // (b, h, n) strides in elements
    int32_t H, N, d;
    int32_t row_blocks;  // ceil(N / ROPE_ROWS)
    double log2_base;
};

constexpr int ROPE_ROWS = 64;  // rows of one (b, h) per workgroup

// A workgroup rotates ROPE_ROWS rows of one (b, h); lane (slot, c) keeps the
// frequencies of chunk c's four pairs and walks the rows slot, slot + S, ...
// (S = 256 / chunks per row). Consecutive lanes touch consecutive 16-byte
// chunks, so each row (and, for contiguous rows, the whole block) is one
// coalesced run. Memory-bound: every byte of X is read once and every byte
// of Y written once.
__global__ void __launch_bounds__(256) rope_bf16_kernel(const RopeArgs a) {
    const int cpr = a.d / 8;
    const int slots = 256 / cpr;
    const int c = threadIdx.x % cpr, slot = threadIdx.x / cpr;
    if (slot >= slots) return;
    const uint32_t wid = work_index(blockIdx.x, gridDim.x);
    const int rb = wid % a.row_blocks;
    const int64_t bh = wid / a.row_blocks;
    const int64_t h = bh % a.H, b = bh / a.H;
    double f[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) f[p] = rope_inv_freq(4 * c + p, a.d, a.log2_base);
    const __bf16 *xb = a.x + b * a.x_sb + h * a.x_sh + 8 * c;
    __bf16 *yb = a.y + b * a.y_sb + h * a.y_sh + 8 * c;
    const int n_end = min(a.N, (rb + 1) * ROPE_ROWS);
    for (int n = rb * ROPE_ROWS + slot; n < n_end; n += slots) {
        const u32x4 v = *(const u32x4 *)(xb + (int64_t)n * a.x_sn);
        *(u32x4 *)(yb + (int64_t)n * a.y_sn) = rope_chunk_f(v, n, f);
    }
}

}  // namespace attn
