/*
 * tile_gemm.h - C ABI of the MI355X (gfx950) bf16 GEMM built on the attention
 * kernel's tile layer (the same 32x32x16 MFMA fragments, swizzled LDS slabs
 * and LDS-DMA staging).
 *
 * The operation is C = A·Bᵀ: the Q/K/V and O projections that sit on either
 * side of attention in a decoder layer ("CS149 L11: Programming Specialized
 * Hardware", section 6, the Llama 3.1 8B chain: Q/K/V GEMMs, QKᵀ, ..., the O
 * GEMM), computed as in that page's matrix-multiply metapipeline (section 5,
 * slides 51-53: slabs of A and B staged on chip, multiplied into an output
 * tile that stays on chip for the whole K loop) with the disjoint-output-tile
 * blocking of "Distilling a 4.5 hour CUDA talk", section 5.
 *
 * Shares attn_status (and attn_status_str) with attn_fwd.h.
 */
#ifndef TILE_GEMM_H
#define TILE_GEMM_H

#include <stdint.h>

#include "attn_fwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * C[m, n] = sum_k A[m, k] * B[n, k], m < M, n < N, k < K.
 *
 *   A: device pointer, bf16, [M, K] row-major, row stride lda elements.
 *   B: device pointer, bf16, [N, K] row-major, row stride ldb elements (the
 *      [out, in] layout of a weight matrix).
 *   C: device pointer, bf16, [M, N] row-major, row stride ldc elements;
 *      written, not read. Products accumulate in fp32 and each element is
 *      rounded to bf16 once (round to nearest even).
 *   stream: a hipStream_t (NULL = the default stream); the call only queues
 *      the work and never synchronizes.
 *
 * Requirements (ATTN_ERR_INVALID otherwise, before any HIP call):
 *   M, N, K >= 0; K % 8 == 0; N % 4 == 0; lda >= K, ldb >= K, ldc >= N;
 *   lda and ldb multiples of 8, ldc a multiple of 4; A and B 16-byte
 *   aligned, C 8-byte aligned; 256 * lda and 256 * ldb below 2^30; M and N
 *   below 2^31. M == 0 or N == 0 queues nothing; K == 0 writes zeros.
 * The caller owns all buffers and keeps them alive until the stream work is
 * done; A and B must not overlap C. HIP launch failures return ATTN_ERR_HIP.
 */
attn_status tile_gemm_bf16_nt(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                              const void *B, int64_t ldb, void *C, int64_t ldc, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TILE_GEMM_H */
