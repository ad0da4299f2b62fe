// C ABI of the gfx950 bf16 GEMM (include/tile_gemm.h): host-side checks and
// the launch of attn::gemm_bf16_nt_kernel.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/tile_gemm.h"
#include "gemm_kernel.hpp"

extern "C" attn_status tile_gemm_bf16_nt(int64_t M, int64_t N, int64_t K, const void *A,
                                         int64_t lda, const void *B, int64_t ldb, void *C,
                                         int64_t ldc, void *stream) {
    using G = attn::GemmCfg;
    if (M < 0 || N < 0 || K < 0) return ATTN_ERR_INVALID;
    if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 30))
        return ATTN_ERR_INVALID;
    if (K % 8 != 0 || N % 4 != 0) return ATTN_ERR_INVALID;
    if (lda < K || ldb < K || ldc < N) return ATTN_ERR_INVALID;
    if (lda % 8 != 0 || ldb % 8 != 0 || ldc % 4 != 0) return ATTN_ERR_INVALID;
    // byte offsets within one 256-row slab stay below 2^31 (the offset that
    // marks a chunk past K as out of range)
    if ((int64_t)G::BM * lda >= ((int64_t)1 << 30) || (int64_t)G::BN * ldb >= ((int64_t)1 << 30))
        return ATTN_ERR_INVALID;
    if (M == 0 || N == 0) return ATTN_OK;
    if (!A || !B || !C) return ATTN_ERR_INVALID;
    if (((uintptr_t)A & 15) || ((uintptr_t)B & 15) || ((uintptr_t)C & 7)) return ATTN_ERR_INVALID;
    const int64_t tiles_m = (M + G::BM - 1) / G::BM, tiles_n = (N + G::BN - 1) / G::BN;
    if (tiles_m * tiles_n >= ((int64_t)1 << 31)) return ATTN_ERR_INVALID;

    attn::GemmArgs a;
    a.a = (const __bf16 *)A;
    a.b = (const __bf16 *)B;
    a.c = (__bf16 *)C;
    a.M = (int32_t)M;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    a.lda = (int32_t)lda;
    a.ldb = (int32_t)ldb;
    a.ldc = (int32_t)ldc;
    a.tiles_m = (int32_t)tiles_m;
    a.tiles_n = (int32_t)tiles_n;
    // 16-byte C rows: the epilogue stores whole row pieces through LDS
    a.stage_c = (ldc % 8 == 0 && ((uintptr_t)C & 15) == 0) ? 1 : 0;
    hipLaunchKernelGGL(attn::gemm_bf16_nt_kernel, dim3((uint32_t)(tiles_m * tiles_n)), dim3(G::NT), 0,
                       (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}
