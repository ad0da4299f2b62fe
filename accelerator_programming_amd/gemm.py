"""ctypes binding of include/tile_gemm.h (argument marshalling only).

``tile_gemm_bf16_nt`` mirrors the C entry point; ``gemm_nt`` wraps it for
torch tensors: C = A·Bᵀ with A [M, K], B [N, K] and C [M, N], all bf16 on the
GPU with unit inner stride. The product runs in the HIP library; there is no
fallback path.
"""
from __future__ import annotations

from . import attn


def tile_gemm_bf16_nt(M: int, N: int, K: int, A: int, lda: int, B: int, ldb: int, C: int,
                      ldc: int, stream: int | None = None) -> None:
    st = attn.lib().tile_gemm_bf16_nt(int(M), int(N), int(K), A, int(lda), B, int(ldb), C,
                                      int(ldc), stream)
    if st != attn.ATTN_OK:
        raise attn.AttnError(st, "tile_gemm_bf16_nt")


def gemm_nt(a, b, out=None, stream=None):
    """C = A·Bᵀ for bf16 device tensors a [M, K] and b [N, K] (row strides
    free, inner stride 1). Writes into ``out`` ([M, N] bf16) when given."""
    import torch
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("gemm_nt needs a [M, K] and b [N, K]")
    for t in (a, b):
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.stride(1) != 1:
            raise ValueError("gemm_nt needs bf16 device tensors with unit inner stride")
    M, K = a.shape
    N = b.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if (tuple(out.shape) != (M, N) or out.dtype != torch.bfloat16 or not out.is_cuda
            or out.stride(1) != 1):
        raise ValueError("out must be a [M, N] bf16 device tensor with unit inner stride")
    s = stream if stream is not None else torch.cuda.current_stream()
    tile_gemm_bf16_nt(M, N, K, a.data_ptr(), a.stride(0), b.data_ptr(), b.stride(0),
                      out.data_ptr(), out.stride(0), s.cuda_stream)
    return out
