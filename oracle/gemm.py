"""fp64 CPU oracle of the bf16 GEMM C = A·Bᵀ (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module. It computes the plain definition
    C[m, n] = sum_k A[m, k] * B[n, k]
(the Q/K/V and O projections of the decoder chain, "CS149 L11: Programming
Specialized Hardware", section 6) in fp64 with numpy's matrix product as the
one library step, on exactly the values the GPU receives (bf16 widened to
fp64, which is exact). It shares nothing with the HIP library.

    gemm_fp64(a, b, rows=None) -> C
        a: [M, K], b: [N, K] (torch tensors or numpy arrays of any float dtype)
        rows: optional int array of row indices m; then C is [len(rows), N].
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def gemm_fp64(a, b, rows=None) -> np.ndarray:
    A = _f64(a)
    B = _f64(b)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[1]:
        raise ValueError("gemm_fp64 needs a [M, K] and b [N, K]")
    if rows is not None:
        A = A[np.asarray(rows, dtype=np.int64)]
    return A @ B.T
