"""Pins of the fp64 GEMM oracle (C = A·Bᵀ) against facts that do not come
from the oracle itself: explicit loops, closed forms, and identities."""
import numpy as np
import pytest

from oracle.gemm import gemm_fp64


def _loops(A, B):
    M, K = A.shape
    N = B.shape[0]
    C = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            s = 0.0
            for k in range(K):
                s += float(A[m, k]) * float(B[n, k])
            C[m, n] = s
    return C


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 4), (7, 2, 9)])
def test_brute_force_loops(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((N, K))
    np.testing.assert_allclose(gemm_fp64(A, B), _loops(A, B), rtol=0, atol=1e-12)


def test_closed_form_ones_times_ramp():
    # A = 1, B[n, k] = n + k: C[m, n] = K n + K (K - 1) / 2
    M, N, K = 4, 6, 10
    A = np.ones((M, K))
    B = np.add.outer(np.arange(N), np.arange(K)).astype(np.float64)
    want = np.tile(K * np.arange(N) + K * (K - 1) / 2, (M, 1))
    np.testing.assert_array_equal(gemm_fp64(A, B), want)


def test_identity_gives_transpose():
    # A = I (M = K): C[m, n] = B[n, m], so C is Bᵀ (B is [N, K], not square)
    K, N = 5, 3
    B = np.arange(N * K, dtype=np.float64).reshape(N, K)
    np.testing.assert_array_equal(gemm_fp64(np.eye(K), B), B.T)


def test_swap_operands_transposes():
    rng = np.random.default_rng(1)
    A = rng.standard_normal((4, 6))
    B = rng.standard_normal((3, 6))
    np.testing.assert_allclose(gemm_fp64(B, A), gemm_fp64(A, B).T, rtol=0, atol=1e-12)


def test_row_subset():
    rng = np.random.default_rng(2)
    A = rng.standard_normal((9, 8))
    B = rng.standard_normal((5, 8))
    rows = np.array([8, 0, 3])
    np.testing.assert_array_equal(gemm_fp64(A, B, rows), gemm_fp64(A, B)[rows])


def test_bf16_inputs_widen_exactly():
    torch = pytest.importorskip("torch")
    a = torch.tensor([[1.5, -2.0, 0.0078125, 3.0]], dtype=torch.bfloat16)
    b = torch.tensor([[2.0, 0.5, 128.0, -1.0]], dtype=torch.bfloat16)
    # 3 - 1 + 1 - 3 = 0 exactly
    assert gemm_fp64(a, b)[0, 0] == 0.0
