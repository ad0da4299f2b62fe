"""Parity of the HIP bf16 GEMM (C = A·Bᵀ) with the fp64 oracle, through the C
ABI.

Bound (same inputs on both sides): the GPU sums the products in fp32 and
rounds once to bf16, so for every element
    |C_gpu - C_ref| <= ulp_bf16(|C_ref| + d) / 2 + d,   d = gamma_K * sum_k |a_mk| |b_nk|
with gamma_K = K u / (1 - K u), u = 2^-24 (any summation order in fp32) and
ulp_bf16(x) = 2^(floor(log2 x) - 7) (8 significant bits). Small-integer
inputs make both sides exact, so that case is compared bit for bit.
"""
import numpy as np
import pytest
import torch

from accelerator_programming_amd import gemm
from accelerator_programming_amd.inputs import G1, G2, GemmWorkload, make_gemm_inputs
from oracle.gemm import gemm_fp64

pytestmark = pytest.mark.gpu


def check(c_gpu, a, b, rows=None):
    A = a.float().cpu().numpy().astype(np.float64)
    B = b.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        A = A[rows]
    ref = gemm_fp64(A, B)
    K = A.shape[1]
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    d = gamma * (np.abs(A) @ np.abs(B).T)
    mag = np.abs(ref) + d
    ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 2.0 ** -126))) - 7)
    tol = 0.5 * ulp + d + 2.0 ** -133
    got = c_gpu.float().cpu().numpy().astype(np.float64)
    if rows is not None and got.shape[0] != len(rows):
        got = got[rows]
    assert np.isfinite(got).all()
    bad = np.abs(got - ref) > tol
    assert not bad.any(), "%d elements out of bound; worst |d| = %.3e" % (
        bad.sum(), np.abs(got - ref).max())


def randn_bf16(*shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16).cuda()


@pytest.mark.parametrize("M,N,K", [
    (300, 264, 200),    # ragged in M and N, K not a multiple of the 32-wide step
    (256, 256, 32),     # exactly one tile and one step
    (512, 768, 1024),   # several tiles and steps
    (1, 4, 8),          # the smallest accepted shape
    (100, 1000, 8),     # one partial step, wide
])
def test_parity_shapes(M, N, K):
    a = randn_bf16(M, K, seed=M + N + K)
    b = randn_bf16(N, K, seed=M * N + K)
    check(gemm.gemm_nt(a, b), a, b)


def test_small_integers_are_exact():
    # entries in {-1, 0, 1} and K = 256: every sum is an integer of magnitude
    # <= 256, exact in fp32 and in bf16
    g = torch.Generator().manual_seed(5)
    a = torch.randint(-1, 2, (257, 256), generator=g).to(torch.bfloat16).cuda()
    b = torch.randint(-1, 2, (260, 256), generator=g).to(torch.bfloat16).cuda()
    c = gemm.gemm_nt(a, b)
    ref = gemm_fp64(a, b)
    np.testing.assert_array_equal(c.float().cpu().numpy().astype(np.float64), ref)


def test_strided_operands_and_output():
    M, N, K = 200, 136, 96
    abig = randn_bf16(M, K + 40, seed=11)
    bbig = randn_bf16(N, K + 24, seed=12)
    a, b = abig[:, 8:8 + K], bbig[:, :K]
    out_big = torch.full((M, N + 20), 7.0, dtype=torch.bfloat16, device="cuda")
    out = out_big[:, :N]
    gemm.gemm_nt(a, b, out=out)
    check(out, a, b)
    # columns past N are untouched
    assert (out_big[:, N:] == 7.0).all()


def test_output_rows_staged_with_a_partial_last_chunk():
    # ldc a multiple of 8 (the epilogue goes through LDS) and N = 268: the
    # last 16-byte piece of each row holds 4 columns of C and 4 past N
    M, N, K = 300, 268, 96
    a = randn_bf16(M, K, seed=13)
    b = randn_bf16(N, K, seed=14)
    out_big = torch.full((M, 280), 7.0, dtype=torch.bfloat16, device="cuda")
    out = out_big[:, :N]
    gemm.gemm_nt(a, b, out=out)
    check(out, a, b)
    assert (out_big[:, N:] == 7.0).all()


def test_k_zero_writes_zeros():
    out = torch.full((64, 32), 3.0, dtype=torch.bfloat16, device="cuda")
    # zero-width operands have no storage: hand the C ABI aligned stand-ins of
    # their own (A and B must not overlap C), which it never reads
    a_stub = torch.empty(8, dtype=torch.bfloat16, device="cuda")
    b_stub = torch.empty(8, dtype=torch.bfloat16, device="cuda")
    gemm.tile_gemm_bf16_nt(64, 32, 0, a_stub.data_ptr(), 0, b_stub.data_ptr(), 0, out.data_ptr(),
                           32, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert (out == 0).all()


def test_non_default_stream_and_repeatability():
    a = randn_bf16(384, 512, seed=21)
    b = randn_bf16(320, 512, seed=22)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c1 = gemm.gemm_nt(a, b, stream=s)
        c2 = gemm.gemm_nt(a, b, stream=s)
    s.synchronize()
    assert torch.equal(c1, c2)
    check(c1, a, b)


@pytest.mark.parametrize("w", [G1, G2], ids=lambda w: w.name.split("_")[0])
def test_full_size_sampled_rows(w):
    a, b = make_gemm_inputs(w, "cuda")
    c = gemm.gemm_nt(a, b)
    rows = np.unique(np.concatenate([[0, 1, w.M - 1, w.M // 2],
                                     np.random.default_rng(w.seed).integers(0, w.M, 28)]))
    check(c[torch.as_tensor(rows, device="cuda")], a, b, rows=rows)
