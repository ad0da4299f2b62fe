"""Tile-layer probes on the GPU: each primitive the attention kernel is built
from, checked bit-exactly with inputs whose products are exact in fp32."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SELFTEST = os.path.join(ROOT, "accelerator_programming_amd", "libattn_tile_selftest.so")


@pytest.fixture(scope="module")
def lib():
    L = ctypes.CDLL(SELFTEST)
    for n in ("tile_selftest_mfma", "tile_selftest_mfma16", "tile_selftest_xhalf"):
        getattr(L, n).restype = ctypes.c_int
        getattr(L, n).argtypes = [ctypes.c_void_p] * 4
    for n in ("tile_selftest_qk", "tile_selftest_pv"):
        getattr(L, n).restype = ctypes.c_int
        getattr(L, n).argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 4
    return L


def stream():
    return torch.cuda.current_stream().cuda_stream


def small_ints(shape, seed, lo=-4, hi=5):
    g = torch.Generator().manual_seed(seed)
    return torch.randint(lo, hi, shape, generator=g).float()


def test_mfma_32x32x16_fragment_layout(lib):
    A = small_ints((32, 16), 1)
    B = small_ints((16, 32), 2)
    Ad, Bd = A.bfloat16().cuda(), B.bfloat16().cuda()
    C = torch.full((32, 32), float("nan"), device="cuda")
    assert lib.tile_selftest_mfma(Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(C.cpu(), A @ B)


def test_mfma_16x16x32_fragment_layout(lib):
    A = small_ints((16, 32), 4)
    B = small_ints((32, 16), 5)
    Ad, Bd = A.bfloat16().cuda(), B.bfloat16().cuda()
    C = torch.full((16, 16), float("nan"), device="cuda")
    assert lib.tile_selftest_mfma16(Ad.data_ptr(), Bd.data_ptr(), C.data_ptr(), stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(C.cpu(), A @ B)


def test_cross_half_max_and_sum(lib):
    x = small_ints((64,), 3, -100, 100) / 8
    xd = x.cuda()
    mx = torch.empty(64, device="cuda")
    sm = torch.empty(64, device="cuda")
    assert lib.tile_selftest_xhalf(xd.data_ptr(), mx.data_ptr(), sm.data_ptr(), stream()) == 0
    torch.cuda.synchronize()
    other = x.roll(32)
    assert torch.equal(mx.cpu(), torch.maximum(x, other))
    assert torch.equal(sm.cpu(), x + other)


@pytest.mark.parametrize("d", [64, 128])
def test_qk_through_swizzled_k_tile(lib, d):
    K = small_ints((32, d), 6, -2, 3)
    Q = small_ints((32, d), 7, -2, 3)
    St = torch.full((32, 32), float("nan"), device="cuda")
    Kd, Qd = K.bfloat16().cuda(), Q.bfloat16().cuda()
    assert lib.tile_selftest_qk(d, Kd.data_ptr(), Qd.data_ptr(), St.data_ptr(), stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(St.cpu(), K @ Q.t())


@pytest.mark.parametrize("d", [64, 128])
def test_pv_through_transposed_v_reads(lib, d):
    # St[key][query] in the accumulator layout; P = St^T rounded to bf16 (exact
    # here: quarter-integers), V small integers -> O = P·V exact in fp32.
    St = small_ints((64, 32), 4) / 4
    V = small_ints((64, d), 5)
    Sd, Vd = St.cuda(), V.bfloat16().cuda()
    O = torch.full((32, d), float("nan"), device="cuda")
    assert lib.tile_selftest_pv(d, Sd.data_ptr(), Vd.data_ptr(), O.data_ptr(), stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(O.cpu(), St.t() @ V)


def test_mfma_rate_probe_counts_every_wave(lib):
    # the probe behind `bench.py --mfma-ceiling`: every wave of every
    # workgroup reports a positive cycle and tick count, cycles at least the
    # 32 per MFMA the pipe needs, and the host rejects bad arguments
    lib.tile_selftest_mfma_rate.restype = ctypes.c_int
    lib.tile_selftest_mfma_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint,
                                            ctypes.c_void_p]
    nb, iters = 8, 200
    out = torch.zeros(nb * 16, dtype=torch.int64, device="cuda")
    assert lib.tile_selftest_mfma_rate(out.data_ptr(), nb, iters, stream()) == 0
    torch.cuda.synchronize()
    o = out.view(-1, 2).cpu()
    assert bool((o[:, 0] >= 32 * 16 * iters).all()) and bool((o[:, 1] > 0).all())
    assert lib.tile_selftest_mfma_rate(out.data_ptr(), 0, iters, stream()) == -1
    assert lib.tile_selftest_mfma_rate(out.data_ptr(), nb, 0, stream()) == -1
    assert lib.tile_selftest_mfma_rate(None, nb, iters, stream()) == -1
