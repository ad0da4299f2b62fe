"""Pins of the oracle's dropout stage (test infrastructure only).

Nothing here re-types the generator: the Philox4x32-10 block is held to the
known-answer vectors published with the generator (Salmon, Moraes, Dror,
Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11, and the test
vectors of its reference distribution, Random123), and the rest are what
dropout and a counter-based generator must satisfy whatever their internals
are - the keep rate, unbiasedness over seeds, the exact form of each kept
value, independence of lse, determinism in (seed, b, h, i, j), and diffusion
and injectivity of the block. Deliberately broken copies of the generator
(a wrong Weyl constant, a wrong multiplier, a missing round, the high and
low product halves swapped) must each fail a pin."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle

# Published Philox4x32-10 known answers: (counter words, key words) -> output
# words, all hexadecimal, word 0 first.
PHILOX_KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


def _philox_with(lib):
    """philox4x32_10 bound to another build of the oracle's C source."""
    def f(ctr, key):
        c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32).reshape(4))
        k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32).reshape(2))
        out = np.empty(4, dtype=np.uint32)
        lib.oracle_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
        return out
    return f


def test_philox_known_answer_vectors(philox=None):
    philox = philox or oracle.philox4x32_10
    for ctr, key, want in PHILOX_KAT:
        got = tuple(int(x) for x in philox(ctr, key))
        assert got == want, "Philox4x32-10%s%s -> %s, published %s" % (
            ctr, key, " ".join("%08x" % x for x in got), " ".join("%08x" % x for x in want))


def inputs(B, Hq, Hkv, N, d, seed, Nkv=None, dv=None):
    g = torch.Generator().manual_seed(seed)
    Nkv = Nkv or N
    dv = dv or d
    q = torch.randn(B, Hq, N, d, generator=g)
    k = torch.randn(B, Hkv, Nkv, d, generator=g)
    v = torch.randn(B, Hkv, Nkv, dv, generator=g)
    return q, k, v


def test_v_identity_exposes_each_kept_probability():
    # V = I (N_kv = d_v): O[i, j] = p_ij keep_ij * 256 / (256 - thr), with p
    # the plain softmax - every element is either 0 or exactly the scaled p
    N, thr = 64, 64
    g = torch.Generator().manual_seed(3)
    q = torch.randn(1, 2, N, 16, generator=g)
    k = torch.randn(1, 2, N, 16, generator=g)
    v = torch.eye(N).reshape(1, 1, N, N).repeat(1, 2, 1, 1)
    P, _, _ = oracle.attention_fp64(q, k, v, False, 0.25)
    O, _, _ = oracle.attention_fp64(q, k, v, False, 0.25, drop_thr=thr, seed=7)
    scaled = P * 256.0 / (256 - thr)
    kept = np.isclose(O, scaled, rtol=1e-12, atol=0)
    dropped = O == 0.0
    assert (kept | dropped).all()
    assert kept.any() and dropped.any()


@pytest.mark.parametrize("thr", [26, 64, 128, 230])
def test_keep_rate_matches_probability(thr):
    # 128 x 128 elements per head, 2 heads: binomial count of kept elements
    N = 128
    g = torch.Generator().manual_seed(thr)
    q = torch.randn(1, 2, N, 8, generator=g)
    k = torch.randn(1, 2, N, 8, generator=g)
    v = torch.eye(N).reshape(1, 1, N, N).repeat(1, 2, 1, 1)
    O, _, _ = oracle.attention_fp64(q, k, v, False, 0.3, drop_thr=thr, seed=99)
    n = O.size
    kept = int((O != 0.0).sum())
    p_keep = 1.0 - thr / 256.0
    z = (kept - n * p_keep) / np.sqrt(n * p_keep * (1 - p_keep))
    assert abs(z) < 5.0, (kept, n * p_keep, z)


def test_neighbouring_decisions_uncorrelated():
    N, thr = 128, 128
    g = torch.Generator().manual_seed(5)
    q = torch.randn(1, 4, N, 8, generator=g)
    k = torch.randn(1, 4, N, 8, generator=g)
    v = torch.eye(N).reshape(1, 1, N, N).repeat(1, 4, 1, 1)
    O, _, _ = oracle.attention_fp64(q, k, v, False, 0.3, drop_thr=thr, seed=1234)
    keep = (O != 0.0).astype(np.float64)
    for a, b in ((keep[..., :-1], keep[..., 1:]),            # key j and j + 1
                 (keep[..., :-1, :], keep[..., 1:, :]),      # row i and i + 1
                 (keep[:, :-1], keep[:, 1:])):               # head h and h + 1
        r = np.corrcoef(a.ravel(), b.ravel())[0, 1]
        assert abs(r) < 0.03, r


def test_unbiased_over_seeds():
    q, k, v = inputs(1, 1, 1, 12, 4, seed=8)
    O, _, _ = oracle.attention_fp64(q, k, v, True, 0.5)
    samples = np.stack([oracle.attention_fp64(q, k, v, True, 0.5, drop_thr=64, seed=s)[0]
                        for s in range(400)])
    mean = samples.mean(0)
    se = samples.std(0) / np.sqrt(len(samples))
    assert (np.abs(mean - O) <= 6 * se + 1e-12).all()


def test_lse_is_that_before_dropout():
    q, k, v = inputs(2, 4, 2, 40, 8, seed=9)
    _, L, _ = oracle.attention_fp64(q, k, v, True, 0.35)
    _, Ld, _ = oracle.attention_fp64(q, k, v, True, 0.35, drop_thr=100, seed=3)
    np.testing.assert_array_equal(L, Ld)


def test_decisions_depend_only_on_position_and_seed():
    q, k, v = inputs(2, 4, 2, 33, 8, seed=10)
    O, _, _ = oracle.attention_fp64(q, k, v, False, 0.3, drop_thr=77, seed=5)
    rows = np.array([[1, 3, 32], [0, 0, 0], [1, 0, 17]])
    Or, _, _ = oracle.attention_fp64(q, k, v, False, 0.3, rows=rows, drop_thr=77, seed=5)
    np.testing.assert_array_equal(Or, O[rows[:, 0], rows[:, 1], rows[:, 2]])
    O2, _, _ = oracle.attention_fp64(q, k, v, False, 0.3, drop_thr=77, seed=5, threads=1)
    np.testing.assert_array_equal(O, O2)
    O3, _, _ = oracle.attention_fp64(q, k, v, False, 0.3, drop_thr=77, seed=6)
    assert not np.array_equal(O, O3)


def test_threshold_out_of_range_is_rejected():
    q, k, v = inputs(1, 1, 1, 4, 4, seed=11)
    with pytest.raises(ValueError):
        oracle.attention_fp64(q, k, v, False, 0.5, drop_thr=256, seed=1)


def test_philox_block_is_injective_on_a_sample():
    outs = {tuple(oracle.philox4x32_10([i, 0, 0, 0], [1, 2])) for i in range(4096)}
    assert len(outs) == 4096


def test_philox_block_diffuses_single_bit_changes():
    # flipping one counter bit changes about half of the 128 output bits
    rng = np.random.default_rng(0)
    flips = []
    for _ in range(200):
        ctr = rng.integers(0, 2 ** 32, 4, dtype=np.uint64).astype(np.uint32)
        key = rng.integers(0, 2 ** 32, 2, dtype=np.uint64).astype(np.uint32)
        bit = rng.integers(0, 128)
        ctr2 = ctr.copy()
        ctr2[bit // 32] ^= np.uint32(1 << (bit % 32))
        a = oracle.philox4x32_10(ctr, key)
        b = oracle.philox4x32_10(ctr2, key)
        flips.append(sum(bin(int(x) ^ int(y)).count("1") for x, y in zip(a, b)))
    flips = np.array(flips)
    assert 60 < flips.mean() < 68
    assert flips.min() > 30


# --------------------------------------------------------------------------
# Mutants of the generator: each must fail the known-answer pin.
# --------------------------------------------------------------------------
PHILOX_MUTANTS = {
    "weyl_constant": ("k[1] += 0xBB67AE85u;", "k[1] += 0xBB67AE86u;"),
    "multiplier": ("(uint64_t)0xD2511F53u * c[0]", "(uint64_t)0xD2511F57u * c[0]"),
    "nine_rounds": ("for (int r = 0; r < 10; ++r) {\n        if (r > 0)",
                    "for (int r = 0; r < 9; ++r) {\n        if (r > 0)"),
    "halves_swapped": ("const uint32_t n1 = (uint32_t)p1;", "const uint32_t n1 = (uint32_t)(p1 >> 16);"),
}


@pytest.mark.parametrize("name", sorted(PHILOX_MUTANTS))
def test_known_answers_catch_generator_mutant(name, tmp_path):
    import ctypes
    src = open(os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")).read()
    old, new = PHILOX_MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor not found: " + old
    path_c = tmp_path / ("mut_%s.c" % name)
    path_c.write_text(src.replace(old, new))
    path_so = tmp_path / ("libmut_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o",
                    str(path_so), str(path_c), "-lm"], check=True)
    lib = ctypes.CDLL(str(path_so))
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_philox4x32_10.argtypes = [ctypes.c_void_p] * 3
    with pytest.raises(AssertionError):
        test_philox_known_answer_vectors(_philox_with(lib))
