"""Pins of the RoPE oracle against properties that do not restate its
formula: a rotation per pair (norms kept), identity at position 0, the
closed form of the first pair (angle = position), and the defining relative
property: a score between rotated q and k depends only on their distance."""
import numpy as np

from oracle.rope import rope_fp64


def test_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((1, 8))
    np.testing.assert_array_equal(rope_fp64(x, 10000.0), x)


def test_pair_norms_are_kept():
    x = np.random.default_rng(1).standard_normal((2, 3, 50, 16))
    y = rope_fp64(x, 500000.0)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-12, atol=1e-14)


def test_first_pair_turns_by_the_position():
    # pair 0 has frequency base^0 = 1: (1, 0) at position n becomes (cos n, sin n)
    N = 40
    x = np.zeros((N, 4))
    x[:, 0] = 1.0
    y = rope_fp64(x, 10000.0)
    n = np.arange(N)
    np.testing.assert_allclose(y[:, 0], np.cos(n), atol=1e-15)
    np.testing.assert_allclose(y[:, 1], np.sin(n), atol=1e-15)


def test_scores_depend_only_on_distance():
    rng = np.random.default_rng(2)
    d = 32
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    N = 64
    Q = rope_fp64(np.tile(q, (N, 1)), 10000.0)
    K = rope_fp64(np.tile(k, (N, 1)), 10000.0)
    S = Q @ K.T
    for delta in (-7, 0, 5, 31):
        diag = np.array([S[i, i - delta] for i in range(max(0, delta), min(N, N + delta))])
        np.testing.assert_allclose(diag, diag[0], rtol=0, atol=1e-11)


def test_position_offset_shifts_rows():
    x = np.random.default_rng(3).standard_normal((10, 8))
    full = rope_fp64(np.concatenate([np.zeros((3, 8)), x]), 10000.0)
    np.testing.assert_allclose(rope_fp64(x, 10000.0, pos0=3), full[3:], atol=1e-14)
