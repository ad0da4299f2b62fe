"""Pins of the RoPE oracle against properties that do not restate its
formula: a rotation per pair (norms kept), identity at position 0, closed
forms of single pairs (pair 0 turns by the position; with d = 4 and
base = 100 pair 1 has frequency exactly 1/10; the last pair of d = 128 turns
by n * base^(-126/128), the frequency the RoFormer paper's schedule gives
it), and the defining relative property: a score between rotated q and k
depends only on their distance. Deliberately broken copies of the oracle (a
halved exponent, a frequency index off by one, the pair's two outputs
swapped, sine with the wrong sign) must each fail a pin."""
import math
import os
import types

import numpy as np
import pytest

import oracle.rope
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


def test_second_pair_closed_form(rope=None):
    # d = 4, base = 100: pair 1 has frequency 100^(-2/4) = 1/10, so (1, 0) in
    # pair 1 at position n becomes (cos(n/10), sin(n/10)); pair 0 is untouched
    # when it holds zeros
    rope = rope or rope_fp64
    N = 50
    x = np.zeros((N, 4))
    x[:, 2] = 1.0
    y = rope(x, 100.0)
    n = np.arange(N)
    np.testing.assert_allclose(y[:, 2], np.cos(n / 10.0), atol=1e-14)
    np.testing.assert_allclose(y[:, 3], np.sin(n / 10.0), atol=1e-14)
    np.testing.assert_array_equal(y[:, :2], 0.0)


def test_last_pair_of_d128(rope=None):
    # (0, 1) in the last pair (k = 63) at position n: the rotation by
    # theta = n * 10000^(-126/128) maps (0, 1) to (-sin theta, cos theta)
    rope = rope or rope_fp64
    d, N = 128, 300
    x = np.zeros((N, d))
    x[:, d - 1] = 1.0
    y = rope(x, 10000.0)
    theta = np.arange(N) * math.exp(-126.0 / 128.0 * math.log(10000.0))
    np.testing.assert_allclose(y[:, d - 2], -np.sin(theta), atol=1e-13)
    np.testing.assert_allclose(y[:, d - 1], np.cos(theta), atol=1e-13)


def test_every_pair_frequency_at_position_one(rope=None):
    # at position 1 pair k turns by base^(-2k/d): read each pair's angle back
    rope = rope or rope_fp64
    d, base = 16, 500000.0
    x = np.zeros((2, d))
    x[:, 0::2] = 1.0
    y = rope(x, base)
    ang = np.arctan2(y[1, 1::2], y[1, 0::2])
    want = np.array([base ** (-2.0 * k / d) for k in range(d // 2)])
    np.testing.assert_allclose(ang, want, rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# Mutants of the oracle's source: each must fail at least one pin.
# --------------------------------------------------------------------------
ROPE_MUTANTS = {
    "half_exponent": ("-2.0 * k / d", "-1.0 * k / d"),
    "index_off_by_one": ("k = np.arange(d // 2, dtype=np.float64)",
                         "k = np.arange(1, d // 2 + 1, dtype=np.float64)"),
    "outputs_swapped": ("Y[..., 0::2] = xe * c - xo * s", "Y[..., 0::2] = xe * s + xo * c"),
    "sine_sign": ("Y[..., 1::2] = xe * s + xo * c", "Y[..., 1::2] = -xe * s + xo * c"),
}

ROPE_PINS = [
    lambda f: test_second_pair_closed_form(f),
    lambda f: test_last_pair_of_d128(f),
    lambda f: test_every_pair_frequency_at_position_one(f),
]


@pytest.mark.parametrize("name", sorted(ROPE_MUTANTS))
def test_pins_catch_rope_mutant(name):
    src = open(os.path.join(os.path.dirname(oracle.rope.__file__), "rope.py")).read()
    old, new = ROPE_MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor not found: " + old
    mod = types.ModuleType("rope_mutant_" + name)
    exec(compile(src.replace(old, new), "rope_mutant.py", "exec"), mod.__dict__)
    caught = 0
    for pin in ROPE_PINS:
        try:
            pin(mod.rope_fp64)
        except AssertionError:
            caught += 1
    assert caught > 0, "mutant %s survived every pin" % name


def test_unmutated_rope_passes_every_pin():
    for pin in ROPE_PINS:
        pin(rope_fp64)
