"""Pins for the fp64 oracle: it is checked against things other than itself.

Each check below follows from the definition of attention forward on the
pages (Q·Kᵀ -> scale -> mask -> softmax as Map(exp) -> Reduce(+) -> Zip(/) ->
×V; "CS149 L11: Programming Specialized Hardware", section 5, slides 48 and
54) or from mathematics, never from the oracle's own code:
  * worked examples with closed forms (tests/golden/*.json);
  * a library routine on tiny inputs (torch's scaled_dot_product_attention in
    fp64, and scipy's logsumexp over explicitly materialized scores);
  * invariants: probability rows sum to one, single key, constant V, causal
    first row, Q = 0 averages, GQA = MHA with repeated heads, key-permutation
    invariance, causal independence of later keys, split/merge through lse,
    key-shift invariance;
  * mutants: deliberately broken copies of the C source must each fail one of
    the pins above (so a dropped term, a wrong sign or a wrong index would be
    caught).
"""
import json
import math
import os
import subprocess

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    # fp32 values: the oracle reads fp32, so references use the same values
    return (torch.randn(shape, generator=g, dtype=torch.float32) * scale).double()


def f32(x):
    """The scale crosses the oracle's interface as fp32."""
    return float(np.float32(x))


def run(q, k, v, causal, scale, lib_path=None, **kw):
    return oracle.attention_fp64(q, k, v, causal, scale, lib_path=lib_path, **kw)[:2]


# --------------------------------------------------------------------------
# Worked examples with closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["two_key_logistic.json", "causal_uniform_3.json"])
def test_golden_closed_forms(name, lib_path=None):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    O, lse = run(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]), g["causal"], g["scale"],
                 lib_path=lib_path)
    np.testing.assert_allclose(O, np.array(g["expected_o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(g["expected_lse"]), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Library routines on tiny inputs
# --------------------------------------------------------------------------
SHAPES = [
    # B, Hq, Hkv, Nq, Nkv, dqk, dv, causal
    (1, 1, 1, 1, 1, 1, 1, False),
    (2, 3, 3, 5, 7, 4, 3, False),
    (1, 4, 2, 6, 6, 5, 2, True),
    (2, 6, 3, 9, 9, 8, 6, True),
    (1, 2, 1, 3, 11, 16, 4, False),
]


def sdpa_reference(q, k, v, causal, scale):
    group = q.shape[1] // k.shape[1]
    kk = k.repeat_interleave(group, dim=1)
    vv = v.repeat_interleave(group, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=causal,
                                                         scale=float(np.float32(scale)))
    s = float(np.float32(scale)) * (q @ kk.transpose(-1, -2))
    if causal:
        n = q.shape[2]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), -math.inf)
    lse = logsumexp(s.numpy(), axis=-1)
    return o.numpy(), lse


@pytest.mark.parametrize("shape", SHAPES)
def test_matches_library_sdpa(shape, lib_path=None):
    B, Hq, Hkv, Nq, Nkv, dqk, dv, causal = shape
    q, k, v = rnd((B, Hq, Nq, dqk), 1), rnd((B, Hkv, Nkv, dqk), 2), rnd((B, Hkv, Nkv, dv), 3)
    scale = 1.0 / math.sqrt(dqk)
    O, lse = run(q, k, v, causal, scale, lib_path=lib_path)
    Oref, lseref = sdpa_reference(q, k, v, causal, scale)
    np.testing.assert_allclose(O, Oref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lseref, rtol=0, atol=1e-12)


def test_rows_subset_matches_full(lib_path=None):
    q, k, v = rnd((2, 4, 9, 8), 4), rnd((2, 2, 9, 8), 5), rnd((2, 2, 9, 5), 6)
    O, lse = run(q, k, v, True, 0.3, lib_path=lib_path)
    rows = np.array([[1, 3, 8], [0, 0, 0], [1, 2, 4]])
    Or, lser = oracle.attention_fp64(q, k, v, True, 0.3, rows=rows, lib_path=lib_path)[:2]
    for r, (b, h, i) in enumerate(rows):
        np.testing.assert_array_equal(Or[r], O[b, h, i])
        assert lser[r] == lse[b, h, i]


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal, lib_path=None):
    # With V = I (N_kv = d_v), O is the probability matrix itself.
    n = 12
    q, k = rnd((1, 2, n, 6), 7), rnd((1, 2, n, 6), 8)
    v = torch.eye(n, dtype=torch.float64).expand(1, 2, n, n).contiguous()
    P, _ = run(q, k, v, causal, 0.7, lib_path=lib_path)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-13)
    assert (P >= 0).all()
    if causal:
        assert np.all(P[..., np.triu_indices(n, 1)[0], np.triu_indices(n, 1)[1]] == 0.0)
        assert np.all(np.diagonal(P, axis1=-2, axis2=-1) > 0)


def test_single_key(lib_path=None):
    q, k, v = rnd((2, 3, 4, 5), 9), rnd((2, 3, 1, 5), 10), rnd((2, 3, 1, 7), 11)
    O, lse = run(q, k, v, False, 0.25, lib_path=lib_path)
    np.testing.assert_allclose(O, np.broadcast_to(v.numpy(), O.shape), rtol=0, atol=1e-15)
    expect = 0.25 * np.einsum("bhid,bhjd->bhi", q.numpy(), k.numpy())
    np.testing.assert_allclose(lse, expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v(causal, lib_path=None):
    q, k = rnd((1, 2, 10, 4), 12, 3.0), rnd((1, 2, 10, 4), 13, 3.0)
    const = np.array([1.5, -2.25, 0.0, 7.0])
    v = torch.from_numpy(np.broadcast_to(const, (1, 2, 10, 4)).copy())
    O, _ = run(q, k, v, causal, 1.0, lib_path=lib_path)
    np.testing.assert_allclose(O, np.broadcast_to(const, O.shape), rtol=0, atol=1e-13)


def test_causal_first_row_attends_to_itself(lib_path=None):
    q, k, v = rnd((2, 2, 8, 6), 14), rnd((2, 2, 8, 6), 15), rnd((2, 2, 8, 3), 16)
    O, lse = run(q, k, v, True, 0.4, lib_path=lib_path)
    np.testing.assert_allclose(O[:, :, 0], v[:, :, 0].numpy(), rtol=0, atol=1e-15)
    expect = f32(0.4) * (q[:, :, 0] * k[:, :, 0]).sum(-1).numpy()
    np.testing.assert_allclose(lse[:, :, 0], expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_q_averages_visible_values(causal, lib_path=None):
    n = 9
    q = torch.zeros((1, 1, n, 4), dtype=torch.float64)
    k, v = rnd((1, 1, n, 4), 17), rnd((1, 1, n, 3), 18)
    O, lse = run(q, k, v, causal, 0.5, lib_path=lib_path)
    vn = v[0, 0].numpy()
    for i in range(n):
        cnt = i + 1 if causal else n
        np.testing.assert_allclose(O[0, 0, i], vn[:cnt].mean(0), rtol=0, atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(cnt)) < 1e-14


def test_gqa_equals_repeated_heads(lib_path=None):
    q, k, v = rnd((2, 6, 7, 4), 19), rnd((2, 2, 7, 4), 20), rnd((2, 2, 7, 5), 21)
    O, lse = run(q, k, v, True, 0.6, lib_path=lib_path)
    O2, lse2 = run(q, k.repeat_interleave(3, 1), v.repeat_interleave(3, 1), True, 0.6,
                   lib_path=lib_path)
    np.testing.assert_allclose(O, O2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-15)


def test_key_permutation_invariance(lib_path=None):
    q, k, v = rnd((1, 2, 5, 6), 22), rnd((1, 2, 13, 6), 23), rnd((1, 2, 13, 4), 24)
    perm = torch.randperm(13, generator=torch.Generator().manual_seed(0))
    O, lse = run(q, k, v, False, 0.45, lib_path=lib_path)
    O2, lse2 = run(q, k[:, :, perm], v[:, :, perm], False, 0.45, lib_path=lib_path)
    np.testing.assert_allclose(O, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-13)


def test_causal_ignores_later_keys(lib_path=None):
    n = 10
    q, k, v = rnd((1, 1, n, 4), 25), rnd((1, 1, n, 4), 26), rnd((1, 1, n, 3), 27)
    O, lse = run(q, k, v, True, 0.5, lib_path=lib_path)
    for i in (0, 4, 8):
        k2, v2 = k.clone(), v.clone()
        k2[:, :, i + 1:] = rnd((1, 1, n - i - 1, 4), 100 + i, 5.0)
        v2[:, :, i + 1:] = rnd((1, 1, n - i - 1, 3), 200 + i, 5.0)
        O2, lse2 = run(q, k2, v2, True, 0.5, lib_path=lib_path)
        np.testing.assert_array_equal(O2[0, 0, : i + 1], O[0, 0, : i + 1])
        np.testing.assert_array_equal(lse2[0, 0, : i + 1], lse[0, 0, : i + 1])
        assert not np.array_equal(O2[0, 0, i + 1:], O[0, 0, i + 1:])


def test_split_merge_through_lse(lib_path=None):
    # Attention over keys A ∪ B equals the lse-weighted merge of the two halves.
    q, k, v = rnd((1, 2, 6, 5), 28), rnd((1, 2, 17, 5), 29), rnd((1, 2, 17, 4), 30)
    O, lse = run(q, k, v, False, 0.8, lib_path=lib_path)
    Oa, la = run(q, k[:, :, :7], v[:, :, :7], False, 0.8, lib_path=lib_path)
    Ob, lb = run(q, k[:, :, 7:], v[:, :, 7:], False, 0.8, lib_path=lib_path)
    lm = np.logaddexp(la, lb)
    Om = np.exp(la - lm)[..., None] * Oa + np.exp(lb - lm)[..., None] * Ob
    np.testing.assert_allclose(lm, lse, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Om, O, rtol=0, atol=1e-13)


def test_key_shift_moves_lse_only(lib_path=None):
    # Adding the same vector c to every key adds scale·(q·c) to each score of a
    # row: the softmax is unchanged and lse moves by exactly that amount.
    q, v = rnd((1, 1, 4, 3), 31), rnd((1, 1, 8, 2), 33)
    k = torch.round(rnd((1, 1, 8, 3), 32) * 1024) / 1024  # k + c stays exact in fp32
    c = torch.tensor([0.5, -1.0, 2.0], dtype=torch.float64)
    O, lse = run(q, k, v, False, 0.9, lib_path=lib_path)
    O2, lse2 = run(q, k + c, v, False, 0.9, lib_path=lib_path)
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-13)
    np.testing.assert_allclose((lse2 - lse)[0, 0], f32(0.9) * (q[0, 0] @ c).numpy(), rtol=0, atol=1e-12)


def test_large_scores_stay_finite(lib_path=None):
    # Scores of several hundred would overflow exp() without the max shift.
    q, k, v = rnd((1, 1, 4, 8), 34, 10.0), rnd((1, 1, 16, 8), 35, 10.0), rnd((1, 1, 16, 2), 36)
    O, lse = run(q, k, v, False, 1.0, lib_path=lib_path)
    assert np.isfinite(O).all() and np.isfinite(lse).all()
    Oref, lseref = sdpa_reference(q, k, v, False, 1.0)
    np.testing.assert_allclose(O, Oref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lseref, rtol=1e-14, atol=0)


def test_rejects_bad_sizes():
    q, k, v = rnd((1, 3, 4, 2), 1), rnd((1, 2, 4, 2), 2), rnd((1, 2, 4, 2), 3)
    with pytest.raises(ValueError):
        oracle.attention_fp64(q, k, v, False, 1.0)  # 3 % 2 != 0
    q2, k2, v2 = rnd((1, 2, 4, 2), 1), rnd((1, 2, 5, 2), 2), rnd((1, 2, 5, 2), 3)
    with pytest.raises(ValueError):
        oracle.attention_fp64(q2, k2, v2, True, 1.0)  # causal needs N_q == N_kv
    with pytest.raises(ValueError):
        oracle.attention_fp64(q2, k2, v2, False, 1.0, rows=[[0, 2, 0]])


# --------------------------------------------------------------------------
# Mutants: each plausible slip in the oracle must fail at least one pin.
# --------------------------------------------------------------------------
MUTANTS = {
    "drop_scale": ("s[j] = J->scale * dot;", "s[j] = dot;"),
    "causal_off_by_one": ("i + 1 < J->Nkv ? i + 1 : J->Nkv", "i < J->Nkv ? i : J->Nkv"),
    "wrong_kv_head": ("const int64_t g = h / group;", "const int64_t g = h % J->Hkv;"),
    "lse_without_max": ("*out_lse = m + log(l);", "*out_lse = log(l);"),
    "no_normalisation": ("const double p = s[j] / l;", "const double p = s[j];"),
    "transposed_k": ("dot += (double)q[c] * (double)k[c];",
                     "dot += (double)q[c] * (double)kbase[c * J->Nkv + j % J->dqk];"),
    "shift_sign": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j] + m);"),
    "v_row_index": ("const float *v = vbase + j * J->dv;", "const float *v = vbase + (n_keys - 1 - j) * J->dv;"),
    "first_key_dropped": ("for (int64_t j = 0; j < n_keys; ++j) {\n        const float *k",
                          "for (int64_t j = 1; j < n_keys; ++j) {\n        const float *k"),
}

PINS = [
    lambda p: [test_golden_closed_forms(n, lib_path=p) for n in ("two_key_logistic.json",
                                                               "causal_uniform_3.json")],
    lambda p: [test_matches_library_sdpa(s, lib_path=p) for s in SHAPES],
    lambda p: [test_probability_rows_sum_to_one(c, lib_path=p) for c in (False, True)],
    lambda p: test_single_key(lib_path=p),
    lambda p: [test_constant_v(c, lib_path=p) for c in (False, True)],
    lambda p: test_causal_first_row_attends_to_itself(lib_path=p),
    lambda p: [test_zero_q_averages_visible_values(c, lib_path=p) for c in (False, True)],
    lambda p: test_gqa_equals_repeated_heads(lib_path=p),
    lambda p: test_key_permutation_invariance(lib_path=p),
    lambda p: test_causal_ignores_later_keys(lib_path=p),
    lambda p: test_split_merge_through_lse(lib_path=p),
    lambda p: test_key_shift_moves_lse_only(lib_path=p),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation anchor not found: " + old
    path_c = tmp_path / ("mut_%s.c" % name)
    path_c.write_text(src.replace(old, new))
    path_so = tmp_path / ("libmut_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o",
                    str(path_so), str(path_c), "-lm"], check=True)
    caught = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(str(path_so))
        except (AssertionError, ValueError):
            caught += 1
    assert caught > 0, "mutant %s survived every pin" % name


def test_unmutated_source_passes_every_pin():
    for pin in PINS:
        pin(None)
