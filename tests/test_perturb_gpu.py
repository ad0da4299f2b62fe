"""Parity with the copy/wait/barrier timing pulled out of its usual shape.

A copy landing in LDS after the barrier that was meant to publish it, or a
read of a ring stage that a later copy already overwrites, gives wrong
numbers only under some timings; a run on one GPU with one compiler proves
nothing about the ordering ("Distilling a 4.5 hour CUDA talk", sections 6
and 7: asynchronous copies need explicit waits). The library is therefore
also built with timing perturbation compiled in (``libattn_fwd_perturb.so``,
``-DATTN_PERTURB``): every kernel takes its work items in a seeded permuted
order and pauses for a pseudo-random number of ``s_sleep`` before each
LDS-DMA (main kernel, GEMM) or each tile copy (wide-head and split-KV
kernels). Arithmetic is unchanged, so each perturbed run must reproduce the
normal build's O and logsumexp bit for bit; each case runs the perturbed
build three times (the pauses differ from run to run) and holds the normal
output to the fp64 oracle at the usual tolerances (max |dO| <= 2e-2,
max |dlse| <= 1e-2).
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from accelerator_programming_amd import attn
from accelerator_programming_amd.inputs import (C3, C4, C5, G1, Workload, make_gemm_inputs,
                                                make_inputs, sample_rows)
from oracle.rope import rope_fp64

pytestmark = pytest.mark.gpu

PERTURB_PATH = os.path.join(os.path.dirname(attn.LIB_PATH), "libattn_fwd_perturb.so")
REPEATS = 3


@pytest.fixture(scope="module")
def libs():
    if not os.path.exists(PERTURB_PATH):
        pytest.fail("%s is not built: run python -m accelerator_programming_amd.build" % PERTURB_PATH)
    return attn.lib(), attn.bind(PERTURB_PATH)


def run_with(L, how, q, k, v, causal, scale, **kw):
    """One attention call through library build L (no torch work in between)."""
    o = torch.empty(tuple(q.shape[:3]) + (v.shape[3],), dtype=q.dtype, device="cuda")
    lse = torch.empty(tuple(q.shape[:3]), device="cuda")
    params = attn.params_for(q, k, v, causal, scale, o)
    plan = ctypes.c_void_p()
    assert L.attn_fwd_create_ex(ctypes.byref(params), ctypes.byref(plan)) == attn.ATTN_OK
    s = torch.cuda.current_stream().cuda_stream
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr())
    try:
        if how == "plain":
            st = L.attn_fwd_run(plan, *ptrs, s)
        elif how == "dropout":
            st = L.attn_fwd_run_dropout(plan, *ptrs, kw["p_drop"], kw["seed"], s)
        elif how == "rope":
            ws = torch.empty(max(16, L.attn_fwd_rope_workspace_bytes(plan)), dtype=torch.uint8,
                             device="cuda")
            st = L.attn_fwd_run_rope(plan, *ptrs, kw["base"], ws.data_ptr(), ws.numel(), s)
        else:  # split
            n = kw.get("n_splits", 0)
            need = L.attn_fwd_split_workspace_bytes(plan, n)
            ws = torch.empty(max(16, need), dtype=torch.uint8, device="cuda")
            st = L.attn_fwd_run_split(plan, *ptrs, n, ws.data_ptr(), ws.numel(), s)
        assert st == attn.ATTN_OK, attn.attn_status_str(st)
        torch.cuda.synchronize()
    finally:
        L.attn_fwd_destroy(plan)
    return o, lse


def check_perturbed(libs, how, q, k, v, causal, scale, **kw):
    L0, L1 = libs
    o0, l0 = run_with(L0, how, q, k, v, causal, scale, **kw)
    for rep in range(REPEATS):
        o1, l1 = run_with(L1, how, q, k, v, causal, scale, **kw)
        assert torch.equal(o1, o0) and torch.equal(l1, l0), "perturbed run %d differs" % rep
    return o0, l0


def oracle_check(o, lse, Oref, Lref, rows=None):
    if rows is not None:
        r = torch.as_tensor(rows)
        o, lse = o[r[:, 0], r[:, 1], r[:, 2]], lse[r[:, 0], r[:, 1], r[:, 2]]
    og = o.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    assert np.abs(og - Oref).max() <= 2e-2, np.abs(og - Oref).max()
    assert np.abs(lg - Lref).max() <= 1e-2, np.abs(lg - Lref).max()


SHAPES = [
    # name, workload
    ("d128_causal_gqa", Workload("pt", 1, 8, 2, 1000, 1000, 128, 128, True, torch.bfloat16, 71)),
    ("d64_full_ragged", Workload("pt", 2, 4, 4, 300, 1000, 64, 64, False, torch.bfloat16, 72)),
    ("d64_fp32_causal", Workload("pt", 1, 2, 1, 190, 190, 64, 64, True, torch.float32, 73)),
    ("wide_v_in_k", C5.with_(Hq=8, Nkv=1000)),
    ("wide_own_v", Workload("pt", 1, 2, 1, 33, 257, 576, 512, False, torch.bfloat16, 74)),
]


@pytest.mark.parametrize("name,w", SHAPES, ids=[s[0] for s in SHAPES])
def test_perturbed_plain(libs, name, w):
    q, k, v = make_inputs(w, "cuda")
    o, lse = check_perturbed(libs, "plain", q, k, v, w.causal, w.softmax_scale)
    Oref, Lref, _ = oracle.attention_fp64(q, k, v, w.causal, w.softmax_scale)
    oracle_check(o, lse, Oref, Lref)


def test_perturbed_dropout(libs):
    w = Workload("ptd", 1, 4, 2, 500, 500, 128, 128, True, torch.bfloat16, 75)
    q, k, v = make_inputs(w, "cuda")
    o, lse = check_perturbed(libs, "dropout", q, k, v, True, w.softmax_scale, p_drop=0.25, seed=99)
    Oref, Lref, _ = oracle.attention_fp64(q, k, v, True, w.softmax_scale, drop_thr=64, seed=99)
    oracle_check(o, lse, Oref, Lref)


def test_perturbed_rope(libs):
    w = Workload("ptr", 1, 4, 2, 400, 400, 128, 128, True, torch.bfloat16, 76)
    q, k, v = make_inputs(w, "cuda")
    o, lse = check_perturbed(libs, "rope", q, k, v, True, w.softmax_scale, base=10000.0)
    Oref, Lref, _ = oracle.attention_fp64(rope_fp64(q, 1e4), rope_fp64(k, 1e4), v, True,
                                          w.softmax_scale)
    oracle_check(o, lse, Oref, Lref)


@pytest.mark.parametrize("shape", [(2, 32, 8, 1, 4096, 128, 0), (2, 8, 2, 4, 1000, 64, 3)],
                         ids=["d128_library_count", "d64_ragged_3"])
def test_perturbed_split(libs, shape):
    B, Hq, Hkv, Nq, Nkv, d, n = shape
    w = Workload("pts", B, Hq, Hkv, Nq, Nkv, d, d, False, torch.bfloat16, 77 + Nkv)
    q, k, v = make_inputs(w, "cuda")
    o, lse = check_perturbed(libs, "split", q, k, v, False, w.softmax_scale, n_splits=n)
    Oref, Lref, _ = oracle.attention_fp64(q, k, v, False, w.softmax_scale)
    oracle_check(o, lse, Oref, Lref)


@pytest.mark.parametrize("shape", [(1, 3, 1, 130, 700, 3), (1, 2, 1, 40, 300, 0)],
                         ids=["wide_ragged_3", "wide_library_count"])
def test_perturbed_wide_split(libs, shape):
    # the wide-head split kernel (V inside K): copies three tiles ahead in
    # each range, ragged rows and a ragged last range
    B, Hq, Hkv, Nq, Nkv, n = shape
    w = Workload("ptws", B, Hq, Hkv, Nq, Nkv, 576, 512, False, torch.bfloat16, 78 + Nkv, v_from_k=True)
    q, k, v = make_inputs(w, "cuda")
    o, lse = check_perturbed(libs, "split", q, k, v, False, w.softmax_scale, n_splits=n)
    Oref, Lref, _ = oracle.attention_fp64(q, k, v, False, w.softmax_scale)
    oracle_check(o, lse, Oref, Lref)


def test_perturbed_c5_split(libs):
    q, k, v = make_inputs(C5, "cuda")
    o, lse = check_perturbed(libs, "split", q, k, v, False, C5.softmax_scale)
    rows = sample_rows(C5, 64)
    Oref, Lref, _ = oracle.attention_fp64(q, k, v, False, C5.softmax_scale, rows=rows)
    oracle_check(o, lse, Oref, Lref, rows=rows)


@pytest.mark.parametrize("w", [C3, C4, C5], ids=["C3", "C4", "C5"])
def test_perturbed_full_size(libs, w):
    # every element bit for bit against the normal build, sampled rows
    # against the oracle
    q, k, v = make_inputs(w, "cuda")
    o, lse = check_perturbed(libs, "plain", q, k, v, w.causal, w.softmax_scale)
    rows = sample_rows(w, 64)
    Oref, Lref, _ = oracle.attention_fp64(q, k, v, w.causal, w.softmax_scale, rows=rows)
    oracle_check(o, lse, Oref, Lref, rows=rows)


def test_perturbed_gemm(libs):
    L0, L1 = libs
    w = G1
    a, b = make_gemm_inputs(w, "cuda")
    # ragged M and N (not multiples of the 256 tile); ldc = N must be a
    # multiple of 4
    a, b = a[:1000, :1032].contiguous(), b[:780, :1032].contiguous()
    M, K = a.shape
    N = b.shape[0]
    outs = []
    for L in (L0,) + (L1,) * REPEATS:
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        st = L.tile_gemm_bf16_nt(M, N, K, a.data_ptr(), K, b.data_ptr(), K, c.data_ptr(), N,
                                 torch.cuda.current_stream().cuda_stream)
        assert st == attn.ATTN_OK
        torch.cuda.synchronize()
        outs.append(c)
    for c in outs[1:]:
        assert torch.equal(c, outs[0])
