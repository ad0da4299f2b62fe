"""The C-ABI boundary on the host: the library loads, exports every function
include/attn_fwd.h declares, and validates its arguments before any HIP call
(so these tests run without a GPU)."""
import ctypes
import math
import os
import re

import pytest

from accelerator_programming_amd import attn
from accelerator_programming_amd.attn import (ATTN_BF16, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED,
                                              ATTN_FP32, ATTN_OK, AttnError, AttnFwdParams)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_fwd.h")
SELFTEST = os.path.join(ROOT, "accelerator_programming_amd", "libattn_tile_selftest.so")


def declared_functions(path):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions(HEADER)
    for n in ("attn_fwd_create", "attn_fwd_run", "attn_fwd_destroy"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = attn.lib()
    for name in declared_functions(HEADER):
        assert hasattr(L, name), name


def test_selftest_library_loads():
    L = ctypes.CDLL(SELFTEST)
    for n in ("tile_selftest_mfma", "tile_selftest_mfma16", "tile_selftest_xhalf", "tile_selftest_qk",
              "tile_selftest_pv",
              "tile_selftest_tr16"):
        assert hasattr(L, n)


def test_params_struct_matches_header_layout():
    # 7 int64 + int32 + float + int32 (+4 padding) + 4 x 3 int64
    assert ctypes.sizeof(AttnFwdParams) == 7 * 8 + 4 + 4 + 4 + 4 + 12 * 8


def create(**kw):
    """Call the C entry point directly (the Python helper normalises causal)."""
    base = dict(B=1, H_q=2, H_kv=1, N=256, d=128, causal=1, scale=1 / math.sqrt(128))
    base.update(kw)
    plan = ctypes.c_void_p()
    st = attn.lib().attn_fwd_create(ctypes.byref(plan), base["B"], base["H_q"], base["H_kv"],
                                    base["N"], base["d"], base["causal"], base["scale"])
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_create")
    return plan.value


def status_of(fn):
    try:
        plan = fn()
    except AttnError as e:
        return e.status
    attn.attn_fwd_destroy(plan)
    return ATTN_OK


@pytest.mark.parametrize("kw,expected", [
    ({}, ATTN_OK),
    (dict(d=64), ATTN_OK),
    (dict(B=0), ATTN_ERR_INVALID),
    (dict(H_q=0), ATTN_ERR_INVALID),
    (dict(N=0), ATTN_ERR_INVALID),
    (dict(N=-5), ATTN_ERR_INVALID),
    (dict(H_q=3, H_kv=2), ATTN_ERR_INVALID),
    (dict(scale=float("nan")), ATTN_ERR_INVALID),
    (dict(scale=float("inf")), ATTN_ERR_INVALID),
    (dict(scale=0.0), ATTN_ERR_INVALID),
    (dict(scale=-0.1), ATTN_ERR_INVALID),
    (dict(causal=2), ATTN_ERR_INVALID),
    (dict(d=96), ATTN_ERR_UNSUPPORTED),
    (dict(d=256), ATTN_ERR_UNSUPPORTED),
])
def test_create_validation(kw, expected):
    assert status_of(lambda: create(**kw)) == expected


def ex_params(**kw):
    p = AttnFwdParams()
    p.B, p.H_q, p.H_kv, p.N, p.d = 2, 4, 2, 300, 64
    p.N_kv, p.d_v = 0, 0
    p.causal, p.scale, p.dtype = 0, 0.125, ATTN_BF16
    for k, v in kw.items():
        if k.endswith("_strides"):
            setattr(p, k, (ctypes.c_int64 * 3)(*v))
        else:
            setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,expected", [
    ({}, ATTN_OK),
    (dict(N_kv=517), ATTN_OK),
    (dict(dtype=ATTN_FP32), ATTN_OK),
    (dict(dtype=ATTN_FP32, d=128), ATTN_ERR_UNSUPPORTED),
    (dict(dtype=7), ATTN_ERR_INVALID),
    (dict(causal=1, N_kv=301), ATTN_ERR_INVALID),
    (dict(d_v=32), ATTN_ERR_UNSUPPORTED),
    # the wide-head variant: d_qk 576 with d_v 512, bf16 only
    (dict(d=576, d_v=512), ATTN_OK),
    (dict(d=576, d_v=512, causal=1), ATTN_OK),
    (dict(d=576, d_v=576), ATTN_ERR_UNSUPPORTED),
    (dict(d=576, d_v=512, dtype=ATTN_FP32), ATTN_ERR_UNSUPPORTED),
    # V as the first 512 columns of the 576-wide K rows
    (dict(d=576, d_v=512, v_strides=(2 * 300 * 576, 300 * 576, 576)), ATTN_OK),
    # V as the first 64 columns of a 128-wide row: legal strides
    (dict(v_strides=(2 * 300 * 128, 300 * 128, 128)), ATTN_OK),
    # row stride smaller than the row
    (dict(q_strides=(4 * 300 * 64, 300 * 64, 56)), ATTN_ERR_INVALID),
    # a stride that breaks 16-byte alignment of bf16 rows
    (dict(k_strides=(2 * 300 * 68, 300 * 68, 68)), ATTN_ERR_INVALID),
    (dict(o_strides=(-1, 300 * 64, 64)), ATTN_ERR_INVALID),
])
def test_create_ex_validation(kw, expected):
    p = ex_params(**kw)
    assert status_of(lambda: attn.attn_fwd_create_ex(p)) == expected


def test_create_null_plan_pointer():
    L = attn.lib()
    assert L.attn_fwd_create(None, 1, 1, 1, 128, 64, 0, 0.125) == ATTN_ERR_INVALID
    assert L.attn_fwd_create_ex(None, None) == ATTN_ERR_INVALID


def test_destroy_null_is_safe():
    attn.attn_fwd_destroy(None)


def test_plan_info_geometry():
    plan = attn.attn_fwd_create(2, 32, 8, 4096, 128, 1, 1 / math.sqrt(128))
    try:
        info = attn.attn_fwd_plan_info(plan)
    finally:
        attn.attn_fwd_destroy(plan)
    assert info["grid"] == 2 * 32 * (4096 // info["tile_q"])
    assert info["block"] % 64 == 0
    assert info["lds_bytes"] <= 160 * 1024


def test_plan_info_geometry_wide_heads():
    p = ex_params(B=1, H_q=128, H_kv=1, N=64, N_kv=8192, d=576, d_v=512, scale=1 / math.sqrt(576))
    plan = attn.attn_fwd_create_ex(p)
    try:
        info = attn.attn_fwd_plan_info(plan)
    finally:
        attn.attn_fwd_destroy(plan)
    assert info["grid"] == 128 * (64 // info["tile_q"])
    assert info["block"] % 64 == 0
    assert info["lds_bytes"] <= 160 * 1024


def test_run_rejects_null_and_misaligned_pointers_before_launch():
    plan = create()
    try:
        L = attn.lib()
        assert L.attn_fwd_run(None, 16, 16, 16, 16, None, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run(plan, None, 16, 16, 16, None, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run(plan, 16, 16, 16, None, None, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run(plan, 16 + 2, 16, 16, 16, None, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run(plan, 16, 16, 16 + 8, 16, None, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run(plan, 16, 16, 16, 16, 18, None) == ATTN_ERR_INVALID
    finally:
        attn.attn_fwd_destroy(plan)


def test_status_strings():
    assert attn.attn_status_str(ATTN_OK) == "ATTN_OK"
    assert attn.attn_status_str(ATTN_ERR_UNSUPPORTED) == "ATTN_ERR_UNSUPPORTED"
    assert attn.attn_status_str(99) == "ATTN_ERR_UNKNOWN"


# ---------------------------------------------------------------------------
# Split-KV entry points: choice, workspace size and argument checks (no launch)
# ---------------------------------------------------------------------------
def split_plan(**kw):
    args = dict(B=1, H_q=32, H_kv=8, N=4, N_kv=4096, d=128, causal=0, scale=1 / math.sqrt(128))
    args.update(kw)
    return attn.attn_fwd_create_ex(ex_params(**args))


def test_split_count_and_workspace_size():
    plan = split_plan()
    try:
        n = attn.attn_fwd_split_count(plan)
        assert 1 <= n <= 64
        rows = 1 * 32 * 4
        assert attn.attn_fwd_split_workspace_bytes(plan, 0) == n * rows * (128 + 1) * 4
        assert attn.attn_fwd_split_workspace_bytes(plan, 3) == 3 * rows * (128 + 1) * 4
        assert attn.attn_fwd_split_workspace_bytes(plan, 65) == -1
    finally:
        attn.attn_fwd_destroy(plan)
    # at most one split per 64-key tile
    plan = split_plan(N_kv=100)
    try:
        assert attn.attn_fwd_split_count(plan) == 2
    finally:
        attn.attn_fwd_destroy(plan)


@pytest.mark.parametrize("kw", [
    dict(causal=1, N=4096),                      # causal
    dict(N=32),                                  # 4 x 32 = 128 query rows per kv head
    dict(d=576, d_v=512, H_q=128, H_kv=1, N=64, N_kv=64, causal=1),  # wide heads, causal
    dict(B=1 << 16, H_q=32, H_kv=8, N=1),         # 2^19 (batch, kv head) pairs
    dict(d=64, d_v=64, dtype=1),                  # fp32
    dict(d=576, d_v=512, B=1024, H_q=128, H_kv=1, N=64, N_kv=64),  # 2^17 wide row tiles
], ids=["causal", "too_many_rows", "wide_causal", "too_many_groups", "fp32", "wide_too_many_tiles"])
def test_split_path_declines_unserved_plans(kw):
    plan = split_plan(**kw)
    try:
        assert attn.attn_fwd_split_count(plan) == 0
        assert attn.attn_fwd_split_workspace_bytes(plan, 0) == -1
        L = attn.lib()
        assert L.attn_fwd_run_split(plan, 16, 16, 16, 16, None, 0, 16, 1 << 30, None) == \
            ATTN_ERR_UNSUPPORTED
    finally:
        attn.attn_fwd_destroy(plan)


def wide_split_plan(**kw):
    args = dict(B=1, H_q=128, H_kv=1, N=64, N_kv=8192, d=576, d_v=512, causal=0,
                scale=1 / math.sqrt(192))
    args.update(kw)
    return attn.attn_fwd_create_ex(ex_params(**args))


def test_wide_split_count_and_workspace_size():
    # 64-row tiles of each (batch, head): 128 of them at 64 rows per head, so
    # two ranges give one workgroup per CU; at least one 32-key tile per range
    plan = wide_split_plan()
    try:
        rows = 128 * 64
        assert attn.attn_fwd_split_count(plan) == 2
        assert attn.attn_fwd_split_workspace_bytes(plan, 0) == 2 * rows * (512 + 1) * 4
        assert attn.attn_fwd_split_workspace_bytes(plan, 7) == 7 * rows * (512 + 1) * 4
        assert attn.attn_fwd_split_workspace_bytes(plan, 65) == -1
    finally:
        attn.attn_fwd_destroy(plan)
    for kw, n in [(dict(H_q=1, N=1, N_kv=40), 2),       # two 32-key tiles
                  (dict(H_q=4, N=65, N_kv=8192), 32),  # 8 row tiles
                  (dict(H_q=1, N=1, N_kv=1 << 20), 64)]:  # the cap
        plan = wide_split_plan(**kw)
        try:
            assert attn.attn_fwd_split_count(plan) == n, kw
        finally:
            attn.attn_fwd_destroy(plan)


def test_wide_split_refuses_a_separate_v_before_launch():
    # the wide split kernel reads V from the copied K tiles: V must be the
    # first 512 columns of K (same pointer and strides); anything else is
    # refused before any HIP call (a problem small enough for the static
    # scratch, so noalloc reaches that check)
    plan = wide_split_plan(H_q=2, N=8, N_kv=256)
    try:
        L = attn.lib()
        need = attn.attn_fwd_split_workspace_bytes(plan, 0)
        assert L.attn_fwd_run_split(plan, 16, 16, 32, 16, None, 0, 16, need, None) == \
            ATTN_ERR_UNSUPPORTED
        assert L.attn_fwd_run_split_noalloc(plan, 16, 16, 32, 16, None, 0, None) == \
            ATTN_ERR_UNSUPPORTED
    finally:
        attn.attn_fwd_destroy(plan)


def test_wide_split_at_full_size_exceeds_the_static_scratch():
    # 2 ranges x 8192 rows x 513 floats = 33.6 MB > 16 MiB
    from accelerator_programming_amd.attn import ATTN_ERR_TOO_LARGE
    plan = wide_split_plan()
    try:
        assert attn.lib().attn_fwd_run_split_noalloc(plan, 16, 16, 16, 16, None, 0, None) == \
            ATTN_ERR_TOO_LARGE
    finally:
        attn.attn_fwd_destroy(plan)


def test_run_split_rejects_bad_arguments_before_launch():
    plan = split_plan()
    try:
        L = attn.lib()
        need = attn.attn_fwd_split_workspace_bytes(plan, 0)
        assert L.attn_fwd_run_split(None, 16, 16, 16, 16, None, 0, 16, need, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run_split(plan, 16, 16, 16, 16, None, 0, None, need, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run_split(plan, 16, 16, 16, 16, None, 0, 24, need, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run_split(plan, 16, 16, 16, 16, None, 0, 16, need - 4, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run_split(plan, 16, 16, 16, 16, None, 65, 16, 1 << 40, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run_split(plan, 16 + 2, 16, 16, 16, None, 0, 16, need, None) == ATTN_ERR_INVALID
    finally:
        attn.attn_fwd_destroy(plan)


def test_dropout_probability_checked_before_any_hip_call():
    L = attn.lib()
    plan = attn.attn_fwd_create(1, 2, 2, 64, 128, True, 0.125)
    P = ctypes.c_void_p(0x1000)
    try:
        for p in (1.0, 1.5, -0.1, float("nan")):
            assert L.attn_fwd_run_dropout(plan, P, P, P, P, None, p, 1, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run_dropout(None, P, P, P, P, None, 0.1, 1, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run_dropout(plan, ctypes.c_void_p(0x1008), P, P, P, None, 0.1, 1,
                                      None) == ATTN_ERR_INVALID
    finally:
        attn.attn_fwd_destroy(plan)


def test_dropout_unsupported_for_wide_heads():
    L = attn.lib()
    p = AttnFwdParams()
    p.B, p.H_q, p.H_kv, p.N, p.d, p.N_kv, p.d_v = 1, 2, 1, 16, 576, 64, 512
    p.causal, p.scale, p.dtype = 0, 0.05, ATTN_BF16
    plan = attn.attn_fwd_create_ex(p)
    P = ctypes.c_void_p(0x1000)
    try:
        assert L.attn_fwd_run_dropout(plan, P, P, P, P, None, 0.1, 1, None) == ATTN_ERR_UNSUPPORTED
    finally:
        attn.attn_fwd_destroy(plan)


def test_rope_arguments_checked_before_any_hip_call():
    L = attn.lib()
    P = ctypes.c_void_p(0x1000)
    assert L.attn_rope_bf16(P, P, 1, 1, 4, 12, None, None, 10000.0, None) == ATTN_ERR_INVALID  # d % 8
    assert L.attn_rope_bf16(P, P, 1, 1, 4, 16, None, None, 1.0, None) == ATTN_ERR_INVALID  # base
    assert L.attn_rope_bf16(P, P, 1, 1, 4, 16, None, None, float("inf"), None) == ATTN_ERR_INVALID
    assert L.attn_rope_bf16(ctypes.c_void_p(0x1004), P, 1, 1, 4, 16, None, None, 1e4,
                            None) == ATTN_ERR_INVALID
    assert L.attn_rope_bf16(P, P, 0, 1, 4, 16, None, None, 1e4, None) == ATTN_OK  # empty
    plan = attn.attn_fwd_create(1, 2, 2, 64, 128, True, 0.125)
    try:
        need = L.attn_fwd_rope_workspace_bytes(plan)
        assert need == 1 * 2 * 64 * 128 * 2
        assert L.attn_fwd_run_rope(plan, P, P, P, P, None, 1e4, P, need - 16,
                                   None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run_rope(plan, P, P, P, P, None, 0.5, P, need, None) == ATTN_ERR_INVALID
    finally:
        attn.attn_fwd_destroy(plan)
    p = AttnFwdParams()
    p.B, p.H_q, p.H_kv, p.N, p.d = 1, 1, 1, 32, 64
    p.causal, p.scale, p.dtype = 0, 0.125, ATTN_FP32
    plan = attn.attn_fwd_create_ex(p)
    try:
        assert L.attn_fwd_rope_workspace_bytes(plan) == -1
        assert L.attn_fwd_run_rope(plan, P, P, P, P, None, 1e4, P, 1 << 20,
                                   None) == ATTN_ERR_UNSUPPORTED
    finally:
        attn.attn_fwd_destroy(plan)


def test_binding_rejects_host_tensors_before_the_c_abi():
    # every run* method of the binding checks its tensors before it passes a
    # pointer on: host memory never reaches a kernel
    import torch
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    o = torch.zeros_like(q)
    op = attn.AttnFwd(q, k, k, False, 0.125, o)
    try:
        for call in (lambda: op.run(q, k, k, o),
                     lambda: op.run_dropout(q, k, k, o, p_drop=0.5, seed=1),
                     lambda: op.run_rope(q, k, k, o, k_rot=k),
                     lambda: op.run_split(q, k, k, o, workspace=k)):
            with pytest.raises(ValueError, match="device tensor"):
                call()
    finally:
        op.close()
    with pytest.raises(ValueError, match="device tensor"):
        attn.attn_rope_bf16(q)


def test_split_noalloc_rejects_bad_arguments_before_any_hip_call():
    # these return before the library looks up its static scratch (no GPU here)
    from accelerator_programming_amd.attn import ATTN_ERR_TOO_LARGE, ATTN_SPLIT_SCRATCH_BYTES
    L = attn.lib()
    plan = split_plan()
    try:
        assert L.attn_fwd_run_split_noalloc(None, 16, 16, 16, 16, None, 0, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run_split_noalloc(plan, 16, None, 16, 16, None, 0, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run_split_noalloc(plan, 16 + 2, 16, 16, 16, None, 0, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run_split_noalloc(plan, 16, 16, 16, 16, 18, 0, None) == ATTN_ERR_INVALID
        assert L.attn_fwd_run_split_noalloc(plan, 16, 16, 16, 16, None, 65, None) == ATTN_ERR_INVALID
    finally:
        attn.attn_fwd_destroy(plan)
    # a plan the split path does not serve (causal)
    plan = split_plan(causal=1, N=4096)
    try:
        assert L.attn_fwd_run_split_noalloc(plan, 16, 16, 16, 16, None, 0, None) == \
            ATTN_ERR_UNSUPPORTED
    finally:
        attn.attn_fwd_destroy(plan)
    # more partial results than the static buffer holds
    plan = split_plan(B=64, N=1)
    try:
        need = attn.attn_fwd_split_workspace_bytes(plan, 64)
        assert need > ATTN_SPLIT_SCRATCH_BYTES
        assert L.attn_fwd_run_split_noalloc(plan, 16, 16, 16, 16, None, 64, None) == \
            ATTN_ERR_TOO_LARGE
        assert attn.attn_status_str(ATTN_ERR_TOO_LARGE) == "ATTN_ERR_TOO_LARGE"
    finally:
        attn.attn_fwd_destroy(plan)
