"""attn_fwd_run_split_noalloc (the split-KV path through the library's static
scratch, for callers that cannot allocate device memory) against
attn_fwd_run_split with a caller workspace, through the C ABI: two calls in
a row, the second with a smaller problem. The two entry points launch the
same kernels with the same split count, so their outputs are bitwise equal;
both are also held to the fp64 oracle at the parity tolerances
(max |dO| <= 2e-2, max |dlse| <= 1e-2)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from accelerator_programming_amd import attn
from accelerator_programming_amd.inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu


def out_like(q, v):
    return torch.empty(q.shape[:3] + v.shape[3:], dtype=q.dtype, device=q.device)


def via_workspace(q, k, v, scale, n_splits):
    o = out_like(q, v)
    lse = torch.empty(q.shape[:3], device=q.device)
    op = attn.AttnFwd(q, k, v, False, scale, o)
    try:
        op.run_split(q, k, v, o, lse, n_splits=n_splits)
    finally:
        op.close()
    return o, lse


def via_static_scratch(q, k, v, scale, n_splits):
    # straight through the C entry point; the plan is the only host object
    o = out_like(q, v)
    lse = torch.empty(q.shape[:3], device=q.device)
    params = attn.params_for(q, k, v, False, scale, o)
    plan = attn.attn_fwd_create_ex(params)
    try:
        st = attn.lib().attn_fwd_run_split_noalloc(
            plan, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            ctypes.c_int32(n_splits), torch.cuda.current_stream().cuda_stream)
        assert st == attn.ATTN_OK, attn.attn_status_str(st)
    finally:
        attn.attn_fwd_destroy(plan)
    return o, lse


def check_twice(shapes):
    for w, ns in shapes:
        q, k, v = make_inputs(w, "cuda")
        print("noalloc case", w.name, "n_splits", ns, flush=True)
        o1, l1 = via_static_scratch(q, k, v, w.softmax_scale, ns)
        o2, l2 = via_workspace(q, k, v, w.softmax_scale, ns)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        Oref, Lref, _ = oracle.attention_fp64(q, k, v, False, w.softmax_scale)
        assert np.abs(o1.float().cpu().numpy() - Oref).max() <= 2e-2
        assert np.abs(l1.cpu().numpy() - Lref).max() <= 1e-2


def test_noalloc_matches_workspace_entry_point_twice():
    check_twice([
        # the larger problem first (its partials fill more of the buffer),
        # then a smaller one that reuses the same buffer
        (Workload("na1", 4, 32, 8, 1, 8192, 128, 128, False, torch.bfloat16, 4101), 0),
        (Workload("na2", 1, 8, 2, 3, 1000, 64, 64, False, torch.bfloat16, 4102), 5),
    ])


def test_noalloc_wide_heads_twice():
    # wide heads with V inside K (d_qk 576, d_v 512): 16 ranges of 256 rows
    # take 8.4 MB of the 16 MiB buffer, then a smaller problem reuses it
    check_twice([
        (Workload("naw1", 1, 16, 1, 16, 2048, 576, 512, False, torch.bfloat16, 4103, v_from_k=True), 0),
        (Workload("naw2", 1, 2, 1, 5, 300, 576, 512, False, torch.bfloat16, 4104, v_from_k=True), 3),
    ])
