"""Register, scratch and LDS budgets of every kernel in every build.

The build records the compiler's per-kernel resource report beside each
library (``<library>.resources.json``). A kernel whose registers leave too few
waves per SIMD for its own workgroup cannot be dispatched at all (the runtime
rejects it), and one that spills to scratch memory is silently slow; the
compiler warns about neither. These CPU tests hold every kernel to what its
launch needs:
  * waves per SIMD (occupancy) at least ceil(workgroup threads / 256), and
    2 for the kernels designed to run two workgroups per CU (split-KV);
  * no scratch memory and no VGPR spills;
  * LDS within the 160 KB of a CU (80 KB where two workgroups share one).
"""
import json
import math
import os

import pytest

PKG = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "accelerator_programming_amd")
LIBS = ["libattn_fwd.so", "libattn_fwd_perturb.so", "libattn_tile_selftest.so"]

# kernel name fragment -> (threads per workgroup, workgroups per CU it is
# designed for); the first fragment that matches a kernel's name applies
BUDGET = [
    ("attn_fwd_wide_vk_split_kernel", 512, 1),
    ("attn_fwd_wide_vk_kernel", 512, 1),
    ("attn_fwd_wide_kernel", 256, 1),
    ("attn_fwd_kernel", 512, 1),
    ("attn_split_kernel", 256, 2),
    ("attn_split_merge", 256, 1),
    ("gemm_bf16_nt_kernel", 512, 1),
    ("rope_bf16_kernel", 256, 1),
    ("_probe", 64, 1),
]
LDS_PER_CU = 160 * 1024


def report(lib):
    path = os.path.join(PKG, lib + ".resources.json")
    if not os.path.exists(path):
        pytest.fail("%s is missing: build with python -m accelerator_programming_amd.build" % path)
    with open(path) as f:
        return json.load(f)


@pytest.mark.parametrize("lib", LIBS)
def test_every_kernel_fits_its_launch(lib):
    kernels = report(lib)
    assert kernels, "no kernels in the resource report of %s" % lib
    for name, r in kernels.items():
        budget = next(((t, w) for frag, t, w in BUDGET if frag in name), None)
        assert budget is not None, "no budget for kernel %s" % name
        threads, per_cu = budget
        need = per_cu * math.ceil(threads / 256)
        assert r["Occupancy [waves/SIMD]"] >= need, (name, r)
        assert r["ScratchSize [bytes/lane]"] == 0, (name, r)
        assert r["VGPRs Spill"] == 0, (name, r)
        assert r["LDS Size [bytes/block]"] * per_cu <= LDS_PER_CU, (name, r)


def test_perturbation_build_has_the_same_kernels():
    assert sorted(report("libattn_fwd.so")) == sorted(report("libattn_fwd_perturb.so"))
