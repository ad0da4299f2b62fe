"""Build the gfx950 HIP libraries in-tree with hipcc.

``python -m accelerator_programming_amd.build`` compiles
``libattn_fwd.so`` (the C-ABI attention library),
``libattn_tile_selftest.so`` (tile-layer probes used by the GPU tests) and
``libattn_fwd_perturb.so`` (the attention library with timing perturbation
compiled in, for the perturbation parity tests only).
Every build compiles from source; nothing is cached.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
ARCH = "gfx950"

# Packed fp32 VALU forms are switched off for every device pass.
HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]

TARGETS = {
    "libattn_fwd.so": ["attn_fwd.hip", "tile_gemm.hip"],
    "libattn_tile_selftest.so": ["tile_selftest.hip"],
    # the same library with timing perturbation compiled in (test use only:
    # permuted workgroup order, pauses before every LDS-DMA)
    "libattn_fwd_perturb.so": ["attn_fwd.hip", "tile_gemm.hip"],
}
TARGET_FLAGS = {
    "libattn_fwd_perturb.so": ["-DATTN_PERTURB=0x5EED1234u"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    return "hipcc"


RESOURCE_REMARK = "-Rpass-analysis=kernel-resource-usage"


def parse_resource_remarks(text: str) -> dict:
    """{kernel: {field: value}} from the compiler's kernel-resource-usage
    remarks (registers, scratch, spills, occupancy, LDS per kernel)."""
    out, cur = {}, None
    for line in text.splitlines():
        if "remark:" not in line or RESOURCE_REMARK not in line:
            continue
        body = line.split("remark:", 1)[1].rsplit("[", 1)[0].strip()
        key, _, val = body.partition(":")
        key, val = key.strip(), val.strip()
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            try:
                cur[key] = int(val)
            except ValueError:
                cur[key] = val
    return out


def build_one(name: str, extra=(), verbose: bool = False) -> str:
    out = os.path.join(PKG, name)
    tmp = out + ".tmp%d" % os.getpid()
    srcs = [os.path.join(CSRC, s) for s in TARGETS[name]]
    cmd = ([hipcc()] + HIPCC_FLAGS + TARGET_FLAGS.get(name, []) + list(extra) + [RESOURCE_REMARK]
           + ["-o", tmp] + srcs)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature; the
    # resource remarks are kept in a file beside the library
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = "\n".join(x for x in (r.stdout + r.stderr).splitlines()
                     if noise not in x and "remark:" not in x)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (name, msgs))
    if verbose and msgs.strip():
        print(msgs)
    with open(out + ".resources.json.tmp", "w") as f:
        json.dump(parse_resource_remarks(r.stderr), f, indent=1, sort_keys=True)
    os.replace(tmp, out)
    os.replace(out + ".resources.json.tmp", out + ".resources.json")
    return out


def build_all(verbose: bool = False) -> list[str]:
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=len(TARGETS)) as ex:
        return list(ex.map(lambda n: build_one(n, verbose=verbose), TARGETS))


if __name__ == "__main__":
    extra = sys.argv[1:]
    for n in TARGETS:
        print(build_one(n, extra=extra, verbose=True))
