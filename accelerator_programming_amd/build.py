"""Build the gfx950 HIP libraries in-tree with hipcc.

``python -m accelerator_programming_amd.build`` compiles
``libattn_fwd.so`` (the C-ABI attention library) and
``libattn_tile_selftest.so`` (tile-layer probes used by the GPU tests).
Every build compiles from source; nothing is cached.
"""
from __future__ import annotations

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
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    return "hipcc"


def build_one(name: str, extra=(), verbose: bool = False) -> str:
    out = os.path.join(PKG, name)
    tmp = out + ".tmp%d" % os.getpid()
    srcs = [os.path.join(CSRC, s) for s in TARGETS[name]]
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra) + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = "\n".join(x for x in (r.stdout + r.stderr).splitlines() if noise not in x)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (name, msgs))
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list[str]:
    return [build_one(n, verbose=verbose) for n in TARGETS]


if __name__ == "__main__":
    extra = sys.argv[1:]
    for n in TARGETS:
        print(build_one(n, extra=extra, verbose=True))
