"""Build libgdn_tree.so in-tree with hipcc for gfx950.

    python -m gated_deltanet_tree_amd.build

Every HIP source is compiled with FP contraction off (the kernels spell out
each fused multiply-add, which keeps the chain, tree and persist kernels
bitwise consistent) and with packed-FP32 instruction selection disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgdn_tree.so")
ARCH = "gfx950"

SOURCES = ["gdn_api.cpp", "gdn_plan.hip", "gdn_recurrent.hip", "gdn_fast.hip", "gdn_accept.hip", "gdn_ddtree.hip", "gdn_snapshot.hip", "gdn_static.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list[str]:
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I" + INCLUDE, "-I" + CSRC,
    ]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + flags() + ["-shared", "-o", tmp] + ["-x", "hip"] + srcs
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libgdn_tree.so")
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise and verbose:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
