"""Build libmedusa.so in-tree with hipcc for gfx950.

Usage: ``python -m speculative_decoding_heads_amd.build`` (or call ``build()``).
Every build recompiles all sources.  Packed FP32 instructions are disabled for
the device code (``-packed-fp32-ops``); hipcc's host pass warns that it does
not know that feature, which is harmless.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmedusa.so")

SOURCES = ["api.cpp", "tree_plan.cpp", "gemm.hip", "topk.hip", "tree.hip", "attn.hip",
           "accept.hip", "compact.hip", "loop.hip", "hydra.hip"]

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", "-Wno-unused-command-line-argument",
         "-I", os.path.join(ROOT, "include")]


def build(verbose=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc] + FLAGS + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
