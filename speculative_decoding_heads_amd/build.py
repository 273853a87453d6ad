"""Build libmedusa.so in-tree with hipcc for gfx950.

Usage: ``python -m speculative_decoding_heads_amd.build`` (or call ``build()``).
Every build recompiles all sources (one hipcc process per source file, run in
parallel, then one link).  Packed FP32 instructions are disabled for the
device code (``-packed-fp32-ops``); hipcc's host pass warns that it does not
know that feature, which is harmless.
"""

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmedusa.so")

SOURCES = ["api.cpp", "tree_plan.cpp", "gemm.hip", "topk.hip", "tree.hip", "attn.hip",
           "accept.hip", "compact.hip", "loop.hip", "hydra.hip", "mtp.hip", "probe.hip"]

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", "-Wno-unused-command-line-argument",
         "-I", os.path.join(ROOT, "include")]

_NOISE = "is not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if _NOISE not in ln]
    return res.returncode, msgs


def build(verbose=False, jobs=None):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    jobs = jobs or min(len(SOURCES), max(1, min(os.cpu_count() or 1, 16)))
    tmpdir = tempfile.mkdtemp(prefix="medusa_build_")
    try:
        objs, cmds = [], []
        for s in SOURCES:
            src = os.path.join(CSRC, s)
            obj = os.path.join(tmpdir, os.path.splitext(s)[0] + ".o")
            lang = ["-x", "hip"] if s.endswith(".hip") else []
            cmds.append([hipcc] + FLAGS + lang + ["-c", src, "-o", obj])
            objs.append(obj)
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for cmd, (rc, msgs) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
            if verbose and msgs:
                print("\n".join(msgs))
        tmp = LIB + ".tmp"
        rc, msgs = _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
        if rc != 0:
            raise RuntimeError("link failed:\n" + "\n".join(msgs))
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
