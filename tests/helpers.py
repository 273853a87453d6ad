"""Shared helpers of the GPU parity tests (not collected by pytest)."""

import os
import sys

import numpy as np
import pytest
import torch

# tolerances: per output row, max|gpu - ref| <= tol * max|ref|
TOL_BF16 = 2e-2
TOL_F32 = 1e-5


def require_gpu():
    from speculative_decoding_heads_amd import medusa as M
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.lib()          # raises if the library is missing: the HIP path must run


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype != torch.float64 else \
        t.detach().cpu().numpy()


def row_rel_err(gpu, ref):
    """max over rows of max|gpu - ref| / max|ref| (rows = last axis)."""
    g = np.asarray(gpu, dtype=np.float64).reshape(-1, np.shape(gpu)[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    num = np.abs(g - r).max(axis=1)
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((num / den).max())


def assert_rows_close(gpu, ref, tol, what=""):
    e = row_rel_err(gpu, ref)
    assert e <= tol, f"{what}: row-relative error {e:.3e} > {tol:.1e}"
    return e


def normal(shape, seed, std=1.0, dtype=torch.bfloat16):
    from speculative_decoding_heads_amd.synth import normal as syn
    return syn(shape, seed, std, "bf16" if dtype == torch.bfloat16 else "f32")
