"""Seeded synthetic inputs for the verify step.

This module only draws random numbers; it holds none of the step's
arithmetic.  It is the one piece shared by the tests, the bench and the CPU
oracle's callers: inputs are drawn here on the host, then handed to both the
device library and the oracle.

Recipe (per workload w and tensor id t: h=0, W=1, LM=2, Kc=3, Vc=4, Q=5):
  * a torch CPU generator seeded with ``seed_of(w, t, chunk)``;
  * float32 normal draws; W and LM scaled by 0.02 (standard deviation), the
    rest standard normal;
  * bf16 workloads round the float32 draws to bf16 (round to nearest even).
Large tensors are drawn in chunks along the leading dimension so host memory
stays bounded.
"""

import torch

TENSOR_IDS = {"h": 0, "W": 1, "LM": 2, "Kc": 3, "Vc": 4, "Q": 5, "E": 6,
              "g1": 7, "Wqkv": 8, "Wo": 9, "g2": 10, "Wgu": 11, "Wd": 12, "Kh": 13, "Vh": 14}
WEIGHT_STD = 0.02


def seed_of(workload, tensor_id, chunk=0):
    """Deterministic 63-bit seed for (workload, tensor, chunk)."""
    s = 2026
    for v in (workload, tensor_id, chunk):
        s = (s * 1_000_003 + v + 1) % (1 << 63)
    return s


def normal(shape, seed, std=1.0, dtype="f32"):
    """N(0, std^2) float32 draws, optionally rounded to bf16, as a CPU tensor.
    dtype: "f32" / "bf16" or torch.float32 / torch.bfloat16."""
    if dtype not in ("f32", "bf16", torch.float32, torch.bfloat16):
        raise ValueError(f"unsupported dtype {dtype!r}")
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16) if dtype in ("bf16", torch.bfloat16) else x


def _chunked(shape, workload, name, std, dtype):
    tid = TENSOR_IDS[name]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.empty(*shape, dtype=tdt)
    lead = shape[0]
    for c in range(lead):
        out[c] = normal(shape[1:], seed_of(workload, tid, c), std, dtype)
    return out


def make_inputs(cfg, names=("h", "W", "LM", "Kc", "Vc", "Q")):
    """Host tensors for one workload (torch CPU tensors, fp32 or bf16).

    h [b, H]; W [K, H, H] ([head, out, in]); LM [V, H];
    Kc, Vc [b, nkv, Pmax, d] with the tree nodes' K/V at slots P..P+T-1;
    Q [b, T, nq, d] (the tree nodes' queries); on request E [V, H], the input
    embedding table a Hydra-style draft adds to h (N(0, 1), the scale of h).
    """
    shapes = {
        "h": (cfg.b, cfg.H),
        "W": (cfg.K, cfg.H, cfg.H),
        "LM": (cfg.V, cfg.H),
        "Kc": (cfg.b, cfg.nkv, cfg.Pmax, cfg.d),
        "Vc": (cfg.b, cfg.nkv, cfg.Pmax, cfg.d),
        "Q": (cfg.b, cfg.T, cfg.nq, cfg.d),
        "E": (cfg.V, cfg.H),
    }
    out = {}
    for n in names:
        std = WEIGHT_STD if n in ("W", "LM") else 1.0
        out[n] = _chunked(shapes[n], cfg.index, n, std, cfg.dtype)
    return out


def mtp_width(H):
    """SwiGLU width of an MTP head layer: 8H/3 rounded up to a multiple of 256
    (11008 at H = 4096, the Llama-7B layer)."""
    return ((8 * H + 2) // 3 + 255) // 256 * 256


def make_mtp_inputs(cfg, F=None):
    """Host tensors of K MTP-style head layers for a workload (bf16):
    g1, g2 [K, H] = 1 + 0.02 N(0, 1); Wqkv [K, (nq + 2 nkv) d, H], Wo [K, H, nq d],
    Wgu [K, 2F, H] (gate / up rows interleaved), Wd [K, H, F] ~ N(0, 0.02^2);
    the heads' caches Kh, Vh [K, b, nkv, Pmax, d] ~ N(0, 1)."""
    c = cfg
    F = F or mtp_width(c.H)
    K = c.K
    shapes = {
        "Wqkv": (K, (c.nq + 2 * c.nkv) * c.d, c.H), "Wo": (K, c.H, c.nq * c.d),
        "Wgu": (K, 2 * F, c.H), "Wd": (K, c.H, F),
        "Kh": (K, c.b, c.nkv, c.Pmax, c.d), "Vh": (K, c.b, c.nkv, c.Pmax, c.d),
    }
    out = {}
    for n in ("g1", "g2"):
        g = normal((K, c.H), seed_of(c.index, TENSOR_IDS[n]), WEIGHT_STD, "f32") + 1.0
        out[n] = g.to(torch.bfloat16)
    for n, shp in shapes.items():
        std = 1.0 if n in ("Kh", "Vh") else WEIGHT_STD
        out[n] = _chunked(shp, c.index, n, std, "bf16")
    return out
