"""Pins for the oracle's MTP-style heads (oracle/mtp.py).

zackli.ai "Speculative Decoding Deep Dive II: Medusa, MTP", section "MTP":
head i is a transformer layer f_{h_i} on h_t, the logits f_u(f_{h_i}(h_t))
with the shared unembedding.  Pins, each independent of the oracle's own
formula:
  * zero output projections (Wo = Wd = 0) reduce every head to the base head
    LM h, exactly;
  * RMSNorm of a hand-computed vector;
  * the attention of the layer against torch's scaled_dot_product_attention
    (a library routine), with grouped query heads, read out through an
    identity output projection;
  * the SwiGLU MLP in closed form on a constant input (gate and up not
    swapped);
  * cache slots at or past P are never read; grouped-query head mapping.
Planted mistakes in a copy of the oracle (CPU only) must fail a pin.
"""

import math

import numpy as np
import pytest
import torch

from oracle import mtp as O
from oracle.mtp import mtp_draft, mtp_head, rmsnorm


def _weights(rng, H, nq, nkv, d, F, scale=0.1):
    return dict(g1=1.0 + 0.1 * rng.standard_normal(H), Wq=scale * rng.standard_normal((nq * d, H)),
                Wk=scale * rng.standard_normal((nkv * d, H)),
                Wv=scale * rng.standard_normal((nkv * d, H)),
                Wo=scale * rng.standard_normal((H, nq * d)), g2=1.0 + 0.1 * rng.standard_normal(H),
                Wg=scale * rng.standard_normal((F, H)), Wu=scale * rng.standard_normal((F, H)),
                Wd=scale * rng.standard_normal((H, F)))


def _head(w, h, Kc, Vc, P, nq, nkv, eps=1e-6, bf16=False):
    return mtp_head(h, w["g1"], w["Wq"], w["Wk"], w["Wv"], w["Wo"], w["g2"], w["Wg"], w["Wu"],
                    w["Wd"], Kc, Vc, P, nq, nkv, eps, bf16)


def test_zero_output_projections_reduce_to_the_base_head():
    rng = np.random.default_rng(1)
    b, H, nq, nkv, d, F, V, P = 2, 16, 4, 2, 4, 24, 30, 5
    heads = []
    for _ in range(3):
        w = _weights(rng, H, nq, nkv, d, F)
        w["Wo"][:] = 0.0
        w["Wd"][:] = 0.0
        heads.append(w)
    h = rng.standard_normal((b, H))
    LM = rng.standard_normal((V, H))
    Kh = rng.standard_normal((3, b, nkv, P + 2, d))
    Vh = rng.standard_normal((3, b, nkv, P + 2, d))
    u, logits, _ = mtp_draft(h, heads, LM, Kh, Vh, [P, P], nq, nkv, 1e-6, bf16=False)
    for i in range(4):
        assert np.array_equal(u[:, i], h)
        assert np.array_equal(logits[:, i], logits[:, 0])
    assert np.allclose(logits[:, 0], h @ LM.T, rtol=0, atol=1e-12)


def test_rmsnorm_hand_values():
    # x = (3, 4): mean square 12.5, so x / sqrt(12.5) = (3, 4) / 3.5355...
    got = rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 2.0]), 0.0)
    assert np.allclose(got, [3 / math.sqrt(12.5), 8 / math.sqrt(12.5)], rtol=0, atol=1e-15)
    # constant rows normalise to sign(c) * g
    got = rmsnorm(np.full((2, 5), -7.0), np.arange(1.0, 6.0), 0.0)
    assert np.allclose(got, -np.arange(1.0, 6.0)[None].repeat(2, 0), rtol=0, atol=1e-14)


@pytest.mark.parametrize("nq,nkv,P", [(4, 4, 6), (4, 2, 9), (6, 3, 0), (2, 1, 3)])
def test_attention_matches_library_sdpa(nq, nkv, P):
    # Wo = identity, MLP off (Wd = 0): y - h is the attention output o
    rng = np.random.default_rng(nq * 10 + nkv + P)
    b, d = 2, 4
    H = nq * d
    F = 8
    w = _weights(rng, H, nq, nkv, d, F, scale=0.3)
    w["Wo"] = np.eye(H)
    w["Wd"][:] = 0.0
    h = rng.standard_normal((b, H))
    Kc = rng.standard_normal((b, nkv, P + 3, d))
    Vc = rng.standard_normal((b, nkv, P + 3, d))
    y, k, v = _head(w, h, Kc, Vc, [P] * b, nq, nkv)
    o = (y - h).reshape(b, nq, d)
    a = rmsnorm(h, w["g1"], 1e-6)
    for s in range(b):
        q = torch.from_numpy((a[s] @ w["Wq"].T).reshape(nq, 1, d))
        keys = np.concatenate([Kc[s, :, :P], (a[s] @ w["Wk"].T).reshape(nkv, 1, d)], axis=1)
        vals = np.concatenate([Vc[s, :, :P], (a[s] @ w["Wv"].T).reshape(nkv, 1, d)], axis=1)
        kk = torch.from_numpy(keys).repeat_interleave(nq // nkv, dim=0)
        vv = torch.from_numpy(vals).repeat_interleave(nq // nkv, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv).numpy()[:, 0]
        assert np.allclose(o[s], ref, rtol=1e-12, atol=1e-12)
        assert np.allclose(k[s], keys[:, P], atol=0) and np.allclose(v[s], vals[:, P], atol=0)


def test_empty_prefix_attends_to_the_current_position_only():
    # one visible key: the softmax weight is exactly 1, so o = v
    rng = np.random.default_rng(3)
    b, nq, nkv, d, F = 2, 2, 2, 4, 8
    H = nq * d
    w = _weights(rng, H, nq, nkv, d, F)
    w["Wo"] = np.eye(H)
    w["Wd"][:] = 0.0
    h = rng.standard_normal((b, H))
    Kc = rng.standard_normal((b, nkv, 4, d))
    Vc = rng.standard_normal((b, nkv, 4, d))
    y, k, v = _head(w, h, Kc, Vc, [0, 0], nq, nkv)
    assert np.allclose(y - h, v.reshape(b, nq * d), rtol=0, atol=1e-14)


def test_swiglu_closed_form_on_a_constant_input():
    # h = 2 (every entry), g2 = 1, Wo = 0: x1 = h and a2 = 1 (the RMS of a
    # constant row is its magnitude), so gate_j = sum_k Wg[j, k] and up_j =
    # sum_k Wu[j, k]; Wd = identity (F = H) gives y_j = 2 + SiLU(gate_j) up_j
    rng = np.random.default_rng(4)
    H = F = 6
    nq = nkv = 2
    d = 3
    w = _weights(rng, H, nq, nkv, d, F)
    w["Wo"][:] = 0.0
    w["g2"] = np.ones(H)
    w["Wd"] = np.eye(H)
    h = np.full((1, H), 2.0)
    y, _, _ = _head(w, h, np.zeros((1, nkv, 1, d)), np.zeros((1, nkv, 1, d)), [0], nq, nkv, eps=0.0)
    for j in range(F):
        gate, up = w["Wg"][j].sum(), w["Wu"][j].sum()
        want = 2.0 + gate / (1.0 + math.exp(-gate)) * up
        assert abs(y[0, j] - want) <= 1e-12


def test_cache_past_the_prefix_is_not_read_and_gqa_mapping():
    rng = np.random.default_rng(5)
    b, nq, nkv, d, F, P = 1, 4, 2, 4, 8, 5
    H = nq * d
    w = _weights(rng, H, nq, nkv, d, F)
    w["Wo"] = np.eye(H)
    w["Wd"][:] = 0.0
    h = rng.standard_normal((b, H))
    Kc = rng.standard_normal((b, nkv, P + 4, d))
    Vc = rng.standard_normal((b, nkv, P + 4, d))
    y0, _, _ = _head(w, h, Kc, Vc, [P], nq, nkv)
    K2, V2 = Kc.copy(), Vc.copy()
    K2[:, :, P:] = 1e3
    V2[:, :, P:] = -1e3
    y1, _, _ = _head(w, h, K2, V2, [P], nq, nkv)
    assert np.array_equal(y0, y1)
    # moving kv head 1's prefix values changes only q heads 2, 3 (floor(h * nkv / nq))
    V3 = Vc.copy()
    V3[:, 1, :P] += 1.0
    y3, _, _ = _head(w, h, Kc, V3, [P], nq, nkv)
    o0, o3 = (y0 - h).reshape(nq, d), (y3 - h).reshape(nq, d)
    assert np.array_equal(o0[:2], o3[:2]) and not np.allclose(o0[2:], o3[2:])


def _pins_fail(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_mistakes_fail_a_pin(monkeypatch):
    # residual dropped after the attention
    real = O.mtp_head

    def no_residual(h, g1, Wq, Wk, Wv, Wo, g2, Wg, Wu, Wd, Kc, Vc, P, nq, nkv, eps, bf16):
        y, k, v = real(np.zeros_like(np.asarray(h, dtype=np.float64)), g1, Wq, Wk, Wv, Wo, g2, Wg,
                       Wu, Wd, Kc, Vc, P, nq, nkv, eps, bf16)
        return y, k, v
    monkeypatch.setattr(O, "mtp_head", no_residual)
    assert _pins_fail(test_zero_output_projections_reduce_to_the_base_head)
    monkeypatch.setattr(O, "mtp_head", real)
    # SiLU dropped from the gate
    real_silu = O.silu
    monkeypatch.setattr(O, "silu", lambda z: np.asarray(z, dtype=np.float64))
    assert _pins_fail(test_swiglu_closed_form_on_a_constant_input)
    monkeypatch.setattr(O, "silu", real_silu)
    # RMSNorm without the mean (sum of squares)
    real_rms = O.rmsnorm

    def rms_sum(x, g, eps):
        x = np.asarray(x, dtype=np.float64)
        return x / np.sqrt((x * x).sum(axis=-1, keepdims=True) + eps) * np.asarray(g, dtype=np.float64)
    monkeypatch.setattr(O, "rmsnorm", rms_sum)
    assert _pins_fail(test_rmsnorm_hand_values) or _pins_fail(test_swiglu_closed_form_on_a_constant_input)
