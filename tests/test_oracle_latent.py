"""Pins of the latent-MoE block oracle (CPU only).

The pages print no worked example of the block, so ``latent_block_ref`` is
pinned by: its bf16 rounding against a brute-force walk over every bf16 value
and against torch's float32 -> bfloat16 conversion; RMS-norm closed forms;
an identity-weight closed form of the whole block; and a pure-Python loop
evaluation on a tiny input.
"""

import math

import numpy as np
import pytest
import torch

import moe_inputs
from oracle.latent import bf16_bits_of, bf16_round, latent_block_ref, rms_norm
from oracle.route import route_ref
from tests.test_oracle_ffn import IdentityExperts, decode_scalar, identity_like


def bf16_value(p: int) -> float:
    """Value of the bf16 bit pattern p, from its fields."""
    sign = -1.0 if p & 0x8000 else 1.0
    e, m = (p >> 7) & 0xFF, p & 0x7F
    if e == 0:
        return sign * m * 2.0 ** -133
    if e == 255:
        return sign * math.inf if m == 0 else math.nan
    return sign * (1 + m / 128.0) * 2.0 ** (e - 127)


def test_bf16_round_brute_force_over_every_value():
    # every finite non-negative bf16 value p and its successor: the value
    # itself, a quarter and three quarters of the way, and the tie (to the
    # even pattern); the negative side mirrors
    pats = np.arange(0, 0x7F80)
    v = np.array([bf16_value(int(p)) for p in pats])
    nxt = np.array([bf16_value(int(p) + 1) for p in pats])  # 0x7F80 = inf for the last
    gap = np.where(np.isinf(nxt), 2.0 ** (127 - 7), nxt - v)
    for x, want in ((v, v), (v + gap / 4, v), (v + 3 * gap / 4, nxt)):
        assert np.array_equal(bf16_round(x), want)
        assert np.array_equal(bf16_round(-x), -want)
    tie = bf16_round(v + gap / 2)
    assert np.array_equal(tie, np.where(pats % 2 == 0, v, nxt))
    assert bf16_round(np.array([np.nan]))[0] != bf16_round(np.array([np.nan]))[0]
    assert np.array_equal(bf16_round(np.array([np.inf, -np.inf, 1e300])), [np.inf, -np.inf, np.inf])


def test_bf16_round_matches_torch_on_float32_values():
    g = np.random.default_rng(5)
    x = np.concatenate([
        g.standard_normal(200000).astype(np.float32) * np.float32(1e3),
        (g.random(50000) * 2.0 ** -126).astype(np.float32),  # float32 subnormals and bf16 subnormals
        np.frombuffer(g.bytes(4 * 100000), dtype=np.float32),  # every exponent
    ])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_round(x.astype(np.float64)), ref)
    assert np.array_equal(bf16_bits_of(ref), moe_inputs.bf16_bits(x))


def test_rms_norm_closed_forms():
    gamma = np.array([1.0, 2.0, -0.5, 3.0])
    # a constant row c: every element becomes gamma * c / sqrt(c^2 + eps)
    for c in (3.0, -0.25):
        out = rms_norm(np.full((1, 4), c), gamma, 1e-6)
        assert np.allclose(out, gamma * c / math.sqrt(c * c + 1e-6), rtol=1e-15)
    # the 3-4-5 row: mean square (9 + 16 + 0 + 0) / 4 = 6.25 -> rms 2.5
    out = rms_norm(np.array([[3.0, 4.0, 0.0, 0.0]]), gamma, 0.0)
    assert np.allclose(out, [[1.2, 3.2, 0.0, 0.0]], rtol=1e-15)
    # eps = 0: invariant under scaling the row
    d = np.random.default_rng(1).standard_normal((3, 16))
    assert np.allclose(rms_norm(d * 7.5, np.ones(16), 0.0), rms_norm(d, np.ones(16), 0.0), rtol=1e-14)


def identity_bits(rows, cols, scale=1.0):
    a = np.zeros((rows, cols), np.float32)
    n = min(rows, cols)
    a[np.arange(n), np.arange(n)] = scale
    return moe_inputs.bf16_bits(a)


def test_block_identity_closed_form():
    # H = D = 64: Wd = Wu = I, gamma = 1; experts W1 = W3 = [I; 0], W2 =
    # 2^e [I | 0]; shared Ws1 = Ws3 = [I; 0], Ws2 = [I | 0]; the gate picks
    # h's own features: Wg[e] = unit vector on feature e.  Then
    #   xl = bf16(h / rms(h)),  yl = sum_j w_j 2^e_j SiLU(xl) xl,
    #   out = bf16(yl) + bf16(SiLU(h) h)
    H = D = 64
    I = Is = 128
    E, k, T, eps = 4, 2, 5, 1e-6
    g = np.random.default_rng(3)
    h_bits = moe_inputs.bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    h = moe_inputs.bf16_to_f32(h_bits).astype(np.float64)
    wts = {"Wg": identity_bits(E, H), "Wd": identity_bits(D, H), "gamma": moe_inputs.bf16_bits(np.ones(D, np.float32)),
           "Wu": identity_bits(H, D), "Ws1": identity_bits(Is, H), "Ws3": identity_bits(Is, H),
           "Ws2": identity_bits(H, Is)}
    b = np.zeros(E, np.float32)
    out, parts = latent_block_ref(h_bits, wts, b, IdentityExperts(E, D, I), k, eps, return_parts=True)
    # router: logits are h's first E features
    assert np.array_equal(parts["z"], h[:, :E].astype(np.float32))
    ids, w = route_ref(h[:, :E].astype(np.float32), b, k)
    assert np.array_equal(parts["ids"], ids) and np.array_equal(parts["w"], w)
    rms = np.sqrt(np.mean(h * h, axis=1, keepdims=True) + eps)
    xl = bf16_round(h / rms)
    assert np.array_equal(moe_inputs.bf16_to_f32(parts["xl_bits"]).astype(np.float64), xl)
    base = xl * xl / (1.0 + np.exp(-xl))
    yl = np.stack([sum(float(w[t, j]) * 2.0 ** int(ids[t, j]) for j in range(k)) * base[t] for t in range(T)])
    assert np.allclose(parts["yl"], yl, rtol=1e-14, atol=0)
    expect = bf16_round(yl) + bf16_round(h * h / (1.0 + np.exp(-h)))
    assert np.allclose(out, expect, rtol=1e-14, atol=0)


def test_block_matches_python_loops_on_tiny_input():
    cfg = moe_inputs.BLOCK_TINY.with_(H=64, Is=32, layer=moe_inputs.BLOCK_TINY.layer.with_(E=4, k=2, D=32, I=32, T=2))
    L = cfg.layer
    h_bits = moe_inputs.block_hidden(cfg)
    wts = moe_inputs.block_dense_weights(cfg)
    b = moe_inputs.block_bias(cfg)
    experts = moe_inputs.ExpertSource(L)
    out = latent_block_ref(h_bits, wts, b, experts, L.k, cfg.eps)
    f = {n: moe_inputs.bf16_to_f32(v).astype(np.float64) for n, v in wts.items()}
    h = moe_inputs.bf16_to_f32(h_bits).astype(np.float64)

    def silu(v):
        return v / (1.0 + math.exp(-v))

    for t in range(L.T):
        hv = list(h[t])
        z = [sum(f["Wg"][e, c] * hv[c] for c in range(cfg.H)) for e in range(L.E)]
        ids, w = route_ref(np.array([z], np.float32), b, L.k)
        dv = [sum(f["Wd"][r, c] * hv[c] for c in range(cfg.H)) for r in range(L.D)]
        rms = math.sqrt(sum(v * v for v in dv) / L.D + cfg.eps)
        xl = [float(bf16_round(f["gamma"][r] * dv[r] / rms)) for r in range(L.D)]
        yl = [0.0] * L.D
        for j in range(L.k):
            (p1, s1), (p3, s3), (p2, s2) = experts[int(ids[0, j])]
            hh = []
            for i in range(L.I):
                gi = sum(decode_scalar(p1, s1, i, c) * xl[c] for c in range(L.D))
                ui = sum(decode_scalar(p3, s3, i, c) * xl[c] for c in range(L.D))
                hh.append(silu(gi) * ui)
            for r in range(L.D):
                yl[r] += float(w[0, j]) * sum(decode_scalar(p2, s2, r, i) * hh[i] for i in range(L.I))
        s = []
        for i in range(cfg.Is):
            gi = sum(f["Ws1"][i, c] * hv[c] for c in range(cfg.H))
            ui = sum(f["Ws3"][i, c] * hv[c] for c in range(cfg.H))
            s.append(float(bf16_round(silu(gi) * ui)))
        yb = [float(bf16_round(v)) for v in yl]
        ref = [sum(f["Wu"][o, r] * yb[r] for r in range(L.D)) + sum(f["Ws2"][o, i] * s[i] for i in range(cfg.Is))
               for o in range(cfg.H)]
        scale = max(abs(v) for v in ref)
        assert np.allclose(out[t], ref, rtol=1e-12, atol=1e-12 * scale), t


def test_token_subset_and_shapes():
    cfg = moe_inputs.BLOCK_TINY
    h_bits = moe_inputs.block_hidden(cfg)
    wts = moe_inputs.block_dense_weights(cfg)
    b = moe_inputs.block_bias(cfg)
    experts = moe_inputs.ExpertSource(cfg.layer)
    out = latent_block_ref(h_bits, wts, b, experts, cfg.layer.k, cfg.eps)
    assert out.shape == (cfg.T, cfg.H) and np.all(np.isfinite(out))
    sub = latent_block_ref(h_bits, wts, b, experts, cfg.layer.k, cfg.eps, tokens=[7, 2])
    assert np.allclose(sub, out[[7, 2]], rtol=1e-12, atol=1e-12)
    # outputs are about unit scale at these weight scales
    assert 0.1 < float(np.sqrt(np.mean(out * out))) < 10


@pytest.mark.parametrize("name", ["block-decode-t8", "block-prefill"])
def test_k3_block_inputs_have_unit_scale(name):
    cfg = moe_inputs.BLOCK_CONFIGS[name]
    wts = moe_inputs.block_dense_weights(cfg)
    assert wts["Wd"].shape == (3584, 7168) and wts["Wu"].shape == (7168, 3584) and wts["Wg"].shape == (896, 7168)
    sd = float(np.std(moe_inputs.bf16_to_f32(wts["Wd"][:64])))
    assert abs(sd * math.sqrt(7168) - 1) < 0.05
