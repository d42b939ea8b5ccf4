"""Pins of the FFN oracle (CPU only).

No worked FFN example exists on the pages, so ``ffn_ref`` is pinned by closed
forms built from exactly representable weights and by an independent
pure-Python loop evaluation on tiny inputs.
"""

import math

import numpy as np

import moe_inputs
from oracle.ffn import ffn_ref
from oracle.route import route_ref


def identity_like(rows, cols, scale_exp=0):
    """(packed, scale) of the [rows, cols] matrix 2**scale_exp * delta(i, j)."""
    codes = np.zeros((rows, cols), np.uint8)
    n = min(rows, cols)
    codes[np.arange(n), np.arange(n)] = 2  # E2M1 code 2 = 1.0
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scale = np.full((rows, cols // 32), 127 + scale_exp, np.uint8)
    return packed, scale


class IdentityExperts:
    """Expert e: W1 = W3 = [I_D; 0] (I x D), W2 = 2**e [I_D | 0] (D x I)."""

    def __init__(self, E, D, I):
        self.E, self.D, self.I = E, D, I

    def __getitem__(self, e):
        return identity_like(self.I, self.D), identity_like(self.I, self.D), identity_like(self.D, self.I, e)

    def __len__(self):
        return self.E


def silu_mul_scalar(g, u):
    return g / (1.0 + math.exp(-g)) * u


def test_identity_weights_closed_form():
    E, D, I, T, k = 4, 128, 256, 5, 2
    g = np.random.default_rng(8)
    x_bits = moe_inputs.bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    x = moe_inputs.bf16_to_f32(x_bits).astype(np.float64)
    ids = np.array([[0, 1], [3, 2], [1, 0], [2, 2], [3, 0]], np.int32)
    w = g.random((T, k)).astype(np.float32)
    out = ffn_ref(x_bits, ids, w, IdentityExperts(E, D, I))
    base = x * (x / (1.0 + np.exp(-x)))  # SiLU(x) * x: gate = up = x
    expect = np.zeros_like(base)
    for t in range(T):
        seen = set()
        for j in range(k):
            e = int(ids[t, j])
            if e not in seen:
                expect[t] += float(w[t, j]) * (2.0 ** e) * base[t]
            seen.add(e)
    assert np.allclose(out, expect, rtol=1e-14, atol=0)


def decode_scalar(packed, scale, r, c):
    """Single weight from the source layout, read nibble by nibble."""
    byte = int(packed[r, c // 2])
    code = (byte >> 4) if (c % 2) else (byte & 15)
    mag = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0][code & 7]
    return (-mag if code & 8 else mag) * 2.0 ** (int(scale[r, c // 32]) - 127)


def test_matches_python_loops_on_tiny_input():
    cfg = moe_inputs.TINY.with_(E=4, k=2, D=64, I=64, T=3)
    batch = moe_inputs.make_batch(cfg)
    ids, w = route_ref(batch.z, batch.b, cfg.k)
    out = ffn_ref(batch.x, ids, w, batch.experts)
    x = moe_inputs.bf16_to_f32(batch.x).astype(np.float64)
    for t in range(cfg.T):
        ref = [0.0] * cfg.D
        for j in range(cfg.k):
            (p1, s1), (p3, s3), (p2, s2) = batch.experts[int(ids[t, j])]
            h = []
            for i in range(cfg.I):
                gi = sum(decode_scalar(p1, s1, i, d) * x[t, d] for d in range(cfg.D))
                ui = sum(decode_scalar(p3, s3, i, d) * x[t, d] for d in range(cfg.D))
                h.append(silu_mul_scalar(gi, ui))
            for d in range(cfg.D):
                ref[d] += float(w[t, j]) * sum(decode_scalar(p2, s2, d, i) * h[i] for i in range(cfg.I))
        assert np.allclose(out[t], ref, rtol=1e-12, atol=1e-12 * max(abs(v) for v in ref))


def test_linearity_slot_order_and_zero_weights():
    cfg = moe_inputs.TINY.with_(T=6)
    batch = moe_inputs.make_batch(cfg)
    ids, w = route_ref(batch.z, batch.b, cfg.k)
    out = ffn_ref(batch.x, ids, w, batch.experts)
    assert np.allclose(ffn_ref(batch.x, ids, 2 * w, batch.experts), 2 * out, rtol=1e-14)
    assert np.all(ffn_ref(batch.x, ids, 0 * w, batch.experts) == 0)
    flip = ids[:, ::-1].copy(), w[:, ::-1].copy()
    assert np.allclose(ffn_ref(batch.x, flip[0], flip[1], batch.experts), out, rtol=1e-13, atol=1e-12)
    # a token subset gives the same rows
    sub = ffn_ref(batch.x, ids, w, batch.experts, tokens=[4, 1])
    assert np.allclose(sub, out[[4, 1]], rtol=1e-13, atol=1e-13)  # BLAS blocking may differ by batch
    # out-of-range ids contribute nothing
    bad = ids.copy()
    bad[:, 1] = cfg.E + 3
    one = ffn_ref(batch.x, ids[:, :1].copy(), w[:, :1].copy(), batch.experts)
    assert np.allclose(ffn_ref(batch.x, bad, w, batch.experts), one, rtol=1e-13, atol=1e-13)
