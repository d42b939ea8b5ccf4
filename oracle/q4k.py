"""Q4_K expert blocks: decode and the routed FFN over them, in fp64 (numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages run K3 with requantized weights besides the native MXFP4 experts: a
trunk rewritten from Q8_0 to Q4_K (Hugging Face card "K3-Stuff", scripts list,
the requant_trunk.c entry), a Q3_K_M quant (llama.cpp page "model: add Kimi-K3
text model", comment by [jukofyork]) and a UD-IQ1_S target (lucebox page
"feat(kimi-k3): ...", "Runtime validation"), while warning that the QAT-trained
MXFP4 experts should never be requantized ("K3-Stuff", Key facts).  They name
these formats without defining them.  This module takes ggml's published
definition of the 4-bit k-quant block (``block_q4_K``), the simplest of the
named ones that needs no lookup table:

* one block covers 256 consecutive weights of a row in 144 bytes: fp16 ``d``
  (bytes 0-1), fp16 ``dmin`` (bytes 2-3), 12 bytes of packed 6-bit
  (scale, min) pairs for the eight 32-weight sub-blocks (bytes 4-15) and 128
  bytes of 4-bit codes (bytes 16-143);
* sub-block j < 4: scale = scales[j] & 63, min = scales[j + 4] & 63;
  sub-block j >= 4: scale = (scales[j + 4] & 15) | (scales[j - 4] >> 6) << 4,
  min = (scales[j + 4] >> 4) | (scales[j] >> 6) << 4;
* code bytes 32c .. 32c + 31 hold sub-block 2c in their low nibbles and
  sub-block 2c + 1 in their high nibbles, element i of the sub-block in byte
  32c + i;
* weight = d * scale * code - dmin * min.

Matrices are [rows, cols] with blocks along each row, as for MXFP4: a tensor
of ``rows`` rows is u8 [rows, cols / 256, 144].
"""

from __future__ import annotations

import numpy as np

from .ffn import ACT_SILU_MUL, ffn_ref, silu_mul

QK_K = 256  # weights per block
BLOCK_BYTES = 144  # bytes per block


def q4k_scale_min(scales: np.ndarray):
    """The eight (scale, min) pairs of each block from its 12 packed bytes.

    scales: u8 [..., 12] -> (sc, m), each int64 [..., 8] with values 0..63.
    """
    s = np.asarray(scales, dtype=np.int64)
    sc = np.empty(s.shape[:-1] + (8,), dtype=np.int64)
    m = np.empty_like(sc)
    for j in range(8):
        if j < 4:
            sc[..., j] = s[..., j] & 63
            m[..., j] = s[..., j + 4] & 63
        else:
            sc[..., j] = (s[..., j + 4] & 15) | ((s[..., j - 4] >> 6) << 4)
            m[..., j] = (s[..., j + 4] >> 4) | ((s[..., j] >> 6) << 4)
    return sc, m


def q4k_codes(qs: np.ndarray) -> np.ndarray:
    """4-bit codes of each block by sub-block: u8 [..., 128] -> int64 [..., 8, 32]."""
    q = np.asarray(qs, dtype=np.int64)
    chunks = q.reshape(q.shape[:-1] + (4, 32))  # chunk c holds sub-blocks 2c (low) and 2c + 1 (high)
    lo = chunks & 15
    hi = chunks >> 4
    return np.stack([lo, hi], axis=-2).reshape(q.shape[:-1] + (8, 32))


def q4k_decode(blocks: np.ndarray) -> np.ndarray:
    """Q4_K blocks u8 [rows, nb, 144] -> fp64 weights [rows, nb * 256]."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    if b.ndim != 3 or b.shape[-1] != BLOCK_BYTES:
        raise ValueError("expected u8 [rows, nb, 144]")
    rows, nb, _ = b.shape
    d = b[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)  # [rows, nb]
    dmin = b[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    sc, m = q4k_scale_min(b[..., 4:16])  # [rows, nb, 8]
    q = q4k_codes(b[..., 16:144])  # [rows, nb, 8, 32]
    w = d[..., None, None] * sc[..., None] * q - dmin[..., None, None] * m[..., None]
    return w.reshape(rows, nb * QK_K)


def expert_ffn_q4k(x: np.ndarray, blocks, act: int = ACT_SILU_MUL) -> np.ndarray:
    """One expert on rows x [n, D] (fp64); blocks = (w1, w3, w2) in Q4_K blocks.

    w1 and w3 are [I, D / 256, 144] (gate and up), w2 is [D, I / 256, 144].
    """
    if act != ACT_SILU_MUL:
        raise ValueError(f"unknown activation {act}")
    b1, b3, b2 = blocks
    g = x @ q4k_decode(b1).T
    u = x @ q4k_decode(b3).T
    return silu_mul(g, u) @ q4k_decode(b2).T


def ffn_q4k_ref(x_bits: np.ndarray, ids: np.ndarray, w: np.ndarray, experts, act: int = ACT_SILU_MUL,
                tokens=None) -> np.ndarray:
    """The routed FFN with Q4_K experts; ``experts[e]`` -> (w1, w3, w2) blocks.

    Same layer and conventions as ``ffn_ref`` (skipped entries contribute
    nothing; fp64 throughout), only the expert encoding differs.
    """
    return ffn_ref(x_bits, ids, w, experts, act, tokens, expert_fn=expert_ffn_q4k)
