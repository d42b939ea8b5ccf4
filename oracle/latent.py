"""The latent-MoE block around the routed experts, in fp64 (numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The llama.cpp page "model: add Kimi-K3 text model" names, in its opening
comment, a latent MoE in which the routed experts run at a latent width; its
dry-run comment lists the tensors of every MoE layer beside the experts —
the gate with its selection bias (exp_probs_b), ffn_routed_down,
ffn_routed_norm and ffn_routed_up — with a hidden (embedding) width of 7168,
896 experts, 16 used and sigmoid gating; a later review comment there names
shared-expert invariants.  The pages give no formula for the block.  The
reading used here and by the GPU library, one step each in this order, for
hidden rows h [T, H]:

    z   = h Wg^T                    gate projection, Wg [E, H]: router logits
    ids, w = route(fp32(z), b)      sigmoid + bias top-k (oracle.route)
    d   = h Wd^T                    ffn_routed_down, Wd [D, H]: hidden -> latent
    xl  = bf16(gamma * d / sqrt(mean(d^2) + eps))      ffn_routed_norm (RMS over D)
    yl  = the routed FFN of xl with ids, w            (oracle.ffn)
    s   = bf16(SiLU(h Ws1^T) * (h Ws3^T))             shared expert, Ws1, Ws3 [Is, H]
    out = bf16(yl) Wu^T + s Ws2^T   ffn_routed_up Wu [H, D]; shared down Ws2 [H, Is]

* h and every dense weight (including gamma) are bf16 values; products and
  sums are fp64.
* Each activation that enters a dense product as its input is a bf16 value
  (xl, yl, s: rounded to nearest, ties to even, straight from fp64); z, d and
  out are not rounded, except that the router takes z as fp32 (its input type).
* The shared expert runs at the hidden width with the routed experts'
  activation (SiLU(g) * u, the only form of the declared hook).
"""

from __future__ import annotations

import numpy as np

from .ffn import bf16_bits_to_f64, ffn_ref, silu_mul
from .route import route_ref

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_round(x) -> np.ndarray:
    """fp64 values rounded to the nearest bf16 value, ties to even (fp64 out).

    bf16 keeps 8 significant bits: a value in [2^(e-1), 2^e) is rounded to a
    multiple of 2^(e-8), and below the smallest normal 2^-126 to a multiple
    of 2^-133.  Results above the largest finite bf16 value become +-inf;
    inf and nan pass through."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
        r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def bf16_bits_of(x) -> np.ndarray:
    """Raw bits (uint16) of values that are already bf16 values."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def rms_norm(d: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """gamma * d / sqrt(mean(d^2) + eps) over the last axis (fp64)."""
    ms = np.mean(d * d, axis=-1, keepdims=True)
    return gamma * d / np.sqrt(ms + eps)


def latent_block_ref(h_bits, wts: dict, b, experts, k: int, eps: float, tokens=None, return_parts: bool = False):
    """The block for every token (or the listed ``tokens``); returns out fp64 [T', H].

    h_bits: bf16 bits [T, H]; wts: bf16 bits of Wg [E, H], Wd [D, H],
    gamma [D], Wu [H, D], Ws1 [Is, H], Ws3 [Is, H], Ws2 [H, Is]; b fp32 [E];
    experts[e]: the source-layout MXFP4 triple of routed expert e.
    With return_parts, also a dict of the intermediate values (z as fp32,
    ids, w, d, xl bits, yl, s)."""
    h_bits = np.asarray(h_bits)
    if tokens is not None:
        h_bits = h_bits[np.asarray(tokens, dtype=np.int64)]
    h = bf16_bits_to_f64(h_bits)
    W = {n: bf16_bits_to_f64(v) for n, v in wts.items()}
    z = (h @ W["Wg"].T).astype(np.float32)
    ids, w = route_ref(z, np.asarray(b, dtype=np.float32), k)
    d = h @ W["Wd"].T
    xl = bf16_round(rms_norm(d, W["gamma"], eps))
    xl_bits = bf16_bits_of(xl)
    yl = ffn_ref(xl_bits, ids, w, experts)
    s = bf16_round(silu_mul(h @ W["Ws1"].T, h @ W["Ws3"].T))
    out = bf16_round(yl) @ W["Wu"].T + s @ W["Ws2"].T
    if return_parts:
        return out, {"z": z, "ids": ids, "w": w, "d": d, "xl_bits": xl_bits, "yl": yl, "s": s}
    return out
