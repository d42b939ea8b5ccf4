"""Routed-expert FFN with MXFP4 weights, in fp64 (numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the layer computes, per token t with routed experts e_j and gate weights
w_j (j = 0..k-1):

    out[t] = sum_j  w_j * W2[e_j] @ act(W1[e_j] @ x_t, W3[e_j] @ x_t)

* Experts run at the latent width ("latent MoE (routed experts run at
  n_expert_latent)", llama.cpp page "model: add Kimi-K3 text model", opening
  comment); the input x is the latent activation.  w1 is [I, D] (logical
  [3072, 3584] for K3, comment "repack_mxfp4_blocks is bit-exact"), w3 the same,
  w2 is [D, I]; MXFP4 blocks run along each matrix's input dimension.
* Each expert is the triple w1 | w2 | w3 (comment "Dry run: prepare_tensors()
  completes"), read here as w1 = gate, w3 = up, w2 = down.
* The pages name the activation "situ" but never define it; the layer takes it
  as a declared elementwise hook whose only form here is act(g, u) = SiLU(g) * u
  = g * sigmoid(g) * u.
* Weights are decoded from the SOURCE layout (``decode_ct``), so this oracle
  never reads the repacked blocks that the GPU path consumes.
* x is the exact bf16 value widened to fp64; everything else is fp64.
"""

from __future__ import annotations

import numpy as np

from .mxfp4 import decode_ct
from .permute import valid_entries

ACT_SILU_MUL = 0


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """SiLU(g) * u = g / (1 + exp(-g)) * u, fp64."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 raw bits -> fp64 (exact: bf16 is the top half of an fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def expert_ffn(x: np.ndarray, src, act: int = ACT_SILU_MUL) -> np.ndarray:
    """One expert on a batch of rows x [n, D] (fp64) -> [n, D] fp64.

    src = ((p1, s1), (p3, s3), (p2, s2)) in the source MXFP4 layout.
    """
    if act != ACT_SILU_MUL:
        raise ValueError(f"unknown activation {act}")
    (p1, s1), (p3, s3), (p2, s2) = src
    W1 = decode_ct(p1, s1)  # [I, D]
    W3 = decode_ct(p3, s3)  # [I, D]
    W2 = decode_ct(p2, s2)  # [D, I]
    g = x @ W1.T
    u = x @ W3.T
    h = silu_mul(g, u)
    return h @ W2.T


def ffn_ref(x_bits: np.ndarray, ids: np.ndarray, w: np.ndarray, experts, act: int = ACT_SILU_MUL,
            tokens=None, expert_fn=expert_ffn) -> np.ndarray:
    """The routed FFN for every token (or the listed ``tokens``), fp64 [T', D].

    x_bits: bf16 bits [T, D]; ids int [T, k]; w fp32 [T, k] (used as given);
    experts: ``experts[e]`` -> source-layout triple of expert e, evaluated by
    ``expert_fn(rows, experts[e], act)`` (another expert encoding passes its
    own).  Invalid entries (id out of range, or repeating an earlier id of the
    same token) contribute nothing.
    """
    ids = np.asarray(ids)
    T, k = ids.shape
    if tokens is None:
        tokens = np.arange(T)
    tokens = np.asarray(tokens, dtype=np.int64)
    x = bf16_bits_to_f64(np.asarray(x_bits)[tokens])
    sub_ids = ids[tokens]
    sub_w = np.asarray(w, dtype=np.float64)[tokens]
    E = len(experts)
    ok = valid_entries(sub_ids, E)
    out = np.zeros((tokens.size, x.shape[1]), dtype=np.float64)
    for e in np.unique(sub_ids[ok]):
        rows, slots = np.nonzero((sub_ids == e) & ok)
        y = expert_fn(x[rows], experts[int(e)], act)
        out[rows] += sub_w[rows, slots][:, None] * y
    return out
