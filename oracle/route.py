"""Sigmoid + bias top-k routing, in fp64 (numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The llama.cpp pull-request page "model: add Kimi-K3 text model" (comment "Dry
run: prepare_tensors() completes ...") gives the routing hyper-parameters:
896 experts, 16 used per token, expert score gating function "sigmoid", and a
per-expert bias tensor ``exp_probs_b``.  The pages do not spell out the rest;
the readings used here (and by the GPU library) are:

* score s[t,e] = sigmoid(z[t,e]) + b[e], in fp64; the bias only steers which
  experts are selected;
* experts are ranked by score, highest first, and among equal scores the lower
  expert index first; the first k are selected, in that order;
* a NaN score ranks below every number (as if it were -inf);
* gate weights are sigmoid(z) of the selected experts (no bias), divided by
  their sum when ``normalize`` is set, then multiplied by ``route_scale``, and
  rounded once to fp32.
"""

from __future__ import annotations

import numpy as np


def sigmoid64(z: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-z)) in fp64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def scores(z: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    """Selection scores s = sigmoid(z) + b (fp64), NaN mapped to -inf."""
    s = sigmoid64(z)
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)[None, :]
    return np.where(np.isnan(s), -np.inf, s)


def route_ref(z: np.ndarray, bias: np.ndarray | None, k: int, normalize: bool = True,
              route_scale: float = 1.0):
    """Top-k routing of every token.

    z: logits [T, E] (fp32); bias: [E] (fp32) or None for zero.
    Returns ids int32 [T, k] (descending score, ties -> lower index) and
    weights fp32 [T, k].
    """
    z = np.asarray(z)
    T, E = z.shape
    assert 1 <= k <= E
    s = scores(z, bias)
    expert = np.broadcast_to(np.arange(E), (T, E))
    # np.lexsort sorts by the LAST key first: primary key -s (score descending),
    # secondary key the expert index (ascending), stable.
    order = np.lexsort((expert, -s), axis=-1)
    ids = order[:, :k].astype(np.int32)
    g = np.take_along_axis(sigmoid64(z), ids.astype(np.int64), axis=1)
    if normalize:
        with np.errstate(invalid="ignore", divide="ignore"):
            g = g / g.sum(axis=1, keepdims=True)
    g = g * float(route_scale)
    return ids, g.astype(np.float32)
