"""Grouping of routed (token, slot) entries by expert (numpy, integer only).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The routed-MoE FFN ("build_moe_ffn" on the llama.cpp page "model: add Kimi-K3
text model", comment "LLAMA_MAX_EXPERTS is 512, Kimi-K3 has 896") runs every
expert on the tokens routed to it.  Entry q = t*k + j is token t's j-th routed
expert.  The readings shared with the GPU library:

* an entry is valid when its id lies in [0, E) and does not repeat an id that
  appears earlier in the same token's row; invalid entries contribute nothing;
* rows of the grouped activations are ordered by (expert, token, slot), i.e. a
  stable sort of the valid entries by expert.
"""

from __future__ import annotations

import numpy as np


def valid_entries(ids: np.ndarray, E: int) -> np.ndarray:
    """Boolean [T, k]: in range and not a repeat within its token's row."""
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    ok = (ids >= 0) & (ids < E)
    for j in range(1, k):
        ok[:, j] &= ~np.any(ids[:, :j] == ids[:, j:j + 1], axis=1)
    return ok


def permute_ref(ids: np.ndarray, E: int):
    """Stable counting sort of the valid entries by expert.

    Returns
      counts   int32 [E]     valid entries per expert
      offsets  int32 [E+1]   exclusive prefix sum of counts
      row_tok  int32 [n]     token of each grouped row (n = number of valid entries)
      slot_row int32 [T*k]   grouped row of entry q, or -1 if q is invalid
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    ok = valid_entries(ids, E).reshape(-1)
    flat = ids.reshape(-1)
    q = np.nonzero(ok)[0]
    order = q[np.argsort(flat[q], kind="stable")]  # by (expert, q)
    counts = np.bincount(flat[q], minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    np.cumsum(counts, out=offsets[1:])
    row_tok = (order // k).astype(np.int32)
    slot_row = np.full(T * k, -1, dtype=np.int32)
    slot_row[order] = np.arange(order.size, dtype=np.int32)
    return counts, offsets, row_tok, slot_row
