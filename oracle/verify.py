"""Expert bytes of a speculative verify batch by width, and the width a cost
hint picks (numpy / Python, integer counts and fp64 rates).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The lucebox page "feat(kimi-k3): add DSpark Q8 artifact and shared
speculative runtime" verifies the current token plus 7 draft proposals per
sequence (section "DSpark acceptance-contract correction": width 8), notes
that routed-expert traffic grows with every verified row ("Kimi-K3 DSpark
workload probe") and adds target cost hints so that a target whose experts
live in external memory does not over-verify (Summary; "Runtime
validation": adaptive verification cut the streamed expert payload from 73.4
to 47.4 GiB).  The pages give no formula; the readings used here and by the
GPU library:

* a verify batch holds S sequences of W rows, row r = s * W + w (w = 0 the
  current token, w >= 1 the proposals); ``ids`` are the routed experts
  [S * W, k] of those rows;
* verifying width w (rows 0 .. w-1 of every sequence) streams every distinct
  expert those rows route to once, so its weight bytes are
  distinct[w - 1] * (bytes of one expert), distinct[w'] = number of distinct
  ids in [0, E) among rows with position <= w' (repeats and ids outside
  [0, E) add nothing);
* a pass of width w commits, per sequence, the target's own next token plus
  the accepted prefix of the w - 1 proposals: 1 + sum_{i=1}^{w-1} prod_{j<=i}
  a_j tokens in expectation, a_j = P(proposal j accepted | proposals before it
  accepted);
* its time is fixed_s + distinct[w - 1] * expert_bytes / bytes_per_s, and
  the hint picks the width with the highest expected committed tokens per
  second (the smallest width among equal rates).
"""

from __future__ import annotations

import numpy as np


def verify_distinct_ref(ids: np.ndarray, S: int, W: int, E: int) -> np.ndarray:
    """distinct[w] for w = 0 .. W-1: distinct experts routed by rows of
    position <= w, over all S sequences (int64 [W])."""
    ids = np.asarray(ids, dtype=np.int64)
    assert ids.shape[0] == S * W
    per_pos = ids.reshape(S, W, -1)
    out = np.zeros(W, dtype=np.int64)
    for w in range(W):
        sel = per_pos[:, : w + 1, :].reshape(-1)
        sel = sel[(sel >= 0) & (sel < E)]
        out[w] = np.unique(sel).size
    return out


def expected_committed(accept, w: int) -> float:
    """Expected tokens one sequence commits in a pass of width w (fp64)."""
    total, run = 1.0, 1.0
    for j in range(w - 1):
        run *= float(accept[j])
        total += run
    return total


def verify_width_choose_ref(distinct, S: int, accept, expert_bytes: float, bytes_per_s: float, fixed_s: float):
    """(best width in 1 .. W, fp64 rates [W] in committed tokens per second).

    accept: [W - 1] acceptance probabilities, or None for all ones."""
    W = len(distinct)
    if accept is None:
        accept = [1.0] * max(W - 1, 0)
    rates = np.zeros(W, dtype=np.float64)
    for w in range(1, W + 1):
        t = fixed_s + float(distinct[w - 1]) * expert_bytes / bytes_per_s
        rates[w - 1] = S * expected_committed(accept, w) / t
    best = int(np.argmax(rates)) + 1  # argmax takes the first maximum: the smallest width
    return best, rates
