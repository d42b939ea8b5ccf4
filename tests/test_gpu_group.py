"""GPU parity of moe_group_by_expert (the permute / scan step): bit-exact
against the oracle's stable counting sort, on every launch path of the
grouping (one fused launch for decode-sized batches, the count / scan / place
kernels for several 64-token chunks or very many experts)."""

import numpy as np
import pytest
import torch

import moe_inputs
from oracle.permute import permute_ref
from oracle.route import route_ref

pytestmark = pytest.mark.gpu


def check(k3, ids, E, what):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    ws = torch.full((max(k3.moe_group_workspace_size(T, E, k), 1),), 0xA5, dtype=torch.uint8, device="cuda")
    counts, offsets, row_tok, slot_row = (t.cpu().numpy() for t in
                                          k3.moe_group_by_expert(torch.from_numpy(ids).cuda(), E, workspace=ws))
    rc, ro, rt, rs = permute_ref(ids, E)
    n = int(ro[-1])
    assert np.array_equal(counts, rc), f"{what}: counts"
    assert np.array_equal(offsets, ro), f"{what}: offsets"
    assert np.array_equal(row_tok[:n], rt), f"{what}: row_tok"
    assert np.array_equal(slot_row, rs), f"{what}: slot_row"
    return counts, offsets, row_tok, slot_row


@pytest.mark.parametrize("name", ["tiny", "decode-t1", "decode-t8", "verify", "prefill"])
def test_configs(k3, name):
    cfg = moe_inputs.CONFIGS[name]
    print(f"[group] {name}", flush=True)
    z, b = moe_inputs.router_inputs(cfg)
    ids, _ = route_ref(z, b if cfg.bias_sigma > 0 else None, cfg.k)
    check(k3, ids, cfg.E, name)


@pytest.mark.parametrize(
    "T,E,k",
    [
        (1, 1, 1),  # one expert, one entry
        (16, 896, 64),  # 1024 entries: the largest single-launch batch
        (17, 896, 64),  # 1088 entries: one chunk, the three-phase single launch
        (64, 896, 16),  # exactly one chunk
        (65, 896, 16),  # two chunks, one token in the second
        (129, 300, 7),  # ragged third chunk, odd k
        (1000, 896, 16),  # 16 chunks, the last one partial
        (40, 5120, 2),  # largest E whose bitmaps and bases fit one launch's LDS
        (40, 5121, 2),  # one expert more: count / scan / place kernels
        (40, 8192, 2),  # largest supported E
        (3000, 8192, 3),  # many chunks and experts
        (5000, 896, 16),  # 79 chunks, the last one partial
    ],
)
def test_shapes(k3, T, E, k):
    print(f"[group] T={T} E={E} k={k}", flush=True)
    g = np.random.default_rng(T * 7 + E + k)
    ids = np.stack([g.permutation(E)[:k] if k <= E else g.integers(0, E, k) for _ in range(T)])
    check(k3, ids, E, f"T={T} E={E} k={k}")


def test_invalid_duplicate_and_hot_ids(k3):
    g = np.random.default_rng(5)
    for T in (7, 300):
        E, k = 40, 6
        ids = g.integers(0, E, size=(T, k)).astype(np.int32)  # random repeats inside rows
        ids[::3, 0] = -1  # out of range
        ids[::4, 5] = E  # out of range
        ids[1::5, 2] = 2**31 - 1
        ids[::2, 1] = 9  # hot expert
        check(k3, ids, E, f"invalid/duplicate T={T}")
        # nothing valid: every count zero, every entry skipped
        c, o, _, s = check(k3, np.full((T, k), -3, np.int32), E, f"all invalid T={T}")
        assert not c.any() and not o.any() and np.all(s == -1)
    # every token on one expert: 4096 rows of expert 3, in token order
    ids = np.full((4096, 1), 3, np.int32)
    c, o, r, s = check(k3, ids, 896, "one hot expert")
    assert c[3] == 4096 and np.array_equal(r[:4096], np.arange(4096)) and np.array_equal(s, np.arange(4096))


def test_determinism(k3):
    cfg = moe_inputs.PREFILL
    z, b = moe_inputs.router_inputs(cfg)
    ids = torch.from_numpy(route_ref(z, b, cfg.k)[0].astype(np.int32)).cuda()
    a = [t.cpu().numpy() for t in k3.moe_group_by_expert(ids, cfg.E)]
    c = [t.cpu().numpy() for t in k3.moe_group_by_expert(ids, cfg.E)]
    for u, v in zip(a, c):
        assert np.array_equal(u, v)
