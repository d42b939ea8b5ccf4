"""GPU parity of moe_verify_width_distinct (integer: bit-exact) against the oracle."""

import numpy as np
import pytest
import torch

import moe_inputs
from oracle.route import route_ref
from oracle.verify import verify_distinct_ref

pytestmark = pytest.mark.gpu


def run(k3, ids, S, W, E):
    got = k3.moe_verify_width_distinct(torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda(), S, W, E)
    return got.cpu().numpy()


def test_verify_workload_routing(k3):
    # the verify workload's routed ids (16 sequences x width 8, Zipf-skewed logits)
    cfg = moe_inputs.VERIFY
    batch = moe_inputs.make_batch(cfg)
    ids, _ = route_ref(batch.z, batch.b, cfg.k)
    got = run(k3, ids, 16, 8, cfg.E)
    want = verify_distinct_ref(ids, 16, 8, cfg.E)
    print(f"[verify] distinct experts by width: {got.tolist()}", flush=True)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("S,W,k,E", [(16, 8, 16, 896), (1, 1, 1, 1), (3, 64, 4, 50), (64, 8, 16, 8192), (7, 5, 64, 300)])
def test_random_ids_with_invalid_entries(k3, S, W, k, E):
    g = np.random.default_rng(S * 1000 + W * 10 + k)
    ids = g.integers(-5, E + 5, size=(S * W, k)).astype(np.int32)
    assert np.array_equal(run(k3, ids, S, W, E), verify_distinct_ref(ids, S, W, E))


def test_edge_cases(k3):
    # no sequences: zeros; every id invalid: zeros; one hot expert everywhere
    z = k3.moe_verify_width_distinct(torch.empty((0, 16), dtype=torch.int32, device="cuda"), 0, 8, 896)
    assert z.cpu().numpy().tolist() == [0] * 8
    bad = np.full((16 * 8, 16), 896, np.int32)
    assert run(k3, bad, 16, 8, 896).tolist() == [0] * 8
    hot = np.tile(np.arange(16, dtype=np.int32), (16 * 8, 1))
    assert run(k3, hot, 16, 8, 896).tolist() == [16] * 8
    # determinism
    g = np.random.default_rng(1)
    ids = g.integers(0, 896, size=(128, 16)).astype(np.int32)
    assert np.array_equal(run(k3, ids, 16, 8, 896), run(k3, ids, 16, 8, 896))
