"""GPU parity of moe_route_topk: ids bit-exact, weights to fp32 rounding."""

import numpy as np
import pytest
import torch

import moe_inputs
from oracle.route import route_ref, scores

pytestmark = pytest.mark.gpu

W_RTOL = 4e-7  # weights: fp64 -> fp32 rounding of sums taken in different orders


def run(k3, z, b, k, normalize=True, route_scale=1.0):
    zd = torch.from_numpy(np.ascontiguousarray(z)).cuda()
    bd = None if b is None else torch.from_numpy(np.ascontiguousarray(b)).cuda()
    ids, w = k3.moe_route_topk(zd, bd, k, normalize, route_scale)
    return ids.cpu().numpy(), w.cpu().numpy()


def check(k3, z, b, k, normalize=True, route_scale=1.0, what=""):
    ids, w = run(k3, z, b, k, normalize, route_scale)
    rid, rw = route_ref(z, b, k, normalize, route_scale)
    if not np.array_equal(ids, rid):
        bad = np.argwhere(ids != rid)
        t = int(bad[0][0])
        s = scores(z[t:t + 1], b)[0]
        gap = abs(s[ids[t]] - s[rid[t]]).max() if len(bad) else 0.0
        raise AssertionError(f"{what}: {len(bad)} id mismatches, first token {t}, fp64 score gap {gap:.3e}")
    fin = np.isfinite(rw)
    assert np.array_equal(fin, np.isfinite(w)), what
    np.testing.assert_allclose(w[fin], rw[fin], rtol=W_RTOL, atol=0, err_msg=what)


@pytest.mark.parametrize("name", ["tiny", "decode-t1", "decode-t8", "verify", "prefill"])
def test_configs(k3, name):
    cfg = moe_inputs.CONFIGS[name]
    print(f"[route] {name}", flush=True)
    z, b = moe_inputs.router_inputs(cfg)
    check(k3, z, b if cfg.bias_sigma > 0 else None, cfg.k, what=name)
    check(k3, z, b, cfg.k, what=name + " (explicit zero bias)")


@pytest.mark.parametrize("E,k", [(8, 1), (8, 8), (896, 16), (1024, 64), (2048, 16), (9000, 16), (12000, 3)])
def test_expert_counts(k3, E, k):
    """No expert cap: LDS-resident scores up to 8192 experts, recomputed beyond."""
    g = np.random.default_rng(E + k)
    T = 37
    z = g.standard_normal((T, E)).astype(np.float32)
    b = (g.standard_normal(E) * 0.5).astype(np.float32)
    check(k3, z, b, k, what=f"E={E} k={k}")


@pytest.mark.parametrize("T", [1, 7, 256, 257])
@pytest.mark.parametrize("E,k", [(8, 3), (200, 16), (256, 16), (257, 5), (513, 16), (896, 16), (1024, 16), (896, 17)])
def test_small_batch_router(k3, T, E, k):
    """Up to 256 tokens (E <= 1024, k <= 16) a workgroup of four waves routes each
    token; shares of fewer than k experts (E = 8, E = 200) leave sentinels among
    the candidates.  T = 257 and k = 17 take the one-wave-per-token kernel."""
    g = np.random.default_rng(1000 * T + E + k)
    z = g.standard_normal((T, E)).astype(np.float32)
    b = (g.standard_normal(E) * 0.5).astype(np.float32)
    check(k3, z, b, k, what=f"T={T} E={E} k={k}")
    z[:, ::3] = 0.25  # exact ties across the four waves' shares
    check(k3, z, None, k, what=f"T={T} E={E} k={k} ties")


def test_ties_nan_and_options(k3):
    z = np.zeros((5, 40), np.float32)
    check(k3, z, np.zeros(40, np.float32), 7, what="all equal")
    g = np.random.default_rng(9)
    z = np.round(g.standard_normal((64, 896)), 1).astype(np.float32)  # many exact ties
    check(k3, z, None, 16, what="rounded logits")
    z[3, 10] = np.nan
    z[5, :] = np.nan
    z[6, 7] = np.inf
    z[7, 100] = -np.inf
    check(k3, z, None, 16, what="nan/inf")
    zz = g.standard_normal((20, 896)).astype(np.float32)
    bb = (g.standard_normal(896) * 0.5).astype(np.float32)
    check(k3, zz, bb, 16, normalize=False, what="unnormalized")
    check(k3, zz, bb, 16, route_scale=2.827, what="scaled")
    check(k3, zz[:, :16].copy(), bb[:16].copy(), 16, what="k == E")


def test_large_batch_router_ties_and_fallback(k3):
    # more than 256 tokens: the one-wave router's filtered selection, and its
    # k-round fallback when more than 64 experts tie at the threshold
    g = np.random.default_rng(10)
    z = np.round(g.standard_normal((300, 896)), 1).astype(np.float32)  # many exact ties
    z[0, :] = 0.25  # every expert equal: fallback
    z[1, :448] = 1.0  # half the experts tie for first place: fallback
    z[2, 5] = np.nan
    z[3, :] = np.nan
    z[4, 9] = np.inf
    check(k3, z, None, 16, what="T=300 rounded/equal/nan")
    b = np.round(g.standard_normal(896) * 0.1, 2).astype(np.float32)
    check(k3, z, b, 16, what="T=300 rounded with bias")
    z2 = g.standard_normal((300, 1024)).astype(np.float32)
    check(k3, z2, None, 64, what="T=300 E=1024 k=64")
    check(k3, z2[:, :70].copy(), None, 64, what="T=300 E=70 k=64")


def test_empty_and_determinism(k3):
    ids, w = k3.moe_route_topk(torch.empty((0, 896), device="cuda"), None, 16)
    assert ids.shape == (0, 16)
    z, b = moe_inputs.router_inputs(moe_inputs.PREFILL)
    a = run(k3, z, b, 16)
    c = run(k3, z, b, 16)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1].view(np.uint32), c[1].view(np.uint32))


@pytest.mark.parametrize("n_close,E,k,T", [(40, 896, 16, 1), (40, 896, 16, 8), (20, 256, 16, 3), (100, 896, 16, 2),
                                           (70, 1024, 64, 1), (17, 896, 16, 300)])
def test_scores_closer_than_fp32_resolves(k3, n_close, E, k, T):
    # n_close experts get logits one fp32 ulp apart near 2.0, whose sigmoids
    # differ by about 2.5e-8: below what an fp32 score resolves, so the fp32
    # pre-filter keeps all of them as candidates and the fp64 scores decide
    # (more than 64 of them: the all-fp64 path); the others sit at 0 (score
    # 0.5, far below), with one token also carrying a bias that lifts an
    # outsider into the top k
    g = np.random.default_rng(n_close + E + k + T)
    z = np.zeros((T, E), np.float32)
    for t in range(T):
        pick = g.choice(E, size=n_close, replace=False)
        z[t, pick] = (np.float32(2.0) + np.arange(n_close, dtype=np.float32) * np.float32(2.0 ** -22))[g.permutation(n_close)]
    b = np.zeros(E, np.float32)
    b[g.integers(0, E)] = np.float32(0.4)
    print(f"[route] {n_close} close scores, E={E} k={k} T={T}", flush=True)
    check(k3, z, b, k, what=f"close scores n={n_close} E={E} k={k} T={T}")
    check(k3, z, None, k, what=f"close scores n={n_close} E={E} k={k} T={T}, no bias")
