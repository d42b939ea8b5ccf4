"""GPU parity of moe_q4k_ffn (the routed FFN over Q4_K experts) against the fp64 oracle.

Bar: the FFN bar (relative L2 error <= 2e-3, max abs error <= 1e-2 * max|ref|)
and, tighter, relative L2 <= 1e-4: the codes enter the MFMA exactly, the
block scales and mins are applied in fp32 and h carries about 16 significant
bits (the bf16 hi + lo pair), so the kernel's error is fp32 rounding, far
below the bar.  Small configs are compared on every output, the K3-shaped
batches on every token (1 token) or chosen tokens (8 tokens; the verify
batch's hottest expert), which the oracle evaluates one expert at a time.
"""

import numpy as np
import pytest
import torch

import moe_inputs
from oracle.q4k import ffn_q4k_ref
from oracle.route import route_ref
from tests.gpu_util import assert_ffn_close, bf16_dev, ffn_errors

pytestmark = pytest.mark.gpu

Q4K_REL_L2 = 1e-4


class Q4KExperts:
    """Q4_K experts in host memory, generated on first use and kept."""

    def __init__(self, cfg, patch=None):
        self.src = moe_inputs.ExpertSourceQ4K(cfg)
        self.cfg = cfg
        self.patch = patch
        self.cache = {}

    def __getitem__(self, e):
        if e not in self.cache:
            m = tuple(a.copy() for a in self.src[e])
            if self.patch is not None:
                self.patch(e, m)
            self.cache[e] = m
        return self.cache[e]

    def __len__(self):
        return self.cfg.E


def upload(host, experts):
    """Device tensors [E, rows, nb, 144] holding the listed experts (the others are never read)."""
    c = host.cfg
    w1 = torch.empty((c.E, c.I, c.D // 256, 144), dtype=torch.uint8, device="cuda")
    w3 = torch.empty_like(w1)
    w2 = torch.empty((c.E, c.D, c.I // 256, 144), dtype=torch.uint8, device="cuda")
    for e in experts:
        b1, b3, b2 = host[int(e)]
        w1[e].copy_(torch.from_numpy(b1))
        w3[e].copy_(torch.from_numpy(b3))
        w2[e].copy_(torch.from_numpy(b2))
    return w1, w3, w2


def used_experts(ids, E):
    ids = np.asarray(ids)
    return sorted({int(e) for e in ids.reshape(-1) if 0 <= e < E})


def run(k3, host, x_bits, ids, w, **kw):
    w1, w3, w2 = upload(host, used_experts(ids, host.cfg.E))
    out = k3.moe_q4k_ffn(bf16_dev(x_bits), torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(),
                         torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda(), w1, w3, w2, **kw)
    return out.cpu().numpy(), (w1, w3, w2)


def check(got, ref, what):
    assert_ffn_close(got, ref, what)
    rel, _, _ = ffn_errors(got, ref)
    assert rel <= Q4K_REL_L2, (what, rel)


def routed_case(cfg, seed=None):
    batch = moe_inputs.make_batch(cfg, seed)
    ids, w = route_ref(batch.z, batch.b, cfg.k)
    return batch, ids.astype(np.int32), w.astype(np.float32)


@pytest.mark.parametrize(
    "E,k,D,I,T",
    [
        (8, 2, 512, 768, 1),  # three blocks per row on the down product's K
        (8, 2, 512, 768, 5),
        (8, 2, 768, 512, 40),  # three blocks per row on gate/up's K
        (8, 2, 256, 256, 3),  # one block per row: a unit is a single stage
        (16, 4, 512, 512, 64),
        (8, 8, 512, 1280, 17),  # k = E: every expert sees every token (two 16-row tiles + 1)
        (200, 64, 512, 512, 8),  # the largest top-k: 512 routed entries
    ],
)
def test_q4k_shapes(k3, E, k, D, I, T):
    cfg = moe_inputs.TINY.with_(E=E, k=k, D=D, I=I, T=T, config_id=60 + T)
    print(f"[q4k] shapes E={E} k={k} D={D} I={I} T={T}", flush=True)
    batch, ids, w = routed_case(cfg)
    host = Q4KExperts(cfg)
    got, _ = run(k3, host, batch.x, ids, w)
    check(got, ffn_q4k_ref(batch.x, ids, w, host), f"q4k {E},{k},{D},{I},{T}")


def test_q4k_tiles_around_their_limits(k3):
    # experts of 1, 7, 8, 9, 15, 16 (one gate/up tile; one or two down tiles,
    # ragged), 17 (two gate/up tiles) and 40 rows; every token checked
    cfg = moe_inputs.TINY.with_(E=24, k=4, D=512, I=768, T=64, config_id=70)
    g = np.random.default_rng(70)
    ids = np.full((cfg.T, cfg.k), -1, np.int32)
    col = {}
    t0 = 0
    for e, n in ((0, 1), (1, 7), (2, 8), (3, 9), (4, 15), (5, 16), (6, 17), (7, 40)):
        for t in (t0 + np.arange(n)) % cfg.T:
            j = col.get(t, 0)
            ids[t, j] = e
            col[t] = j + 1
        t0 += n
    free = np.argwhere(ids < 0)
    fill = 8 + np.arange(len(free)) % 16
    for (t, j), e in zip(free, fill):
        ids[t, j] = e if e not in ids[t] else -1
    counts = [int((ids == e).sum()) for e in range(8)]
    assert counts == [1, 7, 8, 9, 15, 16, 17, 40], counts
    w = g.random((cfg.T, cfg.k)).astype(np.float32)
    batch = moe_inputs.make_batch(cfg)
    host = Q4KExperts(cfg)
    print("[q4k] tiles around their limits", flush=True)
    got, _ = run(k3, host, batch.x, ids, w)
    check(got, ffn_q4k_ref(batch.x, ids, w, host), "q4k tile limits")


def test_q4k_invalid_duplicate_ids_and_nan_weights_on_skipped_entries(k3):
    cfg = moe_inputs.TINY.with_(E=8, k=4, D=512, I=512, T=20, config_id=71)
    batch, ids, w = routed_case(cfg)
    ids[0, 1] = -1
    ids[1, 2] = cfg.E  # out of range
    ids[2, 3] = ids[2, 0]  # repeat within the token
    ids[3, :] = -5  # a token with nothing routed
    w[0, 1] = np.nan
    w[1, 2] = np.inf
    w[2, 3] = np.nan
    w[3, :] = np.nan
    host = Q4KExperts(cfg)
    print("[q4k] invalid and duplicate ids", flush=True)
    got, _ = run(k3, host, batch.x, ids, w)
    ref = ffn_q4k_ref(batch.x, ids, w, host)
    assert np.all(got[3] == 0.0)
    check(got, ref, "q4k skipped entries")


def _special_scales(e, mats):
    # d and dmin at the edges of fp16 in some blocks of every matrix: zero,
    # the smallest subnormal, the largest subnormal, negative values
    specials = [(0x0000, 0x0400), (0x0001, 0x0000), (0x03FF, 0x8400), (0x8800, 0x0C00), (0x0800, 0x8001)]
    for m, b in enumerate(mats):
        rows, nb = b.shape[0], b.shape[1]
        for i, (d, dmin) in enumerate(specials):
            r, t = (7 * i + 3 * e + m) % rows, (i + e) % nb
            b[r, t, 0], b[r, t, 1] = d & 0xFF, d >> 8
            b[r, t, 2], b[r, t, 3] = dmin & 0xFF, dmin >> 8


def test_q4k_fp16_scale_edge_values(k3):
    cfg = moe_inputs.TINY.with_(E=8, k=2, D=512, I=512, T=24, config_id=72)
    batch, ids, w = routed_case(cfg)
    host = Q4KExperts(cfg, patch=_special_scales)
    print("[q4k] fp16 scale edge values", flush=True)
    got, _ = run(k3, host, batch.x, ids, w)
    check(got, ffn_q4k_ref(batch.x, ids, w, host), "q4k fp16 edges")


def test_q4k_large_batch(k3):
    # 2048 tokens, every expert many 16-row tiles, every token checked
    cfg = moe_inputs.TINY.with_(E=40, k=8, D=512, I=512, T=2048, config_id=73)
    batch, ids, w = routed_case(cfg)
    host = Q4KExperts(cfg)
    print("[q4k] large batch", flush=True)
    got, _ = run(k3, host, batch.x, ids, w)
    check(got, ffn_q4k_ref(batch.x, ids, w, host), "q4k large batch")


def test_q4k_deterministic_and_graph_replay(k3):
    cfg = moe_inputs.TINY.with_(E=16, k=4, D=512, I=768, T=33, config_id=74)
    batch, ids, w = routed_case(cfg)
    host = Q4KExperts(cfg)
    x = bf16_dev(batch.x)
    ids_d = torch.from_numpy(ids).cuda()
    w_d = torch.from_numpy(w).cuda()
    w1, w3, w2 = upload(host, used_experts(ids, cfg.E))
    out1 = k3.moe_q4k_ffn(x, ids_d, w_d, w1, w3, w2)
    out2 = k3.moe_q4k_ffn(x, ids_d, w_d, w1, w3, w2)
    assert torch.equal(out1, out2)
    ws = torch.empty(k3.moe_q4k_ffn_workspace_size(cfg.T, cfg.D, cfg.I, cfg.E, cfg.k), dtype=torch.uint8, device="cuda")
    out_g = torch.empty_like(out1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        k3.moe_q4k_ffn(x, ids_d, w_d, w1, w3, w2, out=out_g, workspace=ws)  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        k3.moe_q4k_ffn(x, ids_d, w_d, w1, w3, w2, out=out_g, workspace=ws)
    for _ in range(3):
        out_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out1)
        k3.moe_q4k_ffn(x, ids_d, w_d, w1, w3, w2)  # eager work between the replays
        torch.cuda.synchronize()
    print("[q4k] deterministic, graph replays match", flush=True)


@pytest.mark.parametrize("name,tokens", [("decode-t1", None), ("decode-t8", [0, 5])])
def test_q4k_k3_decode(k3, name, tokens):
    # K3 shapes (896 experts, top-16, D 3584, I 3072; 14 and 12 blocks per row)
    cfg = moe_inputs.CONFIGS[name]
    batch, ids, w = routed_case(cfg)
    host = Q4KExperts(cfg)
    print(f"[q4k] K3 {name}", flush=True)
    got, _ = run(k3, host, batch.x, ids, w)
    sel = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    ref = ffn_q4k_ref(batch.x, ids, w, host, tokens=sel)
    check(got[sel], ref, f"q4k K3 {name}")


def test_q4k_k3_verify_hot_expert_tiles(k3):
    # K3 verify batch (128 tokens, Zipf-skewed routing): the hottest expert has
    # about 127 rows (eight 16-row gate/up and sixteen 8-row down tiles); the
    # checked tokens are its last and first rows and the batch's last token
    cfg = moe_inputs.VERIFY
    batch, ids, w = routed_case(cfg)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.E)
    hot = int(np.argmax(counts))
    rows = np.nonzero((ids == hot).any(axis=1))[0]
    assert counts[hot] > 64, counts[hot]
    sel = np.unique([rows[-1], rows[0], cfg.T - 1])
    host = Q4KExperts(cfg)
    print(f"[q4k] K3 verify, hot expert {hot} with {counts[hot]} rows, tokens {sel.tolist()}", flush=True)
    got, _ = run(k3, host, batch.x, ids, w)
    ref = ffn_q4k_ref(batch.x, ids, w, host, tokens=sel)
    check(got[sel], ref, "q4k K3 verify")


def test_q4k_k3_prefill_two_token_chunks(k3):
    # 20000 tokens at K3 shape run as a chunk of 18688 tokens and one of 1312
    # (32-bit activation offsets); checked: both sides of the chunk boundary,
    # the last token and the last row of each chunk's hottest expert
    cfg = moe_inputs.PREFILL.with_(T=20000, config_id=85)
    batch, ids, w = routed_case(cfg)
    host = Q4KExperts(cfg)
    chunk = 18688
    toks = {chunk - 1, chunk, cfg.T - 1}
    for lo, hi in ((0, chunk), (chunk, cfg.T)):
        sub = ids[lo:hi]
        e = int(np.argmax(np.bincount(sub.reshape(-1), minlength=cfg.E)))
        toks.add(lo + int(np.argwhere(sub == e)[:, 0].max()))
    toks = sorted(toks)
    print(f"[q4k] K3 prefill T={cfg.T}: tokens {toks}", flush=True)
    got, _ = run(k3, host, batch.x, ids, w)
    assert np.all(np.isfinite(got))
    ref = ffn_q4k_ref(batch.x, ids, w, host, tokens=np.array(toks))
    check(got[toks], ref, f"q4k T=20000 tokens {toks}")


@pytest.mark.parametrize("where", ["device", "pinned"])
def test_q4k_ffn_through_expert_cache(k3, where):
    # Q4_K experts staged by moe_expert_cache_route_q4k into 12 slots over 12
    # Zipf-skewed 3-token batches (hits and evictions): every step the FFN on
    # the slots gives exactly the bits of the FFN on the store's experts, the
    # renamed ids follow the oracle's LRU, and the last step matches the oracle
    from oracle.cache import ExpertCacheRef

    cfg = moe_inputs.TINY.with_(E=40, k=4, D=512, I=768, T=3, logits="zipf", config_id=75)
    C = 12
    host = Q4KExperts(cfg)
    w1, w3, w2 = upload(host, range(cfg.E))
    store = [w1, w3, w2] if where == "device" else [t.cpu().pin_memory() for t in (w1, w3, w2)]
    cache = [torch.zeros((C,) + tuple(t.shape[1:]), dtype=torch.uint8, device="cuda") for t in (w1, w3, w2)]
    state = k3.moe_expert_cache_init(cfg.E, C)
    ref = ExpertCacheRef(cfg.E, C)
    print(f"[q4k] through the expert cache, store={where}", flush=True)
    for step in range(12):
        batch, x, z, b = moe_inputs.device.upload_batch(cfg, seed=200 + step)
        ids_d, w_d = k3.moe_route_topk(z, b, cfg.k)
        slot_ids = k3.moe_expert_cache_route(state, cfg.E, C, ids_d, *store, *cache, q4k=True)
        got = k3.moe_q4k_ffn(x, slot_ids, w_d, *cache)
        want = k3.moe_q4k_ffn(x, ids_d, w_d, w1, w3, w2)
        torch.cuda.synchronize()
        ids = ids_d.cpu().numpy()
        ref.route(ids)
        want_slots = np.array([[ref.slot_of[e] if 0 <= e < cfg.E else -1 for e in row] for row in ids], np.int32)
        assert np.array_equal(slot_ids.cpu().numpy(), want_slots), step
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), step
    ids_o, w_o = route_ref(batch.z, batch.b, cfg.k)
    assert np.array_equal(ids, ids_o)
    check(got.cpu().numpy(), ffn_q4k_ref(batch.x, ids_o, w_o, host), "q4k through the cache")
    assert ref.hits_total > 0 and ref.misses_total > C  # the cache filled and evicted
