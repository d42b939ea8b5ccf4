"""GPU parity of the device expert cache (moe_expert_cache_init / _route)
against the oracle's ExpertCacheRef, and of the FFN run on the cache.

Integer work (tables, fetch list, renamed ids, copied bytes): bit-exact.  The
FFN on the cache's slots with the renamed ids must give exactly the bits of
the FFN on the store's experts with the original ids (the same kernels see
the same per-expert operands), and so stays within the oracle bar too.
"""

import numpy as np
import pytest
import torch

import moe_inputs
from moe_inputs.device import upload_experts
from oracle.cache import ExpertCacheRef
from oracle.ffn import ffn_ref
from oracle.route import route_ref
from tests.gpu_util import assert_ffn_close, bf16_dev, expert_blocks

pytestmark = pytest.mark.gpu


def _align(v):
    return (v + 255) // 256 * 256


def read_state(k3, state, E, C):
    """The documented state layout: header, slot_of[E], expert_in[C], order[C],
    fetch[2C], each on a 256-byte boundary."""
    raw = state.cpu().numpy()
    hdr = k3.moe_expert_cache_header(state)
    off = 256
    tables = {}
    for name, n in (("slot_of", E), ("expert_in", C), ("order", C), ("fetch", 2 * C)):
        tables[name] = raw[off:off + 4 * n].view(np.int32).copy()
        off = _align(off + 4 * n)
    assert off == k3.moe_expert_cache_state_size(E, C)
    return hdr, tables


class Store:
    """Random bytes standing for E experts' three matrices (the cache copies
    bytes; it never decodes them)."""

    def __init__(self, E, D, I, seed, where):
        g = np.random.default_rng(seed)
        shapes = ((E, I, D // 32, 17), (E, I, D // 32, 17), (E, D, I // 32, 17))
        self.host = [g.integers(0, 256, size=s, dtype=np.uint8) for s in shapes]
        if where == "device":
            self.t = [torch.from_numpy(a).cuda() for a in self.host]
        else:
            # pinned host memory; "pinned-offset" places each matrix 4 KiB into
            # a larger pinned allocation (a pointer inside it, not its start)
            off = 4096 if where == "pinned-offset" else 0
            self.t = []
            for a in self.host:
                buf = torch.empty(a.size + off + 4096, dtype=torch.uint8, pin_memory=True)
                v = buf[off:off + a.size].view(a.shape)
                v.numpy()[...] = a
                self.t.append(v)


def cache_buffers(C, D, I):
    return (torch.zeros((C, I, D // 32, 17), dtype=torch.uint8, device="cuda"),
            torch.zeros((C, I, D // 32, 17), dtype=torch.uint8, device="cuda"),
            torch.zeros((C, D, I // 32, 17), dtype=torch.uint8, device="cuda"))


def check_step(k3, state, ref, ids, slot_ids, fetch, h, m, cache, store, E, C):
    hdr, tab = read_state(k3, state, E, C)
    got_fetch = [tuple(p) for p in tab["fetch"][:2 * hdr["n_fetch"]].reshape(-1, 2).tolist()]
    assert got_fetch == fetch
    assert np.array_equal(slot_ids.cpu().numpy(), ref_slots(ids, ref, E))
    assert tab["slot_of"].tolist() == ref.slot_of
    assert tab["expert_in"].tolist() == ref.expert_in
    assert tab["order"].tolist() == ref.order
    assert (hdr["step"], hdr["hits"], hdr["misses"], hdr["n_fetch"]) == (ref.step, h, m, m)
    assert (hdr["hits_total"], hdr["misses_total"]) == (ref.hits_total, ref.misses_total)
    assert (hdr["E"], hdr["C"], hdr["tag"]) == (E, C, k3.EXPERT_CACHE_TAG)
    # every filled slot holds its expert's bytes, all three matrices
    held = np.array(ref.expert_in)
    slots = np.flatnonzero(held >= 0)
    for mat in range(3):
        assert np.array_equal(cache[mat].cpu().numpy()[slots], store.host[mat][held[slots]]), mat


def ref_slots(ids, ref, E):
    return np.array([[ref.slot_of[e] if 0 <= e < E else -1 for e in row] for row in ids], dtype=np.int32)


@pytest.mark.parametrize("E,C,T,k,D,I,where", [
    (40, 12, 3, 4, 64, 32, "device"),
    (40, 12, 3, 4, 64, 32, "pinned"),
    (40, 12, 3, 4, 64, 96, "pinned-offset"),
    (896, 160, 8, 16, 32, 32, "device"),   # K3's E, k and decode batch; tiny matrices
    (8192, 8192, 64, 64, 32, 32, "device"),  # the largest E and C: several items per thread
    (6, 6, 2, 3, 32, 64, "device"),        # C = E: nothing is ever evicted
])
def test_tables_fetch_and_bytes_match_oracle(k3, E, C, T, k, D, I, where):
    print(f"[cache] E={E} C={C} T={T} k={k} D={D} I={I} store={where}", flush=True)
    store = Store(E, D, I, seed=E * 7 + C, where=where)
    cache = cache_buffers(C, D, I)
    state = k3.moe_expert_cache_init(E, C)
    ref = ExpertCacheRef(E, C)
    g = np.random.default_rng(E + C + T)
    hot = g.choice(E, size=max(1, min(C, E) // 2), replace=False)
    for step in range(25 if E < 8192 else 6):
        ids = g.integers(-2, E + 2, size=(T, k)).astype(np.int32)  # some ids out of range
        ids[:, 0] = g.choice(hot, size=T)
        if step % 7 == 3:
            ids[:] = ids[0, 0]  # one expert repeated everywhere
        ids_d = torch.from_numpy(ids).cuda()
        slot_ids = k3.moe_expert_cache_route(state, E, C, ids_d, *store.t, *cache)
        torch.cuda.synchronize()
        _, fetch, h, m = ref.route(ids)
        check_step(k3, state, ref, ids, slot_ids, fetch, h, m, cache, store, E, C)
    assert ref.hits_total > 0 and ref.misses_total > 0


def test_empty_batch_and_uninitialised_state(k3):
    E, C, D, I = 40, 12, 32, 32
    store = Store(E, D, I, seed=3, where="device")
    cache = cache_buffers(C, D, I)
    state = k3.moe_expert_cache_init(E, C)
    # T == 0: a no-op (the state is unchanged)
    before = state.clone()
    k3.moe_expert_cache_route(state, E, C, torch.empty((0, 4), dtype=torch.int32, device="cuda"), *store.t, *cache)
    torch.cuda.synchronize()
    assert torch.equal(before, state)
    # a state initialised for other sizes (or never initialised) is left alone:
    # every entry gets -1, nothing is fetched
    other = k3.moe_expert_cache_init(E, C + 1)
    sizes = torch.zeros(k3.moe_expert_cache_state_size(E, C + 1), dtype=torch.uint8, device="cuda")
    ids = torch.tensor([[1, 2, 3, 4]], dtype=torch.int32, device="cuda")
    for st in (other, sizes):
        snap = st.clone()
        sid = k3.moe_expert_cache_route(st, E, C, ids, *store.t, *cache)
        torch.cuda.synchronize()
        assert sid.cpu().numpy().tolist() == [[-1, -1, -1, -1]]
        assert torch.equal(snap[48:], st[48:])  # tables untouched (only n_fetch may be cleared)
    assert not any(bool(c.any()) for c in cache)


def test_pageable_host_store_is_refused(k3):
    E, C, D, I = 8, 4, 32, 32
    state = k3.moe_expert_cache_init(E, C)
    cache = cache_buffers(C, D, I)
    host = [torch.zeros((E, I, 1, 17), dtype=torch.uint8), torch.zeros((E, I, 1, 17), dtype=torch.uint8),
            torch.zeros((E, D, 1, 17), dtype=torch.uint8)]
    ids = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    sid = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    st = k3.lib.moe_expert_cache_route(state.data_ptr(), state.numel(), E, C, ids.data_ptr(), 1, 2, sid.data_ptr(),
                                       *[h.data_ptr() for h in host], *[c.data_ptr() for c in cache], D, I,
                                       torch.cuda.current_stream().cuda_stream)
    assert st == -5  # K3MOE_ERR_UNSUPPORTED: pageable memory the GPU cannot read


def ffn_case(k3, cfg, C, where, steps, seed0):
    """Route `steps` batches of cfg through a cache of C slots; the FFN on the
    cache must give the FFN-on-the-store bits every step."""
    dev = upload_experts(cfg, expert_blocks(k3))
    if where == "pinned":
        store = [t.cpu().pin_memory() for t in (dev.w1, dev.w3, dev.w2)]
    else:
        store = [dev.w1, dev.w3, dev.w2]
    cache = cache_buffers(C, cfg.D, cfg.I)
    state = k3.moe_expert_cache_init(cfg.E, C)
    ref = ExpertCacheRef(cfg.E, C)
    for step in range(steps):
        batch, x, z, b = moe_inputs.device.upload_batch(cfg, seed=seed0 + step)
        ids_d, w_d = k3.moe_route_topk(z, b, cfg.k)
        slot_ids = k3.moe_expert_cache_route(state, cfg.E, C, ids_d, *store, *cache)
        got = k3.moe_mxfp4_ffn(x, slot_ids, w_d, *cache)
        want = k3.moe_mxfp4_ffn(x, ids_d, w_d, dev.w1, dev.w3, dev.w2)
        torch.cuda.synchronize()
        ids = ids_d.cpu().numpy()
        ref.route(ids)
        assert np.array_equal(slot_ids.cpu().numpy(), ref_slots(ids, ref, cfg.E)), step
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), step
        if step == steps - 1:
            ids_o, w_o = route_ref(batch.z, batch.b, cfg.k)
            assert np.array_equal(ids, ids_o)
            assert_ffn_close(got.cpu().numpy(), ffn_ref(batch.x, ids_o, w_o, batch.experts), f"cache step {step}")
    print(f"[cache] hits {ref.hits_total} misses {ref.misses_total}", flush=True)
    assert ref.hits_total > 0 and ref.misses_total > ref.C  # the cache filled and evicted


@pytest.mark.parametrize("where", ["device", "pinned"])
def test_ffn_on_cache_matches_resident(k3, where):
    # 40 experts, top-4, 3-token batches, 12 slots: decode-like batches that
    # evict; the skewed logits give hits
    cfg = moe_inputs.TINY.with_(E=40, k=4, D=512, I=1024, T=3, logits="zipf", config_id=91)
    print(f"[cache] ffn store={where}", flush=True)
    ffn_case(k3, cfg, 12, where, 12, 100)


def test_ffn_on_cache_inside_graph(k3):
    # route + FFN captured once and replayed on new routed ids (copied into the
    # captured input between replays): every replay matches the eager FFN on
    # the store and the oracle's tables
    cfg = moe_inputs.TINY.with_(E=40, k=4, D=512, I=512, T=4, logits="zipf", config_id=92)
    dev = upload_experts(cfg, expert_blocks(k3))
    C = 16
    cache = cache_buffers(C, cfg.D, cfg.I)
    state = k3.moe_expert_cache_init(cfg.E, C)
    ref = ExpertCacheRef(cfg.E, C)
    batches = [moe_inputs.device.upload_batch(cfg, seed=200 + i) for i in range(8)]
    routed = [k3.moe_route_topk(z, b, cfg.k) for _, _, z, b in batches]
    x_in = batches[0][1].clone()
    ids_in = routed[0][0].clone()
    w_in = routed[0][1].clone()
    slot_ids = torch.empty_like(ids_in)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(k3.moe_mxfp4_ffn_workspace_size(cfg.T, cfg.D, cfg.I, C, cfg.k), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            k3.moe_expert_cache_route(state, cfg.E, C, ids_in, dev.w1, dev.w3, dev.w2, *cache, slot_ids=slot_ids)
            k3.moe_mxfp4_ffn(x_in, slot_ids, w_in, *cache, out=out, workspace=ws)
    torch.cuda.synchronize()
    # capture ran nothing: the state is still empty
    assert k3.moe_expert_cache_header(state)["step"] == 0
    for i, ((_, x, _, _), (ids_d, w_d)) in enumerate(zip(batches, routed)):
        x_in.copy_(x)
        ids_in.copy_(ids_d)
        w_in.copy_(w_d)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = k3.moe_mxfp4_ffn(x, ids_d, w_d, dev.w1, dev.w3, dev.w2)
        torch.cuda.synchronize()
        ids = ids_d.cpu().numpy()
        ref.route(ids)
        assert np.array_equal(slot_ids.cpu().numpy(), ref_slots(ids, ref, cfg.E)), i
        assert torch.equal(out.view(torch.int32), want.view(torch.int32)), i
    assert k3.moe_expert_cache_header(state)["step"] == len(batches)


@pytest.mark.slow
def test_k3_decode_t8_through_cache(k3, k3_experts):
    """K3 decode batches of 8 tokens (896 experts, top-16) through a cache of
    160 slots fed from the resident experts: slot ids match the oracle, and
    the FFN on the cache gives the resident FFN's bits, every step."""
    cfg = moe_inputs.DECODE8
    C = 160
    cache = cache_buffers(C, cfg.D, cfg.I)
    state = k3.moe_expert_cache_init(cfg.E, C)
    ref = ExpertCacheRef(cfg.E, C)
    w = k3_experts
    for step in range(6):
        # consecutive decode steps: seeds differ, the hot set comes from the
        # shared zero bias and uniform logits, so hits are rare; repeat one
        # batch to force a step of hits only
        seed = 300 + (step if step != 3 else 2)
        batch, x, z, b = moe_inputs.device.upload_batch(cfg, seed=seed)
        ids_d, w_d = k3.moe_route_topk(z, b, cfg.k)
        slot_ids = k3.moe_expert_cache_route(state, cfg.E, C, ids_d, w.w1, w.w3, w.w2, *cache)
        got = k3.moe_mxfp4_ffn(x, slot_ids, w_d, *cache)
        want = k3.moe_mxfp4_ffn(x, ids_d, w_d, w.w1, w.w3, w.w2)
        torch.cuda.synchronize()
        ids = ids_d.cpu().numpy()
        _, fetch, h, m = ref.route(ids)
        print(f"[cache] K3 decode-t8 step {step}: hits {h} misses {m}", flush=True)
        assert np.array_equal(slot_ids.cpu().numpy(), ref_slots(ids, ref, cfg.E)), step
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), step
        if step == 3:
            assert m == 0
    hdr, tab = read_state(k3, state, cfg.E, C)
    assert tab["order"].tolist() == ref.order and tab["expert_in"].tolist() == ref.expert_in
    assert (hdr["hits_total"], hdr["misses_total"]) == (ref.hits_total, ref.misses_total)
