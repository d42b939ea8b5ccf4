"""The C ABI without a GPU: symbols, host-side argument checks, workspace sizes.

Every call here fails (or succeeds as a no-op) in the host checks, before the
library touches the HIP runtime; the pointer values are never dereferenced.
"""

import os
import re

import pytest

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "k3moe.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_DEVICE, ERR_TOO_LARGE = 0, -1, -2, -3, -4, -5, -6, -7
A = 0x10000  # an aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol(k3):
    names = declared_functions()
    assert set(names) == {"k3moe_status_str", "moe_route_topk", "mxfp4_repack", "mxfp4_dequant", "mxfp4_tile",
                          "moe_mxfp4_ffn_workspace_size", "moe_mxfp4_ffn", "moe_mxfp4_ffn_profiled",
                          "moe_mxfp4_ffn_noalloc", "moe_q4k_ffn_workspace_size", "moe_q4k_ffn",
                          "moe_q4k_ffn_profiled", "moe_group_workspace_size", "moe_group_by_expert",
                          "moe_verify_width_distinct", "moe_verify_width_choose", "moe_expert_cache_state_size",
                          "moe_expert_cache_init", "moe_expert_cache_route", "moe_expert_cache_route_q4k", "moe_latent_block_workspace_size",
                          "moe_latent_block", "moe_latent_block_profiled"}
    for n in names:
        assert hasattr(k3.lib, n), n


def test_status_strings(k3):
    for s in range(-7, 1):
        assert k3.status_str(s) and k3.status_str(s) != "unknown status"
    assert k3.status_str(-99) == "unknown status"


def test_route_checks(k3):
    f = k3.lib.moe_route_topk
    assert f(A, None, 4, 8, 0, 1, 1.0, A, A, None) == ERR_SHAPE  # k < 1
    assert f(A, None, 4, 8, 9, 1, 1.0, A, A, None) == ERR_SHAPE  # k > E
    assert f(A, None, 4, 100, 65, 1, 1.0, A, A, None) == ERR_SHAPE  # k > 64
    assert f(A, None, -1, 8, 2, 1, 1.0, A, A, None) == ERR_SHAPE  # T < 0
    assert f(A, None, 4, 0, 1, 1, 1.0, A, A, None) == ERR_SHAPE  # E < 1
    assert f(None, None, 0, 8, 2, 1, 1.0, None, None, None) == OK  # T == 0: no-op
    assert f(None, None, 4, 8, 2, 1, 1.0, A, A, None) == ERR_NULL
    assert f(A, None, 4, 8, 2, 1, 1.0, None, A, None) == ERR_NULL
    assert f(A + 4, None, 4, 8, 2, 1, 1.0, A, A, None) == ERR_ALIGN
    assert f(A, A + 8, 4, 8, 2, 1, 1.0, A, A, None) == ERR_ALIGN


def test_codec_checks(k3):
    r, d = k3.lib.mxfp4_repack, k3.lib.mxfp4_dequant
    assert r(A, A, 4, 33, A, None) == ERR_SHAPE
    assert r(A, A, 4, 0, A, None) == ERR_SHAPE
    assert r(A, A, -1, 32, A, None) == ERR_SHAPE
    assert r(None, None, 0, 32, None, None) == OK
    assert r(A, None, 4, 32, A, None) == ERR_NULL
    assert r(A, A + 1, 4, 32, A, None) == ERR_ALIGN
    assert d(A, 4, 48, 0, A, None) == ERR_SHAPE
    assert d(A, 4, 64, 2, A, None) == ERR_UNSUPPORTED
    assert d(None, 0, 64, 1, None, None) == OK
    assert d(A, 4, 64, 0, None, None) == ERR_NULL
    assert d(A + 2, 4, 64, 0, A, None) == ERR_ALIGN


def test_tile_checks(k3):
    t = k3.lib.mxfp4_tile
    B = A + 0x100000  # a second aligned fake address, far from A
    assert t(A, 2, 16, 48, B, None) == ERR_SHAPE  # K % 32
    assert t(A, 2, 16, 0, B, None) == ERR_SHAPE
    assert t(A, -1, 16, 64, B, None) == ERR_SHAPE
    assert t(A, 2, 0, 64, B, None) == ERR_SHAPE  # N < 1
    assert t(A, 1 << 40, 1024, 4096, B, None) == ERR_SHAPE  # too many pieces
    assert t(None, 0, 16, 64, None, None) == OK  # nmat == 0: no-op
    assert t(None, 2, 16, 64, B, None) == ERR_NULL
    assert t(A, 2, 16, 64, None, None) == ERR_NULL
    assert t(A + 1, 2, 16, 64, B, None) == ERR_ALIGN
    assert t(A, 2, 16, 64, B + 8, None) == ERR_ALIGN
    # 2 matrices of 16 x 2 blocks = 1088 bytes: destinations that overlap the source
    assert t(A, 2, 16, 64, A, None) == ERR_SHAPE
    assert t(A, 2, 16, 64, A + 1072, None) == ERR_SHAPE
    assert t(A + 1072, 2, 16, 64, A, None) == ERR_SHAPE


def ffn(k3, T=8, D=256, I=256, E=8, k=2, act=0, ws_bytes=None, **ptrs):
    p = dict(x=A, ids=A, w=A, w1=A, w3=A, w2=A, out=A, ws=A)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = k3.moe_mxfp4_ffn_workspace_size(T, D, I, E, k)
    return k3.lib.moe_mxfp4_ffn(p["x"], p["ids"], p["w"], p["w1"], p["w3"], p["w2"], T, D, I, E, k, act, p["out"],
                                p["ws"], ws_bytes, None)


def test_ffn_checks(k3):
    assert ffn(k3, D=96 + 16) == ERR_SHAPE  # D % 32
    assert ffn(k3, I=200) == ERR_SHAPE  # I % 32
    assert ffn(k3, D=65536 + 32) == ERR_SHAPE  # above K3MOE_MAX_DIM_FFN
    assert ffn(k3, I=65536 + 32) == ERR_SHAPE
    assert ffn(k3, E=0) == ERR_SHAPE
    assert ffn(k3, E=8193, k=2) == ERR_SHAPE
    assert ffn(k3, k=0) == ERR_SHAPE
    assert ffn(k3, k=65, E=100) == ERR_SHAPE
    assert ffn(k3, k=9, E=8) == ERR_SHAPE  # k > E
    assert ffn(k3, T=-3) == ERR_SHAPE
    assert ffn(k3, T=2**31, k=1) == ERR_SHAPE  # T * k must stay below 2^31
    assert ffn(k3, act=1) == ERR_UNSUPPORTED
    assert ffn(k3, T=0, x=None, ids=None, w=None, w1=None, w3=None, w2=None, out=None, ws=None, ws_bytes=0) == OK
    assert ffn(k3, w3=None) == ERR_NULL
    assert ffn(k3, ws=None) == ERR_NULL
    assert ffn(k3, out=A + 4) == ERR_ALIGN
    need = k3.moe_mxfp4_ffn_workspace_size(8, 256, 256, 8, 2)
    assert ffn(k3, ws_bytes=need - 1) == ERR_WORKSPACE


@pytest.mark.parametrize("D,I", [(96, 160), (224, 288), (32, 32), (3584, 3072)])
def test_ffn_accepts_multiples_of_32(k3, D, I):
    # shapes that pass every host check fail only at the workspace check here
    # (a 1-byte workspace), before anything is enqueued
    assert k3.moe_mxfp4_ffn_workspace_size(8, D, I, 8, 2) > 0
    assert ffn(k3, D=D, I=I, ws_bytes=1) == ERR_WORKSPACE


def q4k_ffn(k3, T=8, D=256, I=512, E=8, k=2, act=0, ws_bytes=1 << 30, **ptrs):
    p = dict(x=A, ids=A, w=A, w1=A, w3=A, w2=A, out=A, ws=A)
    p.update(ptrs)
    return k3.lib.moe_q4k_ffn(p["x"], p["ids"], p["w"], p["w1"], p["w3"], p["w2"], T, D, I, E, k, act, p["out"],
                              p["ws"], ws_bytes, None)


def test_q4k_ffn_checks(k3):
    # Q4_K blocks cover 256 weights: D and I must be multiples of 256
    assert q4k_ffn(k3, D=128) == ERR_SHAPE
    assert q4k_ffn(k3, I=96) == ERR_SHAPE
    assert q4k_ffn(k3, D=256 + 32) == ERR_SHAPE
    assert q4k_ffn(k3, D=65536 + 256) == ERR_SHAPE
    assert q4k_ffn(k3, k=9, E=8) == ERR_SHAPE
    assert q4k_ffn(k3, T=-1) == ERR_SHAPE
    assert q4k_ffn(k3, act=1) == ERR_UNSUPPORTED
    assert q4k_ffn(k3, T=0, x=None, ids=None, w=None, w1=None, w3=None, w2=None, out=None, ws=None, ws_bytes=0) == OK
    assert q4k_ffn(k3, w2=None) == ERR_NULL
    assert q4k_ffn(k3, ws=None) == ERR_NULL
    assert q4k_ffn(k3, w1=A + 8) == ERR_ALIGN
    need = k3.moe_q4k_ffn_workspace_size(8, 256, 512, 8, 2)
    assert need > 0
    assert q4k_ffn(k3, ws_bytes=need - 1) == ERR_WORKSPACE
    assert k3.moe_q4k_ffn_workspace_size(8, 128, 512, 8, 2) == 0
    assert k3.moe_q4k_ffn_workspace_size(0, 256, 512, 8, 2) == 0
    # the same workspace layout as the MXFP4 path (grouping, h pair, fp32 y)
    assert k3.moe_q4k_ffn_workspace_size(128, 3584, 3072, 896, 16) == k3.moe_mxfp4_ffn_workspace_size(128, 3584, 3072, 896, 16)


def noalloc(k3, T=8, D=256, I=256, E=8, k=2, act=0, **ptrs):
    p = dict(x=A, ids=A, w=A, w1=A, w3=A, w2=A, out=A)
    p.update(ptrs)
    return k3.lib.moe_mxfp4_ffn_noalloc(p["x"], p["ids"], p["w"], p["w1"], p["w3"], p["w2"], T, D, I, E, k, act,
                                        p["out"], None)


def test_ffn_noalloc_checks(k3):
    assert noalloc(k3, D=100) == ERR_SHAPE
    assert noalloc(k3, k=9) == ERR_SHAPE
    assert noalloc(k3, act=3) == ERR_UNSUPPORTED
    assert noalloc(k3, T=0, x=None, ids=None, w=None, w1=None, w3=None, w2=None, out=None) == OK
    assert noalloc(k3, out=None) == ERR_NULL
    assert noalloc(k3, w1=A + 8) == ERR_ALIGN
    # K3 shape: 128 tokens fit the fixed scratch, 4096 do not
    ws = k3.moe_mxfp4_ffn_workspace_size
    assert ws(128, 3584, 3072, 896, 16) <= k3.NOALLOC_SCRATCH_BYTES < ws(4096, 3584, 3072, 896, 16)
    assert noalloc(k3, T=4096, D=3584, I=3072, E=896, k=16) == ERR_TOO_LARGE
    assert "scratch" in k3.status_str(ERR_TOO_LARGE)


def test_workspace_size(k3):
    ws = k3.moe_mxfp4_ffn_workspace_size
    assert ws(0, 3584, 3072, 896, 16) == 0
    assert ws(4, 100, 3072, 896, 16) == 0  # invalid shape -> 0
    a, b = ws(1, 3584, 3072, 896, 16), ws(4096, 3584, 3072, 896, 16)
    assert 0 < a < b
    T, D, I, k = 4096, 3584, 3072, 16
    # at least h (fp16 / bf16) + y (fp16) + the re-laid-out activations
    assert b >= T * k * I * 2 + T * k * D * 2 + T * D * 2
    assert b % 256 == 0


def test_workspace_is_one_token_chunk(k3):
    # past (2^31 - 1) / (2 k max(D, I)) tokens (rounded down to 64) the layer
    # runs in chunks that reuse one chunk's workspace
    ws = k3.moe_mxfp4_ffn_workspace_size
    D, I, E, k = 3584, 3072, 896, 16
    chunk = ((2**31 - 1) // (2 * k * max(D, I))) // 64 * 64
    assert chunk == 18688
    assert ws(chunk, D, I, E, k) == ws(chunk + 1, D, I, E, k) == ws(5 * chunk + 7, D, I, E, k)
    assert ws(chunk - 1, D, I, E, k) < ws(chunk, D, I, E, k)


def group(k3, T=8, E=8, k=2, ws_bytes=None, **ptrs):
    p = dict(ids=A, counts=A, offsets=A, row_tok=A, slot_row=A, ws=A)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = k3.moe_group_workspace_size(T, E, k)
    return k3.lib.moe_group_by_expert(p["ids"], T, E, k, p["counts"], p["offsets"], p["row_tok"], p["slot_row"],
                                      p["ws"], ws_bytes, None)


def test_group_checks(k3):
    assert group(k3, E=0) == ERR_SHAPE
    assert group(k3, E=8193) == ERR_SHAPE
    assert group(k3, k=0) == ERR_SHAPE
    assert group(k3, k=65) == ERR_SHAPE
    assert group(k3, T=-1) == ERR_SHAPE
    assert group(k3, T=2**31, k=1) == ERR_SHAPE  # T * k must stay below 2^31
    assert group(k3, T=0, ids=None, counts=None, offsets=None, row_tok=None, slot_row=None, ws=None,
                 ws_bytes=0) == OK
    assert group(k3, slot_row=None) == ERR_NULL
    assert group(k3, ws=None) == ERR_NULL
    assert group(k3, offsets=A + 4) == ERR_ALIGN
    need = k3.moe_group_workspace_size(8, 8, 2)
    assert need > 0 and need % 256 == 0
    assert group(k3, ws_bytes=need - 1) == ERR_WORKSPACE
    gw = k3.moe_group_workspace_size
    assert gw(0, 896, 16) == 0 and gw(4, 0, 16) == 0
    # chunk tables: one 64-bit token bitmap and one base per (64-token chunk, expert)
    assert gw(4096, 896, 16) >= 64 * 896 * 12


def test_verify_width_checks(k3):
    f = k3.lib.moe_verify_width_distinct
    assert f(A, 16, 0, 896, 16, A, None) == ERR_SHAPE  # W < 1
    assert f(A, 16, 65, 896, 16, A, None) == ERR_SHAPE  # W > 64
    assert f(A, -1, 8, 896, 16, A, None) == ERR_SHAPE
    assert f(A, 16, 8, 0, 16, A, None) == ERR_SHAPE
    assert f(A, 16, 8, 8193, 16, A, None) == ERR_SHAPE
    assert f(A, 16, 8, 896, 65, A, None) == ERR_SHAPE
    assert f(None, 16, 8, 896, 16, A, None) == ERR_NULL
    assert f(A, 16, 8, 896, 16, None, None) == ERR_NULL
    assert f(A + 4, 16, 8, 896, 16, A, None) == ERR_ALIGN


def test_verify_width_choose_matches_oracle(k3):
    # a host call: the library's choice and rates against the oracle's
    import numpy as np

    from oracle.verify import verify_width_choose_ref

    g = np.random.default_rng(21)
    for W in (1, 2, 8, 64):
        distinct = np.cumsum(g.integers(0, 40, size=W)) + 16
        accept = g.random(W - 1)
        for fixed in (0.0, 2e-4, 5e-3):
            best, rates = k3.moe_verify_width_choose(distinct.tolist(), 16, accept.tolist(), 17_547_264.0, 6.3e12, fixed)
            rbest, rrates = verify_width_choose_ref(distinct, 16, accept, 17_547_264.0, 6.3e12, fixed)
            assert best == rbest
            assert np.allclose(rates, rrates, rtol=1e-12, atol=0)
    best, _ = k3.moe_verify_width_choose([16, 16, 16], 4, None, 1e6, 1e9, 0.0)
    assert best == 3
    with pytest.raises(k3.K3MoeError):
        k3.moe_verify_width_choose([16, 20], 4, None, 1e6, 0.0, 0.0)  # no bandwidth


def test_expert_cache_state_size(k3):
    sz = k3.moe_expert_cache_state_size
    assert sz(0, 4) == 0 and sz(4, 0) == 0 and sz(8193, 4) == 0 and sz(4, 8193) == 0
    # header, slot_of[E], expert_in[C], order[C], fetch[2C], each on 256 bytes
    assert sz(896, 160) == 256 + 3584 + 768 + 768 + 1280
    assert sz(8192, 8192) >= 4 * (8192 + 4 * 8192)


def test_expert_cache_checks(k3):
    init, route = k3.lib.moe_expert_cache_init, k3.lib.moe_expert_cache_route
    need = k3.moe_expert_cache_state_size(896, 160)
    assert init(A, need, 0, 160, None) == ERR_SHAPE
    assert init(None, need, 896, 160, None) == ERR_NULL
    assert init(A + 4, need, 896, 160, None) == ERR_ALIGN
    assert init(A, need - 1, 896, 160, None) == ERR_WORKSPACE

    def r(state=A, nbytes=need, E=896, C=160, ids=A, T=8, k=16, sid=A, st=(A, A, A), ca=(A, A, A), D=7168, I=2048):
        return route(state, nbytes, E, C, ids, T, k, sid, *st, *ca, D, I, None)

    assert r(T=0) == OK  # an empty batch is a no-op
    assert r(C=127) == ERR_SHAPE  # 8 x 16 entries may use 128 experts
    assert r(E=100, C=99) == ERR_SHAPE  # ... and 100 experts of 100 (C = E holds any batch)
    assert r(k=0) == ERR_SHAPE and r(k=65) == ERR_SHAPE and r(T=-1) == ERR_SHAPE
    assert r(D=7000) == ERR_SHAPE and r(I=2050) == ERR_SHAPE and r(D=0) == ERR_SHAPE
    assert r(E=0) == ERR_SHAPE and r(C=8193) == ERR_SHAPE
    assert r(state=None) == ERR_NULL and r(ids=None) == ERR_NULL and r(sid=None) == ERR_NULL
    assert r(st=(A, None, A)) == ERR_NULL and r(ca=(A, A, None)) == ERR_NULL
    assert r(state=A + 4) == ERR_ALIGN and r(st=(A + 8, A, A)) == ERR_ALIGN and r(ca=(A, A + 2, A)) == ERR_ALIGN
    assert r(nbytes=need - 1) == ERR_WORKSPACE


def test_expert_cache_q4k_checks(k3):
    # the Q4_K entry: same checks, D and I multiples of 256 (Q4_K blocks)
    route = k3.lib.moe_expert_cache_route_q4k
    need = k3.moe_expert_cache_state_size(896, 160)

    def r(state=A, nbytes=need, E=896, C=160, ids=A, T=8, k=16, sid=A, st=(A, A, A), ca=(A, A, A), D=3584, I=3072):
        return route(state, nbytes, E, C, ids, T, k, sid, *st, *ca, D, I, None)

    assert r(T=0) == OK
    assert r(D=3584 + 32) == ERR_SHAPE and r(I=3072 + 128) == ERR_SHAPE  # multiples of 32 but not of 256
    assert r(C=127) == ERR_SHAPE and r(k=65) == ERR_SHAPE
    assert r(st=(A, A, None)) == ERR_NULL and r(ca=(A, A + 8, A)) == ERR_ALIGN
    assert r(nbytes=need - 1) == ERR_WORKSPACE
    # the MXFP4 entry accepts the same D as a multiple of 32 (it fails later, at the workspace check)
    assert k3.lib.moe_expert_cache_route(A, need - 1, 896, 160, A, 8, 16, A, A, A, A, A, A, A, 3584 + 32, 3072,
                                         None) == ERR_WORKSPACE


K3_BLOCK = dict(H=7168, D=3584, I=3072, Is=3072, E=896, k=16)


def test_latent_block_workspace_size(k3):
    ws = k3.moe_latent_block_workspace_size
    assert ws(0, **K3_BLOCK) == 0
    assert ws(8, 7000, 3584, 3072, 3072, 896, 16) == 0  # H not a multiple of 128
    assert ws(8, 7168, 3584, 3072, 3000, 896, 16) == 0  # Is not a multiple of 64
    assert ws(8, 7168, 3584, 3072, 3072, 8, 16) == 0    # k > E
    for T in (1, 8, 64, 65, 128, 4096):
        n = ws(T, **K3_BLOCK)
        # at least the FFN's own workspace and the block's activations
        assert n >= k3.moe_mxfp4_ffn_workspace_size(T, 3584, 3072, 896, 16) + T * (896 * 4 + 3584 * 4 + 3072 * 2)
    # the first product's sums (at decode the streaming kernel splits K inside
    # a workgroup and writes one fp32 row of 896 + 3584 + 3072 + 3072
    # features per token) fit the shared region
    assert ws(1, **K3_BLOCK) >= 10624 * 4


def test_latent_block_checks(k3):
    f = k3.lib.moe_latent_block
    need = k3.moe_latent_block_workspace_size(8, **K3_BLOCK)

    def call(T=8, H=7168, D=3584, I=3072, Is=3072, E=896, k=16, eps=1e-6, ptr=A, out=A, ws=A, nbytes=need,
             bias=None, ids=None):
        return f(ptr, ptr, bias, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, T, H, D, I, Is, E, k, 1, 1.0, eps, out,
                 ids, None, ws, nbytes, None)

    assert call(T=0, ptr=None, out=None, ws=None) == OK
    assert call(T=-1) == ERR_SHAPE and call(H=7040 + 64) == ERR_SHAPE and call(D=3584 + 32) == ERR_SHAPE
    assert call(Is=3072 + 32) == ERR_SHAPE and call(I=3072 + 16) == ERR_SHAPE and call(k=0) == ERR_SHAPE
    assert call(E=8, k=16) == ERR_SHAPE and call(k=65, E=896) == ERR_SHAPE and call(E=8193) == ERR_SHAPE
    assert call(eps=-1.0) == ERR_SHAPE and call(eps=float("nan")) == ERR_SHAPE and call(H=65536 + 128) == ERR_SHAPE
    assert call(ptr=None) == ERR_NULL and call(out=None) == ERR_NULL and call(ws=None) == ERR_NULL
    assert call(ptr=A + 2) == ERR_ALIGN and call(bias=A + 4) == ERR_ALIGN and call(ids=A + 8) == ERR_ALIGN
    assert call(nbytes=need - 1) == ERR_WORKSPACE
