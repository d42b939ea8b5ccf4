"""moe_mxfp4_ffn_noalloc (the FFN in the library's fixed device scratch)
against moe_mxfp4_ffn on the same inputs, through the C ABI: two calls in a
row, the second on a smaller batch, must give the existing entry point's
bits (and stay within the oracle bar)."""

import ctypes

import numpy as np
import pytest
import torch

import moe_inputs
from moe_inputs.device import upload_experts
from oracle.ffn import ffn_ref
from oracle.route import route_ref
from tests.gpu_util import assert_ffn_close, bf16_dev, expert_blocks

pytestmark = pytest.mark.gpu


def _noalloc(k3, x, ids, w, dev, out):
    T, D = x.shape
    k = ids.shape[1]
    E, I = dev.w1.shape[0], dev.w1.shape[1]
    st = k3.lib.moe_mxfp4_ffn_noalloc(
        ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(w.data_ptr()),
        ctypes.c_void_p(dev.w1.data_ptr()), ctypes.c_void_p(dev.w3.data_ptr()), ctypes.c_void_p(dev.w2.data_ptr()),
        T, D, I, E, k, 0, ctypes.c_void_p(out.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_matches_workspace_entry_point(k3):
    cfg = moe_inputs.TINY.with_(E=40, k=4, D=512, I=1024, T=90, config_id=81)
    dev = upload_experts(cfg, expert_blocks(k3))
    batch = moe_inputs.make_batch(cfg)
    ids, w = route_ref(batch.z, batch.b, cfg.k)
    x = bf16_dev(batch.x)
    ids_d = torch.from_numpy(ids.astype(np.int32)).cuda()
    w_d = torch.from_numpy(w.astype(np.float32)).cuda()
    # call 1: 90 tokens (large-tile and weight-streaming experts); call 2: the
    # first 5 tokens (weight-streaming only, grouped in the gate/up launch);
    # call 3: the first 2 tokens (x read in place)
    for T in (90, 5, 2):
        print(f"[noalloc] T={T}", flush=True)
        want = k3.moe_mxfp4_ffn(x[:T], ids_d[:T], w_d[:T], dev.w1, dev.w3, dev.w2)
        out = torch.full((T, cfg.D), float("nan"), dtype=torch.float32, device="cuda")
        assert _noalloc(k3, x[:T], ids_d[:T], w_d[:T], dev, out) == 0
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want.view(torch.int32)), f"T={T}"
        ref = ffn_ref(batch.x[:T], ids[:T], w[:T], batch.experts)
        assert_ffn_close(out.cpu().numpy(), ref, f"noalloc T={T}")


def test_noalloc_inside_graph_capture(k3):
    # a captured noalloc call replays to the eager bits (the scratch keeps
    # whatever the previous call left; nothing in it needs clearing)
    cfg = moe_inputs.TINY.with_(E=16, k=4, D=512, I=512, T=40, config_id=82)
    dev = upload_experts(cfg, expert_blocks(k3))
    batch = moe_inputs.make_batch(cfg)
    ids, w = route_ref(batch.z, batch.b, cfg.k)
    x = bf16_dev(batch.x)
    ids_d = torch.from_numpy(ids.astype(np.int32)).cuda()
    w_d = torch.from_numpy(w.astype(np.float32)).cuda()
    want = k3.moe_mxfp4_ffn(x, ids_d, w_d, dev.w1, dev.w3, dev.w2)
    out = torch.empty((cfg.T, cfg.D), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert _noalloc(k3, x, ids_d, w_d, dev, out) == 0
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want.view(torch.int32)), f"replay {rep}"
        _ = (x.float() * 3).sum().item()  # unrelated eager work between replays


def test_noalloc_rejects_sizes_beyond_its_scratch(k3):
    # K3 shape at 4096 tokens needs far more than the fixed scratch: status
    # K3MOE_ERR_TOO_LARGE, nothing enqueued (host check)
    A = 0x10000
    st = k3.lib.moe_mxfp4_ffn_noalloc(A, A, A, A, A, A, 4096, 3584, 3072, 896, 16, 0, A, None)
    assert st == -7
