"""GPU parity of moe_latent_block (the latent-MoE block) against the fp64 oracle.

Routing ids bit-exact (the inputs are checked to keep every checked token's
k-th and (k+1)-th scores apart by far more than the fp32 sums can move them);
the block output within the FFN bar: relative L2 error <= 2e-3 and max abs
error <= 1e-2 * max|ref|.  Small shapes on every token, through both dense
kernels (up to 16 tokens the weight-streaming kernel, beyond it the tile
kernel, with and without split-K) and ragged feature segments; the K3 shape
on chosen tokens at decode, verify and prefill sizes.
"""

import numpy as np
import pytest
import torch

import moe_inputs
from moe_inputs.device import upload_experts
from oracle.latent import latent_block_ref
from oracle.route import scores
from tests.gpu_util import assert_ffn_close, expert_blocks

pytestmark = pytest.mark.gpu


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class DenseDev:
    def __init__(self, cfg):
        self.host = moe_inputs.block_dense_weights(cfg)
        self.dev = {n: bf16_dev(v) for n, v in self.host.items()}
        self.bias_host = moe_inputs.block_bias(cfg)
        self.bias = torch.from_numpy(self.bias_host).cuda()


def run_block(k3, cfg, dense, experts, h_bits, **kw):
    L = cfg.layer
    T = h_bits.shape[0]
    ids = torch.empty((T, L.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, L.k), dtype=torch.float32, device="cuda")
    d = dense.dev
    out = k3.moe_latent_block(bf16_dev(h_bits), d["Wg"], dense.bias, d["Wd"], d["gamma"], experts.w1, experts.w3,
                              experts.w2, d["Wu"], d["Ws1"], d["Ws3"], d["Ws2"], L.k, eps=cfg.eps, topk_ids=ids,
                              topk_w=w, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


def check(cfg, dense, h_bits, got, gids, gw, tokens, what):
    L = cfg.layer
    ref, parts = latent_block_ref(h_bits, dense.host, dense.bias_host, moe_inputs.ExpertSource(L), L.k, cfg.eps,
                                  tokens=tokens, return_parts=True)
    # the checked tokens' routing is far from a tie: k-th and (k+1)-th scores
    # differ by much more than fp32 sums over H can move a logit
    s = np.sort(scores(parts["z"], dense.bias_host), axis=1)[:, ::-1]
    margin = float(np.min(s[:, L.k - 1] - s[:, L.k]))
    assert margin > 1e-5, margin
    assert np.array_equal(gids[tokens], parts["ids"]), what
    assert np.allclose(gw[tokens], parts["w"], rtol=1e-5, atol=1e-7), what
    assert_ffn_close(got[tokens], ref, what)


@pytest.fixture(scope="module")
def tiny(k3):
    cfg = moe_inputs.BLOCK_TINY
    experts = upload_experts(cfg.layer, expert_blocks(k3))
    return cfg, DenseDev(cfg), experts


@pytest.mark.parametrize("T", [1, 5, 16, 17, 32, 40, 64, 65, 200, 600, 1100])
def test_tiny_block_every_token(k3, tiny, T):
    # 8 experts top-2, H 256, latent 128, shared 192 (ragged 128-wide
    # segments: gate 8 of 128, shared 192 of 256); T <= 16: streaming kernel,
    # 17 .. 200: the tile kernel with split-K, 600 and 1100: several token
    # tiles, the last one ragged
    cfg, dense, experts = tiny
    cfg = cfg.with_(layer=cfg.layer.with_(T=T))
    h_bits = moe_inputs.block_hidden(cfg, seed=T)
    print(f"[block] tiny T={T}", flush=True)
    got, ids, w = run_block(k3, cfg, dense, experts, h_bits)
    assert np.all(np.isfinite(got))
    check(cfg, dense, h_bits, got, ids, w, np.arange(T), f"tiny T={T}")


def test_tiny_block_deterministic_and_in_a_graph(k3, tiny):
    cfg, dense, experts = tiny
    L = cfg.layer
    d = dense.dev
    hs = [bf16_dev(moe_inputs.block_hidden(cfg, seed=50 + i)) for i in range(4)]
    h_in = hs[0].clone()
    ws = torch.empty(k3.moe_latent_block_workspace_size(L.T, cfg.H, L.D, L.I, cfg.Is, L.E, L.k), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((L.T, cfg.H), dtype=torch.float32, device="cuda")

    def call(h, o):
        return k3.moe_latent_block(h, d["Wg"], dense.bias, d["Wd"], d["gamma"], experts.w1, experts.w3, experts.w2,
                                   d["Wu"], d["Ws1"], d["Ws3"], d["Ws2"], L.k, eps=cfg.eps, out=o, workspace=ws)

    eager = [call(h, torch.empty_like(out)).clone() for h in hs]
    again = call(hs[0], torch.empty_like(out))
    torch.cuda.synchronize()
    assert torch.equal(eager[0].view(torch.int32), again.view(torch.int32))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            call(h_in, out)
    torch.cuda.synchronize()
    for i, h in enumerate(hs):
        h_in.copy_(h)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager[i].view(torch.int32)), i


def test_block_stage_events(k3, tiny):
    cfg, dense, experts = tiny
    h_bits = moe_inputs.block_hidden(cfg, seed=9)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(k3.BLOCK_STAGE_EVENTS)]
    got, _, _ = run_block(k3, cfg, dense, experts, h_bits, stage_events=evs)
    plain, _, _ = run_block(k3, cfg, dense, experts, h_bits)
    assert np.array_equal(got.view(np.int32), plain.view(np.int32))
    ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(len(evs) - 1)]
    assert all(m >= 0 for m in ms)


@pytest.fixture(scope="module")
def k3_dense(k3):
    print("[block] K3 dense weights", flush=True)
    return DenseDev(moe_inputs.BLOCK_DECODE8)


# (workload, token count, checked tokens): decode through the streaming
# kernel, 64 and 128 tokens through the tile kernel with split-K, 4096 tokens
# with one split
K3_CASES = [("block-decode-t1", 1, [0]), ("block-decode-t8", 8, [7]), ("block-decode-t8", 64, [63]),
            ("block-prefill", 128, [127]), ("block-prefill", 4096, [1, 4095])]


@pytest.mark.parametrize("name,T,tokens", K3_CASES)
def test_k3_block(k3, k3_experts, k3_dense, name, T, tokens):
    cfg = moe_inputs.BLOCK_CONFIGS[name]
    cfg = cfg.with_(layer=cfg.layer.with_(T=T))
    dense = k3_dense
    if name == "block-prefill":  # its own selection bias, N(0, 0.5)
        dense = DenseDev.__new__(DenseDev)
        dense.host, dense.dev = k3_dense.host, k3_dense.dev
        dense.bias_host = moe_inputs.block_bias(cfg)
        dense.bias = torch.from_numpy(dense.bias_host).cuda()
    h_bits = moe_inputs.block_hidden(cfg)
    print(f"[block] K3 {name} T={T} tokens {tokens}", flush=True)
    got, ids, w = run_block(k3, cfg, dense, k3_experts, h_bits)
    assert np.all(np.isfinite(got))
    check(cfg, dense, h_bits, got, ids, w, np.array(tokens), f"{name} T={T}")
