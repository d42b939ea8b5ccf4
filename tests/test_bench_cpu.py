"""Host logic of bench.py (no GPU): which GEMM path each workload takes, the
kernel names its roofline reports, and its algorithmic work per launch against
the per-token flop count and per-expert byte count of the K3 shape."""

import os
import sys

import numpy as np
import pytest

import moe_inputs

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

K3_FLOPS_PER_TOKEN = 1_056_964_608  # 2 * k * 3 * D * I at k=16, D=3584, I=3072
K3_EXPERT_BYTES = 17_547_264  # 3 matrices of 3072 x 3584 weights, 17 bytes per 32
GEMM_LAUNCHES = ("gate_up", "gate_up_stream", "down", "down_stream")


@pytest.mark.parametrize(
    "name,path",
    [("tiny", "small"), ("decode-t1", "stream"), ("decode-t8", "stream"), ("verify", "tiled"), ("prefill", "tiled")],
)
def test_gemm_path(name, path):
    assert bench.gemm_path(moe_inputs.CONFIGS[name]) == path


def test_gemm_path_no_size_cliff():
    # prefill far beyond 2^31 bytes of grouped h: still the tiled path (the
    # library runs it in token chunks)
    assert bench.gemm_path(moe_inputs.PREFILL.with_(T=40000)) == "tiled"


@pytest.mark.parametrize(
    "name,launch,kernel",
    [
        ("decode-t1", "gate_up_stream", "ffn_stream_kernel<true, true, true>"),
        ("decode-t8", "gate_up_stream", "ffn_stream_kernel<true, true, false>"),
        ("decode-t8", "down_stream", "ffn_stream_kernel<false, false, false>"),
        ("decode-t1", "gate_up", None),
        ("decode-t8", "down", None),
        ("verify", "gate_up", "ffn_big_kernel<true, 128>"),
        ("verify", "gate_up_stream", "ffn_stream_shared_kernel<true>"),
        ("verify", "down_stream", "ffn_stream_shared_kernel<false>"),
        ("verify", "down", "ffn_big_kernel<false, 64>"),
        ("prefill", "down", "ffn_big_kernel<false, 128>"),
        ("tiny", "gate_up", "ffn_gemm_kernel<NT, true, ...>"),
        ("tiny", "down_stream", None),
    ],
)
def test_kernel_names(name, launch, kernel):
    cfg = moe_inputs.CONFIGS[name]
    info = bench.kernel_info(launch, bench.gemm_path(cfg), cfg.T * cfg.k, cfg.T)
    if kernel is None:
        assert info is None
        return
    got, sources = info
    assert got == kernel
    assert all(os.path.exists(os.path.join(bench.ROOT, s)) for s in sources)


def _counts(cfg, seed=0):
    g = np.random.default_rng(seed)
    ids = np.stack([g.permutation(cfg.E)[: cfg.k] for _ in range(cfg.T)])
    return np.bincount(ids.reshape(-1), minlength=cfg.E)


@pytest.mark.parametrize("name", ["decode-t1", "decode-t8", "verify", "prefill", "tiny"])
def test_work_per_token_and_expert(name):
    cfg = moe_inputs.CONFIGS[name]
    path = bench.gemm_path(cfg)
    counts = _counts(cfg)
    st = bench.routing_stats(counts, path)
    assert st[0] + st[2] == cfg.T * cfg.k and st[1] + st[3] == int((counts > 0).sum())
    flops = sum(bench.launch_work(l, cfg, path, st)[0] for l in GEMM_LAUNCHES)
    if name != "tiny":
        assert flops == K3_FLOPS_PER_TOKEN * cfg.T
    else:
        assert flops == 2 * cfg.k * 3 * cfg.D * cfg.I * cfg.T
    # one more expert served by the streaming kernels adds exactly one
    # expert's matrices to the weight bytes
    if path != "small":
        rb, nb, rs, ns = st
        more = (rb, nb, rs, ns + 1)
        d = sum(bench.launch_work(l, cfg, path, more)[1] - bench.launch_work(l, cfg, path, st)[1]
                for l in GEMM_LAUNCHES)
        assert d == K3_EXPERT_BYTES


def test_large_tile_h_and_y_counted_at_two_bytes():
    cfg = moe_inputs.PREFILL
    st = (1000, 1, 0, 0)  # one large-tile expert with 1000 rows
    _, b = bench.launch_work("down", cfg, "tiled", st)
    mat2 = cfg.D * (cfg.I // 32) * 17
    assert b == mat2 + 1000 * cfg.I * 2 + 1000 * cfg.D * 2
    _, s = bench.launch_work("down", cfg, "small", st)
    assert s == mat2 + 1000 * cfg.I * 4 + 1000 * cfg.D * 4


def test_routing_stats_split_at_sixteen_rows():
    counts = np.array([0, 1, 16, 17, 100, 0, 3])
    assert bench.routing_stats(counts, "tiled") == (117, 2, 20, 3)
    assert bench.routing_stats(counts, "stream") == (0, 0, 137, 5)
    assert bench.routing_stats(counts, "small") == (137, 5, 0, 0)


def test_q4k_accounting():
    # the Q4_K path: every expert in the gate_up / down launches of
    # ffn_q4k_kernel, 144 bytes per 256 weights
    cfg = moe_inputs.DECODE8
    assert bench.kernel_info("gate_up", "q4k")[0] == "ffn_q4k_kernel<true>"
    assert bench.kernel_info("down", "q4k")[0] == "ffn_q4k_kernel<false>"
    assert bench.kernel_info("gate_up_stream", "q4k") is None and bench.kernel_info("down_stream", "q4k") is None
    assert os.path.exists(os.path.join(bench.ROOT, bench.kernel_info("down", "q4k")[1][0]))
    counts = _counts(cfg)
    st = bench.routing_stats(counts, "q4k")
    assert st[0] == cfg.T * cfg.k and st[1] == int((counts > 0).sum()) and st[2] == st[3] == 0
    more = (st[0], st[1] + 1, 0, 0)
    d = sum(bench.launch_work(l, cfg, "q4k", more)[1] - bench.launch_work(l, cfg, "q4k", st)[1]
            for l in GEMM_LAUNCHES)
    assert d == 3 * cfg.I * cfg.D // 256 * 144 == 18579456
    flops = sum(bench.launch_work(l, cfg, "q4k", st)[0] for l in GEMM_LAUNCHES)
    assert flops == K3_FLOPS_PER_TOKEN * cfg.T
    assert set(bench.Q4K_WORKLOADS) <= set(["q4k-" + w for w in moe_inputs.CONFIGS])
