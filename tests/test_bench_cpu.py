"""Host logic of bench.py (no GPU): which GEMM path each workload takes, the
kernel names its roofline reports, and its algorithmic work per launch against
the per-token flop count and per-expert byte count of the K3 shape."""

import os
import sys

import pytest

import moe_inputs

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

K3_FLOPS_PER_TOKEN = 1_056_964_608  # 2 * k * 3 * D * I at k=16, D=3584, I=3072
K3_EXPERT_BYTES = 17_547_264  # 3 matrices of 3072 x 3584 weights, 17 bytes per 32


@pytest.mark.parametrize(
    "name,path",
    [("tiny", "small"), ("decode-t1", "stream"), ("decode-t8", "stream"), ("verify", "tiled"), ("prefill", "tiled")],
)
def test_gemm_path(name, path):
    assert bench.gemm_path(moe_inputs.CONFIGS[name]) == path


@pytest.mark.parametrize(
    "name,stage,kernel",
    [
        ("decode-t1", "gate_up", "ffn_stream_kernel<true, true, true>"),
        ("decode-t8", "gate_up", "ffn_stream_kernel<true, true, false>"),
        ("decode-t8", "down", "ffn_stream_kernel<false, false, false>"),
        ("verify", "gate_up", "ffn_big_kernel<true, 128> + ffn_stream_kernel<true, false, false>"),
        ("verify", "down", "ffn_big_kernel<false, 64> + ffn_stream_kernel<false, false, false>"),
        ("prefill", "down", "ffn_big_kernel<false, 128> + ffn_stream_kernel<false, false, false>"),
    ],
)
def test_kernel_names(name, stage, kernel):
    cfg = moe_inputs.CONFIGS[name]
    got, sources = bench.kernel_info(stage, bench.gemm_path(cfg), cfg.T * cfg.k, cfg.T)
    assert got == kernel
    assert all(os.path.exists(os.path.join(bench.ROOT, s)) for s in sources)


@pytest.mark.parametrize("name", ["decode-t1", "decode-t8", "verify", "prefill"])
def test_work_per_token_and_expert(name):
    cfg = moe_inputs.CONFIGS[name]
    rows = cfg.T * cfg.k
    f_gu, _ = bench.stage_work("gate_up", cfg, rows, 0)
    f_dn, _ = bench.stage_work("down", cfg, rows, 0)
    assert f_gu + f_dn == K3_FLOPS_PER_TOKEN * cfg.T
    # weight bytes of one active expert: the gate/up and down byte counts grow
    # by exactly one expert's matrices per extra active expert
    _, b0 = bench.stage_work("gate_up", cfg, rows, 0)
    _, b1 = bench.stage_work("gate_up", cfg, rows, 1)
    _, d0 = bench.stage_work("down", cfg, rows, 0)
    _, d1 = bench.stage_work("down", cfg, rows, 1)
    assert (b1 - b0) + (d1 - d0) == K3_EXPERT_BYTES
