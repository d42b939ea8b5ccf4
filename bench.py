#!/usr/bin/env python3
"""Routed-expert MXFP4 MoE layer (Kimi-K3 shape) on one MI355X.

One step is one pass of the whole hot path over one batch of tokens whose
inputs already sit in HBM: moe_route_topk (sigmoid + bias top-k) followed by
moe_mxfp4_ffn (grouping by expert, gate/up grouped GEMM with the MXFP4 decode
and the SiLU gating fused in, down grouped GEMM, weighted combine).  All 896
experts (15.7 GB of 17-byte MXFP4 blocks) are resident; the batches rotate over
several seeded routing inputs so successive steps touch different experts.

    python bench.py [--workload prefill|verify|decode-t8|decode-t1|tiny] [--steps K] [--warmup W]

Without --steps, K is chosen so the timed steps take about half a second.

Prints one JSON line (rank 0).  `value` is the wall-clock rate of K steps
replayed from captured HIP graphs (one graph per rotated batch; --eager times
plain launches).  The kernel timing behind "roofline" comes from HIP events
that the library records on its own stream around the dominant stage
(moe_mxfp4_ffn_profiled) in up to 200 eager steps run right after the timed ones; the
stage split comes from a short eager pass with every stage boundary marked.
`python bench.py --copy-calibration` only copies a 256 MiB buffer, the
reference kernel whose rocprofv3 FETCH_SIZE / WRITE_SIZE readings scale the
traffic counters.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "routed-MoE tokens/s at K3 shape; achieved HBM GB/s (decode) / MFMA % (prefill)"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # flop per byte
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
CSRC = "mxfp4_mixture_experts_moe_amd/csrc/"


def gemm_path(cfg) -> str:
    """Which grouped-GEMM kernels moe_mxfp4_ffn launches for this shape (the
    library's own selection rule, restated for labelling the roofline):
    "stream" (weight-streaming only, batches of up to 8 tokens), "tiled"
    (large-tile GEMMs for experts with more than 4 rows, weight-streaming for
    the others) or "small"."""
    entries = cfg.T * cfg.k
    fits = entries * max(cfg.I, cfg.D) * 2 < (1 << 31)
    if cfg.D % 512 == 0 and cfg.I % 512 == 0 and fits:
        return "stream" if cfg.T <= 8 else "tiled"
    return "small"


def kernel_info(stage: str, path: str, entries: int = 0, tokens: int = 0):
    """(kernel name(s) as rocprofv3 reports them, source files) of a stage.
    The large-tile down product takes 128-row tiles from 16384 routed entries
    on, 64-row tiles below."""
    if stage in ("gate_up", "down"):
        flag = "true" if stage == "gate_up" else "false"
        rows = 128 if stage == "gate_up" or entries >= 16384 else 64
        big, stream = f"ffn_big_kernel<{flag}, {rows}>", f"ffn_stream_kernel<{flag}, false, false>"
        if path == "stream":
            # a decode batch is grouped inside the gate/up launch, which reads x in
            # place up to 4 tokens (else x re-laid out by a small launch first)
            if stage == "gate_up":
                nat = "true" if tokens <= 4 else "false"
                return f"ffn_stream_kernel<true, true, {nat}>", [CSRC + "ffn_stream.hip"]
            return stream, [CSRC + "ffn_stream.hip"]
        if path == "tiled":
            return f"{big} + {stream}", [CSRC + "ffn_big.hip", CSRC + "ffn_stream.hip"]
        return f"ffn_gemm_kernel<NT, {flag}, ...>", [CSRC + "ffn.hip"]
    return {"route": ("route_topk_*kernel", [CSRC + "route.hip"]), "group": ("group_*_kernel / permute_x_kernel", [CSRC + "group.hip"]),
            "combine": ("combine_kernel", [CSRC + "ffn.hip"])}[stage]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (0: as many as fill about 0.5 s, 20 to 5000)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill", choices=["prefill", "verify", "decode-t8", "decode-t1", "tiny"])
    ap.add_argument("--rotate", type=int, default=0, help="distinct seeded batches cycled (0: 8 for decode, 4 else)")
    ap.add_argument("--cpu-baseline", dest="cpu_baseline", action="store_true", default=True)
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0, help="tokens the oracle evaluates (0: auto)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 256 MiB buffer 3 times (reference kernel for HBM traffic counters)")
    return ap.parse_args()


def source_sha(rels) -> str:
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(stage: str, workload: str, sources):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(TRAFFIC_DIR, f"{stage}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha") != source_sha(sources):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def stage_work(stage, cfg, rows, n_active):
    """Algorithmic (flops, bytes) of one launch of a stage.

    Weight bytes count every active expert's matrices once (17 bytes per 32
    weights); activation traffic counts each tensor once at its stored width.
    """
    T, D, I, E, k = cfg.T, cfg.D, cfg.I, cfg.E, cfg.k
    mat_w13 = I * (D // 32) * 17
    mat_w2 = D * (I // 32) * 17
    if stage == "gate_up":
        flops = 2.0 * 2 * rows * I * D
        byts = n_active * 2 * mat_w13 + T * D * 2 + rows * I * 4  # x (re-laid-out bf16) in, h hi+lo out
    elif stage == "down":
        flops = 2.0 * rows * D * I
        byts = n_active * mat_w2 + rows * I * 4 + rows * D * 4  # h hi+lo in, y fp32 out
    elif stage == "combine":
        flops = 2.0 * rows * D
        byts = rows * D * 4 + T * D * 4 + T * k * 8
    elif stage == "route":
        flops = 0.0
        byts = T * E * 4 + E * 4 + T * k * 8
    else:  # group
        flops = 0.0
        byts = T * k * 4 * 3 + T * D * 4
    return flops, byts


def cpu_baseline(cfg, batch, sample_tokens):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np

    from oracle.ffn import ffn_ref
    from oracle.route import route_ref

    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS default is one thread per core
        cores = os.cpu_count() or 1
    toks = np.arange(min(sample_tokens, cfg.T))
    t0 = time.perf_counter()
    ids, w = route_ref(batch.z[toks], batch.b, cfg.k)
    ffn_ref(batch.x[toks], ids, w, batch.experts)
    dt = time.perf_counter() - t0
    return {
        "value": len(toks) / dt,
        "unit": "tokens/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"first {len(toks)} of the {cfg.T} tokens of the seed-0 batch: fp64 routing of their "
                  f"logits + the FFN decoding every touched expert from the source MXFP4 layout "
                  f"({dt:.1f} s)",
    }


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for {max(args.gpus, world)}): this layer is built and "
              "measured on one MI355X; sharding is a design note only.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = 1 << 28
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copied {n} bytes 3 times", flush=True)
        return

    import moe_inputs
    import mxfp4_mixture_experts_moe_amd as k3
    from moe_inputs.device import upload_batch, upload_experts

    torch.cuda.set_device(0)
    cfg = moe_inputs.CONFIGS[args.workload]
    rotate = args.rotate or (8 if cfg.T <= 8 else 4)
    t_setup = time.perf_counter()
    dev = upload_experts(cfg, lambda p, s, out: k3.mxfp4_repack(p, s, blocks=out))
    batches = [upload_batch(cfg, seed=s) for s in range(rotate)]
    ws = torch.empty(k3.moe_mxfp4_ffn_workspace_size(cfg.T, cfg.D, cfg.I, cfg.E, cfg.k), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((cfg.T, cfg.D), dtype=torch.float32, device="cuda")
    ids = [torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda") for _ in range(rotate)]
    wts = [torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda") for _ in range(rotate)]
    # distinct experts each batch touches (for the weight-byte accounting)
    n_active = []
    for i, (_, x, z, b) in enumerate(batches):
        k3.moe_route_topk(z, b, cfg.k, ids=ids[i], weights=wts[i])
        n_active.append(int(torch.unique(ids[i]).numel()))
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    steps, warmup = args.steps, args.warmup
    stages = ["route", "group", "gate_up", "down", "combine"]

    def step(i, events=None):
        j = i % rotate
        _, x, z, b = batches[j]
        if events is not None and events[0] is not None:
            events[0].record()
        k3.moe_route_topk(z, b, cfg.k, ids=ids[j], weights=wts[j])
        k3.moe_mxfp4_ffn(x, ids[j], wts[j], dev.w1, dev.w3, dev.w2, out=out, workspace=ws,
                         stage_events=None if events is None else events[1:])

    def busy_head():
        # keep the GPU busy while the host enqueues the measured steps, so no
        # step waits for the host (matters for decode-sized steps)
        torch.cuda._sleep(int(2e7))

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # 1. stage split (eager, all stage boundaries marked) -> dominant stage
    n_split = max(rotate, min(steps, 16) if steps > 0 else 16)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(n_split)]
    busy_head()
    for i in range(n_split):
        step(warmup + i, ev[i])
    torch.cuda.synchronize()
    stage_ms = {s: float(np.mean([ev[i][n].elapsed_time(ev[i][n + 1]) for i in range(n_split)]))
                for n, s in enumerate(stages)}

    if steps <= 0:
        # long enough that clock ramp-up and the first replays do not show
        est_s = sum(stage_ms.values()) * 1e-3
        steps = int(min(5000, max(20, round(0.5 / max(est_s, 1e-6)))))

    # 2. the timed steps: one captured graph per rotated batch, replayed
    graphs = []
    if not args.eager:
        for j in range(rotate):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(j)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if graphs:
            graphs[(warmup + i) % rotate].replay()
        else:
            step(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # 3. eager steps with the dominant stage bracketed by two events on the
    #    library's stream (its per-launch duration for the roofline), and the
    #    eager step time from two events around all of them
    dom = max(stages, key=lambda s: stage_ms[s])
    n = stages.index(dom)
    n_ev = min(steps, 200)
    dev_ev = [[torch.cuda.Event(enable_timing=True) if m in (n, n + 1) else None for m in range(6)]
              for _ in range(n_ev)]
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    busy_head()
    e_start.record()
    for i in range(n_ev):
        step(warmup + i, dev_ev[i])
    e_end.record()
    torch.cuda.synchronize()
    dom_ms = float(np.mean([dev_ev[i][n].elapsed_time(dev_ev[i][n + 1]) for i in range(n_ev)]))
    eager_ms = e_start.elapsed_time(e_end) / n_ev

    rows = cfg.T * cfg.k
    act_ev = [n_active[(warmup + i) % rotate] for i in range(n_ev)]
    act_steps = [n_active[(warmup + i) % rotate] for i in range(steps)]
    flops, byts = stage_work(dom, cfg, rows, float(np.mean(act_ev)))
    bound = "mfma" if flops / max(byts, 1.0) > RIDGE else "hbm"
    dur_s = dom_ms * 1e-3
    if bound == "mfma":
        achieved, peak, unit = flops / dur_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = byts / dur_s / 1e9, PEAK_HBM_GBS, "GB/s"
    kname, ksrc = kernel_info(dom, gemm_path(cfg), cfg.T * cfg.k, cfg.T)
    traffic = stored_traffic(dom, args.workload, ksrc)

    value = cfg.T * steps / elapsed
    weight_bytes = float(np.mean(act_steps)) * (2 * cfg.I * (cfg.D // 32) * 17 + cfg.D * (cfg.I // 32) * 17)
    step_s = elapsed / steps
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded MXFP4 weights for all experts, bf16 N(0,1) activations, seeded router logits)",
        "config": {
            "workload": args.workload,
            "tokens": cfg.T,
            "experts": cfg.E,
            "top_k": cfg.k,
            "latent_dim": cfg.D,
            "expert_intermediate": cfg.I,
            "weights": "MXFP4 E2M1 + E8M0 in 17-byte blocks",
            "routing_inputs_rotated": rotate,
            "mean_active_experts": float(np.mean(act_steps)),
        },
        "roofline": {
            "kernel": kname,
            "bound": bound,
            "achieved": achieved,
            "peak": peak,
            "unit": unit,
            "frac": achieved / peak,
            "traffic": traffic,
            "algorithmic_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": byts,
            "avg_launch_ms": dom_ms,
        },
        "timing": ("graph replay of the step (route + FFN), one captured graph per rotated batch"
                   if graphs else "eager launches"),
        "eager_ms_per_step": eager_ms,
        "step_weight_GBps": weight_bytes / step_s / 1e9,
        "step_mfma_frac": cfg.T * 2 * cfg.k * 3 * cfg.D * cfg.I / step_s / (PEAK_BF16_TFLOPS * 1e12),
        "stages_ms": stage_ms,
        "setup_s": setup_s,
    }
    if args.cpu_baseline:
        sample = args.cpu_sample_tokens or (cfg.T if cfg.T <= 64 else 2)
        result["cpu_baseline"] = cpu_baseline(cfg, batches[0][0], sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
