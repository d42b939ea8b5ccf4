#!/usr/bin/env python3
"""Routed-expert MXFP4 MoE layer (Kimi-K3 shape) on one MI355X.

One step is one pass of the whole hot path over one batch of tokens whose
inputs already sit in HBM: moe_route_topk (sigmoid + bias top-k) followed by
moe_mxfp4_ffn (grouping by expert, gate/up grouped GEMM with the MXFP4 decode
and the SiLU gating fused in, down grouped GEMM, weighted combine).  All 896
experts (15.7 GB of 17-byte MXFP4 blocks) are resident; the batches rotate over
several seeded routing inputs so successive steps touch different experts.

    python bench.py [--workload prefill|verify|decode-t8|decode-t1|tiny|q4k-decode-t1|q4k-decode-t8|q4k-verify]
                    [--steps K] [--warmup W]
                    [--no-extra] [--no-cpu-baseline]

The headline workload (default: prefill, 4096 tokens) gives the JSON line's
`value`.  With the default workload the same process also measures the 8- and
1-token decode batches and the 128-token verify batch on the same resident
experts and reports them under "workloads", the verify cost hint under
"verify_width", 8-token decode with the experts streamed from an external
store (pinned host memory) through an 8 GiB device expert cache under
"expert_cache", the latent-MoE block under "latent_block", and then the
decode and verify batches again with the experts stored as Q4_K blocks
(moe_q4k_ffn), under "workloads" as q4k-decode-t1, q4k-decode-t8 and
q4k-verify (--no-extra skips all of these; --workload q4k-... runs one alone).

Without --steps, K is chosen so the timed steps take about half a second.

Prints one JSON line (rank 0).  `value` is the wall-clock rate of K steps
replayed from captured HIP graphs (one graph per rotated batch; --eager times
plain launches).  The roofline of each workload is that of its longest kernel
launch: its algorithmic flops or bytes per launch over its average duration,
which comes from two HIP events the library records on its own stream right
around that launch (moe_mxfp4_ffn_profiled keeps every launch on that stream)
in up to 200 eager steps run right after the timed ones.  The per-launch
split comes from a short eager pass with every launch boundary marked.
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
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 (and fp16) MFMA
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # flop per byte
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
CSRC = "mxfp4_mixture_experts_moe_amd/csrc/"
STREAM_MAX_ROWS = 16  # experts with more rows go to the large-tile kernels (tiled path)
EXTRA_WORKLOADS = ("decode-t1", "decode-t8", "verify")
# the same batches with the experts stored as Q4_K blocks (moe_q4k_ffn)
Q4K_WORKLOADS = ("q4k-decode-t1", "q4k-decode-t8", "q4k-verify")
Q4K_PREFIX = "q4k-"

# launch slots of one step; event i is recorded right before launch i
LAUNCHES = ("route", "group", "gate_up", "gate_up_stream", "down", "down_stream", "combine")
GEMM_LAUNCHES = ("gate_up", "gate_up_stream", "down", "down_stream")


def gemm_path(cfg) -> str:
    """Which grouped-GEMM kernels moe_mxfp4_ffn launches for this shape (the
    library's own selection rule, restated for labelling the roofline):
    "stream" (weight-streaming only, batches of up to 8 tokens), "tiled"
    (large-tile GEMMs for experts with more than 16 rows, shared-tile
    weight-streaming for the others) or "small" (the small-tile GEMMs for
    every expert)."""
    if cfg.D % 512 == 0 and cfg.I % 512 == 0:
        return "stream" if cfg.T <= 8 else "tiled"
    return "small"


def kernel_info(launch: str, path: str, entries: int = 0, tokens: int = 0):
    """(kernel name as rocprofv3 reports it, source files) of a launch slot;
    None when the path has no launch there.  The large-tile down product takes
    128-row tiles from 16384 routed entries on, 64-row tiles below."""
    big, stream, ffn = CSRC + "ffn_big.hip", CSRC + "ffn_stream.hip", CSRC + "ffn.hip"
    if path == "q4k":
        if launch in ("gate_up", "down"):
            return f"ffn_q4k_kernel<{'true' if launch == 'gate_up' else 'false'}>", [CSRC + "ffn_q4k.hip"]
        if launch in ("gate_up_stream", "down_stream"):
            return None
    if launch in ("gate_up", "down"):
        flag = "true" if launch == "gate_up" else "false"
        if path == "tiled":
            rows = 128 if launch == "gate_up" or entries >= 16384 else 64
            return f"ffn_big_kernel<{flag}, {rows}>", [big]
        if path == "small":
            return f"ffn_gemm_kernel<NT, {flag}, ...>", [ffn]
        return None
    if launch == "gate_up_stream":
        if path == "stream":
            # a decode batch is grouped inside the gate/up launch, which reads x
            # in place up to 4 tokens (else x re-laid out by a small launch first)
            return f"ffn_stream_kernel<true, true, {'true' if tokens <= 4 else 'false'}>", [stream]
        return ("ffn_stream_shared_kernel<true>", [stream]) if path == "tiled" else None
    if launch == "down_stream":
        if path == "tiled":
            return "ffn_stream_shared_kernel<false>", [stream]
        return ("ffn_stream_kernel<false, false, false>", [stream]) if path == "stream" else None
    return {"route": ("route_topk_*kernel", [CSRC + "route.hip"]),
            "group": ("group_*_kernel / permute_x_kernel", [CSRC + "group.hip"]),
            "combine": ("combine_kernel", [ffn])}[launch]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (0: as many as fill about 0.5 s, 20 to 5000)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill",
                    choices=["prefill", "verify", "decode-t8", "decode-t1", "tiny", *Q4K_WORKLOADS])
    ap.add_argument("--block", default=None, choices=[b[0] for b in BLOCK_SIZES],
                    help="measure only the latent-MoE block at this size (prints its result line)")
    ap.add_argument("--rotate", type=int, default=0, help="distinct seeded batches cycled (0: 8 for decode, 4 else)")
    ap.add_argument("--no-extra", dest="extra", action="store_false", default=True,
                    help="measure only the headline workload")
    ap.add_argument("--cpu-baseline", dest="cpu_baseline", action="store_true", default=True)
    ap.add_argument("--no-cpu-baseline", dest="cpu_baseline", action="store_false")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0, help="tokens the oracle evaluates (0: auto)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--serial-launches", action="store_true",
                    help="launch every FFN kernel on the caller's stream (no side-stream branch); the roofline's "
                         "timed launches are always serial, so profiles taken with this flag match them")
    ap.add_argument("--cold-steps", type=int, default=21,
                    help="steps timed one at a time after a 1 GiB cache-evicting read (median reported; 0: none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 256 MiB buffer 3 times (reference kernel for HBM traffic counters)")
    return ap.parse_args()


def source_sha(rels) -> str:
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(launch: str, workload: str, sources):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was taken
    on the current kernel source (else None)."""
    path = os.path.join(TRAFFIC_DIR, f"{launch}_{workload}_traffic.txt")
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


def routing_stats(counts, path: str):
    """Rows and distinct experts each GEMM kind serves, from the per-expert row
    counts of one batch: (rows_big, experts_big, rows_stream, experts_stream).
    "big" is the large-tile (tiled path) or small-tile (small path) launch."""
    rows_big = experts_big = rows_st = experts_st = 0
    for c in counts:
        c = int(c)
        if c == 0:
            continue
        big = (path in ("small", "q4k")) or (path == "tiled" and c > STREAM_MAX_ROWS)
        if big:
            rows_big += c
            experts_big += 1
        else:
            rows_st += c
            experts_st += 1
    return rows_big, experts_big, rows_st, experts_st


def launch_work(launch, cfg, path, stats):
    """Algorithmic (flops, bytes) of one launch.

    Weight bytes count every expert the launch serves once (17 bytes per 32
    weights); activations count x once per token and each grouped row of h
    and y once, at the width the launch stores them in: the large-tile
    kernels keep h and y as scaled fp16 (2 B), the streaming and small-tile
    kernels h as a bf16 pair (4 B) and y as fp32 (4 B).
    """
    T, D, I, E, k = cfg.T, cfg.D, cfg.I, cfg.E, cfg.k
    rows_b, n_b, rows_s, n_s = stats
    mat13, mat2 = matrix_bytes(cfg, path)
    hb = 2 if path == "tiled" else 4  # h bytes per element, big slot
    yb = 2 if path == "tiled" else 4  # y bytes per element, big slot
    if launch == "gate_up":
        return 4.0 * rows_b * I * D, n_b * 2 * mat13 + (T * D * 2 if rows_b else 0) + rows_b * I * hb
    if launch == "gate_up_stream":
        return 4.0 * rows_s * I * D, n_s * 2 * mat13 + min(T, rows_s) * D * 2 + rows_s * I * 4
    if launch == "down":
        return 2.0 * rows_b * D * I, n_b * mat2 + rows_b * I * hb + rows_b * D * yb
    if launch == "down_stream":
        return 2.0 * rows_s * D * I, n_s * mat2 + rows_s * I * 4 + rows_s * D * 4
    if launch == "combine":
        return 2.0 * (rows_b + rows_s) * D, rows_b * D * yb + rows_s * D * 4 + T * D * 4 + T * k * 8
    if launch == "route":
        return 0.0, T * E * 4 + E * 4 + T * k * 8
    return 0.0, T * k * 4 * 3 + T * D * 4  # group: ids in, maps out, x in and re-laid out


def matrix_bytes(cfg, path: str):
    """Bytes of one w1 (or w3) and of one w2 matrix: 17 per 32 MXFP4 weights,
    144 per 256 Q4_K weights."""
    if path == "q4k":
        return cfg.I * (cfg.D // 256) * 144, cfg.D * (cfg.I // 256) * 144
    return cfg.I * (cfg.D // 32) * 17, cfg.D * (cfg.I // 32) * 17


def arithmetic(path: str):
    """(dtype, description) of what the path computes in."""
    if path == "q4k":
        return ("bf16", "Q4_K codes exact in bf16 (as 128 + code); bf16 MFMA with fp32 accumulation, block scales "
                "and mins applied in fp32 (the min terms as fp32 MFMAs); h as a bf16 hi+lo pair; fp32 expert "
                "outputs and combine; fp64 routing scores")
    if path == "tiled":
        return ("bf16+fp16", "MXFP4 weights decoded exactly to bf16 (gate/up) and fp16 (down); bf16 MFMA gate/up, "
                "fp16 MFMA down on h scaled per (row, 256 features); experts with <= 16 rows: bf16 MFMA with h "
                "as a bf16 hi+lo pair; fp32 accumulation; large-tile expert outputs held as scaled fp16; "
                "fp32 combine; fp64 routing scores")
    return ("bf16", "MXFP4 weights decoded exactly to bf16; bf16 MFMA with fp32 accumulation, h as a bf16 hi+lo "
            "pair; fp32 expert outputs and combine; fp64 routing scores")


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


def measure(name, cfg, dev, k3, steps, warmup, rotate, eager, cold_steps=0, serial=False, q4k=False):
    """Time one workload on the resident experts; returns its result fields.
    q4k: the experts in `dev` are Q4_K blocks and the FFN is moe_q4k_ffn."""
    import numpy as np
    import torch

    from moe_inputs.device import upload_batch

    path = "q4k" if q4k else gemm_path(cfg)
    ffn = k3.moe_q4k_ffn if q4k else k3.moe_mxfp4_ffn
    ws_size = k3.moe_q4k_ffn_workspace_size if q4k else k3.moe_mxfp4_ffn_workspace_size
    batches = [upload_batch(cfg, seed=s) for s in range(rotate)]
    ws = torch.empty(max(1, ws_size(cfg.T, cfg.D, cfg.I, cfg.E, cfg.k)), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.T, cfg.D), dtype=torch.float32, device="cuda")
    ids = [torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda") for _ in range(rotate)]
    wts = [torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda") for _ in range(rotate)]
    # realized routing of each batch (for the work accounting)
    stats, n_active = [], []
    for i, (_, x, z, b) in enumerate(batches):
        k3.moe_route_topk(z, b, cfg.k, ids=ids[i], weights=wts[i])
        counts = torch.bincount(ids[i].reshape(-1).long(), minlength=cfg.E).cpu().numpy()
        stats.append(routing_stats(counts, path))
        n_active.append(int((counts > 0).sum()))
    torch.cuda.synchronize()

    # serial: every FFN launch on the caller's stream (moe_mxfp4_ffn_profiled
    # with no events), as in the timed-launch pass below
    no_events = [None] * k3.FFN_STAGE_EVENTS if serial else None

    def step(i, events=None):
        j = i % rotate
        _, x, z, b = batches[j]
        if events is not None and events[0] is not None:
            events[0].record()
        k3.moe_route_topk(z, b, cfg.k, ids=ids[j], weights=wts[j])
        ffn(x, ids[j], wts[j], dev.w1, dev.w3, dev.w2, out=out, workspace=ws,
            stage_events=no_events if events is None else events[1:])

    def busy_head():
        # keep the GPU busy while the host enqueues the measured steps, so no
        # step waits for the host (matters for decode-sized steps)
        torch.cuda._sleep(int(2e7))

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # 1. launch split (eager, every launch boundary marked) -> longest launch
    n_ev_slots = len(LAUNCHES) + 1
    n_split = max(rotate, min(steps, 16) if steps > 0 else 16)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev_slots)] for _ in range(n_split)]
    busy_head()
    for i in range(n_split):
        step(warmup + i, ev[i])
    torch.cuda.synchronize()
    launch_ms = {s: float(np.mean([ev[i][n].elapsed_time(ev[i][n + 1]) for i in range(n_split)]))
                 for n, s in enumerate(LAUNCHES)}

    if steps <= 0:
        # long enough that clock ramp-up and the first replays do not show
        est_s = sum(launch_ms.values()) * 1e-3
        steps = int(min(5000, max(20, round(0.5 / max(est_s, 1e-6)))))

    # 2. the timed steps: one captured graph per rotated batch, replayed
    graphs = []
    if not eager:
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

    # 2b. cold steps: before each one a read of a 1 GiB buffer evicts the
    #     experts from the 256 MiB Infinity Cache and the L2s; each replay is
    #     timed alone by two events, and the median is reported
    cold_ms = []
    if graphs and cold_steps > 0:
        flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")  # 1 GiB
        sink = torch.empty((), dtype=torch.int64, device="cuda")
        ce = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(cold_steps)]
        for i in range(cold_steps):
            torch.sum(flush, dim=0, dtype=torch.int64, out=sink)
            ce[i][0].record()
            graphs[(warmup + i) % rotate].replay()
            ce[i][1].record()
        torch.cuda.synchronize()
        cold_ms = [a.elapsed_time(b) for a, b in ce]
        del flush

    # 3. eager steps with the longest launch bracketed by two events on the
    #    library's stream (its per-launch duration for the roofline), and the
    #    eager step time from two events around all of them
    have = [s for s in LAUNCHES if kernel_info(s, path, cfg.T * cfg.k, cfg.T) is not None]
    # the roofline is that of the longest grouped-GEMM launch (at decode sizes
    # the event pairs around the tiny route / group / combine launches
    # measure mostly their own overhead)
    dom = max([s for s in have if s in GEMM_LAUNCHES], key=lambda s: launch_ms[s])
    n = LAUNCHES.index(dom)
    #    Each step also records two events back to back on the same stream
    #    (nothing between them): their mean interval is the fixed cost an
    #    event pair adds around a launch, which the per-launch duration has
    #    subtracted (the raw interval is reported beside it).
    n_ev = min(steps, 200)
    dev_ev = [[torch.cuda.Event(enable_timing=True) if m in (n, n + 1) else None for m in range(n_ev_slots)]
              for _ in range(n_ev)]
    pair = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    busy_head()
    e_start.record()
    for i in range(n_ev):
        step(warmup + i, dev_ev[i])
        pair[i][0].record()
        pair[i][1].record()
    e_end.record()
    torch.cuda.synchronize()
    dom_raw_ms = float(np.mean([dev_ev[i][n].elapsed_time(dev_ev[i][n + 1]) for i in range(n_ev)]))
    pair_ms = float(np.mean([a.elapsed_time(b) for a, b in pair]))
    dom_ms = dom_raw_ms - pair_ms
    eager_ms = e_start.elapsed_time(e_end) / n_ev

    work = [launch_work(dom, cfg, path, stats[(warmup + i) % rotate]) for i in range(n_ev)]
    flops = float(np.mean([w[0] for w in work]))
    byts = float(np.mean([w[1] for w in work]))
    bound = "mfma" if flops / max(byts, 1.0) > RIDGE else "hbm"
    dur_s = dom_ms * 1e-3
    if bound == "mfma":
        achieved, peak, unit = flops / dur_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = byts / dur_s / 1e9, PEAK_HBM_GBS, "GB/s"
    kname, ksrc = kernel_info(dom, path, cfg.T * cfg.k, cfg.T)
    traffic = stored_traffic(dom, name, ksrc)

    act_steps = [n_active[(warmup + i) % rotate] for i in range(steps)]
    m13, m2 = matrix_bytes(cfg, path)
    expert_bytes = 2 * m13 + m2
    weight_bytes = float(np.mean(act_steps)) * expert_bytes
    step_s = elapsed / steps
    dtype, arith = arithmetic(path)
    res = {
        "value": cfg.T * steps / elapsed,
        "steps": steps,
        "ms_per_step": step_s * 1e3,
        "dtype": dtype,
        "arithmetic": arith,
        "config": {
            "workload": name,
            "tokens": cfg.T,
            "experts": cfg.E,
            "top_k": cfg.k,
            "latent_dim": cfg.D,
            "expert_intermediate": cfg.I,
            "weights": ("Q4_K (ggml block_q4_K): 144-byte blocks of 256 weights" if q4k
                        else "MXFP4 E2M1 + E8M0 in 17-byte blocks"),
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
            "avg_launch_ms_raw_events": dom_raw_ms,
            "event_pair_overhead_ms": pair_ms,
            "launches_timed": n_ev,
        },
        "timing": ("graph replay of the step (route + FFN), one captured graph per rotated batch"
                   if graphs else "eager launches") + (", every FFN launch on one stream" if serial else ""),
        "eager_ms_per_step": eager_ms,
        "step_weight_GBps": weight_bytes / step_s / 1e9,
        "step_hbm_frac": weight_bytes / step_s / (PEAK_HBM_GBS * 1e9),
        "step_mfma_frac": cfg.T * 2 * cfg.k * 3 * cfg.D * cfg.I / step_s / (PEAK_BF16_TFLOPS * 1e12),
        "launches_ms": {s: v for s, v in launch_ms.items() if s in have},
        "_batch0": batches[0][0],
    }
    if cold_ms:
        med = float(np.median(cold_ms))
        cold_act = float(np.mean([n_active[(warmup + i) % rotate] for i in range(len(cold_ms))]))
        res["cold"] = {
            "protocol": "1 GiB read between steps (caches evicted), each step timed alone by HIP events",
            "steps": len(cold_ms),
            "median_ms_per_step": med,
            "tokens_per_s": cfg.T / (med * 1e-3),
            "step_weight_GBps": cold_act * expert_bytes / (med * 1e-3) / 1e9,
            "step_hbm_frac": cold_act * expert_bytes / (med * 1e-3) / (PEAK_HBM_GBS * 1e9),
            "step_mfma_frac": cfg.T * 2 * cfg.k * 3 * cfg.D * cfg.I / (med * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        }
    return res


def q4k_device_experts(cfg, seed: int = 0):
    """All E experts as Q4_K blocks drawn on the device (the recipe of
    moe_inputs.q4k_blocks: uniform code and scale bytes, positive fp16 d and
    dmin with exponent fields 1..3 and uniform mantissas) from a seeded torch
    generator: 16.6 GB at K3 shape, which host generation would take a minute
    to write.  Timing only; the parity tests draw their Q4_K experts on the host."""
    import torch

    from moe_inputs.device import DeviceExperts

    g = torch.Generator(device="cuda")
    g.manual_seed(1000 + seed)

    def mat(rows, cols):
        nb = cols // 256
        b = torch.randint(0, 256, (cfg.E, rows, nb, 144), generator=g, dtype=torch.uint8, device="cuda")
        for off in (0, 2):
            e = torch.randint(1, 4, (cfg.E, rows, nb), generator=g, dtype=torch.int32, device="cuda")
            m = torch.randint(0, 1024, (cfg.E, rows, nb), generator=g, dtype=torch.int32, device="cuda")
            bits = (e << 10) | m
            b[..., off] = (bits & 0xFF).to(torch.uint8)
            b[..., off + 1] = (bits >> 8).to(torch.uint8)
        return b

    return DeviceExperts(mat(cfg.I, cfg.D), mat(cfg.I, cfg.D), mat(cfg.D, cfg.I))


def measure_verify_width(dev, k3, warmup, reps=100):
    """The verify cost hint on the verify workload's seed-0 batch: distinct
    experts by verify width (moe_verify_width_distinct), the FFN step time
    of every truncated width (positions < w of each of the 16 sequences,
    graph replay), a least-squares fit time = fixed + distinct * expert_bytes
    / bytes_per_s, and the width moe_verify_width_choose picks at an
    acceptance of 0.8 per proposal (the pages report 4 of 5 verified rows
    accepted) for experts in HBM and for experts streamed over the host link."""
    import numpy as np
    import torch

    import moe_inputs
    from moe_inputs.device import upload_batch

    cfg = moe_inputs.VERIFY
    S, W = 16, 8
    _, x, z, b = upload_batch(cfg, seed=0)
    ids, wts = k3.moe_route_topk(z, b, cfg.k)
    distinct = k3.moe_verify_width_distinct(ids, S, W, cfg.E)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        k3.moe_verify_width_distinct(ids, S, W, cfg.E, out=distinct)
    ev1.record()
    torch.cuda.synchronize()
    kernel_ms = ev0.elapsed_time(ev1) / reps
    d = distinct.cpu().numpy().astype(np.int64)
    expert_bytes = 2 * cfg.I * (cfg.D // 32) * 17 + cfg.D * (cfg.I // 32) * 17
    ffn_ms = []
    for w in range(1, W + 1):
        rows = torch.tensor([s_ * W + p for s_ in range(S) for p in range(w)], dtype=torch.long, device="cuda")
        xw, iw, ww = x[rows].contiguous(), ids[rows].contiguous(), wts[rows].contiguous()
        T = S * w
        out = torch.empty((T, cfg.D), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(1, k3.moe_mxfp4_ffn_workspace_size(T, cfg.D, cfg.I, cfg.E, cfg.k)), dtype=torch.uint8,
                         device="cuda")
        for _ in range(warmup):
            k3.moe_mxfp4_ffn(xw, iw, ww, dev.w1, dev.w3, dev.w2, out=out, workspace=ws)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            k3.moe_mxfp4_ffn(xw, iw, ww, dev.w1, dev.w3, dev.w2, out=out, workspace=ws)
        g.replay()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(reps):
            g.replay()
        ev1.record()
        torch.cuda.synchronize()
        ffn_ms.append(ev0.elapsed_time(ev1) / reps)
    A = np.stack([np.ones(W), d.astype(np.float64)], axis=1)
    (fixed_ms, ms_per_expert), *_ = np.linalg.lstsq(A, np.array(ffn_ms), rcond=None)
    if fixed_ms < 0:  # no fixed part: a line through the origin
        fixed_ms = 0.0
        ms_per_expert = float(np.dot(d, ffn_ms) / np.dot(d, d))
    model_ms = (A @ np.array([fixed_ms, ms_per_expert])).tolist()
    bytes_per_s = expert_bytes / (ms_per_expert * 1e-3)
    accept = [0.8] * (W - 1)
    best_hbm, rates_hbm = k3.moe_verify_width_choose(d.tolist(), S, accept, expert_bytes, bytes_per_s, fixed_ms * 1e-3)
    host_link = 64e9  # PCIe 5.0 x16, one direction
    best_host, rates_host = k3.moe_verify_width_choose(d.tolist(), S, accept, expert_bytes, host_link, fixed_ms * 1e-3)
    return {
        "sequences": S,
        "width": W,
        "distinct_experts_by_width": d.tolist(),
        "distinct_kernel_ms": kernel_ms,
        "ffn_ms_by_width": ffn_ms,
        "fit": {"fixed_ms": float(fixed_ms), "bytes_per_s": float(bytes_per_s), "model_ms_by_width": model_ms,
                "max_rel_error": float(np.max(np.abs(np.array(model_ms) - np.array(ffn_ms)) / np.array(ffn_ms)))},
        "accept_per_proposal": 0.8,
        "best_width_hbm": best_hbm,
        "committed_tokens_per_s_hbm": rates_hbm,
        "best_width_host_link_64GBps": best_host,
        "committed_tokens_per_s_host_link": rates_host,
    }


BLOCK_SIZES = (("decode-t1", "block-decode-t1", 1), ("decode-t8", "block-decode-t8", 8),
               ("t128", "block-prefill", 128), ("prefill", "block-prefill", 4096))


def block_dense_work(launch, T, E, D, Is, H):
    """Algorithmic (flops, bytes) of one dense product launch of the block:
    weights once, inputs once, fp32 outputs once."""
    if launch == "dense1":
        n = E + D + 2 * Is
        return 2.0 * T * n * H, 2.0 * n * H + 2.0 * T * H + 4.0 * T * n
    n = D + Is
    return 2.0 * T * H * n, 2.0 * H * n + 2.0 * T * n + 4.0 * T * H


def measure_block(label, cfg, dense, dev, k3, warmup, rotate=4, steps=0):
    """The latent-MoE block (moe_latent_block) at cfg's size on resident
    weights: graph-replayed steps over `rotate` seeded hidden batches, a
    stage split from the profiled entry point's events, and the roofline of
    both dense products (event pairs right around each launch, minus the mean
    interval of an empty event pair)."""
    import numpy as np
    import torch

    import moe_inputs

    L = cfg.layer
    T, H, D, I, Is, E, k = L.T, cfg.H, L.D, L.I, cfg.Is, L.E, L.k
    hs = [torch.from_numpy(moe_inputs.block_hidden(cfg, seed=s).view(np.int16)).view(torch.bfloat16).cuda()
          for s in range(rotate)]
    bias = torch.from_numpy(moe_inputs.block_bias(cfg)).cuda()
    ws = torch.empty(k3.moe_latent_block_workspace_size(T, H, D, I, Is, E, k), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    d = dense

    def step(i, events=None):
        k3.moe_latent_block(hs[i % rotate], d["Wg"], bias, d["Wd"], d["gamma"], dev.w1, dev.w3, dev.w2, d["Wu"],
                            d["Ws1"], d["Ws3"], d["Ws2"], k, eps=cfg.eps, out=out, workspace=ws, stage_events=events)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    n_ev = 50
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(k3.BLOCK_STAGE_EVENTS)] for _ in range(n_ev)]
    pair = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    torch.cuda._sleep(int(2e7))
    for i in range(n_ev):
        step(i, evs[i])
        pair[i][0].record()
        pair[i][1].record()
    torch.cuda.synchronize()
    stage = {s: float(np.mean([evs[i][n].elapsed_time(evs[i][n + 1]) for i in range(n_ev)]))
             for n, s in enumerate(k3.BLOCK_STAGES)}
    pair_ms = float(np.mean([a.elapsed_time(b) for a, b in pair]))
    if steps <= 0:
        steps = int(min(5000, max(20, round(0.5 / max(sum(stage.values()) * 1e-3, 1e-6)))))
    graphs = []
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
        graphs[i % rotate].replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kname = "dense_stream_kernel" if T <= 64 else "dense_tile_kernel"
    roof = {}
    for launch in ("dense1", "dense2"):
        kname_l = f"{kname}<{launch[-1]}>"
        flops, byts = block_dense_work(launch, T, E, D, Is, H)
        ms = stage[launch] - pair_ms
        bound = "mfma" if flops / byts > RIDGE else "hbm"
        if bound == "mfma":
            ach, peak, unit = flops / (ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
        else:
            ach, peak, unit = byts / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
        roof[launch] = {"kernel": kname_l, "bound": bound, "achieved": ach, "peak": peak, "unit": unit,
                        "frac": ach / peak, "algorithmic_flops_per_launch": flops,
                        "algorithmic_bytes_per_launch": byts, "avg_launch_ms": ms,
                        "avg_launch_ms_raw_events": stage[launch], "event_pair_overhead_ms": pair_ms}
    step_s = elapsed / steps
    dense_bytes = 2.0 * H * (E + D + 2 * Is) + 2.0 * H * (D + Is)
    return {
        "workload": label,
        "tokens": T,
        "shape": {"hidden": H, "latent": D, "expert_intermediate": I, "shared_intermediate": Is, "experts": E,
                  "top_k": k},
        "steps": steps,
        "ms_per_step": step_s * 1e3,
        "tokens_per_s": T / step_s,
        "timing": "graph replay of moe_latent_block, one captured graph per rotated hidden batch",
        "stages_ms": stage,
        "dense_weight_bytes": dense_bytes,
        "step_dense_GBps": dense_bytes / step_s / 1e9,
        "roofline": roof,
    }


def measure_blocks(dev, k3, warmup, only=None):
    """Every block size (or only the one named) on one set of dense weights."""
    import numpy as np
    import torch

    import moe_inputs

    base = moe_inputs.BLOCK_DECODE8
    host = moe_inputs.block_dense_weights(base)
    dense = {n: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda() for n, v in host.items()}
    res = {}
    for label, name, T in BLOCK_SIZES:
        if only is not None and label != only:
            continue
        cfg = moe_inputs.BLOCK_CONFIGS[name]
        cfg = cfg.with_(layer=cfg.layer.with_(T=T))
        res[label] = measure_block(label, cfg, dense, dev, k3, warmup, rotate=8 if T <= 8 else 4)
    return res


HOST_LINK_PEAK_GBS = 63.0  # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes x 128/130 / 8


def measure_expert_cache(dev, k3, warmup, steps=40, cache_gib=8.0):
    """Decode batches of 8 tokens with the experts in an external store behind
    a device expert cache of cache_gib GiB (the lucebox runtime's 8 GiB): each
    step routes the batch, stages its missing experts into the cache
    (moe_expert_cache_route: plan + fetch, GPU loads from the store) and runs
    the FFN on the cache's slots.  The store is pinned host memory (the fetch
    crosses the host link) or the resident HBM copy (an HBM-to-HBM copy).
    Consecutive steps draw fresh seeded batches; the first `warmup + 24`
    steps fill the cache and are not timed."""
    import numpy as np
    import torch

    import moe_inputs
    from moe_inputs.device import upload_batch

    base = moe_inputs.DECODE8
    E = base.E
    expert_bytes = 2 * base.I * (base.D // 32) * 17 + base.D * (base.I // 32) * 17
    C = int(cache_gib * (1 << 30) // expert_bytes)
    cache = (torch.empty((C, base.I, base.D // 32, 17), dtype=torch.uint8, device="cuda"),
             torch.empty((C, base.I, base.D // 32, 17), dtype=torch.uint8, device="cuda"),
             torch.empty((C, base.D, base.I // 32, 17), dtype=torch.uint8, device="cuda"))
    t0 = time.perf_counter()
    host = []
    for t in (dev.w1, dev.w3, dev.w2):
        h = torch.empty(t.shape, dtype=torch.uint8, pin_memory=True)
        h.copy_(t)
        host.append(h)
    pin_s = time.perf_counter() - t0
    fill = warmup + 24
    out = {"slots": C, "cache_GiB": C * expert_bytes / (1 << 30), "expert_bytes": expert_bytes,
           "host_link_peak_GBps": HOST_LINK_PEAK_GBS, "pin_store_s": pin_s}
    cases = (("uniform", base, host, "pinned host"), ("zipf", base.with_(logits="zipf"), host, "pinned host"),
             ("uniform-hbm-store", base, [dev.w1, dev.w3, dev.w2], "HBM"))
    for name, cfg, store, where in cases:
        batches = [upload_batch(cfg, seed=5000 + i) for i in range(fill + steps)]
        state = k3.moe_expert_cache_init(E, C)
        slot_ids = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
        y = torch.empty((cfg.T, cfg.D), dtype=torch.float32, device="cuda")
        ws = torch.empty(k3.moe_mxfp4_ffn_workspace_size(cfg.T, cfg.D, cfg.I, C, cfg.k), dtype=torch.uint8,
                         device="cuda")
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        misses, hits = [], []
        for i, (_, x, z, b) in enumerate(batches):
            e = evs[i - fill] if i >= fill else None
            if e:
                e[0].record()
            ids, w = k3.moe_route_topk(z, b, cfg.k)
            if e:
                e[1].record()
            k3.moe_expert_cache_route(state, E, C, ids, *store, *cache, slot_ids=slot_ids)
            if e:
                e[2].record()
            k3.moe_mxfp4_ffn(x, slot_ids, w, *cache, out=y, workspace=ws)
            if e:
                e[3].record()
                torch.cuda.synchronize()
                hdr = k3.moe_expert_cache_header(state)
                misses.append(hdr["misses"])
                hits.append(hdr["hits"])
        torch.cuda.synchronize()
        step_ms = np.array([e[0].elapsed_time(e[3]) for e in evs])
        stage_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
        ffn_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
        moved = float(np.sum(misses)) * expert_bytes
        r = {"store": where, "steps": steps, "ms_per_step": float(step_ms.mean()),
             "tokens_per_s": cfg.T * steps / (step_ms.sum() * 1e-3),
             "hit_rate": float(np.sum(hits) / max(1, np.sum(hits) + np.sum(misses))),
             "distinct_experts_per_step": float(np.mean(np.add(hits, misses))),
             "misses_per_step": float(np.mean(misses)), "stage_ms_per_step": float(stage_ms.mean()),
             "ffn_ms_per_step": float(ffn_ms.mean()),
             "staged_GBps": moved / (stage_ms.sum() * 1e-3) / 1e9}
        if where == "HBM":
            # read and write once per staged byte
            r["hbm_GBps"] = 2 * r["staged_GBps"]
            r["frac_of_hbm_peak"] = r["hbm_GBps"] / PEAK_HBM_GBS
        else:
            r["frac_of_host_link_peak"] = r["staged_GBps"] / HOST_LINK_PEAK_GBS
        out[name] = r
    return out


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for {max(args.gpus, world)}): this layer is built and "
              "measured on one MI355X; sharding is a design note only.", file=sys.stderr)
        sys.exit(2)

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
    from moe_inputs.device import upload_experts

    torch.cuda.set_device(0)
    if args.block is not None:
        dev = upload_experts(moe_inputs.PREFILL, lambda p, s, out: k3.mxfp4_tile(k3.mxfp4_repack(p, s), out=out))
        r = measure_blocks(dev, k3, args.warmup, only=args.block)[args.block]
        print(json.dumps({"metric": "latent-MoE block tokens/s at K3 shape", "value": r["tokens_per_s"],
                          "unit": "tokens/s", "n_gpus": 1, "higher_is_better": True, "data": "synthetic",
                          "latent_block": r}), flush=True)
        return
    head_q4k = args.workload.startswith(Q4K_PREFIX)
    cfg = moe_inputs.CONFIGS[args.workload[len(Q4K_PREFIX):] if head_q4k else args.workload]
    t_setup = time.perf_counter()
    if head_q4k:
        dev = q4k_device_experts(cfg)
    else:
        dev = upload_experts(cfg, lambda p, s, out: k3.mxfp4_tile(k3.mxfp4_repack(p, s), out=out))
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    def rot(c):
        return args.rotate or (8 if c.T <= 8 else 4)

    head = measure(args.workload, cfg, dev, k3, args.steps, args.warmup, rot(cfg), args.eager, args.cold_steps,
                   args.serial_launches, q4k=head_q4k)
    batch0 = head.pop("_batch0")
    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": head["steps"],
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": ("synthetic (seeded Q4_K weights for all experts drawn on the device, bf16 N(0,1) activations, "
                 "seeded router logits)" if head_q4k else
                 "synthetic (seeded MXFP4 weights for all experts, bf16 N(0,1) activations, seeded router logits)"),
    }
    result.update({k: v for k, v in head.items() if k not in ("value", "steps", "ms_per_step", "dtype")})
    result["setup_s"] = setup_s
    if args.extra and args.workload == "prefill":
        extra = {}
        for w in EXTRA_WORKLOADS:
            c = moe_inputs.CONFIGS[w]
            r = measure(w, c, dev, k3, 0, args.warmup, rot(c), args.eager, args.cold_steps, args.serial_launches)
            r.pop("_batch0")
            r["tokens_per_s"] = r.pop("value")
            extra[w] = r
        result["workloads"] = extra
        result["verify_width"] = measure_verify_width(dev, k3, args.warmup)
        result["expert_cache"] = measure_expert_cache(dev, k3, args.warmup)
        result["latent_block"] = measure_blocks(dev, k3, args.warmup)
        del dev
        torch.cuda.empty_cache()
        dq = q4k_device_experts(cfg)
        for w in Q4K_WORKLOADS:
            c = moe_inputs.CONFIGS[w[len(Q4K_PREFIX):]]
            r = measure(w, c, dq, k3, 0, args.warmup, rot(c), args.eager, args.cold_steps, args.serial_launches,
                        q4k=True)
            r.pop("_batch0")
            r["tokens_per_s"] = r.pop("value")
            extra[w] = r
        del dq
    if args.cpu_baseline and not head_q4k:
        sample = args.cpu_sample_tokens or (cfg.T if cfg.T <= 64 else 12)  # about 12 s of oracle work at K3 shape
        result["cpu_baseline"] = cpu_baseline(cfg, batch0, sample)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
