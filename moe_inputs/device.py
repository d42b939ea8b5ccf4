"""Upload a workload's synthetic inputs to the GPU.

Data movement only: the caller passes the function that turns source-layout
MXFP4 matrices into device blocks (the library's ``mxfp4_repack`` followed by
``mxfp4_tile``), so this module itself performs none of the method's
arithmetic.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import T_W1, T_W2, T_W3, ExpertSource, LayerConfig, make_batch


@dataclass
class DeviceExperts:
    w1: torch.Tensor  # u8 [E, I, D/32, 17]
    w3: torch.Tensor  # u8 [E, I, D/32, 17]
    w2: torch.Tensor  # u8 [E, D, I/32, 17]


def upload_experts(cfg: LayerConfig, repack, device="cuda", progress=None) -> DeviceExperts:
    """Generate every expert's source-layout matrices and repack them on the device.

    ``repack(packed_dev, scale_dev, out=blocks_view)`` must write the 17-byte
    blocks of one matrix into ``blocks_view``, in the order the FFN reads.
    """
    E, D, I = cfg.E, cfg.D, cfg.I
    w1 = torch.empty((E, I, D // 32, 17), dtype=torch.uint8, device=device)
    w3 = torch.empty_like(w1)
    w2 = torch.empty((E, D, I // 32, 17), dtype=torch.uint8, device=device)
    src = ExpertSource(cfg)
    # two pinned staging slots so host generation overlaps the copies
    big = max(I * D // 2, D * I // 2)
    stage_p = [torch.empty(big, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
    stage_s = [torch.empty(big // 16, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
    dev_p = [torch.empty(big, dtype=torch.uint8, device=device) for _ in range(2)]
    dev_s = [torch.empty(big // 16, dtype=torch.uint8, device=device) for _ in range(2)]
    events = [None, None]
    slot = 0
    for e in range(E):
        for tid, dst in ((T_W1, w1), (T_W3, w3), (T_W2, w2)):
            packed, scale = src.matrix(tid, e)
            if events[slot] is not None:
                events[slot].synchronize()  # staging slot free again
            npk, nsc = packed.size, scale.size
            stage_p[slot][:npk].numpy()[:] = packed.reshape(-1)
            stage_s[slot][:nsc].numpy()[:] = scale.reshape(-1)
            dp = dev_p[slot][:npk]
            ds = dev_s[slot][:nsc]
            dp.copy_(stage_p[slot][:npk], non_blocking=True)
            ds.copy_(stage_s[slot][:nsc], non_blocking=True)
            repack(dp.view(packed.shape), ds.view(scale.shape), dst[e])
            ev = torch.cuda.Event()
            ev.record()
            events[slot] = ev
            slot ^= 1
        if progress is not None and (e + 1) % 128 == 0:
            progress(e + 1, E)
    torch.cuda.synchronize()
    return DeviceExperts(w1, w3, w2)


def upload_batch(cfg: LayerConfig, seed: int | None = None, device="cuda"):
    """Host batch plus its device copies (x as bf16, logits, bias)."""
    b = make_batch(cfg, seed)
    x = torch.from_numpy(b.x.view(np.int16)).view(torch.bfloat16).to(device)
    z = torch.from_numpy(b.z).to(device)
    bias = torch.from_numpy(b.b).to(device)
    return b, x, z, bias
