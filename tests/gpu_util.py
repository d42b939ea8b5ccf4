"""Helpers shared by the GPU parity tests (no arithmetic of the method here)."""

import numpy as np
import torch

# FFN parity bar: relative L2 error and max abs error vs the fp64 oracle.
FFN_REL_L2 = 2e-3
FFN_MAX_ABS_FRAC = 1e-2


def ffn_errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rel_l2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    max_abs = float(np.abs(got - ref).max()) if ref.size else 0.0
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    return rel_l2, max_abs, scale


def assert_ffn_close(got, ref, what=""):
    rel_l2, max_abs, scale = ffn_errors(got, ref)
    print(f"[ffn parity] {what}: rel_l2={rel_l2:.3e} max_abs={max_abs:.3e} max|ref|={scale:.3e}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert rel_l2 <= FFN_REL_L2, (what, rel_l2)
    assert max_abs <= FFN_MAX_ABS_FRAC * scale, (what, max_abs, scale)


def expert_blocks(k3):
    """Upload step of one expert matrix: source layout -> ggml blocks
    (mxfp4_repack) -> the stage-tiled order the FFN reads (mxfp4_tile)."""
    return lambda p, s, out: k3.mxfp4_tile(k3.mxfp4_repack(p, s), out=out)


def to_dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
