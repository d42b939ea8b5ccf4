"""Python binding of libk3moe (the routed-expert MXFP4 MoE layer for MI355X).

Argument marshalling only: every function checks dtypes, devices and
contiguity, allocates outputs with torch when the caller passes none, and calls
the C entry point of the same name (include/k3moe.h) on torch's current HIP
stream.  All arithmetic runs in the library's HIP kernels; there is no CPU or
PyTorch fallback, and importing the package fails loudly when the library has
not been built.
"""

from __future__ import annotations

import ctypes
import os
import struct

import torch

__all__ = [
    "K3MoeError",
    "LIB_PATH",
    "ACT_SILU_MUL",
    "moe_route_topk",
    "mxfp4_repack",
    "mxfp4_dequant",
    "mxfp4_tile",
    "moe_mxfp4_ffn_workspace_size",
    "moe_mxfp4_ffn",
    "moe_mxfp4_ffn_noalloc",
    "NOALLOC_SCRATCH_BYTES",
    "moe_q4k_ffn_workspace_size",
    "moe_q4k_ffn",
    "moe_verify_width_distinct",
    "moe_verify_width_choose",
    "moe_expert_cache_state_size",
    "moe_expert_cache_init",
    "moe_expert_cache_route",
    "moe_expert_cache_header",
    "moe_latent_block_workspace_size",
    "moe_latent_block",
    "BLOCK_STAGES",
    "moe_group_workspace_size",
    "moe_group_by_expert",
    "FFN_STAGES",
    "status_str",
    "lib",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libk3moe.so")
ACT_SILU_MUL = 0
DTYPE_F32, DTYPE_BF16 = 0, 1
MAX_TOPK = 64
MAX_EXPERTS_FFN = 8192

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m mxfp4_mixture_experts_moe_amd.build` "
        "(there is no fallback implementation)"
    )
lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
lib.k3moe_status_str.restype = ctypes.c_char_p
lib.k3moe_status_str.argtypes = [ctypes.c_int]
lib.moe_route_topk.restype = ctypes.c_int
lib.moe_route_topk.argtypes = [_vp, _vp, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _vp]
lib.mxfp4_repack.restype = ctypes.c_int
lib.mxfp4_repack.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp]
lib.mxfp4_dequant.restype = ctypes.c_int
lib.mxfp4_dequant.argtypes = [_vp, _i64, _i64, _i32, _vp, _vp]
lib.mxfp4_tile.restype = ctypes.c_int
lib.mxfp4_tile.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp]
lib.moe_mxfp4_ffn_workspace_size.restype = _sz
lib.moe_mxfp4_ffn_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _i32]
lib.moe_mxfp4_ffn.restype = ctypes.c_int
lib.moe_mxfp4_ffn.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _sz, _vp]
lib.moe_mxfp4_ffn_profiled.restype = ctypes.c_int
lib.moe_mxfp4_ffn_profiled.argtypes = lib.moe_mxfp4_ffn.argtypes + [ctypes.POINTER(ctypes.c_void_p)]
lib.moe_mxfp4_ffn_noalloc.restype = ctypes.c_int
lib.moe_q4k_ffn_workspace_size.restype = _sz
lib.moe_q4k_ffn_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _i32]
lib.moe_q4k_ffn.argtypes = lib.moe_mxfp4_ffn.argtypes
lib.moe_q4k_ffn_profiled.argtypes = lib.moe_mxfp4_ffn_profiled.argtypes
lib.moe_mxfp4_ffn_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp, _vp]
NOALLOC_SCRATCH_BYTES = 64 << 20
lib.moe_group_workspace_size.restype = _sz
lib.moe_group_workspace_size.argtypes = [_i64, _i32, _i32]
lib.moe_group_by_expert.restype = ctypes.c_int
lib.moe_group_by_expert.argtypes = [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
lib.moe_verify_width_distinct.restype = ctypes.c_int
lib.moe_verify_width_distinct.argtypes = [_vp, _i32, _i32, _i32, _i32, _vp, _vp]
lib.moe_verify_width_choose.restype = ctypes.c_int
lib.moe_verify_width_choose.argtypes = [ctypes.POINTER(ctypes.c_int32), _i32, _i32, ctypes.POINTER(ctypes.c_double),
                                        ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)]
lib.moe_expert_cache_state_size.restype = _sz
lib.moe_expert_cache_state_size.argtypes = [_i32, _i32]
lib.moe_expert_cache_init.restype = ctypes.c_int
lib.moe_expert_cache_init.argtypes = [_vp, _sz, _i32, _i32, _vp]
lib.moe_expert_cache_route.restype = ctypes.c_int
lib.moe_expert_cache_route.argtypes = [_vp, _sz, _i32, _i32, _vp, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _i32, _i32, _vp]
lib.moe_expert_cache_route_q4k.argtypes = lib.moe_expert_cache_route.argtypes
EXPERT_CACHE_TAG = 0x4B334543
lib.moe_latent_block_workspace_size.restype = _sz
lib.moe_latent_block_workspace_size.argtypes = [_i64, _i32, _i32, _i32, _i32, _i32, _i32]
_block_args = [_vp] * 12 + [_i64] + [_i32] * 6 + [_i32, _f32, _f32, _vp, _vp, _vp, _vp, _sz, _vp]
lib.moe_latent_block.restype = ctypes.c_int
lib.moe_latent_block.argtypes = _block_args
lib.moe_latent_block_profiled.restype = ctypes.c_int
lib.moe_latent_block_profiled.argtypes = _block_args + [ctypes.POINTER(ctypes.c_void_p)]
BLOCK_STAGE_EVENTS = 7
# launches between consecutive events of moe_latent_block_profiled
BLOCK_STAGES = ("dense1", "mid", "route", "ffn", "dense2", "sum")
FFN_STAGE_EVENTS = 7
# launches between consecutive events of moe_mxfp4_ffn_profiled
FFN_STAGES = ("group", "gate_up", "gate_up_stream", "down", "down_stream", "combine")


class K3MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_str(status)} (status {status})")
        self.status = status


def status_str(status: int) -> str:
    return lib.k3moe_status_str(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise K3MoeError(fn, status)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype | tuple) -> None:
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dts:
        raise TypeError(f"{name}: expected dtype {dts}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def moe_route_topk(logits: torch.Tensor, bias: torch.Tensor | None, k: int, normalize: bool = True,
                   route_scale: float = 1.0, ids: torch.Tensor | None = None, weights: torch.Tensor | None = None):
    """Sigmoid + bias top-k routing. logits f32 [T, E], bias f32 [E] or None.

    Returns (ids int32 [T, k], weights f32 [T, k]).
    """
    _dev(logits, "logits", torch.float32)
    T, E = logits.shape
    if bias is not None:
        _dev(bias, "bias", torch.float32)
        if bias.shape != (E,):
            raise ValueError("bias must be [E]")
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _dev(ids, "ids", torch.int32)
    _dev(weights, "weights", torch.float32)
    if ids.shape != (T, k) or weights.shape != (T, k):
        raise ValueError("ids / weights must be [T, k]")
    _check("moe_route_topk", lib.moe_route_topk(_ptr(logits), _ptr(bias), T, E, k, int(bool(normalize)),
                                                float(route_scale), _ptr(ids), _ptr(weights),
                                                _stream(logits.device)))
    return ids, weights


def mxfp4_repack(packed: torch.Tensor, scale: torch.Tensor, blocks: torch.Tensor | None = None) -> torch.Tensor:
    """compressed-tensors MXFP4 (packed u8 [..., R, K/2], scale u8 [..., R, K/32]) -> u8 [..., R, K/32, 17].

    Leading dimensions are flattened into rows (the layout is row-independent).
    """
    _dev(packed, "packed", torch.uint8)
    _dev(scale, "scale", torch.uint8)
    K = packed.shape[-1] * 2
    if scale.shape[:-1] != packed.shape[:-1] or scale.shape[-1] * 32 != K:
        raise ValueError("scale must be [..., R, K/32] for packed [..., R, K/2]")
    R = packed.numel() // (K // 2)
    if blocks is None:
        blocks = torch.empty((*packed.shape[:-1], K // 32, 17), dtype=torch.uint8, device=packed.device)
    _dev(blocks, "blocks", torch.uint8)
    if blocks.numel() != R * (K // 32) * 17:
        raise ValueError("blocks has the wrong size")
    _check("mxfp4_repack", lib.mxfp4_repack(_ptr(packed), _ptr(scale), R, K, _ptr(blocks), _stream(packed.device)))
    return blocks


def mxfp4_tile(blocks: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """ggml-row-order MXFP4 matrices u8 [..., N, K/32, 17] -> the same blocks in
    the stage-tiled order the FFN entry points read (same shape; leading
    dimensions are separate matrices)."""
    _dev(blocks, "blocks", torch.uint8)
    if blocks.dim() < 3 or blocks.shape[-1] != 17:
        raise ValueError("blocks must be [..., N, K/32, 17]")
    N, nb = blocks.shape[-3], blocks.shape[-2]
    nmat = blocks.numel() // (N * nb * 17) if N * nb else 0
    if out is None:
        out = torch.empty_like(blocks)
    _dev(out, "out", torch.uint8)
    if out.numel() != blocks.numel():
        raise ValueError("out has the wrong size")
    if blocks.numel() == 0:
        return out
    _check("mxfp4_tile", lib.mxfp4_tile(_ptr(blocks), nmat, N, nb * 32, _ptr(out), _stream(blocks.device)))
    return out


def mxfp4_dequant(blocks: torch.Tensor, out_dtype: torch.dtype = torch.float32,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """ggml MXFP4 blocks u8 [..., R, K/32, 17] -> [..., R, K] f32 or bf16."""
    _dev(blocks, "blocks", torch.uint8)
    if blocks.shape[-1] != 17:
        raise ValueError("blocks must end in a 17-byte dimension")
    nb = blocks.shape[-2]
    K = nb * 32
    R = blocks.numel() // (nb * 17)
    code = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}.get(out_dtype)
    if code is None:
        raise TypeError("out_dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty((*blocks.shape[:-2], K), dtype=out_dtype, device=blocks.device)
    _dev(out, "out", out_dtype)
    if out.numel() != R * K:
        raise ValueError("out has the wrong size")
    _check("mxfp4_dequant", lib.mxfp4_dequant(_ptr(blocks), R, K, code, _ptr(out), _stream(blocks.device)))
    return out


def moe_mxfp4_ffn_workspace_size(T: int, D: int, I: int, E: int, k: int) -> int:
    return int(lib.moe_mxfp4_ffn_workspace_size(T, D, I, E, k))


def _ffn_operands(x, ids, weights, w1, w3, w2, out):
    _dev(x, "x", torch.bfloat16)
    _dev(ids, "ids", torch.int32)
    _dev(weights, "weights", torch.float32)
    for n, t in (("w1", w1), ("w3", w3), ("w2", w2)):
        _dev(t, n, torch.uint8)
    T, D = x.shape
    k = ids.shape[1]
    E, I = w1.shape[0], w1.shape[1]
    if ids.shape != (T, k) or weights.shape != (T, k):
        raise ValueError("ids / weights must be [T, k]")
    if w1.shape != (E, I, D // 32, 17) or w3.shape != w1.shape or w2.shape != (E, D, I // 32, 17):
        raise ValueError("expert weights have inconsistent shapes")
    if out is None:
        out = torch.empty((T, D), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    return T, D, I, E, k, out


def _event_handles(stage_events):
    if len(stage_events) != FFN_STAGE_EVENTS:
        raise ValueError(f"stage_events must hold {FFN_STAGE_EVENTS} events")
    handles = (ctypes.c_void_p * FFN_STAGE_EVENTS)()
    for i, ev in enumerate(stage_events):
        if ev is not None and not ev.cuda_event:
            ev.record()  # torch creates its events lazily
        handles[i] = None if ev is None else ev.cuda_event
    return handles


def moe_mxfp4_ffn(x: torch.Tensor, ids: torch.Tensor, weights: torch.Tensor, w1: torch.Tensor, w3: torch.Tensor,
                  w2: torch.Tensor, act: int = ACT_SILU_MUL, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stage_events=None) -> torch.Tensor:
    """Routed-expert FFN. x bf16 [T, D]; ids int32 [T, k]; weights f32 [T, k];
    w1/w3 u8 [E, I, D/32, 17]; w2 u8 [E, D, I/32, 17]. Returns out f32 [T, D].

    stage_events: optional list of FFN_STAGE_EVENTS torch.cuda.Event recorded
    at the launch boundaries (moe_mxfp4_ffn_profiled)."""
    T, D, I, E, k, out = _ffn_operands(x, ids, weights, w1, w3, w2, out)
    need = moe_mxfp4_ffn_workspace_size(T, D, I, E, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace", torch.uint8)
    args = (_ptr(x), _ptr(ids), _ptr(weights), _ptr(w1), _ptr(w3), _ptr(w2), T, D, I, E, k, act, _ptr(out),
            _ptr(workspace), workspace.numel(), _stream(x.device))
    if stage_events is None:
        _check("moe_mxfp4_ffn", lib.moe_mxfp4_ffn(*args))
    else:
        _check("moe_mxfp4_ffn_profiled", lib.moe_mxfp4_ffn_profiled(*args, _event_handles(stage_events)))
    return out


def moe_q4k_ffn_workspace_size(T: int, D: int, I: int, E: int, k: int) -> int:
    return int(lib.moe_q4k_ffn_workspace_size(T, D, I, E, k))


def moe_q4k_ffn(x: torch.Tensor, ids: torch.Tensor, weights: torch.Tensor, w1: torch.Tensor, w3: torch.Tensor,
                w2: torch.Tensor, act: int = ACT_SILU_MUL, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stage_events=None) -> torch.Tensor:
    """Routed-expert FFN over Q4_K experts. x bf16 [T, D]; ids int32 [T, k];
    weights f32 [T, k]; w1/w3 u8 [E, I, D/256, 144]; w2 u8 [E, D, I/256, 144]
    (ggml block_q4_K, row-major). Returns out f32 [T, D].

    stage_events: optional list of FFN_STAGE_EVENTS torch.cuda.Event recorded
    at the launch boundaries (moe_q4k_ffn_profiled)."""
    _dev(x, "x", torch.bfloat16)
    _dev(ids, "ids", torch.int32)
    _dev(weights, "weights", torch.float32)
    for n, t in (("w1", w1), ("w3", w3), ("w2", w2)):
        _dev(t, n, torch.uint8)
    T, D = x.shape
    k = ids.shape[1]
    E, I = w1.shape[0], w1.shape[1]
    if ids.shape != (T, k) or weights.shape != (T, k):
        raise ValueError("ids / weights must be [T, k]")
    if w1.shape != (E, I, D // 256, 144) or w3.shape != w1.shape or w2.shape != (E, D, I // 256, 144):
        raise ValueError("Q4_K expert weights have inconsistent shapes")
    if out is None:
        out = torch.empty((T, D), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    need = moe_q4k_ffn_workspace_size(T, D, I, E, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace", torch.uint8)
    args = (_ptr(x), _ptr(ids), _ptr(weights), _ptr(w1), _ptr(w3), _ptr(w2), T, D, I, E, k, act, _ptr(out),
            _ptr(workspace), workspace.numel(), _stream(x.device))
    if stage_events is None:
        _check("moe_q4k_ffn", lib.moe_q4k_ffn(*args))
    else:
        _check("moe_q4k_ffn_profiled", lib.moe_q4k_ffn_profiled(*args, _event_handles(stage_events)))
    return out


def moe_mxfp4_ffn_noalloc(x: torch.Tensor, ids: torch.Tensor, weights: torch.Tensor, w1: torch.Tensor,
                          w3: torch.Tensor, w2: torch.Tensor, out: torch.Tensor, act: int = ACT_SILU_MUL) -> torch.Tensor:
    """moe_mxfp4_ffn in the library's fixed device scratch (no workspace, no
    allocation: `out` is required). Raises K3MoeError (status -7) when the
    sizes need more than NOALLOC_SCRATCH_BYTES of workspace."""
    T, D, I, E, k, out = _ffn_operands(x, ids, weights, w1, w3, w2, out)
    _check("moe_mxfp4_ffn_noalloc", lib.moe_mxfp4_ffn_noalloc(_ptr(x), _ptr(ids), _ptr(weights), _ptr(w1), _ptr(w3),
                                                              _ptr(w2), T, D, I, E, k, act, _ptr(out),
                                                              _stream(x.device)))
    return out


def moe_group_workspace_size(T: int, E: int, k: int) -> int:
    return int(lib.moe_group_workspace_size(T, E, k))


def moe_group_by_expert(ids: torch.Tensor, E: int, workspace: torch.Tensor | None = None):
    """Grouping of routed entries by expert. ids int32 [T, k].

    Returns (counts int32 [E], offsets int32 [E + 1], row_tok int32 [T * k],
    slot_row int32 [T * k]); row_tok is meaningful up to offsets[E] (its later
    entries are zero here)."""
    _dev(ids, "ids", torch.int32)
    T, k = ids.shape
    dev = ids.device
    counts = torch.zeros(E, dtype=torch.int32, device=dev)
    offsets = torch.zeros(E + 1, dtype=torch.int32, device=dev)
    row_tok = torch.zeros(T * k, dtype=torch.int32, device=dev)
    slot_row = torch.zeros(T * k, dtype=torch.int32, device=dev)
    need = moe_group_workspace_size(T, E, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8)
    _check("moe_group_by_expert", lib.moe_group_by_expert(_ptr(ids), T, E, k, _ptr(counts), _ptr(offsets),
                                                          _ptr(row_tok), _ptr(slot_row), _ptr(workspace),
                                                          workspace.numel(), _stream(dev)))
    return counts, offsets, row_tok, slot_row


def moe_verify_width_distinct(ids: torch.Tensor, S: int, W: int, E: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Distinct experts routed by positions <= w of S sequences of W rows.
    ids int32 [S * W, k] (row r = s * W + w). Returns int32 [W]."""
    _dev(ids, "ids", torch.int32)
    if ids.dim() != 2 or ids.shape[0] != S * W:
        raise ValueError("ids must be [S * W, k]")
    k = ids.shape[1]
    if out is None:
        out = torch.empty(W, dtype=torch.int32, device=ids.device)
    _dev(out, "out", torch.int32)
    if out.numel() != W:
        raise ValueError("out must hold W counts")
    _check("moe_verify_width_distinct", lib.moe_verify_width_distinct(_ptr(ids), S, W, E, k, _ptr(out),
                                                                      _stream(ids.device)))
    return out


def moe_verify_width_choose(distinct, S: int, accept=None, expert_bytes: float = 0.0, bytes_per_s: float = 1.0,
                            fixed_s: float = 0.0):
    """Host call: (best width, [W] expected committed tokens per second).
    distinct: W counts (any int sequence); accept: W - 1 probabilities or None."""
    W = len(distinct)
    d = (ctypes.c_int32 * W)(*[int(v) for v in distinct])
    a = None if accept is None else (ctypes.c_double * max(W - 1, 1))(*[float(v) for v in accept])
    best = ctypes.c_int32(0)
    rates = (ctypes.c_double * W)()
    _check("moe_verify_width_choose", lib.moe_verify_width_choose(d, W, S, a, float(expert_bytes), float(bytes_per_s),
                                                                  float(fixed_s), ctypes.byref(best), rates))
    return int(best.value), [float(r) for r in rates]


def moe_expert_cache_state_size(E: int, C: int) -> int:
    return int(lib.moe_expert_cache_state_size(E, C))


def moe_expert_cache_init(E: int, C: int, state: torch.Tensor | None = None,
                          device: torch.device | str = "cuda") -> torch.Tensor:
    """Empty cache state for E experts and C slots (u8 device tensor)."""
    need = moe_expert_cache_state_size(E, C)
    if state is None:
        state = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _dev(state, "state", torch.uint8)
    _check("moe_expert_cache_init", lib.moe_expert_cache_init(_ptr(state), state.numel(), E, C,
                                                              _stream(state.device)))
    return state


def _store(t: torch.Tensor, name: str) -> None:
    if t.dtype != torch.uint8:
        raise TypeError(f"{name}: expected uint8, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda" and not t.is_pinned():
        raise ValueError(f"{name}: must be a device tensor or pinned host memory")


def moe_expert_cache_route(state: torch.Tensor, E: int, C: int, ids: torch.Tensor, store_w1: torch.Tensor,
                           store_w3: torch.Tensor, store_w2: torch.Tensor, cache_w1: torch.Tensor,
                           cache_w3: torch.Tensor, cache_w2: torch.Tensor,
                           slot_ids: torch.Tensor | None = None, q4k: bool = False) -> torch.Tensor:
    """Stage a batch's routed experts into the C slots; returns slot_ids
    int32 [T, k] (the FFN then runs on cache_w* with slot_ids and E = C).
    store_w*: all E experts, device tensors or pinned host tensors; MXFP4
    blocks, or Q4_K blocks with q4k=True (moe_expert_cache_route_q4k)."""
    _dev(state, "state", torch.uint8)
    _dev(ids, "ids", torch.int32)
    for n, t in (("store_w1", store_w1), ("store_w3", store_w3), ("store_w2", store_w2)):
        _store(t, n)
    for n, t in (("cache_w1", cache_w1), ("cache_w3", cache_w3), ("cache_w2", cache_w2)):
        _dev(t, n, torch.uint8)
    T, k = ids.shape
    I, D = store_w1.shape[1], store_w2.shape[1]
    blk, nbytes = (256, 144) if q4k else (32, 17)
    if store_w1.shape != (E, I, D // blk, nbytes) or store_w3.shape != store_w1.shape or \
            store_w2.shape != (E, D, I // blk, nbytes):
        raise ValueError(f"store matrices must be [E, I, D/{blk}, {nbytes}] and [E, D, I/{blk}, {nbytes}]")
    if cache_w1.shape != (C, I, D // blk, nbytes) or cache_w3.shape != cache_w1.shape or \
            cache_w2.shape != (C, D, I // blk, nbytes):
        raise ValueError(f"cache matrices must be [C, I, D/{blk}, {nbytes}] and [C, D, I/{blk}, {nbytes}]")
    if slot_ids is None:
        slot_ids = torch.empty((T, k), dtype=torch.int32, device=ids.device)
    _dev(slot_ids, "slot_ids", torch.int32)
    if slot_ids.shape != (T, k):
        raise ValueError("slot_ids must be [T, k]")
    fn = "moe_expert_cache_route_q4k" if q4k else "moe_expert_cache_route"
    _check(fn, getattr(lib, fn)(
        _ptr(state), state.numel(), E, C, _ptr(ids), T, k, _ptr(slot_ids), _ptr(store_w1), _ptr(store_w3),
        _ptr(store_w2), _ptr(cache_w1), _ptr(cache_w3), _ptr(cache_w2), D, I, _stream(ids.device)))
    return slot_ids


def moe_expert_cache_header(state: torch.Tensor) -> dict:
    """The state's header fields, copied to the host (synchronizes)."""
    raw = state[:48].cpu().numpy().tobytes()
    step, n_fetch, hits, misses, hits_total, misses_total, E, C, tag, _ = struct.unpack("<4I2Q2i2I", raw)
    return {"step": step, "n_fetch": n_fetch, "hits": hits, "misses": misses, "hits_total": hits_total,
            "misses_total": misses_total, "E": E, "C": C, "tag": tag}


def moe_latent_block_workspace_size(T: int, H: int, D: int, I: int, Is: int, E: int, k: int) -> int:
    return int(lib.moe_latent_block_workspace_size(T, H, D, I, Is, E, k))


def moe_latent_block(h: torch.Tensor, wg: torch.Tensor, bias: torch.Tensor | None, wd: torch.Tensor,
                     gamma: torch.Tensor, w1: torch.Tensor, w3: torch.Tensor, w2: torch.Tensor, wu: torch.Tensor,
                     ws1: torch.Tensor, ws3: torch.Tensor, ws2: torch.Tensor, k: int, normalize: bool = True,
                     route_scale: float = 1.0, eps: float = 1e-6, out: torch.Tensor | None = None,
                     topk_ids: torch.Tensor | None = None, topk_w: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stage_events=None) -> torch.Tensor:
    """Latent-MoE block. h bf16 [T, H]; wg bf16 [E, H]; bias f32 [E] or None;
    wd bf16 [D, H]; gamma bf16 [D]; w1/w3 u8 [E, I, D/32, 17], w2 u8 [E, D,
    I/32, 17]; wu bf16 [H, D]; ws1/ws3 bf16 [Is, H]; ws2 bf16 [H, Is].
    Returns out f32 [T, H]; topk_ids / topk_w (int32 / f32 [T, k]) receive the
    routing when given.  stage_events: BLOCK_STAGE_EVENTS torch.cuda.Event
    (moe_latent_block_profiled)."""
    T, H = h.shape
    E, D, Is = wg.shape[0], wd.shape[0], ws1.shape[0]
    I = w1.shape[1]
    for n, t in (("h", h), ("wg", wg), ("wd", wd), ("gamma", gamma), ("wu", wu), ("ws1", ws1), ("ws3", ws3),
                 ("ws2", ws2)):
        _dev(t, n, torch.bfloat16)
    for n, t in (("w1", w1), ("w3", w3), ("w2", w2)):
        _dev(t, n, torch.uint8)
    shapes = {"wg": (wg, (E, H)), "wd": (wd, (D, H)), "gamma": (gamma, (D,)), "wu": (wu, (H, D)),
              "ws1": (ws1, (Is, H)), "ws3": (ws3, (Is, H)), "ws2": (ws2, (H, Is)),
              "w1": (w1, (E, I, D // 32, 17)), "w3": (w3, (E, I, D // 32, 17)), "w2": (w2, (E, D, I // 32, 17))}
    for n, (t, shp) in shapes.items():
        if tuple(t.shape) != shp:
            raise ValueError(f"{n}: expected shape {shp}, got {tuple(t.shape)}")
    if bias is not None:
        _dev(bias, "bias", torch.float32)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=h.device)
    _dev(out, "out", torch.float32)
    for n, t, dt in (("topk_ids", topk_ids, torch.int32), ("topk_w", topk_w, torch.float32)):
        if t is not None:
            _dev(t, n, dt)
            if tuple(t.shape) != (T, k):
                raise ValueError(f"{n} must be [T, k]")
    need = moe_latent_block_workspace_size(T, H, D, I, Is, E, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=h.device)
    _dev(workspace, "workspace", torch.uint8)
    args = (_ptr(h), _ptr(wg), _ptr(bias), _ptr(wd), _ptr(gamma), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(wu), _ptr(ws1),
            _ptr(ws3), _ptr(ws2), T, H, D, I, Is, E, k, int(bool(normalize)), float(route_scale), float(eps),
            _ptr(out), _ptr(topk_ids), _ptr(topk_w), _ptr(workspace), workspace.numel(), _stream(h.device))
    if stage_events is None:
        _check("moe_latent_block", lib.moe_latent_block(*args))
    else:
        if len(stage_events) != BLOCK_STAGE_EVENTS:
            raise ValueError(f"stage_events must hold {BLOCK_STAGE_EVENTS} events")
        handles = (ctypes.c_void_p * BLOCK_STAGE_EVENTS)()
        for i, ev in enumerate(stage_events):
            if ev is not None and not ev.cuda_event:
                ev.record()
            handles[i] = None if ev is None else ev.cuda_event
        _check("moe_latent_block_profiled", lib.moe_latent_block_profiled(*args, handles))
    return out
