"""Seeded synthetic inputs for the routed-expert MXFP4 MoE layer.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no decoding, routing or matrix products).  Both the fp64
CPU oracle and the GPU library consume what it produces, so neither side ever
takes an input from the other.

Every tensor comes from its own keyed PCG64 stream: activations and router
inputs from ``numpy.random.default_rng([seed, config_id, tensor_id])``, expert
matrices from ``default_rng([seed, 100 + weight_id, tensor_id, expert])`` (all
K3-shaped workloads share one weight set), so any single expert matrix can be
regenerated alone (the FFN oracle only needs the experts a batch actually
routes to).

Workload shapes follow the Kimi-K3 routed experts described on the llama.cpp
pull-request page "model: add Kimi-K3 text model": 896 experts, 16 used,
sigmoid gating with an ``exp_probs_b`` bias (comment "Dry run: prepare_tensors()
completes"), and expert w1 of logical shape [3072, 3584] (comment
"repack_mxfp4_blocks is bit-exact"); the verify width 8 (current token plus 7
proposals) comes from the lucebox page "feat(kimi-k3): add DSpark Q8 artifact
and shared speculative runtime", comment "DSpark acceptance-contract correction".
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# tensor ids used as keys of the per-tensor streams
T_W1, T_W3, T_W2, T_X, T_LOGITS, T_BIAS, T_PERM, T_SINGLE = 1, 2, 3, 4, 5, 6, 7, 8
# latent-MoE block: hidden rows and the dense weights around the experts
T_H, T_WG, T_WD, T_GAMMA, T_WU, T_WS1, T_WS3, T_WS2 = 9, 10, 11, 12, 13, 14, 15, 16


def rng(seed: int, *key: int) -> np.random.Generator:
    """PCG64 stream keyed by (seed, *key)."""
    return np.random.default_rng([int(seed), *[int(k) for k in key]])


def mxfp4_source(g: np.random.Generator, rows: int, cols: int, e_lo: int, e_hi: int):
    """Source-layout MXFP4 matrix with uniform random 4-bit codes.

    Returns ``packed`` u8 [rows, cols/2] (two uniform codes per byte, the
    negative-zero code included) and ``scale`` u8 [rows, cols/32] with E8M0
    exponents uniform over the closed range [e_lo, e_hi].
    """
    assert cols % 32 == 0
    packed = np.frombuffer(g.bytes(rows * cols // 2), dtype=np.uint8).reshape(rows, cols // 2).copy()
    scale = g.integers(e_lo, e_hi + 1, size=(rows, cols // 32), dtype=np.uint8)
    return packed, scale


def q4k_blocks(g: np.random.Generator, rows: int, cols: int, e_lo: int = 1, e_hi: int = 3) -> np.ndarray:
    """Q4_K matrix u8 [rows, cols/256, 144] (ggml ``block_q4_K`` per 256 weights).

    The 12 packed scale/min bytes and the 128 code bytes are uniform random
    bytes; ``d`` and ``dmin`` (bytes 0-1 and 2-3, little-endian fp16) are
    positive with their 5-bit exponent field uniform over [e_lo, e_hi] and a
    uniform 10-bit mantissa (2^-14 up to just below 2^-11 for the defaults), so
    the weights span about the range of the MXFP4 experts' weights.
    """
    assert cols % 256 == 0
    nb = cols // 256
    b = np.frombuffer(g.bytes(rows * nb * 144), dtype=np.uint8).reshape(rows, nb, 144).copy()
    for off in (0, 2):
        e = g.integers(e_lo, e_hi + 1, size=(rows, nb), dtype=np.uint16)
        mant = g.integers(0, 1024, size=(rows, nb), dtype=np.uint16)
        bits = (e << 10) | mant
        b[..., off] = (bits & 0xFF).astype(np.uint8)
        b[..., off + 1] = (bits >> 8).astype(np.uint8)
    return b


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest-even) and return the raw u16 bits.

    Input preparation only: the layer consumes bf16 activations.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits to fp32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class LayerConfig:
    """One synthetic MoE-layer workload."""

    name: str
    config_id: int
    E: int
    k: int
    D: int
    I: int
    T: int
    e_lo: int = 118
    e_hi: int = 124
    logits: str = "normal"  # "normal" | "uniform" | "zipf"
    bias_sigma: float = 0.0  # 0 -> bias is identically zero
    zipf_s: float = 1.1
    seed: int = 0
    weight_id: int = -1  # key of the expert-weight streams; -1 -> config_id
    notes: str = ""

    def with_(self, **kw) -> "LayerConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return LayerConfig(**d)


# The five workloads (shapes from the pages; distributions as stated for each).
TINY = LayerConfig("tiny", 0, E=8, k=2, D=128, I=256, T=64, logits="normal", bias_sigma=0.1,
                   notes="8 experts, top-2, bias N(0,0.1), exps 118..124, 64 tokens")
# All K3-shaped workloads share one set of expert weights (weight_id 2).
K3_WEIGHTS = 2
DECODE1 = LayerConfig("decode-t1", 2, E=896, k=16, D=3584, I=3072, T=1, logits="uniform", weight_id=K3_WEIGHTS,
                      notes="K3 decode, 1 token, uniform logits, zero bias")
DECODE8 = DECODE1.with_(name="decode-t8", config_id=5, T=8, notes="K3 decode, 8 tokens, uniform logits, zero bias")
VERIFY = LayerConfig("verify", 3, E=896, k=16, D=3584, I=3072, T=128, logits="zipf", weight_id=K3_WEIGHTS,
                     notes="K3 speculative verify: 16 sequences x width 8, Zipf(1.1) skewed logits")
PREFILL = LayerConfig("prefill", 4, E=896, k=16, D=3584, I=3072, T=4096, logits="normal", bias_sigma=0.5,
                      weight_id=K3_WEIGHTS, notes="K3 prefill: 4096 tokens, logits N(0,1), bias N(0,0.5)")

CONFIGS = {c.name: c for c in (TINY, DECODE1, DECODE8, VERIFY, PREFILL)}

# Repack/dequant workload: one K3-shaped expert tensor [3072, 3584].
REPACK_ROWS, REPACK_COLS = 3072, 3584
REPACK_CONFIG_ID = 1


def repack_tensor(seed: int = 0, e_lo: int = 0, e_hi: int = 254):
    """One [3072, 3584] source tensor with uniform nibbles and E8M0 in [e_lo, e_hi]."""
    sub = 0 if (e_lo, e_hi) == (0, 254) else 1
    return mxfp4_source(rng(seed, REPACK_CONFIG_ID, T_SINGLE, sub), REPACK_ROWS, REPACK_COLS, e_lo, e_hi)


class ExpertSource:
    """Lazily generated source-layout weights of every expert of one config.

    ``src[e]`` returns ``((p1, s1), (p3, s3), (p2, s2))``: w1 and w3 are
    [I, D] (rows = intermediate features, blocks along D) and w2 is [D, I]
    (rows = latent features, blocks along I).
    """

    def __init__(self, cfg: LayerConfig):
        self.cfg = cfg

    def matrix(self, tensor_id: int, e: int):
        c = self.cfg
        rows, cols = (c.I, c.D) if tensor_id in (T_W1, T_W3) else (c.D, c.I)
        wid = c.config_id if c.weight_id < 0 else c.weight_id
        return mxfp4_source(rng(c.seed, 100 + wid, tensor_id, e), rows, cols, c.e_lo, c.e_hi)

    def __getitem__(self, e: int):
        return self.matrix(T_W1, e), self.matrix(T_W3, e), self.matrix(T_W2, e)

    def __len__(self):
        return self.cfg.E


class ExpertSourceQ4K:
    """Lazily generated Q4_K weights of every expert of one config.

    ``src[e]`` returns ``(w1, w3, w2)``: w1 and w3 u8 [I, D/256, 144], w2 u8
    [D, I/256, 144], each from its own keyed stream (keys 200 + weight id, so
    they never share a stream with the MXFP4 experts).
    """

    def __init__(self, cfg: LayerConfig):
        self.cfg = cfg

    def matrix(self, tensor_id: int, e: int) -> np.ndarray:
        c = self.cfg
        rows, cols = (c.I, c.D) if tensor_id in (T_W1, T_W3) else (c.D, c.I)
        wid = c.config_id if c.weight_id < 0 else c.weight_id
        return q4k_blocks(rng(c.seed, 200 + wid, tensor_id, e), rows, cols)

    def __getitem__(self, e: int):
        return self.matrix(T_W1, e), self.matrix(T_W3, e), self.matrix(T_W2, e)

    def __len__(self):
        return self.cfg.E


def activations(cfg: LayerConfig, seed: int | None = None) -> np.ndarray:
    """x ~ bf16(N(0,1)), shape [T, D], returned as raw bf16 bits (u16)."""
    s = cfg.seed if seed is None else seed
    g = rng(s, cfg.config_id, T_X)
    return bf16_bits(g.standard_normal((cfg.T, cfg.D), dtype=np.float32))


def router_inputs(cfg: LayerConfig, seed: int | None = None):
    """Router logits z [T, E] fp32 and expert bias b [E] fp32.

    * "normal":  z ~ N(0,1)
    * "uniform": z ~ U[0,1)
    * "zipf":    z[t,e] = N(0,1) + ln p_rank(e), p_r proportional to r^-s over
                 a seeded permutation of the experts (a few experts are hot)
    The bias is N(0, bias_sigma), or exactly zero when bias_sigma == 0.
    """
    s = cfg.seed if seed is None else seed
    g = rng(s, cfg.config_id, T_LOGITS)
    T, E = cfg.T, cfg.E
    if cfg.logits == "uniform":
        z = g.random((T, E), dtype=np.float32)
    elif cfg.logits == "normal":
        z = g.standard_normal((T, E), dtype=np.float32)
    elif cfg.logits == "zipf":
        ranks = rng(s, cfg.config_id, T_PERM).permutation(E) + 1  # rank of expert e, 1..E
        p = ranks.astype(np.float64) ** (-cfg.zipf_s)
        p /= p.sum()
        z = (g.standard_normal((T, E)) + np.log(p)[None, :]).astype(np.float32)
    else:
        raise ValueError(cfg.logits)
    if cfg.bias_sigma > 0:
        b = (rng(s, cfg.config_id, T_BIAS).standard_normal(E) * cfg.bias_sigma).astype(np.float32)
    else:
        b = np.zeros(E, np.float32)
    return np.ascontiguousarray(z), b


@dataclass
class Batch:
    """Everything one forward pass of the layer consumes (host side)."""

    cfg: LayerConfig
    x: np.ndarray  # u16 bf16 bits [T, D]
    z: np.ndarray  # f32 [T, E]
    b: np.ndarray  # f32 [E]
    experts: ExpertSource = field(repr=False, default=None)


def make_batch(cfg: LayerConfig, seed: int | None = None) -> Batch:
    z, b = router_inputs(cfg, seed)
    return Batch(cfg, activations(cfg, seed), z, b, ExpertSource(cfg))


# ---------------------------------------------------------------------------
# Latent-MoE block workloads: hidden rows h [T, H] go through the gate
# projection (router logits), ffn_routed_down / _norm into the latent width,
# the routed experts, ffn_routed_up back to H, plus a shared expert (tensor
# names from the llama.cpp page's dry-run comment; hidden width 7168 there).


@dataclass(frozen=True)
class BlockConfig:
    """One synthetic latent-MoE block workload.

    ``layer`` carries the routed part (E, k, latent D, expert I, T, the
    selection bias and the expert weights); its router-logit settings are
    unused, the logits come from the gate projection."""

    name: str
    config_id: int
    layer: LayerConfig
    H: int  # hidden width
    Is: int  # shared-expert intermediate width
    eps: float = 1e-6
    dense_id: int = -1  # key of the dense weight streams; -1 -> config_id
    notes: str = ""

    @property
    def T(self):
        return self.layer.T

    def with_(self, **kw) -> "BlockConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return BlockConfig(**d)


K3_DENSE = 3
BLOCK_TINY = BlockConfig("block-tiny", 20, TINY.with_(E=8, k=2, D=128, I=256, T=40, bias_sigma=0.1, config_id=21),
                         H=256, Is=192, notes="8 experts top-2, H 256, latent 128, shared 192, 40 tokens")
BLOCK_DECODE1 = BlockConfig("block-decode-t1", 22, DECODE1.with_(config_id=23), H=7168, Is=3072, dense_id=K3_DENSE,
                            notes="K3 block decode, 1 token")
BLOCK_DECODE8 = BlockConfig("block-decode-t8", 24, DECODE8.with_(config_id=25), H=7168, Is=3072, dense_id=K3_DENSE,
                            notes="K3 block decode, 8 tokens")
BLOCK_PREFILL = BlockConfig("block-prefill", 26, PREFILL.with_(config_id=27), H=7168, Is=3072, dense_id=K3_DENSE,
                            notes="K3 block prefill, 4096 tokens, bias N(0,0.5)")
BLOCK_CONFIGS = {c.name: c for c in (BLOCK_TINY, BLOCK_DECODE1, BLOCK_DECODE8, BLOCK_PREFILL)}


def block_hidden(cfg: BlockConfig, seed: int | None = None) -> np.ndarray:
    """h ~ bf16(N(0,1)), shape [T, H], as raw bf16 bits."""
    s = cfg.layer.seed if seed is None else seed
    g = rng(s, cfg.config_id, T_H)
    return bf16_bits(g.standard_normal((cfg.T, cfg.H), dtype=np.float32))


def block_dense_weights(cfg: BlockConfig) -> dict:
    """The dense weights as raw bf16 bits: each ~ N(0, 1/fan_in) (so every
    product's outputs are about unit scale), gamma ~ 1 + N(0, 0.1^2)."""
    L = cfg.layer
    wid = cfg.config_id if cfg.dense_id < 0 else cfg.dense_id
    shapes = {"Wg": (T_WG, L.E, cfg.H), "Wd": (T_WD, L.D, cfg.H), "Wu": (T_WU, cfg.H, L.D),
              "Ws1": (T_WS1, cfg.Is, cfg.H), "Ws3": (T_WS3, cfg.Is, cfg.H), "Ws2": (T_WS2, cfg.H, cfg.Is)}
    out = {}
    for name, (tid, rows, cols) in shapes.items():
        g = rng(L.seed, 200 + wid, tid)
        out[name] = bf16_bits(g.standard_normal((rows, cols), dtype=np.float32) * np.float32(cols ** -0.5))
    g = rng(L.seed, 200 + wid, T_GAMMA)
    out["gamma"] = bf16_bits((1.0 + 0.1 * g.standard_normal(L.D)).astype(np.float32))
    return out


def block_bias(cfg: BlockConfig) -> np.ndarray:
    """The selection bias of the routed part (zero when its sigma is 0)."""
    return router_inputs(cfg.layer.with_(T=1))[1]
