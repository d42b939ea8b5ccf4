"""MXFP4 block encodings, written from their definitions (fp64, numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Both encodings are described on the llama.cpp pull-request page "model: add
Kimi-K3 text model", in the review comment "repack_mxfp4_blocks is bit-exact —
0 mismatches over 11,010,048 values":

* Source side (compressed-tensors ``pack_fp4_to_uint8`` / ``decompress_mx_scale``):
  ``weight_packed`` u8 [rows, cols/2] holds element 2i of a row in the LOW
  nibble of byte i and element 2i+1 in the HIGH nibble; bit 3 of a nibble is
  the sign and bits 0..2 index the E2M1 magnitudes [0, .5, 1, 1.5, 2, 3, 4, 6].
  ``weight_scale`` u8 [rows, cols/32] holds one E8M0 exponent e per 32
  consecutive elements of a row; the block scale is 2**(e - 127).

* ggml side (``block_mxfp4``, ``dequantize_row_mxfp4``, ``kvalues_fp4``,
  ``ggml_e8m0_to_fp32_half``): a 17-byte block per 32 elements.  Byte 0 is the
  E8M0 exponent; bytes 1..16 are ``qs``; element j of the block is the LOW
  nibble of qs[j] and element j+16 the HIGH nibble of qs[j].  A nibble indexes
  the doubled table [0,1,2,3,4,6,8,12, 0,-1,-2,-3,-4,-6,-8,-12] and the block
  multiplier is the "half" scale 2**(x - 128).

The same comment states that the repack keeps the represented values ("kvalues
doubled, scale halved, represented value unchanged") and accounts 17 bytes per
32 values (4.25 bits per weight).
"""

from __future__ import annotations

import numpy as np

# E2M1 magnitudes indexed by (code & 7); sign in bit 3 (source-side decode).
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

# ggml kvalues_fp4: doubled E2M1 values, nibble-indexed, sign in bit 3.
KVALUES = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], dtype=np.float64)

BLOCK = 32  # elements per MXFP4 block
BLOCK_BYTES = 17  # ggml block_mxfp4: 1 exponent byte + 16 nibble-pair bytes


def source_codes(packed: np.ndarray) -> np.ndarray:
    """4-bit code of every element of a source-layout row block.

    Element 2i of a row is the low nibble of byte i, element 2i+1 the high one.
    Returns u8 [rows, 2 * packed.shape[1]].
    """
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    codes = np.empty((rows, 2 * half), dtype=np.uint8)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    return codes


def decode_ct(packed: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Source-layout (compressed-tensors) MXFP4 decode, exactly, in fp64.

    value = (-1 if code & 8 else +1) * E2M1[code & 7] * 2**(e - 127), with e the
    exponent of the element's 32-block.  Exact in fp64 for every e in 0..255
    (the largest magnitude, 6 * 2**128, is far inside fp64 range).
    """
    codes = source_codes(packed)
    rows, cols = codes.shape
    scale = np.asarray(scale, dtype=np.uint8)
    assert scale.shape == (rows, cols // BLOCK), (scale.shape, codes.shape)
    magnitude = E2M1[codes & 7]
    signed = np.where((codes & 8) != 0, -magnitude, magnitude)
    block_scale = np.ldexp(1.0, scale.astype(np.int64) - 127)  # fp64, exact
    return signed * np.repeat(block_scale, BLOCK, axis=1)


def repack_ref(packed: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Source layout -> ggml 17-byte blocks, u8 [rows, cols/32, 17].

    A pure re-arrangement: the exponent byte is copied unchanged to byte 0 and
    every 4-bit code is copied unchanged into its ggml position (element j of a
    block -> low nibble of qs[j], element j+16 -> high nibble of qs[j]).
    Keeping codes and exponent byte as they are is what makes the represented
    value unchanged: ggml's doubled table times its halved scale equals the
    source's E2M1 value times 2**(e-127).
    """
    codes = source_codes(packed)
    rows, cols = codes.shape
    nb = cols // BLOCK
    scale = np.asarray(scale, dtype=np.uint8)
    assert scale.shape == (rows, nb)
    c = codes.reshape(rows, nb, BLOCK)
    out = np.empty((rows, nb, BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0] = scale
    out[:, :, 1:] = c[:, :, :16] | (c[:, :, 16:] << 4)
    return out


def unrepack_ref(blocks: np.ndarray):
    """Inverse of ``repack_ref``: ggml blocks -> (packed, scale) source layout."""
    blocks = np.asarray(blocks, dtype=np.uint8)
    rows, nb, nbytes = blocks.shape
    assert nbytes == BLOCK_BYTES
    qs = blocks[:, :, 1:]
    codes = np.concatenate([qs & 0x0F, qs >> 4], axis=2).reshape(rows, nb * BLOCK)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, blocks[:, :, 0].copy()


def dequant_ref(blocks: np.ndarray, out_dtype: str = "f32") -> np.ndarray:
    """ggml ``dequantize_row_mxfp4`` semantics: kvalue * 2**(x - 128).

    Computed exactly in fp64, then rounded once to the output type.  Every
    finite result is representable in fp32 and in bf16 (a kvalue has at most
    two significant bits), so the rounding only matters where the value
    overflows (x >= 254 with large codes), which gives +-inf.  Returns fp32
    [rows, nb*32], or raw bf16 bits (u16) when ``out_dtype == "bf16"``.
    """
    blocks = np.asarray(blocks, dtype=np.uint8)
    rows, nb, nbytes = blocks.shape
    assert nbytes == BLOCK_BYTES
    x = blocks[:, :, 0].astype(np.int64)
    qs = blocks[:, :, 1:]
    kv = np.concatenate([KVALUES[qs & 0x0F], KVALUES[qs >> 4]], axis=2)  # [rows, nb, 32]
    half = np.ldexp(1.0, x - 128)  # fp64, exact
    val64 = (kv * half[:, :, None]).reshape(rows, nb * BLOCK)
    with np.errstate(over="ignore"):
        val32 = val64.astype(np.float32)
    if out_dtype == "f32":
        return val32
    if out_dtype == "bf16":
        import torch

        t = torch.from_numpy(val32).to(torch.bfloat16)  # exact for these values
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(out_dtype)
