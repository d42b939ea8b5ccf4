"""Pins of the oracle's MXFP4 codec (CPU only).

Each test checks oracle/mxfp4.py against something other than itself: the
tables and figures the pages print (tests/golden), the IEEE-754 / OCP FP4 bit
formats, torch's E8M0 decoding, and brute force over every (code, exponent).
"""

import numpy as np
import pytest
import torch

import moe_inputs
from oracle import mxfp4 as mx
from tests.conftest import read_golden


def every_code_exponent_block(exps):
    """Source tensor with one row per exponent; each 32-block holds codes 0..15 twice."""
    codes = np.tile(np.arange(16, dtype=np.uint8), 2)  # element i -> code i % 16
    rows = len(exps)
    c = np.tile(codes, (rows, 1))
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    scale = np.asarray(exps, dtype=np.uint8).reshape(rows, 1)
    return packed, scale, c


def test_tables_match_page():
    g = read_golden("mxfp4_tables.txt")
    assert np.array_equal(mx.E2M1, np.array([float(v) for v in g["e2m1"]]))
    assert np.array_equal(mx.KVALUES, np.array([float(v) for v in g["kvalues_fp4"]]))
    # "kvalues doubled": every kvalue is twice the signed E2M1 value of the same nibble
    signed = np.array([(-1.0 if c & 8 else 1.0) * float(g["e2m1"][c & 7]) for c in range(16)])
    assert np.array_equal(mx.KVALUES, 2.0 * signed)


def test_e2m1_matches_fp4_bit_format():
    """E2M1 = 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 is subnormal."""
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = (0.5 * m) if e == 0 else (2.0 ** (e - 1)) * (1.0 + 0.5 * m)
        v = -v if s else v
        packed = np.array([[c | (c << 4)] * 16], dtype=np.uint8)
        got = mx.decode_ct(packed, np.array([[127]], dtype=np.uint8))
        assert np.all(got == v), (c, got[0, 0], v)
        assert np.all(np.signbit(got) == bool(s))


def test_e8m0_scale_matches_torch_e8m0():
    """The source block scale 2**(e-127) equals torch.float8_e8m0fnu's decode, e = 0..254."""
    e = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(e.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    packed = np.full((255, 16), 0x22, dtype=np.uint8)  # code 2 -> 1.0 everywhere
    got = mx.decode_ct(packed, e.reshape(255, 1))
    assert np.array_equal(got[:, 0], ref)


def test_decode_ct_element_order():
    g = read_golden("repack_block_example.txt")
    packed = np.array([[int(v, 16) for v in g["packed"]]], dtype=np.uint8)
    scale = np.array([[int(g["scale"][0], 16)]], dtype=np.uint8)
    expect = np.array([float(v) for v in g["values"]])
    got = mx.decode_ct(packed, scale)[0]
    assert np.array_equal(got, expect)
    assert np.array_equal(np.signbit(got), np.signbit(expect))  # -0 for code 8


def test_repack_block_example():
    g = read_golden("repack_block_example.txt")
    packed = np.array([[int(v, 16) for v in g["packed"]]], dtype=np.uint8)
    scale = np.array([[int(g["scale"][0], 16)]], dtype=np.uint8)
    block = np.array([int(v, 16) for v in g["block"]], dtype=np.uint8)
    out = mx.repack_ref(packed, scale)
    assert out.shape == (1, 1, 17)
    assert np.array_equal(out[0, 0], block)
    # ggml decode of the block gives the listed values (as IEEE values; code 8 decodes to +0)
    vals = mx.dequant_ref(out)[0]
    assert np.all(vals == np.array([float(v) for v in g["values"]], dtype=np.float32))


def test_value_equality_every_code_and_exponent():
    """dequant(repack(P,S)) == decode(P,S) for all 16 codes x all 256 exponents.

    This is the page's check (element-wise IEEE comparison, 0 mismatches),
    extended to every exponent (including the x < 2 branch the page's tensor did
    not reach).  Results are compared in fp32 as the page's check does.
    """
    packed, scale, codes = every_code_exponent_block(range(256))
    src = mx.decode_ct(packed, scale)
    with np.errstate(over="ignore"):
        ref32 = src.astype(np.float32)
    got = mx.dequant_ref(mx.repack_ref(packed, scale))
    assert int((ref32 != got).sum()) == 0
    # bitwise: the only difference is the sign of zero for code 8 (-0 vs ggml's +0)
    diff = ref32.view(np.uint32) != got.view(np.uint32)
    assert np.all(codes[diff] == 8)
    assert np.all(got[codes == 8] == 0) and not np.any(np.signbit(got[codes == 8]))


def test_subnormal_and_overflow_bit_patterns():
    """ggml half scale 2**(x-128) for x < 2 lands in fp32 subnormals; large x overflows."""
    def one(code, x):
        blk = np.zeros((1, 1, 17), dtype=np.uint8)
        blk[0, 0, 0] = x
        blk[0, 0, 1] = code  # element 0 = low nibble of qs[0]
        return int(mx.dequant_ref(blk).view(np.uint32)[0, 0])

    # IEEE-754 binary32: value = 2**-149 * mantissa field when the exponent field is 0.
    assert one(1, 0) == 0x00200000  # kvalue 1 * 2**-128 = 2**21 * 2**-149
    assert one(1, 1) == 0x00400000  # 2**-127
    assert one(2, 0) == 0x00400000  # 2 * 2**-128
    assert one(4, 0) == 0x00800000  # 4 * 2**-128 = 2**-126, the smallest normal
    assert one(7, 0) == 0x01400000  # 12 * 2**-128 = 1.5 * 2**-125
    assert one(9, 0) == 0x80200000  # -1 * 2**-128
    assert one(1, 2) == 0x00800000  # x = 2: bits (x - 1) << 23, the page's formula
    assert one(1, 200) == (199 << 23)
    assert one(2, 254) == 0x7F000000  # 2 * 2**126 = 2**127
    assert one(4, 254) == 0x7F800000  # 4 * 2**126 overflows to +inf
    assert one(12, 254) == 0xFF800000  # -4 * 2**126 -> -inf
    assert one(1, 255) == 0x7F000000  # 2**127 (formula value; E8M0 255 is outside the configs)
    assert one(0, 255) == 0 and one(8, 255) == 0


def test_dequant_bf16_is_exact():
    packed, scale, _ = every_code_exponent_block(range(256))
    blocks = mx.repack_ref(packed, scale)
    f32 = mx.dequant_ref(blocks, "f32")
    b16 = mx.dequant_ref(blocks, "bf16")
    bits = f32.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0)  # every value (inf included) fits bf16 exactly
    assert np.array_equal(b16, (bits >> 16).astype(np.uint16))


def test_repack_round_trip_is_a_bijection():
    g = np.random.default_rng(7)
    # every byte value at every packed position, and every exponent byte
    packed = np.stack([np.roll(np.arange(256, dtype=np.uint8), r)[:64] for r in range(256)])  # [256, 64]
    scale = g.integers(0, 256, size=(256, 4), dtype=np.uint8)
    blocks = mx.repack_ref(packed, scale)
    p2, s2 = mx.unrepack_ref(blocks)
    assert np.array_equal(p2, packed) and np.array_equal(s2, scale)
    rnd = g.integers(0, 256, size=(5, 7, 17), dtype=np.uint8)
    assert np.array_equal(mx.repack_ref(*mx.unrepack_ref(rnd)), rnd)


def test_repack_check_at_k3_shape():
    """The page's repack check, on a synthetic tensor of the real tensor's shape and exponents."""
    g = read_golden("repack_check_k3_w1.txt")
    rows, cols = int(g["rows"][0]), int(g["cols"][0])
    lo, hi = int(g["e8m0_min"][0]), int(g["e8m0_max"][0])
    packed, scale = moe_inputs.repack_tensor(seed=0, e_lo=lo, e_hi=hi)
    assert packed.shape == (rows, cols // 2) and scale.shape == (rows, cols // 32)
    blocks = mx.repack_ref(packed, scale)
    ref = mx.decode_ct(packed, scale).astype(np.float32)
    got = mx.dequant_ref(blocks)
    assert ref.size == int(g["values"][0])
    assert int((ref != got).sum()) == int(g["mismatched"][0])
    assert float(np.abs(ref - got).max()) == float(g["max_abs_error"][0])
    assert packed.nbytes + scale.nbytes == int(g["bytes_in"][0])
    assert blocks.nbytes == int(g["bytes_out"][0])
    assert f"{blocks.nbytes * 8 / (rows * cols):.4f}" == g["bpw"][0]


@pytest.mark.slow
def test_repack_check_full_exponent_range():
    packed, scale = moe_inputs.repack_tensor(seed=0, e_lo=0, e_hi=254)
    assert scale.min() == 0 and scale.max() == 254
    ref = mx.decode_ct(packed, scale)
    with np.errstate(over="ignore"):
        ref32 = ref.astype(np.float32)
    got = mx.dequant_ref(mx.repack_ref(packed, scale))
    assert int((ref32 != got).sum()) == 0
