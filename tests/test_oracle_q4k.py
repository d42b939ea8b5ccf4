"""Pins of the oracle's Q4_K decode and of the routed FFN over Q4_K experts (CPU only).

The pages name Q4_K without defining it, so nothing here comes from them: the
oracle follows ggml's published block layout, and these tests pin it to a
block encoded by hand (tests/golden/q4k_block_example.txt), to an encoder
written as the inverse of the packing (round trip over every 6-bit value),
to closed forms of the fp16 fields, and to a pure-Python loop evaluation of
the FFN on weights built from their design values.
"""

import numpy as np

from oracle import q4k as q
from tests.conftest import read_golden


def encode_block(d_bits: int, dmin_bits: int, sc, m, codes) -> np.ndarray:
    """144 bytes of one block from its design: fp16 bit patterns of d and dmin,
    eight 6-bit scales and mins, codes [8][32] (sub-block, element)."""
    b = np.zeros(144, dtype=np.uint8)
    b[0], b[1] = d_bits & 0xFF, d_bits >> 8
    b[2], b[3] = dmin_bits & 0xFF, dmin_bits >> 8
    for j in range(4):
        # low six bits: pairs 0..3; top two bits: bits 4..5 of pairs 4..7
        b[4 + j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        b[8 + j] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        # low four bits of pairs 4..7, scale in the low nibble, min in the high
        b[12 + j] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    for c in range(4):
        for i in range(32):
            b[16 + 32 * c + i] = codes[2 * c][i] | (codes[2 * c + 1][i] << 4)
    return b


def test_golden_block_decodes_to_its_design():
    g = read_golden("q4k_block_example.txt")
    raw = np.array([int(v, 16) for v in g["bytes"]], dtype=np.uint8)
    assert raw.size == 144
    sc = [int(v) for v in g["scales"]]
    mn = [int(v) for v in g["mins"]]
    d, dmin = float(g["d"][0]), float(g["dmin"][0])
    expected = np.empty(256)
    for j in range(8):
        for i in range(32):
            code = i % 16 if j % 2 == 0 else (i + 5 * (j // 2)) % 16
            expected[32 * j + i] = d * sc[j] * code - dmin * mn[j]
    got = q.q4k_decode(raw.reshape(1, 1, 144))
    assert got.shape == (1, 256)
    assert np.array_equal(got[0], expected)
    s, mm = q.q4k_scale_min(raw[4:16])
    assert s.tolist() == sc and mm.tolist() == mn


def test_scale_min_round_trip_every_value():
    """Every 6-bit value in every one of the eight (scale, min) slots survives encode -> decode."""
    zeros = [[0] * 32 for _ in range(8)]
    for j in range(8):
        for v in range(64):
            sc = [(7 * t + 3) % 64 for t in range(8)]
            mn = [(11 * t + 5) % 64 for t in range(8)]
            sc[j] = v
            mn[j] = 63 - v
            b = encode_block(0x3C00, 0x3C00, sc, mn, zeros)
            s, m = q.q4k_scale_min(b[4:16])
            assert s.tolist() == sc and m.tolist() == mn, (j, v)


def test_codes_every_nibble_position():
    """Each code position decodes to the value placed there by its design (d = 1, scale 1, min 0)."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(8, 32)).tolist()
    b = encode_block(0x3C00, 0x0000, [1] * 8, [0] * 8, codes)
    got = q.q4k_decode(b.reshape(1, 1, 144))[0]
    assert np.array_equal(got, np.array(codes, dtype=np.float64).reshape(256))


def test_fp16_fields_closed_forms():
    """d and dmin are IEEE half precision: subnormal, negative, zero and the largest finite value."""
    codes = [[(i + j) % 16 for i in range(32)] for j in range(8)]
    sc = [1, 5, 9, 13, 17, 21, 25, 63]
    mn = [63, 2, 4, 8, 16, 32, 1, 0]
    code_arr = np.array(codes, dtype=np.float64)
    for d_bits, d_val in ((0x0001, 2.0 ** -24), (0x03FF, 1023 * 2.0 ** -24), (0xB400, -0.25), (0x0000, 0.0),
                          (0x7BFF, 65504.0), (0x3555, 0.25 * (1 + 341 / 1024))):
        for dmin_bits, dmin_val in ((0x0000, 0.0), (0x8001, -(2.0 ** -24)), (0x3800, 0.5)):
            b = encode_block(d_bits, dmin_bits, sc, mn, codes)
            got = q.q4k_decode(b.reshape(1, 1, 144))[0].reshape(8, 32)
            want = d_val * np.array(sc, dtype=np.float64)[:, None] * code_arr - dmin_val * np.array(mn, dtype=np.float64)[:, None]
            assert np.array_equal(got, want), (hex(d_bits), hex(dmin_bits))


def test_decode_block_and_row_order():
    """Blocks run along the row: row r, block t covers columns 256 t .. 256 t + 255."""
    blocks = np.zeros((3, 2, 144), dtype=np.uint8)
    for r in range(3):
        for t in range(2):
            blocks[r, t] = encode_block(0x3C00, 0x0000, [1] * 8, [0] * 8, [[(r * 2 + t) % 16] * 32 for _ in range(8)])
    got = q.q4k_decode(blocks)
    assert got.shape == (3, 512)
    for r in range(3):
        for t in range(2):
            assert np.all(got[r, 256 * t:256 * (t + 1)] == (r * 2 + t) % 16)


def _design_matrix(rng, rows, cols):
    """Random design values of a Q4_K matrix: its blocks and the weights they stand for."""
    nb = cols // 256
    blocks = np.zeros((rows, nb, 144), dtype=np.uint8)
    w = np.zeros((rows, cols))
    for r in range(rows):
        for t in range(nb):
            d_val = float(rng.integers(1, 9)) / 64.0  # exact in fp16
            dmin_val = float(rng.integers(0, 9)) / 64.0
            d_bits = int(np.float16(d_val).view(np.uint16))
            dmin_bits = int(np.float16(dmin_val).view(np.uint16))
            sc = rng.integers(0, 64, size=8).tolist()
            mn = rng.integers(0, 64, size=8).tolist()
            codes = rng.integers(0, 16, size=(8, 32)).tolist()
            blocks[r, t] = encode_block(d_bits, dmin_bits, sc, mn, codes)
            for j in range(8):
                for i in range(32):
                    w[r, 256 * t + 32 * j + i] = d_val * sc[j] * codes[j][i] - dmin_val * mn[j]
    return blocks, w


def test_ffn_q4k_ref_matches_python_loops():
    """The routed FFN over Q4_K experts against loops over weights built from their design values."""
    import math

    rng = np.random.default_rng(11)
    E, D, I, T, k = 3, 256, 256, 3, 2
    experts, W = [], []
    for _ in range(E):
        b1, w1 = _design_matrix(rng, I, D)
        b3, w3 = _design_matrix(rng, I, D)
        b2, w2 = _design_matrix(rng, D, I)
        experts.append((b1, b3, b2))
        W.append((w1, w3, w2))
    x = (rng.standard_normal((T, D)) * 0.05).astype(np.float32)
    x_bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern is a valid input
    xv = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ids = np.array([[0, 2], [1, 1], [2, 0]])  # token 1 repeats expert 1: its second slot is skipped
    wts = np.array([[0.75, 0.25], [0.5, 2.0], [1.0, -1.0]], dtype=np.float32)
    got = q.ffn_q4k_ref(x_bits, ids, wts, experts)
    want = np.zeros((T, D))
    for t in range(T):
        seen = set()
        for j in range(k):
            e = int(ids[t, j])
            if e in seen:
                continue
            seen.add(e)
            w1, w3, w2 = W[e]
            h = []
            for f in range(I):
                gv = sum(w1[f, c] * xv[t, c] for c in range(D))
                uv = sum(w3[f, c] * xv[t, c] for c in range(D))
                h.append(gv / (1.0 + math.exp(-gv)) * uv)
            for o in range(D):
                want[t, o] += float(wts[t, j]) * sum(w2[o, f] * h[f] for f in range(I))
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
