"""GPU parity of mxfp4_repack / mxfp4_dequant: bit-exact against the oracle;
mxfp4_tile bit-exact against its order built step by step from the definition."""

import numpy as np
import pytest
import torch

import moe_inputs
from oracle import mxfp4 as mx
from tests.gpu_util import to_dev_u8

pytestmark = pytest.mark.gpu


def every_code_and_exponent(rows_per_e=1):
    codes = np.tile(np.arange(16, dtype=np.uint8), 2)
    c = np.tile(codes, (256 * rows_per_e, 1))
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    scale = np.repeat(np.arange(256, dtype=np.uint8), rows_per_e).reshape(-1, 1)
    return packed, scale


def gpu_repack(k3, packed, scale):
    return k3.mxfp4_repack(to_dev_u8(packed), to_dev_u8(scale)).cpu().numpy()


@pytest.mark.parametrize("e_range", [(0, 254), (120, 122)])
def test_repack_dequant_k3_tensor(k3, e_range):
    """The page's repack check at the real tensor's shape: [3072, 3584], bit-exact."""
    print(f"[codec] K3 tensor e in {e_range}", flush=True)
    packed, scale = moe_inputs.repack_tensor(seed=0, e_lo=e_range[0], e_hi=e_range[1])
    ref_blocks = mx.repack_ref(packed, scale)
    blocks_dev = k3.mxfp4_repack(to_dev_u8(packed), to_dev_u8(scale))
    blocks = blocks_dev.cpu().numpy()
    assert blocks.shape == (3072, 112, 17) and blocks.nbytes == 5849088
    assert np.array_equal(blocks, ref_blocks)
    f32 = k3.mxfp4_dequant(blocks_dev, torch.float32).cpu().numpy()
    ref32 = mx.dequant_ref(ref_blocks, "f32")
    assert np.array_equal(f32.view(np.uint32), ref32.view(np.uint32))  # bitwise, +0 for code 8
    b16 = k3.mxfp4_dequant(blocks_dev, torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16, mx.dequant_ref(ref_blocks, "bf16"))
    # the page's value check: dequant(repack(P, S)) == decode(P, S), 0 mismatches
    src = mx.decode_ct(packed, scale)
    with np.errstate(over="ignore"):
        src32 = src.astype(np.float32)
    assert int((src32 != f32).sum()) == 0


def test_every_code_and_exponent_bitwise(k3):
    packed, scale = every_code_and_exponent(rows_per_e=3)
    ref_blocks = mx.repack_ref(packed, scale)
    blocks_dev = k3.mxfp4_repack(to_dev_u8(packed), to_dev_u8(scale))
    assert np.array_equal(blocks_dev.cpu().numpy(), ref_blocks)
    for dt, name in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        got = k3.mxfp4_dequant(blocks_dev, dt).cpu()
        got = got.numpy().view(np.uint32) if dt == torch.float32 else got.view(torch.int16).numpy().view(np.uint16)
        ref = mx.dequant_ref(ref_blocks, name)
        ref = ref.view(np.uint32) if name == "f32" else ref
        assert np.array_equal(got, ref), name


@pytest.mark.parametrize("R,K", [(1, 32), (37, 96), (5, 32 * 1023), (1025, 64), (3, 32 * 4097)])
def test_ragged_sizes(k3, R, K):
    """Block counts that leave partial workgroups (1024 / 256 blocks per workgroup)."""
    g = np.random.default_rng(R * 1000 + K)
    packed = g.integers(0, 256, size=(R, K // 2), dtype=np.uint8)
    scale = g.integers(0, 255, size=(R, K // 32), dtype=np.uint8)
    ref_blocks = mx.repack_ref(packed, scale)
    blocks_dev = k3.mxfp4_repack(to_dev_u8(packed), to_dev_u8(scale))
    assert np.array_equal(blocks_dev.cpu().numpy(), ref_blocks)
    got = k3.mxfp4_dequant(blocks_dev).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), mx.dequant_ref(ref_blocks).view(np.uint32))
    # the output buffer is fully overwritten and nothing past it is touched
    out = torch.full((R * K + 64,), 7.0, device="cuda")
    k3.mxfp4_dequant(blocks_dev, out=out[: R * K].view(R, K))
    torch.cuda.synchronize()
    assert torch.all(out[R * K:] == 7.0)


def test_empty_and_determinism(k3):
    z = torch.empty((0, 16), dtype=torch.uint8, device="cuda")
    zs = torch.empty((0, 1), dtype=torch.uint8, device="cuda")
    assert k3.mxfp4_repack(z, zs).shape == (0, 1, 17)
    packed, scale = moe_inputs.repack_tensor(seed=3, e_lo=118, e_hi=124)
    a = k3.mxfp4_repack(to_dev_u8(packed), to_dev_u8(scale))
    b = k3.mxfp4_repack(to_dev_u8(packed), to_dev_u8(scale))
    assert torch.equal(a, b)
    assert torch.equal(k3.mxfp4_dequant(a), k3.mxfp4_dequant(b))


def tiled_ref(blocks: np.ndarray) -> np.ndarray:
    """Stage-tiled order built as its definition reads: groups of 16 rows one
    after another, a group stage by stage (16 blocks, fewer at the end), a
    stage row by row, a row's blocks in order."""
    N, nb = blocks.shape[-3], blocks.shape[-2]
    out = []
    for m in blocks.reshape(-1, N, nb, 17):
        runs = []
        for g0 in range(0, N, 16):
            for b0 in range(0, nb, 16):
                for r in range(g0, min(g0 + 16, N)):
                    runs.append(m[r, b0:b0 + 16])
        out.append(np.concatenate(runs).reshape(N, nb, 17))
    return np.stack(out).reshape(blocks.shape)


# K3 gate/up and down matrices (16-byte copies), ragged row groups, ragged
# stages (byte copies: 23 and 17 blocks per row), a single block, a single row
@pytest.mark.parametrize("nmat,N,K", [(1, 3072, 3584), (3, 3584, 3072), (2, 40, 512), (2, 37, 736), (1, 5, 96),
                                      (2, 16, 32), (1, 1, 544)])
def test_tile_matches_definition(k3, nmat, N, K):
    print(f"[codec] tile nmat={nmat} N={N} K={K}", flush=True)
    g = np.random.default_rng(N * 7 + K)
    src = g.integers(0, 256, size=(nmat, N, K // 32, 17), dtype=np.uint8)
    got = k3.mxfp4_tile(to_dev_u8(src)).cpu().numpy()
    assert np.array_equal(got, tiled_ref(src))
    # the K3 order: stage s of group G is the contiguous 4352 bytes at
    # (G * (K / 512) + s) * 4352
    if N % 16 == 0 and K % 512 == 0:
        flat = got.reshape(nmat, -1)
        G, s = N // 16 - 1, K // 512 - 1
        piece = flat[:, (G * (K // 512) + s) * 4352:(G * (K // 512) + s + 1) * 4352].reshape(nmat, 16, 16, 17)
        assert np.array_equal(piece, src[:, 16 * G:16 * G + 16, 16 * s:16 * s + 16])


def test_tile_empty_and_out_argument(k3):
    z = torch.empty((0, 16, 2, 17), dtype=torch.uint8, device="cuda")
    assert k3.mxfp4_tile(z).shape == z.shape
    src = to_dev_u8(np.random.default_rng(1).integers(0, 256, size=(2, 20, 3, 17), dtype=np.uint8))
    out = torch.full_like(src, 7)
    assert k3.mxfp4_tile(src, out=out) is out
    assert np.array_equal(out.cpu().numpy(), tiled_ref(src.cpu().numpy()))
