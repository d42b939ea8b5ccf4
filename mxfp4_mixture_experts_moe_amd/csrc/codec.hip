// MXFP4 codec kernels: compressed-tensors layout -> 17-byte ggml blocks,
// ggml blocks -> fp32 / bf16 values, and ggml row order -> the stage-tiled
// order the FFN kernels read.
//
// Layouts (llama.cpp pull request "model: add Kimi-K3 text model", review
// comment "repack_mxfp4_blocks is bit-exact"):
//   source: packed[r][i] holds element 2i (low nibble) and 2i+1 (high nibble);
//           scale[r][b] is the E8M0 exponent of elements 32b..32b+31.
//   ggml:   block = [exponent byte, qs[0..15]], element j = low nibble of
//           qs[j], element j+16 = high nibble; value = kvalues[nibble] *
//           2^(x-128) with kvalues the doubled E2M1 table.
//
// Both kernels treat the data as a flat sequence of blocks: block q (row
// q / nb, block q % nb) reads packed bytes [16q, 16q+16) and scale byte q, and
// owns output bytes [17q, 17q+17) or output elements [32q, 32q+32).
#include "k3moe_internal.h"

namespace k3moe {
namespace {

// ----------------------------------------------------------------------------
// Repack.  A workgroup of 256 threads handles 1024 blocks; thread p builds the
// 68 output bytes of blocks 4p..4p+3 (a dword-aligned run) in registers, writes
// them to LDS, and the workgroup then streams the 17 KB out with 16-byte stores.
constexpr int kRepackBlocksPerWg = 1024;
constexpr int kRepackBytesPerWg = kRepackBlocksPerWg * 17;  // 17408 = 1088 * 16

// qs dwords of one block from its 16 source bytes s0..s3 (little-endian dwords).
// qs[2m] = lo(S[m]) | lo(S[8+m]) << 4 and qs[2m+1] = hi(S[m]) | hi(S[8+m]) << 4.
__device__ __forceinline__ void repack_qs(uint32_t s0, uint32_t s1, uint32_t s2, uint32_t s3, uint32_t q[4]) {
  // bytes m = 0..3 come from s0 (with s2), m = 4..7 from s1 (with s3)
  const uint32_t lo_a = (s0 & 0x0F0F0F0Fu) | ((s2 & 0x0F0F0F0Fu) << 4);  // byte m: qs[2m]
  const uint32_t hi_a = ((s0 >> 4) & 0x0F0F0F0Fu) | (s2 & 0xF0F0F0F0u);  // byte m: qs[2m+1]
  const uint32_t lo_b = (s1 & 0x0F0F0F0Fu) | ((s3 & 0x0F0F0F0Fu) << 4);
  const uint32_t hi_b = ((s1 >> 4) & 0x0F0F0F0Fu) | (s3 & 0xF0F0F0F0u);
  // interleave: qs dword 0 = [lo0, hi0, lo1, hi1], dword 1 = [lo2, hi2, lo3, hi3]
  q[0] = __builtin_amdgcn_perm(hi_a, lo_a, 0x05010400u);
  q[1] = __builtin_amdgcn_perm(hi_a, lo_a, 0x07030602u);
  q[2] = __builtin_amdgcn_perm(hi_b, lo_b, 0x05010400u);
  q[3] = __builtin_amdgcn_perm(hi_b, lo_b, 0x07030602u);
}

__global__ __launch_bounds__(256) void repack_kernel(const uint8_t* __restrict__ packed,
                                                      const uint8_t* __restrict__ scale, int64_t nblocks,
                                                      uint8_t* __restrict__ blocks) {
  __shared__ uint32_t stage[kRepackBytesPerWg / 4];
  const int tid = threadIdx.x;
  const int64_t q0 = (int64_t)blockIdx.x * kRepackBlocksPerWg;
  const int64_t nloc64 = nblocks - q0;
  const int nloc = nloc64 < kRepackBlocksPerWg ? (int)nloc64 : kRepackBlocksPerWg;

  uint32_t o[17];
#pragma unroll
  for (int i = 0; i < 17; ++i) o[i] = 0;
  const int lb0 = tid * 4;  // first local block of this thread
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int lb = lb0 + b;
    if (lb < nloc) {
      const uint4 src = *reinterpret_cast<const uint4*>(packed + (q0 + lb) * 16);
      const uint32_t sc = scale[q0 + lb];
      uint32_t q[4];
      repack_qs(src.x, src.y, src.z, src.w, q);
      // 17 bytes [sc, q] as 5 little-endian words, then shifted to byte offset
      // 17b = 4*(4b) + b inside the 68-byte run.
      const uint32_t wds[5] = {sc | (q[0] << 8), (q[0] >> 24) | (q[1] << 8), (q[1] >> 24) | (q[2] << 8),
                               (q[2] >> 24) | (q[3] << 8), q[3] >> 24};
      // Bytes [b, b+17) of dwords d0..d0+4; the top byte lands at most at byte
      // 19, so nothing spills past the fifth dword.
      const int d0 = 4 * b;  // = (17 * b) / 4 for b in 0..3
      const int sh = 8 * b;  // bit offset of (17 * b) % 4 = b bytes
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        uint32_t v = wds[i] << sh;
        if (sh != 0 && i > 0) v |= wds[i - 1] >> (32 - sh);
        o[d0 + i] |= v;
      }
    }
  }
  // The run of this thread starts at byte 68 * tid = dword 17 * tid.
#pragma unroll
  for (int i = 0; i < 17; ++i) stage[17 * tid + i] = o[i];
  __syncthreads();

  const int nbytes = nloc * 17;
  uint8_t* dst = blocks + q0 * 17;
  const int nvec = nbytes / 16;
  for (int v = tid; v < nvec; v += 256)
    *reinterpret_cast<uint4*>(dst + 16 * v) = *reinterpret_cast<const uint4*>(&stage[4 * v]);
  const uint8_t* stage_b = reinterpret_cast<const uint8_t*>(stage);
  for (int i = nvec * 16 + tid; i < nbytes; i += 256) dst[i] = stage_b[i];
}

// ----------------------------------------------------------------------------
// Dequant.  A workgroup handles 256 blocks (4352 input bytes = 272 x 16 B).
// Eight lanes share a block; lane s writes elements 4s..4s+3 (16 B of fp32 or
// 8 B of bf16), so every store instruction of a wave covers 8 whole blocks.
constexpr int kDqBlocksPerWg = 256;
constexpr int kDqBytesPerWg = kDqBlocksPerWg * 17;

// fp32 bits of kvalues_fp4[n] (doubled E2M1, sign in bit 3, both zero codes +0).
__device__ __forceinline__ uint32_t kvalue_bits(uint32_t n) {
  const uint32_t m = n & 7u;       // magnitude code
  const uint32_t e2 = m >> 1;      // E2M1 exponent field
  const uint32_t mant = m & 1u;    // E2M1 mantissa bit
  // doubled value: m for e2 == 0 (0 or 1), else 2^e2 * (1 + mant/2)
  uint32_t mag = e2 ? (((127u + e2) << 23) | (mant << 22)) : (mant ? 0x3F800000u : 0u);
  const uint32_t sign = (m != 0u) ? ((n & 8u) << 28) : 0u;
  return mag | sign;
}

// 2^(x-128) as fp32: (x-1) << 23 for x >= 2, subnormals 2^-127 / 2^-128 below.
__device__ __forceinline__ float half_scale(uint32_t x) {
  const uint32_t bits = x >= 2u ? ((x - 1u) << 23) : (x == 1u ? 0x00400000u : 0x00200000u);
  return __uint_as_float(bits);
}

template <bool kBf16>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ blocks, int64_t nblocks,
                                                       void* __restrict__ out) {
  __shared__ uint32_t stage[kDqBytesPerWg / 4 + 1];
  const int tid = threadIdx.x;
  const int64_t q0 = (int64_t)blockIdx.x * kDqBlocksPerWg;
  const int64_t nloc64 = nblocks - q0;
  const int nloc = nloc64 < kDqBlocksPerWg ? (int)nloc64 : kDqBlocksPerWg;
  const int nbytes = nloc * 17;
  const uint8_t* src = blocks + q0 * 17;
  const int nvec = nbytes / 16;
  for (int v = tid; v < nvec; v += 256)
    *reinterpret_cast<uint4*>(&stage[4 * v]) = *reinterpret_cast<const uint4*>(src + 16 * v);
  uint8_t* stage_b = reinterpret_cast<uint8_t*>(stage);
  for (int i = nvec * 16 + tid; i < nbytes; i += 256) stage_b[i] = src[i];
  if (tid == 0) stage[kDqBytesPerWg / 4] = 0;
  __syncthreads();

  const int s = tid & 7;
  for (int lb = tid >> 3; lb < nloc; lb += 32) {
    const int base = 17 * lb;
    const uint32_t x = stage_b[base];
    const int off = base + 1 + 4 * (s & 3);  // first of the 4 qs bytes this lane needs
    const uint32_t qd = __builtin_amdgcn_alignbyte(stage[(off >> 2) + 1], stage[off >> 2], off & 3);
    const uint32_t shift = (s >> 2) * 4;  // low nibbles for s < 4, high nibbles for s >= 4
    const float sc = half_scale(x);
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(kvalue_bits((qd >> (8 * i + shift)) & 0xFu)) * sc;
    const int64_t e0 = (q0 + lb) * 32 + 4 * s;
    if (kBf16) {
      // exact: every value has at most 2 significant bits, so the top half is the value
      uint2 pk;
      pk.x = (__float_as_uint(v[0]) >> 16) | (__float_as_uint(v[1]) & 0xFFFF0000u);
      pk.y = (__float_as_uint(v[2]) >> 16) | (__float_as_uint(v[3]) & 0xFFFF0000u);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + e0) = pk;
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + e0) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// ----------------------------------------------------------------------------
// Tile: ggml row order -> stage-tiled order (tiled_block_index).  Workgroup
// (matrix, group G, stage s) moves one piece: its rG rows of wS blocks, row r
// from source blocks (16G + r) * nb + 16s onwards to the piece's row r.  With
// nb a multiple of 16 every row of a piece is 272 bytes at 16-byte aligned
// offsets on both sides and moves as 17 chunks of 16 bytes; otherwise bytes.
template <bool kVec16>
__global__ __launch_bounds__(256) void tile_kernel(const uint8_t* __restrict__ src, int N, int nb, int ngroups,
                                                    int nstages, uint8_t* __restrict__ dst) {
  const int64_t piece = blockIdx.x;
  const int s = (int)(piece % nstages);
  const int64_t mg = piece / nstages;
  const int G = (int)(mg % ngroups);
  const int64_t m = mg / ngroups;
  const int rG = N - 16 * G < 16 ? N - 16 * G : 16;
  const int wS = nb - 16 * s < 16 ? nb - 16 * s : 16;
  const int64_t mat = m * (int64_t)N * nb * 17;
  const int64_t src0 = mat + ((int64_t)16 * G * nb + 16 * s) * 17;  // row 0 of the piece in the source
  const int64_t dst0 = mat + tiled_block_index(N, nb, 16 * G, 16 * s) * 17;
  const int64_t src_row = (int64_t)nb * 17;
  if (kVec16) {
    for (int i = threadIdx.x; i < rG * 17; i += 256) {
      const int r = i / 17, c = i - 17 * r;
      *reinterpret_cast<uint4*>(dst + dst0 + 272 * r + 16 * c) =
          *reinterpret_cast<const uint4*>(src + src0 + src_row * r + 16 * c);
    }
  } else {
    const int row_b = wS * 17;
    for (int i = threadIdx.x; i < rG * row_b; i += 256) {
      const int r = i / row_b, c = i - row_b * r;
      dst[dst0 + (int64_t)row_b * r + c] = src[src0 + src_row * r + c];
    }
  }
}

}  // namespace

hipError_t launch_tile(const uint8_t* src, int64_t nmat, int N, int nb, uint8_t* dst, hipStream_t s) {
  const int ngroups = (N + 15) / 16, nstages = (nb + 15) / 16;
  const int64_t wgs = nmat * ngroups * nstages;
  if (nb % 16 == 0)
    hipLaunchKernelGGL(tile_kernel<true>, dim3((unsigned)wgs), dim3(256), 0, s, src, N, nb, ngroups, nstages, dst);
  else
    hipLaunchKernelGGL(tile_kernel<false>, dim3((unsigned)wgs), dim3(256), 0, s, src, N, nb, ngroups, nstages, dst);
  return hipGetLastError();
}

hipError_t launch_repack(const uint8_t* packed, const uint8_t* scale, int64_t nblocks, uint8_t* blocks,
                         hipStream_t s) {
  const int64_t wgs = (nblocks + kRepackBlocksPerWg - 1) / kRepackBlocksPerWg;
  hipLaunchKernelGGL(repack_kernel, dim3((unsigned)wgs), dim3(256), 0, s, packed, scale, nblocks, blocks);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* blocks, int64_t nblocks, int out_bf16, void* out, hipStream_t s) {
  const int64_t wgs = (nblocks + kDqBlocksPerWg - 1) / kDqBlocksPerWg;
  if (out_bf16)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3((unsigned)wgs), dim3(256), 0, s, blocks, nblocks, out);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3((unsigned)wgs), dim3(256), 0, s, blocks, nblocks, out);
  return hipGetLastError();
}

}  // namespace k3moe
