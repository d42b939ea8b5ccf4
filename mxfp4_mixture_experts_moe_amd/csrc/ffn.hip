// Grouped expert GEMMs with the MXFP4 decode fused in, and the weighted combine.
//
// Shapes (llama.cpp pull request "model: add Kimi-K3 text model"): an expert
// is w1 | w2 | w3 (dry-run comment); w1 and w3 are [I, D] (logical [3072, 3584]
// for K3, repack comment), w2 is [D, I]; every row is stored as 17-byte ggml
// MXFP4 blocks along the contraction dimension.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16, fp32 accumulate): the 16 MFMA rows
// are 16 weight rows (output features), the 16 columns are 16 tokens.  A lane
// owns one weight row and one of four K slices.  One ggml block holds 32
// weights with a single E8M0 exponent; the decode multiplies each 4-bit code by
// that block's scale while converting to bf16 (v_cvt_scalef32_pk_bf16_fp4),
// which is exact for every code and every exponent that keeps the product in
// range, so the MFMA needs no rescale afterwards.  Because qs byte j holds
// elements j and j+16, a decoded dword is the pair (j, j+16); the activations
// are stored in the same order inside each 32-block ("P order": position
// 8i + 2t + h holds element 16h + 4i + t), so A and B agree on K.
//
// Precision: h = SiLU(g) * u is formed in fp32 and handed to the down product
// as two bf16 terms, hi = bf16(h) and lo = bf16(h - hi); both multiply the same
// decoded w2 operand, so h enters with about 16 significant bits while every
// MFMA stays bf16 x bf16 -> fp32.
//
// Work decomposition: a workgroup of 4 waves computes 64 output features for
// one tile of up to 16*NT grouped rows of one expert.  Weight rows are staged
// through LDS one K segment (up to 16 blocks = 272 bytes per row) at a time
// with coalesced loads (in the stage-tiled weight order a segment of 16 rows
// is one contiguous run); each wave decodes its own 16 rows.
#include "k3moe_internal.h"

#include <math.h>

namespace k3moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kFeatPerWg = 64;   // output features per workgroup (16 per wave)
constexpr int kSegBlocks = 16;   // MXFP4 blocks per K segment
constexpr int kLdsRowDw = 68;    // LDS dwords per staged row (16 blocks * 17 B / 4)

// Element of a 32-block stored at P-order position p.
__device__ __forceinline__ int p_to_elem(int p) { return 16 * (p & 1) + 4 * (p >> 3) + ((p >> 1) & 3); }

// Block scale 2^(e-127) as fp32 (e = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return __uint_as_float(e ? (e << 23) : 0x00400000u);
}

// 8 weights (qs dword q = 4 nibble pairs) -> bf16x8 in P order, scaled.
__device__ __forceinline__ bf16x8_t decode_dword(uint32_t q, float sf) {
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sf, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sf, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sf, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sf, 3));
  return __builtin_bit_cast(bf16x8_t, r);
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);  // round to nearest even
}

// Stage K segment `seg` (nbs blocks: 16, fewer in a last segment) of rows
// f0 .. f0 + nrows - 1 of one expert's stage-tiled matrix `w` (N rows x nb
// blocks) into LDS (row r at dword r * kLdsRowDw); rows nrows..63 are left
// as they are (the MFMA rows they feed are never stored).  In the tiled order
// a row's blocks of one segment are contiguous, starting at block
// tiled_block_index(N, nb, row, 16 * seg).
// kVec16 (nb a multiple of 16): every row piece is 272 bytes at a 16-byte
// aligned offset.  Otherwise dword copies when nb is a multiple of 4 (then
// every piece's offset and length are), and byte copies for the rest.
template <bool kVec16>
__device__ __forceinline__ void stage_weights(const uint8_t* __restrict__ w, int N, int nb, int f0, int seg,
                                              int nbs, int nrows, uint32_t* lds) {
  if (kVec16) {
    for (int idx = threadIdx.x; idx < nrows * 17; idx += blockDim.x) {
      const int r = idx / 17, c = idx - r * 17;
      const uint8_t* src = w + tiled_block_index(N, nb, f0 + r, 16 * seg) * 17;
      *reinterpret_cast<uint4*>(lds + r * kLdsRowDw + 4 * c) = *reinterpret_cast<const uint4*>(src + 16 * c);
    }
  } else if ((nb & 3) == 0) {
    const int dpr = nbs * 17 / 4;
    for (int idx = threadIdx.x; idx < nrows * dpr; idx += blockDim.x) {
      const int r = idx / dpr, c = idx - r * dpr;
      const uint8_t* src = w + tiled_block_index(N, nb, f0 + r, 16 * seg) * 17;
      lds[r * kLdsRowDw + c] = *reinterpret_cast<const uint32_t*>(src + 4 * c);
    }
  } else {
    uint8_t* lb = reinterpret_cast<uint8_t*>(lds);
    const int seg_bytes = nbs * 17;
    for (int idx = threadIdx.x; idx < nrows * seg_bytes; idx += blockDim.x) {
      const int r = idx / seg_bytes, c = idx - r * seg_bytes;
      lb[r * kLdsRowDw * 4 + c] = w[tiled_block_index(N, nb, f0 + r, 16 * seg) * 17 + c];
    }
  }
}

// Decode block (4*rnd + g) of the staged segment for LDS row `lrow`: the lane's
// four operands (P-order positions 8i..8i+7, i = 0..3).
__device__ __forceinline__ void decode_block(const uint32_t* lds, int lrow, int rnd, int g, bf16x8_t op[4]) {
  // block 4*rnd + g starts at byte 68*rnd + 17*g = dword 17*rnd + 4*g, byte g
  const uint32_t* L = lds + lrow * kLdsRowDw + 17 * rnd + 4 * g;
  const uint32_t d0 = L[0], d1 = L[1], d2 = L[2], d3 = L[3], d4 = L[4];
  const float sf = e8m0_to_f32((d0 >> (8 * g)) & 0xFFu);
  // qs dword i = bytes g+1+4i .. g+4+4i of d0..d4
  uint32_t q0, q1, q2, q3;
  if (g == 3) {
    q0 = d1; q1 = d2; q2 = d3; q3 = d4;
  } else {
    const int sh = g + 1;
    q0 = __builtin_amdgcn_alignbyte(d1, d0, sh);
    q1 = __builtin_amdgcn_alignbyte(d2, d1, sh);
    q2 = __builtin_amdgcn_alignbyte(d3, d2, sh);
    q3 = __builtin_amdgcn_alignbyte(d4, d3, sh);
  }
  op[0] = decode_dword(q0, sf);
  op[1] = decode_dword(q1, sf);
  op[2] = decode_dword(q2, sf);
  op[3] = decode_dword(q3, sf);
}

template <int NT, bool kGateUp, bool kVec16>
__global__ __launch_bounds__(256) void ffn_gemm_kernel(GemmArgs a) {
  constexpr int kMats = kGateUp ? 2 : 1;
  __shared__ uint32_t wlds[kMats][kFeatPerWg * kLdsRowDw];

  const int64_t tile_idx = blockIdx.x;
  if (tile_idx >= *a.tile_count) return;  // uniform over the workgroup
  const Tile tile = a.tiles[tile_idx];
  const int f0 = blockIdx.y * kFeatPerWg;
  // output features of this workgroup: 64, or 32 in the last feature tile
  // when N is an odd multiple of 32
  const int nfeat = a.N - f0 < kFeatPerWg ? a.N - f0 : kFeatPerWg;
  const int nb = a.K >> 5;
  const size_t row_bytes = (size_t)nb * 17;
  const size_t mat_bytes = (size_t)a.N * row_bytes;
  const uint8_t* wA = a.wa + (size_t)tile.expert * mat_bytes;
  const uint8_t* wB = kGateUp ? a.wb + (size_t)tile.expert * mat_bytes : nullptr;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rho = lane & 15, g = lane >> 4;
  // LDS row (feature f0 + lrow) that feeds MFMA row rho of this wave.  For
  // gate/up the rows are chosen so that a lane's four outputs are four
  // consecutive P-order positions of h (one 8-byte store).  A wave's features
  // are f0 + 32 * (wave / 2) + 0..31 (gate/up) or f0 + 16 * wave + 0..15 (down).
  const int lrow = kGateUp ? 32 * (wave >> 1) + p_to_elem(16 * (wave & 1) + rho) : 16 * wave + rho;
  const bool wave_live = (kGateUp ? 32 * (wave >> 1) : 16 * wave) < nfeat;

  const uint16_t* brow[NT];
  const uint16_t* brow_lo[NT];
  bool bvalid[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int m = nt * 16 + rho;
    bvalid[nt] = m < tile.nrows;
    const int row = tile.row0 + (bvalid[nt] ? m : 0);
    const int64_t src_row = kGateUp ? (int64_t)a.row_tok[row] : (int64_t)row;
    brow[nt] = a.act + src_row * a.K;
    brow_lo[nt] = kGateUp ? nullptr : a.act_lo + src_row * a.K;
  }

  f32x4_t acc[kMats][NT];
#pragma unroll
  for (int mi = 0; mi < kMats; ++mi)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mi][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int seg0 = 0; seg0 < nb; seg0 += kSegBlocks) {
    const int nbs = (nb - seg0) < kSegBlocks ? (nb - seg0) : kSegBlocks;
    __syncthreads();  // previous segment fully consumed
    stage_weights<kVec16>(wA, a.N, nb, f0, seg0 / kSegBlocks, nbs, nfeat, wlds[0]);
    if (kGateUp) stage_weights<kVec16>(wB, a.N, nb, f0, seg0 / kSegBlocks, nbs, nfeat, wlds[kMats - 1]);
    __syncthreads();
    if (!wave_live) continue;  // no feature of this wave exists (uniform over the wave)
    for (int rnd = 0; rnd < ((nbs + 3) >> 2); ++rnd) {
      // lane group g takes block seg0 + 4*rnd + g; in a last round of fewer
      // than four blocks the groups past the end multiply zeros
      const bool blk = 4 * rnd + g < nbs;
      // activations: that block, P-order positions 8i..8i+7
      bf16x8_t bop[NT][4];
      bf16x8_t bop_lo[kGateUp ? 1 : NT][4];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const size_t off = (size_t)(seg0 + 4 * rnd + g) * 32;
        const bool ld = bvalid[nt] && blk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bop[nt][i] = ld ? load_bf16x8(brow[nt] + off + 8 * i) : bf16x8_t{};
          if (!kGateUp) bop_lo[kGateUp ? 0 : nt][i] = ld ? load_bf16x8(brow_lo[nt] + off + 8 * i) : bf16x8_t{};
        }
      }
#pragma unroll
      for (int mi = 0; mi < kMats; ++mi) {
        bf16x8_t aop[4];
        decode_block(wlds[mi], lrow, rnd, g, aop);
        if (!blk)
#pragma unroll
          for (int i = 0; i < 4; ++i) aop[i] = bf16x8_t{};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            acc[mi][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[i], bop[nt][i], acc[mi][nt], 0, 0, 0);
            if (!kGateUp)
              acc[mi][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[i], bop_lo[kGateUp ? 0 : nt][i],
                                                                    acc[mi][nt], 0, 0, 0);
          }
      }
    }
  }
  if (!wave_live) return;

  // Epilogue.  Lane holds rows 4g..4g+3 (features) of column rho (token).
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int m = nt * 16 + rho;
    if (m >= tile.nrows) continue;
    const int64_t row = tile.row0 + m;
    if (kGateUp) {
      uint32_t hb[4], lb[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float gt = acc[0][nt][v], up = acc[kMats - 1][nt][v];
        const float h = gt / (1.0f + expf(-gt)) * up;
        hb[v] = f32_to_bf16_bits(h);
        lb[v] = f32_to_bf16_bits(h - __uint_as_float(hb[v] << 16));
      }
      // P-order positions 16*(wave&1) + 4g + v of I-block (f0/32 + wave/2)
      const int pos = f0 + 32 * (wave >> 1) + 16 * (wave & 1) + 4 * g;
      uint16_t* hrow = reinterpret_cast<uint16_t*>(a.out) + row * a.N;
      uint16_t* lrow_out = reinterpret_cast<uint16_t*>(a.out_lo) + row * a.N;
      *reinterpret_cast<uint2*>(hrow + pos) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
      *reinterpret_cast<uint2*>(lrow_out + pos) = make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
    } else {
      float* yrow = reinterpret_cast<float*>(a.out) + row * a.N;
      const int f = f0 + 16 * wave + 4 * g;
      *reinterpret_cast<float4*>(yrow + f) =
          make_float4(acc[0][nt][0], acc[0][nt][1], acc[0][nt][2], acc[0][nt][3]);
    }
  }
}

template <bool kGateUp>
hipError_t launch_gemm(const GemmArgs& a, int rows_per_tile, hipStream_t s) {
  const dim3 grid((unsigned)a.max_tiles, (unsigned)((a.N + kFeatPerWg - 1) / kFeatPerWg));
  const bool vec16 = ((a.K / 32) % kSegBlocks) == 0;
  const int nt = rows_per_tile / 16;
#define K3_LAUNCH(NT_, V_) hipLaunchKernelGGL((ffn_gemm_kernel<NT_, kGateUp, V_>), grid, dim3(256), 0, s, a)
  if (nt == 1) {
    if (vec16) K3_LAUNCH(1, true); else K3_LAUNCH(1, false);
  } else if (nt == 2) {
    if (vec16) K3_LAUNCH(2, true); else K3_LAUNCH(2, false);
  } else {
    if (vec16) K3_LAUNCH(4, true); else K3_LAUNCH(4, false);
  }
#undef K3_LAUNCH
  return hipGetLastError();
}

// out[t] = sum_j w[t,j] * y[slot_row[t*k+j]], in slot order.  fp32 y only:
// 4 features per thread, slots 16 at a time (all their row indices and
// weights loaded together, then all their y rows: two memory round trips per
// 16 slots, 16 reads in flight).  Rows that may hold fp16 y: 16 features per
// thread (two 16-byte reads and one scale byte per slot), slots 8 at a time
// for large batches, which keeps the thread under 128 VGPRs (four waves per
// SIMD), and 16 at a time for batches too small to fill the GPU, where the
// round trips matter more than the occupancy.
// kMixed: a slot_row entry with kBigRowFlag names a row written by the
// large-tile down kernel, which holds y as fp16 scaled by 2^y_scale[row,
// feature / 32] at the start of the row's fp32 slot.
// OutT: float, or uint16_t for bf16 outputs (rounded to nearest even).
constexpr int kCombineSlots = 16;
template <bool kMixed, int kB, typename OutT = float>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const int8_t* __restrict__ y_scale,
                                                       const int32_t* __restrict__ slot_row,
                                                       const float* __restrict__ w, int64_t T, int D, int k,
                                                       OutT* __restrict__ out) {
  constexpr int kF = kMixed ? 16 : 4;
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
  const int q = D / kF;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * q) return;
  const int64_t t = idx / q;
  const int d = (int)(idx - t * q) * kF;
  float acc[kF] = {};
  for (int j0 = 0; j0 < k; j0 += kB) {
    int32_t r[kB];
    float wj[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int j = j0 + u < k ? j0 + u : k - 1;
      r[u] = slot_row[t * k + j];
      wj[u] = w[t * k + j];
    }
    if constexpr (kMixed) {
      // rows of the large-tile kernels: raw fp16 reads for the whole batch
      // first; fp32 rows (experts served by the streaming kernels) are read
      // when their slot is summed
      f16x8_t h[kB][2];
      float fs[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const bool big = j0 + u < k && r[u] >= 0 && (r[u] & kBigRowFlag);
        if (big) {
          const int64_t row = r[u] & ~kBigRowFlag;
          const f16x8_t* src = reinterpret_cast<const f16x8_t*>(reinterpret_cast<const uint16_t*>(y + row * D) + d);
          h[u][0] = __builtin_nontemporal_load(src);
          h[u][1] = __builtin_nontemporal_load(src + 1);
          fs[u] = ldexpf(1.0f, (int)y_scale[row * (D >> 5) + (d >> 5)]);
        } else {
          h[u][0] = f16x8_t{};
          h[u][1] = f16x8_t{};
          fs[u] = 0.0f;
        }
      }
      // slot order; skipped slots add nothing; an fp32 row is read here (rare)
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (j0 + u >= k || r[u] < 0) continue;
        if (r[u] & kBigRowFlag) {
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[e] += wj[u] * ((float)h[u][e >> 3][e & 7] * fs[u]);
        } else {
          const f32x4_t* src = reinterpret_cast<const f32x4_t*>(y + (int64_t)r[u] * D + d);
#pragma unroll
          for (int c = 0; c < kF / 4; ++c) {
            const f32x4_t x4 = __builtin_nontemporal_load(src + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[4 * c + e] += wj[u] * x4[e];
          }
        }
      }
    } else {
      f32x4_t v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u)
        v[u] = j0 + u < k && r[u] >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(y + (int64_t)r[u] * D + d))
                                        : f32x4_t{};
      // slot order; skipped and out-of-range slots add nothing, whatever
      // their weight (a NaN or inf weight there must not reach the sum)
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (j0 + u >= k || r[u] < 0) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += wj[u] * v[u][e];
      }
    }
  }
  if constexpr (sizeof(OutT) == 4) {
    f32x4_t* o = reinterpret_cast<f32x4_t*>(out + t * D + d);
#pragma unroll
    for (int c = 0; c < kF / 4; ++c) o[c] = f32x4_t{acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]};
  } else {
    // kF bf16 values: 8 bytes (kF = 4) or 32 bytes (kF = 16), aligned since D % 32 == 0
    uint32_t pk[kF / 2];
#pragma unroll
    for (int c = 0; c < kF / 2; ++c)
      pk[c] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[2 * c]) |
              ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[2 * c + 1]) << 16);
    uint2* o = reinterpret_cast<uint2*>(out + t * D + d);
#pragma unroll
    for (int c = 0; c < kF / 4; ++c) o[c] = uint2{pk[2 * c], pk[2 * c + 1]};
  }
}

}  // namespace

hipError_t launch_gate_up(const GemmArgs& a, int rows_per_tile, hipStream_t s) {
  return launch_gemm<true>(a, rows_per_tile, s);
}

hipError_t launch_down(const GemmArgs& a, int rows_per_tile, hipStream_t s) {
  return launch_gemm<false>(a, rows_per_tile, s);
}

hipError_t launch_combine(const float* y, const int8_t* y_scale, bool mixed, const int32_t* slot_row, const float* w,
                          int64_t T, int D, int k, float* out, hipStream_t s) {
  const int64_t n = T * (D / (mixed ? 16 : 4));
  const int64_t blocks = (n + 255) / 256;
  // fewer threads than four waves on every SIMD of the GPU: 16-slot batches
  constexpr int64_t kFewThreads = 4 * 4 * 64 * 256;
  if (mixed && n >= kFewThreads)
    hipLaunchKernelGGL((combine_kernel<true, 8>), dim3((unsigned)blocks), dim3(256), 0, s, y, y_scale, slot_row, w, T, D,
                       k, out);
  else if (mixed)
    hipLaunchKernelGGL((combine_kernel<true, kCombineSlots>), dim3((unsigned)blocks), dim3(256), 0, s, y, y_scale,
                       slot_row, w, T, D, k, out);
  else
    hipLaunchKernelGGL((combine_kernel<false, kCombineSlots>), dim3((unsigned)blocks), dim3(256), 0, s, y, y_scale,
                       slot_row, w, T, D, k, out);
  return hipGetLastError();
}

hipError_t launch_combine_bf16(const float* y, const int8_t* y_scale, bool mixed, const int32_t* slot_row,
                               const float* w, int64_t T, int D, int k, uint16_t* out, hipStream_t s) {
  const int64_t n = T * (D / (mixed ? 16 : 4));
  const int64_t blocks = (n + 255) / 256;
  if (mixed)
    hipLaunchKernelGGL((combine_kernel<true, 8, uint16_t>), dim3((unsigned)blocks), dim3(256), 0, s, y, y_scale,
                       slot_row, w, T, D, k, out);
  else
    hipLaunchKernelGGL((combine_kernel<false, kCombineSlots, uint16_t>), dim3((unsigned)blocks), dim3(256), 0, s, y,
                       y_scale, slot_row, w, T, D, k, out);
  return hipGetLastError();
}

int choose_rows_per_tile(int64_t T, int k, int E) {
  const int64_t entries = T * k;
  const int64_t active = entries < E ? entries : E;
  const int64_t avg = active > 0 ? entries / active : 0;
  if (avg >= 48) return 64;
  if (avg >= 24) return 32;
  return 16;
}

}  // namespace k3moe
