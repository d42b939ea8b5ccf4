// Dense bf16 products and epilogues of the latent-MoE block.
//
// The llama.cpp page "model: add Kimi-K3 text model" runs K3's routed experts
// at a latent width (opening comment, "latent MoE") and lists the dense
// tensors around them — the gate with exp_probs_b, ffn_routed_down,
// ffn_routed_norm, ffn_routed_up (dry-run comment) — and a shared expert
// (review comment on shared-expert invariants).  Every dense product of the
// block has the form P = A W^T with bf16 activations A [T, K] and bf16 weights
// W [N, K] (rows K-contiguous, as a linear layer stores them), fp32 sums:
//   first product:  A = h, K = H; N segments: gate logits (E), latent down
//                   (D), shared gate (Is), shared up (Is);
//   second product: N = H; K segments: the routed latent sum (D, with
//                   ffn_routed_up) and the shared expert's h (Is, with its
//                   down matrix) — the block output is their sum.
//
// Two kernels:
//   tile kernel   (more than 64 tokens): 128 tokens x 128 features per
//                 workgroup of 4 waves (64 x 64 each: 2 x 2 MFMA 32x32x16
//                 bf16 blocks), K in steps of 64 double-buffered in LDS and
//                 filled by direct global -> LDS buffer loads; the eight
//                 16-byte chunks of a 128-byte LDS row are XOR-swizzled by the
//                 row's low 3 bits so that an operand read (32 rows, one chunk
//                 each) touches distinct banks.  Workgroups go to XCDs in
//                 contiguous runs of a grouped order (8 feature tiles x every
//                 token tile), so tiles that share operands share an L2.
//                 Split-K when the tiles alone cannot fill the GPU.
//   stream kernel (up to 64 tokens): bound by the weight stream.  128
//                 features x 32 tokens x up to 7 K steps per workgroup; each
//                 wave loads its 32 weight rows for all its steps straight
//                 into registers (64 contiguous bytes per lane and step, all in
//                 flight at once), the split's 32 token rows are staged in LDS.
// Splits write partial sums that the consumer adds in split order, so every
// result is deterministic.
#include "k3moe_internal.h"

#include <math.h>

namespace k3moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kTile = 128;              // tokens and features of a tile-kernel workgroup
constexpr int kRowB = 2 * kDenseKStep;  // bytes of one K step of a bf16 row (128)
constexpr int kOpB = kTile * kRowB;     // bytes of one operand tile per stage (16 KB)
constexpr int kStreamTok = 32;          // token rows of a stream-kernel workgroup
constexpr int kXcds = 8;
constexpr int kTargetGroups = 512;      // workgroups that fill the GPU (2 per CU)

// Logical work index of workgroup i among `total`: the ids the hardware sends
// to XCD x (i % 8 == x) take the x-th contiguous run of the logical order.
__device__ __forceinline__ int64_t xcd_order(int64_t i, int64_t total) {
  const int64_t q = total / kXcds, r = total % kXcds;
  const int64_t x = i % kXcds, j = i / kXcds;
  return x * q + (x < r ? x : r) + j;
}

// N segment of the tile starting at virtual feature n0 (segments start at
// multiples of the tile width, so a tile never straddles two).
__device__ __forceinline__ int seg_of(const DenseGemmArgs& a, int n0) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < kDenseMaxSeg; ++i)
    if (i < a.nseg && n0 >= a.base[i]) s = i;
  return s;
}

__device__ __forceinline__ uint16_t bf16_bits(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

// LDS byte offset of 16-byte chunk c of row r of an operand tile.
__device__ __forceinline__ int swz(int r, int c) { return r * kRowB + ((c ^ (r & 7)) << 4); }

// Store a lane's 4 consecutive features of one token (masked at the edges).
__device__ __forceinline__ void store4(float* dst, const f32x16_t& acc, int q, int valid) {
  if (valid >= 4) {
    *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u < valid) dst[u] = acc[4 * q + u];
  }
}

__global__ __launch_bounds__(kThreads, 2) void dense_tile_kernel(DenseGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2 * kOpB];  // [buffer][weights | tokens]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nT = a.NV / kTile;
  const int64_t tT = (a.T + kTile - 1) / kTile;
  const int64_t tiles = (int64_t)nT * tT;
  int64_t r = xcd_order(blockIdx.x, tiles * a.splits);
  const int split = (int)(r / tiles);
  r -= (int64_t)split * tiles;
  // grouped order: 8 feature tiles x every token tile, token tile outer
  const int64_t per_group = 8 * tT;
  const int grp = (int)(r / per_group);
  r -= (int64_t)grp * per_group;
  const int gn = nT - 8 * grp < 8 ? nT - 8 * grp : 8;
  const int64_t tt = r / gn;
  const int nt = 8 * grp + (int)(r - tt * gn);

  const int n0 = nt * kTile;
  const int s = seg_of(a, n0);
  const int f0 = n0 - a.base[s];
  const int frows = a.rows[s] - f0 < kTile ? a.rows[s] - f0 : kTile;  // >= 1
  const int64_t t0 = tt * kTile;
  const int trows = a.T - t0 < kTile ? (int)(a.T - t0) : kTile;
  const int ktot = a.ksteps[0] + a.ksteps[1];
  const int kbeg = split * a.split_steps;
  const int kend = kbeg + a.split_steps < ktot ? kbeg + a.split_steps : ktot;

  // per-lane load offsets of the 4 row groups this wave fills (rows
  // 32*wave + 8j + lane/8, the chunk that lands at position lane%8)
  const int lrow = 32 * wave + (lane >> 3);
  const int lchunk = (lane & 7) ^ (lane >> 3);
  uint32_t woff[2][4], aoff[2][4];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      woff[ks][j] = (uint32_t)((lrow + 8 * j) * a.ldw[s][ks] * 2 + 16 * lchunk);
      aoff[ks][j] = (uint32_t)((lrow + 8 * j) * a.lda[ks] * 2 + 16 * lchunk);
    }

  auto issue = [&](int k, int buf) {
    const int ks = k < a.ksteps[0] ? 0 : 1;
    const int kin = k - (ks ? a.ksteps[0] : 0);
    const uint16_t* wb = a.w[s][ks] + (int64_t)f0 * a.ldw[s][ks];
    const uint16_t* ab = a.a[ks] + t0 * a.lda[ks];
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void*)wb, 0, (int)(frows * a.ldw[s][ks] * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t ar =
        __builtin_amdgcn_make_buffer_rsrc((void*)ab, 0, (int)(trows * a.lda[ks] * 2), 0x00020000);
    uint8_t* lb = lds[buf];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row0 = 32 * wave + 8 * j;  // rows of this load; rows past the edge keep stale data,
      if (row0 < frows)                     // which only reaches outputs that are never stored
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, lb + row0 * kRowB, 16, ks ? woff[1][j] : woff[0][j], kin * kRowB,
                                                 0, 0);
      if (row0 < trows)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, lb + kOpB + row0 * kRowB, 16, ks ? aoff[1][j] : aoff[0][j],
                                                 kin * kRowB, 0, 0);
    }
  };

  // wave tile: features 64*fm .. +63, tokens 64*tm .. +63
  const int fm = wave & 1, tm = wave >> 1;
  const bool flive[2] = {64 * fm < frows, 64 * fm + 32 < frows};
  const bool tlive[2] = {64 * tm < trows, 64 * tm + 32 < trows};
  const int hb = lane >> 5, l32 = lane & 31;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

  issue(kbeg, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int k = kbeg; k < kend; ++k) {
    const int buf = (k - kbeg) & 1;
    if (k + 1 < kend) issue(k + 1, buf ^ 1);
    const uint8_t* wl = lds[buf];
    const uint8_t* al = lds[buf] + kOpB;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = 2 * kk + hb;
      bf16x8_t wf[2], af[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        wf[i] = *reinterpret_cast<const bf16x8_t*>(wl + swz(64 * fm + 32 * i + l32, c));
        af[i] = *reinterpret_cast<const bf16x8_t*>(al + swz(64 * tm + 32 * i + l32, c));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (flive[i] && tlive[j]) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], af[j], acc[i][j], 0, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // lane holds, for token 64*tm + 32j + l32, features 64*fm + 32i + 8q + 4hb + 0..3
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int tok = 64 * tm + 32 * j + l32;
    if (!tlive[j] || tok >= trows) continue;
    float* prow = a.p + ((int64_t)split * a.T + t0 + tok) * a.NV + n0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (!flive[i]) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = 64 * fm + 32 * i + 8 * q + 4 * hb;
        if (f < frows) store4(prow + f, acc[i][j], q, frows - f);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void dense_stream_kernel(DenseGemmArgs a) {
  constexpr int kSteps = kDenseStreamSplitSteps;
  __shared__ __attribute__((aligned(16))) uint8_t xs[kSteps][kStreamTok * kRowB];  // 28 KB
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hb = lane >> 5, l32 = lane & 31;
  const int nT = a.NV / kTile;
  const int nt = blockIdx.x % nT;
  const int split = blockIdx.x / nT;
  const int n0 = nt * kTile;
  const int s = seg_of(a, n0);
  const int f0 = n0 - a.base[s];
  const int frows = a.rows[s] - f0 < kTile ? a.rows[s] - f0 : kTile;
  const int64_t t0 = (int64_t)blockIdx.y * kStreamTok;
  const int trows = a.T - t0 < kStreamTok ? (int)(a.T - t0) : kStreamTok;
  const int ktot = a.ksteps[0] + a.ksteps[1];
  const int kbeg = split * a.split_steps;
  const int nsteps = (kbeg + a.split_steps < ktot ? kbeg + a.split_steps : ktot) - kbeg;  // 1..kSteps

  // token rows: wave w fills rows 8w .. 8w+7 of every step (rows past the
  // last token keep stale data, which only reaches outputs never stored)
  const int xrow = 8 * wave + (lane >> 3);
  const int xchunk = (lane & 7) ^ (lane >> 3);
  if (8 * wave < trows) {
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      if (i >= nsteps) break;
      const int k = kbeg + i;
      const int ks = k < a.ksteps[0] ? 0 : 1;
      const int kin = k - (ks ? a.ksteps[0] : 0);
      const uint16_t* ab = a.a[ks] + t0 * a.lda[ks];
      const __amdgpu_buffer_rsrc_t ar =
          __builtin_amdgcn_make_buffer_rsrc((void*)ab, 0, (int)(trows * a.lda[ks] * 2), 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, xs[i] + 8 * wave * kRowB, 16,
                                               (uint32_t)(xrow * a.lda[ks] * 2 + 16 * xchunk), kin * kRowB, 0, 0);
    }
  }
  // weights: lane (row l32 of the wave's 32, half hb) takes bytes 64*hb ..
  // 64*hb + 63 of every step of its row; all steps are loaded up front
  const int frow = 32 * wave + l32;
  const bool wvalid = frow < frows;
  u32x4_t wv[kSteps][4];
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int k = kbeg + i;
    const int ks = k < a.ksteps[0] ? 0 : 1;
    const int kin = k - (ks ? a.ksteps[0] : 0);
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.w[s][ks] + (int64_t)(f0 + frow) * a.ldw[s][ks] +
                                                          kin * kDenseKStep + 32 * hb);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) wv[i][kk] = (wvalid && i < nsteps) ? __builtin_nontemporal_load(src + kk) : u32x4_t{};
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // MFMA rows = the wave's 32 features, columns = the 32 tokens; the K order
  // inside a step is permuted the same way on both operands (substep kk of
  // half hb is chunk 4*hb + kk)
  f32x16_t acc = f32x16_t{};
  if (32 * wave < frows) {
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      if (i >= nsteps) break;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8_t xo = *reinterpret_cast<const bf16x8_t*>(xs[i] + swz(l32, 4 * hb + kk));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, wv[i][kk]), xo, acc, 0, 0, 0);
      }
    }
    if (l32 < trows) {
      float* prow = a.p + ((int64_t)split * a.T + t0 + l32) * a.NV + n0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = 32 * wave + 8 * q + 4 * hb;
        if (f < frows) store4(prow + f, acc, q, frows - f);
      }
    }
  }
}

// One workgroup per token: logits, RMS-normed latent, shared-expert h.
__global__ __launch_bounds__(kThreads) void block_mid_kernel(BlockMidArgs a) {
  __shared__ float red[kThreads / 64];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const float* row = a.p + t * a.NV;
  const int64_t sstride = a.T * a.NV;
  auto col = [&](int c) {
    float v = 0.0f;
    for (int sp = 0; sp < a.splits; ++sp) v += row[sp * sstride + c];
    return v;
  };
  for (int e = tid; e < a.E; e += kThreads) a.z[t * a.E + e] = col(a.base_z + e);
  float ss = 0.0f;
  for (int r = tid; r < a.D; r += kThreads) {
    const float d = col(a.base_d + r);
    ss += d * d;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float total = red[0] + red[1] + red[2] + red[3];
  const float inv = 1.0f / sqrtf(total / (float)a.D + a.eps);
  for (int r = tid; r < a.D; r += kThreads) {
    const float d = col(a.base_d + r);
    const float gm = __uint_as_float((uint32_t)a.gamma[r] << 16);
    a.xl[t * a.D + r] = bf16_bits(gm * (d * inv));
  }
  for (int i = tid; i < a.Is; i += kThreads) {
    const float g = col(a.base_g + i), u = col(a.base_u + i);
    a.s[t * a.Is + i] = bf16_bits(g / (1.0f + expf(-g)) * u);
  }
}

__global__ __launch_bounds__(kThreads) void dense_sum_kernel(const float* __restrict__ p, int splits, int64_t T, int N,
                                                             float* __restrict__ out) {
  const int64_t q = N / 4;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= T * q) return;
  const int64_t sstride = T * N;
  f32x4_t v = *reinterpret_cast<const f32x4_t*>(p + idx * 4);
  for (int sp = 1; sp < splits; ++sp) {
    const f32x4_t w = *reinterpret_cast<const f32x4_t*>(p + sp * sstride + idx * 4);
    v += w;
  }
  *reinterpret_cast<f32x4_t*>(out + idx * 4) = v;
}

}  // namespace

int dense_tile_splits(int64_t T, int NV, int ksteps) {
  const int64_t tiles = (int64_t)(NV / kTile) * ((T + kTile - 1) / kTile);
  if (tiles >= kTargetGroups) return 1;
  int splits = (int)((kTargetGroups + tiles - 1) / tiles);
  const int most = ksteps / 8 > 1 ? ksteps / 8 : 1;  // at least 8 steps per split
  return splits < most ? splits : most;
}

hipError_t launch_dense_gemm(const DenseGemmArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int nT = a.NV / kTile;
  if (a.T <= kDenseStreamMaxTokens) {
    if (a.split_steps > kDenseStreamSplitSteps) return hipErrorInvalidValue;
    const unsigned tchunks = (unsigned)((a.T + kStreamTok - 1) / kStreamTok);
    hipLaunchKernelGGL(dense_stream_kernel, dim3((unsigned)(nT * a.splits), tchunks), dim3(kThreads), 0, s, a);
  } else {
    const int64_t total = (int64_t)nT * ((a.T + kTile - 1) / kTile) * a.splits;
    hipLaunchKernelGGL(dense_tile_kernel, dim3((unsigned)total), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_block_mid(const BlockMidArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  hipLaunchKernelGGL(block_mid_kernel, dim3((unsigned)a.T), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dense_sum(const float* p, int splits, int64_t T, int N, float* out, hipStream_t s) {
  const int64_t n = T * (N / 4);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(dense_sum_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, p,
                     splits, T, N, out);
  return hipGetLastError();
}

}  // namespace k3moe
