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
//   tile kernel   (more than 16 tokens): 128 tokens x 128 features per
//                 workgroup of 4 waves (64 x 64 each: 2 x 2 MFMA 32x32x16
//                 bf16 blocks), K in steps of 64 double-buffered in LDS and
//                 filled by direct global -> LDS buffer loads; the eight
//                 16-byte chunks of a 128-byte LDS row are XOR-swizzled by
//                 (row / 2) % 8 so that an operand read (32 rows, one chunk
//                 each) meets no bank conflict.  Workgroups go to XCDs in
//                 contiguous runs of a grouped order (8 feature tiles x every
//                 token tile), so tiles that share operands share an L2.
//                 Split-K when the tiles alone cannot fill the GPU.
//   stream kernel (up to 16 tokens): bound by the weight stream.  16 features
//                 x 16 tokens x all of K per workgroup, each wave streaming a
//                 contiguous quarter of the 16 weight rows through its own
//                 4-stage LDS ring (3 K steps in flight), the quarters added
//                 through LDS in wave order.
// Splits of the tile kernel write partial sums that the consumer adds in
// split order, so every result is deterministic.
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
constexpr int kStreamRows = 16;         // features and tokens of a stream-kernel workgroup
constexpr int kXcds = 8;
constexpr int kTargetGroups = 512;      // workgroups that fill the GPU (2 per CU)

// Logical work index of workgroup i among `total`: the ids the hardware sends
// to XCD x (i % 8 == x) take the x-th contiguous run of the logical order.
__device__ __forceinline__ int64_t xcd_order(int64_t i, int64_t total) {
  const int64_t q = total / kXcds, r = total % kXcds;
  const int64_t x = i % kXcds, j = i / kXcds;
  return x * q + (x < r ? x : r) + j;
}

// The N segment holding the tile that starts at virtual feature n0
// (segments start at multiples of the tile width, so a tile never straddles
// two).  Fields are picked with constant indices, so they stay in scalar
// registers (an index computed at run time would send the argument struct to
// memory and load it with vector loads, whose waits also drain the weight
// loads in flight).
struct SegView {
  const uint16_t* w[2];
  int64_t ldw[2];
  int rows, base;
};
__device__ __forceinline__ SegView seg_view(const DenseGemmArgs& a, int n0) {
  SegView v{{a.w[0][0], a.w[0][1]}, {a.ldw[0][0], a.ldw[0][1]}, a.rows[0], a.base[0]};
#pragma unroll
  for (int i = 1; i < kDenseMaxSeg; ++i)
    if (i < a.nseg && n0 >= a.base[i]) v = SegView{{a.w[i][0], a.w[i][1]}, {a.ldw[i][0], a.ldw[i][1]}, a.rows[i], a.base[i]};
  return v;
}

__device__ __forceinline__ uint16_t bf16_bits(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

// LDS byte offset of 16-byte chunk c of row r of an operand tile.
__device__ __forceinline__ int swz(int r, int c) { return r * kRowB + ((c ^ (r & 7)) << 4); }
// The tile kernel's operand reads (lanes 0-31: rows r..r+31 at chunk c, lanes
// 32-63: the same rows at chunk c + 1) meet no bank conflict when the key is
// (r / 2) % 8; with r % 8 rows r and r + 8 of a 16-lane group share banks
// (measured on gfx950 with the LDS conflict counters).
__device__ __forceinline__ int swz_tile(int r, int c) { return r * kRowB + ((c ^ ((r >> 1) & 7)) << 4); }

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

// kProduct (1 or 2) only names the block's first or second product, so that
// profiles list the two separately.
template <int kProduct>
__global__ __launch_bounds__(kThreads, 2) void dense_tile_kernel(DenseGemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2 * kOpB];  // [buffer][weights | tokens]
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  const SegView sv = seg_view(a, n0);
  const int f0 = n0 - sv.base;
  const int frows = sv.rows - f0 < kTile ? sv.rows - f0 : kTile;  // >= 1
  const int64_t t0 = tt * kTile;
  const int trows = a.T - t0 < kTile ? (int)(a.T - t0) : kTile;
  const int ktot = a.ksteps[0] + a.ksteps[1];
  const int kbeg = split * a.split_steps;
  const int kend = kbeg + a.split_steps < ktot ? kbeg + a.split_steps : ktot;

  // per-lane load offsets of the 4 row groups this wave fills (rows
  // r = 32*wave + 8j + lane/8, the chunk that lands at position lane%8, i.e.
  // chunk (lane%8) ^ ((r/2) % 8) with (r/2) % 8 = (4j + lane/16) % 8)
  const int lrow = 32 * wave + (lane >> 3);
  uint32_t woff[2][4], aoff[2][4];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lchunk = (lane & 7) ^ ((4 * j + (lane >> 4)) & 7);
      woff[ks][j] = (uint32_t)((lrow + 8 * j) * sv.ldw[ks] * 2 + 16 * lchunk);
      aoff[ks][j] = (uint32_t)((lrow + 8 * j) * a.lda[ks] * 2 + 16 * lchunk);
    }

  auto issue = [&](int k, int buf) {
    const int ks = k < a.ksteps[0] ? 0 : 1;
    const int kin = k - (ks ? a.ksteps[0] : 0);
    const uint16_t* wb = (ks ? sv.w[1] : sv.w[0]) + (int64_t)f0 * (ks ? sv.ldw[1] : sv.ldw[0]);
    const uint16_t* ab = (ks ? a.a[1] : a.a[0]) + t0 * (ks ? a.lda[1] : a.lda[0]);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)wb, 0, (int)(frows * (ks ? sv.ldw[1] : sv.ldw[0]) * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t ar =
        __builtin_amdgcn_make_buffer_rsrc((void*)ab, 0, (int)(trows * (ks ? a.lda[1] : a.lda[0]) * 2), 0x00020000);
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
        wf[i] = *reinterpret_cast<const bf16x8_t*>(wl + swz_tile(64 * fm + 32 * i + l32, c));
        af[i] = *reinterpret_cast<const bf16x8_t*>(al + swz_tile(64 * tm + 32 * i + l32, c));
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

// A step's operands for one lane: weight and token chunks at LDS byte
// addresses a0 and a1 (tokens 2 KB further).  The reads and their wait are one
// asm block: written as plain loads, the compiler would order them behind
// every global -> LDS load in flight and empty the ring each step.
__device__ __forceinline__ void read_step(uint32_t a0, uint32_t a1, bf16x8_t& w0, bf16x8_t& x0, bf16x8_t& w1,
                                          bf16x8_t& x1) {
  asm volatile(
      "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:2048\n\t"
      "ds_read_b128 %2, %5\n\tds_read_b128 %3, %5 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w0), "=&v"(x0), "=&v"(w1), "=&v"(x1)
      : "v"(a0), "v"(a1)
      : "memory");
}

// Weight-streaming product for up to 16 tokens.  A workgroup owns 16 features
// of one segment (the rows of MFMA 16x16x32 blocks) and every token; its 4
// waves take every fourth 64-wide K step (wave w: steps w, w + 4, ...), so at
// any time the workgroup reads 512 contiguous bytes of each of its rows (HBM
// serves that better than four separate 128-byte streams per row), with
// nontemporal weight loads (read once per call).  Every wave has its own ring
// of kRing stages in LDS (one
// 64-wide K step: 16 weight rows and 16 token rows of 128 bytes, chunks
// XOR-swizzled by row) filled by direct global -> LDS loads, and waits for a
// stage with an explicit count of the loads issued after it, so kRing - 1
// steps stay in flight (no barrier in the loop).  Rows past the edge re-read
// the last valid row (their outputs are never stored); the tail re-reads its
// last step, so every stage has the same 4 loads.  The two MFMAs of a step
// take chunks 2g and 2g + 1 for lane group g (the same K order on both
// operands).  The four partial sums are added in wave order through LDS.
template <int kProduct>
__global__ __launch_bounds__(kThreads, 2) void dense_stream_kernel(DenseGemmArgs a) {
  constexpr int kRing = 4;
  constexpr int kStageB = 2 * kStreamRows * kRowB;  // 4 KB: weights, then tokens
  __shared__ __attribute__((aligned(16))) uint8_t ring[4][kRing][kStageB];
  __shared__ f32x4_t red[4][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int n0 = blockIdx.x * kStreamRows;
  const SegView sv = seg_view(a, n0);
  const int f0 = n0 - sv.base;
  const int frows = sv.rows - f0 < kStreamRows ? sv.rows - f0 : kStreamRows;
  if (frows <= 0) return;  // a tile in the padding after a segment (uniform over the workgroup)
  const int64_t t0 = (int64_t)blockIdx.y * kStreamRows;
  const int trows = a.T - t0 < kStreamRows ? (int)(a.T - t0) : kStreamRows;
  const int ktot = a.ksteps[0] + a.ksteps[1];
  const int nst = ktot > wave ? (ktot - wave + 3) / 4 : 0;  // steps wave, wave + 4, ... below ktot
  const int last = nst > 0 ? nst - 1 : 0;

  // load j (0, 1) of an operand moves rows 8j .. 8j+7: lane -> row 8j + lane/8,
  // the chunk that lands at position lane % 8
  const int chunk = (lane & 7) ^ (lane >> 3);
  uint32_t woff[2][2], xoff[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * j + (lane >> 3);
    const int wr = r < frows ? r : frows - 1, xr = r < trows ? r : trows - 1;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      woff[ks][j] = (uint32_t)(wr * sv.ldw[ks] * 2 + 16 * chunk);
      xoff[ks][j] = (uint32_t)(xr * a.lda[ks] * 2 + 16 * chunk);
    }
  }
  // buffer resources of both K segments (built once)
  const __amdgpu_buffer_rsrc_t wrs0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(sv.w[0] + (int64_t)f0 * sv.ldw[0]), 0, (int)(frows * sv.ldw[0] * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t wrs1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(sv.w[1] + (int64_t)f0 * sv.ldw[1]), 0, (int)(frows * sv.ldw[1] * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.a[0] + t0 * a.lda[0]), 0, (int)(trows * a.lda[0] * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.a[1] + t0 * a.lda[1]), 0, (int)(trows * a.lda[1] * 2), 0x00020000);
  const int ks0 = a.ksteps[0];
  auto issue = [&](int i) {
    const int k = wave + 4 * (i < last ? i : last);
    const int ks = k < ks0 ? 0 : 1;
    const int kin = k - (ks ? ks0 : 0);
    const __amdgpu_buffer_rsrc_t wr = ks ? wrs1 : wrs0;
    const __amdgpu_buffer_rsrc_t xr = ks ? xrs1 : xrs0;
    uint8_t* st = ring[wave][i & (kRing - 1)];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, st + 8 * j * kRowB, 16, ks ? woff[1][j] : woff[0][j], kin * kRowB,
                                               0, 2 /* nontemporal */);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, st + (kStreamRows + 8 * j) * kRowB, 16,
                                               ks ? xoff[1][j] : xoff[0][j], kin * kRowB, 0, 0);
  };

  // operand offsets in a stage: row l16, chunks 2g and 2g + 1
  const uint32_t op0 = (uint32_t)swz(l16, 2 * g), op1 = (uint32_t)swz(l16, 2 * g + 1);
  static_assert(kStreamRows * kRowB == 2048, "token rows start 2 KB into a stage");
  f32x4_t acc = f32x4_t{};
  if (nst > 0) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) issue(i);
    for (int i = 0; i < nst; ++i) {
      // stage i has landed once at most the (kRing - 1) later stages' 4 loads each are in flight
      asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
      const uint32_t st = (uint32_t)(uintptr_t)ring[wave][i & (kRing - 1)];
      bf16x8_t w0, x0, w1, x1;
      read_step(st + op0, st + op1, w0, x0, w1, x1);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, x0, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, x1, acc, 0, 0, 0);
      issue(i + kRing);
    }
    // no load may still be landing in this workgroup's LDS when it exits
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  static_assert(kRing == 4, "the wait count above assumes 3 later stages of 4 loads");
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  const f32x4_t sum = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
  // lane holds token l16, features 4g .. 4g+3
  const int f = 4 * g;
  if (l16 < trows && f < frows) {
    float* dst = a.p + (t0 + l16) * a.NV + n0 + f;
    if (frows - f >= 4) {
      *reinterpret_cast<f32x4_t*>(dst) = sum;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (u < frows - f) dst[u] = sum[u];
    }
  }
}

// Block epilogue, first half: one thread per column of the logits, the latent
// and the shared expert, for a.tok_per_wg consecutive tokens (1 for small
// batches, so they spread over more workgroups).  Sums the split partials;
// writes z, the raw latent d (fp32) and the shared expert's h; each workgroup
// also writes, per token, the sum of squares of its latent columns (0 if it
// has none).
constexpr int kMidTok = 8;  // most tokens per workgroup
__global__ __launch_bounds__(kThreads) void block_cols_kernel(BlockMidArgs a) {
  __shared__ float red[kMidTok][kThreads / 64];
  const int tid = threadIdx.x;
  const int c = blockIdx.y * kThreads + tid;  // column blocks on y (a few hundred at most), token chunks on x
  const int64_t sstride = a.T * a.NV;
  const int64_t tb = (int64_t)blockIdx.x * a.tok_per_wg;
  const int nt = a.T - tb < a.tok_per_wg ? (int)(a.T - tb) : a.tok_per_wg;
  for (int u = 0; u < nt; ++u) {
    const int64_t t = tb + u;
    const float* row = a.p + t * a.NV;
    auto col = [&](int cc) {
      float v = 0.0f;
      for (int sp = 0; sp < a.splits; ++sp) v += row[sp * sstride + cc];
      return v;
    };
    float sq = 0.0f;
    if (c < a.E) {
      a.z[t * a.E + c] = col(a.base_z + c);
    } else if (c < a.E + a.D) {
      const int r = c - a.E;
      const float d = col(a.base_d + r);
      a.dbuf[t * a.D + r] = d;
      sq = d * d;
    } else if (c < a.E + a.D + a.Is) {
      const int i = c - a.E - a.D;
      const float gt = col(a.base_g + i), uu = col(a.base_u + i);
      a.s[t * a.Is + i] = bf16_bits(gt / (1.0f + expf(-gt)) * uu);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
    if ((tid & 63) == 0) red[u][tid >> 6] = sq;
  }
  __syncthreads();
  if (tid < nt) a.ssq[(tb + tid) * a.nblk + blockIdx.y] = ((red[tid][0] + red[tid][1]) + red[tid][2]) + red[tid][3];
}

// Second half: xl = bf16(gamma * d / sqrt(mean(d^2) + eps)) for the
// workgroup's tokens.  Each token's sum of squares over its column blocks is
// reduced by 32 lanes (lane j takes blocks j, j + 32, ...; then a fixed
// butterfly), so the order never depends on timing.
__global__ __launch_bounds__(kThreads) void block_norm_kernel(BlockMidArgs a) {
  __shared__ float inv_l[kMidTok];
  const int tid = threadIdx.x;
  const int r = blockIdx.y * kThreads + tid;
  const int64_t tb = (int64_t)blockIdx.x * a.tok_per_wg;
  const int nt = a.T - tb < a.tok_per_wg ? (int)(a.T - tb) : a.tok_per_wg;
  {
    const int u = tid >> 5, j0 = tid & 31;  // 8 tokens x 32 lanes
    float part = 0.0f;
    if (u < nt)
      for (int j = j0; j < a.nblk; j += 32) part += a.ssq[(tb + u) * a.nblk + j];
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) part += __shfl_xor(part, o, 32);
    if (j0 == 0 && u < nt) inv_l[u] = 1.0f / sqrtf(part / (float)a.D + a.eps);
  }
  __syncthreads();
  if (r >= a.D) return;
  const float gm = __uint_as_float((uint32_t)a.gamma[r] << 16);
  for (int u = 0; u < nt; ++u) {
    const int64_t t = tb + u;
    a.xl[t * a.D + r] = bf16_bits(gm * (a.dbuf[t * a.D + r] * inv_l[u]));
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

hipError_t launch_dense_gemm(const DenseGemmArgs& a, int product, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const int nT = a.NV / kTile;
  if (a.T <= kDenseStreamMaxTokens) {
    if (a.splits != 1) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(a.NV / kStreamRows), (unsigned)((a.T + kStreamRows - 1) / kStreamRows));
    if (product == 1)
      hipLaunchKernelGGL(dense_stream_kernel<1>, grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL(dense_stream_kernel<2>, grid, dim3(kThreads), 0, s, a);
  } else {
    const dim3 grid((unsigned)((int64_t)nT * ((a.T + kTile - 1) / kTile) * a.splits));
    if (product == 1)
      hipLaunchKernelGGL(dense_tile_kernel<1>, grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL(dense_tile_kernel<2>, grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

int block_mid_blocks(int E, int D, int Is) { return (E + D + Is + kThreads - 1) / kThreads; }

hipError_t launch_block_mid(const BlockMidArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.tok_per_wg < 1 || a.tok_per_wg > kMidTok) return hipErrorInvalidValue;
  const unsigned tchunks = (unsigned)((a.T + a.tok_per_wg - 1) / a.tok_per_wg);
  hipLaunchKernelGGL(block_cols_kernel, dim3(tchunks, (unsigned)a.nblk), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(block_norm_kernel, dim3(tchunks, (unsigned)((a.D + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, s, a);
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
