// Large-tile grouped GEMMs for batches in which experts receive many tokens
// (prefill-sized batches).  Same arithmetic as ffn.hip (bf16 MFMA with the
// MXFP4 block scale folded into the exact fp4 -> bf16 conversion, fp32
// accumulation, h carried as a bf16 hi + lo pair); only the work decomposition
// differs.
//
// A workgroup of 8 waves (4 along features x 2 along tokens) owns an output
// tile of kF features x kN tokens of one expert and walks K in steps of 128
// (four MXFP4 blocks).  Each step is double-buffered in LDS and filled with
// direct global -> LDS loads, so staging costs no VGPRs:
//   weights:     kMats * kF rows x 68 bytes (the four 17-byte ggml blocks of
//                the row, exactly as stored), one dword per lane per load;
//   activations: kSrc * kN rows x 256 bytes (+16 bytes of padding so the 16
//                tokens a ds_read_b128 touches fall in distinct banks).
// A lane (row rho, lane group g) owns block g of the step for its row: it pulls
// the block's exponent byte and 16 qs bytes out of the raw row once per step
// and converts one qs dword per MFMA slice.
//
// gate/up: kF = 256 features of w1 and of w3, kN = 128 tokens; wave tile
//          64 features x 64 tokens for both matrices.  Weight rows are placed
//          so each lane's four outputs are four consecutive P-order positions of
//          h (8-byte stores of h_hi and h_lo).
// down:    kF = 512 features of w2, kN = 64 tokens; wave tile 128 x 32; the B
//          operand is h_hi and h_lo (two MFMAs per decoded weight operand).
//
// Workgroups are numbered so that those the hardware sends to the same XCD
// (consecutive ids round-robin over 8 XCDs) take a contiguous range of the
// logical work order, which keeps the tiles that share weights (gate/up) or
// activations (down) in one L2.
#include "k3moe_internal.h"

#include <math.h>

namespace k3moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kKStep = 128;     // K per stage (4 MXFP4 blocks)
constexpr int kWRowDw = 17;     // LDS dwords per weight row per stage (68 bytes)
constexpr int kARowDw = 68;     // LDS dwords per activation row per stage (256 + 16 bytes)
constexpr int kARowChunks = 17; // 16-byte chunks per activation row (16 data + 1 pad)
constexpr int kXcds = 8;

template <bool kGateUp>
struct BigCfg;
template <>
struct BigCfg<true> {
  static constexpr int kF = 256, kN = 128, kRG = 4, kTG = 4, kMats = 2, kSrc = 1;
};
template <>
struct BigCfg<false> {
  static constexpr int kF = 512, kN = 64, kRG = 8, kTG = 2, kMats = 1, kSrc = 2;
};

constexpr int kWDw = 2 * 256 * kWRowDw;        // weight dwords per stage (both variants: 512 rows)
constexpr int kADw = 128 * kARowDw;            // activation dwords per stage (both variants: 128 rows)
constexpr int kStageDw = kWDw + kADw;          // 17408 dwords = 69632 bytes

__device__ __forceinline__ int p_to_elem(int p) { return 16 * (p & 1) + 4 * (p >> 3) + ((p >> 1) & 3); }

__device__ __forceinline__ float e8m0_to_f32(uint32_t e) { return __uint_as_float(e ? (e << 23) : 0x00400000u); }

__device__ __forceinline__ bf16x8_t decode_dword(uint32_t q, float sf) {
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sf, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sf, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sf, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sf, 3));
  return __builtin_bit_cast(bf16x8_t, r);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Logical work index of workgroup `i` among `total` valid ones: the ids the
// hardware sends to XCD x (i % 8 == x) get the x-th contiguous slice.
__device__ __forceinline__ int64_t xcd_logical(int64_t i, int64_t total) {
  const int64_t q = total / kXcds, r = total % kXcds;
  const int64_t x = i % kXcds, j = i / kXcds;
  return x * q + (x < r ? x : r) + j;
}

template <bool kGateUp>
__global__ __launch_bounds__(kThreads) void ffn_big_kernel(GemmArgs a) {
  using C = BigCfg<kGateUp>;
  __shared__ uint32_t lds[2][kStageDw];
  __shared__ int32_t tok_src[C::kN];  // source row of every token slot of the tile

  const int n_ftiles = a.N / C::kF;
  const int64_t total = (int64_t)(*a.tile_count) * n_ftiles;
  const int64_t wg = blockIdx.x;
  if (wg >= total) return;  // uniform over the workgroup
  const int64_t logical = xcd_logical(wg, total);
  // gate/up: consecutive logical ids walk the token tiles of one feature tile
  // (they share weights); down: they walk the feature tiles of one token tile
  // (they share the h rows).
  int64_t tile_idx;
  int ftile;
  if (kGateUp) {
    const int64_t ntiles = *a.tile_count;
    // order: feature tile major within runs of the same expert is not known
    // here, so take token tiles fastest inside each feature tile
    ftile = (int)(logical / ntiles);
    tile_idx = logical % ntiles;
  } else {
    tile_idx = logical / n_ftiles;
    ftile = (int)(logical % n_ftiles);
  }
  const Tile tile = a.tiles[tile_idx];
  const int f0 = ftile * C::kF;
  const int K = a.K;
  const int nb = K >> 5;
  const size_t row_bytes = (size_t)nb * 17;
  const size_t mat_bytes = (size_t)a.N * row_bytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wf = wave & 3, wn = wave >> 2;  // 4 waves along features, 2 along tokens
  const int rho = lane & 15, g = lane >> 4;

  if (tid < C::kN) {
    const int m = tid < tile.nrows ? tid : 0;  // padding tokens repeat the first row
    const int row = tile.row0 + m;
    tok_src[tid] = kGateUp ? a.row_tok[row] : row;
  }
  __syncthreads();

  // ---- per-lane load descriptors (constant over K) ----
  // Weights: wave w fills LDS rows 64w..64w+63 (natural feature order, all of
  // one matrix); load j moves flat dword f = 64j + lane of those rows, i.e.
  // byte 4f - 68*(f/17) + (f/17)*row_bytes from the first row.
  const int wmat = (64 * wave) / C::kF;  // matrix of this wave's rows
  const int wrow0 = 64 * wave - wmat * C::kF;
  const uint8_t* wsrc = (wmat == 0 ? a.wa : a.wb) + (size_t)tile.expert * mat_bytes + (size_t)(f0 + wrow0) * row_bytes;
  const uint32_t wstride = (uint32_t)row_bytes - 4 * kWRowDw;
  // Activations: wave w fills rows 16w..16w+15 (272 flat 16-byte chunks), all
  // of one source (x / h_hi for gate/up, h_hi or h_lo for down); load j moves
  // chunk f = 64j + lane of them (row f/17, chunk f%17; chunk 16 is padding and
  // re-reads chunk 15; lanes past the 272 chunks are never issued).
  const int asrc = (16 * wave) / C::kN;
  const uint16_t* abase = (kGateUp || asrc == 0) ? a.act : a.act_lo;
  uint32_t aoffs[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int f = 64 * j + lane;
    int rl = f / kARowChunks;
    int ch = f - rl * kARowChunks;
    ch = ch > 15 ? 15 : ch;
    rl = rl > 15 ? 15 : rl;
    const int t = 16 * wave + rl - asrc * C::kN;
    aoffs[j] = (uint32_t)tok_src[t] * (uint32_t)K + 8 * ch;  // in bf16 elements
  }

  auto issue = [&](int stage, int buf) {
    uint32_t* wl = &lds[buf][0] + 64 * wave * kWRowDw;
    uint32_t* al = &lds[buf][kWDw] + 272 * 4 * wave;
    const uint8_t* wstage = wsrc + (size_t)stage * 68;
#pragma unroll
    for (int j = 0; j < kWRowDw; ++j) {
      const uint32_t f = 64 * j + lane;
      const uint32_t sl = (f * 3856u) >> 16;  // f / 17 for f < 1088
      __builtin_amdgcn_global_load_lds(wstage + 4 * f + sl * wstride, wl + 64 * j, 4, 0, 0);
    }
    const uint16_t* astage = abase + (size_t)stage * kKStep;
#pragma unroll
    for (int j = 0; j < 4; ++j) __builtin_amdgcn_global_load_lds(astage + aoffs[j], al + 256 * j, 16, 0, 0);
    if (lane < 16) __builtin_amdgcn_global_load_lds(astage + aoffs[4], al + 256 * 4, 16, 0, 0);
  };

  // LDS row (relative to the wave's feature range) feeding MFMA row rho of row
  // group rg.  gate/up: row groups (2b, 2b+1) cover I-block b of the wave and
  // MFMA row rho of half t of the block is the feature at P-order position
  // 16t + rho, so a lane's four outputs are consecutive P-order positions.
  int rrow[C::kRG];
#pragma unroll
  for (int rg = 0; rg < C::kRG; ++rg)
    rrow[rg] = kGateUp ? 32 * (rg >> 1) + p_to_elem(16 * (rg & 1) + rho) : 16 * rg + rho;

  f32x4_t acc[C::kMats][C::kRG][C::kTG];
#pragma unroll
  for (int mi = 0; mi < C::kMats; ++mi)
#pragma unroll
    for (int rg = 0; rg < C::kRG; ++rg)
#pragma unroll
      for (int tg = 0; tg < C::kTG; ++tg) acc[mi][rg][tg] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nstages = K / kKStep;
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int s = 0; s < nstages; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstages) issue(s + 1, buf ^ 1);
    const uint32_t* wl = &lds[buf][0];
    const uint32_t* al = &lds[buf][kWDw];

    // Two half-steps of two MFMA slices each.  For every (matrix, row group)
    // the lane pulls the qs dwords of block g it needs for the half (plus the
    // block's exponent byte) out of the raw 17-byte layout.
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t q[C::kMats][C::kRG][2];
      float sf[C::kMats][C::kRG];
#pragma unroll
      for (int mi = 0; mi < C::kMats; ++mi)
#pragma unroll
        for (int rg = 0; rg < C::kRG; ++rg) {
          const int slot = mi * C::kF + wf * (C::kRG * 16) + rrow[rg];
          const uint32_t* L = wl + slot * kWRowDw + 4 * g;  // block g: dword 4g, byte g
          const uint32_t d0 = L[0];
          const uint32_t da = L[2 * half], db = L[2 * half + 1], dc = L[2 * half + 2];
          sf[mi][rg] = e8m0_to_f32(__builtin_amdgcn_ubfe(d0, 8 * g, 8));
          // qs dword i = bytes g+1+4i .. g+4+4i of the block's dwords
          const int sh = (g + 1) & 3;
          const bool whole = g == 3;  // qs starts on a dword boundary
          q[mi][rg][0] = whole ? db : __builtin_amdgcn_alignbyte(db, da, sh);
          q[mi][rg][1] = whole ? dc : __builtin_amdgcn_alignbyte(dc, db, sh);
        }
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * half + ii;
        // activations: block g of the step, P-order positions 8i..8i+7 (chunk 4g+i)
        bf16x8_t bop[C::kSrc][C::kTG];
#pragma unroll
        for (int src = 0; src < C::kSrc; ++src)
#pragma unroll
          for (int tg = 0; tg < C::kTG; ++tg) {
            const int row = src * C::kN + wn * (C::kTG * 16) + tg * 16 + rho;
            bop[src][tg] =
                __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(al + row * kARowDw + 4 * (4 * g + i)));
          }
#pragma unroll
        for (int mi = 0; mi < C::kMats; ++mi)
#pragma unroll
          for (int rg = 0; rg < C::kRG; ++rg) {
            const bf16x8_t aop = decode_dword(q[mi][rg][ii], sf[mi][rg]);
#pragma unroll
            for (int src = 0; src < C::kSrc; ++src)
#pragma unroll
              for (int tg = 0; tg < C::kTG; ++tg)
                acc[mi][rg][tg] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop[src][tg], acc[mi][rg][tg], 0, 0, 0);
          }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- epilogue ----
#pragma unroll
  for (int tg = 0; tg < C::kTG; ++tg) {
    const int m = wn * (C::kTG * 16) + tg * 16 + rho;
    if (m >= tile.nrows) continue;
    const int64_t row = tile.row0 + m;
#pragma unroll
    for (int rg = 0; rg < C::kRG; ++rg) {
      if (kGateUp) {
        uint32_t hb[4], lb[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gt = acc[0][rg][tg][v], up = acc[C::kMats - 1][rg][tg][v];
          const float h = gt / (1.0f + expf(-gt)) * up;
          hb[v] = f32_to_bf16_bits(h);
          lb[v] = f32_to_bf16_bits(h - __uint_as_float(hb[v] << 16));
        }
        const int pos = f0 + 64 * wf + 32 * (rg >> 1) + 16 * (rg & 1) + 4 * g;
        uint16_t* hrow = reinterpret_cast<uint16_t*>(a.out) + row * a.N;
        uint16_t* lrow = reinterpret_cast<uint16_t*>(a.out_lo) + row * a.N;
        *reinterpret_cast<uint2*>(hrow + pos) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        *reinterpret_cast<uint2*>(lrow + pos) = make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
      } else {
        float* yrow = reinterpret_cast<float*>(a.out) + row * a.N;
        const int f = f0 + 128 * wf + 16 * rg + 4 * g;
        *reinterpret_cast<float4*>(yrow + f) =
            make_float4(acc[0][rg][tg][0], acc[0][rg][tg][1], acc[0][rg][tg][2], acc[0][rg][tg][3]);
      }
    }
  }
}

}  // namespace

bool big_gemm_supported(int D, int I) { return (I % BigCfg<true>::kF) == 0 && (D % BigCfg<false>::kF) == 0; }

int big_rows_per_tile(bool gate_up) { return gate_up ? BigCfg<true>::kN : BigCfg<false>::kN; }

hipError_t launch_big_gate_up(const GemmArgs& a, hipStream_t s) {
  const int64_t grid = a.max_tiles * (a.N / BigCfg<true>::kF);
  hipLaunchKernelGGL(ffn_big_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_big_down(const GemmArgs& a, hipStream_t s) {
  const int64_t grid = a.max_tiles * (a.N / BigCfg<false>::kF);
  hipLaunchKernelGGL(ffn_big_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace k3moe
