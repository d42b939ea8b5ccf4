// Large-tile grouped GEMMs for batches in which experts receive many tokens
// (prefill-sized batches).  gate/up has the arithmetic of ffn.hip (bf16 MFMA
// with the MXFP4 block scale folded into the exact fp4 -> bf16 conversion,
// fp32 accumulation).  h leaves it as fp16 scaled by a power of two per
// (row, 256-feature slice) — 11 significant bits where ffn.hip's bf16 hi + lo
// pair needs two MFMAs per product — and the down product takes it with fp16
// MFMAs (w2 blocks converted exactly to fp16): each slice of a row is first
// multiplied by 2^(slice scale - row's largest slice scale), exact in fp16
// except far below the row's largest values, so all slices accumulate into
// one set of fp32 sums, which the epilogue multiplies by 2^(row scale).
//
// A workgroup of 8 waves owns an output tile of kF features x kN tokens of one
// expert; each wave takes kF/8 features and all kN tokens, so every weight row
// is decoded by exactly one wave.  K is walked in steps of 128
// (four MXFP4 blocks).  Each step is double-buffered in LDS and filled with
// direct global -> LDS buffer loads of 16 bytes per lane, so staging costs no
// VGPRs:
//   weights:     kMats * kF rows x 80 bytes: the 16-byte-aligned window that
//                holds the step's 68 bytes of the row (its four 17-byte ggml
//                blocks, exactly as stored) starting at byte 4*(step % 4),
//                chunk-major within each 16-row group;
//   activations: kSrc * kN rows x 256 bytes (+16 bytes of padding), the
//                row's 64-byte quarters rotated by the row (act_rot), so that
//                no operand read meets a bank conflict.
// A lane (row rho, lane group g) owns block g of the step for its row: it reads
// the two 16-byte chunks holding the block, pulls out the exponent byte and the
// 16 qs bytes, and converts one qs dword per MFMA slice (the next slice's
// conversions run between the current slice's MFMAs).  The K loop is
// unrolled by four so the window phase is a compile-time constant.
//
// gate/up: kF = 256 features of w1 and of w3, kN = 128 tokens; wave tile
//          32 features (one I-block) x 128 tokens for both matrices.  The MFMA
//          rows are assigned so each lane's four outputs are four consecutive
//          P-order positions of h (8-byte stores of the scaled fp16 h).
// down:    kF = 512 features of w2, kN = 128 tokens (batches of at least
//          16384 routed entries) or 64; wave tile 64 x kN; the B operand is
//          the rescaled fp16 h.  If any w2 block of the tile has an
//          exponent outside 104..140 (values fp16 cannot hold exactly), the
//          workgroup redoes the tile with bf16 weights and h split into an
//          exact bf16 pair (two MFMAs per operand).
//
// Token groups of 16 with no row of the tile are skipped (no activation loads,
// no MFMAs), so a tile of few rows costs about its weight traffic only.
//
// Workgroups are numbered so that those the hardware sends to the same XCD
// (consecutive ids round-robin over 8 XCDs) take a contiguous range of the
// logical work order, which keeps the tiles that share weights (gate/up) or
// activations (down) in one L2.
#include "k3moe_internal.h"

#include <math.h>

#include <type_traits>

namespace k3moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kKStep = 128;     // K per stage (4 MXFP4 blocks)
constexpr int kWRowDw = 20;     // LDS dwords per weight row per stage: an aligned 80-byte window
constexpr int kWRowChunks = 5;  // 16-byte chunks per weight row window
constexpr int kARowDw = 68;     // LDS dwords per activation row per stage (256 + 16 bytes)
constexpr int kARowChunks = 17; // 16-byte chunks per activation row (16 data + 1 pad)
constexpr int kWGroupDw = 16 * kWRowDw;  // LDS dwords of a 16-row weight group per stage (chunk-major)
constexpr int kXcds = 8;
constexpr int kMaxSlices = 64;  // 256-wide slices of I the down kernel supports (I <= 16384)
constexpr int kRescaleSpan = 64;  // down: largest slice-scale spread of a row for the rescaling K loop

// kTok: token rows of a workgroup tile.  The down product has two: 128-row
// tiles give a workgroup twice the matrix work between barriers (large
// batches), 64-row tiles give twice as many workgroups (batches whose experts
// have few rows, where the weight stream needs every CU).
template <bool kGateUp, int kTok>
struct BigCfg;
template <>
struct BigCfg<true, 128> {  // wave: 2 row groups (32 features) x 8 token groups, 2 matrices
  static constexpr int kF = 256, kN = 128, kRG = 2, kTG = 8, kMats = 2, kSrc = 1;
};
template <>
struct BigCfg<false, 128> {  // wave: 4 row groups (64 features) x 8 token groups, scaled fp16 h
  static constexpr int kF = 512, kN = 128, kRG = 4, kTG = 8, kMats = 1, kSrc = 1;
};
template <>
struct BigCfg<false, 64> {  // wave: 4 row groups (64 features) x 4 token groups, scaled fp16 h
  static constexpr int kF = 512, kN = 64, kRG = 4, kTG = 4, kMats = 1, kSrc = 1;
};

constexpr int kWDw = 2 * 256 * kWRowDw;        // weight dwords per stage (both variants: 512 rows)
constexpr int kADw = 128 * kARowDw;            // activation dwords per stage (both variants: 128 rows)
constexpr int kStageDw = kWDw + kADw;          // 18944 dwords = 75776 bytes

// LDS layouts that keep every ds_read_b128 of the K loop free of bank
// conflicts (measured on gfx950 with the LDS conflict counters: a 16-lane
// read of 16-byte pieces 272 or 80 bytes apart takes two passes; the layouts
// below take one):
//   weights:     a 16-row group of a stage is chunk-major: chunk c of row r at
//                dword 64 c + 4 r, so the 64 lanes reading chunk g of rows
//                rho (lane = rho + 16 g) read 1 KB in order;
//   activations: rows of 256 + 16 bytes; the row's four 64-byte quarters
//                rotated by act_rot(r % 16), so quarter q of row r is stored at
//                quarter (q + act_rot(r)) % 4 and chunk i of a quarter stays
//                at offset 16 i (an immediate of the read).
__device__ __forceinline__ int act_rot(int r) { return (r >> 2) & 3; }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// Both weight chunks (g and g + 1, 256 bytes apart) of the four (matrix, row
// group) pairs, as whole 16-byte reads: with separate reads the compiler
// keeps only the dwords a step's phase uses, and 4- or 8-byte reads of these
// 16-byte-strided rows meet bank conflicts.  One wait for all eight.
__device__ __forceinline__ void read_weight_chunks(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                                   u32x4_t (&c)[4][2]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:256\n\t"
      "ds_read_b128 %2, %9\n\tds_read_b128 %3, %9 offset:256\n\t"
      "ds_read_b128 %4, %10\n\tds_read_b128 %5, %10 offset:256\n\t"
      "ds_read_b128 %6, %11\n\tds_read_b128 %7, %11 offset:256\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(c[0][0]), "=&v"(c[0][1]), "=&v"(c[1][0]), "=&v"(c[1][1]), "=&v"(c[2][0]), "=&v"(c[2][1]),
        "=&v"(c[3][0]), "=&v"(c[3][1])
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
}

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

__device__ __forceinline__ f16x8_t decode_dword_f16(uint32_t q, float sf) {
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, sf, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, sf, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, sf, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, sf, 3));
  return __builtin_bit_cast(f16x8_t, r);
}

// Eight fp16 values as the exact bf16 pair hi = bf16(v), lo = v - hi.
__device__ __forceinline__ void split_f16x8(uint4 b, bf16x8_t& hi, bf16x8_t& lo) {
  const f16x8_t v = __builtin_bit_cast(f16x8_t, b);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float f = (float)v[e];
    hi[e] = (__bf16)f;
    lo[e] = (__bf16)(f - (float)hi[e]);
  }
}

// Logical work index of workgroup `i` among `total` valid ones: the ids the
// hardware sends to XCD x (i % 8 == x) get the x-th contiguous slice.
__device__ __forceinline__ int64_t xcd_logical(int64_t i, int64_t total) {
  const int64_t q = total / kXcds, r = total % kXcds;
  const int64_t x = i % kXcds, j = i / kXcds;
  return x * q + (x < r ? x : r) + j;
}

template <bool kGateUp, int kTok>
__global__ __launch_bounds__(kThreads) void ffn_big_kernel(GemmArgs a) {
  using C = BigCfg<kGateUp, kTok>;
  // One array per buffer: the compiler can then tell that the buffer being
  // read is not the one the LDS-DMA loads in flight write.  With a single
  // array it makes every read of the current buffer wait for the loads just
  // issued into the other one, which serialises loading and computing.
  __shared__ uint32_t lds0[kStageDw], lds1[kStageDw];
  __shared__ int32_t tok_src[C::kN];  // source row of every token slot of the tile
  // down: h scale of every (slice, row), rows contiguous so that the 16 rows of
  // a token group are read without bank conflicts
  __shared__ int8_t hs_l[kGateUp ? 1 : C::kN * kMaxSlices];
  __shared__ int srow_l[kGateUp ? 1 : C::kN];                 // down: largest h scale of every row
  __shared__ float red[kGateUp ? kThreads / 64 * C::kN : 1];   // gate/up: per-wave row maxima of |h|
  __shared__ int sexp[kGateUp ? C::kN : 1];                    // gate/up: h scale exponent per row

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
    // super-tiles of 8 token tiles x fb feature tiles, feature tiles fastest:
    // the workgroups of an XCD round share both the weight rows and the
    // activation rows of a super-tile, so its per-step footprint stays small
    const int64_t ntiles = *a.tile_count;
    const int fb = (n_ftiles % 4 == 0) ? 4 : (n_ftiles % 2 == 0) ? 2 : 1;
    const int fgrp = (int)(logical / (ntiles * fb));
    const int64_t L = logical - (int64_t)fgrp * ntiles * fb;
    const int64_t nfull = ntiles / 8;
    if (L < nfull * 8 * fb) {
      tile_idx = (L / (8 * fb)) * 8 + (L % (8 * fb)) / fb;
      ftile = fgrp * fb + (int)(L % fb);
    } else {
      const int64_t L2 = L - nfull * 8 * fb;
      tile_idx = nfull * 8 + L2 / fb;
      ftile = fgrp * fb + (int)(L2 % fb);
    }
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
  const int rho = lane & 15, g = lane >> 4;

  if (tid < C::kN) {
    const int m = tid < tile.nrows ? tid : 0;  // rows past the tile repeat the first row
    const int row = tile.row0 + m;
    tok_src[tid] = kGateUp ? a.row_tok[row] : row;
  }
  if constexpr (!kGateUp) {
    const int nsl = K >> 8;  // 256-wide slices of h
    for (int i = tid; i < C::kN * nsl; i += kThreads) {
      const int m = i / nsl, sl = i - m * nsl;
      hs_l[sl * C::kN + m] = m < tile.nrows ? a.h_scale[(int64_t)(tile.row0 + m) * nsl + sl] : (int8_t)0;
    }
  }
  __syncthreads();
  // down: true when every row's slice scales lie within kRescaleSpan of its
  // largest (always, for h a gated MLP produces): the K loop then reads h as
  // stored and rescales the fp32 sums at each slice boundary instead
  bool rescale = false;
  if constexpr (!kGateUp) {
    int spread = 0;
    if (tid < C::kN) {
      const int nsl = K >> 8;
      int mx = -128, mn = 127;
      for (int sl = 0; sl < nsl; ++sl) {
        const int v = hs_l[sl * C::kN + tid];
        mx = max(mx, v);
        mn = min(mn, v);
      }
      srow_l[tid] = mx;
      spread = mx - mn;
    }
    rescale = !__syncthreads_or(spread > kRescaleSpan ? 1 : 0);
    // srow_l is read after the barrier that follows the first stage's loads
  }

  // ---- per-lane load descriptors (constant over K) ----
  // All loads are buffer loads straight into LDS: an SGPR resource per source,
  // a per-lane byte offset fixed for the whole kernel, and the K step in the
  // scalar offset.  Out-of-range offsets would read zeros instead of faulting.
  //
  // Weights: loader wave w fills LDS rows 64w..64w+63 (four 16-row groups),
  // all of one matrix; load j moves 16-byte chunk t = 64j + lane of them, in
  // the chunk-major order of each group (group t/80, chunk (t%80)/16, row
  // t%16).  LDS rows are in consumer order: row (mi, consumer wave, row
  // group, rho).
  const int wmat = (64 * wave) / C::kF;  // matrix of the rows this wave loads
  const int wrow0 = 64 * wave - wmat * C::kF;
  const uint8_t* wmat_base = (wmat == 0 ? a.wa : a.wb) + (size_t)tile.expert * mat_bytes + (size_t)f0 * row_bytes;
  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)wmat_base, 0, (int)(C::kF * row_bytes), 0x00020000);
  uint32_t woffs[kWRowChunks];
#pragma unroll
  for (int j = 0; j < kWRowChunks; ++j) {
    const int t = 64 * j + lane;
    const int grp = t / (16 * kWRowChunks), q = t - grp * (16 * kWRowChunks);
    const int sl = 16 * grp + (q & 15), ch = q >> 4;
    const int r_tile = wrow0 + sl;                   // LDS row within the matrix tile
    const int cw = r_tile / (C::kRG * 16);           // consumer wave
    const int r = r_tile - cw * (C::kRG * 16);       // (row group, rho) within the consumer wave
    const int feat_in_wave = kGateUp ? p_to_elem(r) : r;
    // stage-tiled weights (tiled_block_index; N and nb multiples of 16):
    // row f of the tile is row f % 16 of group f / 16, 272 bytes per row in
    // a stage; the K step adds its stage's offset in the scalar offset
    const int f = cw * (C::kRG * 16) + feat_in_wave;
    woffs[j] = (uint32_t)((f >> 4) * 16 * row_bytes) + (uint32_t)(f & 15) * 272u + 16 * ch;
  }
  // Activations: wave w fills rows 16w..16w+15 (272 flat 16-byte chunks), all
  // of one source (x / h_hi for gate/up, h_hi or h_lo for down); load j moves
  // LDS chunk f = 64j + lane of them (row f/17, stored position p = f%17,
  // which holds chunk 4 ((p/4 - act_rot(row)) % 4) + p%4 of the row; position
  // 16 is padding and re-reads chunk 15; lanes past the 272 chunks are never
  // issued).
  const int asrc = (16 * wave) / C::kN;
  const uint16_t* abase = (kGateUp || asrc == 0) ? a.act : a.act_lo;
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)abase, 0, (int)(a.act_rows * (size_t)K * 2), 0x00020000);
  uint32_t aoffs[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const int f = 64 * j + lane;
    int rl = f / kARowChunks;
    int p = f - rl * kARowChunks;
    rl = rl > 15 ? 15 : rl;
    const int ch = p > 15 ? 15 : 4 * (((p >> 2) - act_rot(rl)) & 3) + (p & 3);
    const int t = 16 * wave + rl - asrc * C::kN;
    aoffs[j] = ((uint32_t)tok_src[t] * (uint32_t)K + 8 * ch) * 2;  // bytes
  }

  // Token groups of 16 that hold rows of this tile (the others are skipped:
  // no activation loads, no MFMAs; their output columns are never stored).
  const int ntg = __builtin_amdgcn_readfirstlane((tile.nrows + 15) >> 4);
  const bool aload = asrc < C::kSrc && 16 * wave - asrc * C::kN < 16 * ntg;  // this wave's rows are live

  auto issue = [&](int stage, int buf) {
    uint32_t* const lb = buf ? lds1 : lds0;
    uint32_t* wl = lb + 64 * wave * kWRowDw;
    uint32_t* al = lb + kWDw + 16 * kARowDw * wave;  // 272 chunks per wave
    // 16-byte aligned start of the step's 68 bytes: byte 68 * (stage % 4) of
    // the row's 272 bytes in 512-wide stage stage / 4 (4352 bytes per stage)
    const int wso = 4352 * (stage >> 2) + 64 * (stage & 3);
#pragma unroll
    for (int j = 0; j < kWRowChunks; ++j) __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc, wl + 256 * j, 16, woffs[j], wso, 0, 0);
    if (aload) {
      const int aso = stage * kKStep * 2;
#pragma unroll
      for (int j = 0; j < 4; ++j) __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, al + 256 * j, 16, aoffs[j], aso, 0, 0);
      if (lane < 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, al + 256 * 4, 16, aoffs[4], aso, 0, 0);
    }
  };

  // LDS dword of chunk g of the window of MFMA row rho of row group rg (block g
  // of the step lies in chunks g and g+1, 64 dwords apart).
  int wrow_dw[C::kMats][C::kRG];
#pragma unroll
  for (int mi = 0; mi < C::kMats; ++mi)
#pragma unroll
    for (int rg = 0; rg < C::kRG; ++rg)
      wrow_dw[mi][rg] = ((mi * C::kF + wave * (C::kRG * 16)) / 16 + rg) * kWGroupDw + 64 * g + 4 * rho;
  // LDS dword of this lane's activation chunk 4g (quarter g) in token group 0;
  // chunk 4g + i adds 4 i, token group n adds 16 * kARowDw * n
  const int aread_dw = rho * kARowDw + 16 * ((g + act_rot(rho)) & 3);
  // block g starts at byte 4*phase + g of chunk g; its qs dword i is bytes
  // g+1..g+4 of the dword pair (phase+i, phase+i+1) of the two chunks
  const uint32_t qsel = 0x03020100u + 0x01010101u * (uint32_t)(g + 1);

  f32x4_t acc[C::kMats][C::kRG][C::kTG];
#pragma unroll
  for (int mi = 0; mi < C::kMats; ++mi)
#pragma unroll
    for (int rg = 0; rg < C::kRG; ++rg)
#pragma unroll
      for (int tg = 0; tg < C::kTG; ++tg) acc[mi][rg][tg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // down: h of token group tg in the current 256-wide slice is brought from
  // its slice scale to its row's largest scale by multiplying by hmul[tg] =
  // 2^(slice scale - row scale) <= 1 (two equal fp16 halves), so every slice
  // accumulates into the same fp32 sums, which the epilogue multiplies by
  // 2^(row scale).  The products are exact unless they fall below fp16's
  // normal range, i.e. below 2^-29 of the row's largest |h|.
  uint32_t hmul[kGateUp ? 1 : C::kTG];
  auto slice_mults = [&](int sl) {
#pragma unroll
    for (int tg = 0; tg < (kGateUp ? 1 : C::kTG); ++tg) {
      const int t = tg * 16 + rho;
      const int d = (int)hs_l[sl * C::kN + t] - srow_l[t];
      const uint32_t hb = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)ldexpf(1.0f, d));
      hmul[tg] = hb | (hb << 16);
    }
  };
  auto scale_h = [&](f16x8_t v, int tg) {
    const _Float16 m = __builtin_bit_cast(_Float16, (uint16_t)hmul[tg]);
    return v * m;
  };
  // Rescaling variant: the sums of token row t are kept in units of 2^(scale
  // of the slice being read); entering slice sl they are multiplied by
  // 2^(scale[sl-1] - scale[sl]), after the last slice by 2^(scale - row
  // scale), so the epilogue finds them in row-scale units as above.  The
  // factors are powers of two within 2^+-kRescaleSpan: exact, and with h below
  // 2^15 in every slice's units the sums stay far inside the fp32 range.
  auto rescale_acc = [&](int sl_from, int to_row) {
#pragma unroll
    for (int tg = 0; tg < (kGateUp ? 1 : C::kTG); ++tg) {
      const int t = tg * 16 + rho;
      const int to = to_row ? srow_l[t] : (int)hs_l[(sl_from + 1) * C::kN + t];
      const float f = ldexpf(1.0f, (int)hs_l[sl_from * C::kN + t] - to);
#pragma unroll
      for (int rg = 0; rg < C::kRG; ++rg)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[0][rg][tg][v] *= f;
    }
  };

  const int nstages = K / kKStep;

  // One K step from LDS buffer `buf` whose weight window starts at phase PH.
  // kFull: every token group of the tile is live (the unguarded fast path)
  // down: set when a wave met a w2 block the fp16 path cannot hold exactly
  bool wide_seen = false;
  auto run_stage = [&](auto ph_tag, auto full_tag, auto exact_tag, auto resc_tag, int s) {
    constexpr int PH = decltype(ph_tag)::value;
    constexpr bool kFull = decltype(full_tag)::value;
    constexpr bool kExact = decltype(exact_tag)::value;  // down: the exact bf16-pair pass
    constexpr bool kResc = decltype(resc_tag)::value;    // down, fp16 pass: rescaled sums, h read as stored
    const int buf = PH & 1;  // s % 2 == PH % 2 because s % 4 == PH
    if (s + 1 < nstages) issue(s + 1, buf ^ 1);
    const uint32_t* wl = buf ? lds1 : lds0;
    const uint32_t* al = wl + kWDw;

    // qs dwords and block exponent of block g of every (matrix, row group)
    uint32_t q[C::kMats][C::kRG][4];
    uint32_t eb[C::kMats][C::kRG];
    static_assert(C::kMats * C::kRG == 4, "four (matrix, row group) pairs per wave");
    u32x4_t wc[4][2];
    {
      const uint32_t wb = (uint32_t)(uintptr_t)wl;
      read_weight_chunks(wb + 4u * (uint32_t)wrow_dw[0][0], wb + 4u * (uint32_t)wrow_dw[(1 / C::kRG) % C::kMats][1 % C::kRG],
                         wb + 4u * (uint32_t)wrow_dw[(2 / C::kRG) % C::kMats][2 % C::kRG],
                         wb + 4u * (uint32_t)wrow_dw[(3 / C::kRG) % C::kMats][3 % C::kRG], wc);
    }
#pragma unroll
    for (int mi = 0; mi < C::kMats; ++mi)
#pragma unroll
      for (int rg = 0; rg < C::kRG; ++rg) {
        const u32x4_t c0 = wc[mi * C::kRG + rg][0], c1 = wc[mi * C::kRG + rg][1];
        const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        eb[mi][rg] = __builtin_amdgcn_ubfe(w[PH], 8 * g, 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[mi][rg][i] = __builtin_amdgcn_perm(w[PH + i + 1], w[PH + i], qsel);
      }
    constexpr int kB = C::kTG * C::kSrc;
    const int nlive = kFull ? kB : ntg * C::kSrc;  // operands of live token groups

    if constexpr (kGateUp) {
      // Slice i's weight operands are converted during slice i - 1's MFMAs
      // (one (matrix, row group) pair per token group), so the conversion
      // overlaps the matrix work instead of preceding it.
      constexpr int kPairs = C::kMats * C::kRG;
      // two operand sets used in turn (slice i reads set i % 2 and fills the
      // other), indexed by constants after unrolling, so no register copies
      bf16x8_t ops[2][kPairs];
#pragma unroll
      for (int pr = 0; pr < kPairs; ++pr)
        ops[0][pr] = decode_dword(q[pr / C::kRG][pr % C::kRG][0], e8m0_to_f32(eb[pr / C::kRG][pr % C::kRG]));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x8_t(&aop)[kPairs] = ops[i & 1];
        bf16x8_t(&anext)[kPairs] = ops[(i + 1) & 1];
        // activations: block g of the step, P-order positions 8i..8i+7 (chunk
        // 4g+i); one operand is read ahead while the previous one feeds its MFMAs
        auto bread = [&](int n) {
          return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(al + n * 16 * kARowDw + aread_dw + 4 * i));
        };
        auto convert_next = [&](int pr) {
          return decode_dword(q[pr / C::kRG][pr % C::kRG][i + 1], e8m0_to_f32(eb[pr / C::kRG][pr % C::kRG]));
        };
        bf16x8_t bnext = bread(0);
#pragma unroll
        for (int n = 0; n < kB; ++n) {
          if (!kFull && n >= nlive) break;
          const bf16x8_t bop = bnext;
          // the next operand is read even if its token group is dead (an
          // in-bounds LDS read whose value is then unused): no copy, no branch
          if (n + 1 < kB) bnext = bread(n + 1);
#pragma unroll
          for (int pr = 0; pr < kPairs; ++pr)
            acc[pr / C::kRG][pr % C::kRG][n] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[pr], bop, acc[pr / C::kRG][pr % C::kRG][n], 0, 0, 0);
          if (i + 1 < 4 && n < kPairs) anext[n] = convert_next(n);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (i + 1 < 4 && !kFull) {
#pragma unroll
          for (int pr = 0; pr < kPairs; ++pr)
            if (pr >= nlive) anext[pr] = convert_next(pr);  // fewer live token groups than pairs
        }
      }
    } else {
      if constexpr ((PH & 1) == 0) {  // the step opens a 256-wide slice of h
        if constexpr (kResc) {
          if (s > 0) rescale_acc((s >> 1) - 1, 0);
        } else {
          slice_mults(s >> 1);
        }
      }
      // fp16 holds every w2 value of a block exactly when its exponent byte is
      // in 104..140.  The fp16 pass notes any other block; the workgroup then
      // redoes the tile with the exact pass.
      if constexpr (!kExact) {
        bool wide = false;
#pragma unroll
        for (int rg = 0; rg < C::kRG; ++rg) wide |= (eb[0][rg] - 104u) > 36u;
        wide_seen |= __builtin_amdgcn_ballot_w64(wide) != 0;
        // as in gate/up, slice i's operands are converted during slice i - 1's MFMAs
        f16x8_t ops[2][C::kRG];  // used in turn, as in gate/up
#pragma unroll
        for (int rg = 0; rg < C::kRG; ++rg) ops[0][rg] = decode_dword_f16(q[0][rg][0], e8m0_to_f32(eb[0][rg]));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f16x8_t(&aop)[C::kRG] = ops[i & 1];
          f16x8_t(&anext)[C::kRG] = ops[(i + 1) & 1];
          auto bread = [&](int n) {
            const f16x8_t hv =
                __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4*>(al + n * 16 * kARowDw + aread_dw + 4 * i));
            if constexpr (kResc) return hv;
            else return scale_h(hv, n);
          };
          f16x8_t bnext = bread(0);
#pragma unroll
          for (int n = 0; n < kB; ++n) {
            if (!kFull && n >= nlive) break;
            const f16x8_t bop = bnext;
            if (n + 1 < kB) bnext = bread(n + 1);  // as in gate/up
#pragma unroll
            for (int rg = 0; rg < C::kRG; ++rg)
              acc[0][rg][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[rg], bop, acc[0][rg][n], 0, 0, 0);
            if (i + 1 < 4 && n < C::kRG) anext[n] = decode_dword_f16(q[0][n][i + 1], e8m0_to_f32(eb[0][n]));
            __builtin_amdgcn_sched_barrier(0);
          }
          if (i + 1 < 4 && !kFull) {
#pragma unroll
            for (int rg = 0; rg < C::kRG; ++rg)
              if (rg >= nlive) anext[rg] = decode_dword_f16(q[0][rg][i + 1], e8m0_to_f32(eb[0][rg]));
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x8_t aop[C::kRG];
#pragma unroll
          for (int rg = 0; rg < C::kRG; ++rg) aop[rg] = decode_dword(q[0][rg][i], e8m0_to_f32(eb[0][rg]));
#pragma unroll
          for (int n = 0; n < kB; ++n) {
            if (!kFull && n >= nlive) break;
            bf16x8_t bhi, blo;
            const f16x8_t hv =
                scale_h(__builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4*>(al + n * 16 * kARowDw + aread_dw + 4 * i)), n);
            split_f16x8(__builtin_bit_cast(uint4, hv), bhi, blo);
#pragma unroll
            for (int rg = 0; rg < C::kRG; ++rg) {
              acc[0][rg][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[rg], bhi, acc[0][rg][n], 0, 0, 0);
              acc[0][rg][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[rg], blo, acc[0][rg][n], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  auto k_loop = [&](auto full_tag, auto exact_tag, auto resc_tag) {
    for (int s = 0; s < nstages; s += 4) {
      run_stage(std::integral_constant<int, 0>{}, full_tag, exact_tag, resc_tag, s);
      if (s + 1 < nstages) run_stage(std::integral_constant<int, 1>{}, full_tag, exact_tag, resc_tag, s + 1);
      if (s + 2 < nstages) run_stage(std::integral_constant<int, 2>{}, full_tag, exact_tag, resc_tag, s + 2);
      if (s + 3 < nstages) run_stage(std::integral_constant<int, 3>{}, full_tag, exact_tag, resc_tag, s + 3);
    }
  };
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (!kGateUp && rescale) {
    if (ntg == C::kTG)
      k_loop(std::true_type{}, std::false_type{}, std::true_type{});
    else
      k_loop(std::false_type{}, std::false_type{}, std::true_type{});
    rescale_acc((K >> 8) - 1, 1);  // to row-scale units
  } else {
    if (ntg == C::kTG)
      k_loop(std::true_type{}, std::false_type{}, std::false_type{});
    else
      k_loop(std::false_type{}, std::false_type{}, std::false_type{});
  }
  if constexpr (!kGateUp) {
    if (__syncthreads_or(wide_seen ? 1 : 0)) {  // rare: w2 exponents outside 104..140
#pragma unroll
      for (int rg = 0; rg < C::kRG; ++rg)
#pragma unroll
        for (int tg = 0; tg < C::kTG; ++tg) acc[0][rg][tg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      issue(0, 0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (ntg == C::kTG)
        k_loop(std::true_type{}, std::true_type{}, std::false_type{});
      else
        k_loop(std::false_type{}, std::true_type{}, std::false_type{});
    }
  }

  // ---- epilogue ----
  if constexpr (kGateUp) {
    // h = SiLU(gate) * up, in place of the gate accumulators
#pragma unroll
    for (int rg = 0; rg < C::kRG; ++rg)
#pragma unroll
      for (int tg = 0; tg < C::kTG; ++tg)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float gt = acc[0][rg][tg][v], up = acc[1][rg][tg][v];
          acc[0][rg][tg][v] = gt / (1.0f + expf(-gt)) * up;
        }
    // Scale of each token row of this 256-feature slice: 2^s with s = the
    // exponent of max |h| minus 14, so the scaled values stay below 2^15.
    // Max over the wave's 32 features (lanes g = 0..3), then over the waves
    // through LDS.
#pragma unroll
    for (int tg = 0; tg < C::kTG; ++tg) {
      float m = 0.f;
#pragma unroll
      for (int rg = 0; rg < C::kRG; ++rg)
#pragma unroll
        for (int v = 0; v < 4; ++v) m = fmaxf(m, fabsf(acc[0][rg][tg][v]));
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      if (g == 0) red[wave * C::kN + tg * 16 + rho] = m;
    }
    __syncthreads();
    if (tid < C::kN) {
      float m = 0.f;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) m = fmaxf(m, red[w * C::kN + tid]);
      int sx = (int)((__float_as_uint(m) >> 23) & 0xFFu) - 127 - 14;
      sx = m > 0.f ? (sx < -128 ? -128 : (sx > 113 ? 113 : sx)) : 0;
      sexp[tid] = sx;
      if (tid < tile.nrows) a.h_scale[(int64_t)(tile.row0 + tid) * (a.N >> 8) + ftile] = (int8_t)sx;
    }
    __syncthreads();
#pragma unroll
    for (int tg = 0; tg < C::kTG; ++tg) {
      const int m = tg * 16 + rho;
      if (m >= tile.nrows) continue;
      const int64_t row = tile.row0 + m;
      const int sx = sexp[m];
      uint16_t* hrow = reinterpret_cast<uint16_t*>(a.out) + row * a.N;
#pragma unroll
      for (int rg = 0; rg < C::kRG; ++rg) {
        uint32_t hb[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          hb[v] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)ldexpf(acc[0][rg][tg][v], -sx));
        const int pos = f0 + 32 * wave + 16 * rg + 4 * g;
        *reinterpret_cast<uint2*>(hrow + pos) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
      }
    }
  } else {
    // y as fp16 scaled by 2^sy per (row, 32-feature group), sy = the exponent
    // of the group's max |y| minus 14 (so the scaled values stay below 2^15),
    // stored at the start of the row's fp32 slot: a group is two row groups
    // (rg = 2q, 2q + 1) of the four lane groups g.
#pragma unroll
    for (int tg = 0; tg < C::kTG; ++tg) {
      const int m = tg * 16 + rho;
      const float sc = ldexpf(1.0f, srow_l[m]);  // h's row scale
#pragma unroll
      for (int q = 0; q < C::kRG / 2; ++q) {
        float yv[2][4];
        float mx = 0.f;
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            yv[r2][v] = acc[0][2 * q + r2][tg][v] * sc;
            mx = fmaxf(mx, fabsf(yv[r2][v]));
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        int sy = (int)((__float_as_uint(mx) >> 23) & 0xFFu) - 127 - 14;
        sy = mx > 0.f ? (sy < -128 ? -128 : (sy > 113 ? 113 : sy)) : 0;
        if (m >= tile.nrows) continue;
        const int64_t row = tile.row0 + m;
        uint16_t* yrow = reinterpret_cast<uint16_t*>(reinterpret_cast<float*>(a.out) + row * a.N);
        const int fq = f0 + 64 * wave + 32 * q;  // first feature of the group
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
          uint32_t hb[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) hb[v] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)ldexpf(yv[r2][v], -sy));
          *reinterpret_cast<uint2*>(yrow + fq + 16 * r2 + 4 * g) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        }
        if (g == 0) a.y_scale[row * (a.N >> 5) + (fq >> 5)] = (int8_t)sy;
      }
    }
  }
}

}  // namespace

// Feature tiles must divide the outputs, and K must be a multiple of 4 steps
// (512) so the last 80-byte weight window of a row ends exactly at the row end.
bool big_gemm_supported(int D, int I) {
  return (I % BigCfg<true, 128>::kF) == 0 && (D % BigCfg<false, 128>::kF) == 0 && (D % (4 * kKStep)) == 0 &&
         (I % (4 * kKStep)) == 0 && I <= 256 * kMaxSlices;
}

int big_rows_per_tile(bool gate_up, bool wide_down) {
  return gate_up ? BigCfg<true, 128>::kN : wide_down ? BigCfg<false, 128>::kN : BigCfg<false, 64>::kN;
}

hipError_t launch_big_gate_up(const GemmArgs& a, hipStream_t s) {
  const int64_t grid = a.max_tiles * (a.N / BigCfg<true, 128>::kF);
  hipLaunchKernelGGL((ffn_big_kernel<true, 128>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_big_down(const GemmArgs& a, bool wide, hipStream_t s) {
  if (wide) {
    const int64_t grid = a.max_tiles * (a.N / BigCfg<false, 128>::kF);
    hipLaunchKernelGGL((ffn_big_kernel<false, 128>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  } else {
    const int64_t grid = a.max_tiles * (a.N / BigCfg<false, 64>::kF);
    hipLaunchKernelGGL((ffn_big_kernel<false, 64>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace k3moe
