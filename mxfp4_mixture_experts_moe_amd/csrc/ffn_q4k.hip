// Routed-expert GEMMs over Q4_K expert blocks.
//
// Q4_K (ggml's block_q4_K) holds 256 consecutive weights of a row in 144
// bytes: fp16 d, fp16 dmin, 12 bytes packing eight 6-bit (scale, min) pairs
// (one per 32-weight sub-block), 128 bytes of 4-bit codes (bytes 32c ..
// 32c + 31 carry sub-block 2c in their low nibbles and 2c + 1 in their high
// nibbles); weight = d * scale * code - dmin * min.  The expert tensors are
// read in ggml's own layout, [E][rows][K / 256][144].
//
// Arithmetic.  A code byte placed under the byte 0x43 is the bf16 value
// 128 + code, so one v_perm turns two codes into an exact bf16 pair, and one
// bf16 MFMA per sub-block gives t = sum (128 + code) x = sum code x + 128 Sx,
// Sx the sum of the sub-block's 32 activations.  With ds = d * scale (exact in
// fp32) and C = 128 ds + dmin * min, the sub-block's share of the dot product
// is ds t - C Sx.  ds t is four fp32 FMAs into the lane's accumulator.  The
// C Sx terms of a whole block are two fp32 16x16x4 MFMAs: Sx itself comes
// from bf16 MFMAs of an indicator operand (row r of its 16 is 1 on sub-block
// r / 4 of four) against the activations, which leaves Sx of sub-block g of
// token t in lane (t, g), the A-operand layout of the fp32 MFMA; each lane
// decodes C of sub-blocks g and g + 4 of its own feature, the B-operand
// layout of the same MFMA.  The products are exact, the sums are fp32.
//
// Work decomposition.  The path serves every batch, and is laid out for the
// few-token batches that stream the experts' weight bytes (HBM-bound):
//   - persistent, two workgroups of four waves per CU (two waves per SIMD, so
//     one wave's conversions and scaling overlap the other's MFMA and LDS
//     latencies); a unit is one tile of
//     one expert (gate/up: up to 16 token rows; down: up to 8 rows of h, as
//     h_hi rows 0-7 and h_lo rows 8-15 of the MFMA) times four waves'
//     features (gate/up: 16 features of w1 and of w3 per wave; down: 32 of
//     w2), over the whole K;
//   - a stage is one block (256 K, 144 bytes) of each of a wave's 32 weight
//     rows, copied by direct global -> LDS loads of 16 bytes per lane into the
//     wave's own ring of three stage buffers, two stages ahead of the one it
//     computes; the tile's activation rows for the same 256 K ride in a ring
//     the four waves share (each wave loads its share of the live rows), with
//     one barrier per stage;
//   - the MFMA output is 16 token rows x 16 features; rows of the tile that
//     do not exist read whatever their LDS slot holds and are never stored.
#include "k3moe_internal.h"

#include <math.h>

namespace k3moe {

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;            // waves per workgroup
constexpr int kWgPerCu = 2;          // workgroups per CU (the LDS of two fits)
constexpr int kRing = 3;             // stage buffers
constexpr int kBlkBytes = 144;       // one Q4_K block
constexpr int kStageK = 256;         // one block per row and stage
constexpr int kStageRowBytes = kBlkBytes;  // one row's share of a stage
constexpr int kRowChunks = 9;        // 16-byte chunks of it
constexpr int kMatBytes = 16 * kStageRowBytes;     // a 16-row weight block of a stage
constexpr int kMatInstr = (16 * kRowChunks + 63) / 64;  // 3 loads (the third for 16 lanes)
constexpr int kRB = 2;                             // 16-row weight blocks per wave
constexpr int kW = kRB * kMatInstr;                // weight loads per wave and stage
constexpr int kWBytes = kRB * kMatBytes;           // a wave's stage buffer
constexpr int kBRows = 16;                         // activation rows of a tile in the MFMA
constexpr int kBRowBytes = 528;                    // 512 bytes per row and stage + 16 against bank conflicts
constexpr int kA = kBRows / kWaves;                // activation rows each wave loads
constexpr int kNt = 0;                             // weights: default caching (a 144-byte piece shares cache lines with the next stage's)
static_assert(kWaves * kRing * kWBytes + kRing * kBRows * kBRowBytes <= 160 * 1024 / kWgPerCu, "LDS");
static_assert(2 * kW + kA < 64, "vmcnt range");

template <bool kGateUp>
struct Q4KCfg;
template <>
struct Q4KCfg<true> {
  static constexpr int kFeat = 16, kTileRows = 16;  // per wave: 16 features of w1 and of w3
};
template <>
struct Q4KCfg<false> {
  static constexpr int kFeat = 32, kTileRows = 8;  // per wave: 32 features of w2; rows as h_hi + h_lo
};

// Wave-uniform reads through the constant address space become scalar loads,
// which never wait behind the vector loads in flight.
template <typename T_>
__device__ __forceinline__ const __attribute__((address_space(4))) T_* as_const(const T_* p) {
  return reinterpret_cast<const __attribute__((address_space(4))) T_*>(reinterpret_cast<uintptr_t>(p));
}

// s_waitcnt vmcnt(N): at most N vector-memory operations of this wave
// outstanding; they complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <int kBase>
__device__ __forceinline__ void wait_vm_plus(int b) {
  switch (b) {
    case 0: wait_vm<kBase>(); break;
    case 1: wait_vm<kBase + 1>(); break;
    case 2: wait_vm<kBase + 2>(); break;
    case 3: wait_vm<kBase + 3>(); break;
    case 4: wait_vm<kBase + 4>(); break;
    default: wait_vm<0>(); break;
  }
}

struct Q4Tile {
  int expert, row0, nrows;
};
__device__ __forceinline__ Q4Tile load_q4_tile(const Tile* tiles, int idx) {
  const auto p = as_const(reinterpret_cast<const int32_t*>(tiles) + 4 * idx);
  return Q4Tile{p[0], p[1], p[2]};
}

// The LDS operands of one block of a stage, read in one asm block with its
// own wait (as plain loads the compiler would wait for every global -> LDS
// load in flight before them):
//   x[j]  (j = 0..7): 16 bytes of the activations of sub-block j for this
//         lane's token row (ap = row start + 16 * g; sub-block j at +64 j);
//   hd[r] (r = 0..1): the 16-byte header of the block in weight block r's
//         row of this lane (h0 / h1 = the block's first byte);
//   qd[r][c] (c = 0..3): code bytes 32c + 8g .. 32c + 8g + 7 of the same
//         block (c0 / c1 = the block's first byte + 8g; codes start at +16).
__device__ __forceinline__ void read_block_operands(uint32_t ap, uint32_t h0, uint32_t h1, uint32_t c0, uint32_t c1,
                                                    u32x4_t (&x)[8], u32x4_t (&hd)[2], u32x2_t (&qd)[2][4]) {
  asm volatile(
      "ds_read_b128 %0, %18\n\tds_read_b128 %1, %18 offset:64\n\t"
      "ds_read_b128 %2, %18 offset:128\n\tds_read_b128 %3, %18 offset:192\n\t"
      "ds_read_b128 %4, %18 offset:256\n\tds_read_b128 %5, %18 offset:320\n\t"
      "ds_read_b128 %6, %18 offset:384\n\tds_read_b128 %7, %18 offset:448\n\t"
      "ds_read_b128 %8, %19\n\tds_read_b128 %9, %20\n\t"
      "ds_read_b64 %10, %21 offset:16\n\tds_read_b64 %11, %21 offset:48\n\t"
      "ds_read_b64 %12, %21 offset:80\n\tds_read_b64 %13, %21 offset:112\n\t"
      "ds_read_b64 %14, %22 offset:16\n\tds_read_b64 %15, %22 offset:48\n\t"
      "ds_read_b64 %16, %22 offset:80\n\tds_read_b64 %17, %22 offset:112\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7]),
        "=&v"(hd[0]), "=&v"(hd[1]), "=&v"(qd[0][0]), "=&v"(qd[0][1]), "=&v"(qd[0][2]), "=&v"(qd[0][3]),
        "=&v"(qd[1][0]), "=&v"(qd[1][1]), "=&v"(qd[1][2]), "=&v"(qd[1][3])
      : "v"(ap), "v"(h0), "v"(h1), "v"(c0), "v"(c1)
      : "memory");
}

// 8 codes (one nibble per byte, in the low four bits) -> bf16 128 + code.
__device__ __forceinline__ bf16x8_t codes_to_bf16(uint32_t b0, uint32_t b1) {
  constexpr uint32_t k43 = 0x43434343u;
  u32x4_t r;
  r.x = __builtin_amdgcn_perm(k43, b0, 0x04010400u);
  r.y = __builtin_amdgcn_perm(k43, b0, 0x04030402u);
  r.z = __builtin_amdgcn_perm(k43, b1, 0x04010400u);
  r.w = __builtin_amdgcn_perm(k43, b1, 0x04030402u);
  return __builtin_bit_cast(bf16x8_t, r);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

template <bool kGateUp>
__global__ __launch_bounds__(kWaves * 64, kWgPerCu) void ffn_q4k_kernel(GemmArgs a) {
  using C = Q4KCfg<kGateUp>;
  constexpr int kTileRows = C::kTileRows;
  __shared__ __attribute__((aligned(16))) uint8_t wlds[kWaves][kRing][kWBytes];
  __shared__ __attribute__((aligned(16))) uint8_t alds[kRing][kBRows * kBRowBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int fl = lane & 15, g = lane >> 4;  // MFMA column (feature / token) and lane group
  const int ngr = a.N / C::kFeat / kWaves;   // workgroup units per tile
  const auto row_tok = as_const(a.row_tok);
  const int n_tiles = *as_const(a.tile_count);
  const int64_t n_units = (int64_t)n_tiles * ngr;
  const int64_t nwg = gridDim.x;
  const int64_t wg = blockIdx.x;
  if (wg >= n_units) return;  // uniform over the workgroup; every later barrier is reached by all waves
  const int64_t my_units = (n_units - wg + nwg - 1) / nwg;
  const int nb = a.K >> 8;                  // blocks per row
  const int nst = nb;                       // stages per unit
  const int64_t Q = my_units * nst;
  const uint32_t row_bytes = (uint32_t)nb * kBlkBytes;
  const size_t mat_bytes = (size_t)a.N * row_bytes;
  const uint32_t act_row_bytes = (uint32_t)a.K * 2;

  // per-lane source offsets of a 16-row weight block's stage: chunk c = 64 j +
  // lane is 16 bytes at row c / 9, byte 16 (c % 9) of the row's block
  uint32_t woff[kMatInstr];
#pragma unroll
  for (int j = 0; j < kMatInstr; ++j) {
    const int c = 64 * j + lane;
    const int r = c / kRowChunks, p = c - r * kRowChunks;
    woff[j] = c < 16 * kRowChunks ? (uint32_t)r * row_bytes + 16u * (uint32_t)p : 0u;
  }
  const bool wtail = lane < 16 * kRowChunks - 64 * (kMatInstr - 1);

  struct Cur {
    int64_t u;
    int s, ti, gr;
    Q4Tile tile;
  };
  const int step_ti = (int)(nwg / ngr), step_gr = (int)(nwg % ngr);
  auto load_unit = [&](Cur& c) { c.tile = load_q4_tile(a.tiles, __builtin_amdgcn_readfirstlane(c.ti)); };
  auto next_stage = [&](Cur& c) {
    if (++c.s < nst) return;
    c.s = 0;
    c.u += nwg;
    c.ti += step_ti;
    c.gr += step_gr;
    if (c.gr >= ngr) {
      c.gr -= ngr;
      ++c.ti;
    }
    if (c.u < n_units) load_unit(c);
  };

  // weight loads of cursor c's stage into stage buffer buf (this wave's rows)
  auto issue_w = [&](const Cur& c, int buf) {
    const int fg = kWaves * c.gr + wave;
    const size_t unit_off = (size_t)c.tile.expert * mat_bytes + (size_t)(C::kFeat * fg) * row_bytes;
    uint8_t* dst = &wlds[wave][buf][0];
    const uint32_t wso = (uint32_t)(kStageRowBytes * c.s);
#pragma unroll
    for (int mi = 0; mi < kRB; ++mi) {
      const uint8_t* base =
          kGateUp ? (mi == 0 ? a.wa : a.wb) + unit_off : a.wa + unit_off + (size_t)(16 * mi) * row_bytes;
      const __amdgpu_buffer_rsrc_t wr =
          __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)(16 * row_bytes), 0x00020000);
#pragma unroll
      for (int j = 0; j < kMatInstr; ++j) {
        // every load keeps at least one lane, so each one is issued and counted
        if (j < kMatInstr - 1 || wtail)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              wr, (__attribute__((address_space(3))) void*)(uintptr_t)(dst + mi * kMatBytes + 1024 * j), 16, woff[j],
              wso, 0, kNt);
      }
    }
  };
  // this wave's share (B rows 4 wave .. 4 wave + 3) of the stage's live
  // activation rows; returns how many loads it issued
  auto issue_a = [&](const Cur& c, int buf) -> int {
    uint8_t* dst = &alds[buf][0];
    const uint32_t aso = (uint32_t)(kStageK * 2 * c.s);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.act, 0, (int)((uint32_t)a.act_rows * act_row_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t lr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kGateUp ? a.act : a.act_lo), 0, (int)((uint32_t)a.act_rows * act_row_bytes), 0x00020000);
    int n = 0;
#pragma unroll
    for (int r = 0; r < kA; ++r) {
      const int m = kA * wave + r;
      const int mr = kGateUp ? m : (m < kTileRows ? m : m - kTileRows);
      if (mr < c.tile.nrows) {
        const int row = c.tile.row0 + mr;
        const int xrow = kGateUp ? row_tok[row] : row;
        const uint32_t so = (uint32_t)xrow * act_row_bytes + aso;
        if (lane < kStageK * 2 / 16) {  // 512 bytes: 32 lanes
          if (kGateUp || m < kTileRows)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (__attribute__((address_space(3))) void*)(uintptr_t)(dst + kBRowBytes * m), 16, 16 * lane, so, 0, 0);
          else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                lr, (__attribute__((address_space(3))) void*)(uintptr_t)(dst + kBRowBytes * m), 16, 16 * lane, so, 0, 0);
        }
        ++n;
      }
    }
    return n;
  };

  // indicator operands: row fl of operand j is 1.0 iff fl / 4 == j
  bf16x8_t ind[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t v = (fl >> 2) == j ? 0x3F803F80u : 0u;
    ind[j] = __builtin_bit_cast(bf16x8_t, u32x4_t{v, v, v, v});
  }
  f32x4_t acc[kRB];
#pragma unroll
  for (int mi = 0; mi < kRB; ++mi) acc[mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  Cur ci{wg, 0, (int)(wg / ngr), (int)(wg % ngr), {0, 0, 0}};
  load_unit(ci);
  Cur cc = ci;
  int buf_i = 0, buf_c = 0;
  int a_next = 0;  // this wave's activation loads of stage q + 1
  issue_w(ci, 0);
  issue_a(ci, 0);
  next_stage(ci);
  if (Q > 1) {
    issue_w(ci, 1);
    a_next = issue_a(ci, 1);
    next_stage(ci);
  }
  buf_i = 2;
  Cur ca = ci;  // the stage whose activations the next issue_a loads
  for (int64_t q = 0; q < Q; ++q) {
    // stage q has landed for this wave once at most the loads issued after it
    // are pending: W(q+1), A(q+1) and W(q+2), those that were issued
    if (q + 2 < Q) {
      issue_w(ci, buf_i);
      next_stage(ci);
      wait_vm_plus<2 * kW>(a_next);
    } else if (q + 1 < Q) {
      wait_vm_plus<kW>(a_next);
    } else {
      wait_vm<0>();
    }
    // every wave's share of stage q is in LDS, and every wave is done with
    // stage q - 1, whose activation buffer the next loads refill
    asm volatile("s_barrier" ::: "memory");
    if (q + 2 < Q) {
      a_next = issue_a(ca, buf_i);
      next_stage(ca);
      buf_i = buf_i == kRing - 1 ? 0 : buf_i + 1;
    }
    const uint32_t wl = (uint32_t)(uintptr_t)&wlds[wave][buf_c][0];
    const uint32_t al = (uint32_t)(uintptr_t)&alds[buf_c][0] + kBRowBytes * fl + 16 * g;
    buf_c = buf_c == kRing - 1 ? 0 : buf_c + 1;
    {
      u32x4_t xr[8], hd[2];
      u32x2_t qd[2][4];
      const uint32_t w0 = wl + kStageRowBytes * fl;
      read_block_operands(al, w0, w0 + kMatBytes, w0 + 8 * g, w0 + kMatBytes + 8 * g, xr, hd, qd);
      bf16x8_t xo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xo[j] = __builtin_bit_cast(bf16x8_t, xr[j]);
      // each lane decodes sub-blocks g and g + 4 of its feature's block in
      // both weight blocks: ds = d * scale, nc = -(128 ds + dmin * min)
      float dsa[kRB], dsb[kRB], nca[kRB], ncb[kRB];
#pragma unroll
      for (int mi = 0; mi < kRB; ++mi) {
        const u32x4_t h = hd[mi];
        const float d = f16_bits_to_f32(h.x & 0xFFFFu), dmin = f16_bits_to_f32(h.x >> 16);
        const uint32_t sh = 8u * (uint32_t)g;
        const uint32_t sca = __builtin_amdgcn_ubfe(h.y, sh, 6), ma = __builtin_amdgcn_ubfe(h.z, sh, 6);
        const uint32_t scb = __builtin_amdgcn_ubfe(h.w, sh, 4) | (__builtin_amdgcn_ubfe(h.y, sh + 6, 2) << 4);
        const uint32_t mb = __builtin_amdgcn_ubfe(h.w, sh + 4, 4) | (__builtin_amdgcn_ubfe(h.z, sh + 6, 2) << 4);
        dsa[mi] = d * (float)sca;
        dsb[mi] = d * (float)scb;
        nca[mi] = fmaf(-128.f, dsa[mi], -(dmin * (float)ma));
        ncb[mi] = fmaf(-128.f, dsb[mi], -(dmin * (float)mb));
      }
      // ds of all eight sub-blocks of feature fl: sub-block j sits in lane fl + 16 (j % 4)
      float ds[kRB][8];
#pragma unroll
      for (int mi = 0; mi < kRB; ++mi)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ds[mi][j] = __shfl(dsa[mi], fl + 16 * j, 64);
          ds[mi][4 + j] = __shfl(dsb[mi], fl + 16 * j, 64);
        }
      // Sx of sub-blocks g (s0) and g + 4 (s1) for token fl, in every element
      f32x4_t s0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j0 = 2 * c, j1 = 2 * c + 1;
        if (j0 < 4)
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ind[j0], xo[j0], s0, 0, 0, 0);
        else
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ind[j0 - 4], xo[j0], s1, 0, 0, 0);
        if (j1 < 4)
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ind[j1], xo[j1], s0, 0, 0, 0);
        else
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ind[j1 - 4], xo[j1], s1, 0, 0, 0);
#pragma unroll
        for (int mi = 0; mi < kRB; ++mi) {
          const u32x2_t qv = qd[mi][c];
          const bf16x8_t wlo = codes_to_bf16(qv.x & 0x0F0F0F0Fu, qv.y & 0x0F0F0F0Fu);
          const bf16x8_t whi = codes_to_bf16((qv.x >> 4) & 0x0F0F0F0Fu, (qv.y >> 4) & 0x0F0F0F0Fu);
          const f32x4_t z = f32x4_t{0.f, 0.f, 0.f, 0.f};
          const f32x4_t t0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xo[j0], wlo, z, 0, 0, 0);
          const f32x4_t t1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xo[j1], whi, z, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[mi][v] = fmaf(t1[v], ds[mi][j1], fmaf(t0[v], ds[mi][j0], acc[mi][v]));
        }
      }
      // the min terms (and the 128 Sx the codes carried), one fp32 MFMA per four sub-blocks
#pragma unroll
      for (int mi = 0; mi < kRB; ++mi) {
        acc[mi] = __builtin_amdgcn_mfma_f32_16x16x4f32(s0[0], nca[mi], acc[mi], 0, 0, 0);
        acc[mi] = __builtin_amdgcn_mfma_f32_16x16x4f32(s1[0], ncb[mi], acc[mi], 0, 0, 0);
      }
    }

    if (cc.s == nst - 1) {
      // lane holds tokens (tile rows) 4 g + v of feature fl of each weight block
      const Q4Tile& tile = cc.tile;
      const int fg = kWaves * cc.gr + wave;
      if (kGateUp) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = 4 * g + v;
          if (r < tile.nrows) {
            const float gt = acc[0][v], up = acc[1][v];
            const float h = gt / (1.0f + expf(-gt)) * up;
            const uint32_t hb = f32_to_bf16_bits(h);
            const uint32_t lb = f32_to_bf16_bits(h - __uint_as_float(hb << 16));
            const int64_t at = (int64_t)(tile.row0 + r) * a.N + C::kFeat * fg + fl;
            reinterpret_cast<uint16_t*>(a.out)[at] = (uint16_t)hb;
            reinterpret_cast<uint16_t*>(a.out_lo)[at] = (uint16_t)lb;
          }
        }
      } else {
        // rows 8..15 of the MFMA are the h_lo parts of rows 0..7, 32 lanes on
        f32x4_t sum[kRB];
#pragma unroll
        for (int mi = 0; mi < kRB; ++mi)
#pragma unroll
          for (int v = 0; v < 4; ++v) sum[mi][v] = acc[mi][v] + __shfl_down(acc[mi][v], 32, 64);
        if (g < 2) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r = 4 * g + v;
            if (r < tile.nrows) {
              float* yrow = reinterpret_cast<float*>(a.out) + (int64_t)(tile.row0 + r) * a.N + C::kFeat * fg + fl;
#pragma unroll
              for (int mi = 0; mi < kRB; ++mi) yrow[16 * mi] = sum[mi][v];
            }
          }
        }
      }
#pragma unroll
      for (int mi = 0; mi < kRB; ++mi) acc[mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    next_stage(cc);
  }
}

}  // namespace

bool q4k_gemm_supported(int D, int I) { return D > 0 && I > 0 && (D % 256) == 0 && (I % 256) == 0; }

int q4k_rows_per_tile(bool gate_up) { return gate_up ? Q4KCfg<true>::kTileRows : Q4KCfg<false>::kTileRows; }

hipError_t launch_q4k_gemm(const GemmArgs& a, bool gate_up, hipStream_t s) {
  const int feat = gate_up ? Q4KCfg<true>::kFeat : Q4KCfg<false>::kFeat;
  int64_t grid = a.max_tiles * (a.N / feat / kWaves);
  const int64_t slots = (int64_t)kWgPerCu * device_cu_count();
  if (grid > slots) grid = slots;
  if (grid < 1) grid = 1;
  if (gate_up)
    hipLaunchKernelGGL(ffn_q4k_kernel<true>, dim3((unsigned)grid), dim3(kWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL(ffn_q4k_kernel<false>, dim3((unsigned)grid), dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace k3moe
