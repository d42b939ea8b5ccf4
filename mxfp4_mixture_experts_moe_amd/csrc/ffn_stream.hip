// Weight-streaming grouped GEMMs for batches in which every expert sees only a
// few tokens (decode-sized batches).  Same arithmetic as ffn.hip (bf16 MFMA,
// the MXFP4 block scale folded into the exact fp4 -> bf16 conversion, fp32
// accumulation, h carried as a bf16 hi + lo pair); only the work decomposition
// differs.
//
// With one or two tokens per expert the product is a stream over the active
// experts' weight bytes (about 4 flop per byte), so the kernel is laid out for
// HBM, not for the matrix cores:
//   - every wave works alone: a unit is 32 weight rows of one tile (gate/up:
//     16 features of w1 and of w3 for up to 4 grouped rows; down: 32 features
//     of w2 for up to 2 grouped rows) over the whole K, and the wave stages the
//     unit's weight rows through a private ring of three LDS buffers with
//     direct global -> LDS loads of 16 bytes per lane, two stages ahead of the
//     one it decodes; no workgroup barrier anywhere;
//   - a stage is 16 MXFP4 blocks (512 K) of each row: 272 bytes, 17 aligned
//     16-byte chunks, so rows of 1904 / 1632 bytes stream without over-fetch;
//     the weights are stage-tiled (tiled_block_index), so the stage of a
//     16-row block is one contiguous 4352-byte run and a unit's weights are
//     read front to back (HBM delivers a fifth less when the same bytes are
//     read as 272-byte pieces of rows 1904 bytes apart);
//   - the tile's activation rows for the same 512 K (x for gate/up, h_hi and
//     h_lo for down) ride in the same stage, one 1 KB load per row the tile
//     actually has (the wait counts follow the per-stage load count); for down
//     the h_hi and h_lo rows sit in different MFMA columns, so one MFMA per
//     decoded operand covers both halves of h;
//   - the waves are persistent: one workgroup of four waves per CU, wave w
//     takes units w, w + W, w + 2W, ..., and the ring runs across unit
//     boundaries so the stream never drains between units.
// The MFMA still does the multiply: its 16 columns are the tile's (up to 4)
// rows, the unused columns hold whatever the LDS row slots hold and are never
// stored.
//
// Decode batches (kSelfGroup): the gate/up launch first groups the routed
// entries itself, identically in every workgroup, from the ids (tiles in LDS,
// tokens of a tile's rows in 4-bit fields), and workgroup 0 writes the down
// tile list, tile counts and slot_row for the launches after it.  With kNatX
// it reads x in its natural layout and builds the P-order operand pairs with
// v_perm; otherwise x arrives re-laid out (P order) by a small launch.
#include "k3moe_internal.h"

#include <math.h>

namespace k3moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;            // waves per workgroup (one workgroup per CU)
constexpr int kRing = 3;             // LDS stage buffers per wave
constexpr int kStageK = 512;         // K per stage (16 MXFP4 blocks)
constexpr int kStageRowBytes = 272;  // bytes of one weight row per stage (17 chunks of 16 B)
constexpr int kRowChunks = 17;
constexpr int kRowDw = 68;           // LDS dwords per staged weight row
constexpr int kBRowBytes = 1040;     // LDS bytes per activation row per stage (1024 + 16 padding)
constexpr int kRB = 2;               // 16-row weight blocks per wave and stage
constexpr int kWInstr = kRB * 5;     // global -> LDS weight loads per stage (5 per 16-row block)
constexpr int kNt = 2;               // cache policy of the weight loads: nontemporal (read once per call)

// A unit is kFeat output features of one tile.  gate/up: row block 0 is w1,
// row block 1 is w3, both rows 16*fg .. 16*fg + 15.  down: both row blocks
// are w2, rows 32*fu .. 32*fu + 15 and 32*fu + 16 .. 32*fu + 31.  The tile's
// activation rows: kTileRows x rows (gate/up); kTileRows h_hi rows followed
// by kTileRows h_lo rows (down).
template <bool kGateUp>
struct StreamCfg;
template <>
struct StreamCfg<true> {
  static constexpr int kFeat = 16, kTileRows = 4, kBRows = 4;
};
template <>
struct StreamCfg<false> {
  static constexpr int kFeat = 32, kTileRows = 2, kBRows = 4;
};
template <bool kGateUp>
constexpr int kStageBytes = kRB * 16 * kStageRowBytes + StreamCfg<kGateUp>::kBRows * kBRowBytes;
static_assert(2 * (kWInstr + StreamCfg<true>::kBRows) < 64, "vmcnt range");
static_assert(2 * (kWInstr + StreamCfg<false>::kBRows) < 64, "vmcnt range");
static_assert(kWaves * kRing * kStageBytes<true> <= 160 * 1024, "LDS");
static_assert(kWaves * kRing * kStageBytes<false> <= 160 * 1024, "LDS");

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

// Block (4*rnd + g) of a staged row: four bf16x8 operands (P-order
// positions 8i..8i+7, i = 0..3) from the five dwords d[0..4] (LDS dwords
// 17*rnd + 4*g .. +4 of the row).  The block starts at byte g of d[0], so its
// exponent is byte g and its qs dword i is bytes g+1+4i .. g+4+4i, picked out
// of two neighbouring dwords with v_perm.
__device__ __forceinline__ void decode_dwords(const uint32_t (&d)[5], int g, uint32_t qsel, bf16x8_t op[4]) {
  const float sf = e8m0_to_f32(__builtin_amdgcn_ubfe(d[0], 8 * g, 8));
  op[0] = decode_dword(__builtin_amdgcn_perm(d[1], d[0], qsel), sf);
  op[1] = decode_dword(__builtin_amdgcn_perm(d[2], d[1], qsel), sf);
  op[2] = decode_dword(__builtin_amdgcn_perm(d[3], d[2], qsel), sf);
  op[3] = decode_dword(__builtin_amdgcn_perm(d[4], d[3], qsel), sf);
}

// Tile list and token map are read through the constant address space so that
// the wave-uniform reads become scalar loads: a vector load would have to be
// waited for with the global -> LDS loads still in flight ahead of it.
template <typename T_>
__device__ __forceinline__ const __attribute__((address_space(4))) T_* as_const(const T_* p) {
  return reinterpret_cast<const __attribute__((address_space(4))) T_*>(reinterpret_cast<uintptr_t>(p));
}

struct TileInfo {
  int expert, row0, nrows;
  int toks;  // self-grouping launch: token of tile row m in bits 4m .. 4m+3
};
__device__ __forceinline__ TileInfo load_tile(const Tile* tiles, int idx) {
  const auto p = as_const(reinterpret_cast<const int32_t*>(tiles) + 4 * idx);
  return TileInfo{p[0], p[1], p[2], 0};
}

// Exclusive scan of three counters over the 256 threads of the workgroup, in
// thread order; tot = the workgroup's sums.  Contains two barriers, so every
// thread must call it.
__device__ __forceinline__ void block_scan3(int (&v)[3], int (&tot)[3], int (*wsum)[3]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl[3] = {v[0], v[1], v[2]};
#pragma unroll
  for (int d = 1; d < 64; d <<= 1)
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const int o = __shfl_up(incl[c], d, 64);
      if (lane >= d) incl[c] += o;
    }
  if (lane == 63)
#pragma unroll
    for (int c = 0; c < 3; ++c) wsum[wave][c] = incl[c];
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int x = wsum[w][c];
      before += w < wave ? x : 0;
      all += x;
    }
    v[c] = before + incl[c] - v[c];
    tot[c] = all;
  }
  __syncthreads();
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// The whole stage's activation operands of one lane when x rows sit in LDS in
// their natural order: block 4 rnd + g of each round rnd, 64 bytes at p +
// 256 rnd, as sixteen 16-byte reads and their wait in one asm block, so the
// LDS latency is paid once per stage.  Written as plain loads, the compiler
// orders these reads behind every global -> LDS load in flight, which empties
// the stage ring each step.
__device__ __forceinline__ void read_x_stage(const uint8_t* p, u32x4_t (&q)[4][4]) {
  const uint32_t a = (uint32_t)(uintptr_t)p;  // LDS byte address
  asm volatile(
      "ds_read_b128 %0, %16\n\tds_read_b128 %1, %16 offset:16\n\t"
      "ds_read_b128 %2, %16 offset:32\n\tds_read_b128 %3, %16 offset:48\n\t"
      "ds_read_b128 %4, %16 offset:256\n\tds_read_b128 %5, %16 offset:272\n\t"
      "ds_read_b128 %6, %16 offset:288\n\tds_read_b128 %7, %16 offset:304\n\t"
      "ds_read_b128 %8, %16 offset:512\n\tds_read_b128 %9, %16 offset:528\n\t"
      "ds_read_b128 %10, %16 offset:544\n\tds_read_b128 %11, %16 offset:560\n\t"
      "ds_read_b128 %12, %16 offset:768\n\tds_read_b128 %13, %16 offset:784\n\t"
      "ds_read_b128 %14, %16 offset:800\n\tds_read_b128 %15, %16 offset:816\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(q[0][0]), "=&v"(q[0][1]), "=&v"(q[0][2]), "=&v"(q[0][3]), "=&v"(q[1][0]), "=&v"(q[1][1]),
        "=&v"(q[1][2]), "=&v"(q[1][3]), "=&v"(q[2][0]), "=&v"(q[2][1]), "=&v"(q[2][2]), "=&v"(q[2][3]),
        "=&v"(q[3][0]), "=&v"(q[3][1]), "=&v"(q[3][2]), "=&v"(q[3][3])
      : "v"(a)
      : "memory");
}

// One entry's view of the batch (self-grouping launch).
struct EntryInfo {
  int id, t, rank, cnt, lead;
  unsigned mask;  // tokens that route to the entry's expert
  bool valid;
};

// s_waitcnt vmcnt(N): at most N of this wave's vector-memory operations
// outstanding.  Loads complete in issue order, so after the wait every load
// issued before the newest N has landed (in LDS, for the global -> LDS loads).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// The same with N = kBase + b, b (0..16) known only at run time.
template <int kBase>
__device__ __forceinline__ void wait_vm_plus(int b) {
  switch (b) {
#define K3_CASE(v) \
  case v: wait_vm<kBase + v>(); break;
    K3_CASE(0) K3_CASE(1) K3_CASE(2) K3_CASE(3) K3_CASE(4) K3_CASE(5) K3_CASE(6) K3_CASE(7) K3_CASE(8)
    K3_CASE(9) K3_CASE(10) K3_CASE(11) K3_CASE(12) K3_CASE(13) K3_CASE(14) K3_CASE(15) K3_CASE(16)
#undef K3_CASE
    default: wait_vm<0>(); break;
  }
}

// Where a wave stands in its list of units: unit u = wid + j * nw, K stage s.
struct Cursor {
  int64_t u;
  int s;
  int ti;         // tile of the unit (u / units per tile)
  int fg;         // feature group of the unit (u % units per tile)
  TileInfo tile;  // tile of the unit
};

template <bool kGateUp, bool kSelfGroup, bool kNatX>
__global__ __launch_bounds__(kWaves * 64, 1) void ffn_stream_kernel(GemmArgs a, SelfGroupArgs sg) {
  static_assert(kGateUp || !kSelfGroup, "only the gate/up launch groups");
  static_assert(kSelfGroup || !kNatX, "natural-order x only in the self-grouping launch (x rows by token)");
  using C = StreamCfg<kGateUp>;
  constexpr int kSB = kStageBytes<kGateUp>;
  constexpr int kMatBytes = 16 * kStageRowBytes;  // one 16-row block of a stage
  constexpr int kWBytes = kRB * kMatBytes;        // activation rows start here
  constexpr int kW = kWInstr;                     // weight loads per stage
  constexpr int kTileRows = C::kTileRows;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves][kRing][kSB];
  // self-grouping launch: gate/up tiles {expert | (nrows-1) << 16 | row0 << 18, tokens}
  __shared__ int2 s_tiles[kSelfGroup ? kSelfGroupEntries : 1];
  __shared__ int s_wsum[kWaves][3];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rho = lane & 15, g = lane >> 4;
  const int nfg = a.N / C::kFeat;  // units per tile
  const auto row_tok = as_const(a.row_tok);
  int n_tiles;
  if constexpr (kSelfGroup) {
    // Group the T*k entries in LDS (identically in every workgroup): an entry
    // is skipped if its id is outside [0, E) or repeats an earlier slot of its
    // token; the first entry of each expert (its leader) owns the expert's
    // rows, ordered by token, and its tiles; leaders take rows and tiles in
    // entry order.  The scratch lives in wave 0's first ring buffer, which is
    // not loaded before the last barrier below.
    constexpr int kThreads = kWaves * 64;
    constexpr int kGuRows = StreamCfg<true>::kTileRows, kDnRows = StreamCfg<false>::kTileRows;
    static_assert(kGuRows == 4, "tile rows travel as 2-bit counts and 4 token fields");
    const int tid = threadIdx.x;
    const int n = sg.T * sg.k;
    const int n4 = (n + 3) & ~3;
    int32_t* sid = reinterpret_cast<int32_t*>(&lds[0][0][0]);  // ids, padded with -1
    int32_t* sbase = sid + kSelfGroupEntries;                  // first row of each leader entry
    // Each expert's first entry and token set come from a hash table on the
    // expert id in LDS (linear probing; twice as many slots as entries, so a
    // probe ends at the id's slot or an empty one long before it wraps).
    constexpr int kH = 2 * kSelfGroupEntries;
    static_assert(kH == 1024, "the hash takes the top 10 bits");
    int32_t* hkey = sbase + kSelfGroupEntries;
    int32_t* hfirst = hkey + kH;
    uint32_t* hmask = reinterpret_cast<uint32_t*>(hfirst + kH);
    for (int h = tid; h < kH; h += kThreads) {
      hkey[h] = -1;
      hfirst[h] = 0x7FFFFFFF;
      hmask[h] = 0u;
    }
    for (int i = tid; i < n4; i += kThreads) sid[i] = i < n ? sg.ids[i] : -1;
    __syncthreads();
    int slot[2] = {-1, -1};  // hash slot of the entry's expert; -1: not a valid first slot of its token
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = tid + kThreads * r;
      if (i >= n) continue;
      const int id = sid[i];
      if (id < 0 || id >= sg.E) continue;
      const int t = i / sg.k, j = i - t * sg.k;
      bool dup = false;  // the same expert in an earlier slot of the token
      for (int jj = 0; jj < j; ++jj) dup = dup || sid[t * sg.k + jj] == id;
      if (dup) continue;
      int h = (int)(((uint32_t)id * 2654435761u) >> 22);
      for (int probe = 0; probe < kH; ++probe) {
        const int old = atomicCAS(&hkey[h], -1, id);
        if (old == -1 || old == id) break;
        h = (h + 1) & (kH - 1);
      }
      atomicMin(&hfirst[h], i);
      atomicOr(&hmask[h], 1u << t);
      slot[r] = h;
    }
    __syncthreads();
    EntryInfo en[2];
    int carry[3] = {0, 0, 0};
    const int rounds = n > kThreads ? 2 : 1;  // uniform: every thread takes the scans' barriers
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (r >= rounds) {
        en[r] = EntryInfo{-1, 0, 0, 0, -1, 0u, false};
        continue;
      }
      const int i = tid + kThreads * r;
      EntryInfo& e = en[r];
      e = EntryInfo{-1, 0, 0, 0, -1, 0u, false};
      if (i < n) {
        const int id = sid[i];
        const int t = i / sg.k;
        e.id = id;
        e.t = t;
        if (slot[r] >= 0) {
          const unsigned mask = hmask[slot[r]];
          e.valid = true;
          e.mask = mask;
          e.lead = hfirst[slot[r]];
          e.rank = __popc(mask & ((1u << t) - 1u));
          e.cnt = __popc(mask);
        }
      }
      const bool leader = e.valid && e.lead == i;
      int v[3] = {0, 0, 0};
      if (leader) {
        v[0] = e.cnt;
        v[1] = (e.cnt + kGuRows - 1) / kGuRows;  // gate/up tiles
        v[2] = (e.cnt + kDnRows - 1) / kDnRows;  // down tiles
      }
      int tot[3];
      block_scan3(v, tot, s_wsum);
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        v[c] += carry[c];
        carry[c] += tot[c];
      }
      if (leader) {
        sbase[i] = v[0];
        unsigned m = e.mask;  // the expert's tokens, taken in row order
        for (int jt = 0; jt < (e.cnt + kGuRows - 1) / kGuRows; ++jt) {
          const int nr = e.cnt - kGuRows * jt < kGuRows ? e.cnt - kGuRows * jt : kGuRows;
          int toks = 0;
          for (int mm = 0; mm < nr; ++mm) {
            toks |= __builtin_ctz(m) << (4 * mm);
            m &= m - 1u;
          }
          s_tiles[v[1] + jt] = make_int2(e.id | (nr - 1) << 16 | (v[0] + kGuRows * jt) << 18, toks);
        }
        if (blockIdx.x == 0)
          for (int jt = 0; jt < (e.cnt + kDnRows - 1) / kDnRows; ++jt) {
            Tile tl;
            tl.expert = e.id;
            tl.row0 = v[0] + kDnRows * jt;
            tl.nrows = e.cnt - kDnRows * jt < kDnRows ? e.cnt - kDnRows * jt : kDnRows;
            tl.pad = 0;
            sg.down_tiles[v[2] + jt] = tl;
          }
      }
    }
    __syncthreads();
    if (blockIdx.x == 0) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int i = tid + kThreads * r;
        if (i < n) sg.slot_row[i] = en[r].valid ? sbase[en[r].lead] + en[r].rank : -1;
      }
      if (tid == 0) {
        sg.tile_count[2] = carry[1];
        sg.tile_count[3] = carry[2];
      }
    }
    __syncthreads();  // scratch reads done before the ring is loaded
    n_tiles = __builtin_amdgcn_readfirstlane(carry[1]);
  } else {
    n_tiles = *as_const(a.tile_count);
  }
  const int64_t n_units = (int64_t)n_tiles * nfg;
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  const int64_t wid = (int64_t)blockIdx.x * kWaves + wave;
  if (wid >= n_units) return;  // uniform over the wave; no barriers below
  const int64_t my_units = (n_units - wid + nw - 1) / nw;
  const int nst = a.K / kStageK;
  const int64_t Q = my_units * nst;
  const uint32_t row_bytes = (uint32_t)(a.K >> 5) * 17;
  const size_t mat_bytes = (size_t)a.N * row_bytes;
  const uint32_t act_row_bytes = (uint32_t)a.K * 2;

  // The weights are stage-tiled (tiled_block_index): stage s of a 16-row
  // group is one contiguous run of 16 rows x 272 bytes, laid out exactly as
  // the LDS stage holds it, so chunk c = 64j + lane of one matrix's stage is
  // byte 16c of the run (MFMA row c / 17, chunk c % 17) and the stage adds
  // 4352*s in the scalar offset.  Only the last load of a matrix is partial
  // (lanes < 16).
  constexpr int kInstrPerMat = (16 * kRowChunks + 63) / 64;  // 5
  uint32_t woff[kInstrPerMat];
#pragma unroll
  for (int j = 0; j < kInstrPerMat; ++j) {
    const int c = 64 * j + lane;
    woff[j] = c < 16 * kRowChunks ? 16u * (uint32_t)c : 0u;
  }
  const bool wtail = lane < 16 * kRowChunks - 64 * (kInstrPerMat - 1);  // lanes of the partial load

  // Cursor moves: a wave's units are wid, wid + nw, ...; the tile and
  // feature group step by nw / nfg and nw % nfg with a carry, so no division
  // runs per unit.
  const int step_ti = (int)(nw / nfg), step_fg = (int)(nw % nfg);
  auto load_unit = [&](Cursor& c) {
    const int tile_idx = __builtin_amdgcn_readfirstlane(c.ti);
    if constexpr (kSelfGroup) {
      const int2 pk = s_tiles[tile_idx];
      const int p0 = __builtin_amdgcn_readfirstlane(pk.x);
      c.tile = TileInfo{p0 & 0xFFFF, (p0 >> 18) & 0x3FF, ((p0 >> 16) & 3) + 1, __builtin_amdgcn_readfirstlane(pk.y)};
    } else {
      c.tile = load_tile(a.tiles, tile_idx);
    }
  };
  auto next_unit = [&](Cursor& c) -> bool {
    c.s = 0;
    c.u += nw;
    c.ti += step_ti;
    c.fg += step_fg;
    if (c.fg >= nfg) {
      c.fg -= nfg;
      ++c.ti;
    }
    if (c.u >= n_units) return false;
    load_unit(c);
    return true;
  };

  // Issue side.  The unit's weight-block resources and activation row
  // offsets are set up once per unit (a wave issues at most one scalar
  // instruction every four cycles, so per-stage address arithmetic would
  // cost more than the stage's loads); a stage only adds its offsets.
  const uint8_t* wbase[kRB];
  uint32_t xsrc[kTileRows];
  int xrows = 0;
  auto prep_issue = [&](const Cursor& c) {
    const size_t unit_off = (size_t)c.tile.expert * mat_bytes + (size_t)(C::kFeat * c.fg) * row_bytes;
#pragma unroll
    for (int mi = 0; mi < kRB; ++mi)
      wbase[mi] = kGateUp ? (mi == 0 ? a.wa : a.wb) + unit_off : a.wa + unit_off + (size_t)(16 * mi) * row_bytes;
    xrows = c.tile.nrows;
#pragma unroll
    for (int m = 0; m < kTileRows; ++m) {
      const int row = c.tile.row0 + (m < xrows ? m : 0);
      const int xrow = kSelfGroup ? (c.tile.toks >> (4 * m)) & 15 : (kGateUp ? row_tok[row] : row);
      xsrc[m] = (uint32_t)xrow * act_row_bytes;
    }
  };
  // Stage ci.s of the issue cursor's unit into ring buffer `buf`; returns
  // how many activation loads it issued.
  auto issue = [&](const Cursor& c, int buf) -> int {
    uint8_t* dst = &lds[wave][buf][0];
    const uint32_t wso = (uint32_t)(16 * kStageRowBytes * c.s);
#pragma unroll
    for (int mi = 0; mi < kRB; ++mi) {
      const __amdgpu_buffer_rsrc_t wr =
          __builtin_amdgcn_make_buffer_rsrc((void*)wbase[mi], 0, (int)(16 * row_bytes), 0x00020000);
#pragma unroll
      for (int j = 0; j < kInstrPerMat - 1; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (__attribute__((address_space(3))) void*)(uintptr_t)(dst + mi * kMatBytes + 1024 * j),
                                                 16, woff[j], wso, 0, kNt);
      if (wtail)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, (__attribute__((address_space(3))) void*)(uintptr_t)(dst + mi * kMatBytes + 1024 * (kInstrPerMat - 1)), 16,
            woff[kInstrPerMat - 1], wso, 0, kNt);
    }
    uint8_t* bdst = dst + kWBytes;
    const uint32_t aso = (uint32_t)(kStageK * 2 * c.s);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.act, 0, (int)((uint32_t)a.act_rows * act_row_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t lr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kGateUp ? a.act : a.act_lo), 0, (int)((uint32_t)a.act_rows * act_row_bytes), 0x00020000);
#pragma unroll
    for (int m = 0; m < kTileRows; ++m) {
      if (m < xrows) {
        // (an array element passed straight as the scalar offset makes the
        // host pass drop this kernel's launch stub without a diagnostic)
        const uint32_t so = xsrc[m] + aso;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)(uintptr_t)(bdst + kBRowBytes * m),
                                                 16, 16 * lane, so, 0, 0);
        if (!kGateUp)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              lr, (__attribute__((address_space(3))) void*)(uintptr_t)(bdst + kBRowBytes * (kTileRows + m)), 16, 16 * lane,
              so, 0, 0);
      }
    }
    return (kGateUp ? 1 : 2) * xrows;
  };
  // Advances the issue cursor by one stage; false once its units are done.
  auto advance_issue = [&](Cursor& c) -> bool {
    if (++c.s < nst) return true;
    if (!next_unit(c)) return false;
    prep_issue(c);
    return true;
  };
  auto advance_compute = [&](Cursor& c) {
    if (++c.s == nst) next_unit(c);
  };

  f32x4_t acc[kRB][2];  // per row block: the even and the odd rounds
#pragma unroll
  for (int mi = 0; mi < kRB; ++mi) acc[mi][0] = acc[mi][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint32_t qsel = 0x03020100u + 0x01010101u * (uint32_t)(g + 1);
  Cursor ci{wid, 0, (int)(wid / nfg), (int)(wid % nfg), {0, 0, 0, 0}};  // issue side
  load_unit(ci);
  prep_issue(ci);
  Cursor cc = ci;  // compute side
  int buf_i = 0, buf_c = 0;
  issue(ci, buf_i);
  advance_issue(ci);
  buf_i = 1;
  int b_next = 0;  // activation loads of stage q + 1
  if (Q > 1) {
    b_next = issue(ci, buf_i);
    advance_issue(ci);
    buf_i = 2;
  }
  // B column rho reads LDS activation row brow: for gate/up the tile's row
  // rho; for down h_hi row rho (columns 0 .. kTileRows-1) or h_lo row
  // rho - kTileRows (the next kTileRows columns), so one MFMA multiplies both
  // halves of h (added in the epilogue).  Columns without a row read row 0
  // (a broadcast; their sums are dropped).
  auto brow_of = [&](int nrows) {
    const bool has = kGateUp ? rho < nrows : (rho < 2 * kTileRows && (rho % kTileRows) < nrows);
    return has ? rho : 0;
  };
  int boff = kWBytes + kBRowBytes * brow_of(cc.tile.nrows);

  for (int64_t q = 0; q < Q; ++q) {
    // Stage q's loads are the oldest outstanding ones: wait until only the
    // loads of stages q+1 and q+2 (and whatever follows them) may be pending.
    if (q + 2 < Q) {
      const int b2 = issue(ci, buf_i);
      advance_issue(ci);
      buf_i = buf_i == kRing - 1 ? 0 : buf_i + 1;
      wait_vm_plus<2 * kW>(b_next + b2);
      b_next = b2;
    } else if (q + 1 < Q) {
      wait_vm_plus<kW>(b_next);
    } else {
      wait_vm<0>();
    }
    const uint8_t* st = &lds[wave][buf_c][0];
    buf_c = buf_c == kRing - 1 ? 0 : buf_c + 1;
    const uint32_t* wl = reinterpret_cast<const uint32_t*>(st);
    const uint8_t* bl = st + boff;
    // Every LDS read of the stage first (the activation operands of the four
    // rounds, the five weight dwords per round and row block), then the
    // decodes two rounds at a time and the MFMAs on four accumulator chains
    // (row block x round parity), so neither the LDS latency nor an MFMA's
    // dependence on the previous one is exposed each round.
    bf16x8_t bop[4][4];
    if constexpr (kNatX) {
      // x rows in natural order: P-order dword t of operand i pairs
      // elements 4i + t and 16 + 4i + t of block 4*rnd + g
      u32x4_t q[4][4];  // per round: elements 0-7, 8-15, 16-23, 24-31
      read_x_stage(bl + 64 * g, q);
#pragma unroll
      for (int rnd = 0; rnd < 4; ++rnd)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4_t& L = q[rnd][i >> 1];
          const u32x4_t& H = q[rnd][2 + (i >> 1)];
          const uint32_t l0 = (i & 1) ? L.z : L.x, l1 = (i & 1) ? L.w : L.y;
          const uint32_t h0 = (i & 1) ? H.z : H.x, h1 = (i & 1) ? H.w : H.y;
          uint4 r;
          r.x = __builtin_amdgcn_perm(h0, l0, 0x05040100u);
          r.y = __builtin_amdgcn_perm(h0, l0, 0x07060302u);
          r.z = __builtin_amdgcn_perm(h1, l1, 0x05040100u);
          r.w = __builtin_amdgcn_perm(h1, l1, 0x07060302u);
          bop[rnd][i] = __builtin_bit_cast(bf16x8_t, r);
        }
    } else {
#pragma unroll
      for (int rnd = 0; rnd < 4; ++rnd)
#pragma unroll
        for (int i = 0; i < 4; ++i) bop[rnd][i] = *reinterpret_cast<const bf16x8_t*>(bl + 64 * (4 * rnd + g) + 16 * i);
    }
    uint32_t wd[kRB][4][5];
#pragma unroll
    for (int mi = 0; mi < kRB; ++mi)
#pragma unroll
      for (int rnd = 0; rnd < 4; ++rnd)
#pragma unroll
        for (int j = 0; j < 5; ++j) wd[mi][rnd][j] = wl[(16 * mi + rho) * kRowDw + 17 * rnd + 4 * g + j];
#pragma unroll
    for (int r0 = 0; r0 < 4; r0 += 2) {
      bf16x8_t aop[kRB][2][4];
#pragma unroll
      for (int mi = 0; mi < kRB; ++mi)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) decode_dwords(wd[mi][r0 + rr], g, qsel, aop[mi][rr]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
#pragma unroll
          for (int mi = 0; mi < kRB; ++mi)
            acc[mi][rr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[mi][rr][i], bop[r0 + rr][i], acc[mi][rr], 0, 0, 0);
    }

    if (cc.s == nst - 1) {
      // Epilogue of the unit: lane holds, for tile row rho, features 4g + v
      // of each 16-row block.
      const TileInfo& tile = cc.tile;
      const int fg = cc.fg;
      f32x4_t sum[kRB];
#pragma unroll
      for (int mi = 0; mi < kRB; ++mi) sum[mi] = acc[mi][0] + acc[mi][1];
      if (!kGateUp) {
        // y = (h_hi part in column rho) + (h_lo part in column rho + kTileRows)
#pragma unroll
        for (int mi = 0; mi < kRB; ++mi)
#pragma unroll
          for (int v = 0; v < 4; ++v) sum[mi][v] += __shfl_down(sum[mi][v], kTileRows, 16);
      }
      if (rho < tile.nrows) {
        const int64_t row = tile.row0 + rho;
        if (kGateUp) {
          uint32_t hb[4], lb[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float gt = sum[0][v], up = sum[1][v];
            const float h = gt / (1.0f + expf(-gt)) * up;
            hb[v] = f32_to_bf16_bits(h);
            lb[v] = f32_to_bf16_bits(h - __uint_as_float(hb[v] << 16));
          }
          // feature 16*fg + 4g + v is element e = 16*(fg&1) + 4g + v of
          // I-block fg/2, stored at its P-order position 8g + 2v + (fg&1)
          const int pos = 32 * (fg >> 1) + 8 * g + (fg & 1);
          uint16_t* hrow = reinterpret_cast<uint16_t*>(a.out) + row * a.N + pos;
          uint16_t* lrow = reinterpret_cast<uint16_t*>(a.out_lo) + row * a.N + pos;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            hrow[2 * v] = (uint16_t)hb[v];
            lrow[2 * v] = (uint16_t)lb[v];
          }
        } else {
          float* yrow = reinterpret_cast<float*>(a.out) + row * a.N + C::kFeat * fg + 4 * g;
#pragma unroll
          for (int mi = 0; mi < kRB; ++mi)
            *reinterpret_cast<float4*>(yrow + 16 * mi) = make_float4(sum[mi][0], sum[mi][1], sum[mi][2], sum[mi][3]);
        }
      }
#pragma unroll
      for (int mi = 0; mi < kRB; ++mi) acc[mi][0] = acc[mi][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    advance_compute(cc);
    if (cc.s == 0 && q + 1 < Q) boff = kWBytes + kBRowBytes * brow_of(cc.tile.nrows);
  }
}

// Shared-tile streaming, for batches a grouping launch has grouped (verify,
// the few-row experts of prefill).  A stage's decode and MFMA work per wave is
// that of ffn_stream_kernel, but the four waves of a workgroup take four
// consecutive feature groups of ONE tile, so the tile's activation rows travel
// once per stage into a ring the workgroup shares: 16 rows (gate/up: 16 token
// rows; down: 8 h_hi rows, then the same 8 rows of h_lo), so every MFMA column
// is a live row and an expert with up to 16 (gate/up) / 8 (down) rows streams
// its weights once.  Each wave loads its share of a stage's live activation
// rows (B rows 4w .. 4w+3 that the tile has) and waits for exactly the loads
// it issued; one barrier per stage, after each wave's wait for its own loads of
// that stage, completes the stage for all waves and frees the activation
// buffer the previous stage used, which the loads issued right after the
// barrier refill.  The barrier is a bare s_barrier: a fenced one would also
// wait for the two weight stages in flight.
template <bool kGateUp>
struct SharedCfg;
template <>
struct SharedCfg<true> {
  static constexpr int kFeat = 16, kTileRows = 16;
};
template <>
struct SharedCfg<false> {
  static constexpr int kFeat = 32, kTileRows = 8;
};
constexpr int kSharedBRows = 16;
constexpr int kSharedABytes = kSharedBRows * kBRowBytes;
constexpr int kSharedWBytes = kRB * 16 * kStageRowBytes;
static_assert(kWaves * kRing * kSharedWBytes + kRing * kSharedABytes <= 160 * 1024, "LDS");

template <bool kGateUp>
__global__ __launch_bounds__(kWaves * 64, 1) void ffn_stream_shared_kernel(GemmArgs a) {
  using C = SharedCfg<kGateUp>;
  constexpr int kTileRows = C::kTileRows;
  constexpr int kMatBytes = 16 * kStageRowBytes;
  constexpr int kW = kWInstr;        // weight loads per stage and wave
  constexpr int kA = kSharedBRows / kWaves;  // activation loads per stage and wave
  static_assert(2 * kW + kA < 64, "vmcnt range");
  __shared__ __attribute__((aligned(16))) uint8_t wlds[kWaves][kRing][kSharedWBytes];
  __shared__ __attribute__((aligned(16))) uint8_t alds[kRing][kSharedABytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rho = lane & 15, g = lane >> 4;
  const int ngr = a.N / C::kFeat / kWaves;  // workgroup units per tile
  const auto row_tok = as_const(a.row_tok);
  const int n_tiles = *as_const(a.tile_count);
  const int64_t n_units = (int64_t)n_tiles * ngr;
  const int64_t nwg = gridDim.x;
  const int64_t wg = blockIdx.x;
  if (wg >= n_units) return;  // uniform over the workgroup; every later barrier is reached by all waves
  const int64_t my_units = (n_units - wg + nwg - 1) / nwg;
  const int nst = a.K / kStageK;
  const int64_t Q = my_units * nst;
  const uint32_t row_bytes = (uint32_t)(a.K >> 5) * 17;
  const size_t mat_bytes = (size_t)a.N * row_bytes;
  const uint32_t act_row_bytes = (uint32_t)a.K * 2;

  constexpr int kInstrPerMat = (16 * kRowChunks + 63) / 64;  // 5
  uint32_t woff[kInstrPerMat];
#pragma unroll
  for (int j = 0; j < kInstrPerMat; ++j) {
    const int c = 64 * j + lane;
    woff[j] = c < 16 * kRowChunks ? 16u * (uint32_t)c : 0u;
  }
  const bool wtail = lane < 16 * kRowChunks - 64 * (kInstrPerMat - 1);

  // Cursor: the workgroup's units are wg, wg + nwg, ...; tile u / ngr and
  // group u % ngr step with a carry; the wave's feature group is 4 * group + wave.
  struct SCursor {
    int64_t u;
    int s, ti, gr;
    TileInfo tile;
  };
  const int step_ti = (int)(nwg / ngr), step_gr = (int)(nwg % ngr);
  auto load_unit = [&](SCursor& c) { c.tile = load_tile(a.tiles, __builtin_amdgcn_readfirstlane(c.ti)); };
  auto next_stage = [&](SCursor& c) {
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

  // weight loads of the issue cursor's stage (this wave's feature group)
  auto issue_w = [&](const SCursor& c, int buf) {
    const int fg = kWaves * c.gr + wave;
    const size_t unit_off = (size_t)c.tile.expert * mat_bytes + (size_t)(C::kFeat * fg) * row_bytes;
    uint8_t* dst = &wlds[wave][buf][0];
    const uint32_t wso = (uint32_t)(16 * kStageRowBytes * c.s);
#pragma unroll
    for (int mi = 0; mi < kRB; ++mi) {
      const uint8_t* base =
          kGateUp ? (mi == 0 ? a.wa : a.wb) + unit_off : a.wa + unit_off + (size_t)(16 * mi) * row_bytes;
      const __amdgpu_buffer_rsrc_t wr =
          __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)(16 * row_bytes), 0x00020000);
#pragma unroll
      for (int j = 0; j < kInstrPerMat - 1; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (__attribute__((address_space(3))) void*)(uintptr_t)(dst + mi * kMatBytes + 1024 * j),
                                                 16, woff[j], wso, 0, kNt);
      if (wtail)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, (__attribute__((address_space(3))) void*)(uintptr_t)(dst + mi * kMatBytes + 1024 * (kInstrPerMat - 1)), 16,
            woff[kInstrPerMat - 1], wso, 0, kNt);
    }
  };
  // this wave's share (B rows 4 * wave .. 4 * wave + 3) of the stage's live
  // activation rows (B row m: gate/up token row m of the tile; down h_hi row
  // m, or h_lo row m - 8); columns of absent rows read whatever their LDS row
  // holds and are never stored.  Returns how many loads it issued.
  auto issue_a = [&](const SCursor& c, int buf) -> int {
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
        if (kGateUp || m < kTileRows)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)(uintptr_t)(dst + kBRowBytes * m),
                                                   16, 16 * lane, so, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(lr, (__attribute__((address_space(3))) void*)(uintptr_t)(dst + kBRowBytes * m),
                                                   16, 16 * lane, so, 0, 0);
        ++n;
      }
    }
    return n;
  };

  f32x4_t acc[kRB][2];
#pragma unroll
  for (int mi = 0; mi < kRB; ++mi) acc[mi][0] = acc[mi][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint32_t qsel = 0x03020100u + 0x01010101u * (uint32_t)(g + 1);

  SCursor ci{wg, 0, (int)(wg / ngr), (int)(wg % ngr), {0, 0, 0, 0}};
  load_unit(ci);
  SCursor cc = ci;
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
  SCursor ca = ci;  // the stage whose activations the next issue_a loads
  for (int64_t q = 0; q < Q; ++q) {
    // stage q landed for this wave once at most the loads issued after it
    // are pending: W(q+1), A(q+1), W(q+2) (those that were issued)
    if (q + 2 < Q) {
      issue_w(ci, buf_i);
      next_stage(ci);
      wait_vm_plus<2 * kW>(a_next);
    } else if (q + 1 < Q) {
      wait_vm_plus<kW>(a_next);
    } else {
      wait_vm<0>();
    }
    asm volatile("s_barrier" ::: "memory");
    if (q + 2 < Q) {
      a_next = issue_a(ca, buf_i);
      next_stage(ca);
      buf_i = buf_i == kRing - 1 ? 0 : buf_i + 1;
    }
    const uint32_t* wl = reinterpret_cast<const uint32_t*>(&wlds[wave][buf_c][0]);
    const uint8_t* bl = &alds[buf_c][0] + kBRowBytes * rho;
    buf_c = buf_c == kRing - 1 ? 0 : buf_c + 1;
    bf16x8_t bop[4][4];
#pragma unroll
    for (int rnd = 0; rnd < 4; ++rnd)
#pragma unroll
      for (int i = 0; i < 4; ++i) bop[rnd][i] = *reinterpret_cast<const bf16x8_t*>(bl + 64 * (4 * rnd + g) + 16 * i);
    uint32_t wd[kRB][4][5];
#pragma unroll
    for (int mi = 0; mi < kRB; ++mi)
#pragma unroll
      for (int rnd = 0; rnd < 4; ++rnd)
#pragma unroll
        for (int j = 0; j < 5; ++j) wd[mi][rnd][j] = wl[(16 * mi + rho) * kRowDw + 17 * rnd + 4 * g + j];
#pragma unroll
    for (int r0 = 0; r0 < 4; r0 += 2) {
      bf16x8_t aop[kRB][2][4];
#pragma unroll
      for (int mi = 0; mi < kRB; ++mi)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) decode_dwords(wd[mi][r0 + rr], g, qsel, aop[mi][rr]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
#pragma unroll
          for (int mi = 0; mi < kRB; ++mi)
            acc[mi][rr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[mi][rr][i], bop[r0 + rr][i], acc[mi][rr], 0, 0, 0);
    }

    if (cc.s == nst - 1) {
      // lane holds, for tile row rho (down: h_hi part in columns 0-7, h_lo
      // part in columns 8-15), features 4g + v of each 16-row block
      const TileInfo& tile = cc.tile;
      const int fg = kWaves * cc.gr + wave;
      f32x4_t sum[kRB];
#pragma unroll
      for (int mi = 0; mi < kRB; ++mi) sum[mi] = acc[mi][0] + acc[mi][1];
      if (!kGateUp) {
#pragma unroll
        for (int mi = 0; mi < kRB; ++mi)
#pragma unroll
          for (int v = 0; v < 4; ++v) sum[mi][v] += __shfl_down(sum[mi][v], kTileRows, 16);
      }
      if (rho < tile.nrows) {
        const int64_t row = tile.row0 + rho;
        if (kGateUp) {
          uint32_t hb[4], lb[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float gt = sum[0][v], up = sum[1][v];
            const float h = gt / (1.0f + expf(-gt)) * up;
            hb[v] = f32_to_bf16_bits(h);
            lb[v] = f32_to_bf16_bits(h - __uint_as_float(hb[v] << 16));
          }
          const int pos = 32 * (fg >> 1) + 8 * g + (fg & 1);
          uint16_t* hrow = reinterpret_cast<uint16_t*>(a.out) + row * a.N + pos;
          uint16_t* lrow = reinterpret_cast<uint16_t*>(a.out_lo) + row * a.N + pos;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            hrow[2 * v] = (uint16_t)hb[v];
            lrow[2 * v] = (uint16_t)lb[v];
          }
        } else {
          float* yrow = reinterpret_cast<float*>(a.out) + row * a.N + C::kFeat * fg + 4 * g;
#pragma unroll
          for (int mi = 0; mi < kRB; ++mi)
            *reinterpret_cast<float4*>(yrow + 16 * mi) = make_float4(sum[mi][0], sum[mi][1], sum[mi][2], sum[mi][3]);
        }
      }
#pragma unroll
      for (int mi = 0; mi < kRB; ++mi) acc[mi][0] = acc[mi][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    next_stage(cc);
  }
}

int cu_count() {
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

template <bool kGateUp, bool kSelfGroup, bool kNatX>
hipError_t launch_stream(const GemmArgs& a, const SelfGroupArgs& sg, hipStream_t s) {
  const int64_t max_units = a.max_tiles * (a.N / StreamCfg<kGateUp>::kFeat);
  int64_t grid = (max_units + kWaves - 1) / kWaves;
  const int cus = cu_count();
  if (grid > cus) grid = cus;
  if (grid < 1) grid = 1;  // the self-grouping launch needs workgroup 0 in any case
  hipLaunchKernelGGL((ffn_stream_kernel<kGateUp, kSelfGroup, kNatX>), dim3((unsigned)grid), dim3(kWaves * 64), 0, s, a,
                     sg);
  return hipGetLastError();
}

}  // namespace

// K must be whole stages (rows of 16-block multiples, so every row and every
// stage window starts 16-byte aligned); I must hold whole 32-feature blocks.
bool stream_gemm_supported(int D, int I) { return (D % kStageK) == 0 && (I % kStageK) == 0; }

int stream_rows_per_tile(bool gate_up) { return gate_up ? StreamCfg<true>::kTileRows : StreamCfg<false>::kTileRows; }

hipError_t launch_stream_down(const GemmArgs& a, hipStream_t s) { return launch_stream<false, false, false>(a, {}, s); }

int stream_shared_rows_per_tile(bool gate_up) {
  return gate_up ? SharedCfg<true>::kTileRows : SharedCfg<false>::kTileRows;
}

hipError_t launch_stream_shared(const GemmArgs& a, bool gate_up, hipStream_t s) {
  const int feat = gate_up ? SharedCfg<true>::kFeat : SharedCfg<false>::kFeat;
  const int64_t max_units = a.max_tiles * (a.N / feat / kWaves);
  int64_t grid = max_units;
  const int cus = cu_count();
  if (grid > cus) grid = cus;
  if (grid < 1) grid = 1;
  if (gate_up)
    hipLaunchKernelGGL(ffn_stream_shared_kernel<true>, dim3((unsigned)grid), dim3(kWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL(ffn_stream_shared_kernel<false>, dim3((unsigned)grid), dim3(kWaves * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stream_gate_up_grouped(const GemmArgs& a, const SelfGroupArgs& sg, bool natural_x, hipStream_t s) {
  return natural_x ? launch_stream<true, true, true>(a, sg, s) : launch_stream<true, true, false>(a, sg, s);
}

}  // namespace k3moe
