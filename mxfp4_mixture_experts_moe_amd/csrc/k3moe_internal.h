// Internal declarations shared by the k3moe HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "k3moe.h"
#include <stddef.h>
#include <stdint.h>

namespace k3moe {

// ---------------------------------------------------------------------------
// Grouped-GEMM work list.  One tile = up to `rows_per_tile` consecutive grouped
// rows of one expert (rows of an expert are contiguous after grouping).
struct Tile {
  int32_t expert;
  int32_t row0;   // first grouped row
  int32_t nrows;  // 1..rows_per_tile
  int32_t pad;
};

// Tokens per grouping chunk: one 64-bit bitmap per (chunk, expert).
constexpr int kChunkTokens = 64;
// Tile lists: 0 / 1 = gate/up / down tiles of experts with many rows, 2 / 3 =
// gate/up / down tiles of experts with few rows (see GroupArgs::split_rows).
constexpr int kTileLists = 4;
// The smallest tile height any GEMM variant uses; sizes the tile list.
constexpr int kMinTileRows = 2;
// Set in slot_row (FFN only) on rows of experts served by the large-tile
// kernels, whose y rows are stored as scaled fp16 (grouped rows stay below
// 2^21 on that path, so the bit is free).
constexpr int32_t kBigRowFlag = 1 << 30;

// Byte layout of the moe_mxfp4_ffn workspace (every region 256-byte aligned).
struct FfnWorkspace {
  size_t counts, offsets, tile_count, tiles[kTileLists], row_tok, slot_row, chunk_base, chunk_mask;
  size_t x_perm, h, h_lo, h_scale, y, y_scale;
  size_t total;
  int64_t max_tiles, n_chunks;
};

FfnWorkspace ffn_workspace_layout(int64_t T, int32_t D, int32_t I, int32_t E, int32_t k);
// Tokens per chunk of moe_mxfp4_ffn (min(T, the largest chunk whose
// activations the GEMM kernels address with 32-bit offsets)).
int64_t ffn_chunk_tokens(int64_t T, int32_t D, int32_t I, int32_t k);

// Workspace of the stand-alone grouping call (tile lists and chunk tables; the
// caller's buffers receive counts, offsets, row_tok and slot_row).  Its tile
// lists use one tile height for every expert.
constexpr int kGroupTileRows = 64;
struct GroupWorkspace {
  size_t tile_count, tiles[kTileLists], chunk_base, chunk_mask;
  size_t total;
  int64_t max_tiles, n_chunks;
};
GroupWorkspace group_workspace_layout(int64_t T, int32_t E, int32_t k);

// ---------------------------------------------------------------------------
// Launchers (host side; enqueue only, return the hipError_t of the launch).
hipError_t launch_route_topk(const float* z, const float* bias, int64_t T, int E, int k, int normalize,
                             float route_scale, int32_t* ids, float* w, hipStream_t s);
hipError_t launch_repack(const uint8_t* packed, const uint8_t* scale, int64_t nblocks, uint8_t* blocks,
                         hipStream_t s);
hipError_t launch_dequant(const uint8_t* blocks, int64_t nblocks, int out_bf16, void* out, hipStream_t s);
hipError_t launch_tile(const uint8_t* src, int64_t nmat, int N, int nb, uint8_t* dst, hipStream_t s);

// Stage-tiled order of an MXFP4 matrix of N rows x nb 17-byte blocks (the
// order mxfp4_tile writes and the FFN kernels read): rows in groups of 16 and
// a group's blocks in stages of 16 (the last group / stage may be shorter);
// groups one after another, a group stage by stage, a stage row by row, a
// row's blocks in order.  So a stage of a group (16 rows x 16 blocks, 4352
// bytes) is one contiguous piece, and a kernel that streams a 16-row group
// one 512-wide K stage at a time reads memory front to back.  Block index of
// block b of row r.
__host__ __device__ inline int64_t tiled_block_index(int N, int nb, int r, int b) {
  const int G = r >> 4, rr = r & 15, s = b >> 4, bb = b & 15;
  const int rG = N - 16 * G < 16 ? N - 16 * G : 16;
  const int wS = nb - 16 * s < 16 ? nb - 16 * s : 16;
  return (int64_t)16 * G * nb + (int64_t)16 * s * rG + (int64_t)rr * wS + bb;
}

struct GroupArgs {
  const int32_t* ids;
  const uint16_t* x;  // bf16 bits [T, D]
  int64_t T;
  int D, E, k;
  int rows_per_tile[kTileLists];  // tile height of each list
  int split_rows;                 // experts with more rows go to lists 0/1, the others to 2/3
  int flag_big_rows;              // mark the slot_row entries of lists 0/1 experts with kBigRowFlag
  // workspace views
  int32_t* counts;
  int32_t* offsets;
  int32_t* tile_count;  // [kTileLists]
  Tile* tiles[kTileLists];
  int32_t* row_tok;
  int32_t* slot_row;
  int32_t* chunk_base;
  unsigned long long* chunk_mask;
  uint16_t* x_perm;  // null: no re-laid-out copy of x (a GEMM that reads x in its natural order)
};
hipError_t launch_group(const GroupArgs& a, hipStream_t s);
// x [T, D] -> x_perm in the P order of the GEMM operands (the re-layout the
// grouping launch also does), for batches grouped inside the gate/up launch.
hipError_t launch_permute_x(const uint16_t* x, uint16_t* xp, int64_t T, int D, hipStream_t s);

struct GemmArgs {
  const uint16_t* act;      // gate/up: x_perm [T, D] (rows via row_tok); down: h_hi [rows, I]
  const uint16_t* act_lo;   // down only: h_lo [rows, I] (h = h_hi + h_lo)
  int64_t act_rows;         // rows of act (and act_lo)
  const int32_t* row_tok;   // gate/up only
  const uint8_t* wa;        // w1 (gate/up) or w2 (down)
  const uint8_t* wb;        // w3 (gate/up) or unused
  const Tile* tiles;
  const int32_t* tile_count;
  int64_t max_tiles;
  int K;      // contraction length (D for gate/up, I for down)
  int N;      // output features (I for gate/up, D for down)
  void* out;     // gate/up: h_hi bf16 [rows, I] (P-order blocks); down: y f32 [rows, D]
  void* out_lo;  // gate/up: h_lo bf16 [rows, I]
  // Large-tile kernels only: h of their rows is carried as fp16 scaled by
  // 2^-h_scale[row, I-slice of 256] instead of h_hi + h_lo (written by the
  // gate/up kernel into `out`, read by the down kernel from `act`).
  int8_t* h_scale;  // [rows, I / 256]
  // Large-tile down kernel only: its y rows are fp16 scaled by 2^y_scale[row,
  // 32-feature group], stored at the start of the row's fp32 slot of `out`.
  int8_t* y_scale;  // [rows, N / 32]
};
hipError_t launch_gate_up(const GemmArgs& a, int rows_per_tile, hipStream_t s);
hipError_t launch_down(const GemmArgs& a, int rows_per_tile, hipStream_t s);

bool big_gemm_supported(int D, int I);
// wide_down: the down product's 128-row tiles (else 64-row tiles)
int big_rows_per_tile(bool gate_up, bool wide_down);
hipError_t launch_big_gate_up(const GemmArgs& a, hipStream_t s);
hipError_t launch_big_down(const GemmArgs& a, bool wide, hipStream_t s);

bool stream_gemm_supported(int D, int I);
int stream_rows_per_tile(bool gate_up);
// Shared-tile streaming GEMMs (batches grouped by a grouping launch): tiles of
// 16 rows (gate/up) or 8 rows (down), one tile per workgroup at a time.
int stream_shared_rows_per_tile(bool gate_up);
hipError_t launch_stream_shared(const GemmArgs& a, bool gate_up, hipStream_t s);
hipError_t launch_stream_down(const GemmArgs& a, hipStream_t s);

// Streaming gate/up that groups the routed entries itself (batches of at most
// kSelfGroupEntries entries, experts below 2^16): every workgroup builds the
// gate/up tiles in LDS from the ids, and workgroup 0 writes what the kernels
// after it read (the down tile list, tile_count[2..3], slot_row), so no
// grouping launch precedes it.  `a.act` is x [T, D] in its natural layout
// (natural_x) or in P order (launch_permute_x).
constexpr int kSelfGroupEntries = 512;
struct SelfGroupArgs {
  const int32_t* ids;   // [T, k]
  int T, E, k;          // T <= 16 (tokens travel as 4-bit fields)
  int32_t* tile_count;  // [kTileLists]; entries 2 and 3 are written
  Tile* down_tiles;     // list 3: 2-row down tiles
  int32_t* slot_row;    // [T * k]: grouped row of each entry, -1 if skipped
};
hipError_t launch_stream_gate_up_grouped(const GemmArgs& a, const SelfGroupArgs& sg, bool natural_x, hipStream_t s);

// Q4_K expert GEMMs (ggml block_q4_K, [E][rows][K / 256][144]): tiles of 16
// token rows (gate/up) or 8 rows of h (down).  D and I multiples of 256.
bool q4k_gemm_supported(int D, int I);
int q4k_rows_per_tile(bool gate_up);
hipError_t launch_q4k_gemm(const GemmArgs& a, bool gate_up, hipStream_t s);
// Compute units of the current device (cached per device).
int device_cu_count();

// mixed: rows whose slot_row entry carries kBigRowFlag hold scaled fp16 y.
hipError_t launch_combine(const float* y, const int8_t* y_scale, bool mixed, const int32_t* slot_row, const float* w,
                          int64_t T, int D, int k,
                          float* out, hipStream_t s);

// Verify batches: distinct[w] = distinct experts routed by the rows of
// position <= w of S sequences of W rows (W <= kMaxVerifyWidth, E <= 8192).
constexpr int kMaxVerifyWidth = 64;
hipError_t launch_verify_distinct(const int32_t* ids, int S, int W, int E, int k, int32_t* distinct, hipStream_t s);

// Device expert cache (state layout inside the caller's buffer; the header
// type is public, k3moe_expert_cache_header).
struct CacheState {
  k3moe_expert_cache_header* header;
  int32_t* slot_of;    // [E]: slot of expert e, -1 if not cached
  int32_t* expert_in;  // [C]: expert in slot s, -1 if empty
  int32_t* order;      // [C]: slots, least recently used first
  int32_t* fetch;      // [2C]: (expert, slot) of the last batch's misses
  size_t bytes;        // total state bytes
  int32_t E, C;
};
CacheState cache_state_view(void* state, int32_t E, int32_t C);
hipError_t launch_cache_init(const CacheState& st, hipStream_t s);
hipError_t launch_cache_plan(const CacheState& st, const int32_t* ids, int64_t n, int32_t* slot_ids, hipStream_t s);
struct CacheFetchArgs {
  const k3moe_expert_cache_header* header;
  const int32_t* fetch;
  const uint8_t *store_w1, *store_w3, *store_w2;  // device-readable store [E, ...]
  uint8_t *cache_w1, *cache_w3, *cache_w2;        // slots [C, ...]
  int64_t mat13, mat2;                            // bytes of one w1 / w3 and one w2 matrix
  int32_t E, C;
};
hipError_t launch_cache_fetch(const CacheFetchArgs& a, hipStream_t s);

// Token-tile height the FFN uses for a batch of T tokens with k routed experts.
int choose_rows_per_tile(int64_t T, int k, int E);

// combine with a bf16 output (round to nearest even) instead of fp32.
hipError_t launch_combine_bf16(const float* y, const int8_t* y_scale, bool mixed, const int32_t* slot_row,
                               const float* w, int64_t T, int D, int k, uint16_t* out, hipStream_t s);

// ---------------------------------------------------------------------------
// Dense bf16 GEMMs of the latent-MoE block: P[split][t][n] = sum over the
// split's K steps of A[t, k] * W[n, k] (fp32 accumulation).  N is made of up to
// kDenseMaxSeg segments (each its own [rows, K] matrix, placed at a multiple
// of kDenseSegAlign in P's row), K of up to 2 segments (each its own A and,
// per N segment, its own W).  K segments are whole 64-wide steps.
constexpr int kDenseMaxSeg = 4;
constexpr int kDenseKStep = 64;
constexpr int kDenseSegAlign = 128;
struct DenseGemmArgs {
  const uint16_t* a[2];  // bf16 [T, K_ks], row stride lda[ks] elements
  int64_t lda[2];
  int ksteps[2];  // K_ks / 64 (ksteps[1] = 0: one K segment)
  int nseg;
  int rows[kDenseMaxSeg];  // output features of segment s
  int base[kDenseMaxSeg];  // offset of segment s in P's row (a multiple of kDenseSegAlign)
  const uint16_t* w[kDenseMaxSeg][2];  // bf16 [rows, K_ks], row stride ldw[s][ks] elements
  int64_t ldw[kDenseMaxSeg][2];
  int64_t T;
  int NV;           // P's row length (the last segment's end, rounded up to kDenseSegAlign)
  int split_steps;  // K steps per split (the last split takes what is left)
  int splits;
  float* p;  // [splits][T][NV]
};
// Tokens up to which the weight-streaming kernel serves a product (one split;
// each 16-token chunk re-reads the weights); beyond, the 128 x 128 tile kernel.
constexpr int64_t kDenseStreamMaxTokens = 16;
// product: 1 or 2 (the block's first or second product; names the kernel only)
hipError_t launch_dense_gemm(const DenseGemmArgs& a, int product, hipStream_t s);
// Splits the tile kernel uses for T tokens and NV features over `ksteps` steps.
int dense_tile_splits(int64_t T, int NV, int ksteps);

// Block epilogue after the first product (segments: gate logits [E], latent
// [D], shared gate [Is], shared up [Is]): z fp32 [T, E]; xl bf16 [T, D] =
// RMS-normed latent times gamma; s bf16 [T, Is] = SiLU(g) * u.  Two launches
// (column sums, then the norm), both parallel over tokens and columns.
struct BlockMidArgs {
  const float* p;  // [splits][T][NV]
  int splits, NV;
  int64_t T;
  int E, D, Is;
  int base_z, base_d, base_g, base_u;
  const uint16_t* gamma;  // bf16 [D]
  float eps;
  float* z;
  uint16_t* xl;
  uint16_t* s;
  float* dbuf;  // [T, D] raw latent (fp32)
  float* ssq;   // [T, nblk] per-workgroup sums of squares of the latent
  int nblk;     // block_mid_blocks(E, D, Is)
  int tok_per_wg;  // tokens per workgroup, 1..8
};
int block_mid_blocks(int E, int D, int Is);
hipError_t launch_block_mid(const BlockMidArgs& a, hipStream_t s);
// out[t][n] = sum over splits of p[split][t][n] (n < N, row length N).
hipError_t launch_dense_sum(const float* p, int splits, int64_t T, int N, float* out, hipStream_t s);

}  // namespace k3moe
