// Grouping of routed (token, slot) entries by expert, the GEMM tile list, and
// the activation re-layout the GEMM consumes.
//
// The routed-MoE FFN ("build_moe_ffn", llama.cpp pull request "model: add
// Kimi-K3 text model", LLAMA_MAX_EXPERTS comment) runs every expert on the
// tokens routed to it.  Rows of the grouped activations are ordered by
// (expert, token, slot); an entry whose id is outside [0, E) or repeats an id
// earlier in its token's row is skipped.
//
// Tokens are cut into chunks of 64.  For every (chunk, expert) a 64-bit LDS
// bitmap records which tokens of the chunk chose the expert (atomic OR, so the
// result does not depend on thread order).  A single-workgroup scan turns the
// per-chunk popcounts into per-expert offsets and per-(chunk, expert) bases;
// an entry's grouped row is then base + popcount(bitmap & tokens before it).
// Small batches (one chunk) run all phases in one launch.  Tile counts and
// row offsets are packed in 21-bit fields when one scan serves all three, so
// that path needs at most 2^21 - 1 rows (it serves at most 1024 entries).
#include "k3moe_internal.h"

namespace k3moe {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kMaxExpertsPerScanThread = 8;  // 8 * 1024 = K3MOE_MAX_EXPERTS_FFN

__device__ __forceinline__ bool entry_expert(const int32_t* ids_t, int j, int E, int& e_out) {
  const int e = ids_t[j];
  if (e < 0 || e >= E) return false;
  for (int jj = 0; jj < j; ++jj)
    if (ids_t[jj] == e) return false;
  e_out = e;
  return true;
}

// Phase 1: token bitmaps of chunk c into mask[0..E) (LDS). Ends with a barrier.
__device__ __forceinline__ void build_masks(const int32_t* __restrict__ ids, int64_t T, int k, int E, int64_t c,
                            unsigned long long* mask) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  for (int e = tid; e < E; e += nthr) mask[e] = 0ull;
  __syncthreads();
  const int64_t t0 = c * kChunkTokens;
  for (int idx = tid; idx < kChunkTokens * k; idx += nthr) {
    const int tl = idx / k, j = idx - tl * k;
    const int64_t t = t0 + tl;
    int e;
    if (t < T && entry_expert(ids + t * k, j, E, e)) atomicOr(&mask[e], 1ull << tl);
  }
  __syncthreads();
}

// Block-wide exclusive scan of one int per thread (blockDim.x == 1024).
__device__ __forceinline__ int block_exclusive_scan(int v, int* total_out) {
  __shared__ int wave_tot[kScanThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < kScanThreads / 64; ++w) {
    const int tw = wave_tot[w];
    if (w < wave) before += tw;
    total += tw;
  }
  __syncthreads();  // wave_tot may be reused by the next call
  *total_out = total;
  return before + incl - v;
}

// Block-wide exclusive scan of one uint64 per thread (blockDim.x == 1024);
// used with three counters packed in 21-bit fields, so one scan serves all.
__device__ __forceinline__ uint64_t block_exclusive_scan_u64(uint64_t v, uint64_t* total_out) {
  __shared__ uint64_t wave_tot64[kScanThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot64[wave] = incl;
  __syncthreads();
  uint64_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kScanThreads / 64; ++w) {
    const uint64_t tw = wave_tot64[w];
    if (w < wave) before += tw;
    total += tw;
  }
  *total_out = total;
  return before + incl - v;
}

// Phase 2 (one workgroup of 1024 threads): per-expert counts and offsets, the
// two tile lists (one per tile height), and base[c][e] = offsets[e] + rows of e
// in chunks before c.
// masks: [n_chunks][E] (global, or LDS when n_chunks == 1); base: [n_chunks][E].
__device__ __forceinline__ void scan_experts(const unsigned long long* masks, int64_t n_chunks, int E, int rpt0, int rpt1,
                             int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                             int32_t* __restrict__ tile_count, Tile* __restrict__ tiles0, Tile* __restrict__ tiles1,
                             int32_t* base) {
  const int tid = threadIdx.x;
  const int e0 = tid * kMaxExpertsPerScanThread;
  // pass 1: this thread's row and tile totals (counts are recomputed in pass 2
  // rather than kept in a per-thread array)
  int my_rows = 0, my_tiles0 = 0, my_tiles1 = 0;
  for (int i = 0; i < kMaxExpertsPerScanThread; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    int cnt = 0;
    for (int64_t c = 0; c < n_chunks; ++c) cnt += __popcll(masks[c * E + e]);
    my_rows += cnt;
    my_tiles0 += (cnt + rpt0 - 1) / rpt0;
    my_tiles1 += (cnt + rpt1 - 1) / rpt1;
  }
  int total_rows, total_tiles0, total_tiles1;
  int row_off = block_exclusive_scan(my_rows, &total_rows);
  int tile_off0 = block_exclusive_scan(my_tiles0, &total_tiles0);
  int tile_off1 = block_exclusive_scan(my_tiles1, &total_tiles1);
  // pass 2: offsets, per-chunk bases and tiles of each expert
  for (int i = 0; i < kMaxExpertsPerScanThread; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    offsets[e] = row_off;
    int run = row_off;
    for (int64_t c = 0; c < n_chunks; ++c) {
      base[c * E + e] = run;
      run += __popcll(masks[c * E + e]);
    }
    const int cnt = run - row_off;
    counts[e] = cnt;
    for (int r = 0; r < cnt; r += rpt0) {
      Tile tl;
      tl.expert = e;
      tl.row0 = row_off + r;
      tl.nrows = cnt - r < rpt0 ? cnt - r : rpt0;
      tl.pad = 0;
      tiles0[tile_off0++] = tl;
    }
    for (int r = 0; r < cnt; r += rpt1) {
      Tile tl;
      tl.expert = e;
      tl.row0 = row_off + r;
      tl.nrows = cnt - r < rpt1 ? cnt - r : rpt1;
      tl.pad = 0;
      tiles1[tile_off1++] = tl;
    }
    row_off = run;
  }
  if (tid == 0) {
    offsets[E] = total_rows;
    tile_count[0] = total_tiles0;
    tile_count[1] = total_tiles1;
  }
}

// Phase 3: grouped row of every entry of chunk c.
__device__ __forceinline__ void place_entries(const int32_t* __restrict__ ids, int64_t T, int k, int E, int64_t c,
                              const unsigned long long* mask_c, const int32_t* base_c, int32_t* __restrict__ row_tok,
                              int32_t* __restrict__ slot_row) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int64_t t0 = c * kChunkTokens;
  for (int idx = tid; idx < kChunkTokens * k; idx += nthr) {
    const int tl = idx / k, j = idx - tl * k;
    const int64_t t = t0 + tl;
    if (t >= T) continue;
    int e;
    int32_t row = -1;
    if (entry_expert(ids + t * k, j, E, e)) {
      const unsigned long long before = tl ? (mask_c[e] & ((1ull << tl) - 1ull)) : 0ull;
      row = base_c[e] + __popcll(before);
      row_tok[row] = (int32_t)t;
    }
    slot_row[t * k + j] = row;
  }
}

// Activation re-layout: inside every 32-element block of a row, position
// p = 8i + 2t + h holds element 16h + 4i + t (i, t in 0..3, h in 0..1).  This
// is the order in which the GEMM decodes a block's nibble pairs (qs byte j
// holds elements j and j+16), so both MFMA operands see the same K order.
__device__ __forceinline__ void perm_group(const uint16_t* __restrict__ xrow, uint16_t* __restrict__ prow, int g) {
  const int b = g >> 2, i = g & 3;
  const uint2 lo = *reinterpret_cast<const uint2*>(xrow + 32 * b + 4 * i);
  const uint2 hi = *reinterpret_cast<const uint2*>(xrow + 32 * b + 16 + 4 * i);
  uint4 o;
  o.x = __builtin_amdgcn_perm(hi.x, lo.x, 0x05040100u);  // elements 4i,   16+4i
  o.y = __builtin_amdgcn_perm(hi.x, lo.x, 0x07060302u);  // elements 4i+1, 17+4i
  o.z = __builtin_amdgcn_perm(hi.y, lo.y, 0x05040100u);  // elements 4i+2, 18+4i
  o.w = __builtin_amdgcn_perm(hi.y, lo.y, 0x07060302u);  // elements 4i+3, 19+4i
  *reinterpret_cast<uint4*>(prow + 8 * g) = o;
}

__device__ __forceinline__ void permute_chunk_rows(const uint16_t* __restrict__ x, uint16_t* __restrict__ xp, int64_t T, int D,
                                   int64_t c) {
  const int groups = D / 8;
  const int64_t t0 = c * kChunkTokens;
  const int64_t nt = (T - t0) < kChunkTokens ? (T - t0) : kChunkTokens;
  for (int64_t idx = threadIdx.x; idx < nt * groups; idx += blockDim.x) {
    const int64_t tl = idx / groups;
    const int g = (int)(idx - tl * groups);
    const int64_t t = t0 + tl;
    perm_group(x + t * D, xp + t * D, g);
  }
}

__global__ __launch_bounds__(256) void group_count_kernel(GroupArgs a) {
  extern __shared__ unsigned long long lmask[];
  const int64_t c = blockIdx.x;
  build_masks(a.ids, a.T, a.k, a.E, c, lmask);
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) {
    const unsigned long long m = lmask[e];
    a.chunk_mask[c * a.E + e] = m;
    a.chunk_base[c * a.E + e] = __popcll(m);  // per-chunk count; the scan turns it into a base
  }
}

// Multi-chunk scan (one workgroup of 1024 threads).  chunk_base holds the
// per-(chunk, expert) counts on entry and the per-(chunk, expert) bases on exit.
__global__ __launch_bounds__(kScanThreads) void group_scan_kernel(GroupArgs a, int64_t n_chunks) {
  extern __shared__ int32_t ltot[];  // [E] per-expert totals
  const int E = a.E, tid = threadIdx.x;
  for (int e = tid; e < E; e += kScanThreads) ltot[e] = 0;
  __syncthreads();
  const int64_t n = n_chunks * E;
  for (int64_t i = tid; i < n; i += kScanThreads) {
    const int32_t v = a.chunk_base[i];
    if (v) atomicAdd(&ltot[(int)(i % E)], v);
  }
  __syncthreads();
  // offsets and tiles: thread t owns experts 8t..8t+7
  const int rpt0 = a.rows_per_tile[0], rpt1 = a.rows_per_tile[1];
  const int e0 = tid * kMaxExpertsPerScanThread;
  int my_rows = 0, my_tiles0 = 0, my_tiles1 = 0;
  for (int i = 0; i < kMaxExpertsPerScanThread; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    const int cnt = ltot[e];
    my_rows += cnt;
    my_tiles0 += (cnt + rpt0 - 1) / rpt0;
    my_tiles1 += (cnt + rpt1 - 1) / rpt1;
  }
  int total_rows, total_tiles0, total_tiles1;
  int row_off = block_exclusive_scan(my_rows, &total_rows);
  int tile_off0 = block_exclusive_scan(my_tiles0, &total_tiles0);
  int tile_off1 = block_exclusive_scan(my_tiles1, &total_tiles1);
  for (int i = 0; i < kMaxExpertsPerScanThread; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    const int cnt = ltot[e];
    a.counts[e] = cnt;
    a.offsets[e] = row_off;
    for (int r = 0; r < cnt; r += rpt0) {
      Tile tl;
      tl.expert = e;
      tl.row0 = row_off + r;
      tl.nrows = cnt - r < rpt0 ? cnt - r : rpt0;
      tl.pad = 0;
      a.tiles[0][tile_off0++] = tl;
    }
    for (int r = 0; r < cnt; r += rpt1) {
      Tile tl;
      tl.expert = e;
      tl.row0 = row_off + r;
      tl.nrows = cnt - r < rpt1 ? cnt - r : rpt1;
      tl.pad = 0;
      a.tiles[1][tile_off1++] = tl;
    }
    ltot[e] = row_off;  // reuse: the expert's first grouped row
    row_off += cnt;
  }
  if (tid == 0) {
    a.offsets[E] = total_rows;
    a.tile_count[0] = total_tiles0;
    a.tile_count[1] = total_tiles1;
  }
  __syncthreads();
  // bases: expert-parallel running sums over the chunks (loads kept in flight)
  for (int e = tid; e < E; e += kScanThreads) {
    int run = ltot[e];
    int64_t c = 0;
    for (; c + 8 <= n_chunks; c += 8) {
      int32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = a.chunk_base[(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a.chunk_base[(c + u) * E + e] = run;
        run += v[u];
      }
    }
    for (; c < n_chunks; ++c) {
      const int32_t v = a.chunk_base[c * E + e];
      a.chunk_base[c * E + e] = run;
      run += v;
    }
  }
}

// Grouped rows of chunk c (part blockIdx.y of kPlaceParts) and the re-laid-out
// activations of its tokens.
constexpr int kPlaceParts = 8;
__global__ __launch_bounds__(256) void group_place_kernel(GroupArgs a) {
  const int64_t c = blockIdx.x;
  const int part = blockIdx.y;
  const int64_t t0 = c * kChunkTokens;
  const unsigned long long* mask_c = a.chunk_mask + c * a.E;
  const int32_t* base_c = a.chunk_base + c * a.E;
  for (int idx = part * blockDim.x + threadIdx.x; idx < kChunkTokens * a.k; idx += kPlaceParts * blockDim.x) {
    const int tl = idx / a.k, j = idx - tl * a.k;
    const int64_t t = t0 + tl;
    if (t >= a.T) continue;
    int e;
    int32_t row = -1;
    if (entry_expert(a.ids + t * a.k, j, a.E, e)) {
      const unsigned long long before = tl ? (mask_c[e] & ((1ull << tl) - 1ull)) : 0ull;
      row = base_c[e] + __popcll(before);
      a.row_tok[row] = (int32_t)t;
    }
    a.slot_row[t * a.k + j] = row;
  }
  const int groups = a.D / 8;
  const int64_t nt = (a.T - t0) < kChunkTokens ? (a.T - t0) : kChunkTokens;
  for (int64_t idx = part * blockDim.x + threadIdx.x; idx < nt * groups; idx += kPlaceParts * blockDim.x) {
    const int64_t tl = idx / groups;
    const int g = (int)(idx - tl * groups);
    perm_group(a.x + (t0 + tl) * a.D, a.x_perm + (t0 + tl) * a.D, g);
  }
}

// All phases for a batch of at most one chunk (T <= 64), one launch.
// LDS: E bitmaps (8 B) + E bases (4 B).
__global__ __launch_bounds__(kScanThreads) void group_fused_kernel(GroupArgs a) {
  extern __shared__ unsigned long long lmask[];
  int32_t* lbase = reinterpret_cast<int32_t*>(lmask + a.E);
  build_masks(a.ids, a.T, a.k, a.E, 0, lmask);
  scan_experts(lmask, 1, a.E, a.rows_per_tile[0], a.rows_per_tile[1], a.counts, a.offsets, a.tile_count,
               a.tiles[0], a.tiles[1], lbase);
  __syncthreads();
  place_entries(a.ids, a.T, a.k, a.E, 0, lmask, lbase, a.row_tok, a.slot_row);
  permute_chunk_rows(a.x, a.x_perm, a.T, a.D, 0);
}

// All phases for a batch of at most 64 tokens and 1024 entries (decode-sized),
// one launch: thread i owns entry i for the whole kernel, the activation
// re-layout is issued first (it does not depend on the ids), and one packed
// scan yields row offsets and both tile lists.
// LDS: E bitmaps (8 B) + E first rows (4 B).
constexpr int kField = 21;  // bits per packed counter
__global__ __launch_bounds__(kScanThreads) void group_small_kernel(GroupArgs a) {
  extern __shared__ unsigned long long lmask[];
  int32_t* lbase = reinterpret_cast<int32_t*>(lmask + a.E);
  __shared__ int32_t lids[kScanThreads];
  const int tid = threadIdx.x, E = a.E, k = a.k;
  const int entries = (int)a.T * k;
  const int my = tid < entries ? a.ids[tid] : -1;
  permute_chunk_rows(a.x, a.x_perm, a.T, a.D, 0);
  for (int i = tid; i < E; i += kScanThreads) lmask[i] = 0ull;
  lids[tid] = my;
  __syncthreads();
  // skip ids outside [0, E) and repeats of an earlier slot of the same token
  int e = -1;
  if (tid < entries && my >= 0 && my < E) {
    const int t = tid / k, j = tid - t * k;
    bool first = true;
    for (int jj = 0; jj < j; ++jj) first = first && lids[t * k + jj] != my;
    if (first) e = my;
  }
  if (e >= 0) atomicOr(&lmask[e], 1ull << (tid / k));
  __syncthreads();

  const int rpt0 = a.rows_per_tile[0], rpt1 = a.rows_per_tile[1];
  const int e0 = tid * kMaxExpertsPerScanThread;
  uint64_t mine = 0;
  for (int i = 0; i < kMaxExpertsPerScanThread; ++i) {
    const int ex = e0 + i;
    if (ex >= E) break;
    const uint64_t cnt = (uint64_t)__popcll(lmask[ex]);
    mine += cnt | ((cnt + rpt0 - 1) / rpt0) << kField | ((cnt + rpt1 - 1) / rpt1) << (2 * kField);
  }
  uint64_t total;
  const uint64_t off = block_exclusive_scan_u64(mine, &total);
  constexpr uint64_t kMask = (1ull << kField) - 1;
  int row_off = (int)(off & kMask), tile_off0 = (int)((off >> kField) & kMask), tile_off1 = (int)(off >> (2 * kField));
  for (int i = 0; i < kMaxExpertsPerScanThread; ++i) {
    const int ex = e0 + i;
    if (ex >= E) break;
    const int cnt = __popcll(lmask[ex]);
    a.counts[ex] = cnt;
    a.offsets[ex] = row_off;
    lbase[ex] = row_off;
    for (int r = 0; r < cnt; r += rpt0) {
      Tile tl;
      tl.expert = ex;
      tl.row0 = row_off + r;
      tl.nrows = cnt - r < rpt0 ? cnt - r : rpt0;
      tl.pad = 0;
      a.tiles[0][tile_off0++] = tl;
    }
    for (int r = 0; r < cnt; r += rpt1) {
      Tile tl;
      tl.expert = ex;
      tl.row0 = row_off + r;
      tl.nrows = cnt - r < rpt1 ? cnt - r : rpt1;
      tl.pad = 0;
      a.tiles[1][tile_off1++] = tl;
    }
    row_off += cnt;
  }
  if (tid == 0) {
    a.offsets[E] = (int)(total & kMask);
    a.tile_count[0] = (int)((total >> kField) & kMask);
    a.tile_count[1] = (int)(total >> (2 * kField));
  }
  __syncthreads();
  if (tid < entries) {
    const int t = tid / k;
    int32_t row = -1;
    if (e >= 0) {
      row = lbase[e] + __popcll(lmask[e] & ((1ull << t) - 1ull));
      a.row_tok[row] = t;
    }
    a.slot_row[tid] = row;
  }
}

}  // namespace

hipError_t launch_group(const GroupArgs& a, hipStream_t s) {
  const int64_t n_chunks = (a.T + kChunkTokens - 1) / kChunkTokens;
  const size_t fused_lds = (size_t)a.E * (sizeof(unsigned long long) + sizeof(int32_t));
  // leave room for the scan's static LDS (64 ints) under the 64 KB limit
  if (n_chunks == 1 && fused_lds <= 60 * 1024) {
    if (a.T * a.k <= kScanThreads)
      hipLaunchKernelGGL(group_small_kernel, dim3(1), dim3(kScanThreads), fused_lds, s, a);
    else
      hipLaunchKernelGGL(group_fused_kernel, dim3(1), dim3(kScanThreads), fused_lds, s, a);
    return hipGetLastError();
  }
  const size_t mask_lds = (size_t)a.E * sizeof(unsigned long long);
  hipLaunchKernelGGL(group_count_kernel, dim3((unsigned)n_chunks), dim3(256), mask_lds, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(kScanThreads), (size_t)a.E * sizeof(int32_t), s, a, n_chunks);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(group_place_kernel, dim3((unsigned)n_chunks, kPlaceParts), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace k3moe
