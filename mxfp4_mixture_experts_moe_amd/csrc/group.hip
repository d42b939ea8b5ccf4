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
// Small batches (one chunk) run all phases in one launch.
//
// Each expert's rows are cut into GEMM tiles in two lists (gate/up, down),
// chosen by the expert's row count: the large-tile lists for experts with
// more than split_rows rows, the weight-streaming lists for the others.
#include "k3moe_internal.h"

namespace k3moe {
namespace {

constexpr int kScanThreads = 1024;
// Experts per scan thread: thread t owns experts t*n .. t*n + n - 1 with
// n = ceil(E / kScanThreads) (at most 8 for the largest expert count, 8192),
// so the block scan runs in expert order.  As few as possible (one up to 1024
// experts): the owner also writes its experts' tiles one after another.

// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for every
// outstanding global load and store of the wave (its release fence), which
// would put the latency of stores nobody in the workgroup reads on the
// critical path; no wave here reads global memory another wave of the same
// workgroup wrote.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
  lds_barrier();
  const int64_t t0 = c * kChunkTokens;
  for (int idx = tid; idx < kChunkTokens * k; idx += nthr) {
    const int tl = idx / k, j = idx - tl * k;
    const int64_t t = t0 + tl;
    int e;
    if (t < T && entry_expert(ids + t * k, j, E, e)) atomicOr(&mask[e], 1ull << tl);
  }
  lds_barrier();
}

// Block-wide exclusive scan of N ints per thread (blockDim.x == 1024): v[i]
// becomes the sum of v[i] over lower threads, total[i] the sum over all.
template <int N>
__device__ __forceinline__ void block_exclusive_scan_n(int (&v)[N], int (&total)[N]) {
  __shared__ int wave_tot[kScanThreads / 64][N];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl[N];
#pragma unroll
  for (int i = 0; i < N; ++i) incl[i] = v[i];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1)
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int o = __shfl_up(incl[i], d, 64);
      if (lane >= d) incl[i] += o;
    }
  if (lane == 63)
#pragma unroll
    for (int i = 0; i < N; ++i) wave_tot[wave][i] = incl[i];
  lds_barrier();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    int before = 0, tot = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      const int tw = wave_tot[w][i];
      if (w < wave) before += tw;
      tot += tw;
    }
    v[i] = before + incl[i] - v[i];
    total[i] = tot;
  }
  lds_barrier();  // wave_tot may be reused by the next call
}

// Tile lists.  An expert with more than split_rows rows goes to lists 0
// (gate/up) and 1 (down), one with fewer to lists 2 and 3; list L cuts the
// expert's rows into tiles of rows_per_tile[L].
struct TileSpec {
  int rpt[kTileLists];
  int split;
};
__device__ __forceinline__ TileSpec tile_spec(const GroupArgs& a) {
  TileSpec t;
#pragma unroll
  for (int L = 0; L < kTileLists; ++L) t.rpt[L] = a.rows_per_tile[L];
  t.split = a.split_rows;
  return t;
}
__device__ __forceinline__ int tiles_in_list(const TileSpec& t, int cnt, int L) {
  const bool first_pair = cnt > t.split;
  if (cnt == 0 || (L < 2) != first_pair) return 0;
  return (cnt + t.rpt[L] - 1) / t.rpt[L];
}
// v[0] += cnt, v[1 + L] += tiles of list L.
__device__ __forceinline__ void add_expert(const TileSpec& t, int cnt, int (&v)[1 + kTileLists]) {
  v[0] += cnt;
#pragma unroll
  for (int L = 0; L < kTileLists; ++L) v[1 + L] += tiles_in_list(t, cnt, L);
}
// Writes the tiles of expert e (rows row0 .. row0 + cnt) and advances the
// per-list write positions in off[1 + L].
__device__ __forceinline__ void emit_tiles(const GroupArgs& a, const TileSpec& t, int e, int row0, int cnt,
                                           int (&off)[1 + kTileLists]) {
#pragma unroll
  for (int L = 0; L < kTileLists; ++L) {
    if (tiles_in_list(t, cnt, L) == 0) continue;
    for (int r = 0; r < cnt; r += t.rpt[L]) {
      Tile tl;
      tl.expert = e;
      tl.row0 = row0 + r;
      tl.nrows = cnt - r < t.rpt[L] ? cnt - r : t.rpt[L];
      tl.pad = 0;
      a.tiles[L][off[1 + L]++] = tl;
    }
  }
}
__device__ __forceinline__ void write_totals(const GroupArgs& a, int E, const int (&total)[1 + kTileLists]) {
  a.offsets[E] = total[0];
#pragma unroll
  for (int L = 0; L < kTileLists; ++L) a.tile_count[L] = total[1 + L];
}

// Phase 2 (one workgroup of 1024 threads): per-expert counts and offsets, the
// tile lists, and base[c][e] = offsets[e] + rows of e in chunks before c.
// masks: [n_chunks][E] (global, or LDS when n_chunks == 1); base: [n_chunks][E].
__device__ __forceinline__ void scan_experts(const GroupArgs& a, const unsigned long long* masks, int64_t n_chunks,
                                             int32_t* base) {
  const int tid = threadIdx.x, E = a.E;
  const TileSpec ts = tile_spec(a);
  const int per = (E + kScanThreads - 1) / kScanThreads;
  const int e0 = tid * per;
  // pass 1: this thread's row and tile totals (counts are recomputed in pass 2
  // rather than kept in a per-thread array)
  int v[1 + kTileLists] = {0, 0, 0, 0, 0};
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    int cnt = 0;
    for (int64_t c = 0; c < n_chunks; ++c) cnt += __popcll(masks[c * E + e]);
    add_expert(ts, cnt, v);
  }
  int total[1 + kTileLists];
  block_exclusive_scan_n(v, total);
  // pass 2: offsets, per-chunk bases and tiles of each expert
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    const int row_off = v[0];
    a.offsets[e] = row_off;
    int run = row_off;
    for (int64_t c = 0; c < n_chunks; ++c) {
      base[c * E + e] = run;
      run += __popcll(masks[c * E + e]);
    }
    const int cnt = run - row_off;
    a.counts[e] = cnt;
    emit_tiles(a, ts, e, row_off, cnt, v);
    v[0] = run;
  }
  if (tid == 0) write_totals(a, E, total);
}

// Phase 3: grouped row of every entry of chunk c.
__device__ __forceinline__ void place_entries(const int32_t* __restrict__ ids, int64_t T, int k, int E, int64_t c,
                              const unsigned long long* mask_c, const int32_t* base_c, int32_t* __restrict__ row_tok,
                              int32_t* __restrict__ slot_row, int flag_split) {
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
      // one chunk: its bitmap holds the expert's whole count
      if (flag_split >= 0 && __popcll(mask_c[e]) > flag_split) row |= kBigRowFlag;
    }
    slot_row[t * k + j] = row;
  }
}

// Activation re-layout: inside every 32-element block of a row, position
// p = 8i + 2t + h holds element 16h + 4i + t (i, t in 0..3, h in 0..1).  This
// is the order in which the GEMM decodes a block's nibble pairs (qs byte j
// holds elements j and j+16), so both MFMA operands see the same K order.
//
// Re-layout of the rows [t0, t0 + nt) of x into xp; this thread takes work
// items idx0, idx0 + stride, ... (item = one 8-element group of a row; idx0
// and stride are below 2^31).  The loads of kBatch items are issued before
// the first store, so a thread waits for one memory round trip per batch, not
// per item.  Items past the end are clamped onto the last one, which is then
// written more than once with the same bytes: no branch around the loads.
// The (row, group) of an item is stepped along, not divided out per item.
template <int kBatch>
__device__ __forceinline__ void permute_rows(const uint16_t* __restrict__ x, uint16_t* __restrict__ xp, int64_t t0,
                                             int64_t nt, int D, uint32_t idx0, uint32_t stride) {
  const uint32_t groups = (uint32_t)D / 8;
  if (groups == 0 || nt <= 0) return;
  const int64_t total = nt * groups;
  const uint32_t drow = stride / groups, dg = stride % groups;
  int64_t idx = idx0, row = t0 + idx0 / groups;
  uint32_t g = idx0 % groups;
  while (idx < total) {
    uint2 lo[kBatch], hi[kBatch];
    int64_t rows[kBatch];
    uint32_t grp[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool in = idx < total;
      rows[u] = in ? row : t0 + nt - 1;
      grp[u] = in ? g : groups - 1;
      const uint16_t* xrow = x + rows[u] * D;
      const uint32_t b = grp[u] >> 2, i = grp[u] & 3;
      lo[u] = *reinterpret_cast<const uint2*>(xrow + 32 * b + 4 * i);
      hi[u] = *reinterpret_cast<const uint2*>(xrow + 32 * b + 16 + 4 * i);
      idx += stride;
      row += drow;
      g += dg;
      if (g >= groups) {
        g -= groups;
        ++row;
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      uint4 o;
      o.x = __builtin_amdgcn_perm(hi[u].x, lo[u].x, 0x05040100u);  // elements 4i,   16+4i
      o.y = __builtin_amdgcn_perm(hi[u].x, lo[u].x, 0x07060302u);  // elements 4i+1, 17+4i
      o.z = __builtin_amdgcn_perm(hi[u].y, lo[u].y, 0x05040100u);  // elements 4i+2, 18+4i
      o.w = __builtin_amdgcn_perm(hi[u].y, lo[u].y, 0x07060302u);  // elements 4i+3, 19+4i
      *reinterpret_cast<uint4*>(xp + rows[u] * D + 8 * grp[u]) = o;
    }
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
  // totals: expert-parallel sums over the chunks, kScanLoads loads in flight
  // (the loads of consecutive threads are consecutive in memory)
  constexpr int kScanLoads = 8;
  for (int e = tid; e < E; e += kScanThreads) {
    int sum = 0;
    int64_t c = 0;
    for (; c + kScanLoads <= n_chunks; c += kScanLoads) {
      int32_t v[kScanLoads];
#pragma unroll
      for (int u = 0; u < kScanLoads; ++u) v[u] = a.chunk_base[(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < kScanLoads; ++u) sum += v[u];
    }
    for (; c < n_chunks; ++c) sum += a.chunk_base[c * E + e];
    ltot[e] = sum;
  }
  lds_barrier();
  // offsets and tiles: thread t owns experts 8t..8t+7
  const TileSpec ts = tile_spec(a);
  const int per = (E + kScanThreads - 1) / kScanThreads;
  const int e0 = tid * per;
  int v[1 + kTileLists] = {0, 0, 0, 0, 0};
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    add_expert(ts, ltot[e], v);
  }
  int total[1 + kTileLists];
  block_exclusive_scan_n(v, total);
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e >= E) break;
    const int cnt = ltot[e];
    a.counts[e] = cnt;
    a.offsets[e] = v[0];
    emit_tiles(a, ts, e, v[0], cnt, v);
    ltot[e] = v[0];  // reuse: the expert's first grouped row
    v[0] += cnt;
  }
  if (tid == 0) write_totals(a, E, total);
  lds_barrier();
  // bases: expert-parallel running sums over the chunks (loads kept in flight)
  for (int e = tid; e < E; e += kScanThreads) {
    int run = ltot[e];
    int64_t c = 0;
    for (; c + kScanLoads <= n_chunks; c += kScanLoads) {
      int32_t v[kScanLoads];
#pragma unroll
      for (int u = 0; u < kScanLoads; ++u) v[u] = a.chunk_base[(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < kScanLoads; ++u) {
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
      if (a.flag_big_rows && a.counts[e] > a.split_rows) row |= kBigRowFlag;
    }
    a.slot_row[t * a.k + j] = row;
  }
  const int64_t nt = (a.T - t0) < kChunkTokens ? (a.T - t0) : kChunkTokens;
  if (a.x_perm) permute_rows<8>(a.x, a.x_perm, t0, nt, a.D, part * blockDim.x + threadIdx.x, kPlaceParts * blockDim.x);
}

// All phases for a batch of at most one chunk (T <= 64), one launch.
// LDS: E bitmaps (8 B) + E bases (4 B).
__global__ __launch_bounds__(kScanThreads) void group_fused_kernel(GroupArgs a) {
  extern __shared__ unsigned long long lmask[];
  int32_t* lbase = reinterpret_cast<int32_t*>(lmask + a.E);
  build_masks(a.ids, a.T, a.k, a.E, 0, lmask);
  scan_experts(a, lmask, 1, lbase);
  lds_barrier();
  place_entries(a.ids, a.T, a.k, a.E, 0, lmask, lbase, a.row_tok, a.slot_row, a.flag_big_rows ? a.split_rows : -1);
  if (a.x_perm) permute_rows<4>(a.x, a.x_perm, 0, a.T, a.D, threadIdx.x, blockDim.x);
}

// All phases for a batch of at most 64 tokens and 1024 entries (decode-sized),
// one launch: thread i owns entry i for the whole kernel, one scan yields
// row offsets and the tile lists, and the activation re-layout comes last,
// where nothing waits for its stores.
// LDS: E bitmaps (8 B) + E first rows (4 B).
__global__ __launch_bounds__(kScanThreads) void group_small_kernel(GroupArgs a) {
  extern __shared__ unsigned long long lmask[];
  int32_t* lbase = reinterpret_cast<int32_t*>(lmask + a.E);
  __shared__ int32_t lids[kScanThreads];
  const int tid = threadIdx.x, E = a.E, k = a.k;
  const int entries = (int)a.T * k;
  const int my = tid < entries ? a.ids[tid] : -1;
  for (int i = tid; i < E; i += kScanThreads) lmask[i] = 0ull;
  lids[tid] = my;
  lds_barrier();
  // skip ids outside [0, E) and repeats of an earlier slot of the same token
  int e = -1;
  if (tid < entries && my >= 0 && my < E) {
    const int t = tid / k, j = tid - t * k;
    bool first = true;
    for (int jj = 0; jj < j; ++jj) first = first && lids[t * k + jj] != my;
    if (first) e = my;
  }
  if (e >= 0) atomicOr(&lmask[e], 1ull << (tid / k));
  lds_barrier();

  const TileSpec ts = tile_spec(a);
  const int per = (E + kScanThreads - 1) / kScanThreads;
  const int e0 = tid * per;
  int v[1 + kTileLists] = {0, 0, 0, 0, 0};
  for (int i = 0; i < per; ++i) {
    const int ex = e0 + i;
    if (ex >= E) break;
    add_expert(ts, __popcll(lmask[ex]), v);
  }
  int total[1 + kTileLists];
  block_exclusive_scan_n(v, total);
  for (int i = 0; i < per; ++i) {
    const int ex = e0 + i;
    if (ex >= E) break;
    const int cnt = __popcll(lmask[ex]);
    a.counts[ex] = cnt;
    a.offsets[ex] = v[0];
    lbase[ex] = v[0];
    emit_tiles(a, ts, ex, v[0], cnt, v);
    v[0] += cnt;
  }
  if (tid == 0) write_totals(a, E, total);
  lds_barrier();
  if (tid < entries) {
    const int t = tid / k;
    int32_t row = -1;
    if (e >= 0) {
      row = lbase[e] + __popcll(lmask[e] & ((1ull << t) - 1ull));
      a.row_tok[row] = t;
      if (a.flag_big_rows && __popcll(lmask[e]) > a.split_rows) row |= kBigRowFlag;
    }
    a.slot_row[tid] = row;
  }
  if (a.x_perm) permute_rows<4>(a.x, a.x_perm, 0, a.T, a.D, tid, kScanThreads);
}

// Activation re-layout only, for batches the gate/up launch groups itself.
__global__ __launch_bounds__(256) void permute_x_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ xp,
                                                         int64_t T, int D) {
  permute_rows<4>(x, xp, 0, T, D, blockIdx.x * blockDim.x + threadIdx.x, gridDim.x * blockDim.x);
}

}  // namespace

hipError_t launch_permute_x(const uint16_t* x, uint16_t* xp, int64_t T, int D, hipStream_t s) {
  const int64_t items = T * (int64_t)(D / 8);  // 8-element groups, four per thread
  int64_t blocks = (items + 4 * 256 - 1) / (4 * 256);
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  hipLaunchKernelGGL(permute_x_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, xp, T, D);
  return hipGetLastError();
}

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
