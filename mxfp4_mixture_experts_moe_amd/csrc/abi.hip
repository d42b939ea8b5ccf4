// Host side of the k3moe C ABI: argument checks, workspace layout, launches.
// Every check runs before anything is enqueued; nothing here aborts.
#include "k3moe.h"
#include "k3moe_internal.h"

#include <math.h>
#include <sys/syscall.h>
#include <unistd.h>

#include <atomic>
#include <mutex>

namespace k3moe {

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int64_t ffn_chunk_tokens(int64_t T, int32_t D, int32_t I, int32_t k) {
  // The GEMM kernels address x, h and the grouped rows through buffer
  // resources with 32-bit byte offsets: a chunk keeps k * max(D, I) * 2 bytes
  // per token below 2^31.  Chunks start on a multiple of 64 tokens (16-byte
  // aligned ids and weights for every k).
  const int64_t per_token = 2 * (int64_t)k * (int64_t)(D > I ? D : I);
  int64_t tc = (((int64_t)1 << 31) - 1) / per_token;
  tc = tc >= 64 ? tc / 64 * 64 : tc;
  if (tc < 1) tc = 1;
  return T < tc ? T : tc;
}

FfnWorkspace ffn_workspace_layout(int64_t T, int32_t D, int32_t I, int32_t E, int32_t k) {
  FfnWorkspace w{};
  const int64_t entries = T * (int64_t)k;
  const int64_t active = entries < E ? entries : E;
  w.max_tiles = entries / kMinTileRows + active;
  w.n_chunks = (T + kChunkTokens - 1) / kChunkTokens;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  w.counts = take(sizeof(int32_t) * (size_t)E);
  w.offsets = take(sizeof(int32_t) * (size_t)(E + 1));
  w.tile_count = take(kTileLists * sizeof(int32_t));
  for (int L = 0; L < kTileLists; ++L) w.tiles[L] = take(sizeof(Tile) * (size_t)(w.max_tiles > 0 ? w.max_tiles : 1));
  w.row_tok = take(sizeof(int32_t) * (size_t)entries);
  w.slot_row = take(sizeof(int32_t) * (size_t)entries);
  w.chunk_base = take(sizeof(int32_t) * (size_t)(w.n_chunks * E));
  w.chunk_mask = take(sizeof(unsigned long long) * (size_t)(w.n_chunks * E));
  w.x_perm = take(sizeof(uint16_t) * (size_t)(T * D));
  w.h = take(sizeof(uint16_t) * (size_t)(entries * I));
  w.h_lo = take(sizeof(uint16_t) * (size_t)(entries * I));
  w.h_scale = take((size_t)entries * (size_t)((I + 255) / 256));
  w.y = take(sizeof(float) * (size_t)(entries * D));
  w.y_scale = take((size_t)entries * (size_t)(D / 32));
  w.total = off;
  return w;
}

GroupWorkspace group_workspace_layout(int64_t T, int32_t E, int32_t k) {
  GroupWorkspace w{};
  const int64_t entries = T * (int64_t)k;
  const int64_t active = entries < E ? entries : E;
  w.max_tiles = entries / kGroupTileRows + active;
  w.n_chunks = (T + kChunkTokens - 1) / kChunkTokens;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  w.tile_count = take(kTileLists * sizeof(int32_t));
  for (int L = 0; L < kTileLists; ++L) w.tiles[L] = take(sizeof(Tile) * (size_t)(w.max_tiles > 0 ? w.max_tiles : 1));
  w.chunk_base = take(sizeof(int32_t) * (size_t)(w.n_chunks * E));
  w.chunk_mask = take(sizeof(unsigned long long) * (size_t)(w.n_chunks * E));
  w.total = off;
  return w;
}

}  // namespace k3moe

using namespace k3moe;

namespace {

constexpr int kMaxDevices = 64;

bool misaligned(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int device_status(hipError_t e) { return e == hipSuccess ? K3MOE_OK : K3MOE_ERR_DEVICE; }

// ---------------------------------------------------------------------------
// Side stream (default priority) and fork / join events of the calling host
// thread on each device, created by the thread's first call outside a graph
// capture that has experts of both GEMM kinds.  A thread other than the
// process's main thread destroys them when it exits; the main thread's are
// left to the end of the process (its thread-local objects are destroyed
// during exit, possibly after the HIP runtime).
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
struct ThreadSideStreams {
  SideStream dev[kMaxDevices];
  bool tried[kMaxDevices] = {};
  ~ThreadSideStreams() {
    if ((pid_t)syscall(SYS_gettid) == getpid()) return;
    for (int d = 0; d < kMaxDevices; ++d) {
      if (dev[d].s) (void)hipStreamDestroy(dev[d].s);
      if (dev[d].fork) (void)hipEventDestroy(dev[d].fork);
      if (dev[d].join) (void)hipEventDestroy(dev[d].join);
    }
  }
};
thread_local ThreadSideStreams t_side;

// The calling thread's side stream for a call on `caller`, or nullptr when the
// launches must stay on `caller`: no side stream yet and `caller` is being
// captured (creating one then is not allowed), the runtime refused one, or the
// side stream already belongs to an open capture other than `caller`'s (it
// joined that capture through an earlier call of this thread).
SideStream* side_stream(hipStream_t caller) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  unsigned long long cid = 0;
  if (hipStreamGetCaptureInfo(caller, &cs, &cid) != hipSuccess) return nullptr;
  SideStream& ss = t_side.dev[dev];
  if (!t_side.tried[dev]) {
    if (cs != hipStreamCaptureStatusNone) return nullptr;
    t_side.tried[dev] = true;
    if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
      if (ss.s) (void)hipStreamDestroy(ss.s);
      if (ss.fork) (void)hipEventDestroy(ss.fork);
      if (ss.join) (void)hipEventDestroy(ss.join);
      ss = SideStream{};
    }
  }
  if (!ss.s) return nullptr;
  hipStreamCaptureStatus side_cs = hipStreamCaptureStatusNone;
  unsigned long long side_id = 0;
  if (hipStreamGetCaptureInfo(ss.s, &side_cs, &side_id) != hipSuccess) return nullptr;
  if (side_cs != hipStreamCaptureStatusNone && (cs != hipStreamCaptureStatusActive || side_id != cid)) return nullptr;
  return &ss;
}

// ---------------------------------------------------------------------------
// Fixed scratch of moe_mxfp4_ffn_noalloc: one copy per device, held from the
// library's first use on that device until the process ends.  Host code never
// passes the array's name (a host-side stand-in) to a kernel; it uses the
// device address looked up once per device.
static __device__ __align__(256) uint8_t scratch[K3MOE_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (nullptr if the runtime
// refuses the lookup).
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress((void**)&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

// ---------------------------------------------------------------------------
int ffn_shape_status(int64_t T, int32_t D, int32_t I, int32_t E, int32_t k) {
  if (T < 0 || D <= 0 || I <= 0 || (D % 32) != 0 || (I % 32) != 0) return K3MOE_ERR_SHAPE;
  if (D > K3MOE_MAX_DIM_FFN || I > K3MOE_MAX_DIM_FFN) return K3MOE_ERR_SHAPE;
  if (E < 1 || E > K3MOE_MAX_EXPERTS_FFN || k < 1 || k > E || k > K3MOE_MAX_TOPK) return K3MOE_ERR_SHAPE;
  // grouped rows are int32 inside the kernels
  if (T * (int64_t)k > 0x7FFFFFFF || T > 0x7FFFFFFF) return K3MOE_ERR_SHAPE;
  return K3MOE_OK;
}

// Events recorded at the launch boundaries (moe_mxfp4_ffn_profiled).
enum { kEvGroup = 0, kEvGateUp, kEvGateUpStream, kEvDown, kEvDownStream, kEvCombine, kEvEnd };
static_assert(kEvEnd + 1 == K3MOE_FFN_STAGE_EVENTS, "event slots");

// One chunk of at most ffn_chunk_tokens() tokens: grouping, gate/up, down,
// combine, enqueued on `s` (the streaming launches on a side stream when
// `side` is set).
int run_ffn_chunk(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1,
                  const uint8_t* w3, const uint8_t* w2, int64_t T, int32_t D, int32_t I, int32_t E, int32_t k,
                  void* out, bool out_bf16, uint8_t* ws, hipStream_t s, void* const* stage_events,
                  bool allow_side) {
  const FfnWorkspace L = ffn_workspace_layout(T, D, I, E, k);
  const int64_t entries = T * (int64_t)k;
  const int64_t active = entries < E ? entries : E;
  // GEMM kernels.  With D and I multiples of 512 every expert is served by
  // the kernel that suits its row count: the large-tile GEMMs for experts
  // with more than kStreamMaxRows rows (MFMA-bound), the weight-streaming
  // GEMMs for the others (HBM-bound; in a grouped batch the shared-tile
  // form, whose 16-row gate/up and 8-row down tiles stream an expert of up
  // to 16 rows once).  Batches of up to kStreamOnlyTokens tokens send every
  // expert to the streaming kernels (an expert with more rows than a tile
  // takes several, whose repeated weight reads mostly hit the caches), so
  // decode steps skip the large-tile launches.  Other shapes use the general
  // small-tile GEMMs for every expert.
  constexpr int kStreamMaxRows = 16;
  constexpr int kStreamOnlyTokens = 8;
  const bool tiled = big_gemm_supported(D, I) && stream_gemm_supported(D, I);
  const bool stream_only = tiled && T <= kStreamOnlyTokens;
  const bool big_lists = !tiled || !stream_only;  // lists 0/1 may hold tiles
  const bool stream_lists = tiled;                // lists 2/3 may hold tiles
  const int rpt_small = choose_rows_per_tile(T, k, E);
  // 128-row down tiles once the batch is large enough that the large-tile
  // down product still has about four workgroups per CU with them
  constexpr int64_t kWideDownEntries = 16384;
  const bool wide_down = entries >= kWideDownEntries;

  GroupArgs g{};
  g.ids = topk_ids;
  g.x = static_cast<const uint16_t*>(x_bf16);
  g.T = T;
  g.D = D;
  g.E = E;
  g.k = k;
  g.rows_per_tile[0] = tiled ? big_rows_per_tile(true, false) : rpt_small;
  g.rows_per_tile[1] = tiled ? big_rows_per_tile(false, wide_down) : rpt_small;
  // A streaming-only batch of at most kSelfGroupEntries entries is grouped by
  // the gate/up launch itself (no grouping launch), in the per-wave streaming
  // form's 4-row gate/up and 2-row down tiles.  Up to kNaturalXTokens tokens
  // that launch also reads x in place; larger decode batches have x re-laid
  // out first by a small launch, as the operand reads of pre-permuted x keep
  // the gate/up stream faster.  Grouped batches stream in the shared-tile form.
  constexpr int kNaturalXTokens = 4;
  const bool self_group = stream_only && entries <= kSelfGroupEntries && E <= 0xFFFF;
  const bool natural_x = self_group && T <= kNaturalXTokens;
  g.rows_per_tile[2] = self_group ? stream_rows_per_tile(true) : stream_shared_rows_per_tile(true);
  g.rows_per_tile[3] = self_group ? stream_rows_per_tile(false) : stream_shared_rows_per_tile(false);
  g.split_rows = tiled ? (stream_only ? kStreamOnlyTokens : kStreamMaxRows) : 0;
  g.flag_big_rows = tiled ? 1 : 0;  // the large-tile down kernel's rows hold scaled fp16 y
  g.counts = reinterpret_cast<int32_t*>(ws + L.counts);
  g.offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  g.tile_count = reinterpret_cast<int32_t*>(ws + L.tile_count);
  for (int l = 0; l < kTileLists; ++l) g.tiles[l] = reinterpret_cast<Tile*>(ws + L.tiles[l]);
  g.row_tok = reinterpret_cast<int32_t*>(ws + L.row_tok);
  g.slot_row = reinterpret_cast<int32_t*>(ws + L.slot_row);
  g.chunk_base = reinterpret_cast<int32_t*>(ws + L.chunk_base);
  g.chunk_mask = reinterpret_cast<unsigned long long*>(ws + L.chunk_mask);
  g.x_perm = reinterpret_cast<uint16_t*>(ws + L.x_perm);
  auto mark = [&](int i) -> bool {
    if (!stage_events || !stage_events[i]) return true;
    return hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), s) == hipSuccess;
  };
  if (!mark(kEvGroup)) return K3MOE_ERR_DEVICE;
  hipError_t err = self_group ? (natural_x ? hipSuccess : launch_permute_x(g.x, g.x_perm, T, D, s)) : launch_group(g, s);
  if (err != hipSuccess) return K3MOE_ERR_DEVICE;

  // Upper bounds of the list lengths (sum over experts of ceil(n_e / rpt)):
  // an expert in lists 0/1 has more than split_rows rows.
  const int64_t big_experts = tiled ? (entries / (kStreamMaxRows + 1) < active ? entries / (kStreamMaxRows + 1) : active)
                                    : active;
  GemmArgs gu{};
  gu.act = g.x_perm;
  gu.act_rows = T;
  gu.row_tok = g.row_tok;
  gu.wa = w1;
  gu.wb = w3;
  gu.K = D;
  gu.N = I;
  gu.out = ws + L.h;
  gu.out_lo = ws + L.h_lo;
  gu.h_scale = reinterpret_cast<int8_t*>(ws + L.h_scale);
  GemmArgs dn{};
  dn.act = reinterpret_cast<const uint16_t*>(ws + L.h);
  dn.act_lo = reinterpret_cast<const uint16_t*>(ws + L.h_lo);
  dn.act_rows = entries;
  dn.row_tok = nullptr;
  dn.wa = w2;
  dn.wb = nullptr;
  dn.K = I;
  dn.N = D;
  dn.out = ws + L.y;
  dn.h_scale = reinterpret_cast<int8_t*>(ws + L.h_scale);
  dn.y_scale = reinterpret_cast<int8_t*>(ws + L.y_scale);

  // Experts of both kinds in one call (and no stage events to record): the
  // streaming launches run on a side stream beside the large-tile launches;
  // they read the same inputs and write other rows of h and y.  The combine
  // waits for both branches.
  SideStream* side = (allow_side && big_lists && stream_lists && !stage_events) ? side_stream(s) : nullptr;
  hipStream_t ss = s;
  if (side) {
    if (hipEventRecord(side->fork, s) != hipSuccess || hipStreamWaitEvent(side->s, side->fork, 0) != hipSuccess)
      return K3MOE_ERR_DEVICE;
    ss = side->s;
  }

  // gate/up
  if (!mark(kEvGateUp)) return K3MOE_ERR_DEVICE;
  if (big_lists) {
    gu.tiles = g.tiles[0];
    gu.tile_count = g.tile_count;
    gu.max_tiles = entries / g.rows_per_tile[0] + big_experts;
    err = tiled ? launch_big_gate_up(gu, s) : launch_gate_up(gu, rpt_small, s);
    if (err != hipSuccess) return K3MOE_ERR_DEVICE;
  }
  if (!mark(kEvGateUpStream)) return K3MOE_ERR_DEVICE;
  if (stream_lists) {
    gu.tiles = g.tiles[2];
    gu.tile_count = g.tile_count + 2;
    const int64_t r = g.rows_per_tile[2];
    gu.max_tiles = (entries + (r - 1) * active) / r;  // bounds the sum of ceil(n_e / r) over experts
    if (self_group) {
      SelfGroupArgs sg{};
      sg.ids = topk_ids;
      sg.T = (int)T;
      sg.E = E;
      sg.k = k;
      sg.tile_count = g.tile_count;
      sg.down_tiles = g.tiles[3];
      sg.slot_row = g.slot_row;
      gu.act = natural_x ? static_cast<const uint16_t*>(x_bf16) : g.x_perm;
      gu.row_tok = nullptr;
      err = launch_stream_gate_up_grouped(gu, sg, natural_x, ss);
    } else {
      err = launch_stream_shared(gu, true, ss);
    }
    if (err != hipSuccess) return K3MOE_ERR_DEVICE;
  }

  // down
  if (!mark(kEvDown)) return K3MOE_ERR_DEVICE;
  if (big_lists) {
    dn.tiles = g.tiles[1];
    dn.tile_count = g.tile_count + 1;
    dn.max_tiles = entries / g.rows_per_tile[1] + big_experts;
    err = tiled ? launch_big_down(dn, wide_down, s) : launch_down(dn, rpt_small, s);
    if (err != hipSuccess) return K3MOE_ERR_DEVICE;
  }
  if (!mark(kEvDownStream)) return K3MOE_ERR_DEVICE;
  if (stream_lists) {
    dn.tiles = g.tiles[3];
    dn.tile_count = g.tile_count + 3;
    const int64_t r = g.rows_per_tile[3];
    dn.max_tiles = (entries + (r - 1) * active) / r;  // bounds the sum of ceil(n_e / r) over experts
    err = self_group ? launch_stream_down(dn, ss) : launch_stream_shared(dn, false, ss);
    if (err != hipSuccess) return K3MOE_ERR_DEVICE;
  }
  if (side) {
    if (hipEventRecord(side->join, side->s) != hipSuccess || hipStreamWaitEvent(s, side->join, 0) != hipSuccess)
      return K3MOE_ERR_DEVICE;
  }
  if (!mark(kEvCombine)) return K3MOE_ERR_DEVICE;

  // Rows of the large-tile down kernel hold scaled fp16 y; a streaming-only
  // batch has none, so its combine reads fp32 rows only.
  const bool mixed_rows = tiled && !stream_only;
  if (out_bf16)
    err = launch_combine_bf16(reinterpret_cast<const float*>(ws + L.y), reinterpret_cast<const int8_t*>(ws + L.y_scale),
                              mixed_rows, g.slot_row, topk_w, T, D, k, static_cast<uint16_t*>(out), s);
  else
    err = launch_combine(reinterpret_cast<const float*>(ws + L.y), reinterpret_cast<const int8_t*>(ws + L.y_scale),
                         mixed_rows, g.slot_row, topk_w, T, D, k, static_cast<float*>(out), s);
  if (err != hipSuccess || !mark(kEvEnd)) return K3MOE_ERR_DEVICE;
  return K3MOE_OK;
}

// The FFN over all T tokens, one chunk of ffn_chunk_tokens() after another
// (the chunks reuse one workspace; stream order serialises them).
int run_ffn(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1, const uint8_t* w3,
            const uint8_t* w2, int64_t T, int32_t D, int32_t I, int32_t E, int32_t k, void* out, bool out_bf16,
            uint8_t* ws, hipStream_t s, void* const* stage_events, bool allow_side) {
  const int64_t tc = ffn_chunk_tokens(T, D, I, k);
  for (int64_t t0 = 0; t0 < T; t0 += tc) {
    const int64_t n = T - t0 < tc ? T - t0 : tc;
    void* o = static_cast<uint8_t*>(out) + t0 * D * (out_bf16 ? 2 : 4);
    const int st = run_ffn_chunk(static_cast<const uint16_t*>(x_bf16) + t0 * D, topk_ids + t0 * k, topk_w + t0 * k,
                                 w1, w3, w2, n, D, I, E, k, o, out_bf16, ws, s, stage_events, allow_side);
    if (st != K3MOE_OK) return st;
  }
  return K3MOE_OK;
}

// The FFN over Q4_K experts, one chunk: grouping (every expert in lists 0/1,
// 16-row gate/up and 8-row down tiles, x read in place), the two Q4_K GEMMs,
// combine.  Events (if given) mark the same launch boundaries as the MXFP4
// path's; the streaming slots stay empty.
int run_q4k_chunk(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1,
                  const uint8_t* w3, const uint8_t* w2, int64_t T, int32_t D, int32_t I, int32_t E, int32_t k,
                  float* out, uint8_t* ws, hipStream_t s, void* const* stage_events) {
  const FfnWorkspace L = ffn_workspace_layout(T, D, I, E, k);
  const int64_t entries = T * (int64_t)k;
  const int64_t active = entries < E ? entries : E;
  GroupArgs g{};
  g.ids = topk_ids;
  g.x = static_cast<const uint16_t*>(x_bf16);
  g.T = T;
  g.D = D;
  g.E = E;
  g.k = k;
  g.rows_per_tile[0] = g.rows_per_tile[2] = q4k_rows_per_tile(true);
  g.rows_per_tile[1] = g.rows_per_tile[3] = q4k_rows_per_tile(false);
  g.split_rows = -1;  // every expert in lists 0 / 1
  g.flag_big_rows = 0;
  g.counts = reinterpret_cast<int32_t*>(ws + L.counts);
  g.offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  g.tile_count = reinterpret_cast<int32_t*>(ws + L.tile_count);
  for (int l = 0; l < kTileLists; ++l) g.tiles[l] = reinterpret_cast<Tile*>(ws + L.tiles[l]);
  g.row_tok = reinterpret_cast<int32_t*>(ws + L.row_tok);
  g.slot_row = reinterpret_cast<int32_t*>(ws + L.slot_row);
  g.chunk_base = reinterpret_cast<int32_t*>(ws + L.chunk_base);
  g.chunk_mask = reinterpret_cast<unsigned long long*>(ws + L.chunk_mask);
  g.x_perm = nullptr;
  auto mark = [&](int i) -> bool {
    if (!stage_events || !stage_events[i]) return true;
    return hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), s) == hipSuccess;
  };
  if (!mark(kEvGroup) || launch_group(g, s) != hipSuccess) return K3MOE_ERR_DEVICE;

  GemmArgs gu{};
  gu.act = static_cast<const uint16_t*>(x_bf16);
  gu.act_rows = T;
  gu.row_tok = g.row_tok;
  gu.wa = w1;
  gu.wb = w3;
  gu.tiles = g.tiles[0];
  gu.tile_count = g.tile_count;
  const int64_t r_gu = q4k_rows_per_tile(true);
  gu.max_tiles = (entries + (r_gu - 1) * active) / r_gu;  // bounds the sum of ceil(n_e / r) over experts
  gu.K = D;
  gu.N = I;
  gu.out = ws + L.h;
  gu.out_lo = ws + L.h_lo;
  if (!mark(kEvGateUp) || launch_q4k_gemm(gu, true, s) != hipSuccess || !mark(kEvGateUpStream))
    return K3MOE_ERR_DEVICE;

  GemmArgs dn{};
  dn.act = reinterpret_cast<const uint16_t*>(ws + L.h);
  dn.act_lo = reinterpret_cast<const uint16_t*>(ws + L.h_lo);
  dn.act_rows = entries;
  dn.wa = w2;
  dn.tiles = g.tiles[1];
  dn.tile_count = g.tile_count + 1;
  const int64_t r_dn = q4k_rows_per_tile(false);
  dn.max_tiles = (entries + (r_dn - 1) * active) / r_dn;
  dn.K = I;
  dn.N = D;
  dn.out = ws + L.y;
  if (!mark(kEvDown) || launch_q4k_gemm(dn, false, s) != hipSuccess || !mark(kEvDownStream) || !mark(kEvCombine))
    return K3MOE_ERR_DEVICE;
  if (launch_combine(reinterpret_cast<const float*>(ws + L.y), nullptr, false, g.slot_row, topk_w, T, D, k, out, s) !=
          hipSuccess ||
      !mark(kEvEnd))
    return K3MOE_ERR_DEVICE;
  return K3MOE_OK;
}

int q4k_shape_status(int64_t T, int32_t D, int32_t I, int32_t E, int32_t k) {
  const int st = ffn_shape_status(T, D, I, E, k);
  if (st != K3MOE_OK) return st;
  return q4k_gemm_supported(D, I) ? K3MOE_OK : K3MOE_ERR_SHAPE;
}

// Argument checks shared by the FFN entry points (workspace excluded).
int ffn_arg_status(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1,
                   const uint8_t* w3, const uint8_t* w2, int64_t T, int32_t D, int32_t I, int32_t E, int32_t k,
                   int32_t act, const float* out) {
  const int st = ffn_shape_status(T, D, I, E, k);
  if (st != K3MOE_OK) return st;
  if (act != K3MOE_ACT_SILU_MUL) return K3MOE_ERR_UNSUPPORTED;
  if (T == 0) return K3MOE_OK;
  if (!x_bf16 || !topk_ids || !topk_w || !w1 || !w3 || !w2 || !out) return K3MOE_ERR_NULL;
  if (misaligned(x_bf16) || misaligned(topk_ids) || misaligned(topk_w) || misaligned(w1) || misaligned(w3) ||
      misaligned(w2) || misaligned(out))
    return K3MOE_ERR_ALIGN;
  return K3MOE_OK;
}

}  // namespace

extern "C" {

const char* k3moe_status_str(int status) {
  switch (status) {
    case K3MOE_OK: return "ok";
    case K3MOE_ERR_NULL: return "a required pointer is NULL";
    case K3MOE_ERR_SHAPE: return "a size argument is out of range or inconsistent";
    case K3MOE_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case K3MOE_ERR_WORKSPACE: return "workspace is smaller than moe_mxfp4_ffn_workspace_size()";
    case K3MOE_ERR_UNSUPPORTED: return "unsupported enum value";
    case K3MOE_ERR_DEVICE: return "the HIP runtime refused a launch";
    case K3MOE_ERR_TOO_LARGE:
      return "the sizes need more workspace than the library's fixed scratch holds (K3MOE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int moe_route_topk(const float* logits, const float* bias, int64_t T, int32_t E, int32_t k, int32_t normalize,
                   float route_scale, int32_t* topk_ids, float* topk_w, void* stream) {
  if (T < 0 || E < 1 || k < 1 || k > E || k > K3MOE_MAX_TOPK) return K3MOE_ERR_SHAPE;
  if (T > (int64_t)0x7FFFFFFF * 4) return K3MOE_ERR_SHAPE;  // grid limit
  if (T == 0) return K3MOE_OK;
  if (!logits || !topk_ids || !topk_w) return K3MOE_ERR_NULL;
  if (misaligned(logits) || misaligned(bias) || misaligned(topk_ids) || misaligned(topk_w)) return K3MOE_ERR_ALIGN;
  return device_status(launch_route_topk(logits, bias, T, E, k, normalize, route_scale, topk_ids, topk_w,
                                         static_cast<hipStream_t>(stream)));
}

int mxfp4_repack(const uint8_t* packed, const uint8_t* scale, int64_t R, int64_t K, uint8_t* blocks,
                 void* stream) {
  if (R < 0 || K <= 0 || (K % 32) != 0) return K3MOE_ERR_SHAPE;
  const int64_t nblocks = R * (K / 32);
  if (nblocks / 1024 > 0x7FFFFFFF) return K3MOE_ERR_SHAPE;
  if (R == 0) return K3MOE_OK;
  if (!packed || !scale || !blocks) return K3MOE_ERR_NULL;
  if (misaligned(packed) || misaligned(scale) || misaligned(blocks)) return K3MOE_ERR_ALIGN;
  return device_status(launch_repack(packed, scale, nblocks, blocks, static_cast<hipStream_t>(stream)));
}

int mxfp4_tile(const uint8_t* src, int64_t nmat, int64_t N, int64_t K, uint8_t* dst, void* stream) {
  if (nmat < 0 || N < 1 || N > 0x7FFFFFFF || K <= 0 || (K % 32) != 0 || K / 32 > 0x7FFFFFFF) return K3MOE_ERR_SHAPE;
  const int64_t nb = K / 32;
  const int64_t pieces = ((N + 15) / 16) * ((nb + 15) / 16);
  if (nmat > 0 && pieces > 0x7FFFFFFF / nmat) return K3MOE_ERR_SHAPE;
  if (nmat == 0) return K3MOE_OK;
  if (!src || !dst) return K3MOE_ERR_NULL;
  if (misaligned(src) || misaligned(dst)) return K3MOE_ERR_ALIGN;
  const uint64_t bytes = (uint64_t)nmat * (uint64_t)N * (uint64_t)nb * 17u;
  const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
  if (a < b + bytes && b < a + bytes) return K3MOE_ERR_SHAPE;  // overlapping buffers
  return device_status(launch_tile(src, nmat, (int)N, (int)nb, dst, static_cast<hipStream_t>(stream)));
}

int mxfp4_dequant(const uint8_t* blocks, int64_t R, int64_t K, int32_t out_dtype, void* out, void* stream) {
  if (R < 0 || K <= 0 || (K % 32) != 0) return K3MOE_ERR_SHAPE;
  if (out_dtype != K3MOE_DTYPE_F32 && out_dtype != K3MOE_DTYPE_BF16) return K3MOE_ERR_UNSUPPORTED;
  const int64_t nblocks = R * (K / 32);
  if (nblocks / 256 > 0x7FFFFFFF) return K3MOE_ERR_SHAPE;
  if (R == 0) return K3MOE_OK;
  if (!blocks || !out) return K3MOE_ERR_NULL;
  if (misaligned(blocks) || misaligned(out)) return K3MOE_ERR_ALIGN;
  return device_status(launch_dequant(blocks, nblocks, out_dtype == K3MOE_DTYPE_BF16, out,
                                      static_cast<hipStream_t>(stream)));
}

size_t moe_mxfp4_ffn_workspace_size(int64_t T, int32_t D, int32_t I, int32_t E, int32_t k) {
  if (ffn_shape_status(T, D, I, E, k) != K3MOE_OK || T == 0) return 0;
  return ffn_workspace_layout(ffn_chunk_tokens(T, D, I, k), D, I, E, k).total;
}

int moe_mxfp4_ffn(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1,
                  const uint8_t* w3, const uint8_t* w2, int64_t T, int32_t D, int32_t I, int32_t E, int32_t k,
                  int32_t act, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return moe_mxfp4_ffn_profiled(x_bf16, topk_ids, topk_w, w1, w3, w2, T, D, I, E, k, act, out, workspace,
                                workspace_bytes, stream, nullptr);
}

int moe_mxfp4_ffn_profiled(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1,
                           const uint8_t* w3, const uint8_t* w2, int64_t T, int32_t D, int32_t I, int32_t E,
                           int32_t k, int32_t act, float* out, void* workspace, size_t workspace_bytes,
                           void* stream, void* const* stage_events) {
  int st = ffn_arg_status(x_bf16, topk_ids, topk_w, w1, w3, w2, T, D, I, E, k, act, out);
  if (st != K3MOE_OK || T == 0) return st;
  if (!workspace) return K3MOE_ERR_NULL;
  if (misaligned(workspace)) return K3MOE_ERR_ALIGN;
  if (workspace_bytes < moe_mxfp4_ffn_workspace_size(T, D, I, E, k)) return K3MOE_ERR_WORKSPACE;
  return run_ffn(x_bf16, topk_ids, topk_w, w1, w3, w2, T, D, I, E, k, out, false, static_cast<uint8_t*>(workspace),
                 static_cast<hipStream_t>(stream), stage_events, true);
}

int moe_mxfp4_ffn_noalloc(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1,
                          const uint8_t* w3, const uint8_t* w2, int64_t T, int32_t D, int32_t I, int32_t E,
                          int32_t k, int32_t act, float* out, void* stream) {
  int st = ffn_arg_status(x_bf16, topk_ids, topk_w, w1, w3, w2, T, D, I, E, k, act, out);
  if (st != K3MOE_OK || T == 0) return st;
  if (moe_mxfp4_ffn_workspace_size(T, D, I, E, k) > (size_t)K3MOE_NOALLOC_SCRATCH_BYTES) return K3MOE_ERR_TOO_LARGE;
  void* ws = scratch_ptr();
  if (!ws) return K3MOE_ERR_DEVICE;
  // every launch on the caller's stream: no side stream (creating one may allocate)
  return run_ffn(x_bf16, topk_ids, topk_w, w1, w3, w2, T, D, I, E, k, out, false, static_cast<uint8_t*>(ws),
                 static_cast<hipStream_t>(stream), nullptr, false);
}

size_t moe_q4k_ffn_workspace_size(int64_t T, int32_t D, int32_t I, int32_t E, int32_t k) {
  if (q4k_shape_status(T, D, I, E, k) != K3MOE_OK || T == 0) return 0;
  return ffn_workspace_layout(ffn_chunk_tokens(T, D, I, k), D, I, E, k).total;
}

int moe_q4k_ffn(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1,
                const uint8_t* w3, const uint8_t* w2, int64_t T, int32_t D, int32_t I, int32_t E, int32_t k,
                int32_t act, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  return moe_q4k_ffn_profiled(x_bf16, topk_ids, topk_w, w1, w3, w2, T, D, I, E, k, act, out, workspace,
                              workspace_bytes, stream, nullptr);
}

int moe_q4k_ffn_profiled(const void* x_bf16, const int32_t* topk_ids, const float* topk_w, const uint8_t* w1,
                         const uint8_t* w3, const uint8_t* w2, int64_t T, int32_t D, int32_t I, int32_t E, int32_t k,
                         int32_t act, float* out, void* workspace, size_t workspace_bytes, void* stream,
                         void* const* stage_events) {
  int st = ffn_arg_status(x_bf16, topk_ids, topk_w, w1, w3, w2, T, D, I, E, k, act, out);
  if (st != K3MOE_OK) return st;
  st = q4k_shape_status(T, D, I, E, k);
  if (st != K3MOE_OK || T == 0) return st;
  if (!workspace) return K3MOE_ERR_NULL;
  if (misaligned(workspace)) return K3MOE_ERR_ALIGN;
  if (workspace_bytes < moe_q4k_ffn_workspace_size(T, D, I, E, k)) return K3MOE_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t tc = ffn_chunk_tokens(T, D, I, k);
  for (int64_t t0 = 0; t0 < T; t0 += tc) {
    const int64_t n = T - t0 < tc ? T - t0 : tc;
    st = run_q4k_chunk(static_cast<const uint16_t*>(x_bf16) + t0 * D, topk_ids + t0 * k, topk_w + t0 * k, w1, w3, w2,
                       n, D, I, E, k, out + t0 * D, static_cast<uint8_t*>(workspace), s, stage_events);
    if (st != K3MOE_OK) return st;
  }
  return K3MOE_OK;
}

int moe_verify_width_distinct(const int32_t* topk_ids, int32_t S, int32_t W, int32_t E, int32_t k, int32_t* distinct,
                              void* stream) {
  if (S < 0 || W < 1 || W > K3MOE_MAX_VERIFY_WIDTH || E < 1 || E > K3MOE_MAX_EXPERTS_FFN || k < 1 ||
      k > K3MOE_MAX_TOPK)
    return K3MOE_ERR_SHAPE;
  if ((int64_t)S * W * k > 0x7FFFFFFF) return K3MOE_ERR_SHAPE;
  if (!distinct) return K3MOE_ERR_NULL;
  if (S > 0 && !topk_ids) return K3MOE_ERR_NULL;
  if (misaligned(topk_ids) || misaligned(distinct)) return K3MOE_ERR_ALIGN;
  return device_status(launch_verify_distinct(topk_ids, S, W, E, k, distinct, static_cast<hipStream_t>(stream)));
}

int moe_verify_width_choose(const int32_t* distinct, int32_t W, int32_t S, const double* accept, double expert_bytes,
                            double bytes_per_s, double fixed_s, int32_t* best_w, double* rates) {
  if (W < 1 || W > K3MOE_MAX_VERIFY_WIDTH || S < 1) return K3MOE_ERR_SHAPE;
  if (!distinct || !best_w) return K3MOE_ERR_NULL;
  if (!(expert_bytes >= 0.0) || !(bytes_per_s > 0.0) || !(fixed_s >= 0.0)) return K3MOE_ERR_SHAPE;
  int best = 1;
  double best_rate = -1.0;
  double committed = 1.0, run = 1.0;  // expected tokens one sequence commits at width w
  for (int w = 1; w <= W; ++w) {
    if (w > 1) {
      run *= accept ? accept[w - 2] : 1.0;
      committed += run;
    }
    const double t = fixed_s + (double)distinct[w - 1] * expert_bytes / bytes_per_s;
    const double rate = (double)S * committed / t;
    if (rates) rates[w - 1] = rate;
    if (rate > best_rate) {  // strictly higher: ties keep the smaller width
      best_rate = rate;
      best = w;
    }
  }
  *best_w = best;
  return K3MOE_OK;
}

size_t moe_expert_cache_state_size(int32_t E, int32_t C) {
  if (E < 1 || C < 1 || E > K3MOE_MAX_EXPERTS_FFN || C > K3MOE_MAX_EXPERTS_FFN) return 0;
  return cache_state_view(nullptr, E, C).bytes;
}

int moe_expert_cache_init(void* state, size_t state_bytes, int32_t E, int32_t C, void* stream) {
  const size_t need = moe_expert_cache_state_size(E, C);
  if (need == 0) return K3MOE_ERR_SHAPE;
  if (!state) return K3MOE_ERR_NULL;
  if (misaligned(state)) return K3MOE_ERR_ALIGN;
  if (state_bytes < need) return K3MOE_ERR_WORKSPACE;
  return device_status(launch_cache_init(cache_state_view(state, E, C), static_cast<hipStream_t>(stream)));
}

// A pointer the GPU can read, for the store: device memory as it is, pinned
// host memory through its device mapping; nullptr for anything else.
static const uint8_t* device_readable(const uint8_t* p) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of an unknown pointer
    return nullptr;
  }
  if (at.type == hipMemoryTypeDevice) return p;
  if (at.type == hipMemoryTypeHost && at.devicePointer) return static_cast<const uint8_t*>(at.devicePointer);
  return nullptr;
}

// Both cache entry points: `block` weights per `bytes` bytes (MXFP4: 32 per 17,
// Q4_K: 256 per 144); the experts are copied whole, so the kernels never look
// inside the blocks.
static int cache_route(void* state, size_t state_bytes, int32_t E, int32_t C, const int32_t* topk_ids, int64_t T,
                       int32_t k, int32_t* slot_ids, const uint8_t* store_w1, const uint8_t* store_w3,
                       const uint8_t* store_w2, uint8_t* cache_w1, uint8_t* cache_w3, uint8_t* cache_w2, int32_t D,
                       int32_t I, int32_t block, int32_t bytes, void* stream) {
  const size_t need = moe_expert_cache_state_size(E, C);
  if (need == 0 || T < 0 || k < 1 || k > K3MOE_MAX_TOPK) return K3MOE_ERR_SHAPE;
  if (D <= 0 || I <= 0 || (D % block) != 0 || (I % block) != 0 || D > K3MOE_MAX_DIM_FFN || I > K3MOE_MAX_DIM_FFN)
    return K3MOE_ERR_SHAPE;
  if (T * (int64_t)k > 0x7FFFFFFF) return K3MOE_ERR_SHAPE;
  const int64_t entries = T * (int64_t)k;
  if ((int64_t)C < (entries < E ? entries : (int64_t)E)) return K3MOE_ERR_SHAPE;
  if (T == 0) return K3MOE_OK;
  if (!state || !topk_ids || !slot_ids || !store_w1 || !store_w3 || !store_w2 || !cache_w1 || !cache_w3 || !cache_w2)
    return K3MOE_ERR_NULL;
  if (misaligned(state) || misaligned(topk_ids) || misaligned(slot_ids) || misaligned(store_w1) ||
      misaligned(store_w3) || misaligned(store_w2) || misaligned(cache_w1) || misaligned(cache_w3) ||
      misaligned(cache_w2))
    return K3MOE_ERR_ALIGN;
  if (state_bytes < need) return K3MOE_ERR_WORKSPACE;
  CacheFetchArgs f{};
  f.store_w1 = device_readable(store_w1);
  f.store_w3 = device_readable(store_w3);
  f.store_w2 = device_readable(store_w2);
  if (!f.store_w1 || !f.store_w3 || !f.store_w2) return K3MOE_ERR_UNSUPPORTED;
  const CacheState st = cache_state_view(state, E, C);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_cache_plan(st, topk_ids, entries, slot_ids, s) != hipSuccess) return K3MOE_ERR_DEVICE;
  f.header = st.header;
  f.fetch = st.fetch;
  f.cache_w1 = cache_w1;
  f.cache_w3 = cache_w3;
  f.cache_w2 = cache_w2;
  f.mat13 = (int64_t)I * (D / block) * bytes;
  f.mat2 = (int64_t)D * (I / block) * bytes;
  f.E = E;
  f.C = C;
  return device_status(launch_cache_fetch(f, s));
}

int moe_expert_cache_route(void* state, size_t state_bytes, int32_t E, int32_t C, const int32_t* topk_ids, int64_t T,
                           int32_t k, int32_t* slot_ids, const uint8_t* store_w1, const uint8_t* store_w3,
                           const uint8_t* store_w2, uint8_t* cache_w1, uint8_t* cache_w3, uint8_t* cache_w2, int32_t D,
                           int32_t I, void* stream) {
  return cache_route(state, state_bytes, E, C, topk_ids, T, k, slot_ids, store_w1, store_w3, store_w2, cache_w1,
                     cache_w3, cache_w2, D, I, 32, 17, stream);
}

int moe_expert_cache_route_q4k(void* state, size_t state_bytes, int32_t E, int32_t C, const int32_t* topk_ids,
                               int64_t T, int32_t k, int32_t* slot_ids, const uint8_t* store_w1,
                               const uint8_t* store_w3, const uint8_t* store_w2, uint8_t* cache_w1,
                               uint8_t* cache_w3, uint8_t* cache_w2, int32_t D, int32_t I, void* stream) {
  return cache_route(state, state_bytes, E, C, topk_ids, T, k, slot_ids, store_w1, store_w3, store_w2, cache_w1,
                     cache_w3, cache_w2, D, I, 256, 144, stream);
}

// ---------------------------------------------------------------------------
// Latent-MoE block.

struct BlockPlan {
  int base_z, base_d, base_g, base_u, NV1;  // first product's segments (virtual feature offsets)
  int ksteps1, split1_steps, splits1;
  int ksteps2, split2_steps, splits2;
  size_t z, xl, s, ids, w, yl, dbuf, ssq, region, total;  // workspace offsets (256-aligned); region: products' partials and
                                               // the FFN's workspace, which never live at the same time
};

static int dense_split_steps(int64_t T, int NV, int ksteps, int* splits) {
  int steps;
  if (T <= kDenseStreamMaxTokens) {
    steps = ksteps;  // the streaming kernel splits K among its own waves
  } else {
    const int n = dense_tile_splits(T, NV, ksteps);
    steps = (ksteps + n - 1) / n;
  }
  *splits = (ksteps + steps - 1) / steps;
  return steps;
}

static BlockPlan block_plan(int64_t T, int32_t H, int32_t D, int32_t I, int32_t Is, int32_t E, int32_t k) {
  auto up = [](int64_t v, int64_t a) { return (v + a - 1) / a * a; };
  BlockPlan P{};
  P.base_z = 0;
  P.base_d = (int)up(E, kDenseSegAlign);
  P.base_g = P.base_d + (int)up(D, kDenseSegAlign);
  P.base_u = P.base_g + (int)up(Is, kDenseSegAlign);
  P.NV1 = P.base_u + (int)up(Is, kDenseSegAlign);
  P.ksteps1 = H / kDenseKStep;
  P.split1_steps = dense_split_steps(T, P.NV1, P.ksteps1, &P.splits1);
  P.ksteps2 = D / kDenseKStep + Is / kDenseKStep;
  P.split2_steps = dense_split_steps(T, H, P.ksteps2, &P.splits2);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (size_t)up((int64_t)(off + bytes), 256);
    return o;
  };
  P.z = take((size_t)T * E * 4);
  P.xl = take((size_t)T * D * 2);
  P.s = take((size_t)T * Is * 2);
  P.ids = take((size_t)T * k * 4);
  P.w = take((size_t)T * k * 4);
  P.yl = take((size_t)T * D * 2);
  P.dbuf = take((size_t)T * D * 4);
  P.ssq = take((size_t)T * block_mid_blocks(E, D, Is) * 4);
  size_t region = (size_t)P.splits1 * T * P.NV1 * 4;
  if (P.splits2 > 1 && (size_t)P.splits2 * T * H * 4 > region) region = (size_t)P.splits2 * T * H * 4;
  const size_t ffn = moe_mxfp4_ffn_workspace_size(T, D, I, E, k);
  if (ffn > region) region = ffn;
  P.region = take(region);
  P.total = off;
  return P;
}

static int block_shape_status(int64_t T, int32_t H, int32_t D, int32_t I, int32_t Is, int32_t E, int32_t k,
                              float eps) {
  if (T < 0 || k < 1 || E < k || k > K3MOE_MAX_TOPK || E > K3MOE_MAX_EXPERTS_FFN) return K3MOE_ERR_SHAPE;
  if (H <= 0 || D <= 0 || I <= 0 || Is <= 0 || H % 128 || D % 64 || Is % 64 || I % 32) return K3MOE_ERR_SHAPE;
  if (H > K3MOE_MAX_DIM_FFN || D > K3MOE_MAX_DIM_FFN || I > K3MOE_MAX_DIM_FFN || Is > K3MOE_MAX_DIM_FFN)
    return K3MOE_ERR_SHAPE;
  if (T * (int64_t)k > 0x7FFFFFFF || !(eps >= 0.0f) || !isfinite(eps)) return K3MOE_ERR_SHAPE;
  // launch grids: tile-kernel workgroups and epilogue rows fit 32-bit counts
  const BlockPlan P = block_plan(T > 0 ? T : 1, H, D, I, Is, E, k);
  const int64_t tiles1 = (int64_t)(P.NV1 / 128) * ((T + 127) / 128) * P.splits1;
  if (tiles1 > 0x7FFFFFFF || T * (int64_t)(H / 4) / 256 > 0x7FFFFFFF) return K3MOE_ERR_SHAPE;
  return K3MOE_OK;
}

size_t moe_latent_block_workspace_size(int64_t T, int32_t H, int32_t D, int32_t I, int32_t Is, int32_t E, int32_t k) {
  if (block_shape_status(T, H, D, I, Is, E, k, 0.0f) != K3MOE_OK || T == 0) return 0;
  return block_plan(T, H, D, I, Is, E, k).total;
}

int moe_latent_block_profiled(const void* h_bf16, const void* wg, const float* bias, const void* wd, const void* gamma,
                              const uint8_t* w1, const uint8_t* w3, const uint8_t* w2, const void* wu,
                              const void* ws1, const void* ws3, const void* ws2, int64_t T, int32_t H, int32_t D,
                              int32_t I, int32_t Is, int32_t E, int32_t k, int32_t normalize, float route_scale,
                              float eps, float* out, int32_t* topk_ids, float* topk_w, void* workspace,
                              size_t workspace_bytes, void* stream, void* const* events) {
  const int st = block_shape_status(T, H, D, I, Is, E, k, eps);
  if (st != K3MOE_OK) return st;
  if (T == 0) return K3MOE_OK;
  if (!h_bf16 || !wg || !wd || !gamma || !w1 || !w3 || !w2 || !wu || !ws1 || !ws3 || !ws2 || !out || !workspace)
    return K3MOE_ERR_NULL;
  const void* ptrs[] = {h_bf16, wg, bias, wd, gamma, w1, w3, w2, wu, ws1, ws3, ws2, out, topk_ids, topk_w, workspace};
  for (const void* q : ptrs)
    if (misaligned(q)) return K3MOE_ERR_ALIGN;
  const BlockPlan P = block_plan(T, H, D, I, Is, E, k);
  if (workspace_bytes < P.total) return K3MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* z = reinterpret_cast<float*>(ws + P.z);
  uint16_t* xl = reinterpret_cast<uint16_t*>(ws + P.xl);
  uint16_t* sh = reinterpret_cast<uint16_t*>(ws + P.s);
  int32_t* ids = topk_ids ? topk_ids : reinterpret_cast<int32_t*>(ws + P.ids);
  float* wts = topk_w ? topk_w : reinterpret_cast<float*>(ws + P.w);
  uint16_t* yl = reinterpret_cast<uint16_t*>(ws + P.yl);
  float* region = reinterpret_cast<float*>(ws + P.region);
  auto mark = [&](int i) { return !events || !events[i] || hipEventRecord((hipEvent_t)events[i], s) == hipSuccess; };

  // first product: gate | latent down | shared gate | shared up, all on h
  DenseGemmArgs g1{};
  g1.a[0] = static_cast<const uint16_t*>(h_bf16);
  g1.lda[0] = H;
  g1.ksteps[0] = P.ksteps1;
  g1.nseg = 4;
  const void* w1seg[4] = {wg, wd, ws1, ws3};
  const int rows1[4] = {E, D, Is, Is};
  const int base1[4] = {P.base_z, P.base_d, P.base_g, P.base_u};
  for (int i = 0; i < 4; ++i) {
    g1.rows[i] = rows1[i];
    g1.base[i] = base1[i];
    g1.w[i][0] = static_cast<const uint16_t*>(w1seg[i]);
    g1.ldw[i][0] = H;
  }
  g1.T = T;
  g1.NV = P.NV1;
  g1.split_steps = P.split1_steps;
  g1.splits = P.splits1;
  g1.p = region;
  if (!mark(0) || launch_dense_gemm(g1, 1, s) != hipSuccess) return K3MOE_ERR_DEVICE;

  BlockMidArgs m{};
  m.p = region;
  m.splits = P.splits1;
  m.NV = P.NV1;
  m.T = T;
  m.E = E;
  m.D = D;
  m.Is = Is;
  m.base_z = P.base_z;
  m.base_d = P.base_d;
  m.base_g = P.base_g;
  m.base_u = P.base_u;
  m.gamma = static_cast<const uint16_t*>(gamma);
  m.eps = eps;
  m.z = z;
  m.xl = xl;
  m.s = sh;
  m.dbuf = reinterpret_cast<float*>(ws + P.dbuf);
  m.ssq = reinterpret_cast<float*>(ws + P.ssq);
  m.nblk = block_mid_blocks(E, D, Is);
  m.tok_per_wg = T >= 512 ? 8 : 1;
  if (!mark(1) || launch_block_mid(m, s) != hipSuccess) return K3MOE_ERR_DEVICE;
  if (!mark(2) || launch_route_topk(z, bias, T, E, k, normalize, route_scale, ids, wts, s) != hipSuccess)
    return K3MOE_ERR_DEVICE;
  if (!mark(3)) return K3MOE_ERR_DEVICE;
  const int fst = run_ffn(xl, ids, wts, w1, w3, w2, T, D, I, E, k, yl, true, reinterpret_cast<uint8_t*>(region), s,
                          nullptr, events == nullptr);
  if (fst != K3MOE_OK) return fst;

  // second product: [yl | s] (K segments) times [Wu | Ws2], one sum
  DenseGemmArgs g2{};
  g2.a[0] = yl;
  g2.lda[0] = D;
  g2.ksteps[0] = D / kDenseKStep;
  g2.a[1] = sh;
  g2.lda[1] = Is;
  g2.ksteps[1] = Is / kDenseKStep;
  g2.nseg = 1;
  g2.rows[0] = H;
  g2.base[0] = 0;
  g2.w[0][0] = static_cast<const uint16_t*>(wu);
  g2.ldw[0][0] = D;
  g2.w[0][1] = static_cast<const uint16_t*>(ws2);
  g2.ldw[0][1] = Is;
  g2.T = T;
  g2.NV = H;
  g2.split_steps = P.split2_steps;
  g2.splits = P.splits2;
  g2.p = P.splits2 == 1 ? out : region;
  if (!mark(4) || launch_dense_gemm(g2, 2, s) != hipSuccess || !mark(5)) return K3MOE_ERR_DEVICE;
  if (P.splits2 > 1 && launch_dense_sum(region, P.splits2, T, H, out, s) != hipSuccess) return K3MOE_ERR_DEVICE;
  if (!mark(6)) return K3MOE_ERR_DEVICE;
  return K3MOE_OK;
}

int moe_latent_block(const void* h_bf16, const void* wg, const float* bias, const void* wd, const void* gamma,
                     const uint8_t* w1, const uint8_t* w3, const uint8_t* w2, const void* wu, const void* ws1,
                     const void* ws3, const void* ws2, int64_t T, int32_t H, int32_t D, int32_t I, int32_t Is,
                     int32_t E, int32_t k, int32_t normalize, float route_scale, float eps, float* out,
                     int32_t* topk_ids, float* topk_w, void* workspace, size_t workspace_bytes, void* stream) {
  return moe_latent_block_profiled(h_bf16, wg, bias, wd, gamma, w1, w3, w2, wu, ws1, ws3, ws2, T, H, D, I, Is, E, k,
                                   normalize, route_scale, eps, out, topk_ids, topk_w, workspace, workspace_bytes,
                                   stream, nullptr);
}

static int group_shape_status(int64_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || E > K3MOE_MAX_EXPERTS_FFN || k < 1 || k > K3MOE_MAX_TOPK) return K3MOE_ERR_SHAPE;
  if (T * (int64_t)k > 0x7FFFFFFF) return K3MOE_ERR_SHAPE;
  return K3MOE_OK;
}

size_t moe_group_workspace_size(int64_t T, int32_t E, int32_t k) {
  if (group_shape_status(T, E, k) != K3MOE_OK || T == 0) return 0;
  return group_workspace_layout(T, E, k).total;
}

int moe_group_by_expert(const int32_t* topk_ids, int64_t T, int32_t E, int32_t k, int32_t* counts, int32_t* offsets,
                        int32_t* row_tok, int32_t* slot_row, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = group_shape_status(T, E, k);
  if (st != K3MOE_OK) return st;
  if (T == 0) return K3MOE_OK;
  if (!topk_ids || !counts || !offsets || !row_tok || !slot_row || !workspace) return K3MOE_ERR_NULL;
  if (misaligned(topk_ids) || misaligned(counts) || misaligned(offsets) || misaligned(row_tok) ||
      misaligned(slot_row) || misaligned(workspace))
    return K3MOE_ERR_ALIGN;
  const GroupWorkspace L = group_workspace_layout(T, E, k);
  if (workspace_bytes < L.total) return K3MOE_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  GroupArgs g{};
  g.ids = topk_ids;
  g.x = nullptr;  // D == 0: no activation re-layout
  g.T = T;
  g.D = 0;
  g.E = E;
  g.k = k;
  // every expert in lists 0/1, cut into tiles of kGroupTileRows rows
  for (int l = 0; l < kTileLists; ++l) g.rows_per_tile[l] = kGroupTileRows;
  g.split_rows = 0;
  g.counts = counts;
  g.offsets = offsets;
  g.tile_count = reinterpret_cast<int32_t*>(ws + L.tile_count);
  for (int l = 0; l < kTileLists; ++l) g.tiles[l] = reinterpret_cast<Tile*>(ws + L.tiles[l]);
  g.row_tok = row_tok;
  g.slot_row = slot_row;
  g.chunk_base = reinterpret_cast<int32_t*>(ws + L.chunk_base);
  g.chunk_mask = reinterpret_cast<unsigned long long*>(ws + L.chunk_mask);
  g.x_perm = nullptr;
  return device_status(launch_group(g, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
