// Device expert cache in front of an external expert store.
//
// The Hugging Face card "K3-Stuff" (llama-cpp-patches item 2) pages the routed
// experts in from disk on demand, the page cache acting as the hot-expert
// cache with least-recently-used eviction; the lucebox page "feat(kimi-k3):
// add DSpark Q8 artifact and shared speculative runtime" ("Runtime
// validation") runs the target with SSD-routed experts behind an 8 GiB device
// expert cache.  Here the store is any memory the GPU can read (host memory
// pinned and mapped, or device memory) holding all E experts as 17-byte
// blocks; the cache is C expert slots in HBM with the same per-expert layout,
// so the FFN runs on it unchanged with slot numbers in place of expert ids.
//
// Per batch, all on the device (no host synchronization, graph-capturable):
//   plan  (one workgroup): mark the experts the batch uses, find hits and
//         misses, give the i-th miss (increasing expert order) the i-th slot of
//         the least-recently-used order that no hit holds, evict what it held,
//         rebuild the order (untouched slots, then hit slots, then filled
//         slots), write the fetch list, rename every entry to its slot;
//   fetch (persistent grid): copy each listed expert's three matrices from the
//         store into its slot with 16-byte loads, many in flight per thread.
#include "k3moe.h"
#include "k3moe_internal.h"

namespace k3moe {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPlanThreads = 1024;
constexpr int kMaxPer = (K3MOE_MAX_EXPERTS_FFN + kPlanThreads - 1) / kPlanThreads;  // items per thread (8)

__device__ __forceinline__ void lds_sync() { __syncthreads(); }

// Block-wide exclusive scan of two counters in thread order (1024 threads);
// tot = the sums.  Every thread must call it.
__device__ __forceinline__ void scan2(int (&v)[2], int (&tot)[2], int (*wsum)[2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl[2] = {v[0], v[1]};
#pragma unroll
  for (int d = 1; d < 64; d <<= 1)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int o = __shfl_up(incl[c], d, 64);
      if (lane >= d) incl[c] += o;
    }
  if (lane == 63) {
    wsum[wave][0] = incl[0];
    wsum[wave][1] = incl[1];
  }
  lds_sync();
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    int before = 0, all = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      const int x = wsum[w][c];
      before += w < wave ? x : 0;
      all += x;
    }
    v[c] = before + incl[c] - v[c];
    tot[c] = all;
  }
  lds_sync();
}

__global__ __launch_bounds__(256) void cache_init_kernel(CacheState st) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < st.E) st.slot_of[i] = -1;
  if (i < st.C) {
    st.expert_in[i] = -1;
    st.order[i] = (int32_t)i;
  }
  if (i == 0) {
    k3moe_expert_cache_header h{};
    h.E = st.E;
    h.C = st.C;
    h.tag = K3MOE_EXPERT_CACHE_TAG;
    *st.header = h;
  }
}

__global__ __launch_bounds__(kPlanThreads) void cache_plan_kernel(CacheState st, const int32_t* __restrict__ ids,
                                                                   int64_t n, int32_t* __restrict__ slot_ids) {
  __shared__ uint32_t used[(K3MOE_MAX_EXPERTS_FFN + 31) / 32];
  __shared__ int32_t l_slot[K3MOE_MAX_EXPERTS_FFN];  // slot_of
  __shared__ int32_t l_exp[K3MOE_MAX_EXPERTS_FFN];   // expert_in
  __shared__ int32_t l_vict[K3MOE_MAX_EXPERTS_FFN];  // i-th victim slot
  __shared__ int32_t l_miss[K3MOE_MAX_EXPERTS_FFN];  // i-th missing expert
  __shared__ int wsum[kPlanThreads / 64][2];
  const int tid = threadIdx.x;
  const int E = st.E, C = st.C;
  // a state that was not initialised for these sizes is left alone: no slot,
  // no fetch (uniform over the workgroup)
  const k3moe_expert_cache_header hd0 = *st.header;
  if (hd0.tag != K3MOE_EXPERT_CACHE_TAG || hd0.E != E || hd0.C != C) {
    for (int64_t q = tid; q < n; q += kPlanThreads) slot_ids[q] = -1;
    if (tid == 0) st.header->n_fetch = 0u;
    return;
  }
  // the old order stays in registers: thread t owns positions t*pc .. t*pc +
  // pc - 1 (read before the barriers that precede every write of the new one)
  const int pc = (C + kPlanThreads - 1) / kPlanThreads;
  int ord[kMaxPer];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int p = tid * pc + i;
    const int o = (i < pc && p < C) ? st.order[p] : 0;
    ord[i] = (o >= 0 && o < C) ? o : 0;  // the tables are read defensively: never an index out of range
  }
  for (int e = tid; e < E; e += kPlanThreads) {
    const int v = st.slot_of[e];
    l_slot[e] = (v >= 0 && v < C) ? v : -1;
  }
  for (int s = tid; s < C; s += kPlanThreads) {
    const int v = st.expert_in[s];
    l_exp[s] = (v >= 0 && v < E) ? v : -1;
  }
  for (int w = tid; w < (E + 31) / 32; w += kPlanThreads) used[w] = 0u;
  lds_sync();
  for (int64_t q = tid; q < n; q += kPlanThreads) {
    const int e = ids[q];
    if (e >= 0 && e < E) atomicOr(&used[e >> 5], 1u << (e & 31));
  }
  lds_sync();
  auto is_used = [&](int e) { return (used[e >> 5] >> (e & 31)) & 1u; };

  // misses (used, not cached) in expert order: thread t owns experts
  // t*pe .. t*pe + pe - 1; hits counted alongside
  const int pe = (E + kPlanThreads - 1) / kPlanThreads;
  int v[2] = {0, 0}, tot[2];
  for (int i = 0; i < pe; ++i) {
    const int e = tid * pe + i;
    if (e < E && is_used(e)) ++v[l_slot[e] < 0 ? 0 : 1];
  }
  scan2(v, tot, wsum);
  const int h = tot[1];
  int m = tot[0];
  {
    int r = v[0];
    for (int i = 0; i < pe; ++i) {
      const int e = tid * pe + i;
      if (e < E && is_used(e) && l_slot[e] < 0) l_miss[r++] = e;
    }
  }
  // order positions: hit (its slot holds a used expert) or not
  bool hit[kMaxPer];
  int u[2] = {0, 0};  // non-hit, hit positions of this thread
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int p = tid * pc + i;
    hit[i] = false;
    if (i < pc && p < C) {
      const int ex = l_exp[ord[i]];
      hit[i] = ex >= 0 && is_used(ex);
      ++u[hit[i] ? 1 : 0];
    }
  }
  int utot[2];
  scan2(u, utot, wsum);  // u[0] = rank among non-hit positions, u[1] = among hits
  const int n_free = utot[0];
  m = m < n_free ? m : n_free;  // C >= distinct experts per batch is checked on the host
  // victims: the first m non-hit positions; new order = untouched non-hit
  // positions, then hit positions, then victims (in miss order)
  int32_t* const order = st.order;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int p = tid * pc + i;
    if (i < pc && p < C) {
      const int s = ord[i];
      if (hit[i]) {
        order[(n_free - m) + u[1]] = s;
        ++u[1];
      } else {
        const int r = u[0]++;
        if (r < m) {
          l_vict[r] = s;
          order[(C - m) + r] = s;
        } else {
          order[r - m] = s;
        }
      }
    }
  }
  lds_sync();
  // fill: the i-th miss into the i-th victim (distinct slots, distinct
  // experts; an evicted expert is never one this batch uses)
  for (int i = tid; i < m; i += kPlanThreads) {
    const int s = l_vict[i], e = l_miss[i];
    const int old = l_exp[s];
    if (old >= 0) l_slot[old] = -1;
    l_exp[s] = e;
    l_slot[e] = s;
    st.fetch[2 * i] = e;
    st.fetch[2 * i + 1] = s;
  }
  lds_sync();
  for (int e = tid; e < E; e += kPlanThreads) st.slot_of[e] = l_slot[e];
  for (int s = tid; s < C; s += kPlanThreads) st.expert_in[s] = l_exp[s];
  for (int64_t q = tid; q < n; q += kPlanThreads) {
    const int e = ids[q];
    slot_ids[q] = (e >= 0 && e < E) ? l_slot[e] : -1;
  }
  if (tid == 0) {
    k3moe_expert_cache_header hd = hd0;
    hd.step += 1;
    hd.n_fetch = (uint32_t)m;
    hd.hits = (uint32_t)h;
    hd.misses = (uint32_t)m;
    hd.hits_total += (uint64_t)h;
    hd.misses_total += (uint64_t)m;
    *st.header = hd;
  }
}

// Copy the fetch list's experts from the store into their slots.  D and I are
// multiples of 32, so every matrix is 17 * 32 * n bytes: whole 16-byte chunks.
__global__ __launch_bounds__(256) void cache_fetch_kernel(CacheFetchArgs a) {
  int n_fetch = (int)__builtin_amdgcn_readfirstlane((int)a.header->n_fetch);
  n_fetch = n_fetch < a.C ? n_fetch : a.C;
  const int64_t c13 = a.mat13 / 16, c2 = a.mat2 / 16;  // chunks per matrix
  const int64_t per = 2 * c13 + c2;                    // chunks per expert
  const int64_t total = (int64_t)n_fetch * per;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  constexpr int kUnroll = 8;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; base < total; base += stride * kUnroll) {
    u32x4_t v[kUnroll];
    u32x4_t* dst[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = base + stride * u;
      dst[u] = nullptr;
      if (c >= total) continue;
      const int i = (int)(c / per);
      int64_t r = c - (int64_t)i * per;
      const int e = a.fetch[2 * i], s = a.fetch[2 * i + 1];
      if (e < 0 || e >= a.E || s < 0 || s >= a.C) continue;  // never written by the plan
      const uint8_t* src;
      uint8_t* d;
      if (r < c13) {
        src = a.store_w1 + (size_t)e * a.mat13;
        d = a.cache_w1 + (size_t)s * a.mat13;
      } else if (r < 2 * c13) {
        r -= c13;
        src = a.store_w3 + (size_t)e * a.mat13;
        d = a.cache_w3 + (size_t)s * a.mat13;
      } else {
        r -= 2 * c13;
        src = a.store_w2 + (size_t)e * a.mat2;
        d = a.cache_w2 + (size_t)s * a.mat2;
      }
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src) + r);
      dst[u] = reinterpret_cast<u32x4_t*>(d) + r;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (dst[u]) *dst[u] = v[u];
  }
}

int cache_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

}  // namespace

CacheState cache_state_view(void* state, int32_t E, int32_t C) {
  auto align = [](size_t v) { return (v + 255) / 256 * 256; };
  uint8_t* b = static_cast<uint8_t*>(state);
  CacheState st{};
  size_t off = 0;
  st.header = reinterpret_cast<k3moe_expert_cache_header*>(b + off);
  off = align(off + sizeof(k3moe_expert_cache_header));
  st.slot_of = reinterpret_cast<int32_t*>(b + off);
  off = align(off + sizeof(int32_t) * (size_t)E);
  st.expert_in = reinterpret_cast<int32_t*>(b + off);
  off = align(off + sizeof(int32_t) * (size_t)C);
  st.order = reinterpret_cast<int32_t*>(b + off);
  off = align(off + sizeof(int32_t) * (size_t)C);
  st.fetch = reinterpret_cast<int32_t*>(b + off);
  off = align(off + sizeof(int32_t) * 2 * (size_t)C);
  st.bytes = off;
  st.E = E;
  st.C = C;
  return st;
}

hipError_t launch_cache_init(const CacheState& st, hipStream_t s) {
  const int n = st.E > st.C ? st.E : st.C;
  hipLaunchKernelGGL(cache_init_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, st);
  return hipGetLastError();
}

hipError_t launch_cache_plan(const CacheState& st, const int32_t* ids, int64_t n, int32_t* slot_ids, hipStream_t s) {
  hipLaunchKernelGGL(cache_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, st, ids, n, slot_ids);
  return hipGetLastError();
}

hipError_t launch_cache_fetch(const CacheFetchArgs& a, hipStream_t s) {
  if (a.mat13 % 16 != 0 || a.mat2 % 16 != 0) return hipErrorInvalidValue;
  const int grid = 4 * cache_cu_count();
  hipLaunchKernelGGL(cache_fetch_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace k3moe
