// Sigmoid + bias top-k router (one 64-lane wavefront per token).
//
// Routing parameters from the llama.cpp pull request "model: add Kimi-K3 text
// model", converter dry-run comment: 896 experts, 16 used, sigmoid expert
// score gating, per-expert bias exp_probs_b.  Scores are evaluated in fp64 so
// that the selected ids are reproducible bit for bit; ties go to the lower
// expert index; NaN scores rank last.
//
// Up to 1024 experts (16 per lane) one wave handles a token with the logits
// in registers: lane l owns experts l, l + 64, l + 128, ....  An fp32 score
// pre-filters: the k-th of the 64 fp32 lane-bests (a bitwise radix select over
// ballots) bounds the k-th fp32 score from below, so every expert of the exact
// top k has an fp32 score no lower than that bound minus a small margin (the
// fp32 error bound is stated at route_score32); those candidates (at most 64)
// are scored in fp64 and each counts how many of the others rank before it,
// which places the top k in order without a sort.
// Otherwise (heavy ties, non-finite scores at the threshold) the fp64 scores of
// all experts are used: the 64 fp64 lane-bests are sorted, the experts ranking
// at or before the k-th of them are compacted and sorted, and with more than
// 64 of those each lane sorts its experts and k rounds take the wave's best
// head (DPP exchanges inside 16-lane rows, row swaps across rows).  Larger E
// falls back to a kernel that writes the scores to LDS (or recomputes them)
// and, in round r, picks the best expert ranking strictly after round r-1's
// pick; it needs no "taken" flags, so nothing limits E.
#include "k3moe_internal.h"

#include <math.h>

namespace k3moe {
namespace {

constexpr int kWaveSize = 64;

__device__ __forceinline__ double sigmoid64(float z) { return 1.0 / (1.0 + exp(-(double)z)); }

__device__ __forceinline__ double route_score(float z, float b) {
  double s = sigmoid64(z) + (double)b;
  return isnan(s) ? -INFINITY : s;
}

// The same score in fp32 from the hardware exp2 and reciprocal (a pre-filter
// only: every decision is taken on the fp64 score).  With u = 2^-24:
// -z * log2(e) is off by at most 2|z|u in the exponent, v_exp_f32 and
// v_rcp_f32 are within 1 ulp (2u) of their results, and the add rounds by u,
// so e^-z carries a relative error of at most (2|z| + 2)u and the sigmoid an
// absolute one of at most 3u + 2u * sigma(1 - sigma)(|z| + 1) <= 4u
// (sigma(1 - sigma)|z| <= 0.224).  Outputs flushed to zero (exponents below
// -126) move the sigmoid by less than 2^-126, an overflow to +inf gives the
// limit 0.  With the bias add (u of the sum): |score32 - score| <=
// 5u(1 + |score|) < 2^-21 (1 + |score|).
__device__ __forceinline__ float route_score32(float z, float b) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.44269504088896341f);
  const float s = __builtin_amdgcn_rcpf(1.0f + e) + b;
  return isnan(s) ? -INFINITY : s;
}

// The k-th largest (1 <= k <= 64) of the wave's 64 values, none NaN: the
// largest x that at least k lanes reach, found one bit at a time on integer
// keys that order like the floats.
__device__ __forceinline__ float wave_kth_largest(float v, int k) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t key = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  uint32_t x = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = x | (1u << bit);
    if (__builtin_popcountll(__builtin_amdgcn_ballot_w64(key >= c)) >= k) x = c;
  }
  return __uint_as_float((x & 0x80000000u) ? (x & 0x7FFFFFFFu) : ~x);
}

// (sa, ea) ranks before (sb, eb): higher score, or equal score and lower index.
__device__ __forceinline__ bool ranks_before(double sa, int ea, double sb, int eb) {
  return sa > sb || (sa == sb && ea < eb);
}

// (s, e) of the lane DPP control kCtrl names (within a row of 16 lanes).
template <int kCtrl>
__device__ __forceinline__ void dpp_pair(double s, int e, double& os, int& oe) {
  const uint64_t b = __double_as_longlong(s);
  const uint32_t lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)b, kCtrl, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), kCtrl, 0xF, 0xF, false);
  os = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  oe = __builtin_amdgcn_mov_dpp(e, kCtrl, 0xF, 0xF, false);
}

// Value of lane ^ 16 (kRows = 16) or lane ^ 32 (kRows = 32): the gfx950 row
// swaps exchange the odd 16- (32-) lane rows of their first operand with the
// even rows of their second; with both operands equal, an even row finds its
// partner's value in the second result and an odd row in the first.
template <int kRows>
__device__ __forceinline__ uint32_t swap_rows(uint32_t v, int lane) {
  if (kRows == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}
template <int kRows>
__device__ __forceinline__ void swap_pair(double s, int e, int lane, double& os, int& oe) {
  const uint64_t b = __double_as_longlong(s);
  const uint32_t lo = swap_rows<kRows>((uint32_t)b, lane);
  const uint32_t hi = swap_rows<kRows>((uint32_t)(b >> 32), lane);
  os = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  oe = (int)swap_rows<kRows>((uint32_t)e, lane);
}

// Wave-wide best (s, e) under ranks_before, in every lane: inside each
// 16-lane row, exchanges with lane ^ 1 and ^ 2 (quad permutes) and with the
// mirrored lane of the 8-lane half and of the row (DPP); then with the other
// rows (lane ^ 16, lane ^ 32).
__device__ __forceinline__ void wave_best(double& bs, int& be, int lane) {
  double os;
  int oe;
#define K3_TAKE                       \
  if (ranks_before(os, oe, bs, be)) { \
    bs = os;                          \
    be = oe;                          \
  }
  dpp_pair<0xB1>(bs, be, os, oe);  // quad_perm [1,0,3,2]
  K3_TAKE
  dpp_pair<0x4E>(bs, be, os, oe);  // quad_perm [2,3,0,1]
  K3_TAKE
  dpp_pair<0x141>(bs, be, os, oe);  // row_half_mirror
  K3_TAKE
  dpp_pair<0x140>(bs, be, os, oe);  // row_mirror
  K3_TAKE
  swap_pair<16>(bs, be, lane, os, oe);
  K3_TAKE
  swap_pair<32>(bs, be, lane, os, oe);
  K3_TAKE
#undef K3_TAKE
}

// Sort N (s, e) pairs held in registers so that x[0] ranks first (bitonic
// network; N is a power of two, every index compile-time).
template <int N>
__device__ __forceinline__ void sort_desc(double (&sc)[N], int (&ix)[N]) {
#pragma unroll
  for (int kk = 2; kk <= N; kk <<= 1)
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int l = i ^ j;
        if (l > i) {
          // first half of each kk-block ends up ranked first, second half last
          const bool first = (i & kk) == 0;
          const bool swap = first ? ranks_before(sc[l], ix[l], sc[i], ix[i]) : ranks_before(sc[i], ix[i], sc[l], ix[l]);
          if (swap) {
            const double ts = sc[i];
            sc[i] = sc[l];
            sc[l] = ts;
            const int te = ix[i];
            ix[i] = ix[l];
            ix[l] = te;
          }
        }
      }
}

// (s, e) of lane ^ S, by DPP and row swaps only (no LDS round trip): quad
// permutes for S = 1, 2; for S = 4 the half-row mirror (lane ^ 7 within 8)
// followed by the quad reversal (^ 3); for S = 8 the row mirror (^ 15 within
// 16) followed by the half-row mirror (^ 7); row swaps for S = 16, 32.
template <int S>
__device__ __forceinline__ void xor_pair(double s, int e, int lane, double& os, int& oe) {
  if constexpr (S == 1) {
    dpp_pair<0xB1>(s, e, os, oe);  // quad_perm [1,0,3,2]
  } else if constexpr (S == 2) {
    dpp_pair<0x4E>(s, e, os, oe);  // quad_perm [2,3,0,1]
  } else if constexpr (S == 4) {
    double ts;
    int te;
    dpp_pair<0x141>(s, e, ts, te);  // row_half_mirror
    dpp_pair<0x1B>(ts, te, os, oe);  // quad_perm [3,2,1,0]
  } else if constexpr (S == 8) {
    double ts;
    int te;
    dpp_pair<0x140>(s, e, ts, te);   // row_mirror
    dpp_pair<0x141>(ts, te, os, oe);  // row_half_mirror
  } else {
    static_assert(S == 16 || S == 32, "lane xor stride");
    swap_pair<S>(s, e, lane, os, oe);
  }
}

// One compare-exchange step of the bitonic network (runs of SIZE, partner
// lane ^ STRIDE) and the steps after it within the same merge.  In a run
// sorted first-ranked-first the lower lane of each pair keeps the earlier-
// ranked entry; runs with bit SIZE set sort the other way (the last run, size
// 64, sorts first-ranked-first).
template <int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_steps(double& cs, int& ce, int lane) {
  double os;
  int oe;
  xor_pair<STRIDE>(cs, ce, lane, os, oe);
  const bool keep_first = ((lane & STRIDE) == 0) == ((lane & SIZE) == 0);
  const bool take = keep_first ? ranks_before(os, oe, cs, ce) : ranks_before(cs, ce, os, oe);
  if (take) {
    cs = os;
    ce = oe;
  }
  if constexpr (STRIDE > 1) bitonic_steps<SIZE, STRIDE / 2>(cs, ce, lane);
}
template <int SIZE>
__device__ __forceinline__ void bitonic_merges(double& cs, int& ce, int lane) {
  bitonic_steps<SIZE, SIZE / 2>(cs, ce, lane);
  if constexpr (SIZE < kWaveSize) bitonic_merges<SIZE * 2>(cs, ce, lane);
}

// Bitonic sort of one (s, e) per lane across the wave, first-ranked in lane 0.
// The entries are distinct experts or identical sentinels, so "ranks before"
// is a strict order on them.
__device__ __forceinline__ void wave_sort64(double& cs, int& ce, int lane) { bitonic_merges<2>(cs, ce, lane); }

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// The k (<= 64) best (s, e) of the wave's NPER-per-lane entries, first-ranked
// in lane 0, with no per-lane sort and no k rounds.  Of the 64 lane-bests, the
// k-th ranks at or after every entry of the top k (the k lane-bests before it
// are k entries ranking at or before it), so the top k are among the entries
// that rank at or before it.  When at most 64 entries qualify they are
// compacted through `ls` / `le` (this wave's 64 doubles and 64 ints of LDS)
// and sorted once; otherwise (heavy ties) nothing is written to out_* and the
// caller takes its k-round path.  Wave-uniform result.
template <int NPER>
__device__ __forceinline__ bool wave_topk_filtered(const double (&sc)[NPER], const int (&ix)[NPER], int k, int lane,
                                                    double* ls, int* le, double& out_s, int& out_e) {
  double bs = sc[0];
  int be = ix[0];
#pragma unroll
  for (int j = 1; j < NPER; ++j)
    if (ranks_before(sc[j], ix[j], bs, be)) {
      bs = sc[j];
      be = ix[j];
    }
  wave_sort64(bs, be, lane);
  const double ts = readlane_f64(bs, k - 1);
  const int te = __builtin_amdgcn_readlane(be, k - 1);
  unsigned qual = 0u;
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < NPER; ++j) {
    const bool q = (sc[j] == ts && ix[j] == te) || ranks_before(sc[j], ix[j], ts, te);
    qual |= (q ? 1u : 0u) << j;
    cnt += q ? 1 : 0;
  }
  int incl = cnt;
#pragma unroll
  for (int d = 1; d < kWaveSize; d <<= 1) {
    const int o = __shfl_up(incl, d, kWaveSize);
    if (lane >= d) incl += o;
  }
  const int total = __builtin_amdgcn_readlane(incl, kWaveSize - 1);
  if (total > kWaveSize) return false;
  int pos = incl - cnt;
#pragma unroll
  for (int j = 0; j < NPER; ++j)
    if (qual & (1u << j)) {
      ls[pos] = sc[j];
      le[pos] = ix[j];
      ++pos;
    }
  // LDS accesses of one wave complete in order; the fences keep the compiler
  // from moving the reads below above these writes.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  double cs = -INFINITY;
  int ce = INT_MAX;  // sentinel: ranks after every real expert
  if (lane < total) {
    cs = ls[lane];
    ce = le[lane];
  }
  wave_sort64(cs, ce, lane);
  out_s = cs;
  out_e = ce;
  return true;
}

// Register-resident router: NPER experts per lane (E <= 64 * NPER).  Each lane
// sorts its experts once; a round takes the wave's best head and the lane that
// owned it moves to its next expert.
template <int NPER>
__global__ __launch_bounds__(256) void route_topk_reg_kernel(const float* __restrict__ z, const float* __restrict__ bias,
                                                              int64_t T, int E, int k, int normalize, float route_scale,
                                                              int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWaveSize) + threadIdx.x / kWaveSize;
  if (t >= T) return;  // whole wave leaves; the kernel has no block-level barrier
  const float* zt = z + t * (int64_t)E;

  // all loads first (indices clamped into range), then the scores
  float zv[NPER], bv[NPER];
#pragma unroll
  for (int j = 0; j < NPER; ++j) zv[j] = zt[min(lane + kWaveSize * j, E - 1)];
  if (bias) {
#pragma unroll
    for (int j = 0; j < NPER; ++j) bv[j] = bias[min(lane + kWaveSize * j, E - 1)];
  } else {
#pragma unroll
    for (int j = 0; j < NPER; ++j) bv[j] = 0.0f;
  }
  // candidates: fp64 score, expert, logit and bias; the top k by rank: gate
  // value and expert
  __shared__ double fs[4][kWaveSize];
  __shared__ int fe[4][kWaveSize];
  __shared__ float cz[4][kWaveSize], cb[4][kWaveSize];
  __shared__ double tg[4][kWaveSize];
  __shared__ int te[4][kWaveSize];
  const int wv = threadIdx.x / kWaveSize;
  int my_id = 0;

  // fp32 pre-filter.  Of the 64 fp32 lane-bests, the k-th (m) is at most the
  // k-th best fp32 score overall (k distinct experts score at least m); an
  // expert of the fp64 top k cannot score below (k-th best fp32) - 2 * err in
  // fp32 (err: the fp32 error bound above), else the k experts above that
  // k-th value would all outrank it in fp64.  So every expert within a margin
  // of m, taken as 2^-16 * (1 + |m|) (16 times 2 * err), is a candidate; the
  // candidates (at least k, at most 64) are scored in fp64, each one's rank
  // among them is counted, and the first k land in rank order.  A non-finite
  // m or more than 64 candidates (heavy ties) take the fp64 path below.
  bool done = false;
  double g = 0.0;
  {
    float s32[NPER];
    float lb = -INFINITY;
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const int e = lane + kWaveSize * j;
      s32[j] = e < E ? route_score32(zv[j], bv[j]) : -INFINITY;
      lb = fmaxf(lb, s32[j]);
    }
    const float m = wave_kth_largest(lb, k);
    if (isfinite(m)) {
      const float theta = m - ldexpf(1.0f + fabsf(m), -16);
      // slots by ballots: item j of a lane goes after every candidate of
      // items < j and after item j of the lanes below (the order is
      // irrelevant: the ranks are counted next)
      uint64_t mask[NPER];
      int total = 0;
#pragma unroll
      for (int j = 0; j < NPER; ++j) {
        mask[j] = __builtin_amdgcn_ballot_w64(s32[j] >= theta);  // experts past E score -inf
        total += __builtin_popcountll(mask[j]);
      }
      if (total <= kWaveSize) {
        int base = 0;
#pragma unroll
        for (int j = 0; j < NPER; ++j) {
          const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask[j] >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)mask[j], 0u));
          if ((mask[j] >> lane) & 1ull) {
            fe[wv][base + below] = lane + kWaveSize * j;
            cz[wv][base + below] = zv[j];
            cb[wv][base + below] = bv[j];
          }
          base += __builtin_popcountll(mask[j]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // slots past the candidates hold sentinels, which rank after every
        // candidate, so the rank count below runs in blocks of 8
        double cs = -INFINITY, cg = 0.0;
        int ce = INT_MAX;
        if (lane < total) {
          ce = fe[wv][lane];
          cg = sigmoid64(cz[wv][lane]);
          cs = cg + (double)cb[wv][lane];
          cs = isnan(cs) ? -INFINITY : cs;  // the value route_score gives
        }
        fs[wv][lane] = cs;
        fe[wv][lane] = ce;
        tg[wv][lane] = 0.0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // candidates are distinct experts, so the ranks 0 .. total-1 are
        // distinct and the top k are exactly ranks 0 .. k-1
        // (all 8 entries read first, the test without short-circuit
        // branches, so the reads overlap)
        int rank = 0;
        for (int j0 = 0; j0 < total; j0 += 8) {
          double os[8];
          int oe[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            os[u] = fs[wv][j0 + u];
            oe[u] = fe[wv][j0 + u];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) rank += (int)((os[u] > cs) | ((os[u] == cs) & (oe[u] < ce)));
        }
        if (lane < total && rank < k) {
          tg[wv][rank] = cg;
          te[wv][rank] = ce;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < k) {
          my_id = te[wv][lane];
          g = tg[wv][lane];
        }
        done = true;
      }
    }
  }

  // fp64 path: lanes 0..k-1 end with the top k in rank order: filtered
  // selection, or (more than 64 entries at or before the threshold) sorted
  // lanes and k rounds
  if (!done) {
    double sc[NPER];
    int ix[NPER];
#pragma unroll
    for (int j = 0; j < NPER; ++j) {
      const int e = lane + kWaveSize * j;
      // experts past E carry index INT_MAX, so they rank after every real expert
      sc[j] = e < E ? route_score(zv[j], bv[j]) : -INFINITY;
      ix[j] = e < E ? e : INT_MAX;
    }
    double fs_out;
    if (!wave_topk_filtered<NPER>(sc, ix, k, lane, fs[wv], fe[wv], fs_out, my_id)) {
    sort_desc<NPER>(sc, ix);
    for (int r = 0; r < k; ++r) {
      double bs = sc[0];
      int be = ix[0];
      wave_best(bs, be, lane);
      if (lane == r) my_id = be;
      if (lane == (be & (kWaveSize - 1))) {  // k <= E, so be is a real expert owned by this lane
#pragma unroll
        for (int j = 0; j + 1 < NPER; ++j) {
          sc[j] = sc[j + 1];
          ix[j] = ix[j + 1];
        }
        sc[NPER - 1] = -INFINITY;
        ix[NPER - 1] = INT_MAX;
      }
    }
    }
  }

  if (!done && lane < k) g = sigmoid64(zt[my_id]);
  double sum = g;
  if (normalize) {
    // in rank order; on the fast path from LDS in blocks of 8 (the slots
    // past k hold zeros, which leave the sum unchanged)
    sum = 0.0;
    if (done) {
      for (int r0 = 0; r0 < k; r0 += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += tg[wv][r0 + u];
      }
    } else {
      for (int r = 0; r < k; ++r) sum += readlane_f64(g, r);  // lane by lane
    }
  }
  if (lane < k) {
    double v = normalize ? g / sum : g;
    v = v * (double)route_scale;
    ids[t * k + lane] = my_id;
    w[t * k + lane] = (float)v;
  }
}

template <bool kScoresInLds>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ z, const float* __restrict__ bias,
                                                          int64_t T, int E, int k, int normalize, float route_scale,
                                                          int32_t* __restrict__ ids, float* __restrict__ w) {
  extern __shared__ double lds_scores[];
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = threadIdx.x / kWaveSize;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWaveSize) + wave;
  if (t >= T) return;  // whole wave leaves; the kernel has no block-level barrier
  const float* zt = z + t * (int64_t)E;
  double* s = lds_scores + (size_t)wave * (kScoresInLds ? E : 0);

  if (kScoresInLds) {
    for (int e = lane; e < E; e += kWaveSize) s[e] = route_score(zt[e], bias ? bias[e] : 0.0f);
    // LDS accesses of one wave complete in order; the fence keeps the compiler
    // from moving the reads below above these writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  double prev_s = INFINITY;
  int prev_e = -1;  // nothing ranks before (+inf, -1)
  int my_id = 0;
  for (int r = 0; r < k; ++r) {
    double best_s = -INFINITY;
    int best_e = INT_MAX;  // sentinel: ranks after every real expert
    for (int e = lane; e < E; e += kWaveSize) {
      const double se = kScoresInLds ? s[e] : route_score(zt[e], bias ? bias[e] : 0.0f);
      if (ranks_before(prev_s, prev_e, se, e) && ranks_before(se, e, best_s, best_e)) {
        best_s = se;
        best_e = e;
      }
    }
#pragma unroll
    for (int m = 1; m < kWaveSize; m <<= 1) {
      const double os = __shfl_xor(best_s, m, kWaveSize);
      const int oe = __shfl_xor(best_e, m, kWaveSize);
      if (ranks_before(os, oe, best_s, best_e)) {
        best_s = os;
        best_e = oe;
      }
    }
    if (lane == r) my_id = best_e;
    prev_s = best_s;
    prev_e = best_e;
  }

  // Gate weights: sigmoid(z) of the selected experts (lane r holds slot r).
  double g = 0.0;
  if (lane < k) g = sigmoid64(zt[my_id]);
  double sum = g;
  if (normalize) {
    // Sum in slot order 0..k-1 so the result does not depend on a tree shape.
    sum = 0.0;
    for (int r = 0; r < k; ++r) sum += readlane_f64(g, r);  // lane by lane
  }
  if (lane < k) {
    double v = normalize ? g / sum : g;
    v = v * (double)route_scale;
    ids[t * k + lane] = my_id;
    w[t * k + lane] = (float)v;
  }
}

}  // namespace

hipError_t launch_route_topk(const float* z, const float* bias, int64_t T, int E, int k, int normalize,
                             float route_scale, int32_t* ids, float* w, hipStream_t s) {
  if (E <= 16 * kWaveSize) {
    const int64_t blocks = (T + 3) / 4;
#define K3_ROUTE(NP)                                                                                            \
  hipLaunchKernelGGL(route_topk_reg_kernel<NP>, dim3((unsigned)blocks), dim3(256), 0, s, z, bias, T, E, k, \
                     normalize, route_scale, ids, w)
    if (E <= kWaveSize) K3_ROUTE(1);
    else if (E <= 2 * kWaveSize) K3_ROUTE(2);
    else if (E <= 4 * kWaveSize) K3_ROUTE(4);
    else if (E <= 8 * kWaveSize) K3_ROUTE(8);
    else K3_ROUTE(16);
#undef K3_ROUTE
    return hipGetLastError();
  }
  const size_t per_wave = (size_t)E * sizeof(double);
  constexpr size_t kLdsBudget = 64 * 1024;
  if (per_wave <= kLdsBudget) {
    int waves = (int)(kLdsBudget / per_wave);
    waves = waves > 4 ? 4 : waves;
    const int64_t blocks = (T + waves - 1) / waves;
    hipLaunchKernelGGL(route_topk_kernel<true>, dim3((unsigned)blocks), dim3(waves * kWaveSize), per_wave * waves, s,
                       z, bias, T, E, k, normalize, route_scale, ids, w);
  } else {
    const int64_t blocks = (T + 3) / 4;
    hipLaunchKernelGGL(route_topk_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, z, bias, T, E, k,
                       normalize, route_scale, ids, w);
  }
  return hipGetLastError();
}

}  // namespace k3moe
