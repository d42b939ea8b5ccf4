// Sigmoid + bias top-k router (one 64-lane wavefront per token).
//
// Routing parameters from the llama.cpp pull request "model: add Kimi-K3 text
// model", converter dry-run comment: 896 experts, 16 used, sigmoid expert
// score gating, per-expert bias exp_probs_b.  Scores are evaluated in fp64 so
// that the selected ids are reproducible bit for bit; ties go to the lower
// expert index; NaN scores rank last.
//
// Each wave first writes the E scores of its token to LDS (when they fit),
// then runs k selection rounds.  Round r picks, among the experts that rank
// strictly after the one picked in round r-1, the best one: every lane scans
// its strided share of experts, then a 6-step butterfly reduces the 64
// candidates.  No "already taken" flags are needed, so nothing limits E; when
// E scores do not fit in LDS the scores are recomputed from the logits each
// round instead.
#include "k3moe_internal.h"

#include <math.h>

namespace k3moe {
namespace {

constexpr int kWaveSize = 64;

__device__ __forceinline__ double route_score(float z, float b) {
  double s = 1.0 / (1.0 + exp(-(double)z)) + (double)b;
  return isnan(s) ? -INFINITY : s;
}

// (sa, ea) ranks before (sb, eb): higher score, or equal score and lower index.
__device__ __forceinline__ bool ranks_before(double sa, int ea, double sb, int eb) {
  return sa > sb || (sa == sb && ea < eb);
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
  if (lane < k) g = 1.0 / (1.0 + exp(-(double)zt[my_id]));
  double sum = g;
  if (normalize) {
    // Sum in slot order 0..k-1 so the result does not depend on a tree shape.
    sum = 0.0;
    for (int r = 0; r < k; ++r) sum += __shfl(g, r, kWaveSize);
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
