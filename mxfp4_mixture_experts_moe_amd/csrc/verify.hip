// Distinct routed experts of a speculative verify batch by verify width.
//
// The lucebox page "feat(kimi-k3): add DSpark Q8 artifact and shared
// speculative runtime" verifies [current token] + 7 draft proposals per
// sequence and adds target cost hints so that external-memory targets do not
// over-verify (expert traffic grows with every verified row).  The bytes a
// verify pass of width w streams are those of the distinct experts its rows
// route to; this kernel counts them for every width at once.
//
// Rows are S sequences x W positions (row r = s * W + w).  One workgroup:
// every entry lowers first[e], the earliest position at which expert e is
// routed (LDS atomic min), then a histogram of first[] over positions and a
// running sum give distinct[w] = #{e : first[e] <= w}.  Integer work only;
// the result does not depend on thread timing.
#include "k3moe_internal.h"

namespace k3moe {
namespace {

constexpr int kThreads = 1024;

__global__ __launch_bounds__(kThreads) void verify_distinct_kernel(const int32_t* __restrict__ ids, int S, int W,
                                                                      int E, int k, int32_t* __restrict__ distinct) {
  extern __shared__ int32_t first[];  // [E]
  __shared__ int32_t hist[kMaxVerifyWidth];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kThreads) first[e] = W;  // W = not routed
  for (int w = tid; w < W; w += kThreads) hist[w] = 0;
  __syncthreads();
  const int64_t n = (int64_t)S * W * k;
  for (int64_t q = tid; q < n; q += kThreads) {
    const int e = ids[q];
    if (e >= 0 && e < E) {
      const int w = (int)((q / k) % W);
      atomicMin(&first[e], w);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    const int w = first[e];
    if (w < W) atomicAdd(&hist[w], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < W; ++w) {
      run += hist[w];
      distinct[w] = run;
    }
  }
}

}  // namespace

hipError_t launch_verify_distinct(const int32_t* ids, int S, int W, int E, int k, int32_t* distinct, hipStream_t s) {
  hipLaunchKernelGGL(verify_distinct_kernel, dim3(1), dim3(kThreads), (size_t)E * sizeof(int32_t), s, ids, S, W, E, k,
                     distinct);
  return hipGetLastError();
}

}  // namespace k3moe
