// Aux-loss-free load balancing: the per-expert router bias update.
//
// Method: "MoE大模型专家并行与动态路由优化" section 八 (DeepSeekV3Gate): each
// token is counted at the argmax of its bias-adjusted logits, and the bias
// moves toward balance, bias += alpha * (mean_count - count).  Section 3.3
// presents this as the way to balance load without dropping tokens.
//
// The argmax of the adjusted logits is slot 0 of the router's top-k (largest
// adjusted logit, ties to the lower id), so the kernel reads topk_idx[t, 0].
// One workgroup: an LDS histogram of slot 0 over all tokens, then per expert
// the page's fp32 arithmetic with one rounding per operation (no fused
// multiply-add): mean = fp32(sum(count) / E), d = fp32(mean - count),
// step = fp32(alpha * d), bias = fp32(bias + step).
#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int kBalanceThreads = 1024;

__global__ __launch_bounds__(kBalanceThreads) void bias_update_kernel(
    const int32_t* __restrict__ idx, int T, int K, int E, float alpha,
    float* __restrict__ bias, int32_t* __restrict__ counts_out) {
  __shared__ int hist[kMaxExperts];
  __shared__ int wsum[kBalanceThreads / 64];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kBalanceThreads) hist[e] = 0;
  __syncthreads();
  // eight loads per thread in flight, then their histogram updates
  for (int t0 = 0; t0 < T; t0 += kBalanceThreads * 8) {
    int ids[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + u * kBalanceThreads + tid;
      ids[u] = t < T ? idx[(int64_t)t * K] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (ids[u] >= 0 && ids[u] < E) atomicAdd(&hist[ids[u]], 1);
  }
  __syncthreads();
  // total of the counts (integer, exact)
  int part = 0;
  for (int e = tid; e < E; e += kBalanceThreads) part += hist[e];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
  if ((tid & 63) == 0) wsum[tid >> 6] = part;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < kBalanceThreads / 64; ++w) total += wsum[w];
  {
    // separate roundings: HIP contracts a * b + c into an FMA by default
#pragma clang fp contract(off)
    const float mean = __fdiv_rn((float)total, (float)E);
    for (int e = tid; e < E; e += kBalanceThreads) {
      const float d = mean - (float)hist[e];
      const float step = alpha * d;
      bias[e] = bias[e] + step;
      if (counts_out) counts_out[e] = hist[e];
    }
  }
}

}  // namespace

hipError_t launch_bias_update(const int32_t* idx, int T, int K, int E, float alpha, float* bias,
                              int32_t* counts, hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(kBalanceThreads), 0, s, idx, T, K, E,
                     alpha, bias, counts);
  return hipGetLastError();
}

}  // namespace moe
