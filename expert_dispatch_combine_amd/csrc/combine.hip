// Weighted combine in original token order, atomic-free and deterministic.
//
// Method: "46. MoE Expert Parallel | MoE 专家并行" combine_expert_outputs and
// "专家并行（Expert Parallelism）" Combine; the per-workgroup gather is
// combine_tokens.  Each workgroup handles TB tokens; their rows/gates are
// staged in LDS.
#include "combine_block.hpp"

namespace moe {

namespace {

template <bool VEC, int U, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ route_row,
                                                      const float* __restrict__ gate,
                                                      float* __restrict__ out, int T, int K,
                                                      int h, int TB) {
  __shared__ int s_row[kMaxTB * kMaxTopK];
  __shared__ float s_gate[kMaxTB * kMaxTopK];
  combine_tokens<VEC, U, NT>(blockIdx.x, y, route_row, gate, out, T, K, h, TB, s_row, s_gate);
}

}  // namespace

hipError_t launch_combine(const float* y, const int32_t* route_row, const float* gate,
                          float* out, int T, int K, int h, hipStream_t s) {
  if (T == 0 || h == 0) return hipSuccess;
  const CombineShape c = combine_shape(T, K, h);
  with_combine_variant(c, [&](auto vec, auto u, auto nt) {
    hipLaunchKernelGGL((combine_kernel<decltype(vec)::value, decltype(u)::value,
                                       decltype(nt)::value>),
                       dim3(c.grid), dim3(256), 0, s, y, route_row, gate, out, T, K, h, c.TB);
  });
  return hipGetLastError();
}

}  // namespace moe
