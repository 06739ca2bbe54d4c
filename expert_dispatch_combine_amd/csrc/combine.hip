// Weighted combine in original token order, atomic-free and deterministic.
//
// Method: "46. MoE Expert Parallel | MoE 专家并行" combine_expert_outputs (weighted
// expert outputs added back into their tokens' rows, starting from zeros) and
// "专家并行（Expert Parallelism）" Combine.  Instead of scattering with
// index_add, every token GATHERS its own accepted expert rows:
//   out[t] = sum_{k ascending, route_row[t,k] >= 0} gate[t,k] * Y[route_row[t,k]]
// in fp32, so each output element is written once by one thread in a fixed
// order.  Each workgroup handles TB tokens; their rows/gates are staged in LDS.
#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int kMaxTB = 64;

template <bool VEC>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ route_row,
                                                      const float* __restrict__ gate,
                                                      float* __restrict__ out, int T, int K,
                                                      int h, int TB) {
  __shared__ int s_row[kMaxTB * kMaxTopK];
  __shared__ float s_gate[kMaxTB * kMaxTopK];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TB;
  const int ntok = min(TB, T - t0);
  for (int j = tid; j < ntok * K; j += 256) {
    s_row[j] = route_row[(size_t)t0 * K + j];
    s_gate[j] = gate[(size_t)t0 * K + j];
  }
  __syncthreads();
  const int hv = VEC ? h / 4 : h;  // vectors per row
  const int total = ntok * hv;
  for (int i = tid; i < total; i += 256) {
    const int tl = i / hv, c = i - tl * hv;
    const int* rows = s_row + tl * K;
    const float* gs = s_gate + tl * K;
    if (VEC) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int k = 0; k < K; ++k) {
        const int r = rows[k];
        if (r < 0) continue;
        const float g = gs[k];
        const float4 v = ((const float4*)(y + (size_t)r * h))[c];
        acc.x = fmaf(g, v.x, acc.x);
        acc.y = fmaf(g, v.y, acc.y);
        acc.z = fmaf(g, v.z, acc.z);
        acc.w = fmaf(g, v.w, acc.w);
      }
      ((float4*)(out + (size_t)(t0 + tl) * h))[c] = acc;
    } else {
      float acc = 0.f;
      for (int k = 0; k < K; ++k) {
        const int r = rows[k];
        if (r < 0) continue;
        acc = fmaf(gs[k], y[(size_t)r * h + c], acc);
      }
      out[(size_t)(t0 + tl) * h + c] = acc;
    }
  }
}

}  // namespace

hipError_t launch_combine(const float* y, const int32_t* route_row, const float* gate,
                          float* out, int T, int K, int h, hipStream_t s) {
  if (T == 0 || h == 0) return hipSuccess;
  const bool vec = (h % 4) == 0;
  const int hv = vec ? h / 4 : h;
  int TB = (1024 + hv - 1) / hv;  // about 4 vectors per thread
  if (TB > kMaxTB) TB = kMaxTB;
  if (TB < 1) TB = 1;
  const int grid = (T + TB - 1) / TB;
  if (vec)
    hipLaunchKernelGGL((combine_kernel<true>), dim3(grid), dim3(256), 0, s, y, route_row, gate,
                       out, T, K, h, TB);
  else
    hipLaunchKernelGGL((combine_kernel<false>), dim3(grid), dim3(256), 0, s, y, route_row,
                       gate, out, T, K, h, TB);
  return hipGetLastError();
}

}  // namespace moe
