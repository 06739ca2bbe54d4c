// Weighted combine in original token order, atomic-free and deterministic.
//
// Method: "46. MoE Expert Parallel | MoE 专家并行" combine_expert_outputs (weighted
// expert outputs added back into their tokens' rows, starting from zeros) and
// "专家并行（Expert Parallelism）" Combine.  Instead of scattering with
// index_add, every token GATHERS its own accepted expert rows:
//   out[t] = sum_{k ascending, route_row[t,k] >= 0} gate[t,k] * Y[route_row[t,k]]
// in fp32, so each output element is written once by one thread in a fixed
// order.  Each workgroup handles TB tokens; their rows/gates are staged in LDS.
#include <type_traits>

#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int kMaxTB = 64;

// Each thread takes U output vectors at a time and issues the U loads of one
// k before their FMAs, so it waits on memory K times per U vectors.
template <bool VEC, int U>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ route_row,
                                                      const float* __restrict__ gate,
                                                      float* __restrict__ out, int T, int K,
                                                      int h, int TB) {
  __shared__ int s_row[kMaxTB * kMaxTopK];
  __shared__ float s_gate[kMaxTB * kMaxTopK];
  using V = typename std::conditional<VEC, float4, float>::type;
  constexpr int NV = VEC ? 4 : 1;
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TB;
  const int ntok = min(TB, T - t0);
  for (int j = tid; j < ntok * K; j += 256) {
    s_row[j] = route_row[(size_t)t0 * K + j];
    s_gate[j] = gate[(size_t)t0 * K + j];
  }
  __syncthreads();
  const int hv = h / NV;  // vectors per row
  const int total = ntok * hv;
  const V* yv = (const V*)y;
  V* ov = (V*)(out + (size_t)t0 * h);
  for (int i0 = tid; i0 < total; i0 += 256 * U) {
    int tl[U], c[U];
    float acc[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(i0 + u * 256, total - 1);
      tl[u] = i / hv;
      c[u] = i - tl[u] * hv;
#pragma unroll
      for (int q = 0; q < NV; ++q) acc[u][q] = 0.f;
    }
    for (int k = 0; k < K; ++k) {
      V v[U];
      int r[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        r[u] = s_row[tl[u] * K + k];
        if (r[u] >= 0) v[u] = yv[(size_t)r[u] * hv + c[u]];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (r[u] < 0) continue;
        const float g = s_gate[tl[u] * K + k];
        const float* vf = (const float*)&v[u];
#pragma unroll
        for (int q = 0; q < NV; ++q) acc[u][q] = fmaf(g, vf[q], acc[u][q]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u * 256 >= total) continue;
      V o;
      float* of = (float*)&o;
#pragma unroll
      for (int q = 0; q < NV; ++q) of[q] = acc[u][q];
      ov[(size_t)tl[u] * hv + c[u]] = o;
    }
  }
}

}  // namespace

hipError_t launch_combine(const float* y, const int32_t* route_row, const float* gate,
                          float* out, int T, int K, int h, hipStream_t s) {
  if (T == 0 || h == 0) return hipSuccess;
  constexpr int U = 4;
  const bool vec = (h % 4) == 0;
  const int hv = vec ? h / 4 : h;
  int TB = 256 * U / hv;  // about U vectors per thread
  if (TB > kMaxTB) TB = kMaxTB;
  if (TB < 1) TB = 1;
  const int grid = (T + TB - 1) / TB;
  // one token per workgroup and rows of up to 2048 vectors: every thread
  // takes all its vectors in one trip (no partly idle second trip)
  const int u1 = (hv + 255) / 256;
  if (vec && TB == 1 && u1 > U && u1 <= 8) {
    switch (u1) {
      case 5:
        hipLaunchKernelGGL((combine_kernel<true, 5>), dim3(grid), dim3(256), 0, s, y,
                           route_row, gate, out, T, K, h, TB);
        break;
      case 6:
        hipLaunchKernelGGL((combine_kernel<true, 6>), dim3(grid), dim3(256), 0, s, y,
                           route_row, gate, out, T, K, h, TB);
        break;
      case 7:
        hipLaunchKernelGGL((combine_kernel<true, 7>), dim3(grid), dim3(256), 0, s, y,
                           route_row, gate, out, T, K, h, TB);
        break;
      default:
        hipLaunchKernelGGL((combine_kernel<true, 8>), dim3(grid), dim3(256), 0, s, y,
                           route_row, gate, out, T, K, h, TB);
        break;
    }
  } else if (vec)
    hipLaunchKernelGGL((combine_kernel<true, U>), dim3(grid), dim3(256), 0, s, y, route_row,
                       gate, out, T, K, h, TB);
  else
    hipLaunchKernelGGL((combine_kernel<false, U>), dim3(grid), dim3(256), 0, s, y, route_row,
                       gate, out, T, K, h, TB);
  return hipGetLastError();
}

}  // namespace moe
