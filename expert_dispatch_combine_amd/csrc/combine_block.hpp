// The combine of one workgroup's tokens, shared by the combine kernel and the
// fused combine + ledger kernel.
//
// Method: "46. MoE Expert Parallel | MoE 专家并行" combine_expert_outputs (weighted
// expert outputs added back into their tokens' rows, starting from zeros) and
// "专家并行（Expert Parallelism）" Combine.  Instead of scattering with
// index_add, every token GATHERS its own accepted expert rows:
//   out[t] = sum_{k ascending, route_row[t,k] >= 0} gate[t,k] * Y[route_row[t,k]]
// in fp32, so each output element is written once by one thread in a fixed
// order.
#pragma once

#include <type_traits>

#include "moe_internal.hpp"

namespace moe {


// Expert outputs are read once: nontemporal loads (large outputs, see NT).
__device__ __forceinline__ float ntl(const float* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float4 ntl(const float4* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return __builtin_bit_cast(float4, v);
}
constexpr int kMaxTB = 64;  // tokens per combine workgroup
// LDS of one combine workgroup: the tokens' rows and gates
constexpr int kCombineLdsBytes = kMaxTB * kMaxTopK * 8;

// Workgroup shape of the combine for T tokens of h fp32 values.  vec: rows
// are read as float4; TB tokens per workgroup; U vectors per thread and trip.
struct CombineShape {
  bool vec, nt;
  int TB, U, grid;
};

inline CombineShape combine_shape(int T, int K, int h) {
  CombineShape c;
  c.vec = (h % 4) == 0;
  // expert outputs of up to T*K rows: nontemporal reads above the LLC size
  c.nt = (int64_t)T * K * h * 4 > ((int64_t)256 << 20);
  c.U = 4;
  const int hv = c.vec ? h / 4 : h;
  int TB = 256 * c.U / hv;  // about U vectors per thread
  if (TB > kMaxTB) TB = kMaxTB;
  if (TB < 1) TB = 1;
  c.TB = TB;
  c.grid = (T + TB - 1) / TB;
  // one token per workgroup and rows of up to 2048 vectors: every thread
  // takes all its vectors in one trip (no partly idle second trip)
  const int u1 = (hv + 255) / 256;
  if (c.vec && TB == 1 && u1 > c.U && u1 <= 8) c.U = u1;
  return c;
}

// Workgroup b's tokens [b TB, b TB + TB).  Each thread takes U output vectors
// at a time; the U loads of route k + 1 are issued before the FMAs of route
// k, so one route's rows are always in flight while the previous one is
// added.  s_row / s_gate: LDS of TB * K entries.
// NT: read the expert outputs with nontemporal loads (chosen when they
// outgrow the 256 MB last-level cache; smaller ones are still resident there
// from the expert GEMM that wrote them, and plain loads hit it).
template <bool VEC, int U, bool NT>
__device__ __forceinline__ void combine_tokens(int b, const float* __restrict__ y,
                                               const int32_t* __restrict__ route_row,
                                               const float* __restrict__ gate,
                                               float* __restrict__ out, int T, int K, int h,
                                               int TB, int* s_row, float* s_gate) {
  using V = typename std::conditional<VEC, float4, float>::type;
  constexpr int NV = VEC ? 4 : 1;
  const int tid = threadIdx.x;
  const int t0 = b * TB;
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
    V v[U];
    int r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      r[u] = s_row[tl[u] * K];
      if (r[u] >= 0) v[u] = NT ? ntl(&yv[(size_t)r[u] * hv + c[u]]) : yv[(size_t)r[u] * hv + c[u]];
    }
    for (int k = 0; k < K; ++k) {
      V vn[U];
      int rn[U];
      const int kn = k + 1 < K ? k + 1 : k;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        rn[u] = k + 1 < K ? s_row[tl[u] * K + kn] : -1;
        if (rn[u] >= 0)
          vn[u] = NT ? ntl(&yv[(size_t)rn[u] * hv + c[u]]) : yv[(size_t)rn[u] * hv + c[u]];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (r[u] >= 0) {
          const float g = s_gate[tl[u] * K + k];
          const float* vf = (const float*)&v[u];
#pragma unroll
          for (int q = 0; q < NV; ++q) acc[u][q] = fmaf(g, vf[q], acc[u][q]);
        }
        v[u] = vn[u];
        r[u] = rn[u];
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

template <bool NT, class F>
inline void with_combine_u(const CombineShape& c, F&& f) {
  using std::integral_constant;
  using N = integral_constant<bool, NT>;
  if (!c.vec) return f(integral_constant<bool, false>(), integral_constant<int, 4>(), N());
  switch (c.U) {
    case 5: return f(integral_constant<bool, true>(), integral_constant<int, 5>(), N());
    case 6: return f(integral_constant<bool, true>(), integral_constant<int, 6>(), N());
    case 7: return f(integral_constant<bool, true>(), integral_constant<int, 7>(), N());
    case 8: return f(integral_constant<bool, true>(), integral_constant<int, 8>(), N());
    default: return f(integral_constant<bool, true>(), integral_constant<int, 4>(), N());
  }
}

// Calls f(integral_constant<bool, VEC>, integral_constant<int, U>,
// integral_constant<bool, NT>) for the combine variant `c` selects.
template <class F>
inline void with_combine_variant(const CombineShape& c, F&& f) {
  if (c.nt) return with_combine_u<true>(c, f);
  return with_combine_u<false>(c, f);
}

}  // namespace moe
