// Router: logits = x W_g^T on bf16 MFMA (or fp32 FMA), then per token the K
// largest (biased) logits and the softmax over them, plus the optional
// pre-capacity expert histogram.
//
// Method: "MoE大模型专家并行与动态路由优化" section 一 (g = Softmax(TopK(W_g x)))
// and 3.1 (TopKGate: bias-free linear gate, topk, softmax of the top-k logits).
// Tie rule (not fixed by the page): equal logits -> lower expert id first.
#include "moe_internal.hpp"

namespace moe {

namespace {

// --------------------------------------------------------------------------
// top-k + softmax of one token held by a group of G lanes.
// Lane j of the group holds experts j, j+G, j+2G, ... (at most VMAX of them).
// K rounds of (lane-local best, butterfly reduce over the group); the winner
// is (largest value, then smallest id).  After the rounds, lane k < K of the
// group holds slot k's (value, id); the softmax is formed from those.
// --------------------------------------------------------------------------
__device__ __forceinline__ void better(float& v, int& e, float v2, int e2) {
  if (v2 > v || (v2 == v && e2 < e)) {
    v = v2;
    e = e2;
  }
}

template <int G, int VMAX>
__device__ __forceinline__ void topk_group(const float (&val)[VMAX], int E, int K, int gl,
                                           float& slot_v, int& slot_e) {
  uint32_t taken = 0;
  slot_v = -INFINITY;
  slot_e = 0x7fffffff;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < VMAX; ++j) {
      const int e = gl + j * G;
      if (e < E && !((taken >> j) & 1u)) better(bv, be, val[j], e);
    }
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, G);
      const int oe = __shfl_xor(be, off, G);
      better(bv, be, ov, oe);
    }
    // every lane of the group now holds the winner
    if (be % G == gl && be < E) taken |= 1u << (be / G);
    if (gl == k) {
      slot_v = bv;
      slot_e = be;
    }
  }
}

// Softmax over the K slots held by lanes 0..K-1 of a G-lane group (G >= K is
// guaranteed by the launcher: groups are at least K lanes wide).
template <int G>
__device__ __forceinline__ float topk_gate(float slot_v, int gl, int K) {
  const float vmax = __shfl(slot_v, 0, G);
  const float w = (gl < K) ? expf(slot_v - vmax) : 0.0f;
  float s = w;
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, G);
  return w / s;
}

// --------------------------------------------------------------------------
// Standalone top-k kernel over fp32 logits in global memory.
// --------------------------------------------------------------------------
template <int G, int VMAX>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   const float* __restrict__ bias,
                                                   int32_t* __restrict__ idx,
                                                   float* __restrict__ gate,
                                                   int32_t* __restrict__ load, int T, int E,
                                                   int K, int tokens_per_block) {
  __shared__ int hist[kMaxExperts];
  const int tid = threadIdx.x;
  const int gl = tid % G;
  const int grp = tid / G;
  constexpr int GPB = 256 / G;  // groups per block
  if (load) {
    for (int e = tid; e < E; e += 256) hist[e] = 0;
    __syncthreads();
  }
  const int t_begin = blockIdx.x * tokens_per_block;
  const int t_end = min(T, t_begin + tokens_per_block);
  for (int t = t_begin + grp; t < t_end; t += GPB) {
    float val[VMAX];
    const float* row = logits + (size_t)t * E;
#pragma unroll
    for (int j = 0; j < VMAX; ++j) {
      const int e = gl + j * G;
      float v = -INFINITY;
      if (e < E) {
        v = row[e];
        if (bias) v = v + bias[e];
      }
      val[j] = v;
    }
    float sv;
    int se;
    topk_group<G, VMAX>(val, E, K, gl, sv, se);
    const float g = topk_gate<G>(sv, gl, K);
    if (gl < K) {
      idx[(size_t)t * K + gl] = se;
      gate[(size_t)t * K + gl] = g;
      if (load) atomicAdd(&hist[se], 1);
    }
  }
  if (load) {
    __syncthreads();
    for (int e = tid; e < E; e += 256)
      if (hist[e]) atomicAdd(&load[e], hist[e]);
  }
}

// --------------------------------------------------------------------------
// bf16 router product on MFMA (v_mfma_f32_16x16x32_bf16), fused with the
// top-k when the workgroup's expert tile covers all E experts.
//
// Workgroup: 256 threads = 4 waves, 16 tokens x EB = 16*NT experts.  The
// reduction dim (h) is split across the 4 waves by 32-wide k-steps (wave w
// takes steps w, w+4, ...); partial sums are added in LDS in wave order, so
// the result is deterministic.  MFMA operands: A = W_g rows (experts), B = x
// rows (tokens), both read straight from global memory (16 bytes per lane).
// Lane l supplies row (l % 16) and k-group (l / 16) * 8 .. +7 of each
// 32-wide step; the accumulator lane l holds token (l % 16) and experts
// (l / 16) * 4 + 0..3 of its 16x16 tile.
// --------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(256) void router_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg,
    const float* __restrict__ bias, float* __restrict__ logits, int32_t* __restrict__ idx,
    float* __restrict__ gate, int32_t* __restrict__ load, int T, int h, int E, int K,
    int fuse_topk) {
  constexpr int EB = 16 * NT;
  __shared__ float red[4][NT][64][4];
  __shared__ float tile[16][EB + 1];
  __shared__ int hist[EB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * 16;
  const int e0 = blockIdx.y * EB;
  const int tok = t0 + (lane & 15);
  const int kg = (lane >> 4) * 8;
  const uint16_t* xrow = x + (size_t)min(tok, T - 1) * h + kg;
  const uint16_t* wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    wrow[nt] = wg + (size_t)min(e0 + nt * 16 + (lane & 15), E - 1) * h + kg;

  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // wave w takes k-steps w, w+4, ...; each trip issues the loads of U steps
  // before their MFMAs, so a wave waits on memory once per U steps
  constexpr int U = NT == 4 ? 4 : 8;
  const int nsteps = h / 32;
  for (int s0 = wave; s0 < nsteps; s0 += 4 * U) {
    uint4 xb[U], wa[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s0 + 4 * u) * 32;
      if (s0 + 4 * u < nsteps) {
        xb[u] = *(const uint4*)(xrow + k);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) wa[u][nt] = *(const uint4*)(wrow[nt] + k);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + 4 * u < nsteps)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wa[u][nt]),
                                                            __builtin_bit_cast(bf16x8, xb[u]),
                                                            acc[nt], 0, 0, 0);
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][nt][lane][r] = acc[nt][r];
  __syncthreads();
  // fixed-order sum over the 4 waves; thread -> (nt, lane) pairs
  for (int p = tid; p < NT * 64; p += 256) {
    const int nt = p / 64, l = p % 64;
    const int tt = l & 15;
    const int t = t0 + tt;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = ((red[0][nt][l][r] + red[1][nt][l][r]) + red[2][nt][l][r]) + red[3][nt][l][r];
      const int el = nt * 16 + (l >> 4) * 4 + r;
      const int e = e0 + el;
      tile[tt][el] = v;
      if (t < T && e < E) logits[(size_t)t * E + e] = v;
    }
  }
  if (!fuse_topk) return;
  // ---- fused top-k (this workgroup holds all E experts of its 16 tokens)
  if (load) {
    for (int e = tid; e < E; e += 256) hist[e] = 0;
  }
  __syncthreads();
  // 16 lanes per token: 4 waves x 4 tokens -> 16 tokens in one pass
  constexpr int G = 16;
  constexpr int VMAX = NT;  // E <= 16 * NT
  const int gl = tid % G;
  const int tt = tid / G;
  const int t = t0 + tt;
  float val[VMAX];
#pragma unroll
  for (int j = 0; j < VMAX; ++j) {
    const int e = gl + j * G;
    float v = -INFINITY;
    if (e < E) {
      v = tile[tt][e];
      if (bias) v = v + bias[e];
    }
    val[j] = v;
  }
  float sv;
  int se;
  topk_group<G, VMAX>(val, E, K, gl, sv, se);
  const float g = topk_gate<G>(sv, gl, K);
  if (t < T && gl < K) {
    idx[(size_t)t * K + gl] = se;
    gate[(size_t)t * K + gl] = g;
    if (load) atomicAdd(&hist[se], 1);
  }
  if (load) {
    __syncthreads();
    for (int e = tid; e < E; e += 256)
      if (hist[e]) atomicAdd(&load[e], hist[e]);
  }
}

// fp32 router product: one thread per logit, sequential fp32 FMA over h.
__global__ __launch_bounds__(256) void router_f32_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ wg,
                                                         float* __restrict__ logits, int T,
                                                         int h, int E) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  const float* a = x + (size_t)t * h;
  const float* b = wg + (size_t)e * h;
  float acc = 0.f;
  for (int j = 0; j < h; ++j) acc = fmaf(a[j], b[j], acc);
  logits[i] = acc;
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <int G, int VMAX>
hipError_t launch_topk_t(const float* logits, const float* bias, int32_t* idx, float* gate,
                         int32_t* load, int T, int E, int K, hipStream_t s) {
  constexpr int GPB = 256 / G;
  const int tpb = GPB * 4;
  const int grid = (T + tpb - 1) / tpb;
  hipLaunchKernelGGL((topk_kernel<G, VMAX>), dim3(grid), dim3(256), 0, s, logits, bias, idx,
                     gate, load, T, E, K, tpb);
  return hipGetLastError();
}

int pow2ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

}  // namespace

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_topk_softmax(const float* logits, const float* bias, int32_t* idx,
                               float* gate, int32_t* load, int T, int E, int K,
                               hipStream_t s) {
  if (T == 0) return hipSuccess;
  // group width: at least K lanes (the softmax reads slots from lanes < K)
  int G = pow2ceil(E);
  if (G > 64) G = 64;
  if (G < pow2ceil(K)) G = pow2ceil(K);
  if (G <= 64 && E <= G) {
    switch (G) {
      case 1: return launch_topk_t<1, 1>(logits, bias, idx, gate, load, T, E, K, s);
      case 2: return launch_topk_t<2, 1>(logits, bias, idx, gate, load, T, E, K, s);
      case 4: return launch_topk_t<4, 1>(logits, bias, idx, gate, load, T, E, K, s);
      case 8: return launch_topk_t<8, 1>(logits, bias, idx, gate, load, T, E, K, s);
      case 16: return launch_topk_t<16, 1>(logits, bias, idx, gate, load, T, E, K, s);
      case 32: return launch_topk_t<32, 1>(logits, bias, idx, gate, load, T, E, K, s);
      default: return launch_topk_t<64, 1>(logits, bias, idx, gate, load, T, E, K, s);
    }
  }
  const int v = pow2ceil((E + 63) / 64);
  switch (v) {
    case 2: return launch_topk_t<64, 2>(logits, bias, idx, gate, load, T, E, K, s);
    case 4: return launch_topk_t<64, 4>(logits, bias, idx, gate, load, T, E, K, s);
    case 8: return launch_topk_t<64, 8>(logits, bias, idx, gate, load, T, E, K, s);
    default: return launch_topk_t<64, 16>(logits, bias, idx, gate, load, T, E, K, s);
  }
}

hipError_t launch_router_gemm_bf16(const uint16_t* x, const uint16_t* wg, float* logits,
                                   int T, int h, int E, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int gx = (T + 15) / 16;
  const int NT = E <= 16 ? 1 : (E <= 32 ? 2 : 4);
  const int gy = (E + 16 * NT - 1) / (16 * NT);
  switch (NT) {
    case 1:
      hipLaunchKernelGGL((router_bf16_kernel<1>), dim3(gx, gy), dim3(256), 0, s, x, wg,
                         nullptr, logits, nullptr, nullptr, nullptr, T, h, E, 0, 0);
      break;
    case 2:
      hipLaunchKernelGGL((router_bf16_kernel<2>), dim3(gx, gy), dim3(256), 0, s, x, wg,
                         nullptr, logits, nullptr, nullptr, nullptr, T, h, E, 0, 0);
      break;
    default:
      hipLaunchKernelGGL((router_bf16_kernel<4>), dim3(gx, gy), dim3(256), 0, s, x, wg,
                         nullptr, logits, nullptr, nullptr, nullptr, T, h, E, 0, 0);
      break;
  }
  return hipGetLastError();
}

// Fused router product + top-k for E <= 64 (one workgroup holds every expert
// of its 16 tokens).  K <= 16 (the 16-lane groups hold one slot per lane).
hipError_t launch_router_topk_bf16(const uint16_t* x, const uint16_t* wg, const float* bias,
                                   float* logits, int32_t* idx, float* gate, int32_t* load,
                                   int T, int h, int E, int K, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int gx = (T + 15) / 16;
  const int NT = E <= 16 ? 1 : (E <= 32 ? 2 : 4);
  switch (NT) {
    case 1:
      hipLaunchKernelGGL((router_bf16_kernel<1>), dim3(gx, 1), dim3(256), 0, s, x, wg, bias,
                         logits, idx, gate, load, T, h, E, K, 1);
      break;
    case 2:
      hipLaunchKernelGGL((router_bf16_kernel<2>), dim3(gx, 1), dim3(256), 0, s, x, wg, bias,
                         logits, idx, gate, load, T, h, E, K, 1);
      break;
    default:
      hipLaunchKernelGGL((router_bf16_kernel<4>), dim3(gx, 1), dim3(256), 0, s, x, wg, bias,
                         logits, idx, gate, load, T, h, E, K, 1);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_router_gemm_f32(const float* x, const float* wg, float* logits, int T,
                                  int h, int E, hipStream_t s) {
  const int64_t n = (int64_t)T * E;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(router_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     x, wg, logits, T, h, E);
  return hipGetLastError();
}

}  // namespace moe
