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

// (value, id) of the group's best lane in every lane of the group (groups of
// up to 16 lanes exchange by DPP, see dpp_partner)
template <int G>
__device__ __forceinline__ void group_best(float& bv, int& be) {
  if constexpr (G <= 16) {
    if constexpr (G >= 2) better(bv, be, dpp_partner<0>(bv), dpp_partner<0>(be));
    if constexpr (G >= 4) better(bv, be, dpp_partner<1>(bv), dpp_partner<1>(be));
    if constexpr (G >= 8) better(bv, be, dpp_partner<2>(bv), dpp_partner<2>(be));
    if constexpr (G >= 16) better(bv, be, dpp_partner<3>(bv), dpp_partner<3>(be));
  } else {
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, G);
      const int oe = __shfl_xor(be, off, G);
      better(bv, be, ov, oe);
    }
  }
}

// sum over the group in every lane of the group
template <int G>
__device__ __forceinline__ float group_sum(float s) {
  if constexpr (G <= 16) {
    if constexpr (G >= 2) s += dpp_partner<0>(s);
    if constexpr (G >= 4) s += dpp_partner<1>(s);
    if constexpr (G >= 8) s += dpp_partner<2>(s);
    if constexpr (G >= 16) s += dpp_partner<3>(s);
  } else {
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, G);
  }
  return s;
}

// vmax receives the largest value (slot 0's, known to every lane).
template <int G, int VMAX>
__device__ __forceinline__ void topk_group(const float (&val)[VMAX], int E, int K, int gl,
                                           float& slot_v, int& slot_e, float& vmax) {
  uint32_t taken = 0;
  slot_v = -INFINITY;
  slot_e = 0x7fffffff;
  vmax = -INFINITY;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < VMAX; ++j) {
      const int e = gl + j * G;
      if (e < E && !((taken >> j) & 1u)) better(bv, be, val[j], e);
    }
    group_best<G>(bv, be);
    // every lane of the group now holds the winner
    if (k == 0) vmax = bv;
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
__device__ __forceinline__ float topk_gate(float slot_v, float vmax, int gl, int K) {
  const float w = (gl < K) ? expf(slot_v - vmax) : 0.0f;
  return w / group_sum<G>(w);
}

// Most h ranges a router product is split into (the top-k kernels add the
// partial products of at most this many ranges).
constexpr int kMaxRouterSplit = 8;

// Logits e_j = gl + j*G (j < VMAX, e_j < E) of one token from the KS partial
// products at pt[e + k * pstride], added in range order.  Every load is
// issued before the first addition: the partials were just written by other
// XCDs, so each dependent load would cost a full memory round trip.  Ranges
// k >= KS re-read range KS - 1 (a cache hit) and are not added; lanes past E
// read logit E - 1 and discard it.
template <int VMAX, int G>
__device__ __forceinline__ void sum_parts(const float* __restrict__ pt, int KS, int64_t pstride,
                                          int gl, int E, float (&v)[VMAX]) {
  float p[VMAX][kMaxRouterSplit];
#pragma unroll
  for (int j = 0; j < VMAX; ++j) {
    const int e = min(gl + j * G, E - 1);
#pragma unroll
    for (int k = 0; k < kMaxRouterSplit; ++k) p[j][k] = pt[e + min(k, KS - 1) * pstride];
  }
#pragma unroll
  for (int j = 0; j < VMAX; ++j) {
    v[j] = p[j][0];
#pragma unroll
    for (int k = 1; k < kMaxRouterSplit; ++k)
      if (k < KS) v[j] += p[j][k];
  }
}

// Logit biases of this lane's experts e_j = gl + j*G (lanes past E read
// bias[E - 1] and never use it), every load issued before the first is used:
// a bias read where it is added would cost a memory round trip per expert
// and per token.
template <int VMAX, int G>
__device__ __forceinline__ void lane_bias(const float* __restrict__ bias, int gl, int E,
                                          float (&b)[VMAX]) {
#pragma unroll
  for (int j = 0; j < VMAX; ++j) b[j] = bias[min(gl + j * G, E - 1)];
}

// --------------------------------------------------------------------------
// Standalone top-k kernel over fp32 logits in global memory.  With `parts`
// the logits are first formed as the sum of KS partial products over
// disjoint h ranges, added in range order (deterministic), and written out.
// --------------------------------------------------------------------------
template <int G, int VMAX>
__global__ __launch_bounds__(256) void topk_kernel(float* __restrict__ logits,
                                                   const float* __restrict__ parts, int KS,
                                                   int64_t pstride,
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
  float bv[VMAX];
  if (bias) lane_bias<VMAX, G>(bias, gl, E, bv);
  for (int t = t_begin + grp; t < t_end; t += GPB) {
    float val[VMAX];
    float* row = logits + (size_t)t * E;
    float ps[VMAX];
    if (parts) sum_parts<VMAX, G>(parts + (size_t)t * E, KS, pstride, gl, E, ps);
#pragma unroll
    for (int j = 0; j < VMAX; ++j) {
      const int e = gl + j * G;
      float v = -INFINITY;
      if (e < E) {
        if (parts) {
          v = ps[j];
          row[e] = v;
        } else {
          v = row[e];
        }
        if (bias) v = v + bv[j];
      }
      val[j] = v;
    }
    float sv;
    int se;
    float vm;
    topk_group<G, VMAX>(val, E, K, gl, sv, se, vm);
    const float g = topk_gate<G>(sv, vm, gl, K);
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
// Top-k by selection for E > 64: one wave per token, lane l holding experts
// l, l+64, ... as order-preserving integer keys.  The K-th largest key is
// found bit by bit from the top with wave-wide ballot counts (32 steps, no
// data exchange between lanes); the winners are the keys above it plus the
// lowest-id keys equal to it (the tie rule), compacted into LDS in id order;
// lanes 0..K-1 then rank their winner among the K by (value, then lower id)
// and write slot rank.  The softmax is over the K biased logits, as in the
// group kernel above.
// --------------------------------------------------------------------------
// larger float -> larger key (finite values and infinities); -0 and +0 share
// the key of +0, as they compare equal
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) == 0) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int VMAX>
__global__ __launch_bounds__(256) void topk_select_kernel(float* __restrict__ logits,
                                                          const float* __restrict__ parts,
                                                          int KS, int64_t pstride,
                                                          const float* __restrict__ bias,
                                                          int32_t* __restrict__ idx,
                                                          float* __restrict__ gate,
                                                          int32_t* __restrict__ load, int T,
                                                          int E, int K) {
  __shared__ uint32_t wkey[4][kMaxTopK];
  __shared__ int wid[4][kMaxTopK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  const bool valid = t < T;  // uniform per wave; idle waves still reach the barrier
  // keys; 0 (below every finite value and -inf) pads lanes past E
  uint32_t key[VMAX];
  float ps[VMAX], bv[VMAX];
  if (valid && bias) lane_bias<VMAX, 64>(bias, lane, E, bv);
  if (valid && parts) sum_parts<VMAX, 64>(parts + (size_t)t * E, KS, pstride, lane, E, ps);
#pragma unroll
  for (int j = 0; j < VMAX; ++j) {
    const int e = lane + 64 * j;
    uint32_t k = 0;
    if (valid && e < E) {
      float* row = logits + (size_t)t * E;
      float v;
      if (parts) {
        v = ps[j];
        row[e] = v;
      } else {
        v = row[e];
      }
      if (bias) v = v + bv[j];
      k = order_key(v);
    }
    key[j] = k;
  }
  // thr = largest value with at least K keys >= thr, i.e. the K-th largest key
  uint32_t thr = 0;
  if (valid) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < VMAX; ++j) cnt += __popcll(__ballot(key[j] >= cand));
      if (cnt >= K) thr = cand;
    }
  }
  int ngt = 0;
#pragma unroll
  for (int j = 0; j < VMAX; ++j) ngt += __popcll(__ballot(valid && key[j] > thr));
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int neq = 0, nwin = 0;
#pragma unroll
  for (int j = 0; j < VMAX; ++j) {
    const bool eq = valid && key[j] == thr;
    const uint64_t eqm = __ballot(eq);
    const bool sel =
        (valid && key[j] > thr) || (eq && neq + __popcll(eqm & below) < K - ngt);
    const uint64_t wm = __ballot(sel);
    if (sel) {
      const int p = nwin + __popcll(wm & below);
      wkey[wave][p] = key[j];
      wid[wave][p] = lane + 64 * j;
    }
    neq += __popcll(eqm);
    nwin += __popcll(wm);
  }
  __syncthreads();
  if (!valid || lane >= K) return;
  const uint32_t kq = wkey[wave][lane];
  const int iq = wid[wave][lane];
  int rank = 0;
  uint32_t kmax = 0;
  for (int p = 0; p < K; ++p) {
    const uint32_t kp = wkey[wave][p];
    rank += (kp > kq) || (kp == kq && wid[wave][p] < iq);
    kmax = max(kmax, kp);
  }
  const float vmax = key_float(kmax);
  float sum = 0.f;
  for (int p = 0; p < K; ++p) sum += expf(key_float(wkey[wave][p]) - vmax);
  idx[(size_t)t * K + rank] = iq;
  gate[(size_t)t * K + rank] = expf(key_float(kq) - vmax) / sum;
  if (load) atomicAdd(&load[iq], 1);
}

template <int VMAX>
hipError_t launch_topk_select_t(float* logits, const float* parts, int KS, const float* bias,
                                int32_t* idx, float* gate, int32_t* load, int T, int E, int K,
                                hipStream_t s) {
  hipLaunchKernelGGL((topk_select_kernel<VMAX>), dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s,
                     logits, parts, KS, (int64_t)T * E, bias, idx, gate, load, T, E, K);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// bf16 router product on MFMA (v_mfma_f32_16x16x32_bf16) fused with the
// top-k, for short batches with E <= 64 (one workgroup holds every expert of
// its 16 tokens).
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
    float* __restrict__ gate, int32_t* __restrict__ load, int T, int h, int E, int K) {
  constexpr int EB = 16 * NT;
  __shared__ float red[4][NT][64][4];
  __shared__ float tile[16][EB + 1];
  __shared__ int hist[EB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * 16;
  const int tok = t0 + (lane & 15);
  const int kg = (lane >> 4) * 8;
  const uint16_t* xrow = x + (size_t)min(tok, T - 1) * h + kg;
  const uint16_t* wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    wrow[nt] = wg + (size_t)min(nt * 16 + (lane & 15), E - 1) * h + kg;

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
      const int e = el;
      tile[tt][el] = v;
      if (t < T && e < E) logits[(size_t)t * E + e] = v;
    }
  }
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
  float bv[VMAX];
  if (bias) lane_bias<VMAX, G>(bias, gl, E, bv);
  float val[VMAX];
#pragma unroll
  for (int j = 0; j < VMAX; ++j) {
    const int e = gl + j * G;
    float v = -INFINITY;
    if (e < E) {
      v = tile[tt][e];
      if (bias) v = v + bv[j];
    }
    val[j] = v;
  }
  float sv;
  int se;
  float vm;
  topk_group<G, VMAX>(val, E, K, gl, sv, se, vm);
  const float g = topk_gate<G>(sv, vm, gl, K);
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

// --------------------------------------------------------------------------
// Tiled bf16 router product for long batches or many experts
// (v_mfma_f32_32x32x16_bf16).  A workgroup (4 waves) owns TT tokens x EE
// experts and one of KS equal h ranges; both operands are staged through a
// double-buffered, XOR-swizzled LDS tile in 64-wide k-chunks, prefetched
// RD chunks ahead in registers, so every x row is read once per expert tile
// and every W_g row once per token tile (instead of once per 16 tokens).
// The waves form a GT x (4/GT) grid over the tile's 32 x 32 MFMA blocks.
// KS > 1: the workgroup writes its partial product to parts[ks]; the top-k
// kernel adds the KS partials in range order.  Workgroups of one range are
// placed on the same XCDs (blockIdx % KS == range) so its W_g slice stays in
// their L2.  With KS == 1 and all experts in one tile, the top-k and softmax
// run in the same workgroup on the logits tile held in LDS.
// --------------------------------------------------------------------------
template <int TT, int EE, int GT>
struct RouterTile {
  static constexpr int GE = 4 / GT;
  static constexpr int WT = TT / 32 / GT;   // token blocks per wave
  static constexpr int WE = EE / 32 / GE;   // expert blocks per wave
  static constexpr int QX = TT * 8 / 256;   // 16-byte quads of x per thread and chunk
  static constexpr int QW = EE * 8 / 256;   // quads of W_g per thread and chunk
  static constexpr int NQ = QX + QW;
  static constexpr int RD = NQ > 8 ? 3 : 4; // chunks in flight in registers
  static constexpr int STAGE = (TT + EE) * 64;  // bf16 per LDS stage: x rows, then W_g rows
  static constexpr int PITCH = EE + 1;          // fp32 logits tile (fused top-k)
  static constexpr int LDS_BYTES =
      2 * STAGE * 2 > TT * PITCH * 4 ? 2 * STAGE * 2 : TT * PITCH * 4;
  static_assert(WT >= 1 && WE >= 1 && QX >= 1 && QW >= 1, "tile shape");
};

// quad q of LDS row r (64 bf16 per row) lives at quad q ^ ((r >> 1) & 7)
__device__ __forceinline__ int rt_slot(int r, int q) { return r * 64 + ((q ^ ((r >> 1) & 7)) << 3); }

// Top-k + softmax of the TT tokens of a logits tile in LDS ([TT][PITCH]),
// G lanes per token, 256 / G tokens per pass.  hist: LDS expert histogram or
// NULL.
template <int G, int TT, int EE, int PITCH>
__device__ __forceinline__ void tile_topk(const float* tile, const float* __restrict__ bias,
                                          int32_t* __restrict__ idx, float* __restrict__ gate,
                                          int* hist, int t0, int T, int E, int K) {
  constexpr int VMAX = EE / G;
  static_assert(VMAX <= 32, "one bit per slot of the taken mask");
  const int tid = threadIdx.x;
  const int gl = tid % G;
  float bv[VMAX];
  if (bias) lane_bias<VMAX, G>(bias, gl, E, bv);
  for (int p = 0; p < TT / (256 / G); ++p) {
    const int tl = p * (256 / G) + tid / G;
    const int t = t0 + tl;
    float val[VMAX];
#pragma unroll
    for (int j = 0; j < VMAX; ++j) {
      const int e = gl + j * G;
      float v = -INFINITY;
      if (e < E) {
        v = tile[tl * PITCH + e];
        if (bias) v = v + bv[j];
      }
      val[j] = v;
    }
    float sv, vm;
    int se;
    topk_group<G, VMAX>(val, E, K, gl, sv, se, vm);
    const float g = topk_gate<G>(sv, vm, gl, K);
    if (t < T && gl < K) {
      idx[(size_t)t * K + gl] = se;
      gate[(size_t)t * K + gl] = g;
      if (hist) atomicAdd(&hist[se], 1);
    }
  }
}

template <int TT, int EE, int GT>
__global__ __launch_bounds__(256) void router_tiled_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg,
    const float* __restrict__ bias, float* __restrict__ logits, float* __restrict__ parts,
    int32_t* __restrict__ idx, float* __restrict__ gate, int32_t* __restrict__ load, int T,
    int h, int E, int K, int KS, int fuse) {
  using S = RouterTile<TT, EE, GT>;
  __shared__ __attribute__((aligned(16))) char lds[S::LDS_BYTES];
  __shared__ int hist[EE];
  uint16_t* stg = (uint16_t*)lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lg = lane >> 5;
  const int ks = blockIdx.x % KS;
  const int t0 = (blockIdx.x / KS) * TT;
  const int e0 = blockIdx.y * EE;
  const int nch = h / 64 / KS;
  const int kbase = ks * nch * 64;

  // global sources and LDS slots of this thread's quads (x rows, then W_g rows)
  const uint16_t* src[S::NQ];
  int dst[S::NQ];
#pragma unroll
  for (int j = 0; j < S::NQ; ++j) {
    const bool isx = j < S::QX;
    const int c = tid + 256 * (isx ? j : j - S::QX);
    const int r = c >> 3, q = c & 7;
    if (isx)
      src[j] = x + (size_t)min(t0 + r, T - 1) * h + kbase + q * 8;
    else
      src[j] = wg + (size_t)min(e0 + r, E - 1) * h + kbase + q * 8;
    dst[j] = rt_slot(isx ? r : TT + r, q);
  }
  // MFMA fragments: lane (row li, half lg) supplies k = 32 lg + 8 s .. +7 of
  // the chunk at k-step s, for both operands
  const int wt = wave % GT, we = wave / GT;
  int xfr[S::WT], wfr[S::WE];
#pragma unroll
  for (int a = 0; a < S::WT; ++a) xfr[a] = rt_slot(32 * (wt * S::WT + a) + li, 4 * lg);
#pragma unroll
  for (int b = 0; b < S::WE; ++b) wfr[b] = rt_slot(TT + 32 * (we * S::WE + b) + li, 4 * lg);

  f32x16 acc[S::WT][S::WE];
#pragma unroll
  for (int a = 0; a < S::WT; ++a)
#pragma unroll
    for (int b = 0; b < S::WE; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  u32x4 reg[S::RD][S::NQ];
#pragma unroll
  for (int d = 0; d < S::RD; ++d)
    if (d < nch)
#pragma unroll
      for (int j = 0; j < S::NQ; ++j) reg[d][j] = *(const u32x4*)(src[j] + d * 64);
#pragma unroll
  for (int j = 0; j < S::NQ; ++j) *(u32x4*)(stg + dst[j]) = reg[0][j];
  __syncthreads();

  // chunk c: refill register slot SLOT with chunk c + RD, MFMAs on LDS stage
  // c & 1, then stage chunk c + 1 (slot NSLOT) into the other LDS buffer
#define MOE_ROUTER_CHUNK(SLOT, NSLOT, c, HAS_NEXT, REFILL)                                   \
  do {                                                                                       \
    if (REFILL) {                                                                            \
      _Pragma("unroll") for (int j = 0; j < S::NQ; ++j) reg[SLOT][j] =                       \
          *(const u32x4*)(src[j] + ((c) + S::RD) * 64);                                      \
    }                                                                                        \
    const uint16_t* st_ = stg + ((c) & 1) * S::STAGE;                                        \
    _Pragma("unroll") for (int s4 = 0; s4 < 4; ++s4) {                                       \
      bf16x8 xf_[S::WT], wf_[S::WE];                                                         \
      _Pragma("unroll") for (int a = 0; a < S::WT; ++a) xf_[a] =                             \
          *(const bf16x8*)(st_ + (xfr[a] ^ (s4 << 3)));                                      \
      _Pragma("unroll") for (int b = 0; b < S::WE; ++b) wf_[b] =                             \
          *(const bf16x8*)(st_ + (wfr[b] ^ (s4 << 3)));                                      \
      _Pragma("unroll") for (int a = 0; a < S::WT; ++a)                                      \
        _Pragma("unroll") for (int b = 0; b < S::WE; ++b) acc[a][b] =                        \
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf_[b], xf_[a], acc[a][b], 0, 0, 0);      \
    }                                                                                        \
    if (HAS_NEXT) {                                                                          \
      uint16_t* nst_ = stg + (((c) + 1) & 1) * S::STAGE;                                     \
      _Pragma("unroll") for (int j = 0; j < S::NQ; ++j) *(u32x4*)(nst_ + dst[j]) =           \
          reg[NSLOT][j];                                                                     \
    }                                                                                        \
    __syncthreads();                                                                         \
  } while (0)

  int c0 = 0;
  for (; c0 + 2 * S::RD <= nch; c0 += S::RD) {
#pragma unroll
    for (int p = 0; p < S::RD; ++p) MOE_ROUTER_CHUNK(p, (p + 1) % S::RD, c0 + p, true, true);
  }
#pragma unroll
  for (int p = 0; p < 2 * S::RD; ++p) {
    const int c = c0 + p;
    if (c < nch)
      MOE_ROUTER_CHUNK(p % S::RD, (p + 1) % S::RD, c, c + 1 < nch, c + S::RD < nch);
  }
#undef MOE_ROUTER_CHUNK

  // accumulator lane: token 32 a' + li, experts 32 b' + 8 q + 4 lg + 0..3
  if (!fuse) {
    float* out = KS > 1 ? parts + (size_t)ks * T * E : logits;
#pragma unroll
    for (int a = 0; a < S::WT; ++a) {
      const int t = t0 + 32 * (wt * S::WT + a) + li;
      if (t >= T) continue;
#pragma unroll
      for (int b = 0; b < S::WE; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = e0 + 32 * (we * S::WE + b) + 8 * q + 4 * lg;
          float* o = out + (size_t)t * E + e;
          if (e + 3 < E && (E & 3) == 0) {
            *(float4*)o = make_float4(acc[a][b][4 * q], acc[a][b][4 * q + 1],
                                      acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (e + i < E) o[i] = acc[a][b][4 * q + i];
          }
        }
    }
    return;
  }

  // ---- fused top-k: this workgroup holds every expert of its TT tokens
  float* tile = (float*)lds;  // [TT][PITCH]; the staging buffers are free
#pragma unroll
  for (int a = 0; a < S::WT; ++a)
#pragma unroll
    for (int b = 0; b < S::WE; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tl = 32 * (wt * S::WT + a) + li;
        const int el = 32 * (we * S::WE + b) + 8 * (r >> 2) + 4 * lg + (r & 3);
        tile[tl * S::PITCH + el] = acc[a][b][r];
      }
  if (load)
    for (int e = tid; e < EE; e += 256) hist[e] = 0;
  __syncthreads();
  for (int i = tid; i < TT * E; i += 256) {
    const int tl = i / E, e = i - tl * E;
    if (t0 + tl < T) logits[(size_t)(t0 + tl) * E + e] = tile[tl * S::PITCH + e];
  }
  // the narrowest lane group that holds K slots (fewer passes over the tile)
  int* hp = load ? hist : nullptr;
  bool done = false;
  if constexpr (EE / 4 <= 32)
    if (K <= 4) {
      tile_topk<4, TT, EE, S::PITCH>(tile, bias, idx, gate, hp, t0, T, E, K);
      done = true;
    }
  if constexpr (EE / 8 <= 32)
    if (!done && K <= 8) {
      tile_topk<8, TT, EE, S::PITCH>(tile, bias, idx, gate, hp, t0, T, E, K);
      done = true;
    }
  if (!done) tile_topk<16, TT, EE, S::PITCH>(tile, bias, idx, gate, hp, t0, T, E, K);
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
  // sequential fp32 FMAs over h; the loads of 8 terms go out before their FMAs
  float acc = 0.f;
  int j = 0;
  for (; j + 8 <= h; j += 8) {
    float av[8], bv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      av[u] = a[j + u];
      bv[u] = b[j + u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = fmaf(av[u], bv[u], acc);
  }
  for (; j < h; ++j) acc = fmaf(a[j], b[j], acc);
  logits[i] = acc;
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <int G, int VMAX>
hipError_t launch_topk_t(float* logits, const float* parts, int KS, const float* bias,
                         int32_t* idx, float* gate, int32_t* load, int T, int E, int K,
                         hipStream_t s) {
  constexpr int GPB = 256 / G;
  const int tpb = GPB * 4;
  const int grid = (T + tpb - 1) / tpb;
  hipLaunchKernelGGL((topk_kernel<G, VMAX>), dim3(grid), dim3(256), 0, s, logits, parts, KS,
                     (int64_t)T * E, bias, idx, gate, load, T, E, K, tpb);
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

hipError_t launch_topk_parts(float* logits, const float* parts, int KS, const float* bias,
                             int32_t* idx, float* gate, int32_t* load, int T, int E, int K,
                             hipStream_t s) {
  if (T == 0) return hipSuccess;
  // group width: at least K lanes (the softmax reads slots from lanes < K)
  int G = pow2ceil(E);
  if (G > 64) G = 64;
  if (G < pow2ceil(K)) G = pow2ceil(K);
  if (G <= 64 && E <= G) {
    switch (G) {
      case 1: return launch_topk_t<1, 1>(logits, parts, KS, bias, idx, gate, load, T, E, K, s);
      case 2: return launch_topk_t<2, 1>(logits, parts, KS, bias, idx, gate, load, T, E, K, s);
      case 4: return launch_topk_t<4, 1>(logits, parts, KS, bias, idx, gate, load, T, E, K, s);
      case 8: return launch_topk_t<8, 1>(logits, parts, KS, bias, idx, gate, load, T, E, K, s);
      case 16: return launch_topk_t<16, 1>(logits, parts, KS, bias, idx, gate, load, T, E, K, s);
      case 32: return launch_topk_t<32, 1>(logits, parts, KS, bias, idx, gate, load, T, E, K, s);
      default: return launch_topk_t<64, 1>(logits, parts, KS, bias, idx, gate, load, T, E, K, s);
    }
  }
  const int v = pow2ceil((E + 63) / 64);
  switch (v) {
    case 2:
      return launch_topk_select_t<2>(logits, parts, KS, bias, idx, gate, load, T, E, K, s);
    case 4:
      return launch_topk_select_t<4>(logits, parts, KS, bias, idx, gate, load, T, E, K, s);
    case 8:
      return launch_topk_select_t<8>(logits, parts, KS, bias, idx, gate, load, T, E, K, s);
    default:
      return launch_topk_select_t<16>(logits, parts, KS, bias, idx, gate, load, T, E, K, s);
  }
}

hipError_t launch_topk_softmax(const float* logits, const float* bias, int32_t* idx,
                               float* gate, int32_t* load, int T, int E, int K,
                               hipStream_t s) {
  // without partial sums the kernel only reads the logits
  return launch_topk_parts(const_cast<float*>(logits), nullptr, 1, bias, idx, gate, load, T, E,
                           K, s);
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
                         logits, idx, gate, load, T, h, E, K);
      break;
    case 2:
      hipLaunchKernelGGL((router_bf16_kernel<2>), dim3(gx, 1), dim3(256), 0, s, x, wg, bias,
                         logits, idx, gate, load, T, h, E, K);
      break;
    default:
      hipLaunchKernelGGL((router_bf16_kernel<4>), dim3(gx, 1), dim3(256), 0, s, x, wg, bias,
                         logits, idx, gate, load, T, h, E, K);
      break;
  }
  return hipGetLastError();
}

namespace {

// Tile shape of the tiled router product for E experts.
struct RouterPlan {
  int tt, ee;   // tokens x experts per workgroup
  int ks;       // h ranges (partial products) per tile
  bool fuse;    // top-k in the same kernel
};

// Shape and split of the tiled router product; ks counts the h ranges the
// workspace must hold partial products for (1: none).
RouterPlan router_plan(int T, int h, int E, int K, size_t parts_room) {
  RouterPlan p;
  if (E <= 32) { p.tt = 128; p.ee = 32; }
  else if (E <= 64) { p.tt = 64; p.ee = 64; }
  else if (E <= 128) { p.tt = 64; p.ee = 128; }
  else { p.tt = 128; p.ee = 128; }  // several expert tiles: x is re-read per tile
  const int64_t tiles = (int64_t)((T + p.tt - 1) / p.tt) * ((E + p.ee - 1) / p.ee);
  // split h while the launch still fits one workgroup per CU (256 CUs)
  p.ks = 1;
  while (p.ks < kMaxRouterSplit && tiles * p.ks * 2 <= 256 && (h / 64) % (p.ks * 2) == 0 &&
         (size_t)(p.ks * 2) * T * E * sizeof(float) <= parts_room)
    p.ks *= 2;
  p.fuse = p.ks == 1 && E <= p.ee && K <= 16;
  return p;
}

// The small-batch fused kernel (16 tokens per workgroup) serves E <= 64 until
// a batch gives the tiled one a full launch of 64-token tiles.
bool use_tiled_router(int T, int E, int K) {
  return E > 64 || K > 16 || T >= 64 * 256;
}

template <int TT, int EE, int GT>
hipError_t launch_router_tiled_t(const uint16_t* x, const uint16_t* wg, const float* bias,
                                 float* logits, float* parts, int32_t* idx, float* gate,
                                 int32_t* load, int T, int h, int E, int K, int KS, bool fuse,
                                 hipStream_t s) {
  const dim3 grid((unsigned)((T + TT - 1) / TT * KS), (unsigned)((E + EE - 1) / EE));
  hipLaunchKernelGGL((router_tiled_kernel<TT, EE, GT>), grid, dim3(256), 0, s, x, wg, bias,
                     logits, parts, idx, gate, load, T, h, E, K, KS, fuse ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

size_t router_parts_bytes(int T, int h, int E, int K) {
  if (T <= 0 || !use_tiled_router(T, E, K)) return 0;
  const RouterPlan p = router_plan(T, h, E, K, (size_t)-1);
  return p.ks > 1 ? (size_t)p.ks * T * E * sizeof(float) : 0;
}

// bf16 router: product (MFMA) + top-k + softmax (+ histogram).  `ws` (16-byte
// aligned, ws_bytes long, may be NULL) holds the partial products of a split
// h; without room for them the product runs unsplit.
hipError_t launch_router_bf16(const uint16_t* x, const uint16_t* wg, const float* bias,
                              float* logits, int32_t* idx, float* gate, int32_t* load, int T,
                              int h, int E, int K, void* ws, size_t ws_bytes, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (!use_tiled_router(T, E, K))
    return launch_router_topk_bf16(x, wg, bias, logits, idx, gate, load, T, h, E, K, s);
  const size_t room = (ws && ((uintptr_t)ws & 15) == 0) ? ws_bytes : 0;
  const RouterPlan p = router_plan(T, h, E, K, room);
  float* parts = p.ks > 1 ? (float*)ws : nullptr;
  hipError_t err;
  if (p.ee == 32)
    err = launch_router_tiled_t<128, 32, 4>(x, wg, bias, logits, parts, idx, gate, load, T, h,
                                            E, K, p.ks, p.fuse, s);
  else if (p.ee == 64)
    err = launch_router_tiled_t<64, 64, 2>(x, wg, bias, logits, parts, idx, gate, load, T, h,
                                           E, K, p.ks, p.fuse, s);
  else if (p.tt == 64)
    err = launch_router_tiled_t<64, 128, 2>(x, wg, bias, logits, parts, idx, gate, load, T, h,
                                            E, K, p.ks, p.fuse, s);
  else
    err = launch_router_tiled_t<128, 128, 2>(x, wg, bias, logits, parts, idx, gate, load, T, h,
                                             E, K, p.ks, p.fuse, s);
  if (err != hipSuccess || p.fuse) return err;
  return launch_topk_parts(logits, parts, p.ks, bias, idx, gate, load, T, E, K, s);
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
