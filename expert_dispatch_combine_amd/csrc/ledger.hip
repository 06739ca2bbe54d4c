// Counters-only ledger of one routed batch: per-expert loads, accepted
// routes, local vs cross-rank routes under an expert -> rank map, the
// accepted-route traffic matrix between logical ranks, and the per-expert gate
// sums behind the auxiliary-loss term P_i.
//
// Method: "47. MoE Expert Parallel" Step 3 / summarize (loads, capacity,
// overflow, bytes, balance), "46. MoE Expert Parallel" TODO 2 (a route is
// local iff the token's source rank equals its expert's owner rank),
// "MoE大模型专家并行与动态路由优化" 2.2 (round-robin owner e % N) and 3.2
// (f_i, P_i, L_aux).
//
// Every counter is an integer, so the result does not depend on the order in
// which routes are added.  The gate sums are integers too: each fp32 gate
// (in [0, 1]) is rounded to a multiple of 2^-32 and the multiples are added
// exactly in 64 bits (the sum of at most 2^31 gates stays below 2^63); the
// host divides by 2^32.  Each route adds at most 2^-33 of rounding error.
//
// Device part: one workgroup per 512 routes builds LDS histograms and a
// second kernel adds the per-block partials (one wave per output value).  Up
// to kSmallLedgerRoutes routes one workgroup takes them all and writes the
// final area itself.  In the combine's launch (combine_ledger_kernel) the
// first workgroups count 1024 routes each into parts of the stage of their
// own, which the host adds.  The stage may be page-locked host memory (its
// device address), which spares a copy.  The host finishes the few scalar
// formulas in float64.
#include "combine_block.hpp"

namespace moe {

namespace {

constexpr int RPBL = kLedgerRoutesPerBlock;

struct LedgerWs {
  int32_t* blk_load;   // [nb][E]
  uint64_t* blk_P;     // [nb][E] gate sums, units of 2^-32
  int64_t* blk_cnt;    // [nb][LC_N]
  int32_t* blk_pair;   // [nb][n_ep*n_ep]
  char* fin;           // final area
  size_t fin_bytes;
  size_t total;
};

LedgerWs carve(void* ws, int64_t A, int E, int n_ep) {
  const int64_t nb = A > 0 ? (A + RPBL - 1) / RPBL : 1;
  char* p = (char*)ws;
  LedgerWs w;
  size_t o = 0;
  w.blk_load = (int32_t*)(p + o);
  o = align_up(o + (size_t)nb * E * sizeof(int32_t), 256);
  w.blk_P = (uint64_t*)(p + o);
  o = align_up(o + (size_t)nb * E * sizeof(uint64_t), 256);
  w.blk_cnt = (int64_t*)(p + o);
  o = align_up(o + (size_t)nb * LC_N * sizeof(int64_t), 256);
  w.blk_pair = (int32_t*)(p + o);
  o = align_up(o + (size_t)nb * n_ep * n_ep * sizeof(int32_t), 256);
  w.fin = p + o;
  w.fin_bytes = ledger_stage_bytes(E, n_ep);
  o = align_up(o + w.fin_bytes, 256);
  w.total = o;
  return w;
}

// Final area layout (8 bytes each): loads[E] int64, P[E] uint64 (units of
// 2^-32), counters[LC_N] int64, pair[n_ep * n_ep] int64.  The stage holds the
// part count (int64), then that many final areas of partials.
struct FinalArea {
  int64_t* load;
  uint64_t* P;
  int64_t* cnt;
  int64_t* pair;
};

__device__ __forceinline__ FinalArea final_area(char* fin, int E) {
  return {(int64_t*)fin, (uint64_t*)(fin + (size_t)E * 8), (int64_t*)(fin + (size_t)2 * E * 8),
          (int64_t*)(fin + (size_t)(2 * E + LC_N) * 8)};
}

// gate (in [0, 1]) -> nearest multiple of 2^-32, as an integer
__device__ __forceinline__ unsigned long long gate_fixed(float g) {
  return __double2ull_rn((double)g * 4294967296.0);
}

// LDS of one ledger workgroup, carved from a byte array (8-byte sums first).
constexpr int kLedgerLdsBytes = kMaxExperts * (8 + 4 + 4) + kMaxRanks * kMaxRanks * 4 + LC_N * 4;

// Workgroup b of the ledger: RPB routes from b * RPB.  FINAL: write part b of
// the stage `fin` (of nparts parts; workgroup 0 writes the count) instead of
// the per-block partials.  `lds`: kLedgerLdsBytes, 8-byte aligned.
template <int RPB, bool FINAL>
__device__ __forceinline__ void ledger_block(
    int b, const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const int32_t* __restrict__ route_row, const int32_t* __restrict__ src,
    const int32_t* __restrict__ owner, int64_t A, int K, int E, int n_ep,
    int32_t* __restrict__ blk_load, uint64_t* __restrict__ blk_P,
    int64_t* __restrict__ blk_cnt, int32_t* __restrict__ blk_pair, char* __restrict__ fin,
    int nparts, char* lds) {
  constexpr int PER_THREAD = RPB / 256;
  unsigned long long* s_P = (unsigned long long*)lds;
  int* s_load = (int*)(lds + kMaxExperts * 8);
  int* s_owner = s_load + kMaxExperts;
  int* s_pair = s_owner + kMaxExperts;
  int* s_cnt = s_pair + kMaxRanks * kMaxRanks;
  const int tid = threadIdx.x;
  const int np = n_ep * n_ep;
  for (int e = tid; e < E; e += 256) {
    s_load[e] = 0;
    s_P[e] = 0ull;
    s_owner[e] = owner[e];
  }
  for (int j = tid; j < np; j += 256) s_pair[j] = 0;
  if (tid < LC_N) s_cnt[tid] = 0;

  const int64_t base = (int64_t)b * RPB;
  const int n = (int)min((int64_t)RPB, A - base);
  int c_lall = 0, c_call = 0, c_lacc = 0, c_cacc = 0, c_acc = 0, c_bad_id = 0, c_bad_rank = 0;
  // batches of U routes per thread; every global load of a batch is issued
  // before any of them is used.  The first batch's loads overlap the LDS
  // initialisation above; the barrier that publishes it follows them.
  constexpr int U = PER_THREAD < 8 ? PER_THREAD : 8;
  for (int u0 = 0; u0 < PER_THREAD; u0 += U) {
    if (u0 > 0 && u0 * 256 >= n) break;  // block-uniform
    int ids[U], rows[U], srcs[U];
    float gs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = (u0 + u) * 256 + tid;
      const int64_t i = base + (j < n ? j : 0);
      ids[u] = idx[i];
      gs[u] = gate[i];
      rows[u] = route_row[i];
      srcs[u] = src[i / K];
    }
    if (u0 == 0) __syncthreads();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = (u0 + u) * 256 + tid;
      if (j >= n) continue;
      const int id = ids[u];
      if (id < 0 || id >= E) {
        ++c_bad_id;
        continue;
      }
      atomicAdd(&s_load[id], 1);
      atomicAdd(&s_P[id], gate_fixed(gs[u]));
      const int row = rows[u];
      if (row >= 0) ++c_acc;
      const int sr = srcs[u];
      const int orank = s_owner[id];
      if (sr < 0 || sr >= n_ep || orank < 0 || orank >= n_ep) {
        ++c_bad_rank;
        continue;
      }
      const bool local = sr == orank;
      c_lall += local;
      c_call += !local;
      if (row >= 0) {
        c_lacc += local;
        c_cacc += !local;
        atomicAdd(&s_pair[sr * n_ep + orank], 1);
      }
    }
  }
  // wave sums of the scalar counters (DPP within rows, then the four rows),
  // then one LDS atomic per wave
  int vals[7] = {c_lall, c_call, c_lacc, c_cacc, c_acc, c_bad_id, c_bad_rank};
#pragma unroll
  for (int q = 0; q < 7; ++q) vals[q] = wave_sum(vals[q]);
  if ((tid & 63) == 0) {
    atomicAdd(&s_cnt[LC_LOCAL_ALL], vals[0]);
    atomicAdd(&s_cnt[LC_CROSS_ALL], vals[1]);
    atomicAdd(&s_cnt[LC_LOCAL_ACC], vals[2]);
    atomicAdd(&s_cnt[LC_CROSS_ACC], vals[3]);
    atomicAdd(&s_cnt[LC_ACCEPTED], vals[4]);
    atomicAdd(&s_cnt[LC_INVALID_ID], vals[5]);
    atomicAdd(&s_cnt[LC_INVALID_RANK], vals[6]);
  }
  __syncthreads();

  if (FINAL) {
    if (b == 0 && tid == 0) *(int64_t*)fin = nparts;
    const FinalArea f = final_area(fin + 8 + (size_t)b * ledger_final_bytes(E, n_ep), E);
    for (int e = tid; e < E; e += 256) {
      f.P[e] = s_P[e];
      f.load[e] = s_load[e];
    }
    for (int j = tid; j < np; j += 256) f.pair[j] = s_pair[j];
    if (tid < LC_N) f.cnt[tid] = s_cnt[tid];
    return;
  }
  for (int e = tid; e < E; e += 256) {
    blk_P[(size_t)b * E + e] = s_P[e];
    blk_load[(size_t)b * E + e] = s_load[e];
  }
  for (int j = tid; j < np; j += 256) blk_pair[(size_t)b * np + j] = s_pair[j];
  if (tid < LC_N) blk_cnt[(size_t)b * LC_N + tid] = s_cnt[tid];
}

template <int RPB, bool FINAL>
__global__ __launch_bounds__(256) void ledger_partial_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const int32_t* __restrict__ route_row, const int32_t* __restrict__ src,
    const int32_t* __restrict__ owner, int64_t A, int K, int E, int n_ep,
    int32_t* __restrict__ blk_load, uint64_t* __restrict__ blk_P,
    int64_t* __restrict__ blk_cnt, int32_t* __restrict__ blk_pair, char* __restrict__ fin) {
  __shared__ __attribute__((aligned(16))) char lds[kLedgerLdsBytes];
  ledger_block<RPB, FINAL>(blockIdx.x, idx, gate, route_row, src, owner, A, K, E, n_ep,
                           blk_load, blk_P, blk_cnt, blk_pair, fin, 1, lds);
}

// The combine and the ledger in one launch: blocks 0 .. nled-1 (dispatched
// first, and the longest) each count kLedgerPartRoutes routes into their own
// part of the stage, blocks nled.. are the combine's workgroups.  The two
// read the same routes and write disjoint outputs.
constexpr int kLedgerPartRoutes = kSmallLedgerRoutes / kLedgerStageParts;
template <bool VEC, int U, bool NT>
__global__ __launch_bounds__(256) void combine_ledger_kernel(
    const float* __restrict__ y, const int32_t* __restrict__ route_row,
    const float* __restrict__ gate, float* __restrict__ out, int T, int K, int h, int TB,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ src,
    const int32_t* __restrict__ owner, int E, int n_ep, int nled, char* __restrict__ fin) {
  constexpr int LDS = kLedgerLdsBytes > kCombineLdsBytes ? kLedgerLdsBytes : kCombineLdsBytes;
  __shared__ __attribute__((aligned(16))) char lds[LDS];
  if ((int)blockIdx.x < nled) {
    ledger_block<kLedgerPartRoutes, true>(blockIdx.x, idx, gate, route_row, src, owner,
                                          (int64_t)T * K, K, E, n_ep, nullptr, nullptr, nullptr,
                                          nullptr, fin, nled, lds);
    return;
  }
  combine_tokens<VEC, U, NT>(blockIdx.x - nled, y, route_row, gate, out, T, K, h, TB, (int*)lds,
                         (float*)(lds + kMaxTB * kMaxTopK * 4));
}

// final[q] = sum over blocks of the per-block partial q; one wave per q, its
// lanes take blocks lane, lane + 64, ... (integers: any order is exact)
__global__ __launch_bounds__(256) void ledger_reduce_kernel(
    int nb, int E, int n_ep, const int32_t* __restrict__ blk_load,
    const uint64_t* __restrict__ blk_P, const int64_t* __restrict__ blk_cnt,
    const int32_t* __restrict__ blk_pair, char* __restrict__ fin) {
  const int np = n_ep * n_ep;
  const int lane = threadIdx.x & 63;
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int items = 2 * E + LC_N + np;
  if (blockIdx.x == 0 && threadIdx.x == 0) *(int64_t*)fin = 1;  // one part
  if (q >= items) return;  // whole waves leave together
  const FinalArea fa = final_area(fin + 8, E);
  uint64_t s = 0;  // two's complement: signed partials add up the same way
  if (q < E) {
    for (int b = lane; b < nb; b += 64) s += (uint64_t)(int64_t)blk_load[(size_t)b * E + q];
  } else if (q < 2 * E) {
    for (int b = lane; b < nb; b += 64) s += blk_P[(size_t)b * E + (q - E)];
  } else if (q < 2 * E + LC_N) {
    for (int b = lane; b < nb; b += 64) s += (uint64_t)blk_cnt[(size_t)b * LC_N + (q - 2 * E)];
  } else {
    const int j = q - 2 * E - LC_N;
    for (int b = lane; b < nb; b += 64) s += (uint64_t)(int64_t)blk_pair[(size_t)b * np + j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)s, off, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(s >> 32), off, 64);
    s += ((uint64_t)hi << 32) | lo;
  }
  if (lane != 0) return;
  if (q < E) fa.load[q] = (int64_t)s;
  else if (q < 2 * E) fa.P[q - E] = s;
  else if (q < 2 * E + LC_N) fa.cnt[q - 2 * E] = (int64_t)s;
  else fa.pair[q - 2 * E - LC_N] = (int64_t)s;
}

}  // namespace

size_t ledger_ws_bytes(int64_t A, int E, int n_ep) { return carve(nullptr, A, E, n_ep).total; }

hipError_t launch_ledger(const int32_t* idx, const float* gate, const int32_t* route_row,
                         const int32_t* src, const int32_t* owner, int T, int K, int E,
                         int n_ep, void* ws, void* fin_dst, void** final_area_out,
                         size_t* final_bytes, hipStream_t s) {
  const int64_t A = (int64_t)T * K;
  LedgerWs w = carve(ws, A, E, n_ep);
  char* fin = fin_dst ? (char*)fin_dst : w.fin;
  *final_area_out = fin;
  *final_bytes = w.fin_bytes;
  if (A > 0 && A <= kSmallLedgerRoutes) {
    hipLaunchKernelGGL((ledger_partial_kernel<kSmallLedgerRoutes, true>), dim3(1), dim3(256), 0,
                       s, idx, gate, route_row, src, owner, A, K, E, n_ep, nullptr, nullptr,
                       nullptr, nullptr, fin);
    return hipGetLastError();
  }
  const int nb = A > 0 ? (int)((A + RPBL - 1) / RPBL) : 0;
  if (nb > 0) {
    hipLaunchKernelGGL((ledger_partial_kernel<RPBL, false>), dim3(nb), dim3(256), 0, s, idx,
                       gate, route_row, src, owner, A, K, E, n_ep, w.blk_load, w.blk_P,
                       w.blk_cnt, w.blk_pair, nullptr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int items = 2 * E + LC_N + n_ep * n_ep;
  hipLaunchKernelGGL(ledger_reduce_kernel, dim3((items + 3) / 4), dim3(256), 0, s, nb, E, n_ep,
                     w.blk_load, w.blk_P, w.blk_cnt, w.blk_pair, fin);
  return hipGetLastError();
}

hipError_t launch_combine_ledger(const float* y, const int32_t* route_row, const float* gate,
                                 float* out, const int32_t* idx, const int32_t* src,
                                 const int32_t* owner, int T, int K, int h, int E, int n_ep,
                                 void* ws, void* fin_dst, void** final_area_out,
                                 size_t* final_bytes, hipStream_t s) {
  const int64_t A = (int64_t)T * K;
  if (A == 0 || h == 0 || A > kSmallLedgerRoutes) {  // two launches
    hipError_t err = launch_combine(y, route_row, gate, out, T, K, h, s);
    if (err != hipSuccess) return err;
    return launch_ledger(idx, gate, route_row, src, owner, T, K, E, n_ep, ws, fin_dst,
                         final_area_out, final_bytes, s);
  }
  LedgerWs w = carve(ws, A, E, n_ep);
  char* fin = fin_dst ? (char*)fin_dst : w.fin;
  *final_area_out = fin;
  *final_bytes = w.fin_bytes;
  const CombineShape c = combine_shape(T, K, h);
  const int nled = (int)((A + kLedgerPartRoutes - 1) / kLedgerPartRoutes);
  with_combine_variant(c, [&](auto vec, auto u, auto nt) {
    hipLaunchKernelGGL((combine_ledger_kernel<decltype(vec)::value, decltype(u)::value,
                                              decltype(nt)::value>),
                       dim3(c.grid + nled), dim3(256), 0, s, y, route_row, gate, out, T, K, h,
                       c.TB, idx, src, owner, E, n_ep, nled, fin);
  });
  return hipGetLastError();
}

}  // namespace moe
