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
// Device part: one workgroup per 2048 routes builds integer histograms in LDS
// and per-expert gate sums in float64 with a fixed summation order; a second
// kernel adds the per-block partials in block order.  Integer counters are
// exact, and the float64 sums are deterministic run to run.  The host
// finishes the few scalar formulas in float64.
#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int RPBL = kLedgerRoutesPerBlock;
constexpr int PER_THREAD = RPBL / 256;

struct LedgerWs {
  int32_t* blk_load;   // [nb][E]
  double* blk_P;       // [nb][E]
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
  w.blk_P = (double*)(p + o);
  o = align_up(o + (size_t)nb * E * sizeof(double), 256);
  w.blk_cnt = (int64_t*)(p + o);
  o = align_up(o + (size_t)nb * LC_N * sizeof(int64_t), 256);
  w.blk_pair = (int32_t*)(p + o);
  o = align_up(o + (size_t)nb * n_ep * n_ep * sizeof(int32_t), 256);
  w.fin = p + o;
  w.fin_bytes = (size_t)(2 * E + LC_N + n_ep * n_ep) * 8;
  o = align_up(o + w.fin_bytes, 256);
  w.total = o;
  return w;
}

__global__ __launch_bounds__(256) void ledger_partial_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const int32_t* __restrict__ route_row, const int32_t* __restrict__ src,
    const int32_t* __restrict__ owner, int64_t A, int K, int E, int n_ep,
    int32_t* __restrict__ blk_load, double* __restrict__ blk_P, int64_t* __restrict__ blk_cnt,
    int32_t* __restrict__ blk_pair) {
  __shared__ int s_load[kMaxExperts];
  __shared__ int s_pair[kMaxRanks * kMaxRanks];
  __shared__ int s_idx[RPBL];
  __shared__ float s_gate[RPBL];
  __shared__ double s_part[kMaxExperts];
  __shared__ int s_cnt[LC_N];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int np = n_ep * n_ep;
  for (int e = tid; e < E; e += 256) s_load[e] = 0;
  for (int j = tid; j < np; j += 256) s_pair[j] = 0;
  if (tid < LC_N) s_cnt[tid] = 0;
  __syncthreads();

  const int64_t base = (int64_t)b * RPBL;
  const int n = (int)min((int64_t)RPBL, A - base);
  int c_lall = 0, c_call = 0, c_lacc = 0, c_cacc = 0, c_acc = 0, c_bad_id = 0, c_bad_rank = 0;
#pragma unroll
  for (int u = 0; u < PER_THREAD; ++u) {
    const int j = u * 256 + tid;
    if (j >= n) continue;
    const int64_t i = base + j;
    const int id = idx[i];
    const bool valid = id >= 0 && id < E;
    s_idx[j] = valid ? id : -1;
    s_gate[j] = gate[i];
    if (!valid) {
      ++c_bad_id;
      continue;
    }
    atomicAdd(&s_load[id], 1);
    const int row = route_row[i];
    if (row >= 0) ++c_acc;
    const int sr = src[i / K];
    const int orank = owner[id];
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
  // wave sums of the scalar counters, then one LDS atomic per wave
  int vals[7] = {c_lall, c_call, c_lacc, c_cacc, c_acc, c_bad_id, c_bad_rank};
#pragma unroll
  for (int q = 0; q < 7; ++q) {
    int v = vals[q];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    vals[q] = v;
  }
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

  // per-expert gate sums, fixed order: S threads per expert, thread `sl`
  // takes routes sl, sl+S, ...; the S partials are then added in sl order
  const int S = (E >= 256) ? 1 : (256 / E);
  for (int w = tid; w < E * S; w += 256) {
    const int e = w % E, sl = w / E;
    double sum = 0.0;
    for (int j = sl; j < n; j += S)
      if (s_idx[j] == e) sum += (double)s_gate[j];
    s_part[w] = sum;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    double sum = 0.0;
    for (int sl = 0; sl < S; ++sl) sum += s_part[sl * E + e];
    blk_P[(size_t)b * E + e] = sum;
    blk_load[(size_t)b * E + e] = s_load[e];
  }
  for (int j = tid; j < np; j += 256) blk_pair[(size_t)b * np + j] = s_pair[j];
  if (tid < LC_N) blk_cnt[(size_t)b * LC_N + tid] = s_cnt[tid];
}

// final[q] = sum over blocks (in block order) of the per-block partial q
__global__ __launch_bounds__(256) void ledger_reduce_kernel(
    int nb, int E, int n_ep, const int32_t* __restrict__ blk_load,
    const double* __restrict__ blk_P, const int64_t* __restrict__ blk_cnt,
    const int32_t* __restrict__ blk_pair, char* __restrict__ fin) {
  const int np = n_ep * n_ep;
  const int q = blockIdx.x * 256 + threadIdx.x;
  int64_t* f_load = (int64_t*)fin;
  double* f_P = (double*)(fin + (size_t)E * 8);
  int64_t* f_cnt = (int64_t*)(fin + (size_t)2 * E * 8);
  int64_t* f_pair = (int64_t*)(fin + (size_t)(2 * E + LC_N) * 8);
  if (q < E) {
    int64_t s = 0;
    for (int b = 0; b < nb; ++b) s += blk_load[(size_t)b * E + q];
    f_load[q] = s;
  } else if (q < 2 * E) {
    const int e = q - E;
    double s = 0.0;
    for (int b = 0; b < nb; ++b) s += blk_P[(size_t)b * E + e];
    f_P[e] = s;
  } else if (q < 2 * E + LC_N) {
    const int c = q - 2 * E;
    int64_t s = 0;
    for (int b = 0; b < nb; ++b) s += blk_cnt[(size_t)b * LC_N + c];
    f_cnt[c] = s;
  } else if (q < 2 * E + LC_N + np) {
    const int j = q - 2 * E - LC_N;
    int64_t s = 0;
    for (int b = 0; b < nb; ++b) s += blk_pair[(size_t)b * np + j];
    f_pair[j] = s;
  }
}

}  // namespace

size_t ledger_ws_bytes(int64_t A, int E, int n_ep) { return carve(nullptr, A, E, n_ep).total; }

hipError_t launch_ledger(const int32_t* idx, const float* gate, const int32_t* route_row,
                         const int32_t* src, const int32_t* owner, int T, int K, int E,
                         int n_ep, void* ws, void** final_area, size_t* final_bytes,
                         hipStream_t s) {
  const int64_t A = (int64_t)T * K;
  LedgerWs w = carve(ws, A, E, n_ep);
  const int nb = A > 0 ? (int)((A + RPBL - 1) / RPBL) : 0;
  if (nb > 0) {
    hipLaunchKernelGGL(ledger_partial_kernel, dim3(nb), dim3(256), 0, s, idx, gate, route_row,
                       src, owner, A, K, E, n_ep, w.blk_load, w.blk_P, w.blk_cnt, w.blk_pair);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const int items = 2 * E + LC_N + n_ep * n_ep;
  hipLaunchKernelGGL(ledger_reduce_kernel, dim3((items + 255) / 256), dim3(256), 0, s, nb, E,
                     n_ep, w.blk_load, w.blk_P, w.blk_cnt, w.blk_pair, w.fin);
  *final_area = w.fin;
  *final_bytes = w.fin_bytes;
  return hipGetLastError();
}

}  // namespace moe
