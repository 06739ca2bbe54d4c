// Locality-aware expert placement: the expert x source-rank affinity counts
// on the device, and the expert -> rank map that maximises the routes kept
// local, on the host.
//
// Method: "46. MoE Expert Parallel" Step 3 (a more local expert placement
// cuts cross-rank dispatch; watch whether the per-rank load gets skewed) and
// TODO 2 (a route is local iff its token's source rank owns its expert);
// "MoE大模型专家并行与动态路由优化" 2.2 (uniform placement of E / N experts per
// device; topology-aware placement matches experts to devices with the
// Hungarian algorithm on an affinity matrix).
//
// affinity[e][r] = routes to expert e from tokens of source rank r (all
// routes, or the accepted ones).  Placing e on r keeps affinity[e][r] routes
// local, so the best map with E / n_ep experts per rank is a linear
// assignment of the E experts to E slots (slot j on rank j / (E / n_ep)),
// solved exactly with the shortest-augmenting-path Hungarian method in
// integer arithmetic.
#include <cstring>
#include <vector>

#include "moe.h"
#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int kAffLds = 8192;  // counts kept in LDS per workgroup (32 KB)

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

// One workgroup per 4096 routes.  Counts go to an LDS histogram when the
// E x n_ep matrix fits, else straight to device memory; the integer sums do
// not depend on the order of the atomic adds.  Invalid ids or ranks are not
// counted (the ledger reports them).
template <bool LDS>
__global__ __launch_bounds__(256) void affinity_kernel(const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ route_row,
                                                       const int32_t* __restrict__ src,
                                                       int64_t A, int K, int E, int n_ep,
                                                       int32_t* __restrict__ counts) {
  __shared__ int32_t hist[LDS ? kAffLds : 1];
  const int n = E * n_ep;
  if (LDS) {
    for (int i = threadIdx.x; i < n; i += 256) hist[i] = 0;
    __syncthreads();
  }
  const int64_t base = (int64_t)blockIdx.x * 4096;
  for (int j = threadIdx.x; j < 4096; j += 256) {
    const int64_t i = base + j;
    if (i >= A) break;
    if (route_row && route_row[i] < 0) continue;
    const int e = idx[i];
    const int r = src[i / K];
    if (e < 0 || e >= E || r < 0 || r >= n_ep) continue;
    if (LDS) atomicAdd(&hist[e * n_ep + r], 1);
    else atomicAdd(&counts[e * n_ep + r], 1);
  }
  if (LDS) {
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += 256)
      if (hist[i]) atomicAdd(&counts[i], hist[i]);
  }
}

}  // namespace

hipError_t launch_affinity(const int32_t* idx, const int32_t* route_row, const int32_t* src,
                           int T, int K, int E, int n_ep, int32_t* counts, hipStream_t s) {
  const int n = E * n_ep;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024),
                     dim3(256), 0, s, counts, n);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t A = (int64_t)T * K;
  if (A == 0) return hipSuccess;
  const unsigned grid = (unsigned)((A + 4095) / 4096);
  if (n <= kAffLds)
    hipLaunchKernelGGL(affinity_kernel<true>, dim3(grid), dim3(256), 0, s, idx, route_row, src, A,
                       K, E, n_ep, counts);
  else
    hipLaunchKernelGGL(affinity_kernel<false>, dim3(grid), dim3(256), 0, s, idx, route_row, src,
                       A, K, E, n_ep, counts);
  return hipGetLastError();
}

// Minimum-cost perfect assignment of an n x n integer cost matrix (row i to
// column col[i]) by successive shortest augmenting paths with row and column
// potentials (the Hungarian method, O(n^3)).
static void assign_min_cost(const std::vector<int64_t>& cost, int n, std::vector<int>& col) {
  const int64_t INF = INT64_MAX / 4;
  std::vector<int64_t> u(n + 1, 0), v(n + 1, 0), minv(n + 1);
  std::vector<int> p(n + 1, 0), way(n + 1, 0);  // p[j]: row matched to column j (1-based)
  std::vector<char> used(n + 1);
  for (int i = 1; i <= n; ++i) {
    p[0] = i;
    int j0 = 0;
    std::fill(minv.begin(), minv.end(), INF);
    std::fill(used.begin(), used.end(), 0);
    do {
      used[j0] = 1;
      const int i0 = p[j0];
      int64_t delta = INF;
      int j1 = 0;
      for (int j = 1; j <= n; ++j) {
        if (used[j]) continue;
        const int64_t cur = cost[(size_t)(i0 - 1) * n + (j - 1)] - u[i0] - v[j];
        if (cur < minv[j]) {
          minv[j] = cur;
          way[j] = j0;
        }
        if (minv[j] < delta) {
          delta = minv[j];
          j1 = j;
        }
      }
      for (int j = 0; j <= n; ++j) {
        if (used[j]) {
          u[p[j]] += delta;
          v[j] -= delta;
        } else {
          minv[j] -= delta;
        }
      }
      j0 = j1;
    } while (p[j0] != 0);
    do {
      const int j1 = way[j0];
      p[j0] = p[j1];
      j0 = j1;
    } while (j0);
  }
  col.assign(n, -1);
  for (int j = 1; j <= n; ++j)
    if (p[j] > 0) col[p[j] - 1] = j - 1;
}

}  // namespace moe

extern "C" {

int moe_expert_rank_affinity(const moe_cfg* cfg, const int32_t* topk_idx,
                             const int32_t* route_row, const int32_t* src_rank, int32_t n_ep,
                             int32_t* affinity, void* stream) {
  if (!cfg || cfg->T < 0 || cfg->E <= 0 || cfg->K <= 0 || cfg->K > cfg->E)
    return MOE_ERR_INVALID_ARG;
  if (n_ep < 1 || n_ep > moe::kMaxRanks || cfg->E > moe::kMaxExperts) return MOE_ERR_INVALID_ARG;
  if (!affinity) return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!topk_idx || !src_rank)) return MOE_ERR_INVALID_ARG;
  if ((int64_t)cfg->T * cfg->K > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  return moe::launch_affinity(topk_idx, route_row, src_rank, cfg->T, cfg->K, cfg->E, n_ep,
                              affinity, (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}

int moe_place_experts(const int32_t* affinity, int32_t E, int32_t n_ep, int32_t* owner) {
  if (!affinity || !owner || E <= 0 || n_ep <= 0 || E % n_ep != 0) return MOE_ERR_INVALID_ARG;
  if (E > moe::kMaxExperts) return MOE_ERR_UNSUPPORTED;
  for (int64_t i = 0; i < (int64_t)E * n_ep; ++i)
    if (affinity[i] < 0) return MOE_ERR_INVALID_ARG;
  const int per = E / n_ep;
  // cost of expert e in slot j = -(routes kept local on slot j's rank)
  std::vector<int64_t> cost((size_t)E * E);
  for (int e = 0; e < E; ++e)
    for (int j = 0; j < E; ++j) cost[(size_t)e * E + j] = -(int64_t)affinity[(size_t)e * n_ep + j / per];
  std::vector<int> col;
  moe::assign_min_cost(cost, E, col);
  for (int e = 0; e < E; ++e) owner[e] = col[e] / per;
  return MOE_OK;
}

}  // extern "C"
