// Capacity-limited dispatch: expert histogram, per-expert offsets, each
// route's rank within its expert, the capacity drop, and the gather of the
// accepted token rows into contiguous per-expert segments.
//
// Method: "MoE大模型专家并行与动态路由优化" 3.3 (capacity loop: routes in
// (token, k-slot) order, accept while the expert holds fewer than `capacity`)
// with capacity = ceil((A/E) * capacity_factor) from "47. MoE Expert Parallel"
// Step 3; dispatch = moving each accepted token to its expert
// ("专家并行（Expert Parallelism）", Dispatch).
//
// The sequential loop is a stable counting sort by expert: a route's rank is
// the number of earlier routes (row-major over [T, K]) with the same expert.
//   count kernel  : LDS histogram of each 1024-route block  -> counts[b][E+1]
//   slot kernel   : prefix over earlier blocks + in-block wave multisplit
//                   (ballots on the id bits) -> rank, row, row_token, offsets
//   gather kernel : x_disp[row] = x[row_token[row]] with 16-byte vectors
// Up to kSmallDispatchRoutes routes (16-byte-vector rows) all three run as one
// launch: every block histograms all A routes itself (the expert totals and
// the counts before its own 16 routes), so no block waits on another.
#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int RPB = kDispatchRoutesPerBlock;  // routes per block
constexpr int CHUNK = 256;                    // routes per pass (one per thread)
constexpr int NPASS = RPB / CHUNK;            // passes of the slot kernel
constexpr int COL_LOADS = 32;                 // count-matrix loads in flight per thread

__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ idx,
                                                    int64_t A, int E,
                                                    int32_t* __restrict__ counts) {
  __shared__ int hist[kMaxExperts + 1];
  const int tid = threadIdx.x;
  for (int e = tid; e <= E; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * RPB;
  // all of this thread's ids are loaded before the first is counted (a load
  // under the bounds check, counted at once, would cost a round trip each)
  int ids[NPASS];
#pragma unroll
  for (int j = 0; j < NPASS; ++j) ids[j] = idx[min(base + j * 256 + tid, A - 1)];
#pragma unroll
  for (int j = 0; j < NPASS; ++j) {
    if (base + j * 256 + tid < A) {
      const int id = ids[j];
      const int bin = (id >= 0 && id < E) ? id : E;  // bin E: invalid ids
      atomicAdd(&hist[bin], 1);
    }
  }
  __syncthreads();
  int32_t* out = counts + (size_t)blockIdx.x * (E + 1);
  for (int e = tid; e <= E; e += 256) out[e] = hist[e];
}

__device__ __forceinline__ int block_exclusive_scan(int v, int* sh_wave, int tid) {
  // 256 threads = 4 waves
  const int lane = tid & 63, wave = tid >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) sh_wave[wave] = incl;
  __syncthreads();
  int prefix = 0;
  for (int w = 0; w < wave; ++w) prefix += sh_wave[w];
  __syncthreads();
  return prefix + incl - v;
}

// Exclusive scan over experts of min(tot[e], cap) into off[0..E] (off[E] =
// R); E <= kMaxExperts = 4 * 256.
__device__ __forceinline__ void accepted_offsets(const int* tot, int* off, int E, int64_t cap,
                                                 int* sh_wave, int tid) {
  const int per_thread = (E + 255) / 256;
  int accv[4];
  int my_acc = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * per_thread + j;
    accv[j] = (j < per_thread && e < E) ? (int)min((int64_t)tot[e], cap) : 0;
    my_acc += accv[j];
  }
  int excl = block_exclusive_scan(my_acc, sh_wave, tid);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * per_thread + j;
    if (j < per_thread && e < E) {
      off[e] = excl;
      excl += accv[j];
    }
  }
  if (tid == 255) off[E] = excl;
  __syncthreads();
}

__global__ __launch_bounds__(256) void slot_kernel(
    const int32_t* __restrict__ idx, int64_t A, int K, int E, int64_t cap, int nblocks,
    const int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ route_rank, int32_t* __restrict__ route_row,
    int32_t* __restrict__ row_token, int32_t* __restrict__ load_out) {
  __shared__ int run[kMaxExperts];       // next rank per expert for this block
  __shared__ int off[kMaxExperts + 1];   // exclusive prefix of accepted counts
  __shared__ int wcnt[4][kMaxExperts];   // per-wave counts of the current pass
  __shared__ int ptot[kMaxExperts];     // partial column sums (S slices)
  __shared__ int pbef[kMaxExperts];
  __shared__ int sh_wave[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const int64_t base = (int64_t)b * RPB;
  // this block's expert ids, loaded first so that they arrive during step 1
  int ids[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int64_t i = base + p * CHUNK + tid;
    ids[p] = i < A ? idx[i] : -1;
  }

  // 1. per expert: routes in earlier blocks (-> run) and in all blocks (load)
  //    -> accepted = min(load, cap) -> exclusive scan over experts (-> off).
  //    S threads share one expert's column of the count matrix.  The counts
  //    were written by other XCDs, so each round trip is a full memory
  //    latency: up to 32 loads per thread are issued before their sums.
  const int S = (E >= 256) ? 1 : (256 / E);
  for (int w = tid; w < E * S; w += 256) {
    const int e = w % E, sl = w / E;
    int bef = 0, tot = 0;
    for (int bb0 = sl; bb0 < nblocks; bb0 += COL_LOADS * S) {
      int c[COL_LOADS];
#pragma unroll
      for (int u = 0; u < COL_LOADS; ++u) {
        const int bb = bb0 + u * S;
        c[u] = bb < nblocks ? counts[(size_t)bb * (E + 1) + e] : 0;
      }
#pragma unroll
      for (int u = 0; u < COL_LOADS; ++u) {
        tot += c[u];
        bef += (bb0 + u * S < b) ? c[u] : 0;
      }
    }
    ptot[w] = tot;
    pbef[w] = bef;
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    int bef = 0, tot = 0;
    for (int sl = 0; sl < S; ++sl) {
      tot += ptot[sl * E + e];
      bef += pbef[sl * E + e];
    }
    run[e] = bef;
    ptot[e] = tot;  // each e is read and written by this thread only
    if (b == 0 && load_out) load_out[e] = tot;
  }
  __syncthreads();
  accepted_offsets(ptot, off, E, cap, sh_wave, tid);
  if (b == 0)
    for (int e = tid; e <= E; e += 256) offsets[e] = off[e];

  // 2. ranks of this block's routes, 256 at a time
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int64_t i = base + p * CHUNK + tid;
    const int id = ids[p];
    const bool valid = (i < A) && id >= 0 && id < E;
    for (int e = tid; e < 4 * E; e += 256) (&wcnt[0][0])[e / E * kMaxExperts + e % E] = 0;
    __syncthreads();
    // lanes of this wave holding the same expert id
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = valid && ((id >> bit) & 1);
      const uint64_t bm = __ballot(on);
      m &= on ? bm : ~bm;
    }
    const int below = __popcll(m & lt_mask);
    if (valid && below == 0) wcnt[wave][id] = __popcll(m);
    __syncthreads();
    int rank = -1;
    if (valid) {
      int prefix = run[id];
      for (int w = 0; w < wave; ++w) prefix += wcnt[w][id];
      rank = prefix + below;
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) run[e] += wcnt[0][e] + wcnt[1][e] + wcnt[2][e] + wcnt[3][e];
    if (i < A) {
      route_rank[i] = rank;
      int row = -1;
      if (valid && (int64_t)rank < cap) {
        row = off[id] + rank;
        row_token[row] = (int)(i / K);
      }
      route_row[i] = row;
    }
    __syncthreads();
  }
}

// Copy NR token rows: xd[dst[r]] = x[src[r]] for r < NR with dst[r] >= 0
// (row indices, in LDS; every src[r] is a valid token, also where dst[r] < 0).
// The NR * row_vecs 16-byte vectors are spread over the 256 threads; each
// thread issues U loads before their stores.  The loads are unconditional
// (positions past the last vector re-read it, rows without a destination
// read their source row and are not stored): loads under a per-lane
// condition had the compiler wait for each before it issued the next, one
// memory round trip per vector.  With a scale (FP8 payload) each 16-byte
// vector of eight bf16 becomes eight E4M3 codes (8 bytes) of the
// destination row.
// NT: nontemporal stores of the dispatched rows (chosen when they outgrow the
// 256 MB last-level cache, which could not keep them for the expert GEMM).
template <int NR, int U, bool NT = false>
__device__ __forceinline__ void copy_rows(const u32x4* __restrict__ x, void* __restrict__ xd,
                                          const int* dst, const int* src, int row_vecs,
                                          const float* __restrict__ q_scale) {
  const int nv = NR * row_vecs;
  const float scale = q_scale ? *q_scale : 0.0f;
  const float rscale = scale != 0.0f ? __fdiv_rn(1.0f, scale) : 0.0f;
  for (int j0 = threadIdx.x; j0 < nv; j0 += 256 * U) {
    u32x4 v[U];
    int64_t to[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = min(j0 + u * 256, nv - 1);
      const int r = j / row_vecs;
      const int c = j - r * row_vecs;
      v[u] = x[(int64_t)src[r] * row_vecs + c];
      to[u] = (j0 + u * 256 < nv && dst[r] >= 0) ? (int64_t)dst[r] * row_vecs + c : -1;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (to[u] < 0) continue;
      if (q_scale) ((uint2*)xd)[to[u]] = quantize8(v[u], scale, rscale);
      else if (NT) __builtin_nontemporal_store(v[u], &((u32x4*)xd)[to[u]]);
      else ((u32x4*)xd)[to[u]] = v[u];
    }
  }
}

// x_disp[row] = x[row_token[row]] for row < R = offsets[E]; rows are
// row_vecs 16-byte vectors long.  Each workgroup moves ROWS rows.
template <int ROWS, bool NT>
__global__ __launch_bounds__(256) void gather_kernel(const u32x4* __restrict__ x,
                                                     const int32_t* __restrict__ row_token,
                                                     const int32_t* __restrict__ offsets,
                                                     int E, int row_vecs,
                                                     void* __restrict__ xd,
                                                     const float* __restrict__ q_scale) {
  __shared__ int dst[ROWS], src[ROWS];
  const int R = offsets[E];
  const int r0 = blockIdx.x * ROWS;
  if (r0 >= R) return;
  if (threadIdx.x < ROWS) {
    const int r = r0 + threadIdx.x;
    dst[threadIdx.x] = r < R ? r : -1;
    src[threadIdx.x] = r < R ? row_token[r] : 0;
  }
  __syncthreads();
  copy_rows<ROWS, 8, NT>(x, xd, dst, src, row_vecs, q_scale);
}

// The whole dispatch for A <= kSmallDispatchRoutes in one launch; block b
// owns routes [16b, 16b + 16).
constexpr int SBR = 16;
constexpr int SBL = 8;  // route ids loaded per thread at once
__global__ __launch_bounds__(256) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, int A, int K, int E, int64_t cap,
    const u32x4* __restrict__ x, int row_vecs, int32_t* __restrict__ offsets,
    int32_t* __restrict__ route_rank, int32_t* __restrict__ route_row,
    int32_t* __restrict__ row_token, int32_t* __restrict__ load_out, void* __restrict__ xd,
    const float* __restrict__ q_scale) {
  __shared__ int tot[kMaxExperts], bef[kMaxExperts], off[kMaxExperts + 1];
  __shared__ int sh_wave[4];
  __shared__ int dst[SBR], src[SBR], own_id[SBR];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = blockIdx.x * SBR;
  for (int e = tid; e < E; e += 256) tot[e] = bef[e] = 0;
  __syncthreads();
  // all routes: totals, and the routes before this block (the stable order).
  // SBL loads per thread in flight; lanes of a wave with the same expert
  // are found with ballots on the id bits, and one of them adds their count.
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int i0 = 0; i0 < A; i0 += 256 * SBL) {
    int ids[SBL];
#pragma unroll
    for (int u = 0; u < SBL; ++u) {
      const int i = i0 + u * 256 + tid;
      ids[u] = i < A ? idx[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < SBL; ++u) {
      const int i = i0 + u * 256 + tid;
      const int id = ids[u];
      if (i >= base && i < base + SBR) own_id[i - base] = id;  // this block's routes
      const bool valid = id >= 0 && id < E;
      uint64_t m = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool on = valid && ((id >> bit) & 1);
        const uint64_t bm = __ballot(on);
        m &= on ? bm : ~bm;
      }
      const uint64_t before = __ballot(i < base);
      if (valid && (m & lt_mask) == 0) {
        atomicAdd(&tot[id], __popcll(m));
        const int nb = __popcll(m & before);
        if (nb) atomicAdd(&bef[id], nb);
      }
    }
  }
  __syncthreads();
  accepted_offsets(tot, off, E, cap, sh_wave, tid);
  if (blockIdx.x == 0) {
    for (int e = tid; e <= E; e += 256) offsets[e] = off[e];
    if (load_out)
      for (int e = tid; e < E; e += 256) load_out[e] = tot[e];
  }
  if (wave == 0) {
    // rank = routes before the block + lanes below with the same expert
    const int i = base + lane;
    int id = -1;
    if (lane < SBR && i < A) id = own_id[lane];  // kept by the histogram pass
    const bool valid = lane < SBR && i < A && id >= 0 && id < E;
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = valid && ((id >> bit) & 1);
      const uint64_t bm = __ballot(on);
      m &= on ? bm : ~bm;
    }
    const int rank = valid ? bef[id] + __popcll(m & lt_mask) : -1;
    int row = -1;
    if (valid && (int64_t)rank < cap) {
      row = off[id] + rank;
      row_token[row] = i / K;
    }
    if (lane < SBR && i < A) {
      route_rank[i] = rank;
      route_row[i] = row;
    }
    if (lane < SBR) {
      dst[lane] = row;
      src[lane] = i < A ? i / K : 0;  // a valid token also past the last route
    }
  }
  if (!xd) return;  // routing metadata only (uniform)
  __syncthreads();
  copy_rows<SBR, 8>(x, xd, dst, src, row_vecs, q_scale);
}

// the same gather for rows that are not a whole number of 16-byte vectors
__global__ __launch_bounds__(256) void gather_bytes_kernel(const uint8_t* __restrict__ x,
                                                           const int32_t* __restrict__ row_token,
                                                           const int32_t* __restrict__ offsets,
                                                           int E, int64_t row_bytes,
                                                           uint8_t* __restrict__ xd) {
  const int R = offsets[E];
  const int64_t row = blockIdx.x;
  if (row >= R) return;
  const int t = row_token[row];
  for (int64_t c = threadIdx.x; c < row_bytes; c += 256)
    xd[row * row_bytes + c] = x[(int64_t)t * row_bytes + c];
}

}  // namespace

size_t dispatch_ws_bytes(int64_t A, int E) {
  const int64_t nb = (A + RPB - 1) / RPB;
  return align_up((size_t)(nb > 0 ? nb : 1) * (size_t)(E + 1) * sizeof(int32_t), 256);
}

static hipError_t gather_rows(const void* x, const int32_t* row_token, const int32_t* offsets,
                              int E, int64_t row_bytes, int64_t r_max, void* dst, hipStream_t s,
                              const float* q_scale) {
  if (r_max == 0) return hipSuccess;
  const bool vec = row_bytes % 16 == 0 && ((uintptr_t)x & 15u) == 0 &&
                   ((uintptr_t)dst & 15u) == 0;
  if (q_scale && !vec) return hipErrorInvalidValue;
  if (vec) {
    constexpr int ROWS = 16;
    const int64_t grid = (r_max + ROWS - 1) / ROWS;
    if (r_max * row_bytes > ((int64_t)256 << 20))
      hipLaunchKernelGGL((gather_kernel<ROWS, true>), dim3((unsigned)grid), dim3(256), 0, s,
                         (const u32x4*)x, row_token, offsets, E, (int)(row_bytes / 16), dst,
                         q_scale);
    else
      hipLaunchKernelGGL((gather_kernel<ROWS, false>), dim3((unsigned)grid), dim3(256), 0, s,
                         (const u32x4*)x, row_token, offsets, E, (int)(row_bytes / 16), dst,
                         q_scale);
  } else {
    hipLaunchKernelGGL(gather_bytes_kernel, dim3((unsigned)r_max), dim3(256), 0, s,
                       (const uint8_t*)x, row_token, offsets, E, row_bytes, (uint8_t*)dst);
  }
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* row_token, const int32_t* offsets,
                              int E, int64_t row_bytes, int64_t r_max, void* dst,
                              hipStream_t s) {
  return gather_rows(x, row_token, offsets, E, row_bytes, r_max, dst, s, nullptr);
}

hipError_t launch_dispatch(const void* x, const int32_t* topk_idx, int64_t A, int K, int E,
                           int64_t cap, int64_t row_bytes, int64_t r_max,
                           int32_t* offsets, int32_t* route_rank, int32_t* route_row,
                           int32_t* row_token, void* x_disp, int32_t* load, void* ws,
                           hipStream_t s, const float* q_scale) {
  const bool vec = row_bytes % 16 == 0 && ((uintptr_t)x & 15u) == 0 &&
                   ((uintptr_t)x_disp & 15u) == 0;
  if (q_scale && !vec) return hipErrorInvalidValue;  // the FP8 path needs vector rows
  if (A > 0 && A <= kSmallDispatchRoutes && r_max > 0 && vec) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3((unsigned)((A + SBR - 1) / SBR)), dim3(256),
                       0, s, topk_idx, (int)A, K, E, cap, (const u32x4*)x,
                       (int)(row_bytes / 16), offsets, route_rank, route_row, row_token, load,
                       x_disp, q_scale);
    return hipGetLastError();
  }
  const int nb = (int)((A + RPB - 1) / RPB);
  int32_t* counts = (int32_t*)ws;
  if (nb > 0) {
    hipLaunchKernelGGL(count_kernel, dim3(nb), dim3(256), 0, s, topk_idx, A, E, counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // at least one block so that the offsets (all zero) are written
  hipLaunchKernelGGL(slot_kernel, dim3(nb > 0 ? nb : 1), dim3(256), 0, s, topk_idx, A, K, E,
                     cap, nb, counts, offsets, route_rank, route_row, row_token, load);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || r_max == 0 || !x_disp) return err;
  return gather_rows(x, row_token, offsets, E, row_bytes, r_max, x_disp, s, q_scale);
}

}  // namespace moe
