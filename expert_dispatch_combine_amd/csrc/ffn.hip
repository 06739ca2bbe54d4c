// Expert FFN over ragged expert segments: a grouped GEMM on bf16 MFMA.
//
// Method: "MoE大模型专家并行与动态路由优化" section 一, FFN(x) = W2 sigma(W1 x + b1)
// + b2 per expert, sigma = GELU (tanh form).  Each expert e owns the rows
// [offsets[e], offsets[e+1]) of the dispatched buffer:
//   GEMM1: H[r, n] = GELU(sum_k x_disp[r, k] W1[e, n, k] + b1[e, n])  -> bf16
//   GEMM2: Y[r, n] = sum_k H[r, k] W2[e, n, k] + b2[e, n]             -> fp32
// Both products read the activation rows and the weight rows along the
// contiguous reduction dimension ("NT" layout), so both operands stream as
// 16-byte vectors.
//
// Kernel shape (gfx950): 256 threads = 4 waves in a 2 x 2 grid, tile
// BM = 128 rows x BN (128 or 64) weight rows, BK = 64, double-buffered LDS
// (rows padded by 16 bytes), v_mfma_f32_32x32x16_bf16 with the WEIGHT tile as
// the MFMA A operand and the activation tile as the B operand, so each
// accumulator lane holds one activation row and 4 consecutive output columns
// (8-byte bf16 / 16-byte fp32 stores in the epilogue).
//
// Scheduling is on the device (no host sync): every workgroup derives the
// per-expert tile counts from `offsets`, maps its id to a logical tile with an
// XCD-aware permutation (consecutive logical tiles run on the same XCD, so
// they share its L2), and exits if it has none.  Logical tiles are ordered per
// expert, then in groups of 8 weight tiles, then row tiles fastest, so tiles
// that run together share their weight and activation panels.
#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int BM = 128;
constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row (16-byte pad)
constexpr int NGROUP = 8;           // weight tiles per scheduling group
constexpr int NXCD = 8;             // XCDs of an MI355X

__device__ __forceinline__ float gelu_tanh_f(float u) {
  // 0.5 u (1 + tanh(z)) == u * sigmoid(2 z),  z = sqrt(2/pi) (u + 0.044715 u^3)
  const float z = 0.7978845608028654f * (u + 0.044715f * u * u * u);
  return u / (1.0f + __expf(-2.0f * z));
}

struct TileInfo {
  int e, row0, row_end, n0;
};

// Find this workgroup's tile.  Returns false if it has none.
template <int BN>
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int E, int N,
                                          TileInfo* sh, int tid) {
  const int ntn = N / BN;
  if (tid < 64) {
    const int lane = tid;
    const int per = (E + 63) / 64;
    const int ebeg = min(E, lane * per), eend = min(E, ebeg + per);
    int mine = 0;
    for (int e = ebeg; e < eend; ++e) {
      const int rows = offsets[e + 1] - offsets[e];
      mine += (rows + BM - 1) / BM * ntn;
    }
    int incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    const int total = __shfl(incl, 63, 64);
    const int per_xcd = (total + NXCD - 1) / NXCD;
    const int bid = blockIdx.x;
    int L = -1;
    if (bid < per_xcd * NXCD) L = (bid % NXCD) * per_xcd + bid / NXCD;
    if (L >= total) L = -1;
    if (lane == 0) sh->e = -1;
    if (L >= 0) {
      int p = incl - mine;
      for (int e = ebeg; e < eend; ++e) {
        const int o0 = offsets[e], o1 = offsets[e + 1];
        const int nmt = (o1 - o0 + BM - 1) / BM;
        const int t = nmt * ntn;
        if (L >= p && L < p + t) {
          const int r = L - p;
          const int ng = r / (nmt * NGROUP);
          const int within = r - ng * nmt * NGROUP;
          const int mt = within % nmt;
          const int nt = ng * NGROUP + within / nmt;
          sh->e = e;
          sh->row0 = o0 + mt * BM;
          sh->row_end = o1;
          sh->n0 = nt * BN;
        }
        p += t;
      }
    }
  }
  __syncthreads();
  return sh->e >= 0;
}

// EPI 0: out = bf16(GELU(acc + bias)),  EPI 1: out = fp32(acc + bias)
template <int BN, int EPI>
__global__ __launch_bounds__(256, 2) void grouped_gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
    const float* __restrict__ bias, void* __restrict__ out,
    const int32_t* __restrict__ offsets, int E, int N, int Kd) {
  constexpr int TM = 2;        // 32-row MFMA tiles per wave (wave covers 64 rows)
  constexpr int TN = BN / 64;  // 32-col MFMA tiles per wave (wave covers BN/2 cols)
  constexpr int ACH = BM * BK / 8 / 256;  // 16-byte chunks per thread per stage (A)
  constexpr int WCH = BN * BK / 8 / 256;  // (W)
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][BN * LDS_STRIDE];
  __shared__ TileInfo tinfo;

  const int tid = threadIdx.x;
  if (!find_tile<BN>(offsets, E, N, &tinfo, tid)) return;
  const int e = tinfo.e, row0 = tinfo.row0, row_end = tinfo.row_end, n0 = tinfo.n0;

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // global source pointers of this thread's staging chunks (k offset added per stage)
  const uint16_t* a_src[ACH];
  int a_lds[ACH];
#pragma unroll
  for (int j = 0; j < ACH; ++j) {
    const int c = tid + j * 256;
    const int r = c >> 3, cc = c & 7;
    const int row = min(row0 + r, row_end - 1);
    a_src[j] = A + (size_t)row * Kd + cc * 8;
    a_lds[j] = r * LDS_STRIDE + cc * 8;
  }
  const uint16_t* w_src[WCH];
  int w_lds[WCH];
  const uint16_t* wbase = W + ((size_t)e * N + n0) * Kd;
#pragma unroll
  for (int j = 0; j < WCH; ++j) {
    const int c = tid + j * 256;
    const int r = c >> 3, cc = c & 7;
    w_src[j] = wbase + (size_t)r * Kd + cc * 8;
    w_lds[j] = r * LDS_STRIDE + cc * 8;
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment offsets inside a stage
  const int kq = (lane >> 5) * 8;
  int a_frag[TM], w_frag[TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) a_frag[tm] = (wm * 64 + tm * 32 + (lane & 31)) * LDS_STRIDE + kq;
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
    w_frag[tn] = (wn * (BN / 2) + tn * 32 + (lane & 31)) * LDS_STRIDE + kq;

  const int nk = Kd / BK;
  u32x4 a_reg[ACH], w_reg[WCH];
#define MOE_GLOAD(k0)                                                              \
  do {                                                                             \
    _Pragma("unroll") for (int j = 0; j < ACH; ++j) a_reg[j] =                     \
        *(const u32x4*)(a_src[j] + (k0));                                          \
    _Pragma("unroll") for (int j = 0; j < WCH; ++j) w_reg[j] =                     \
        *(const u32x4*)(w_src[j] + (k0));                                          \
  } while (0)
#define MOE_LSTORE(buf)                                                            \
  do {                                                                             \
    _Pragma("unroll") for (int j = 0; j < ACH; ++j)                                \
        *(u32x4*)(&As[(buf)][a_lds[j]]) = a_reg[j];                                \
    _Pragma("unroll") for (int j = 0; j < WCH; ++j)                                \
        *(u32x4*)(&Ws[(buf)][w_lds[j]]) = w_reg[j];                                \
  } while (0)
  MOE_GLOAD(0);
  MOE_LSTORE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) MOE_GLOAD((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 wf[TN], af[TM];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        wf[tn] = *(const bf16x8*)(&Ws[buf][w_frag[tn] + kk * 16]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        af[tm] = *(const bf16x8*)(&As[buf][a_frag[tm] + kk * 16]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[tn], af[tm], acc[tm][tn],
                                                                0, 0, 0);
    }
    if (more) MOE_LSTORE(buf ^ 1);
    __syncthreads();
  }
#undef MOE_GLOAD
#undef MOE_LSTORE

  // epilogue: lane holds row (lane % 32) of each 32-row tile and, for
  // g = 0..3, columns 8g + 4*(lane/32) + 0..3 of each 32-col tile
  const float* bptr = bias + (size_t)e * N;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int m = row0 + wm * 64 + tm * 32 + (lane & 31);
    if (m >= row_end) continue;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * (BN / 2) + tn * 32 + g * 8 + (lane >> 5) * 4;
        const float4 b = *(const float4*)(bptr + n);
        float v0 = acc[tm][tn][4 * g + 0] + b.x;
        float v1 = acc[tm][tn][4 * g + 1] + b.y;
        float v2 = acc[tm][tn][4 * g + 2] + b.z;
        float v3 = acc[tm][tn][4 * g + 3] + b.w;
        if (EPI == 0) {
          v0 = gelu_tanh_f(v0);
          v1 = gelu_tanh_f(v1);
          v2 = gelu_tanh_f(v2);
          v3 = gelu_tanh_f(v3);
          uint2 pk;
          pk.x = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
          pk.y = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
          *(uint2*)((uint16_t*)out + (size_t)m * N + n) = pk;
        } else {
          *(float4*)((float*)out + (size_t)m * N + n) = make_float4(v0, v1, v2, v3);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- fp32 path
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int E,
                                             int row) {
  int lo = 0, hi = E;  // offsets[lo] <= row < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= row) lo = mid;
    else hi = mid;
  }
  return lo;
}

template <int EPI>
__global__ __launch_bounds__(256) void ffn_f32_kernel(const float* __restrict__ A,
                                                      const float* __restrict__ W,
                                                      const float* __restrict__ bias,
                                                      float* __restrict__ out,
                                                      const int32_t* __restrict__ offsets,
                                                      int E, int N, int Kd, int64_t r_max) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= r_max * N) return;
  const int row = (int)(i / N), n = (int)(i % N);
  if (row >= offsets[E]) return;
  const int e = expert_of_row(offsets, E, row);
  const float* a = A + (size_t)row * Kd;
  const float* w = W + ((size_t)e * N + n) * Kd;
  float acc = 0.f;
  for (int k = 0; k < Kd; ++k) acc = fmaf(a[k], w[k], acc);
  acc += bias[(size_t)e * N + n];
  out[(size_t)row * N + n] = (EPI == 0) ? gelu_tanh_f(acc) : acc;
}

template <int BN, int EPI>
hipError_t launch_gemm(const uint16_t* A, const uint16_t* W, const float* bias, void* out,
                       const int32_t* offsets, int E, int N, int Kd, int64_t r_max,
                       hipStream_t s) {
  // upper bound of the tile count: sum_e ceil(rows_e / BM) <= r_max / BM + E
  const int64_t mt = r_max / BM + E;
  int64_t grid = mt * (N / BN);
  grid = (grid + NXCD - 1) / NXCD * NXCD;
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<BN, EPI>), dim3((unsigned)grid), dim3(256), 0,
                     s, A, W, bias, out, offsets, E, N, Kd);
  return hipGetLastError();
}

// Weight-tile width: 128 when that already gives the chip (256 CUs x 2
// workgroups) enough tiles, else 64.
template <int EPI>
hipError_t launch_gemm_auto(const uint16_t* A, const uint16_t* W, const float* bias,
                            void* out, const int32_t* offsets, int E, int N, int Kd,
                            int64_t r_max, hipStream_t s) {
  const int64_t est_tiles_128 = ((r_max + BM - 1) / BM) * (N / 128);
  if (N % 128 == 0 && est_tiles_128 >= 512)
    return launch_gemm<128, EPI>(A, W, bias, out, offsets, E, N, Kd, r_max, s);
  return launch_gemm<64, EPI>(A, W, bias, out, offsets, E, N, Kd, r_max, s);
}

}  // namespace

hipError_t launch_ffn_bf16(const uint16_t* xd, const int32_t* offsets, const uint16_t* w1,
                           const float* b1, const uint16_t* w2, const float* b2,
                           uint16_t* hbuf, float* y, int E, int h, int F, int64_t r_max,
                           hipStream_t s) {
  if (r_max == 0) return hipSuccess;
  hipError_t err = launch_gemm_auto<0>(xd, w1, b1, hbuf, offsets, E, F, h, r_max, s);
  if (err != hipSuccess) return err;
  return launch_gemm_auto<1>(hbuf, w2, b2, y, offsets, E, h, F, r_max, s);
}

hipError_t launch_ffn_f32(const float* xd, const int32_t* offsets, const float* w1,
                          const float* b1, const float* w2, const float* b2, float* hbuf,
                          float* y, int E, int h, int F, int64_t r_max, hipStream_t s) {
  if (r_max == 0) return hipSuccess;
  int64_t n1 = r_max * F, n2 = r_max * h;
  hipLaunchKernelGGL((ffn_f32_kernel<0>), dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0,
                     s, xd, w1, b1, hbuf, offsets, E, F, h, r_max);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((ffn_f32_kernel<1>), dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0,
                     s, hbuf, w2, b2, y, offsets, E, h, F, r_max);
  return hipGetLastError();
}

}  // namespace moe
