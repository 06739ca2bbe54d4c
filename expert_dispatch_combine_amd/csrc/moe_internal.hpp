// Internal declarations shared by the HIP translation units of libmoe.
// Device helpers (bf16 conversion, MFMA operand types) and the launchers each
// kernel file exports to the C-ABI layer in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Limits of the kernels (validated on the host before any launch).
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxRanks = 64;

// Routes handled by one workgroup of the dispatch count / slot kernels.
constexpr int kDispatchRoutesPerBlock = 1024;
// routes up to which the whole dispatch runs as one launch
constexpr int kSmallDispatchRoutes = 8192;
// Routes handled by one workgroup of the ledger partial kernel.
constexpr int kLedgerRoutesPerBlock = 512;
// routes up to which one workgroup computes the whole ledger
constexpr int kSmallLedgerRoutes = 4096;
// Scalar counters of the ledger, per block and in the final area.
enum LedgerCounter {
  LC_LOCAL_ALL = 0,
  LC_CROSS_ALL,
  LC_LOCAL_ACC,
  LC_CROSS_ACC,
  LC_ACCEPTED,
  LC_INVALID_ID,
  LC_INVALID_RANK,
  LC_COUNT_PAD,
  LC_N = 8
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t v) {
  return __uint_as_float(v << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- workspace
// Byte sizes of the per-call workspace regions (a call uses its own regions
// from offset 0; regions of different calls may overlap).
size_t dispatch_ws_bytes(int64_t A, int E);
size_t ledger_ws_bytes(int64_t A, int E, int n_ep);
// Bytes of the ledger's compact result (device final area == host stage).
__host__ __device__ inline size_t ledger_final_bytes(int E, int n_ep) {
  return (size_t)(2 * E + LC_N + n_ep * n_ep) * 8;
}
// The ledger's stage: an int64 count of parts, then up to kLedgerStageParts
// final areas of integer partials, which the host adds (exactly, in any
// order) when it decodes the stage.
constexpr int kLedgerStageParts = 4;
inline size_t ledger_stage_bytes(int E, int n_ep) {
  return 8 + (size_t)kLedgerStageParts * ledger_final_bytes(E, n_ep);
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the first HIP error.
// bias[e] += alpha * (mean - count[e]), count = histogram of topk_idx[:, 0]
hipError_t launch_bias_update(const int32_t* idx, int T, int K, int E, float alpha, float* bias,
                              int32_t* counts, hipStream_t s);
hipError_t launch_router_topk_bf16(const uint16_t* x, const uint16_t* wg, const float* bias,
                                   float* logits, int32_t* idx, float* gate, int32_t* load,
                                   int T, int h, int E, int K, hipStream_t s);
hipError_t launch_router_gemm_f32(const float* x, const float* wg, float* logits, int T,
                                  int h, int E, hipStream_t s);
// bf16 router, every batch shape: product + top-k + softmax (+ histogram).
hipError_t launch_router_bf16(const uint16_t* x, const uint16_t* wg, const float* bias,
                              float* logits, int32_t* idx, float* gate, int32_t* load, int T,
                              int h, int E, int K, void* ws, size_t ws_bytes, hipStream_t s);
// Workspace bytes launch_router_bf16 uses for split partial products (0: none).
size_t router_parts_bytes(int T, int h, int E, int K);
hipError_t launch_topk_parts(float* logits, const float* parts, int KS, const float* bias,
                             int32_t* idx, float* gate, int32_t* load, int T, int E, int K,
                             hipStream_t s);
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);
hipError_t launch_topk_softmax(const float* logits, const float* bias, int32_t* idx,
                               float* gate, int32_t* load, int T, int E, int K,
                               hipStream_t s);

// ---- cross-lane exchanges by DPP (no LDS round trip)
// Value of a partner lane in the same 16-lane row: step 0 pairs lane ^ 1,
// step 1 lane ^ 2 (quad permutes), step 2 mirrors each 8-lane half, step 3
// each 16-lane row.  For a group of G <= 16 aligned lanes, steps 0 ..
// log2(G) - 1 in this order combine every lane with the whole group.
template <int STEP>
__device__ __forceinline__ int dpp_partner(int v) {
  constexpr int ctrl = STEP == 0 ? 0xB1 : STEP == 1 ? 0x4E : STEP == 2 ? 0x141 : 0x140;
  return __builtin_amdgcn_mov_dpp(v, ctrl, 0xF, 0xF, false);
}
template <int STEP>
__device__ __forceinline__ float dpp_partner(float v) {
  return __int_as_float(dpp_partner<STEP>(__float_as_int(v)));
}
// inclusive prefix sum over the 64 lanes of a wave (every lane active): a
// shift-and-add scan inside each 16-lane row (lanes shifted in from outside
// the row read 0), then the totals of the lower rows
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (int)(threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// sum over the 64 lanes of a wave (every lane active), returned to all lanes
__device__ __forceinline__ int wave_sum(int v) {
  v += dpp_partner<0>(v);
  v += dpp_partner<1>(v);
  v += dpp_partner<2>(v);
  v += dpp_partner<3>(v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// ---- OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
// infinities; 0x7F/0xFF = NaN; largest finite 448), as in "MoE大模型专家并行与
// 动态路由优化" 4.3 (FP8 all-to-all payload).

// nearest E4M3 code, ties to even; magnitudes above 464 (and NaN) -> NaN code
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (!(a <= 464.0f)) return sign | 0x7Fu;
  if (a < 0x1p-6f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);  // spacing 2^-9
  int lead = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;            // a is normal
  int q = (int)__builtin_rintf(__builtin_ldexpf(a, 3 - lead));           // 8 .. 16
  if (q == 16) {
    ++lead;
    q = 8;
  }
  return sign | ((uint32_t)(lead + 7) << 3) | (uint32_t)(q - 8);
}

// value of an E4M3 code (never called on the NaN code by the quantiser's output)
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e == 0 ? (float)m * 0x1p-9f
                           : __builtin_ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
  return (c & 0x80u) ? -mag : mag;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// eight bf16 (one 16-byte vector) -> eight E4M3 codes: code(bf16(x / scale)),
// rscale = RN(1 / scale); a zero scale (all-zero activations) gives zero codes.
// bf16(x / scale) with x / scale the correctly rounded fp32 quotient: the
// product x * rscale lies within 3 fp32 ulps of the quotient, so it rounds to
// the same bf16 unless its low 16 bits are within 4 of the bf16 rounding
// midpoint; only then is the quotient divided out exactly.  The codes come
// from gfx950's packed conversion (round to nearest even, the OCP E4M3
// encoding; it equals e4m3_code on every bf16 value up to 464 in magnitude),
// from e4m3_code beyond that range.  Both rare cases are tested once per
// vector, so the common path has no branch.
__device__ __forceinline__ uint2 quantize8(u32x4 v, float scale, float rscale) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  typedef float f32x2v_ __attribute__((ext_vector_type(2)));
  if (scale == 0.0f) return make_uint2(0u, 0u);
  float x[8], q[8];
  bool near = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w = v[i >> 1];
    x[i] = __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
    q[i] = x[i] * rscale;
    near |= (__float_as_uint(q[i]) & 0xFFFFu) - 0x7FFCu <= 8u;
  }
  if (near) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((__float_as_uint(q[i]) & 0xFFFFu) - 0x7FFCu <= 8u) q[i] = __fdiv_rn(x[i], scale);
  }
  // bf16 rounding (nearest even, packed conversion), widened back to fp32
  float b[8];
  bool in_range = true;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const uint32_t p = __builtin_bit_cast(
        uint32_t, __builtin_convertvector(f32x2v_{q[i], q[i + 1]}, bf16x2v));
    b[i] = __uint_as_float(p << 16);
    b[i + 1] = __uint_as_float(p & 0xFFFF0000u);
    in_range = in_range & (fabsf(b[i]) <= 464.0f) & (fabsf(b[i + 1]) <= 464.0f);
  }
  if (!in_range)
    return make_uint2(e4m3_code(b[0]) | (e4m3_code(b[1]) << 8) | (e4m3_code(b[2]) << 16) |
                          (e4m3_code(b[3]) << 24),
                      e4m3_code(b[4]) | (e4m3_code(b[5]) << 8) | (e4m3_code(b[6]) << 16) |
                          (e4m3_code(b[7]) << 24));
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(b[0], b[1], 0, false);
  const int hi = __builtin_amdgcn_cvt_pk_fp8_f32(b[4], b[5], 0, false);
  return make_uint2((uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(b[2], b[3], lo, true),
                    (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(b[6], b[7], hi, true));
}

// dst[row] = x[row_token[row]] for row < offsets[E] (rows of row_bytes bytes;
// r_max bounds offsets[E]).
hipError_t launch_gather_rows(const void* x, const int32_t* row_token, const int32_t* offsets,
                              int E, int64_t row_bytes, int64_t r_max, void* dst,
                              hipStream_t s);
// q_scale: NULL for a plain row copy, else the device address of the FP8
// scale; then x holds bf16 rows and x_disp receives E4M3 codes (h bytes/row).
// x_disp == NULL: routing metadata only, no row is copied.
hipError_t launch_dispatch(const void* x, const int32_t* topk_idx, int64_t A, int K, int E,
                           int64_t cap, int64_t row_bytes, int64_t r_max,
                           int32_t* offsets, int32_t* route_rank, int32_t* route_row,
                           int32_t* row_token, void* x_disp, int32_t* load, void* ws,
                           hipStream_t s, const float* q_scale = nullptr);
// FP8 payload: per-tensor scale = bf16(max|x| / 448) of n bf16 values
// (partials in ws: at least kFp8AmaxBlocks floats), and the receiver's
// dequantisation x_disp[r] = bf16(value(code) * scale) for r < offsets[E].
constexpr int kFp8AmaxBlocks = 1024;
hipError_t launch_fp8_scale(const uint16_t* x, int64_t n, float* scale, void* ws, hipStream_t s);
hipError_t launch_fp8_dequantize(const uint8_t* xq, const float* scale, const int32_t* offsets,
                                 int E, int h, int64_t r_max, uint16_t* x_disp, hipStream_t s);

// row_token == nullptr: xd holds the dispatched rows; else xd is the token
// matrix x (x_rows rows) and row r reads x[row_token[r]] (y's storage may
// serve as the staging buffer of that gather).
hipError_t launch_ffn_bf16(const uint16_t* xd, const int32_t* row_token, int64_t x_rows,
                           const int32_t* offsets, const uint16_t* w1, const float* b1,
                           const uint16_t* w2, const float* b2, uint16_t* hbuf, float* y, int E,
                           int h, int F, int64_t A, int64_t cap, int64_t r_max, bool packed,
                           hipStream_t s);
// The expert FFN on the FP8 payload: GEMM1 reads E4M3 codes xq [R_max, h] and
// widens them to bf16 x *scale while staging them.  ffn_fp8_supported: false
// where GEMM1 would take the tiled shape (bf16 activations only).
bool ffn_fp8_supported(int E, int F, int64_t A, int64_t cap, bool packed);
hipError_t launch_ffn_fp8(const uint8_t* xq, const float* scale, const int32_t* offsets,
                          const uint16_t* w1, const float* b1, const uint16_t* w2,
                          const float* b2, uint16_t* hbuf, float* y, int E, int h, int F,
                          int64_t A, int64_t cap, int64_t r_max, bool packed, hipStream_t s);
// Row-major [E, N, K] bf16 -> packed fragment blocks (N % 32 == 0, K % 64 == 0).
hipError_t launch_pack_weights(const uint16_t* w, uint16_t* wp, int E, int N, int Kd,
                               hipStream_t s);
hipError_t launch_ffn_f32(const float* xd, const int32_t* row_token, const int32_t* offsets,
                          const float* w1, const float* b1, const float* w2, const float* b2,
                          float* hbuf, float* y, int E, int h, int F, int64_t r_max,
                          hipStream_t s);

hipError_t launch_combine(const float* y, const int32_t* route_row, const float* gate,
                          float* out, int T, int K, int h, hipStream_t s);

// Ledger: per-block partials then a fixed-order reduction into `final_area`
// (layout: loads[E] int64 | P[E] uint64, sums of gates in units of 2^-32 |
//  counters[LC_N] int64 | pairs[n_ep*n_ep] int64), preceded by the stage's
// int64 part count.
// fin_dst: device-accessible destination of the final area (e.g. the device
// address of page-locked host memory), or NULL for the area in `ws`.
hipError_t launch_ledger(const int32_t* idx, const float* gate, const int32_t* route_row,
                         const int32_t* src, const int32_t* owner, int T, int K, int E,
                         int n_ep, void* ws, void* fin_dst, void** final_area,
                         size_t* final_bytes, hipStream_t s);
// The combine and the ledger of the same routes: one launch up to
// kSmallLedgerRoutes routes (one ledger workgroup per 1024 routes, each
// writing its own integer partials into the stage, beside the combine's
// workgroups), else launch_combine then launch_ledger.  Same out and the same
// decoded ledger as those two.
hipError_t launch_combine_ledger(const float* y, const int32_t* route_row, const float* gate,
                                 float* out, const int32_t* idx, const int32_t* src,
                                 const int32_t* owner, int T, int K, int h, int E, int n_ep,
                                 void* ws, void* fin_dst, void** final_area,
                                 size_t* final_bytes, hipStream_t s);

}  // namespace moe
