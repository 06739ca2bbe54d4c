// Expert FFN over ragged expert segments: grouped GEMMs on bf16 MFMA.
//
// Method: "MoE大模型专家并行与动态路由优化" section 一, FFN(x) = W2 sigma(W1 x + b1)
// + b2 per expert, sigma = GELU (tanh form).  Each expert e owns the rows
// [offsets[e], offsets[e+1]) of the dispatched buffer:
//   GEMM1: H[r, n] = GELU(sum_k x_disp[r, k] W1[e, n, k] + b1[e, n])  -> bf16
//   GEMM2: Y[r, n] = sum_k H[r, k] W2[e, n, k] + b2[e, n]             -> fp32
// The MFMA is v_mfma_f32_32x32x16_bf16 with the WEIGHT rows as operand A and
// the activation rows as operand B: an accumulator lane then holds one
// activation row and 4 consecutive output columns (8-byte bf16 / 16-byte fp32
// stores).  Within a 16-wide k-step a lane supplies 8 consecutive k of its
// row; which 8 is a free choice as long as both operands agree.
//
// Weights come in one of two layouts:
//  * row-major [E, N, K] as the caller stores them;
//  * packed (moe_pack_expert_weights): per expert, per 32-row tile, per
//    64-wide k-chunk, one 4 KB block laid out exactly as a wave's lanes hold
//    its MFMA fragments -- lane l = (row l%32, half l/32), k-step q holds
//    k = 32*(l/32) + 8q .. +7 at byte (64 q + l) * 16.  A wave then reads each
//    fragment as one contiguous 1 KB load and a 32-row strip of a weight as
//    one linear stream, which is what HBM serves at full rate (row-major
//    fragments touch 32 rows x 32 bytes per load and run ~30% slower).
//
// Four kernel shapes, chosen per launch on the host:
//  * streaming (rows per expert up to a few hundred: weight-bandwidth bound).
//    A workgroup takes ALL rows of one expert (up to 160, in 32-row MFMA
//    tiles) and 32*WN*TN weight rows, so each weight byte crosses HBM once.
//    Weights are read once, with nontemporal loads (streamed past the caches
//    that keep the activations), and the fp32 outputs of the second GEMM are
//    written with nontemporal stores.
//    Weights go straight from global memory into a register ring PD chunks
//    deep (no LDS), TN 32-row strips per wave (up to four where a launch
//    still gives every CU a workgroup); activations are shared by the 4
//    waves through a double-buffered, XOR-swizzled LDS tile, loaded two or
//    four chunks ahead.  WK waves split each 64-wide k-chunk when the weight
//    dim is too short to give the chip enough work; their partial sums are
//    added in LDS in a fixed order.
//  * tiled (hundreds of rows per expert, weight dim not a multiple of 128):
//    128 x 64 tiles with both operands double-buffered in LDS, 4 waves in a
//    2 x 2 grid.
//  * wide (hundreds of rows per expert, MFMA bound): 256 x 256 tiles at one
//    workgroup per CU (each wave 128 x 128, which halves the LDS fragment
//    reads per MFMA of a 128 x 128 tiling) or 128 x 128 tiles at two per CU;
//    global loads two chunks ahead, issued and staged a quarter per k-step
//    between the MFMAs.
//  * wide with weights in registers (packed weights, 512 or more rows per
//    expert): 256 x 256 tiles, each wave all 256 rows x 64 weight rows of
//    its own, its weight fragments loaded straight into registers; only the
//    activations go through LDS.  An expert's last, partial row tile stages
//    and multiplies only its 32-row sub-tiles that hold rows (2, 4 or 8),
//    and each XCD runs those cheaper tiles after all its whole ones, so they
//    fill the end of the launch.
//
// Scheduling is on the device (no host sync): every workgroup derives the
// per-expert tile counts from `offsets`, maps its id to a logical tile with an
// XCD-aware permutation (consecutive logical tiles run on the same XCD and
// share its L2) and exits if it has none.  Logical tiles are ordered by
// expert, then groups of 8 weight tiles, then row tiles fastest (the
// weights-in-registers kernel takes the partial row tiles out of that order
// and runs them last).  Where the
// capacity fits one row tile of the streaming shape, every expert has one row
// tile whatever the routing, so the map needs no `offsets` and the weight
// prefetch starts before the expert's row range is read.
#include <type_traits>

#include "moe_internal.hpp"

namespace moe {

namespace {

constexpr int NGROUP = 8;  // weight tiles per scheduling group
constexpr int NXCD = 8;    // XCDs of an MI355X
constexpr int PBLK = 2048; // bf16 elements of one packed block (32 rows x 64 k)

__device__ __forceinline__ float gelu_tanh_f(float u) {
  // 0.5 u (1 + tanh(z)) == u * sigmoid(2 z),  z = sqrt(2/pi) (u + 0.044715 u^3)
  const float z = 0.7978845608028654f * (u + 0.044715f * u * u * u);
  return u / (1.0f + __expf(-2.0f * z));
}

// The same GELU for a bf16 result: the hardware base-2 exponential and
// reciprocal (each within a couple of fp32 ulps) replace the IEEE division,
// far below the bf16 rounding that follows.  -2 z log2(e) = u (k0 + k1 u^2).
__device__ __forceinline__ float gelu_tanh_bf16(float u) {
  constexpr float k0 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
  constexpr float k1 = k0 * 0.044715f;
  const float t = u * fmaf(k1, u * u, k0);
  return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// eight E4M3 codes (lo: codes 0-3, hi: 4-7) -> eight bf16 of value * scale,
// the receiver's dequantisation of the FP8 payload.  gfx950's packed
// conversion widens two OCP E4M3 codes (bias 7, 3 mantissa bits, subnormals
// m * 2^-9) to fp32 exactly; the product of a 4-bit and an 8-bit significand
// is exact in fp32 and is rounded once to bf16.
typedef float f32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 dequant8(uint32_t lo, uint32_t hi, float scale) {
  const f32x2v v0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
  const f32x2v v1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  const f32x2v v2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
  const f32x2v v3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  u32x4 o;
  o[0] = pack_bf16x2(v0[0] * scale, v0[1] * scale);
  o[1] = pack_bf16x2(v1[0] * scale, v1[1] * scale);
  o[2] = pack_bf16x2(v2[0] * scale, v2[1] * scale);
  o[3] = pack_bf16x2(v3[0] * scale, v3[1] * scale);
  return o;
}

// Activation elements of the first GEMM: bf16 (AB = 2 bytes) or E4M3 codes
// of the FP8 dispatch payload (AB = 1), widened to bf16 x scale when staged.
template <int AB>
struct ActIn {
  using V = typename std::conditional<AB == 2, u32x4, uint2>::type;  // 8 elements
  static __device__ __forceinline__ u32x4 widen(const V& v, float scale) {
    if constexpr (AB == 2) {
      (void)scale;
      return v;
    } else {
      return dequant8(v.x, v.y, scale);
    }
  }
};

struct TileInfo {
  int e, row0, row_end, n0;
};

// Find this workgroup's (expert, row tile, weight tile).  False: no tile.
template <int BM, int BN>
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int E, int N,
                                          TileInfo* sh, int tid) {
  const int ntn = (N + BN - 1) / BN;
  if (tid < 64) {
    const int lane = tid;
    if (lane == 0) sh->e = -1;
    const int per = (E + 63) / 64;
    const int ebeg = min(E, lane * per), eend = min(E, ebeg + per);
    int mine = 0;
    for (int e = ebeg; e < eend; ++e) {
      const int rows = offsets[e + 1] - offsets[e];
      mine += (rows + BM - 1) / BM * ntn;
    }
    const int incl = wave_incl_scan(mine);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    const int per_xcd = (total + NXCD - 1) / NXCD;
    const int bid = blockIdx.x;
    int L = -1;
    if (bid < per_xcd * NXCD) L = (bid % NXCD) * per_xcd + bid / NXCD;
    if (L >= total) L = -1;
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

// The tile map of the weights-in-registers kernel.  Each XCD walks its share
// of the experts' whole BM-row tiles first (in find_tile's order: expert,
// groups of 8 weight tiles, row tiles fastest), then its share of the
// experts' last, partial row tiles, which cost less (only their 32-row
// sub-tiles that hold rows run MFMAs) and so fill the end of the launch.
// Needs grid / NXCD >= ceil(TF / NXCD) + ceil(TP / NXCD) workgroups per XCD
// (TF whole, TP partial tiles).
template <int BM, int BN>
__device__ __forceinline__ bool find_tile_partial_last(const int32_t* __restrict__ offsets,
                                                       int E, int N, TileInfo* sh, int tid) {
  const int ntn = (N + BN - 1) / BN;
  if (tid < 64) {
    const int lane = tid;
    if (lane == 0) sh->e = -1;
    const int per = (E + 63) / 64;
    const int ebeg = min(E, lane * per), eend = min(E, ebeg + per);
    int mf = 0, mp = 0;
    for (int e = ebeg; e < eend; ++e) {
      const int rows = offsets[e + 1] - offsets[e];
      mf += rows / BM * ntn;
      mp += (rows % BM != 0) ? ntn : 0;
    }
    const int incf = wave_incl_scan(mf), incp = wave_incl_scan(mp);
    const int TF = __builtin_amdgcn_readlane(incf, 63), TP = __builtin_amdgcn_readlane(incp, 63);
    const int pf = (TF + NXCD - 1) / NXCD, pp = (TP + NXCD - 1) / NXCD;
    const int x = blockIdx.x % NXCD, j = blockIdx.x / NXCD;
    const int nfx = max(0, min(pf, TF - x * pf)), npx = max(0, min(pp, TP - x * pp));
    int L = -1;
    const bool part = j >= nfx;
    if (!part) L = x * pf + j;
    else if (j - nfx < npx) L = x * pp + (j - nfx);
    if (L >= 0) {
      int p = part ? incp - mp : incf - mf;
      for (int e = ebeg; e < eend; ++e) {
        const int o0 = offsets[e], o1 = offsets[e + 1];
        const int nfull = (o1 - o0) / BM;
        const int t = part ? (((o1 - o0) % BM != 0) ? ntn : 0) : nfull * ntn;
        if (L >= p && L < p + t) {
          const int r = L - p;
          int mt, nt;
          if (part) {
            mt = nfull;
            nt = r;
          } else {
            const int ng = r / (nfull * NGROUP);
            const int within = r - ng * nfull * NGROUP;
            mt = within % nfull;
            nt = ng * NGROUP + within / nfull;
          }
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

// Epilogue of one 32x32 accumulator: lane holds row m and, for q = 0..3,
// columns n + 8q .. n + 8q + 3.  EPI 0: bf16(GELU(acc + b)), EPI 1: acc + b.
template <int EPI>
__device__ __forceinline__ void store_tile(const f32x16& acc, const float* __restrict__ bptr,
                                           void* __restrict__ out, int m, int n, int N) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int nn = n + q * 8;
    const float4 b = *(const float4*)(bptr + nn);
    float v0 = acc[4 * q + 0] + b.x;
    float v1 = acc[4 * q + 1] + b.y;
    float v2 = acc[4 * q + 2] + b.z;
    float v3 = acc[4 * q + 3] + b.w;
    if (EPI == 0) {
      uint2 pk;
      pk.x = pack_bf16x2(gelu_tanh_bf16(v0), gelu_tanh_bf16(v1));
      pk.y = pack_bf16x2(gelu_tanh_bf16(v2), gelu_tanh_bf16(v3));
      *(uint2*)((uint16_t*)out + (size_t)m * N + nn) = pk;
    } else {
      *(float4*)((float*)out + (size_t)m * N + nn) = make_float4(v0, v1, v2, v3);
    }
  }
}

// Activation LDS tile: rows of 64 bf16 (8 quads); quad q of row r is stored at
// quad q ^ ((r >> 1) & 7).  Two consecutive rows share one 256-byte bank
// window, so this spreads any 16 consecutive rows read at one quad over all
// 16 bank groups (conflict-free ds_read_b128).
__device__ __forceinline__ int act_slot(int r, int q) { return r * 64 + ((q ^ ((r >> 1) & 7)) << 3); }

// ==========================================================================
// streaming kernel
// ==========================================================================
// OCC = workgroups per CU the kernel is built for.  With OCC 1 (launches with
// at most one workgroup per CU) each wave owns twice the registers, spent on
// deeper prefetch: 8 weight chunks and 4 activation chunks in flight.
// TN = 32-row weight strips per wave.  With TN 2 or 4 (at OCC 1) each
// staged activation chunk and each activation fragment read from LDS serves
// TN times the weights, which divides the activation loads per weight byte
// by TN; the ring then holds 4 (TN 2) or 2 (TN 4) chunks of all strips, the
// same bytes in flight per CU as 8 waves with one strip and 4 chunks each.
template <int MT, int WN, int WK, int OCC, int TN = 1>
struct StreamShape {
  static constexpr int BM = 32 * MT;         // activation rows per workgroup
  static constexpr int BN = 32 * WN * TN;    // weight rows per workgroup
  static constexpr int KC = 64;              // k per chunk (one LDS stage)
  static constexpr int KW = KC / WK;         // k per wave and chunk
  static constexpr int KSTEPS = KW / 16;     // MFMA k-steps per wave and chunk
  // chunks in the weight ring: 16 KB in flight per wave at two workgroups
  // per CU (8 KB when a wave takes only 16 k of a chunk, to stay within the
  // register budget), 32 KB at one (8 chunks of one strip, 4 of two, 2 of
  // four)
  static constexpr int PD = OCC == 1 ? (TN == 4 ? 2 : TN == 2 ? 4 : 8) : ((256 / KW) < 8 ? (256 / KW) : 8);
  // activation register slots: chunk c + AD is loaded while chunk c computes.
  // Loads complete in issue order, so the wait for chunk c + 1's activations
  // also waits for every weight load issued before them: with AD = 4 those
  // are weights of chunk c at the latest (already needed), with AD = 2 they
  // include chunk c + 1's, which shortens the weight lookahead.  (AD = 4
  // outgrows the registers of 160-row tiles at occupancy 2, and of four
  // strips per wave; with TN 4 the ring is 2 chunks deep, so the weights
  // issued before chunk c + 1's activations are again those of chunk c.)
  static constexpr int AD = TN == 4 ? 2 : OCC == 1 || MT <= 4 ? 4 : 2;
  static constexpr int STAGE = BM * KC;      // bf16 elements of one LDS stage
  static constexpr int ACT_BYTES = 2 * STAGE * 2;
  static constexpr int RED_BYTES = (WK - 1) * WN * MT * 16 * 64 * 4;
  // epilogue: 32 output rows at a time, rows padded by 16 bytes
  static constexpr int OUT_ROW_BYTES(int esz) { return BN * esz + 16; }
  static constexpr int OUT_BYTES = 32 * (BN * 4 + 16);
  static constexpr int M1 = ACT_BYTES > RED_BYTES ? ACT_BYTES : RED_BYTES;
  static constexpr int LDS_BYTES = M1 > OUT_BYTES ? M1 : OUT_BYTES;
};

// one_rt != 0: the host guarantees that every expert's rows fit one row tile
// (rows <= BM), so tile L is (expert L / (N/BN), weight tile L % (N/BN)) with
// no look at `offsets`: the weight prefetch is issued before the expert's row
// range arrives, and a workgroup of an empty expert leaves after reading it.
// rowmap != nullptr: activation row r is A[rowmap[r]] (the dispatch gather,
// done by the loads themselves: A is then the token matrix x).
// AB: activation bytes per element, 2 (bf16) or 1 (E4M3 codes, widened to
// bf16 x *ascale before they are staged in LDS).
template <int MT, int WN, int WK, int EPI, bool PK, int OCC, int AB, int TN>
__global__ __launch_bounds__(256, OCC) void stream_gemm_kernel(
    const void* __restrict__ A, const uint16_t* __restrict__ W,
    const float* __restrict__ bias, void* __restrict__ out,
    const int32_t* __restrict__ offsets, int E, int N, int Kd, int one_rt,
    const int32_t* __restrict__ rowmap, const float* __restrict__ ascale) {
  using S = StreamShape<MT, WN, WK, OCC, TN>;
  static_assert(TN == 1 || WK == 1, "strips per wave without a k split");
  using AI = ActIn<AB>;
  using AV = typename AI::V;
  static_assert(S::PD % S::AD == 0 && S::PD % 2 == 0, "ring sizes");
  // the epilogue stages all BM output rows at once when they fit in 48 KB
  constexpr int OUT_ALL = MT * 32 * (S::BN * (EPI == 0 ? 2 : 4) + 16);
  constexpr bool ONE_PASS = OUT_ALL <= 48 * 1024;
  constexpr int LDS_SZ = ONE_PASS && OUT_ALL > S::LDS_BYTES ? OUT_ALL : S::LDS_BYTES;
  __shared__ __attribute__((aligned(16))) char lds[LDS_SZ];
  __shared__ TileInfo tinfo;
  uint16_t* act = (uint16_t*)lds;  // [2][BM rows][8 quads], swizzled

  const int tid = threadIdx.x;
  int e, row0 = 0, row_end = 0, n0;
  if (one_rt) {
    const int ntn = N / S::BN;
    const int total = E * ntn;
    const int per_xcd = (total + NXCD - 1) / NXCD;
    const int bid = blockIdx.x;
    const int L = bid < per_xcd * NXCD ? (bid % NXCD) * per_xcd + bid / NXCD : total;
    if (L >= total) return;
    e = L / ntn;
    n0 = (L - e * ntn) * S::BN;
  } else {
    if (!find_tile<S::BM, S::BN>(offsets, E, N, &tinfo, tid)) return;
    e = tinfo.e, row0 = tinfo.row0, row_end = tinfo.row_end, n0 = tinfo.n0;
  }
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, kw = wave / WN;
  const int li = lane & 31, lg = lane >> 5;
  const int nchunks = Kd / S::KC;

  // ---- weights: base of this lane's fragments; chunk c / k-step s adds
  //      c * CSTR + s * QSTR
  const uint16_t* wp;
  constexpr int CSTR = PK ? PBLK : S::KC;
  constexpr int QSTR = PK ? 512 : 8;
  if (PK)
    wp = W + ((size_t)e * (N / 32) + (n0 + wn * TN * 32) / 32) * nchunks * PBLK +
         (kw * S::KSTEPS * 64 + lane) * 8;
  else
    wp = W + ((size_t)e * N + n0 + wn * TN * 32 + li) * Kd + kw * S::KW + lg * (S::KW / 2);
  const size_t tstr = PK ? (size_t)nchunks * PBLK : (size_t)32 * Kd;  // next strip
  u32x4 wr[S::PD][TN][S::KSTEPS];
#pragma unroll
  for (int p = 0; p < S::PD - 1; ++p)
    if (p < nchunks)
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int q = 0; q < S::KSTEPS; ++q)
          wr[p][t][q] = __builtin_nontemporal_load((const u32x4*)(wp + t * tstr + p * CSTR + q * QSTR));
  if (one_rt) {
    row0 = offsets[e];
    row_end = offsets[e + 1];
    if (row_end <= row0) return;  // empty expert (uniform)
  }

  // ---- activations: this thread stages MT quads per chunk (row c/8, quad c%8)
  const char* ap[MT];
  int alds[MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int c = tid + 256 * j;
    const int r = c >> 3, q = c & 7;
    const int row = min(row0 + r, row_end - 1);
    ap[j] = (const char*)A + ((size_t)(rowmap ? rowmap[row] : row) * Kd + q * 8) * AB;
    alds[j] = act_slot(r, q);
  }
  const float asc = AB == 1 ? *ascale : 0.0f;
  // activation fragments: the quad of the chunk that matches the weights' k
  int afrag[MT][S::KSTEPS];
#pragma unroll
  for (int tm = 0; tm < MT; ++tm)
#pragma unroll
    for (int s = 0; s < S::KSTEPS; ++s) {
      const int r = tm * 32 + li;
      const int q = PK ? lg * 4 + kw * S::KSTEPS + s
                       : (kw * S::KW + lg * (S::KW / 2) + s * 8) >> 3;
      afrag[tm][s] = act_slot(r, q);
    }

  f32x16 acc[MT][TN];
#pragma unroll
  for (int tm = 0; tm < MT; ++tm)
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tm][t][r] = 0.f;

  // activations: chunk 0 straight into LDS stage 0, chunks 1 .. AD-1 into
  // register slots; chunk c+AD is always in flight while chunk c is computed
  AV areg[S::AD][MT];
#pragma unroll
  for (int j = 0; j < MT; ++j) areg[0][j] = *(const AV*)(ap[j]);
#pragma unroll
  for (int a = 1; a < S::AD; ++a)
    if (a < nchunks)
#pragma unroll
      for (int j = 0; j < MT; ++j) areg[a][j] = *(const AV*)(ap[j] + a * S::KC * AB);
#pragma unroll
  for (int j = 0; j < MT; ++j) *(u32x4*)(act + alds[j]) = AI::widen(areg[0][j], asc);
  __syncthreads();

  // One k-chunk c (PD is a multiple of AD and of 2, so every slot index is
  // compile-time): issue the activations of chunk c+AD into slot c%AD and
  // the weights of chunk c+PD-1 into the ring slot freed by chunk c-1 (both
  // before the MFMAs, so the memory pipe stays fed while they run), MFMAs on
  // chunk c (weights from ring slot SLOT, activations from LDS stage STG),
  // stage chunk c+1 (register slot (c+1)%AD, loaded AD-1 chunks earlier) into
  // the other LDS buffer.  In the
  // steady-state loop every condition is compile-time true, so the body has
  // no branches and the compiler counts the loads in flight exactly.
#define MOE_STREAM_CHUNK(SLOT, STG, ASLOT, NSLOT, c, HAS_NEXT, HAS_NEXTA, REFILL)      \
  do {                                                                                \
    const uint16_t* stage_ = act + (STG) * S::STAGE;                                  \
    if (HAS_NEXTA) {                                                                  \
      _Pragma("unroll") for (int j = 0; j < MT; ++j) areg[ASLOT][j] =                 \
          *(const AV*)(ap[j] + ((c) + S::AD) * S::KC * AB);                           \
    }                                                                                 \
    if (REFILL) {                                                                     \
      _Pragma("unroll") for (int t = 0; t < TN; ++t)                                  \
        _Pragma("unroll") for (int q = 0; q < S::KSTEPS; ++q)                         \
          wr[((SLOT) + S::PD - 1) % S::PD][t][q] = __builtin_nontemporal_load(        \
              (const u32x4*)(wp + t * tstr + ((c) + S::PD - 1) * CSTR + q * QSTR));   \
    }                                                                                 \
    if constexpr (OCC == 1) {                                                         \
      /* one wave per SIMD: nothing else hides LDS latency, so every fragment */      \
      /* of the chunk is read before the first MFMA (the scheduling barrier */        \
      /* keeps the compiler from sinking the reads next to their uses) */             \
      bf16x8 xf_[S::KSTEPS][MT];                                                      \
      _Pragma("unroll") for (int s = 0; s < S::KSTEPS; ++s)                           \
        _Pragma("unroll") for (int tm = 0; tm < MT; ++tm) xf_[s][tm] =                \
            *(const bf16x8*)(stage_ + afrag[tm][s]);                                  \
      __builtin_amdgcn_sched_barrier(0);                                              \
      _Pragma("unroll") for (int s = 0; s < S::KSTEPS; ++s)                           \
        _Pragma("unroll") for (int t = 0; t < TN; ++t) {                              \
          const bf16x8 wa = __builtin_bit_cast(bf16x8, wr[SLOT][t][s]);               \
          _Pragma("unroll") for (int tm = 0; tm < MT; ++tm)                           \
            acc[tm][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, xf_[s][tm],       \
                                                                 acc[tm][t], 0, 0, 0); \
        }                                                                             \
    } else {                                                                          \
      _Pragma("unroll") for (int s = 0; s < S::KSTEPS; ++s) {                         \
        _Pragma("unroll") for (int tm = 0; tm < MT; ++tm) {                           \
          const bf16x8 xb = *(const bf16x8*)(stage_ + afrag[tm][s]);                  \
          _Pragma("unroll") for (int t = 0; t < TN; ++t)                              \
            acc[tm][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                     \
                __builtin_bit_cast(bf16x8, wr[SLOT][t][s]), xb, acc[tm][t], 0, 0, 0); \
        }                                                                             \
      }                                                                               \
    }                                                                                 \
    if (HAS_NEXT) {                                                                   \
      uint16_t* nst_ = act + ((STG) ^ 1) * S::STAGE;                                  \
      _Pragma("unroll") for (int j = 0; j < MT; ++j) *(u32x4*)(nst_ + alds[j]) =      \
          AI::widen(areg[NSLOT][j], asc);                                             \
    }                                                                                 \
    __syncthreads();                                                                  \
  } while (0)

  // steady state: chunks c+1, c+AD and c+PD-1 all exist (PD >= AD)
  int c0 = 0;
  for (; c0 + 2 * S::PD <= nchunks; c0 += S::PD) {
#pragma unroll
    for (int p = 0; p < S::PD; ++p)
      MOE_STREAM_CHUNK(p, p & 1, p % S::AD, (p + 1) % S::AD, c0 + p, true, true, true);
  }
  // tail: the last (fewer than 2*PD) chunks
#pragma unroll
  for (int p = 0; p < 2 * S::PD; ++p) {
    const int c = c0 + p;
    if (c < nchunks)
      MOE_STREAM_CHUNK(p % S::PD, p & 1, p % S::AD, (p + 1) % S::AD, c, c + 1 < nchunks,
                       c + S::AD < nchunks, c + S::PD - 1 < nchunks);
  }
#undef MOE_STREAM_CHUNK

  // ---- k-split waves: add partial sums in wave order through LDS
  if (WK > 1) {
    float* red = (float*)lds;
    if (kw > 0) {
#pragma unroll
      for (int tm = 0; tm < MT; ++tm)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          red[((((kw - 1) * WN + wn) * MT + tm) * 16 + r) * 64 + lane] = acc[tm][0][r];
    }
    __syncthreads();
    if (kw == 0) {
#pragma unroll
      for (int k2 = 1; k2 < WK; ++k2)
#pragma unroll
        for (int tm = 0; tm < MT; ++tm)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[tm][0][r] += red[((((k2 - 1) * WN + wn) * MT + tm) * 16 + r) * 64 + lane];
    }
  }

  // ---- epilogue: bias (+ GELU, bf16), 32 rows at a time through LDS, then
  //      written out as whole contiguous row segments (the accumulator layout
  //      would otherwise scatter each store over 32 rows)
  constexpr int ESZ = EPI == 0 ? 2 : 4;
  constexpr int ROWB = S::OUT_ROW_BYTES(ESZ);
  constexpr int CPR = S::BN * ESZ / 16;  // 16-byte chunks per output row
  float4 bq[TN][4];
  {
    const float* bptr = bias + (size_t)e * N + n0 + wn * TN * 32 + lg * 4;
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) bq[t][q] = *(const float4*)(bptr + t * 32 + q * 8);
  }
  char* tile = lds;
  if constexpr (ONE_PASS) {
    __syncthreads();  // LDS free: k-loop / reduction done
    if (kw == 0) {
#pragma unroll
      for (int tm = 0; tm < MT; ++tm) {
        if (row0 + tm * 32 >= row_end) break;  // uniform
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          char* rowp = tile + (tm * 32 + li) * ROWB + ((wn * TN + t) * 32 + lg * 4) * ESZ;
          const float v0 = acc[tm][t][4 * q + 0] + bq[t][q].x, v1 = acc[tm][t][4 * q + 1] + bq[t][q].y;
          const float v2 = acc[tm][t][4 * q + 2] + bq[t][q].z, v3 = acc[tm][t][4 * q + 3] + bq[t][q].w;
          if (EPI == 0) {
            uint2 pk;
            pk.x = pack_bf16x2(gelu_tanh_bf16(v0), gelu_tanh_bf16(v1));
            pk.y = pack_bf16x2(gelu_tanh_bf16(v2), gelu_tanh_bf16(v3));
            *(uint2*)(rowp + q * 8 * ESZ) = pk;
          } else {
            *(float4*)(rowp + q * 8 * ESZ) = make_float4(v0, v1, v2, v3);
          }
        }
      }
    }
    __syncthreads();
    const int rows = min(S::BM, row_end - row0);
    char* gout = (char*)out + ((size_t)row0 * N + n0) * ESZ;
    for (int i = tid; i < rows * CPR; i += 256) {
      const int r = i / CPR, c = i - r * CPR;
      const u32x4 v = *(const u32x4*)(tile + r * ROWB + c * 16);
      u32x4* dst = (u32x4*)(gout + (size_t)r * N * ESZ + c * 16);
      if (EPI == 1) __builtin_nontemporal_store(v, dst);  // Y: read back only by the combine
      else *dst = v;                                       // H: read next by the second GEMM
    }
    return;
  }
#pragma unroll
  for (int tm = 0; tm < MT; ++tm) {
    if (row0 + tm * 32 >= row_end) break;  // uniform
    __syncthreads();  // LDS free: previous pass copied out / reduction read
    if (kw == 0) {
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        char* rowp = tile + li * ROWB + ((wn * TN + t) * 32 + lg * 4) * ESZ;
        const float v0 = acc[tm][t][4 * q + 0] + bq[t][q].x, v1 = acc[tm][t][4 * q + 1] + bq[t][q].y;
        const float v2 = acc[tm][t][4 * q + 2] + bq[t][q].z, v3 = acc[tm][t][4 * q + 3] + bq[t][q].w;
        if (EPI == 0) {
          uint2 pk;
          pk.x = pack_bf16x2(gelu_tanh_bf16(v0), gelu_tanh_bf16(v1));
          pk.y = pack_bf16x2(gelu_tanh_bf16(v2), gelu_tanh_bf16(v3));
          *(uint2*)(rowp + q * 8 * ESZ) = pk;
        } else {
          *(float4*)(rowp + q * 8 * ESZ) = make_float4(v0, v1, v2, v3);
        }
      }
    }
    __syncthreads();
    const int rows = min(32, row_end - (row0 + tm * 32));
    char* gout = (char*)out + ((size_t)(row0 + tm * 32) * N + n0) * ESZ;
    for (int i = tid; i < rows * CPR; i += 256) {
      const int r = i / CPR, c = i - r * CPR;
      const u32x4 v = *(const u32x4*)(tile + r * ROWB + c * 16);
      u32x4* dst = (u32x4*)(gout + (size_t)r * N * ESZ + c * 16);
      if (EPI == 1) __builtin_nontemporal_store(v, dst);  // Y: read back only by the combine
      else *dst = v;                                       // H: read next by the second GEMM
    }
  }
}

// ==========================================================================
// tiled kernel (both operands in LDS)
// ==========================================================================
constexpr int TBM = 128;
constexpr int TBK = 64;
constexpr int TLDS = TBK + 8;  // bf16 elements per padded LDS row (16-byte pad)

template <int BN, int EPI, bool PK>
__global__ __launch_bounds__(256, 2) void tiled_gemm_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
    const float* __restrict__ bias, void* __restrict__ out,
    const int32_t* __restrict__ offsets, int E, int N, int Kd,
    const int32_t* __restrict__ rowmap) {
  constexpr int TM = 2;        // 32-row MFMA tiles per wave (wave covers 64 rows)
  constexpr int TN = BN / 64;  // 32-col MFMA tiles per wave (wave covers BN/2 cols)
  constexpr int ACH = TBM * TBK / 8 / 256;  // 16-byte chunks per thread per stage (A)
  constexpr int WCH = BN * TBK / 8 / 256;   // (W)
  // packed weights need no padding: a block's fragment reads are linear
  constexpr int WSTAGE = PK ? BN * TBK : BN * TLDS;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][TBM * TLDS];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][WSTAGE];
  __shared__ TileInfo tinfo;

  const int tid = threadIdx.x;
  if (!find_tile<TBM, BN>(offsets, E, N, &tinfo, tid)) return;
  const int e = tinfo.e, row0 = tinfo.row0, row_end = tinfo.row_end, n0 = tinfo.n0;

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int nk = Kd / TBK;

  const uint16_t* a_src[ACH];
  int a_lds[ACH];
#pragma unroll
  for (int j = 0; j < ACH; ++j) {
    const int c = tid + j * 256;
    const int r = c >> 3, cc = c & 7;
    const int row = min(row0 + r, row_end - 1);
    a_src[j] = A + (size_t)(rowmap ? rowmap[row] : row) * Kd + cc * 8;
    a_lds[j] = r * TLDS + cc * 8;
  }
  // weight staging: row-major -> 16-byte chunk (row c/8, quad c%8) of the
  // tile; packed -> quad `tid` of 32-row block j (one 4 KB block per j)
  const uint16_t* w_src[WCH];
  int w_lds[WCH];
  constexpr int WKSTR = PK ? PBLK : TBK;  // element stride of one k-stage
#pragma unroll
  for (int j = 0; j < WCH; ++j) {
    if (PK) {
      w_src[j] = W + ((size_t)e * (N / 32) + n0 / 32 + j) * nk * PBLK + tid * 8;
      w_lds[j] = j * PBLK + tid * 8;
    } else {
      const int c = tid + j * 256;
      const int r = c >> 3, cc = c & 7;
      w_src[j] = W + ((size_t)e * N + n0 + r) * Kd + cc * 8;
      w_lds[j] = r * TLDS + cc * 8;
    }
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment offsets: k-step kk covers k = kk*16 + 8*(lane/32) (row-major)
  // or k = 32*(lane/32) + 8*kk (packed); both operands use the same map
  const int li = lane & 31, lg = lane >> 5;
  int a_frag[TM], w_frag[TN];
  constexpr int KK_STEP = PK ? 8 : 16;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
    a_frag[tm] = (wm * 64 + tm * 32 + li) * TLDS + (PK ? lg * 32 : lg * 8);
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
    w_frag[tn] = PK ? (wn * (BN / 64) + tn) * PBLK + lane * 8
                    : (wn * (BN / 2) + tn * 32 + li) * TLDS + lg * 8;
  constexpr int WKK_STEP = PK ? 512 : 16;  // packed: k-step kk is quad kk of the block

  u32x4 a_reg[ACH], w_reg[WCH];
#pragma unroll
  for (int j = 0; j < ACH; ++j) a_reg[j] = *(const u32x4*)(a_src[j]);
#pragma unroll
  for (int j = 0; j < WCH; ++j) w_reg[j] = *(const u32x4*)(w_src[j]);
#pragma unroll
  for (int j = 0; j < ACH; ++j) *(u32x4*)(&As[0][a_lds[j]]) = a_reg[j];
#pragma unroll
  for (int j = 0; j < WCH; ++j) *(u32x4*)(&Ws[0][w_lds[j]]) = w_reg[j];
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
#pragma unroll
      for (int j = 0; j < ACH; ++j) a_reg[j] = *(const u32x4*)(a_src[j] + (kt + 1) * TBK);
#pragma unroll
      for (int j = 0; j < WCH; ++j) w_reg[j] = *(const u32x4*)(w_src[j] + (kt + 1) * WKSTR);
    }
#pragma unroll
    for (int kk = 0; kk < TBK / 16; ++kk) {
      bf16x8 wf[TN], af[TM];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        wf[tn] = *(const bf16x8*)(&Ws[buf][w_frag[tn] + kk * WKK_STEP]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        af[tm] = *(const bf16x8*)(&As[buf][a_frag[tm] + kk * KK_STEP]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[tn], af[tm], acc[tm][tn],
                                                                0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < ACH; ++j) *(u32x4*)(&As[buf ^ 1][a_lds[j]]) = a_reg[j];
#pragma unroll
      for (int j = 0; j < WCH; ++j) *(u32x4*)(&Ws[buf ^ 1][w_lds[j]]) = w_reg[j];
    }
    __syncthreads();
  }

  const float* bptr = bias + (size_t)e * N;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int m = row0 + wm * 64 + tm * 32 + li;
    if (m >= row_end) continue;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      store_tile<EPI>(acc[tm][tn], bptr, out, m, n0 + wn * (BN / 2) + tn * 32 + lg * 4, N);
  }
}

// ==========================================================================
// wide tiled kernel: WBM activation rows x BN weight rows per workgroup
// ==========================================================================
// Each of the 4 waves (2 x 2) owns WBM/2 rows x BN/2 columns, i.e. WBM/64 x
// BN/64 MFMA tiles; with 256 x 256 a 16-wide k-step costs 8 fragment reads
// from LDS for 16 MFMAs (half the LDS traffic per MFMA of 128 x 128).
// Both operands are staged through XOR-swizzled, double-buffered LDS tiles
// (64 k per stage); the global loads run two chunks ahead in registers and
// the LDS fragment reads one k-step ahead of their MFMAs.  Loads and LDS
// staging are spread over the four k-steps: issued in one burst they held
// each chunk's first step up by several hundred ns.  256 x 256: one
// workgroup per CU (the accumulators fill the AGPRs); 128 x 128: two.
// AB: activation bytes per element, 2 (bf16) or 1 (E4M3 codes, widened to
// bf16 x *ascale when staged; a code quad occupies the low half of its slot).
template <int WBM, int BN, int EPI, bool PK, int OCC, int AB>
__global__ __launch_bounds__(256, OCC) void wide_gemm_kernel(
    const void* __restrict__ A, const uint16_t* __restrict__ W,
    const float* __restrict__ bias, void* __restrict__ out,
    const int32_t* __restrict__ offsets, int E, int N, int Kd,
    const int32_t* __restrict__ rowmap, const float* __restrict__ ascale) {
  constexpr int TM = WBM / 64;         // 32-row MFMA tiles per wave
  constexpr int TN = BN / 64;          // 32-column MFMA tiles per wave
  constexpr int AQ = WBM * 8 / 256;    // 16-byte quads per thread and chunk: activations
  constexpr int WQ = BN * 8 / 256;     // weights
  constexpr int NQ = AQ + WQ;
  constexpr int ASTG = WBM * 64;       // bf16 elements of one activation stage
  constexpr int STG = ASTG + BN * 64;  // one stage: activations, then weights
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STG];
  __shared__ TileInfo tinfo;

  const int tid = threadIdx.x;
  if (!find_tile<WBM, BN>(offsets, E, N, &tinfo, tid)) return;
  const int e = tinfo.e, row0 = tinfo.row0, row_end = tinfo.row_end, n0 = tinfo.n0;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int li = lane & 31, lg = lane >> 5;
  const int nk = Kd / 64;

  // staging: quad j of this thread is row (tid / 8) + 32 j, quad tid % 8 of
  // the chunk (packed weights: quad tid of the 4 KB block of strip j, copied
  // linearly).  Sources are 32-bit element offsets from per-tile bases;
  // chunk c adds c * 64 (activations, row-major weights) or c * PBLK.  The
  // swizzle of row r + 32 j equals that of r, so LDS slots step by 32 rows.
  // rowmap: the base is the token matrix and the offsets name token rows (the
  // host keeps its element count below 2^32)
  const uint16_t* abase = (const uint16_t*)A + (rowmap ? 0 : (size_t)row0 * Kd);
  const uint8_t* abase8 = (const uint8_t*)A + (rowmap ? 0 : (size_t)row0 * Kd);
  const float asc = AB == 1 ? *ascale : 0.0f;
  const uint16_t* wbase = PK ? W + ((size_t)e * (N / 32) + n0 / 32) * nk * PBLK
                             : W + ((size_t)e * N + n0) * Kd;
  const int sr = tid >> 3, sq = tid & 7;
  // (unsigned, so that the loads take a scalar base plus a 32-bit offset)
  uint32_t aoff[AQ];
#pragma unroll
  for (int j = 0; j < AQ; ++j) {
    const int row = min(row0 + sr + 32 * j, row_end - 1);
    aoff[j] = rowmap ? (uint32_t)rowmap[row] * (uint32_t)Kd + sq * 8
                     : (uint32_t)((row - row0) * Kd + sq * 8);
  }
  const uint32_t woff0 = PK ? tid * 8 : sr * Kd + sq * 8;
  const uint32_t wjstr = PK ? nk * PBLK : 32 * Kd;  // next quad of this thread
  const int adst = act_slot(sr, sq);
  const int wdst = PK ? ASTG + tid * 8 : ASTG + act_slot(sr, sq);
  constexpr int WDJ = PK ? PBLK : 32 * 64;     // LDS step of the next quad
  constexpr int WCSTR = PK ? PBLK : 64;

  // fragments at k-step 0; step s XORs (s << 3) (packed: k = 32 lg + 8 s)
  // or (2 s << 3) (row-major: k = 16 s + 8 lg) into the slot
  int afr[TM], wfr[TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
    afr[tm] = act_slot(wm * (WBM / 2) + tm * 32 + li, PK ? 4 * lg : lg);
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
    wfr[tn] = PK ? ASTG + (wn * TN + tn) * PBLK + lane * 8
                 : ASTG + act_slot(wn * (BN / 2) + tn * 32 + li, lg);
  constexpr int SSH = PK ? 3 : 4;          // slot XOR of step s: s << SSH
  constexpr int WSTEP = PK ? 512 : 0;      // packed weights: step s adds s * 512

  f32x16 acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.f;

  // activation quad at element offset `o`: 8 bf16, or 8 E4M3 codes in the
  // low half of the slot (widened when staged)
  auto load_act = [](const uint16_t* b16, const uint8_t* b8, uint32_t o) -> u32x4 {
    if constexpr (AB == 2) {
      (void)b8;
      return *(const u32x4*)(b16 + o);
    } else {
      (void)b16;
      const uint2 v = *(const uint2*)(b8 + o);
      return u32x4{v.x, v.y, 0u, 0u};
    }
  };
  auto widen_act = [](const u32x4& v, float scale) -> u32x4 {
    if constexpr (AB == 2) {
      (void)scale;
      return v;
    } else {
      return dequant8(v[0], v[1], scale);
    }
  };
  // global -> registers two chunks ahead; LDS fragments one k-step ahead
  u32x4 reg[2][NQ];
#define MOE_WIDE_LOAD(SLOT, c)                                                               \
  do {                                                                                       \
    _Pragma("unroll") for (int j = 0; j < AQ; ++j) reg[SLOT][j] =                            \
        load_act(abase, abase8, aoff[j] + (uint32_t)(c) * 64u);                              \
    _Pragma("unroll") for (int j = 0; j < WQ; ++j) reg[SLOT][AQ + j] =                       \
        *(const u32x4*)(wbase + (woff0 + j * wjstr + (uint32_t)(c) * WCSTR));                \
  } while (0)
#define MOE_WIDE_STORE(SLOT)                                                                 \
  do {                                                                                       \
    uint16_t* st_ = lds + (SLOT) * STG;                                                      \
    _Pragma("unroll") for (int j = 0; j < AQ; ++j) *(u32x4*)(st_ + adst + j * 32 * 64) =     \
        widen_act(reg[SLOT][j], asc);                                                        \
    _Pragma("unroll") for (int j = 0; j < WQ; ++j) *(u32x4*)(st_ + wdst + j * WDJ) =         \
        reg[SLOT][AQ + j];                                                                   \
  } while (0)
#define MOE_WIDE_FRAGS(B, st_, s4)                                                           \
  do {                                                                                       \
    _Pragma("unroll") for (int tm = 0; tm < TM; ++tm) fa[B][tm] =                            \
        *(const bf16x8*)((st_) + (afr[tm] ^ ((s4) << SSH)));                                 \
    _Pragma("unroll") for (int tn = 0; tn < TN; ++tn) fw[B][tn] =                            \
        *(const bf16x8*)((st_) + (PK ? wfr[tn] + (s4) * WSTEP : (wfr[tn] ^ ((s4) << SSH)))); \
  } while (0)
  // chunk c (in LDS stage and register slot SLOT = c & 1), per k-step: a
  // quarter of chunk c + 2's global loads into the slot, the next step's
  // fragment reads, this step's MFMAs, then a quarter of chunk c + 1's quads
  // into the other LDS buffer (nobody reads it until the barrier), so that
  // load issue and staging overlap the MFMAs; the scheduling barriers keep
  // that order.  In the steady-state loop REFILL and NEXT are compile-time
  // true: without branches the compiler waits only for chunk c + 1's loads
  // before staging them.
  constexpr int QPS = NQ / 4;  // quads staged per k-step
#define MOE_WIDE_CHUNK(SLOT, c, REFILL, NEXT)                                                \
  do {                                                                                       \
    const uint16_t* st = lds + (SLOT) * STG;                                                 \
    uint16_t* nst = lds + ((SLOT) ^ 1) * STG;                                                \
    MOE_WIDE_FRAGS(0, st, 0);                                                                \
    _Pragma("unroll") for (int s4 = 0; s4 < 4; ++s4) {                                       \
      if (REFILL) {                                                                          \
        _Pragma("unroll") for (int jj = 0; jj < QPS; ++jj) {                                 \
          const int j = s4 * QPS + jj;                                                       \
          if (j < AQ)                                                                        \
            reg[SLOT][j] = load_act(abase, abase8, aoff[j] + (uint32_t)((c) + 2) * 64u);     \
          else                                                                               \
            reg[SLOT][j] = *(const u32x4*)(wbase + (woff0 + (j - AQ) * wjstr +               \
                                                    (uint32_t)((c) + 2) * WCSTR));           \
        }                                                                                    \
      }                                                                                      \
      if (s4 < 3) MOE_WIDE_FRAGS((s4 + 1) & 1, st, s4 + 1);                                 \
      __builtin_amdgcn_sched_barrier(0);                                                     \
      _Pragma("unroll") for (int tm = 0; tm < TM; ++tm)                                      \
        _Pragma("unroll") for (int tn = 0; tn < TN; ++tn) acc[tm][tn] =                      \
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[s4 & 1][tn], fa[s4 & 1][tm],          \
                                                    acc[tm][tn], 0, 0, 0);                   \
      if (NEXT) {                                                                            \
        _Pragma("unroll") for (int jj = 0; jj < QPS; ++jj) {                                 \
          const int j = s4 * QPS + jj;                                                       \
          if (j < AQ)                                                                        \
            *(u32x4*)(nst + adst + j * 32 * 64) = widen_act(reg[(SLOT) ^ 1][j], asc);        \
          else                                                                               \
            *(u32x4*)(nst + wdst + (j - AQ) * WDJ) = reg[(SLOT) ^ 1][j];                     \
        }                                                                                    \
      }                                                                                      \
      __builtin_amdgcn_sched_barrier(0);                                                     \
    }                                                                                        \
    __syncthreads();                                                                         \
  } while (0)
  bf16x8 fa[2][TM], fw[2][TN];
  MOE_WIDE_LOAD(0, 0);
  if (nk > 1) MOE_WIDE_LOAD(1, 1);
  MOE_WIDE_STORE(0);
  __syncthreads();
  int c0 = 0;
  for (; c0 + 4 <= nk; c0 += 2) {
    MOE_WIDE_CHUNK(0, c0, true, true);
    MOE_WIDE_CHUNK(1, c0 + 1, true, true);
  }
  // tail: the last two or three chunks (c0 is even)
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int c = c0 + p;
    if (c < nk) MOE_WIDE_CHUNK(p & 1, c, c + 2 < nk, c + 1 < nk);
  }
#undef MOE_WIDE_CHUNK
#undef MOE_WIDE_LOAD
#undef MOE_WIDE_STORE
#undef MOE_WIDE_FRAGS

  const float* bptr = bias + (size_t)e * N;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int m = row0 + wm * (WBM / 2) + tm * 32 + li;
    if (m >= row_end) continue;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      store_tile<EPI>(acc[tm][tn], bptr, out, m, n0 + wn * (BN / 2) + tn * 32 + lg * 4, N);
  }
}

// ==========================================================================
// wide kernel with weights in registers: 256 activation rows x 256 weight rows
// ==========================================================================
// For the MFMA-bound shapes with packed weights.  Each of the 4 waves owns all
// 256 rows of the tile and 64 weight rows of its own (8 x 2 MFMA tiles, the
// 256 accumulator registers), so each weight fragment serves exactly one
// wave: it goes from global memory straight into a register ring PD chunks
// deep (one contiguous 1 KB load per fragment in the packed layout), and only
// the activations are staged through LDS (double-buffered, XOR-swizzled):
// per 16-wide k-step a wave reads 8 activation fragments for 16 MFMAs and no
// weight fragment from LDS.  Activations of chunk c + 1 are loaded while
// chunk c is computed and staged after its MFMAs; one barrier per chunk.
// The tile's weight rows beyond N (N % 256 != 0, N % 64 == 0) leave whole
// waves idle but present at the barriers.
// TM = 32-row sub-tiles that hold rows (8 for a whole tile; a partial last
// tile of up to 64 or 128 rows runs with 2 or 4: only those sub-tiles are
// staged, read and multiplied).
constexpr int W2_BM = 256, W2_BN = 256;
constexpr int W2_STAGE = W2_BM * 64;  // bf16 elements of one activation stage

template <int EPI, int AB, int TM>
__device__ __forceinline__ void wide2_tile(const void* __restrict__ A,
                                           const uint16_t* __restrict__ W,
                                           const float* __restrict__ bias,
                                           void* __restrict__ out, int N, int Kd,
                                           const int32_t* __restrict__ rowmap,
                                           const float* __restrict__ ascale, int e, int row0,
                                           int row_end, int n0, uint16_t* act) {
  constexpr int TN = 2, PD = 3, AQ = TM;  // AQ: activation quads per thread and chunk
  constexpr int STAGE = W2_STAGE;
  using AI = ActIn<AB>;
  using AV = typename AI::V;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, lg = lane >> 5;
  const int nk = Kd / 64;
  const int ncol = n0 + wave * 64;                          // this wave's first weight row
  const bool active = __builtin_amdgcn_readfirstlane(ncol < N ? 1 : 0) != 0;

  // weights: strip t of this wave, chunk c, k-step q at
  // wp + t * sstr + c * PBLK + q * 512 (lane's 8 elements)
  const uint16_t* wp = W + ((size_t)e * (N / 32) + (active ? ncol / 32 : 0)) * nk * PBLK + lane * 8;
  const uint32_t sstr = (uint32_t)nk * PBLK;
  u32x4 wr[PD][TN][4];

  // activations: quad j of this thread is row (tid >> 3) + 32 j, quad tid & 7
  const int sr = tid >> 3, sq = tid & 7;
  // byte offsets from a per-tile base (the token matrix when rowmap gathers:
  // the host keeps its byte count below 2^32)
  const char* abase = (const char*)A + (rowmap ? 0 : (size_t)row0 * Kd * AB);
  uint32_t aoff[AQ];
#pragma unroll
  for (int j = 0; j < AQ; ++j) {
    const int row = min(row0 + sr + 32 * j, row_end - 1);
    const uint32_t r = rowmap ? (uint32_t)rowmap[row] : (uint32_t)(row - row0);
    aoff[j] = (r * (uint32_t)Kd + sq * 8) * AB;
  }
  const int adst = act_slot(sr, sq);            // + 32 * 64 * j for quad j
  const float asc = AB == 1 ? *ascale : 0.0f;
  // fragment of k-step s for MFMA tile tm: row 32 tm + li, quad 4 lg + s
  const int fbase = li * 64, fsw = (li >> 1) & 7;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.f;

  // prologue: weights of chunks 0 .. PD-2, activations of chunk 0 -> LDS,
  // activations of chunk 1 in flight
  if (active) {
#pragma unroll
    for (int p = 0; p < PD - 1; ++p)
      if (p < nk)
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            wr[p][t][q] = __builtin_nontemporal_load(
                (const u32x4*)(wp + t * sstr + (uint32_t)p * PBLK + q * 512));
  }
  AV areg[AQ];
#pragma unroll
  for (int j = 0; j < AQ; ++j) areg[j] = *(const AV*)(abase + aoff[j]);
#pragma unroll
  for (int j = 0; j < AQ; ++j) *(u32x4*)(act + adst + j * 32 * 64) = AI::widen(areg[j], asc);
  if (nk > 1)
#pragma unroll
    for (int j = 0; j < AQ; ++j) areg[j] = *(const AV*)(abase + aoff[j] + 64u * AB);
  __syncthreads();

  // chunk c: weights of chunk c + PD - 1 into ring slot (SLOT + PD - 1) % PD,
  // per k-step 8 activation fragments then 16 MFMAs (weights from slot SLOT),
  // then chunk c + 1's activations into the other stage and chunk c + 2's
  // loads issued; one barrier.
#define MOE_W2_CHUNK(SLOT, c, REFILL, NEXT, NEXT2)                                          \
  do {                                                                                      \
    if (REFILL && active) {                                                                 \
      _Pragma("unroll") for (int t = 0; t < TN; ++t)                                        \
        _Pragma("unroll") for (int q = 0; q < 4; ++q)                                       \
          wr[((SLOT) + PD - 1) % PD][t][q] = __builtin_nontemporal_load(                    \
              (const u32x4*)(wp + t * sstr + (uint32_t)((c) + PD - 1) * PBLK + q * 512));   \
    }                                                                                       \
    const uint16_t* st_ = act + ((c) & 1) * STAGE;                                          \
    if (active) {                                                                           \
      bf16x8 xf[2][TM];                                                                     \
      _Pragma("unroll") for (int tm = 0; tm < TM; ++tm) xf[0][tm] =                         \
          *(const bf16x8*)(st_ + fbase + tm * 32 * 64 + (((4 * lg) ^ fsw) << 3));           \
      _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                       \
        if (s < 3) {                                                                        \
          _Pragma("unroll") for (int tm = 0; tm < TM; ++tm) xf[(s + 1) & 1][tm] =           \
              *(const bf16x8*)(st_ + fbase + tm * 32 * 64 +                                 \
                               (((4 * lg + s + 1) ^ fsw) << 3));                            \
        }                                                                                   \
        _Pragma("unroll") for (int tn = 0; tn < TN; ++tn) {                                 \
          const bf16x8 wa = __builtin_bit_cast(bf16x8, wr[SLOT][tn][s]);                    \
          _Pragma("unroll") for (int tm = 0; tm < TM; ++tm) acc[tm][tn] =                   \
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, xf[s & 1][tm], acc[tm][tn], 0, 0, \
                                                      0);                                   \
        }                                                                                   \
      }                                                                                     \
    }                                                                                       \
    if (NEXT) {                                                                             \
      uint16_t* nst_ = act + (((c) + 1) & 1) * STAGE;                                       \
      _Pragma("unroll") for (int j = 0; j < AQ; ++j)                                        \
        *(u32x4*)(nst_ + adst + j * 32 * 64) = AI::widen(areg[j], asc);                     \
    }                                                                                       \
    if (NEXT2) {                                                                            \
      _Pragma("unroll") for (int j = 0; j < AQ; ++j) areg[j] =                              \
          *(const AV*)(abase + aoff[j] + (uint32_t)((c) + 2) * 64u * AB);                   \
    }                                                                                       \
    __syncthreads();                                                                        \
  } while (0)

  int c0 = 0;
  for (; c0 + 2 * PD <= nk; c0 += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) MOE_W2_CHUNK(p, c0 + p, true, true, true);
  }
#pragma unroll
  for (int p = 0; p < 2 * PD; ++p) {
    const int c = c0 + p;
    if (c < nk) MOE_W2_CHUNK(p % PD, c, c + PD - 1 < nk, c + 1 < nk, c + 2 < nk);
  }
#undef MOE_W2_CHUNK

  if (!active) return;
  const float* bptr = bias + (size_t)e * N;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int m = row0 + tm * 32 + li;
    if (m >= row_end) continue;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      store_tile<EPI>(acc[tm][tn], bptr, out, m, ncol + tn * 32 + lg * 4, N);
  }
}

template <int EPI, int AB>
__global__ __launch_bounds__(256, 1) void wide2_gemm_kernel(
    const void* __restrict__ A, const uint16_t* __restrict__ W,
    const float* __restrict__ bias, void* __restrict__ out,
    const int32_t* __restrict__ offsets, int E, int N, int Kd,
    const int32_t* __restrict__ rowmap, const float* __restrict__ ascale) {
  __shared__ __attribute__((aligned(16))) uint16_t act[2 * W2_STAGE];
  __shared__ TileInfo tinfo;
  if (!find_tile_partial_last<W2_BM, W2_BN>(offsets, E, N, &tinfo, threadIdx.x)) return;
  const int e = tinfo.e, row0 = tinfo.row0, row_end = tinfo.row_end, n0 = tinfo.n0;
  const int rows = __builtin_amdgcn_readfirstlane(min(W2_BM, row_end - row0));
  if (rows > 128)
    wide2_tile<EPI, AB, 8>(A, W, bias, out, N, Kd, rowmap, ascale, e, row0, row_end, n0, act);
  else if (rows > 64)
    wide2_tile<EPI, AB, 4>(A, W, bias, out, N, Kd, rowmap, ascale, e, row0, row_end, n0, act);
  else
    wide2_tile<EPI, AB, 2>(A, W, bias, out, N, Kd, rowmap, ascale, e, row0, row_end, n0, act);
}

// ==========================================================================
// weight packing: row-major [E, N, K] -> fragment blocks (see file header)
// ==========================================================================
__global__ __launch_bounds__(256) void pack_weights_kernel(const u32x4* __restrict__ src,
                                                           u32x4* __restrict__ dst, int E,
                                                           int N, int Kd) {
  const int nchunks = Kd / 64;
  const int64_t nq = (int64_t)E * N * Kd / 8;   // 16-byte quads
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= nq) return;
  const int64_t blk = p >> 8;                   // 256 quads per block
  const int w = (int)(p & 255);
  const int q = w >> 6, l = w & 63;
  const int c = (int)(blk % nchunks);
  const int64_t t = blk / nchunks;              // e * (N/32) + 32-row tile
  const int nt = (int)(t % (N / 32));
  const int e = (int)(t / (N / 32));
  const int n = nt * 32 + (l & 31);
  const int k = c * 64 + (l >> 5) * 32 + q * 8;
  dst[p] = src[(((int64_t)e * N + n) * Kd + k) >> 3];
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
  // sequential fp32 FMAs over k; the loads of 8 k go out before their FMAs
  float acc = 0.f;
  int k = 0;
  for (; k + 8 <= Kd; k += 8) {
    float av[8], wv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      av[u] = a[k + u];
      wv[u] = w[k + u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = fmaf(av[u], wv[u], acc);
  }
  for (; k < Kd; ++k) acc = fmaf(a[k], w[k], acc);
  acc += bias[(size_t)e * N + n];
  out[(size_t)row * N + n] = (EPI == 0) ? gelu_tanh_f(acc) : acc;
}

// ---------------------------------------------------------------- launchers
// Upper bound of the tile count: sum_e ceil(rows_e / BM) <= r_max / BM + E,
// rounded up to whole XCD rounds.
int64_t grid_for(int64_t r_max, int BM, int E, int N, int BN) {
  int64_t g = (r_max / BM + E) * ((N + BN - 1) / BN);
  return (g + NXCD - 1) / NXCD * NXCD;
}

// Launch arguments shared by every GEMM shape.  A: activations (bf16, or
// E4M3 codes when the launcher's AB is 1, scaled by *ascale); rowmap: row r
// of the tile reads A[rowmap[r]] (the gather of the dispatch), or nullptr.
struct GemmArgs {
  const void* A;
  const uint16_t* W;
  const float* bias;
  void* out;
  const int32_t* offsets;
  int E, N, Kd;
  int64_t r_max;
  const int32_t* rowmap;
  const float* ascale;
  hipStream_t s;
};

template <int MT, int WN, int WK, int EPI, bool PK, int OCC, int AB, int TN = 1>
hipError_t launch_stream(const GemmArgs& g, bool static_map) {
  // static_map: every expert's rows fit one row tile (see the kernel)
  const int one_rt = static_map ? 1 : 0;
  const int64_t grid = one_rt ? ((int64_t)g.E * (g.N / (32 * WN * TN)) + NXCD - 1) / NXCD * NXCD
                              : grid_for(g.r_max, 32 * MT, g.E, g.N, 32 * WN * TN);
  hipLaunchKernelGGL((stream_gemm_kernel<MT, WN, WK, EPI, PK, OCC, AB, TN>), dim3((unsigned)grid),
                     dim3(256), 0, g.s, g.A, g.W, g.bias, g.out, g.offsets, g.E, g.N, g.Kd, one_rt,
                     g.rowmap, g.ascale);
  return hipGetLastError();
}

template <int MT, int WN, int WK, int EPI, bool PK, int AB>
hipError_t launch_stream_occ(const GemmArgs& g, bool occ1, bool static_map) {
  // built only for the tall tiles, where one workgroup per CU is the common case
  if constexpr (MT >= 4 && WN == 2)
    if (occ1) return launch_stream<MT, WN, WK, EPI, PK, 1, AB>(g, static_map);
  return launch_stream<MT, WN, WK, EPI, PK, 2, AB>(g, static_map);
}

template <int MT, int EPI, bool PK, int AB>
hipError_t launch_stream_mt(const GemmArgs& g, int wn, bool occ1, bool static_map, int tn) {
  if constexpr (MT <= 4) {
    // (four strips fit the registers with packed weights only)
    if constexpr (PK)
      if (tn == 4) return launch_stream<MT, 4, 1, EPI, PK, 1, AB, 4>(g, static_map);
    if (tn >= 2) return launch_stream<MT, 4, 1, EPI, PK, 1, AB, 2>(g, static_map);
  }
  if (wn == 4) return launch_stream_occ<MT, 4, 1, EPI, PK, AB>(g, occ1, static_map);
  // the 4-way k split keeps MT <= 3 (its reduction and ring outgrow the registers)
  if (wn == 2 || MT >= 4) return launch_stream_occ<MT, 2, 2, EPI, PK, AB>(g, occ1, static_map);
  if constexpr (MT < 4) return launch_stream_occ<MT, 1, 4, EPI, PK, AB>(g, occ1, static_map);
  return hipErrorInvalidValue;
}

template <int WBM, int BN, int EPI, bool PK, int OCC, int AB>
hipError_t launch_wide(const GemmArgs& g) {
  const int64_t grid = grid_for(g.r_max, WBM, g.E, g.N, BN);
  hipLaunchKernelGGL((wide_gemm_kernel<WBM, BN, EPI, PK, OCC, AB>), dim3((unsigned)grid),
                     dim3(256), 0, g.s, g.A, g.W, g.bias, g.out, g.offsets, g.E, g.N, g.Kd,
                     g.rowmap, g.ascale);
  return hipGetLastError();
}

template <int EPI, int AB>
hipError_t launch_wide2(const GemmArgs& g) {
  // whole and partial tiles are split over the XCDs separately, which can
  // take one workgroup per XCD more than their sum
  const int64_t grid = grid_for(g.r_max, W2_BM, g.E, g.N, W2_BN) + NXCD;
  hipLaunchKernelGGL((wide2_gemm_kernel<EPI, AB>), dim3((unsigned)grid), dim3(256), 0, g.s, g.A,
                     g.W, g.bias, g.out, g.offsets, g.E, g.N, g.Kd, g.rowmap, g.ascale);
  return hipGetLastError();
}

template <int BN, int EPI, bool PK>
hipError_t launch_tiled(const GemmArgs& g) {
  const int64_t grid = grid_for(g.r_max, TBM, g.E, g.N, BN);
  hipLaunchKernelGGL((tiled_gemm_kernel<BN, EPI, PK>), dim3((unsigned)grid), dim3(256), 0, g.s,
                     (const uint16_t*)g.A, g.W, g.bias, g.out, g.offsets, g.E, g.N, g.Kd,
                     g.rowmap);
  return hipGetLastError();
}

// Shape choice.  rows_typ = the rows a typical expert holds, min(capacity,
// ceil(A/E)); rows_max = min(capacity, A) bounds every expert.
//  - packed weights, rows_typ >= 512 (MFMA bound, long segments): the wide
//    kernel with weights in registers, both GEMMs (N a multiple of 64; the
//    waves of a last, partial weight tile idle).
//  - row-major weights, rows_typ >= 512, N % 256 == 0, first GEMM (N = F,
//    the long weight dim): wide kernel, 256 x 256 tiles.
//  - rows_typ >= 384, N % 128 == 0: wide kernel, 128 x 128 tiles, two
//    workgroups per CU (finer tiles quantise better over 256 CUs; for the
//    second GEMM they were as fast or faster than 256 x 256).
//  - rows_typ >= 384, other N (multiple of 64): tiled 128 x 64 kernel.
//  - else streaming, with the row tile covering every expert's rows when
//    rows_max <= 160 (each weight byte read once), else 128-row tiles; the
//    weight-tile width 32*WN is the widest that still gives >= 256
//    workgroups (one per CU), narrower ones split the k-chunk across waves.
//    Tiles of up to 128 rows take four weight strips per wave instead
//    (512-wide weight tiles, one workgroup per CU) with packed weights when
//    N is a multiple of 512 and that leaves at least 256 tiles, else two
//    (256-wide) under the same rule.
// Whether launch_gemm_auto takes a wide shape, whose loads address
// activations by 32-bit offsets (bytes with weights in registers, elements
// in the LDS-staged one).
bool takes_wide_shape(bool packed, bool first, int N, int64_t rows_typ) {
  return (packed && rows_typ >= 512) || (rows_typ >= 512 && N % 256 == 0 && first) ||
         (rows_typ >= 384 && N % 128 == 0);
}

// Whether the tiled shape serves this GEMM (it reads bf16 activations only).
bool takes_tiled_shape(int N, int64_t rows_typ) {
  return rows_typ >= 384 && N % 128 != 0;
}

template <int EPI, bool PK, int AB>
hipError_t launch_gemm_auto(const GemmArgs& g, int64_t rows_typ, int64_t rows_max) {
  const int E = g.E, N = g.N;
  if constexpr (PK)
    if (rows_typ >= 512) return launch_wide2<EPI, AB>(g);
  // the LDS-staged 256 x 256 tiles serve the first GEMM on row-major weights only
  if constexpr (EPI == 0 && !PK)
    if (rows_typ >= 512 && N % 256 == 0) return launch_wide<256, 256, EPI, PK, 1, AB>(g);
  if (rows_typ >= 384 && N % 128 == 0) return launch_wide<128, 128, EPI, PK, 2, AB>(g);
  if (rows_typ >= 384) {
    if constexpr (AB == 2) return launch_tiled<64, EPI, PK>(g);
    return hipErrorNotSupported;
  }
  int mt = (int)((rows_max + 31) / 32);
  if (mt > 5) mt = 4;
  if (mt < 1) mt = 1;
  // Static tile map when every expert fits one row tile and a typical
  // expert fills at least half of it: with many empty experts their
  // workgroups would prefetch weights for nothing.
  const bool one_rt = rows_max <= 32 * mt && 2 * rows_typ >= 32 * mt;
  const int64_t bm = 32 * mt;
  const int64_t mtiles = (g.r_max + bm - 1) / bm > E ? (g.r_max + bm - 1) / bm : E;
  int wn = 1;
  if (N % 128 == 0 && mtiles * (N / 128) >= 256) wn = 4;
  else if (mtiles * (N / 64) >= 256 || mt >= 4) wn = 2;
  // at most one workgroup of work per CU: build for occupancy 1 and prefetch deeper
  const bool occ1 = mtiles * (N / (32 * wn)) <= 256;
  // two or four weight strips per wave (256 or 512 weight rows per
  // workgroup, one workgroup per CU) where that still gives every CU a
  // workgroup
  int tn = 1;
  if (mt <= 4 && wn == 4) {
    if (PK && N % 512 == 0 && mtiles * (N / 512) >= 256) tn = 4;
    else if (N % 256 == 0 && mtiles * (N / 256) >= 256) tn = 2;
  }
  switch (mt) {
    case 1: return launch_stream_mt<1, EPI, PK, AB>(g, wn, occ1, one_rt, tn);
    case 2: return launch_stream_mt<2, EPI, PK, AB>(g, wn, occ1, one_rt, tn);
    case 3: return launch_stream_mt<3, EPI, PK, AB>(g, wn, occ1, one_rt, tn);
    case 4: return launch_stream_mt<4, EPI, PK, AB>(g, wn, occ1, one_rt, tn);
    default: return launch_stream_mt<5, EPI, PK, AB>(g, wn, occ1, one_rt, tn);
  }
}

// row_token != nullptr: xd is the token matrix x (x_rows rows) and row r's
// activations are x[row_token[r]].  GEMM1 gathers them in its own loads,
// except in a wide shape when x occupies 4 GiB or more (its loads take
// 32-bit offsets): then the rows are first copied into y's storage
// (R_max rows of h bf16 fit in the R_max x h fp32 of y), which GEMM1 reads
// before GEMM2 overwrites it.
template <bool PK>
hipError_t launch_ffn_bf16_t(const uint16_t* xd, const int32_t* row_token, int64_t x_rows,
                             const int32_t* offsets, const uint16_t* w1, const float* b1,
                             const uint16_t* w2, const float* b2, uint16_t* hbuf, float* y,
                             int E, int h, int F, int64_t A, int64_t cap, int64_t r_max,
                             hipStream_t s) {
  if (r_max == 0) return hipSuccess;
  const int64_t avg = (A + E - 1) / E;
  const int64_t rows_typ = avg < cap ? avg : cap;
  const int64_t rows_max = A < cap ? A : cap;
  if (row_token && takes_wide_shape(PK, true, F, rows_typ) &&
      x_rows * h * 2 > (int64_t)UINT32_MAX) {
    hipError_t err = launch_gather_rows(xd, row_token, offsets, E, (int64_t)h * 2, r_max, y, s);
    if (err != hipSuccess) return err;
    xd = (const uint16_t*)y;
    row_token = nullptr;
  }
  hipError_t err = launch_gemm_auto<0, PK, 2>(
      {xd, w1, b1, hbuf, offsets, E, F, h, r_max, row_token, nullptr, s}, rows_typ, rows_max);
  if (err != hipSuccess) return err;
  return launch_gemm_auto<1, PK, 2>({hbuf, w2, b2, y, offsets, E, h, F, r_max, nullptr, nullptr, s},
                                    rows_typ, rows_max);
}

// The expert FFN on the FP8 dispatch payload: GEMM1 reads the E4M3 codes of
// the dispatched rows and widens them to bf16 x scale as it stages them;
// GEMM2 is the bf16 one.  hipErrorNotSupported where GEMM1 would take the
// tiled shape.
template <bool PK>
hipError_t launch_ffn_fp8_t(const uint8_t* xq, const float* scale, const int32_t* offsets,
                            const uint16_t* w1, const float* b1, const uint16_t* w2,
                            const float* b2, uint16_t* hbuf, float* y, int E, int h, int F,
                            int64_t A, int64_t cap, int64_t r_max, hipStream_t s) {
  if (r_max == 0) return hipSuccess;
  const int64_t avg = (A + E - 1) / E;
  const int64_t rows_typ = avg < cap ? avg : cap;
  const int64_t rows_max = A < cap ? A : cap;
  hipError_t err = launch_gemm_auto<0, PK, 1>(
      {xq, w1, b1, hbuf, offsets, E, F, h, r_max, nullptr, scale, s}, rows_typ, rows_max);
  if (err != hipSuccess) return err;
  return launch_gemm_auto<1, PK, 2>({hbuf, w2, b2, y, offsets, E, h, F, r_max, nullptr, nullptr, s},
                                    rows_typ, rows_max);
}

}  // namespace

hipError_t launch_ffn_bf16(const uint16_t* xd, const int32_t* row_token, int64_t x_rows,
                           const int32_t* offsets, const uint16_t* w1, const float* b1,
                           const uint16_t* w2, const float* b2, uint16_t* hbuf, float* y, int E,
                           int h, int F, int64_t A, int64_t cap, int64_t r_max, bool packed,
                           hipStream_t s) {
  if (packed)
    return launch_ffn_bf16_t<true>(xd, row_token, x_rows, offsets, w1, b1, w2, b2, hbuf, y, E,
                                   h, F, A, cap, r_max, s);
  return launch_ffn_bf16_t<false>(xd, row_token, x_rows, offsets, w1, b1, w2, b2, hbuf, y, E, h,
                                  F, A, cap, r_max, s);
}

bool ffn_fp8_supported(int E, int F, int64_t A, int64_t cap, bool packed) {
  const int64_t avg = E > 0 ? (A + E - 1) / E : 0;
  const int64_t rows_typ = avg < cap ? avg : cap;
  if (packed && rows_typ >= 512) return true;  // weights in registers: any N % 64 == 0
  return !takes_tiled_shape(F, rows_typ);
}

hipError_t launch_ffn_fp8(const uint8_t* xq, const float* scale, const int32_t* offsets,
                          const uint16_t* w1, const float* b1, const uint16_t* w2,
                          const float* b2, uint16_t* hbuf, float* y, int E, int h, int F,
                          int64_t A, int64_t cap, int64_t r_max, bool packed, hipStream_t s) {
  if (packed)
    return launch_ffn_fp8_t<true>(xq, scale, offsets, w1, b1, w2, b2, hbuf, y, E, h, F, A, cap,
                                  r_max, s);
  return launch_ffn_fp8_t<false>(xq, scale, offsets, w1, b1, w2, b2, hbuf, y, E, h, F, A, cap,
                                 r_max, s);
}

hipError_t launch_pack_weights(const uint16_t* w, uint16_t* wp, int E, int N, int Kd,
                               hipStream_t s) {
  const int64_t nq = (int64_t)E * N * Kd / 8;
  if (nq == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, s,
                     (const u32x4*)w, (u32x4*)wp, E, N, Kd);
  return hipGetLastError();
}

hipError_t launch_ffn_f32(const float* xd, const int32_t* row_token, const int32_t* offsets,
                          const float* w1, const float* b1, const float* w2, const float* b2,
                          float* hbuf, float* y, int E, int h, int F, int64_t r_max,
                          hipStream_t s) {
  if (r_max == 0) return hipSuccess;
  if (row_token) {  // rows of x into y's storage first (read before GEMM2 writes y)
    hipError_t err = launch_gather_rows(xd, row_token, offsets, E, (int64_t)h * 4, r_max, y, s);
    if (err != hipSuccess) return err;
    xd = y;
  }
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
