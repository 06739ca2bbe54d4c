// FP8 (OCP E4M3) dispatch payload: the per-tensor scale and the receiver's
// dequantisation.
//
// Method: "MoE大模型专家并行与动态路由优化" 4.3 (FP8/INT8 communication
// quantisation): scale = max|x| / 448 over the bf16 hidden states, payload =
// (x / scale) as E4M3 (the quantising gather lives in dispatch.hip), and the
// receiver widens the codes back to bf16 and multiplies by the scale.  In bf16
// tensor arithmetic each quotient or product is formed in fp32 and rounded to
// bf16 once; the E4M3 rounding is to nearest, ties to even.
//
// amax: |x| of a finite bf16 value orders like its 15-bit pattern, so the
// maximum is taken on integers (order-independent, hence deterministic):
// per-block maxima, then one workgroup combines them and forms the scale.
#include "moe_internal.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void fp8_amax_kernel(const u32x4* __restrict__ x, int64_t nvec,
                                                       uint32_t* __restrict__ partial) {
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * 256) {
    const u32x4 v = x[i];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      m = max(m, v[q] & 0x7FFFu);
      m = max(m, (v[q] >> 16) & 0x7FFFu);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  __shared__ uint32_t wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    partial[blockIdx.x] = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
}

// scale = bf16(fp32(amax) / 448), stored as the fp32 value of that bf16
__global__ __launch_bounds__(256) void fp8_scale_kernel(const uint32_t* __restrict__ partial,
                                                        int nb, float* __restrict__ scale) {
  uint32_t m = 0;
  for (int b = threadIdx.x; b < nb; b += 256) m = max(m, partial[b]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  __shared__ uint32_t wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t amax_bits = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    const float amax = __uint_as_float(amax_bits << 16);
    *scale = __uint_as_float(bf16_rne_bits(__fdiv_rn(amax, 448.0f)) << 16);
  }
}

// x_disp[r] = bf16(value(code) * scale) for rows r < R = offsets[E]; the
// product of a 4-bit and an 8-bit significand is exact in fp32, so one
// rounding to bf16 follows.  One thread per 8 codes.
__global__ __launch_bounds__(256) void fp8_dequant_kernel(const uint2* __restrict__ xq,
                                                          const float* __restrict__ scale_p,
                                                          const int32_t* __restrict__ offsets,
                                                          int E, int vecs_per_row,
                                                          u32x4* __restrict__ xd) {
  const int64_t nvec = (int64_t)offsets[E] * vecs_per_row;
  const float scale = *scale_p;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * 256) {
    const uint2 c = xq[i];
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t w = p < 2 ? c.x : c.y;
      const uint32_t c0 = (w >> (16 * (p & 1))) & 0xFFu, c1 = (w >> (16 * (p & 1) + 8)) & 0xFFu;
      const uint32_t lo = bf16_rne_bits(e4m3_value(c0) * scale);
      const uint32_t hi = bf16_rne_bits(e4m3_value(c1) * scale);
      o[p] = lo | (hi << 16);
    }
    xd[i] = o;
  }
}

}  // namespace

hipError_t launch_fp8_scale(const uint16_t* x, int64_t n, float* scale, void* ws,
                            hipStream_t s) {
  const int64_t nvec = n / 8;
  int nb = (int)((nvec + 256 * 16 - 1) / (256 * 16));
  if (nb < 1) nb = 1;
  if (nb > kFp8AmaxBlocks) nb = kFp8AmaxBlocks;
  uint32_t* partial = (uint32_t*)ws;
  hipLaunchKernelGGL(fp8_amax_kernel, dim3(nb), dim3(256), 0, s, (const u32x4*)x, nvec,
                     partial);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(fp8_scale_kernel, dim3(1), dim3(256), 0, s, partial, nb, scale);
  return hipGetLastError();
}

hipError_t launch_fp8_dequantize(const uint8_t* xq, const float* scale, const int32_t* offsets,
                                 int E, int h, int64_t r_max, uint16_t* x_disp, hipStream_t s) {
  if (r_max == 0) return hipSuccess;
  const int vpr = h / 8;
  int64_t grid = (r_max * vpr + 255) / 256;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(fp8_dequant_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     (const uint2*)xq, scale, offsets, E, vpr, (u32x4*)x_disp);
  return hipGetLastError();
}

}  // namespace moe
