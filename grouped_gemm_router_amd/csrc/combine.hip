// combine.hip -- gather the expert outputs back to token order, weight them
// by the gate and sum.
//
// "Dense GEMM to TP MoE" §2.2 step 6: gather back in the original order,
// multiply by the gate weight, sum.  "DeepGEMM walkthrough" §2.1: the shared
// expert is added with weight one.
//
// One workgroup per token.  Each thread owns 8 consecutive columns (one
// 16-byte bf16 piece, two for fp32; two such pieces at a time for fp32 Y):
// it issues the row loads of four terms at a time, accumulates in fp32 in
// ascending j with fused multiply-adds (the shared rows last, weight one),
// and stores once.  HBM traffic is one read of every used Y row and one
// write of out.
#include "moe_internal.h"

namespace {

using namespace moe;

template <int YSIZE>
__device__ __forceinline__ void load8(const void *base, size_t elem, float v[8]) {
  if (YSIZE == 2) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + elem);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + elem);
    const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + elem + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

constexpr int kMaxTerms = MOE_MAX_TOPK + 8;

template <int YSIZE, int OSIZE>
__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ Y,
                                                      const int32_t *__restrict__ flat_to_row,
                                                      const float *__restrict__ topk_w, int T,
                                                      int k, int d, int n_shared,
                                                      void *__restrict__ out) {
  __shared__ int s_row[kMaxTerms];
  __shared__ float s_w[kMaxTerms];
  const int t = blockIdx.x;
  const int nterm = k + n_shared;
  if (threadIdx.x < nterm) {
    const int j = threadIdx.x;
    if (j < k) {
      s_row[j] = flat_to_row[(size_t)t * k + j];
      s_w[j] = topk_w[(size_t)t * k + j];
    } else {
      s_row[j] = flat_to_row[(size_t)T * k + (size_t)(j - k) * T + t];
      s_w[j] = 1.0f;
    }
  }
  __syncthreads();
  const long long nrows = (long long)T * k + (long long)n_shared * T;
  const int npiece = d / 8;
  // PP column pieces per thread and round (p, p + blockDim.x, ...); terms in
  // groups of 4; all row loads of a group are issued before the first is
  // used, and accumulation stays in ascending j.  Two pieces for fp32 Y
  // (measured faster on the Mixtral shapes), one for bf16 Y (two measured
  // slower on the DeepSeek FP8 shapes: 0.12 -> 0.14 ms)
  constexpr int PP = YSIZE == 4 ? 2 : 1;
  for (int p0 = threadIdx.x; p0 < npiece; p0 += PP * blockDim.x) {
    float acc[PP][8];
#pragma unroll
    for (int h = 0; h < PP; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
    for (int j0 = 0; j0 < nterm; j0 += 4) {
      float v[PP][4][8];
#pragma unroll
      for (int h = 0; h < PP; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = j0 + q, p = p0 + h * blockDim.x;
          const int row = j < nterm ? s_row[j] : -1;
          if (p < npiece && row >= 0 && row < nrows) {  // else: dropped entry (or bad index)
            load8<YSIZE>(Y, (size_t)row * d + (size_t)p * 8, v[h][q]);
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[h][q][i] = 0.f;
          }
        }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + q;
        if (j >= nterm) break;
        const int row = s_row[j];
        if (row < 0 || row >= nrows) continue;
        const float w = j < k ? s_w[j] : 1.0f;
#pragma unroll
        for (int h = 0; h < PP; ++h)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            acc[h][i] = j < k ? fmaf(w, v[h][q][i], acc[h][i]) : acc[h][i] + v[h][q][i];
      }
    }
#pragma unroll
    for (int h = 0; h < PP; ++h) {
      const int p = p0 + h * blockDim.x;
      if (p >= npiece) break;
      if (OSIZE == 2) {
        uint4 o;
        o.x = f32_to_bf16_bits(acc[h][0]) | ((uint32_t)f32_to_bf16_bits(acc[h][1]) << 16);
        o.y = f32_to_bf16_bits(acc[h][2]) | ((uint32_t)f32_to_bf16_bits(acc[h][3]) << 16);
        o.z = f32_to_bf16_bits(acc[h][4]) | ((uint32_t)f32_to_bf16_bits(acc[h][5]) << 16);
        o.w = f32_to_bf16_bits(acc[h][6]) | ((uint32_t)f32_to_bf16_bits(acc[h][7]) << 16);
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + (size_t)t * d + (size_t)p * 8) = o;
      } else {
        float *o = static_cast<float *>(out) + (size_t)t * d + (size_t)p * 8;
        *reinterpret_cast<float4 *>(o) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        *reinterpret_cast<float4 *>(o + 4) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
      }
    }
  }
}

}  // namespace

hipError_t launch_combine(const void *Y, int y_dt, const int32_t *flat_to_row,
                          const float *topk_w, int T, int k, int d, int n_shared, void *out,
                          int out_dt, hipStream_t s) {
  const dim3 grid(T), block(d >= 2048 ? 256 : 64);
  if (y_dt == MOE_BF16 && out_dt == MOE_BF16)
    hipLaunchKernelGGL((combine_kernel<2, 2>), grid, block, 0, s, Y, flat_to_row, topk_w, T, k, d,
                       n_shared, out);
  else if (y_dt == MOE_BF16)
    hipLaunchKernelGGL((combine_kernel<2, 4>), grid, block, 0, s, Y, flat_to_row, topk_w, T, k, d,
                       n_shared, out);
  else if (out_dt == MOE_BF16)
    hipLaunchKernelGGL((combine_kernel<4, 2>), grid, block, 0, s, Y, flat_to_row, topk_w, T, k, d,
                       n_shared, out);
  else
    hipLaunchKernelGGL((combine_kernel<4, 4>), grid, block, 0, s, Y, flat_to_row, topk_w, T, k, d,
                       n_shared, out);
  return hipGetLastError();
}
