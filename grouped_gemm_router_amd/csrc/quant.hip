// quant.hip -- block FP8 (E4M3) quantisation of a matrix.
//
// "DeepGEMM walkthrough" §2.3 and §5.1: FP8 needs a scale per token, per
// group or per block, because one global scale crushes small values next to
// outliers.  For each block: s = absmax / 448 (1 for an all-zero block) and
// q = E4M3 round-to-nearest-even of (v / s), IEEE fp32 division, saturating.
//
// One workgroup (256 threads) per block; 16 threads x 8 values cover a
// 128-wide row piece, 16 row pieces per pass (one pass for 1 x 128 blocks,
// eight for 128 x 128).  absmax is a wave reduction followed by a 4-wave
// reduction in LDS.  This prepares weights once; activations are quantised
// inside the permutation and the gate/up GEMM epilogue instead.
#include "moe_internal.h"

namespace {

using namespace moe;

template <int ESIZE>
__device__ __forceinline__ void load8f(const void *src, size_t elem, float v[8]) {
  if (ESIZE == 2) {
    const uint4 raw = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src) + elem);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(src) + elem);
    const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(src) + elem + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// 128 x 128 blocks (br == 128) or 1 x 128 blocks (br == 1) over [R][C].
template <int ESIZE>
__global__ __launch_bounds__(256) void quant_kernel(const void *__restrict__ src, int R, int C,
                                                    int br, uint8_t *__restrict__ q,
                                                    float *__restrict__ scale) {
  __shared__ float s_red[4];
  const int nbc = C / 128;
  const int b = blockIdx.x;
  const int rb = b / nbc, cb = b % nbc;
  const int tid = threadIdx.x;
  const int col = cb * 128 + (tid & 15) * 8;  // 8 columns per thread
  const int r_in = tid >> 4;                  // 16 rows per pass
  const int passes = (br + 15) / 16;
  float amax = 0.f;
  for (int p = 0; p < passes; ++p) {
    const int r = p * 16 + r_in;
    if (r < br) {
      float v[8];
      load8f<ESIZE>(src, (size_t)(rb * br + r) * C + col, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) s_red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
  if (tid == 0) scale[(size_t)rb * nbc + cb] = sc;
  for (int p = 0; p < passes; ++p) {
    const int r = p * 16 + r_in;
    if (r < br) {
      float v[8];
      load8f<ESIZE>(src, (size_t)(rb * br + r) * C + col, v);
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3(v[i] / sc) << (8 * i);
#pragma unroll
      for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3(v[4 + i] / sc) << (8 * i);
      *reinterpret_cast<uint2 *>(q + (size_t)(rb * br + r) * C + col) = make_uint2(lo, hi);
    }
  }
}

}  // namespace

hipError_t launch_quantize_fp8(const void *src, int src_dt, int R, int C, int br, int bc,
                               uint8_t *q, float *scale, hipStream_t s) {
  (void)bc;
  const dim3 grid((R / br) * (C / 128)), block(256);
  if (src_dt == MOE_BF16)
    hipLaunchKernelGGL((quant_kernel<2>), grid, block, 0, s, src, R, C, br, q, scale);
  else
    hipLaunchKernelGGL((quant_kernel<4>), grid, block, 0, s, src, R, C, br, q, scale);
  return hipGetLastError();
}
