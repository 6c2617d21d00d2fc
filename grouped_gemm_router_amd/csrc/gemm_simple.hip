// gemm_simple.hip -- general grouped GEMM on the vector ALUs (fp32 FMA).
//
// Same contract and device-side tile scheduler as the MFMA kernels ("Dense
// GEMM to TP MoE" §2.1-2.3: one launch, ragged M_i, sizes read on the GPU;
// "DeepGEMM walkthrough" §5.3: rows past the end of a group are masked), for
// the cases the MFMA kernels do not take: fp32 operands (exact fp32 products
// and fp32 accumulation) and shapes off the MFMA tile grid.  It is the path
// of the small fp32 layer, which is launch-bound.
//
// Tile 64 rows x 64 columns, K staged through LDS 16 at a time; each of the
// 256 threads accumulates a 4 x 4 patch (two with SwiGLU: gate and up).
#include "moe_internal.h"

namespace {

using namespace moe;

constexpr int SBM = 64, SBN = 64, SBK = 16;

template <int ESIZE>
__device__ __forceinline__ float ld(const void *p, size_t i) {
  if (ESIZE == 2) return bf16_bits_to_f32(static_cast<const uint16_t *>(p)[i]);
  return static_cast<const float *>(p)[i];
}

template <int ESIZE, int OSIZE, bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_simple_kernel(
    const void *__restrict__ A, const void *__restrict__ B, const void *__restrict__ B2,
    void *__restrict__ C, const int32_t *__restrict__ offsets, int G, int rows, int N, int K,
    int nt_count) {
  __shared__ int s_x[8];
  __shared__ float As[SBK][SBM + 1];
  __shared__ float Bs[SBK][SBN + 1];
  __shared__ float B2s[SWIGLU ? SBK : 1][SBN + 1];

  const int w = (int)blockIdx.x;
  const Sched sc = sched_lookup(offsets, G, rows, SBM, nt_count, kTileChunk, SWIGLU, s_x,
                                [w](int total) { return tile_of_workgroup(w, total); });
  if (sc.L < 0) return;
  const Tile tile = sc.tile;
  const int n0 = tile.nt * SBN;
  const size_t boff = (size_t)tile.g * N * K;

  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[4][4], acc2[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = acc2[i][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += SBK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int r = e / SBK, kk = e % SBK;
      const int m = tile.m0 + r, n = n0 + r, kg = k0 + kk;
      As[kk][r] = (m < tile.mend && kg < K) ? ld<ESIZE>(A, (size_t)m * K + kg) : 0.f;
      Bs[kk][r] = (n < N && kg < K) ? ld<ESIZE>(B, boff + (size_t)n * K + kg) : 0.f;
      if (SWIGLU) B2s[kk][r] = (n < N && kg < K) ? ld<ESIZE>(B2, boff + (size_t)n * K + kg) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < SBK; ++kk) {
      float a[4], b[4], b2[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b[j] = Bs[kk][tx + 16 * j];
        if (SWIGLU) b2[j] = B2s[kk][tx + 16 * j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if (SWIGLU) acc2[i][j] = fmaf(a[i], b2[j], acc2[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = tile.m0 + ty * 4 + i;
    if (m >= tile.mend) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n >= N) continue;
      float v = acc[i][j];
      if (SWIGLU) v = v / (1.0f + expf(-v)) * acc2[i][j];
      if (OSIZE == 2)
        static_cast<uint16_t *>(C)[(size_t)m * N + n] = f32_to_bf16_bits(v);
      else
        static_cast<float *>(C)[(size_t)m * N + n] = v;
    }
  }
}

template <int ESIZE, int OSIZE>
hipError_t launch_t(const void *A, const void *B, const void *B2, void *C, const int32_t *offsets,
                    int G, int rows, int N, int K, int epi, hipStream_t s) {
  const int nt = (N + SBN - 1) / SBN;
  const long long bound = (long long)host_row_tile_bound(rows, G, SBM) * nt;
  const dim3 grid((unsigned)((bound + 7) / 8 * 8)), block(256);
  if (epi == MOE_EPI_SWIGLU)
    hipLaunchKernelGGL((gemm_simple_kernel<ESIZE, OSIZE, true>), grid, block, 0, s, A, B, B2, C,
                       offsets, G, rows, N, K, nt);
  else
    hipLaunchKernelGGL((gemm_simple_kernel<ESIZE, OSIZE, false>), grid, block, 0, s, A, B, B2, C,
                       offsets, G, rows, N, K, nt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_simple(const void *A, const void *B, const void *B2, int ab_dt, void *C,
                              int c_dt, const int32_t *offsets, int G, int rows, int N, int K,
                              int epi, hipStream_t s) {
  if (ab_dt == MOE_BF16)
    return c_dt == MOE_BF16 ? launch_t<2, 2>(A, B, B2, C, offsets, G, rows, N, K, epi, s)
                            : launch_t<2, 4>(A, B, B2, C, offsets, G, rows, N, K, epi, s);
  return c_dt == MOE_BF16 ? launch_t<4, 2>(A, B, B2, C, offsets, G, rows, N, K, epi, s)
                          : launch_t<4, 4>(A, B, B2, C, offsets, G, rows, N, K, epi, s);
}
