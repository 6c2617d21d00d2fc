// gemm_simple.hip -- grouped GEMM for fp32 operands (fp32 matrix cores) and
// for shapes off the bf16 MFMA tile grid (vector ALUs).
//
// Same contract and device-side tile scheduler as the MFMA kernels ("Dense
// GEMM to TP MoE" §2.1-2.3: one launch, ragged M_i, sizes read on the GPU;
// "DeepGEMM walkthrough" §5.3: rows past the end of a group are masked), for
// the cases the MFMA kernels do not take: fp32 operands (exact fp32 products
// and fp32 accumulation) and shapes off the MFMA tile grid.  It is the path
// of the small fp32 layer, which is launch-bound.
//
// Two kernels:
//   * fp32 operands, N % 32 == 0: the fp32 matrix cores
//     (v_mfma_f32_32x32x2_f32, fp32 products and sums).  A workgroup owns a
//     32 x 32 output tile (SwiGLU: 32 gate and the 32 matching up columns);
//     K moves through LDS 64 columns at a time (16-byte coalesced loads into
//     registers, the next chunk's issued before the current one is
//     multiplied; rows, columns and K past the end read as zero), each of the four
//     waves takes 16 of the 64 columns (8 MFMAs per operand), and the four
//     partial tiles are added in wave order through LDS before the epilogue.
//     32-row tiles keep the small fp32 layer's GEMMs (a few hundred rows)
//     spread over ~100-200 workgroups instead of 8-16.
//   * anything else (bf16 off the MFMA tile grid): 64 rows x 64 columns on
//     the vector ALUs, K staged through LDS 16 at a time; each of the 256
//     threads accumulates a 4 x 4 patch (two with SwiGLU: gate and up).
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
    int ldb, int nt_count) {
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
  const size_t boff = (size_t)tile.g * N * ldb;

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
      Bs[kk][r] = (n < N && kg < K) ? ld<ESIZE>(B, boff + (size_t)n * ldb + kg) : 0.f;
      if (SWIGLU) B2s[kk][r] = (n < N && kg < K) ? ld<ESIZE>(B2, boff + (size_t)n * ldb + kg) : 0.f;
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

// ---- fp32 on the matrix cores ----------------------------------------------
constexpr int FBM = 32, FBN = 32, FKC = 64, FPAD = FKC + 4;

template <bool SWIGLU, int OSIZE>
__global__ __launch_bounds__(256) void gemm_f32_mfma_kernel(
    const float *__restrict__ A, const float *__restrict__ B, const float *__restrict__ B2,
    void *__restrict__ C, const int32_t *__restrict__ offsets, int G, int rows, int N, int K,
    int ldb, int nt_count) {
  constexpr int NB = SWIGLU ? 2 : 1;  // B operands (gate, up)
  __shared__ int s_x[8];
  __shared__ float As[FBM][FPAD];
  __shared__ float Bs[NB * FBN][FPAD];
  __shared__ float red[4][NB][FBM][FBN + 1];
  const int w = (int)blockIdx.x;
  const Sched sc = sched_lookup(offsets, G, rows, FBM, nt_count, kTileChunk, SWIGLU, s_x,
                                [w](int total) { return tile_of_workgroup(w, total); });
  if (sc.L < 0) return;
  const Tile tile = sc.tile;
  const int n0 = tile.nt * FBN;
  const size_t boff = (size_t)tile.g * N * ldb;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x16{};
  // A chunk: 32 rows x 64 columns = 512 16-byte pieces, two per thread; B the
  // same per operand.  The next chunk's pieces are loaded into registers
  // while the current chunk is multiplied.
  float4 ra[2], rb[NB][2];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = i * 256 + tid, r = q / (FKC / 4), c = (q % (FKC / 4)) * 4;
      const int m = tile.m0 + r, kg = k0 + c;
      ra[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (m < tile.mend && kg < K) ra[i] = *reinterpret_cast<const float4 *>(A + (size_t)m * K + kg);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        rb[b][i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (kg < K)
          rb[b][i] = *reinterpret_cast<const float4 *>((b ? B2 : B) + boff + (size_t)(n0 + r) * ldb + kg);
      }
    }
  };
  load(0);
  for (int k0 = 0; k0 < K; k0 += FKC) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = i * 256 + tid, r = q / (FKC / 4), c = (q % (FKC / 4)) * 4;
      As[r][c] = ra[i].x; As[r][c + 1] = ra[i].y; As[r][c + 2] = ra[i].z; As[r][c + 3] = ra[i].w;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        Bs[b * FBN + r][c] = rb[b][i].x; Bs[b * FBN + r][c + 1] = rb[b][i].y;
        Bs[b * FBN + r][c + 2] = rb[b][i].z; Bs[b * FBN + r][c + 3] = rb[b][i].w;
      }
    }
    __syncthreads();
    if (k0 + FKC < K) load(k0 + FKC);
    // wave wv: columns 16 wv .. 16 wv + 15 of the chunk, two per MFMA (lane
    // l: row / column l % 32, column offset l / 32)
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const int kk = wv * 16 + st * 2 + (lane >> 5);
      const float a = As[lane & 31][kk];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, Bs[b * FBN + (lane & 31)][kk], acc[b], 0,
                                                       0, 0);
    }
    __syncthreads();
  }
  // 32x32 accumulator layout: lane holds column lane % 32, register r holds
  // row 8 (r / 4) + 4 (lane / 32) + r % 4
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      red[wv][b][8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)][lane & 31] = acc[b][r];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < FBM * FBN / 256; ++i) {
    const int q = i * 256 + tid, r = q / FBN, c = q % FBN;
    const int m = tile.m0 + r, n = n0 + c;
    float v = ((red[0][0][r][c] + red[1][0][r][c]) + red[2][0][r][c]) + red[3][0][r][c];
    if (SWIGLU) {
      const float u = ((red[0][1][r][c] + red[1][1][r][c]) + red[2][1][r][c]) + red[3][1][r][c];
      v = v / (1.0f + expf(-v)) * u;
    }
    if (m < tile.mend) {
      if (OSIZE == 2)
        static_cast<uint16_t *>(C)[(size_t)m * N + n] = f32_to_bf16_bits(v);
      else
        static_cast<float *>(C)[(size_t)m * N + n] = v;
    }
  }
}

template <int OSIZE>
hipError_t launch_f32_mfma(const void *A, const void *B, const void *B2, void *C,
                           const int32_t *offsets, int G, int rows, int N, int K, int ldb,
                           int epi, hipStream_t s) {
  const int nt = N / FBN;
  const long long bound = (long long)host_row_tile_bound(rows, G, FBM) * nt;
  const dim3 grid((unsigned)bound), block(256);
  const float *a = static_cast<const float *>(A), *b = static_cast<const float *>(B),
              *b2 = static_cast<const float *>(B2);
  if (epi == MOE_EPI_SWIGLU)
    hipLaunchKernelGGL((gemm_f32_mfma_kernel<true, OSIZE>), grid, block, 0, s, a, b, b2, C,
                       offsets, G, rows, N, K, ldb, nt);
  else
    hipLaunchKernelGGL((gemm_f32_mfma_kernel<false, OSIZE>), grid, block, 0, s, a, b, b2, C,
                       offsets, G, rows, N, K, ldb, nt);
  return hipGetLastError();
}

template <int ESIZE, int OSIZE>
hipError_t launch_t(const void *A, const void *B, const void *B2, void *C, const int32_t *offsets,
                    int G, int rows, int N, int K, int ldb, int epi, hipStream_t s) {
  const int nt = (N + SBN - 1) / SBN;
  const long long bound = (long long)host_row_tile_bound(rows, G, SBM) * nt;
  const dim3 grid((unsigned)((bound + 7) / 8 * 8)), block(256);
  if (epi == MOE_EPI_SWIGLU)
    hipLaunchKernelGGL((gemm_simple_kernel<ESIZE, OSIZE, true>), grid, block, 0, s, A, B, B2, C,
                       offsets, G, rows, N, K, ldb, nt);
  else
    hipLaunchKernelGGL((gemm_simple_kernel<ESIZE, OSIZE, false>), grid, block, 0, s, A, B, B2, C,
                       offsets, G, rows, N, K, ldb, nt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_simple(const void *A, const void *B, const void *B2, int ab_dt, void *C,
                              int c_dt, const int32_t *offsets, int G, int rows, int N, int K,
                              int ldb, int epi, hipStream_t s) {
  if (ab_dt == MOE_BF16)
    return c_dt == MOE_BF16 ? launch_t<2, 2>(A, B, B2, C, offsets, G, rows, N, K, ldb, epi, s)
                            : launch_t<2, 4>(A, B, B2, C, offsets, G, rows, N, K, ldb, epi, s);
  if (N % FBN == 0)
    return c_dt == MOE_BF16 ? launch_f32_mfma<2>(A, B, B2, C, offsets, G, rows, N, K, ldb, epi, s)
                            : launch_f32_mfma<4>(A, B, B2, C, offsets, G, rows, N, K, ldb, epi, s);
  return c_dt == MOE_BF16 ? launch_t<4, 2>(A, B, B2, C, offsets, G, rows, N, K, ldb, epi, s)
                          : launch_t<4, 4>(A, B, B2, C, offsets, G, rows, N, K, ldb, epi, s);
}
