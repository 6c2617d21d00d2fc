// gemm_fp8.hip -- FP8 (E4M3) block-scaled grouped GEMM on gfx950 MFMA.
//
// "DeepGEMM walkthrough" §2.3: C ~ (A_q / scale_A)(B_q / scale_B) scale_C;
// §5.1: scales per token / group / block, woven into the GEMM, accumulation
// kept in fp32; §4.3 grouped GEMM over the expert-contiguous layout; §5.2
// double buffering; §5.3 masked tails.  Stored scales here are the
// dequantisation multipliers s (the reciprocal of the page's scale), so
//   C[r][n] = sum_kb sA[r][kb] * sB[g][n/128][kb] * (sum_{k in kb} Aq Bq).
//
// Design:
//   * workgroup = 256 threads (2 x 2 waves), tile 128 rows x 256 B-rows,
//     BK = 128 = the scale block, so one K step is one scale block;
//   * each wave owns 64 x 128 = 4 x 8 blocks of v_mfma_scale_f32_16x16x128
//     _f8f6f4 (E4M3 x E4M3, unit E8M0 scales): one instruction covers a whole
//     128-deep scale block, so its result P is exactly the inner sum and is
//     folded as acc += P * (sA[row] * sB) -- the promotion to fp32 happens
//     once per 128 K, on 4 values per lane per block;
//   * SwiGLU: B-tile rows 0..127 are 128 gate rows (one 128-row scale
//     block) and rows 128..255 the matching up rows; wave column wn takes
//     gate rows [64 wn, +64) and up rows [128 + 64 wn, +64);
//   * activation and output scales are stored group-major, [K/128][rows];
//   * E4M3 output: each output row's 128 h-columns of the tile are one
//     1 x 128 quantisation group; absmax over 16 lanes, then over the two
//     wave columns through LDS; s = absmax / 448; q = RNE(h / s).
#include "moe_internal.h"

namespace {

using namespace moe;

constexpr int FBM = 128, FBN = 256, FBK = 128, FNTH = 256;
constexpr int PIECES = FBK / 16;              // 16-byte pieces per tile row (8)
constexpr int A_PIECES = FBM * PIECES;        // 1024
constexpr int B_PIECES = FBN * PIECES;        // 2048
constexpr int A_LOADS = A_PIECES / FNTH;      // 4
constexpr int B_LOADS = B_PIECES / FNTH;      // 8

__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row >> 1) & 7); }

template <bool SWIGLU>
__device__ __forceinline__ int b_row16(int wn, int nb) {
  return SWIGLU ? ((nb & 4) ? 128 : 0) + wn * 64 + (nb & 3) * 16 : wn * 128 + nb * 16;
}

template <bool SWIGLU, bool OUT_FP8>
__global__ __launch_bounds__(FNTH, 1) void gemm_fp8_kernel(
    const uint8_t *__restrict__ Aq, const float *__restrict__ As, const uint8_t *__restrict__ Bq,
    const float *__restrict__ Bs, const uint8_t *__restrict__ B2q,
    const float *__restrict__ B2s, void *__restrict__ C, float *__restrict__ Cs,
    const int32_t *__restrict__ offsets, int G, int rows, int N, int K, int ldb, int nt_count) {
  __shared__ u32x4 lA[2][A_PIECES];
  __shared__ u32x4 lB[2][B_PIECES];
  __shared__ __attribute__((aligned(16))) float lS[2][FBM];
  __shared__ float s_amax[2][FBM];
  __shared__ int s_x[8];

  const int w = (int)blockIdx.x;
  const Sched sc = sched_lookup(offsets, G, rows, FBM, nt_count, kTileChunk, SWIGLU, s_x,
                                [w](int total) { return tile_of_workgroup(w, total); });
  if (sc.L < 0) return;
  const Tile tile = sc.tile;

  const int tid = threadIdx.x;
  const int lane = lane_id(), wv = tid / kWave;
  const int wm = wv >> 1, wn = wv & 1;
  const int KB = K / 128, NB = N / 128;

  // global sources: A rows lrow + 32 i (i < 4), B rows lrow + 32 i (i < 8)
  const int lrow = tid >> 3, lpc = tid & 7;
  const uint8_t *pa[A_LOADS];
  const uint8_t *pb[B_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int m = min(tile.m0 + lrow + 32 * i, tile.mend - 1);  // dead rows: the last row
    pa[i] = Aq + (size_t)m * K + lpc * 16;
  }
  const size_t goff = (size_t)tile.g * N * ldb;
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int r = lrow + 32 * i;
    int n;
    const uint8_t *base;
    if (SWIGLU) {
      n = tile.nt * 128 + (r & 127);
      base = r < 128 ? Bq : B2q;
    } else {
      n = min(tile.nt * 256 + r, N - 1);
      base = Bq;
    }
    pb[i] = base + goff + (size_t)n * ldb + lpc * 16;
  }
  // activation scale row handled by this thread (threads < 128)
  const int srow = min(tile.m0 + tid, tile.mend - 1);
  const float *psa = As + srow;  // [K/128][rows]
  // weight scales of this wave column: [g][n-block][kb]
  const float *psb;
  const float *psb2 = nullptr;
  if (SWIGLU) {
    psb = Bs + ((size_t)tile.g * NB + tile.nt) * KB;
    psb2 = B2s + ((size_t)tile.g * NB + tile.nt) * KB;
  } else {
    psb = Bs + ((size_t)tile.g * NB + min(tile.nt * 2 + wn, NB - 1)) * KB;
  }

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{};

  u32x4 ra[A_LOADS], rb[B_LOADS];
  float rs = 0.f;
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) ra[i] = *reinterpret_cast<const u32x4 *>(pa[i]);
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) rb[i] = *reinterpret_cast<const u32x4 *>(pb[i]);
  if (tid < FBM) rs = psa[0];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int r = lrow + 32 * i;
    lA[0][r * PIECES + swz(r, lpc)] = ra[i];
  }
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int r = lrow + 32 * i;
    lB[0][r * PIECES + swz(r, lpc)] = rb[i];
  }
  if (tid < FBM) lS[0][tid] = rs;
  __syncthreads();

  const int fr = lane & 15;    // fragment row
  const int fq = lane >> 4;    // which 32-byte quarter of the 128-byte row
  for (int kb = 0; kb < KB; ++kb) {
    const int st = kb & 1;
    if (kb + 1 < KB) {
      const int k0 = (kb + 1) * FBK;
#pragma unroll
      for (int i = 0; i < A_LOADS; ++i) ra[i] = *reinterpret_cast<const u32x4 *>(pa[i] + k0);
#pragma unroll
      for (int i = 0; i < B_LOADS; ++i) rb[i] = *reinterpret_cast<const u32x4 *>(pb[i] + k0);
      if (tid < FBM) rs = psa[(size_t)(kb + 1) * rows];
    }
    const float sb = psb[kb];
    const float sb2 = SWIGLU ? psb2[kb] : sb;
    i32x8 a[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int r = wm * 64 + mi * 16 + fr;
      const u32x4 lo = lA[st][r * PIECES + swz(r, 2 * fq)];
      const u32x4 hi = lA[st][r * PIECES + swz(r, 2 * fq + 1)];
      a[mi] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    // combined scale sA[row] * sB for the 4 rows this lane holds per m-block
    f32x4 sa[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      sa[mi] = *reinterpret_cast<const f32x4 *>(&lS[st][wm * 64 + mi * 16 + 4 * fq]);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const int r = b_row16<SWIGLU>(wn, nb) + fr;
      const u32x4 lo = lB[st][r * PIECES + swz(r, 2 * fq)];
      const u32x4 hi = lB[st][r * PIECES + swz(r, 2 * fq + 1)];
      const i32x8 b = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      const float s_n = (SWIGLU && (nb & 4)) ? sb2 : sb;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            a[mi], b, f32x4{}, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mi][nb][i] = fmaf(p[i], sa[mi][i] * s_n, acc[mi][nb][i]);
      }
    }
    if (kb + 1 < KB) {
#pragma unroll
      for (int i = 0; i < A_LOADS; ++i) {
        const int r = lrow + 32 * i;
        lA[st ^ 1][r * PIECES + swz(r, lpc)] = ra[i];
      }
#pragma unroll
      for (int i = 0; i < B_LOADS; ++i) {
        const int r = lrow + 32 * i;
        lB[st ^ 1][r * PIECES + swz(r, lpc)] = rb[i];
      }
      if (tid < FBM) lS[st ^ 1][tid] = rs;
    }
    __syncthreads();
  }

  // epilogue.  16x16 accumulator layout: lane holds column lane%16 and rows
  // 4*(lane/16) + i.
  const int col = lane & 15;
  if (SWIGLU) {
    float h[4][4][4];
    float rmax[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mx = 0.f;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const float g = acc[mi][nb][i], u = acc[mi][nb + 4][i];
          const float v = g / (1.0f + expf(-g)) * u;
          h[mi][nb][i] = v;
          mx = fmaxf(mx, fabsf(v));
        }
        rmax[mi][i] = mx;
      }
    if (OUT_FP8) {
      // row absmax: over the 16 lanes that share rows, then the 2 wave columns
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float mx = group_max(rmax[mi][i], 16);
          if (col == 0) s_amax[wn][wm * 64 + mi * 16 + 4 * fq + i] = mx;
        }
      __syncthreads();
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = wm * 64 + mi * 16 + 4 * fq + i;
        const int m = tile.m0 + rl;
        if (m >= tile.mend) continue;
        if (OUT_FP8) {
          const float amax = fmaxf(s_amax[0][rl], s_amax[1][rl]);
          const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int n = tile.nt * 128 + wn * 64 + nb * 16 + col;
            static_cast<uint8_t *>(C)[(size_t)m * N + n] = (uint8_t)f32_to_e4m3(h[mi][nb][i] / sc);
          }
          if (wn == 0 && col == 0) Cs[(size_t)tile.nt * rows + m] = sc;
        } else {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int n = tile.nt * 128 + wn * 64 + nb * 16 + col;
            static_cast<uint16_t *>(C)[(size_t)m * N + n] = f32_to_bf16_bits(h[mi][nb][i]);
          }
        }
      }
  } else {
    const int nbase = tile.nt * 256 + wn * 128;
    const bool live = nbase < N;  // a half tile past N (N % 256 == 128)
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = tile.m0 + wm * 64 + mi * 16 + 4 * fq + i;
        float sc = 1.0f;
        if (OUT_FP8) {
          float mx = 0.f;
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) mx = fmaxf(mx, fabsf(acc[mi][nb][i]));
          mx = group_max(mx, 16);
          sc = mx > 0.f ? mx / 448.0f : 1.0f;
        }
        if (m >= tile.mend || !live) continue;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          const int n = nbase + nb * 16 + col;
          if (OUT_FP8)
            static_cast<uint8_t *>(C)[(size_t)m * N + n] = (uint8_t)f32_to_e4m3(acc[mi][nb][i] / sc);
          else
            static_cast<uint16_t *>(C)[(size_t)m * N + n] = f32_to_bf16_bits(acc[mi][nb][i]);
        }
        if (OUT_FP8 && col == 0) Cs[(size_t)(tile.nt * 2 + wn) * rows + m] = sc;
      }
  }
}

}  // namespace

hipError_t launch_gemm_fp8(const uint8_t *Aq, const float *As, const uint8_t *Bq, const float *Bs,
                           const uint8_t *B2q, const float *B2s, void *C, int c_dt, float *C_scale,
                           const int32_t *offsets, int G, int rows, int N, int K, int ldb,
                           int epi, hipStream_t s) {
  const bool swiglu = epi == MOE_EPI_SWIGLU;
  const int nt = swiglu ? N / 128 : (N + 255) / 256;
  const long long bound = (long long)host_row_tile_bound(rows, G, FBM) * nt;
  const dim3 grid((unsigned)((bound + 7) / 8 * 8)), block(FNTH);
  const bool f8 = c_dt == MOE_E4M3;
  if (swiglu) {
    if (f8)
      hipLaunchKernelGGL((gemm_fp8_kernel<true, true>), grid, block, 0, s, Aq, As, Bq, Bs, B2q,
                         B2s, C, C_scale, offsets, G, rows, N, K, ldb, nt);
    else
      hipLaunchKernelGGL((gemm_fp8_kernel<true, false>), grid, block, 0, s, Aq, As, Bq, Bs, B2q,
                         B2s, C, C_scale, offsets, G, rows, N, K, ldb, nt);
  } else {
    if (f8)
      hipLaunchKernelGGL((gemm_fp8_kernel<false, true>), grid, block, 0, s, Aq, As, Bq, Bs, B2q,
                         B2s, C, C_scale, offsets, G, rows, N, K, ldb, nt);
    else
      hipLaunchKernelGGL((gemm_fp8_kernel<false, false>), grid, block, 0, s, Aq, As, Bq, Bs, B2q,
                         B2s, C, C_scale, offsets, G, rows, N, K, ldb, nt);
  }
  return hipGetLastError();
}
