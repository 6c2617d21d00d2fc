// gemm_bf16.hip -- grouped GEMM on bf16 MFMA for gfx950, one launch over
// ragged groups.
//
// "DeepGEMM walkthrough" §4.2 (load tiles, multiply on the matrix cores,
// accumulate in registers, write back), §4.3 (many GEMMs of different M in
// one launch over an expert-contiguous layout), §5.2 (double-buffered shared
// memory), §5.3 (rows past a group's end are masked); "Dense GEMM to TP MoE"
// §2.1-2.3 (grouped, not batched: N and K shared, M_i ragged; expert sizes
// stay on the GPU).
//
// Design (CDNA4, 64-wide waves):
//   * workgroup = 256 threads (4 waves, 2 x 2), output tile 256 x 256, BK 64;
//     each wave owns a 128 x 128 sub-tile = 4 x 4 v_mfma_f32_32x32x16_bf16
//     blocks, 256 fp32 accumulators per lane (kept in AGPRs);
//   * A and B tiles are staged through LDS, double buffered (2 x 64 KB):
//     global loads of step k+1 are in flight while step k is multiplied;
//     rows are 128 B (8 pieces of 16 B) and piece c of row r is stored at
//     c ^ ((r >> 1) & 7), so the 16-lane phases of ds_read_b128 that read
//     one piece column of 16 rows hit 16 distinct bank groups;
//   * SwiGLU: the B tile holds 128 gate rows then the 128 matching up rows;
//     wave column wn multiplies gate rows [64 wn, +64) and up rows
//     [128 + 64 wn, +64), so the epilogue pairs silu(gate) * up in registers;
//   * the tile scheduler reads the device offsets array (no host round trip
//     of expert sizes), and the XCD-aware remap keeps tiles that share
//     weight columns / activation rows on one XCD (one L2);
//   * ragged tails: A rows past the group end are still loaded (clamped to
//     the buffer) and multiplied, but never stored.
#include "moe_internal.h"

namespace {

using namespace moe;

constexpr int BM = 256, BN = 256, BK = 64, NTH = 256;
constexpr int PIECES = BK / 8;               // 16-byte pieces per tile row
constexpr int TILE_PIECES = BM * PIECES;     // pieces per operand tile (2048)
constexpr int LOADS = TILE_PIECES / NTH;     // pieces per thread per operand (8)

__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row >> 1) & 7); }

// B-tile row of wave column wn, 32-row block nb
template <bool SWIGLU>
__device__ __forceinline__ int b_row(int wn, int nb) {
  return SWIGLU ? ((nb & 2) ? 128 : 0) + wn * 64 + (nb & 1) * 32 : wn * 128 + nb * 32;
}

template <bool SWIGLU, bool OUT_F32>
__global__ __launch_bounds__(NTH, 1) void gemm_bf16_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B,
    const uint16_t *__restrict__ B2, void *__restrict__ C, const int32_t *__restrict__ offsets,
    int G, int rows, int N, int K, int nt_count) {
  __shared__ u32x4 lds[2][2][TILE_PIECES];  // [stage][A, B][row * 8 + piece]
  __shared__ int s_cum[MOE_MAX_GROUPS + 1];
  __shared__ int s_tmp[4];

  sched_build<NTH>(offsets, G, rows, BM, s_cum, s_tmp);
  const int total = s_cum[G] * nt_count;
  const int L = xcd_remap(blockIdx.x, total);
  if (L < 0) return;
  const Tile tile = sched_tile(L, s_cum, G, offsets, rows, BM, nt_count, 8);

  const int tid = threadIdx.x;
  const int lane = lane_id(), wv = tid / kWave;
  const int wm = wv >> 1, wn = wv & 1;

  // per-thread global source pointers for the 8 A rows and 8 B rows it loads
  const int lrow = tid >> 3, lpc = tid & 7;  // rows lrow + 32 i, piece lpc
  const uint16_t *pa[LOADS];
  const uint16_t *pb[LOADS];
  const size_t goff = (size_t)tile.g * N * K;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int r = lrow + 32 * i;
    const int m = min(tile.m0 + r, rows - 1);
    pa[i] = A + (size_t)m * K + lpc * 8;
    if (SWIGLU) {
      const int n = tile.nt * 128 + (r & 127);
      pb[i] = (r < 128 ? B : B2) + goff + (size_t)n * K + lpc * 8;
    } else {
      const int n = tile.nt * 256 + r;
      pb[i] = B + goff + (size_t)n * K + lpc * 8;
    }
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  u32x4 ra[LOADS], rb[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    ra[i] = *reinterpret_cast<const u32x4 *>(pa[i]);
    rb[i] = *reinterpret_cast<const u32x4 *>(pb[i]);
  }
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int r = lrow + 32 * i;
    lds[0][0][r * PIECES + swz(r, lpc)] = ra[i];
    lds[0][1][r * PIECES + swz(r, lpc)] = rb[i];
  }
  __syncthreads();

  const int KT = K / BK;
  const int fr = lane & 31;    // row of the fragment this lane supplies
  const int fh = lane >> 5;    // which 8-wide k half of a 16-wide step
  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < KT) {
      const int k0 = (kt + 1) * BK;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        ra[i] = *reinterpret_cast<const u32x4 *>(pa[i] + k0);
        rb[i] = *reinterpret_cast<const u32x4 *>(pb[i] + k0);
      }
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int pc = ks * 2 + fh;
      bf16x8 a[4], b[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int r = wm * 128 + mi * 32 + fr;
        a[mi] = *reinterpret_cast<const bf16x8 *>(&lds[st][0][r * PIECES + swz(r, pc)]);
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int r = b_row<SWIGLU>(wn, nb) + fr;
        b[nb] = *reinterpret_cast<const bf16x8 *>(&lds[st][1][r * PIECES + swz(r, pc)]);
      }
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mi][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[nb], acc[mi][nb], 0, 0, 0);
    }
    if (kt + 1 < KT) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int r = lrow + 32 * i;
        lds[st ^ 1][0][r * PIECES + swz(r, lpc)] = ra[i];
        lds[st ^ 1][1][r * PIECES + swz(r, lpc)] = rb[i];
      }
    }
    __syncthreads();
  }

  // epilogue.  32x32 accumulator layout: lane holds column lane%32, and
  // register r holds row 8*(r/4) + 4*(lane/32) + r%4.
  const int col = lane & 31;
  const int rbase = 4 * (lane >> 5);
  if (SWIGLU) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = tile.m0 + wm * 128 + mi * 32 + 8 * (r >> 2) + rbase + (r & 3);
          if (m < tile.mend) {
            const int n = tile.nt * 128 + wn * 64 + nb * 32 + col;
            const float g = acc[mi][nb][r], u = acc[mi][nb + 2][r];
            const float h = g / (1.0f + expf(-g)) * u;
            if (OUT_F32)
              static_cast<float *>(C)[(size_t)m * N + n] = h;
            else
              static_cast<uint16_t *>(C)[(size_t)m * N + n] = f32_to_bf16_bits(h);
          }
        }
  } else {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = tile.m0 + wm * 128 + mi * 32 + 8 * (r >> 2) + rbase + (r & 3);
          if (m < tile.mend) {
            const int n = tile.nt * 256 + wn * 128 + nb * 32 + col;
            const float v = acc[mi][nb][r];
            if (OUT_F32)
              static_cast<float *>(C)[(size_t)m * N + n] = v;
            else
              static_cast<uint16_t *>(C)[(size_t)m * N + n] = f32_to_bf16_bits(v);
          }
        }
  }
}

}  // namespace

bool gemm_bf16_mfma_supports(int N, int K, int epi) {
  if (K % BK != 0 || K <= 0) return false;
  return epi == MOE_EPI_SWIGLU ? (N % 128 == 0) : (N % 256 == 0);
}

hipError_t launch_gemm_bf16_mfma(const void *A, const void *B, const void *B2, void *C, int c_dt,
                                 const int32_t *offsets, int G, int rows, int N, int K, int epi,
                                 hipStream_t s) {
  const int nt = epi == MOE_EPI_SWIGLU ? N / 128 : N / 256;
  const long long bound = (long long)host_row_tile_bound(rows, G, BM) * nt;
  const dim3 grid((unsigned)((bound + 7) / 8 * 8)), block(NTH);
  const uint16_t *a = static_cast<const uint16_t *>(A);
  const uint16_t *b = static_cast<const uint16_t *>(B);
  const uint16_t *b2 = static_cast<const uint16_t *>(B2);
  if (epi == MOE_EPI_SWIGLU) {
    if (c_dt == MOE_F32)
      hipLaunchKernelGGL((gemm_bf16_kernel<true, true>), grid, block, 0, s, a, b, b2, C, offsets,
                         G, rows, N, K, nt);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<true, false>), grid, block, 0, s, a, b, b2, C, offsets,
                         G, rows, N, K, nt);
  } else {
    if (c_dt == MOE_F32)
      hipLaunchKernelGGL((gemm_bf16_kernel<false, true>), grid, block, 0, s, a, b, b2, C, offsets,
                         G, rows, N, K, nt);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<false, false>), grid, block, 0, s, a, b, b2, C,
                         offsets, G, rows, N, K, nt);
  }
  return hipGetLastError();
}
