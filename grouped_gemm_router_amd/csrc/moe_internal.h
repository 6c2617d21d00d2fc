// moe_internal.h -- device helpers and host launcher declarations shared by
// the HIP translation units of libmoe.so.  Written for gfx950 (CDNA4):
// 64-lane wavefronts, MFMA matrix cores, 160 KB of LDS per CU, 8 XCDs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte piece

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// binary32 -> bfloat16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// binary32 -> OCP E4M3FN, round to nearest even, saturating to +-448; the
// input's sign is kept (so tiny values give +0 / -0).  Normal results keep
// the top 3 mantissa bits and round on the 20 discarded ones; results below
// 2^-6 are multiples of 2^-9 and are rounded as an integer count of 2^-9.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                 // NaN in, NaN out
  if (a >= 0x43e00000u) return sign | 0x7eu;         // |v| >= 448
  if (a < 0x3c800000u) {                             // |v| < 2^-6
    float m = rintf(__uint_as_float(a) * 512.0f);    // exact scale, RNE
    return sign | (uint32_t)m;                       // m == 8 is 2^-6 (code 8)
  }
  uint32_t e = (a >> 23) - 127u + 7u;                // 1..15
  uint32_t r = (a >> 20) & 7u;
  uint32_t rem = a & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
  if (r == 8u) { r = 0; ++e; }
  return sign | (e << 3) | r;
}

// four values -> four packed E4M3 codes (byte i = value i) with
// v_cvt_pk_fp8_f32: round to nearest even, identical to f32_to_e4m3 for
// every value in [-448, 448] (checked on the device for all codes, all
// midpoints between neighbouring codes and 8M random values); callers scale
// into that range first
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// ---------------------------------------------------------------------------
// wavefront reductions (butterfly; every lane ends with the result, and the
// combination order is fixed, so results are deterministic)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// max over aligned groups of `width` lanes (width a power of two <= 64)
__device__ __forceinline__ float group_max(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---------------------------------------------------------------------------
// waits and barriers of the LDS-direct pipelines
// ---------------------------------------------------------------------------

// s_waitcnt vmcnt(N), leaving the other counters unconstrained (gfx9 layout:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int imm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
  __builtin_amdgcn_s_waitcnt(imm);
}

// s_waitcnt vmcnt(N) lgkmcnt(0): this wave's LDS reads are complete too
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  constexpr int imm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4);
  __builtin_amdgcn_s_waitcnt(imm);
}

// workgroup barrier without the release fence of __syncthreads(), which
// would drain every LDS-direct load still in flight; callers have already
// waited (vmcnt) for the loads the next stage reads
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

typedef __attribute__((address_space(3))) void lds_void;

// ---------------------------------------------------------------------------
// device-side group/tile scheduler shared by the grouped GEMM kernels.
//
// Each group g owns rows [o_g, o_g + M_g) with o_g the largest of
// clamp(offsets[h], 0, rows) over h <= g and M_g = o_{g+1} - o_g, so the
// groups never hold more than `rows` rows in all.  Group g is cut into
// mt_g = ceil(M_g / BM) row tiles and nt column tiles.  Groups are taken in
// index order, or (by_class) in three classes by size -- M_g > 128, then
// 64 < M_g <= 128, then the rest -- each class in index order: the tallest
// tiles first, so a launch of long tiles does not end on a round of them.
// Measured on the DeepSeek shapes (one 100-170 row tile per routed expert,
// the shared expert last): gate/up (K 7168) 1-2 % faster by class, the
// down projection (K 2048, short tiles) 3-4 % slower, so only the SwiGLU
// launches take the class order.  Inside a group the linear tile id
// walks chunks of `chunk` column tiles, and inside a chunk each row tile of
// the group across the chunk's column tiles in turn, so tiles that run at
// the same time share both weight columns and activation rows.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int sched_class(int m) { return m > 128 ? 0 : (m > 64 ? 1 : 2); }

// Exclusive scan over the 64 lanes of a wave; *total gets the sum.  DPP
// (no LDS round trips): a Hillis-Steele scan inside each row of 16 lanes
// (row_shr 1, 2, 4, 8; a lane whose source lies outside its row adds 0),
// then lane 15 of each row pair is added into the row above it (row_bcast15
// into rows 1 and 3) and lane 31 into the upper half (row_bcast31 into rows
// 2 and 3).  Must be called by a whole wave.
__device__ __forceinline__ int wave_exclusive_scan(int v, int *total) {
  int incl = v;
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xf, 0xf, false);  // row_shr:1
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xf, 0xf, false);  // row_shr:2
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xf, 0xf, false);  // row_shr:4
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xf, 0xf, false);  // row_shr:8
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x142, 0xa, 0xf, false);  // row_bcast:15
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x143, 0xc, 0xf, false);  // row_bcast:31
  *total = __builtin_amdgcn_readlane(incl, kWave - 1);
  return incl - v;
}

// Inclusive running maximum over the 64 lanes of a wave, for values >= 0
// (DPP as in wave_exclusive_scan; a lane without a source takes 0, the
// identity here).  Must be called by a whole wave.
__device__ __forceinline__ int wave_inclusive_max(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return v;
}

struct Tile {
  int g;     // group
  int m0;    // first row of the tile
  int mend;  // one past the last valid row of the tile (<= group end)
  int nt;    // column tile index
};

// Tile order.  Linear tile ids run group by group (size classes as above);
// inside a group, chunks of kTileChunk column tiles, and inside a chunk the
// column tiles fastest: all of the chunk's column tiles of row tile 0, then
// those of row tile 1, and so on.  Workgroup w takes tile w: the hardware
// deals consecutive workgroups to the 8 XCDs in turn, so XCD x takes column
// tiles x and x + 8 of every chunk for every row tile of the group -- its
// concurrent tiles share those columns' weights in its L2 -- and every XCD
// works on the same expert at the same time (the weights are then shared
// through the 256 MB MALL instead of 8 experts competing for it).  Measured
// on the Mixtral shapes against giving each XCD its own contiguous range of
// tiles: gate/up 2.00 -> 1.87 ms, down 1.23 -> 1.04 ms; against dealing each
// XCD 32 consecutive tiles of every round of 256 (two row tiles of 16
// columns): gate/up 1.72 -> 1.76 ms, with the same L2 hit count.
constexpr int kTileChunk = 16;

// Result of sched_lookup: the workgroup's tile, the tile count and the
// linear id that was looked up (-1: nothing to do).
struct Sched {
  Tile tile;
  int total;
  int L;
};

// The first wave's part of sched_lookup for runs of at most RUN groups per
// lane: each lane loads the offsets of its run (all loads unconditional,
// the index clamped to G, so that they are in flight at once -- a load under
// a lane condition gets its own wait), three DPP scans give every group its
// first tile id, and the lane whose run holds the picked id writes the tile.
template <int RUN, class Pick>
__device__ __forceinline__ void sched_wave(const int32_t *__restrict__ offsets, int G, int rows,
                                           int BM, int nt_count, int chunk, bool by_class,
                                           int *s_x, Pick pick) {
  const int lane = threadIdx.x;
  const int per = (G + kWave - 1) / kWave;
  const int g0 = lane * per;
  const int n = max(0, min(G, g0 + per) - g0);  // groups in this lane's run
  int o[RUN + 1];
#pragma unroll
  for (int i = 0; i <= RUN; ++i) o[i] = offsets[min(g0 + i, G)];
#pragma unroll
  for (int i = 0; i <= RUN; ++i) o[i] = (i <= n) ? min(max(o[i], 0), rows) : 0;
  // Make the clamped offsets non-decreasing (each becomes the largest
  // offset up to its group), so the groups' rows never add up to more than
  // `rows` and the tile count stays within host_row_tile_bound whatever the
  // array holds: a running maximum inside the run, then the maximum of the
  // runs of all lower lanes.
  int run_max = o[0];
#pragma unroll
  for (int i = 1; i <= RUN; ++i) {
    if (i <= n) {
      o[i] = max(o[i], o[i - 1]);
      run_max = o[i];
    }
  }
  {
    const int incl = wave_inclusive_max(run_max);
    int before = __shfl_up(incl, 1, kWave);
    if (lane == 0) before = 0;
#pragma unroll
    for (int i = 0; i <= RUN; ++i)
      if (i <= n) o[i] = max(o[i], before);
  }
  // row tiles of this lane's run, per class
  int t0 = 0, t1 = 0, t2 = 0;
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    if (i < n) {
      const int m = max(o[i + 1] - o[i], 0);
      const int c = by_class ? sched_class(m) : 0;
      const int t = (m + BM - 1) / BM;
      if (c == 0) t0 += t; else if (c == 1) t1 += t; else t2 += t;
    }
  }
  int T0, T1, T2;
  int q0 = wave_exclusive_scan(t0, &T0);
  int q1 = wave_exclusive_scan(t1, &T1) + T0;
  int q2 = wave_exclusive_scan(t2, &T2) + T0 + T1;
  const int total = (T0 + T1 + T2) * nt_count;
  const int L = pick(total);  // wave-uniform
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    if (i < n) {
      const int m = max(o[i + 1] - o[i], 0);
      const int c = by_class ? sched_class(m) : 0;
      const int t = (m + BM - 1) / BM;
      int at;
      if (c == 0) { at = q0; q0 += t; } else if (c == 1) { at = q1; q1 += t; } else { at = q2; q2 += t; }
      const int li = L - at * nt_count;  // tile id inside the group
      if (L >= 0 && li >= 0 && li < t * nt_count) {
        // chunks of `chunk` column tiles, column tiles fastest within a chunk
        const int per_chunk = chunk * t;
        const int ch = li / per_chunk;
        const int within = li - ch * per_chunk;
        const int cw = min(chunk, nt_count - ch * chunk);
        const int mt = within / cw;
        const int m0 = o[i] + mt * BM;
        s_x[0] = g0 + i;
        s_x[1] = m0;
        s_x[2] = min(o[i] + m, m0 + BM);
        s_x[3] = ch * chunk + (within - mt * cw);
      }
    }
  }
  if (lane == 0) {
    s_x[4] = total;
    s_x[5] = L;
  }
}

// The device tile scheduler.  Groups have clamped offsets o[g] =
// max over h <= g of min(max(offsets[h], 0), rows) (non-decreasing, at most
// rows) and m_g = o[g+1] - o[g] rows, cut
// into ceil(m_g / BM) row tiles of nt_count column tiles each; with
// by_class the groups are taken class by class (sched_class), in group order
// inside a class.  pick(total) maps the total tile count to the linear id
// this workgroup runs (or -1); the result holds that id's tile.
//
// The first wave alone does the work, in registers (sched_wave, compiled for
// a few run lengths: up to 64, 256, 512 and MOE_MAX_GROUPS groups), and
// writes the tile to s_x (8 ints of LDS); the block meets at one barrier.
// Must be called by all threads.
template <class Pick>
__device__ __forceinline__ Sched sched_lookup(const int32_t *__restrict__ offsets, int G, int rows,
                                              int BM, int nt_count, int chunk, bool by_class,
                                              int *s_x, Pick pick) {
  constexpr int kRun = (MOE_MAX_GROUPS + kWave - 1) / kWave;  // groups per lane at most
  if (threadIdx.x < kWave) {
    const int per = (G + kWave - 1) / kWave;  // wave-uniform
    if (per <= 1)
      sched_wave<1>(offsets, G, rows, BM, nt_count, chunk, by_class, s_x, pick);
    else if (per <= 4)
      sched_wave<4>(offsets, G, rows, BM, nt_count, chunk, by_class, s_x, pick);
    else if (per <= 8)
      sched_wave<8>(offsets, G, rows, BM, nt_count, chunk, by_class, s_x, pick);
    else
      sched_wave<kRun>(offsets, G, rows, BM, nt_count, chunk, by_class, s_x, pick);
  }
  __syncthreads();
  Sched r;
  r.tile.g = s_x[0];
  r.tile.m0 = s_x[1];
  r.tile.mend = s_x[2];
  r.tile.nt = s_x[3];
  r.total = s_x[4];
  r.L = s_x[5];
  return r;
}

// Linear tile id of workgroup w, or -1 for a workgroup with nothing to do.
__device__ __forceinline__ int tile_of_workgroup(int w, int total) { return w < total ? w : -1; }

// Upper bound on the number of row tiles over all groups, known on the host:
// sum_g ceil(M_g / BM) <= floor(rows / BM) + G.
inline int host_row_tile_bound(int rows, int G, int BM) { return rows / BM + G; }

}  // namespace moe

// ---------------------------------------------------------------------------
// host launchers (one per translation unit); return hipSuccess or an error.
// Arguments are validated by the C-ABI layer before these are called.
// ---------------------------------------------------------------------------

size_t route_ws_bytes(int T, int d, int E);

hipError_t launch_router_stats(const float *prob_sums, const int32_t *counts, int T, int E, int k,
                               float alpha, float *f, float *P, float *summary, hipStream_t s);
// prob_sums: [ceil(T/16)][E] per-block sums of the softmax probabilities, or null
hipError_t launch_route(const void *x, const void *w_router, int dt, const float *bias,
                        int T, int d, int E, int k, unsigned flags, float *logits,
                        int32_t *topk_idx, float *topk_w, float *prob_sums, float *ws,
                        hipStream_t s);

size_t permute_ws_bytes(int T, int k, int E);
// device address of moe_permute_noalloc's static scratch on the current
// device (MOE_PERMUTE_NOALLOC_SCRATCH_BYTES bytes)
hipError_t permute_noalloc_scratch(void **ptr);
// capacity: rows kept per expert (INT_MAX: drop-less); overflow and
// n_overflow may be null
hipError_t launch_permute(const void *x, int x_dt, int T, int d, const int32_t *topk_idx,
                          int k, int E, int n_shared, int capacity, int out_dt, void *x_perm,
                          float *x_perm_scale, int32_t *counts, int32_t *offsets,
                          int32_t *perm_src, int32_t *flat_to_row, int32_t *overflow,
                          int32_t *n_overflow, void *ws, hipStream_t s);

// Grouped GEMM launchers.  ldb: elements from one weight row (B, B2) to the
// next, >= K.  ws: the tail-split workspace of gemm_bf16_split_ws_bytes
// bytes, or null (no split); cus: compute units of the device the launch
// runs on.
hipError_t launch_gemm_bf16_mfma(const void *A, const void *B, const void *B2, void *C,
                                 int c_dt, const int32_t *offsets, int G, int rows, int N,
                                 int K, int ldb, int epi, void *ws, int cus, hipStream_t s);
bool gemm_bf16_mfma_supports(int N, int K, int epi);
size_t gemm_bf16_split_ws_bytes(int G, int rows, int N, int K, int epi, int cus);

hipError_t launch_gemm_simple(const void *A, const void *B, const void *B2, int ab_dt,
                              void *C, int c_dt, const int32_t *offsets, int G, int rows,
                              int N, int K, int ldb, int epi, hipStream_t s);

bool gemm_fp8_ring_supports(int rows, int N, int K, int ldb);
hipError_t launch_gemm_fp8_ring(const uint8_t *Aq, const float *As, const uint8_t *Bq,
                                const float *Bs, const uint8_t *B2q, const float *B2s, void *C,
                                int c_dt, float *C_scale, const int32_t *offsets, int G,
                                int rows, int N, int K, int ldb, int epi, hipStream_t s);
hipError_t launch_gemm_fp8(const uint8_t *Aq, const float *As, const uint8_t *Bq,
                           const float *Bs, const uint8_t *B2q, const float *B2s, void *C,
                           int c_dt, float *C_scale, const int32_t *offsets, int G, int rows,
                           int N, int K, int ldb, int epi, hipStream_t s);

hipError_t launch_combine(const void *Y, int y_dt, const int32_t *flat_to_row,
                          const float *topk_w, int T, int k, int d, int n_shared, void *out,
                          int out_dt, hipStream_t s);

hipError_t launch_quantize_fp8(const void *src, int src_dt, int R, int C, int br, int bc,
                               uint8_t *q, float *scale, hipStream_t s);
