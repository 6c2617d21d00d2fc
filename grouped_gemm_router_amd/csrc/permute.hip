// permute.hip -- per-expert histogram, exclusive prefix sum and stable
// scatter of tokens into expert-contiguous rows.
//
// "Dense GEMM to TP MoE" §2.2 steps 3-4: count the tokens of every expert,
// take the prefix sum to get each expert's offset in the permuted buffer,
// scatter the tokens there; §4.2: offsets = cumsum(counts) - counts.
// "DeepGEMM walkthrough" §4.3: tokens of one expert laid out contiguously
// turn expert compute into a list of contiguous GEMMs.
//
// Up to T*k = 32768 entries with bf16 / fp32 rows, one launch
// (perm_fused_kernel below: every workgroup histograms all entries itself,
// so none waits for another); beyond that, and for E4M3 rows (whose
// quantising copy needs more registers than a 1024-thread workgroup
// leaves), three launches.  All deterministic (counts are sums, ranks
// come from flat order, never from the order of atomics):
//   1. rank     one wave per block of 64 tokens: each lane (token) ORs its
//               k experts into a per-expert 64-bit LDS bitmap; the rank of
//               (t, j) inside the block is popcount(bitmap & lanes-below);
//               the block's count per expert is popcount(bitmap).
//               Ranks are parked in flat_to_row, counts in the workspace.
//   2. scan     one workgroup: per expert, exclusive prefix over blocks
//               (in place), then the exclusive prefix over experts of the
//               kept counts -> offsets (and of the dropped counts -> where
//               each expert's dropped entries start in the overflow list).
//               With a capacity ("Dense GEMM to TP MoE" §5.1: cap the
//               tokens per expert, excess to a fallback path) an expert
//               keeps its first `capacity` entries in flat order; the rest
//               get flat_to_row = -1 and are listed in `overflow`.
//   3. scatter  row = offsets[e] + block prefix + rank -> perm_src /
//               flat_to_row; then the
//               row copy: every source row is read once and stored to its k
//               destinations (plus the shared-expert rows), in 16-byte
//               pieces; with E4M3 output each 1 x 128 group is quantised
//               (absmax over 16 lanes, s = absmax / 448, RNE) on the way.
// Rows within an expert come out in ascending flat index t*k + j, exactly as
// a stable sort by expert id orders them.
#include <atomic>

#include "moe_internal.h"

namespace {

using namespace moe;

constexpr int kBlk = 64;  // tokens per rank block (one wave)

// ---- 1. rank ---------------------------------------------------------------
// KMAX >= k: a lane loads its token's k expert ids once, all loads
// unconditional (token and slot indices clamped into range) so that they
// are in flight together, and keeps them for both passes.
template <int KMAX>
__global__ __launch_bounds__(256) void perm_rank_kernel(const int32_t *__restrict__ idx, int T,
                                                        int k, int E, int nblk,
                                                        int32_t *__restrict__ blk_counts,
                                                        int32_t *__restrict__ flat_to_row) {
  extern __shared__ unsigned long long bits[];  // [4][E]
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  const int b = blockIdx.x * 4 + wv;
  unsigned long long *mine = bits + (size_t)wv * E;
  const int t = b * kBlk + lane;
  const bool live = (b < nblk) && (t < T);
  int ev[KMAX];
  const size_t row = (size_t)min(t, T - 1) * k;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) ev[j] = idx[row + min(j, k - 1)];
  for (int e = lane; e < E; e += kWave) mine[e] = 0ull;
  __syncthreads();
  if (live) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k && ev[j] >= 0 && ev[j] < E) atomicOr(&mine[ev[j]], 1ull << lane);
  }
  __syncthreads();
  if (live) {
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (j < k) {
        const int e = ev[j];
        int r = -1;
        if (e >= 0 && e < E) r = __popcll(mine[e] & below);
        flat_to_row[(size_t)t * k + j] = r;
      }
    }
  }
  if (b < nblk)
    for (int e = lane; e < E; e += kWave) blk_counts[(size_t)b * E + e] = __popcll(mine[e]);
}

// ---- 2. scan ---------------------------------------------------------------
// Thread e walks its expert's column of block counts 16 blocks at a time (the
// 16 loads are independent, so they are in flight together) and leaves the
// exclusive prefix over blocks in place; the exclusive prefix over experts
// becomes offsets.  The scatter adds the two.
// Exclusive prefix over the 1024 threads of v (fixed combination order);
// every thread gets its own prefix, and *total receives the sum.
__device__ __forceinline__ int block_excl_scan(int v, int *s_wave, int *total) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  int wave_total;
  const int incl = wave_exclusive_scan(v, &wave_total) + v;  // DPP, no LDS round trips
  if (lane == kWave - 1) s_wave[wv] = incl;
  __syncthreads();
  int base = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wv) base += s_wave[w];
    all += s_wave[w];
  }
  __syncthreads();  // s_wave is reused by the next scan
  *total = all;
  return base + incl - v;
}

// Each expert keeps at most `cap` rows (cap = INT_MAX: drop-less).
// offsets = exclusive prefix of the kept counts; ovf_start = exclusive
// prefix of the dropped counts (where each expert's dropped entries start
// in the overflow list); *n_overflow (if given) = all dropped entries.
// cnt [nblk][E] holds the block counts; blk [nblk][E] receives each block's
// exclusive prefix per expert (blk may be cnt itself).  Called by all 1024
// threads of the workgroup.
__device__ __forceinline__ void scan_blocks(int T, int E, int n_shared, int nblk, int cap,
                                            const int32_t *cnt, int32_t *__restrict__ blk,
                                            int32_t *__restrict__ counts,
                                            int32_t *__restrict__ offsets,
                                            int32_t *__restrict__ ovf_start,
                                            int32_t *__restrict__ n_overflow, int *s_wave,
                                            int *s_part, int *s_tot) {
  const int tid = threadIdx.x;
  // R threads per expert (thread r of expert e takes a contiguous run of
  // token blocks), so the per-block counts are read with many loads in
  // flight even when E is small
  const int R = max(1, min(1024 / E, nblk));
  const int e = tid % E, r = tid / E;
  const bool act = r < R && tid < R * E;
  const int per = (nblk + R - 1) / R;
  const int b_lo = min(nblk, r * per), b_hi = min(nblk, b_lo + per);
  int mine = 0;
  if (act) {
    for (int b0 = b_lo; b0 < b_hi; b0 += 16) {
      int c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = (b0 + i < b_hi) ? cnt[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) mine += c[i];
    }
    s_part[r * E + e] = mine;
  }
  __syncthreads();
  if (act) {
    // exclusive prefix of expert e over the runs before r, then the run's
    // blocks in order (the counts are read again)
    int run = 0;
    for (int q = 0; q < r; ++q) run += s_part[q * E + e];
    for (int b0 = b_lo; b0 < b_hi; b0 += 16) {
      int c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = (b0 + i < b_hi) ? cnt[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (b0 + i < b_hi) blk[(size_t)(b0 + i) * E + e] = run;
        run += c[i];
      }
    }
    if (r == R - 1) s_tot[e] = run;
  }
  __syncthreads();
  int total = 0;
  if (tid < E) {
    total = s_tot[tid];
    counts[tid] = total;
  }
  const int kept = min(total, cap);
  int routed, dropped;
  const int excl = block_excl_scan(kept, s_wave, &routed);
  const int oexcl = block_excl_scan(total - kept, s_wave, &dropped);
  if (tid < E) {
    offsets[tid] = excl;
    ovf_start[tid] = oexcl;
  }
  if (tid == 0) {
    offsets[E] = routed;
    for (int s = 0; s < n_shared; ++s) offsets[E + s + 1] = routed + (s + 1) * T;
    if (n_overflow) *n_overflow = dropped;
  }
}

__global__ __launch_bounds__(1024) void perm_scan_kernel(int T, int E, int n_shared, int nblk,
                                                         int cap, int32_t *__restrict__ blk,
                                                         int32_t *__restrict__ counts,
                                                         int32_t *__restrict__ offsets,
                                                         int32_t *__restrict__ ovf_start,
                                                         int32_t *__restrict__ n_overflow) {
  __shared__ int s_wave[16];
  __shared__ int s_part[1024];  // [r][E]: count of expert e over thread r's blocks
  __shared__ int s_tot[MOE_MAX_EXPERTS];
  scan_blocks(T, E, n_shared, nblk, cap, blk, blk, counts, offsets, ovf_start, n_overflow, s_wave,
              s_part, s_tot);
}

// ---- 3. scatter + row copy ----------------------------------------------------
// Maximum over each aligned group of 8 lanes, by DPP (no LDS round
// trips): swap neighbours (quad_perm 1,0,3,2), then pairs (quad_perm
// 2,3,0,1), then the two quads of the group (row_half_mirror).
__device__ __forceinline__ float group_max8(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                   0, __builtin_bit_cast(int, v), 0xb1, 0xf, 0xf, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                   0, __builtin_bit_cast(int, v), 0x4e, 0xf, 0xf, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                   0, __builtin_bit_cast(int, v), 0x141, 0xf, 0xf, false)));
  return v;
}

// Row copy of tokens [t0, t1): every source row is read once and stored to
// the rows in s_row ([(t1 - t0) * k], -1 = dropped) and to its shared-expert
// rows (shared_base + s*T + t), in 16-byte pieces; with E4M3 output each
// 1 x 128 group is quantised on the way.  Called by the whole workgroup
// after s_row is complete.
template <int ESIZE, bool QUANT>
__device__ __forceinline__ void copy_rows(const void *__restrict__ xv, int T, int d, int k,
                                          int n_shared, int t0, int t1, const int *s_row,
                                          size_t shared_base, void *__restrict__ x_perm,
                                          float *__restrict__ x_scale) {
  // scales are stored group-major, [d/128][rows], rows = T*k + n_shared*T
  const size_t srows = (size_t)T * (k + n_shared);
  const char *x = static_cast<const char *>(xv);
  if (!QUANT) {
    // 16-byte pieces; d * ESIZE is a multiple of 16
    const int cpr = d * ESIZE / 16;
    const int items = (t1 - t0) * cpr;
    uint4 *dst = static_cast<uint4 *>(x_perm);
    // U pieces per thread and round: all loads are issued before the first
    // store, so each thread keeps U reads in flight
    constexpr int U = 8;
    for (int it0 = threadIdx.x; it0 < items; it0 += U * blockDim.x) {
      uint4 v[U];
      int tt[U], c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int it = it0 + u * blockDim.x;
        tt[u] = it < items ? it / cpr : -1;
        c[u] = it - (it / cpr) * cpr;
        v[u] = tt[u] >= 0 ? reinterpret_cast<const uint4 *>(x + (size_t)(t0 + tt[u]) * d * ESIZE)[c[u]]
                          : uint4{0u, 0u, 0u, 0u};
      }
      for (int j = 0; j < k; ++j) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int row = tt[u] >= 0 ? s_row[tt[u] * k + j] : -1;
          if (row >= 0) dst[(size_t)row * cpr + c[u]] = v[u];
        }
      }
      for (int sh = 0; sh < n_shared; ++sh) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (tt[u] >= 0) dst[(shared_base + (size_t)sh * T + t0 + tt[u]) * cpr + c[u]] = v[u];
      }
    }
  } else {
    // one 1 x 128 group per 8 lanes, 16 elements (one 16-byte E4M3 store)
    // per lane
    const int gpr = d / 128;
    const int items = (t1 - t0) * gpr;
    const int lane8 = threadIdx.x & 7;
    uint8_t *dst = static_cast<uint8_t *>(x_perm);
    // every 8-lane group iterates the same number of times (the group max
    // below needs its whole group); each iteration takes HG groups (stride
    // apart) and issues all their loads before using any
    constexpr int HG = 8;
    const int stride = blockDim.x >> 3;
    const int rounds = (items + HG * stride - 1) / (HG * stride);
    for (int rd = 0; rd < rounds; ++rd) {
      float v[HG][16];
      int its[HG];
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        const int it = rd * HG * stride + h * stride + (threadIdx.x >> 3);
        its[h] = it;
        if (it < items) {
          const int tt = it / gpr, gi = it - tt * gpr;
          const size_t e0 = (size_t)(t0 + tt) * d + gi * 128 + lane8 * 16;
          if (ESIZE == 2) {
            const uint4 r0 = *reinterpret_cast<const uint4 *>(x + e0 * 2);
            const uint4 r1 = *reinterpret_cast<const uint4 *>(x + e0 * 2 + 16);
            const uint32_t w[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              v[h][2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
              v[h][2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float4 a = *reinterpret_cast<const float4 *>(x + e0 * 4 + 16 * i);
              v[h][4 * i] = a.x; v[h][4 * i + 1] = a.y; v[h][4 * i + 2] = a.z; v[h][4 * i + 3] = a.w;
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) v[h][i] = 0.f;
        }
      }
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        const int it = its[h];
        const bool ok = it < items;
        const int tt = ok ? it / gpr : 0, gi = ok ? it - tt * gpr : 0;
        const int t = t0 + tt;
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[h][i]));
        amax = group_max8(amax);
        const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
        // v / sc is at most 448 in magnitude, so the hardware conversion
        // gives exactly the codes of f32_to_e4m3
        const uint4 q = make_uint4(e4m3x4(v[h][0] / sc, v[h][1] / sc, v[h][2] / sc, v[h][3] / sc),
                                   e4m3x4(v[h][4] / sc, v[h][5] / sc, v[h][6] / sc, v[h][7] / sc),
                                   e4m3x4(v[h][8] / sc, v[h][9] / sc, v[h][10] / sc, v[h][11] / sc),
                                   e4m3x4(v[h][12] / sc, v[h][13] / sc, v[h][14] / sc, v[h][15] / sc));
        if (ok) {
          for (int j = 0; j < k + n_shared; ++j) {
            size_t row;
            if (j < k) {
              const int r = s_row[tt * k + j];
              if (r < 0) continue;
              row = (size_t)r;
            } else {
              row = shared_base + (size_t)(j - k) * T + t;
            }
            *reinterpret_cast<uint4 *>(dst + row * d + gi * 128 + lane8 * 16) = q;
            if (lane8 == 0) x_scale[(size_t)gi * srows + row] = sc;
          }
        }
      }
    }
  }
}

template <int ESIZE, bool QUANT>
__global__ __launch_bounds__(256) void perm_scatter_kernel(
    const void *__restrict__ xv, int T, int d, const int32_t *__restrict__ idx, int k, int E,
    int n_shared, int tpb, const int32_t *__restrict__ blk_base,
    const int32_t *__restrict__ offsets, int32_t *__restrict__ perm_src,
    int32_t *__restrict__ flat_to_row, void *__restrict__ x_perm, float *__restrict__ x_scale,
    int cap, const int32_t *__restrict__ ovf_start, int32_t *__restrict__ overflow) {
  extern __shared__ int s_row[];  // [tpb * k]
  const int t0 = blockIdx.x * tpb;
  const int t1 = min(t0 + tpb, T);
  const int nent = (t1 - t0) * k;
  // shared-expert rows follow the routed rows: row = offsets[E] + s*T + t
  const size_t shared_base = (size_t)offsets[E];
  for (int i = threadIdx.x; i < (t1 - t0) * n_shared; i += blockDim.x) {
    const int s = i / (t1 - t0), t = t0 + i % (t1 - t0);
    flat_to_row[(size_t)T * k + (size_t)s * T + t] = (int32_t)(shared_base + (size_t)s * T + t);
  }
  for (int i = threadIdx.x; i < nent; i += blockDim.x) {
    const size_t f = (size_t)t0 * k + i;
    const int e = idx[f];
    int row = -1;
    if (e >= 0 && e < E) {
      const int t = (int)(f / k);
      const int r = blk_base[(size_t)(t / kBlk) * E + e] + flat_to_row[f];  // rank in expert
      if (r < cap) {
        row = offsets[e] + r;
        perm_src[row] = (int32_t)f;
      } else if (overflow) {
        overflow[ovf_start[e] + (r - cap)] = (int32_t)f;
      }
    }
    flat_to_row[f] = row;
    s_row[i] = row;
  }
  __syncthreads();
  copy_rows<ESIZE, QUANT>(xv, T, d, k, n_shared, t0, t1, s_row, shared_base, x_perm, x_scale);
}


// ---- one launch: histogram + prefix + scatter (T k <= kFusedMaxEntries) ----
// Every workgroup counts all T*k entries itself (per-wave LDS bins, so no
// workgroup waits for another): the entries before its first token give each
// expert's rank base for its own tokens, all of them give the counts, and
// the exclusive prefix over experts of the kept counts gives the offsets
// (of the dropped counts, the overflow starts).  It then ranks its own
// entries in flat order, places them like the scatter kernel and copies its
// rows.  Workgroup 0 writes counts, offsets and n_overflow.  Each workgroup
// reads all of topk_idx (at most 128 KB, from L2), which is why the three
// launches above take over for larger T*k (measured on the DeepSeek shapes,
// T k = 32768: one launch 128 us against 130 us for the three).
constexpr int kFusedMaxEntries = 32768;
constexpr int kFusedThreads = 1024;  // 16 waves: the row copy needs loads in flight
// copies of the histogram bins per workgroup (thread i counts into copy
// i % copies): with few experts the LDS atomics of one instruction would
// otherwise meet on a handful of addresses; [copies][2][E] stays 8 KB
__host__ __device__ inline int fused_copies(int E) { return E <= 16 ? 64 : (E <= 256 ? 4 : 1); }

// exclusive prefix of v over the workgroup's kFusedThreads threads (fixed
// order); *total gets the sum
__device__ __forceinline__ int fused_excl_scan(int v, int *s_wave, int *total) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  int wt;
  const int ex = wave_exclusive_scan(v, &wt);
  if (lane == 0) s_wave[wv] = wt;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kFusedThreads / kWave; ++w) {
    if (w < wv) base += s_wave[w];
    all += s_wave[w];
  }
  __syncthreads();  // s_wave is reused by the next scan
  *total = all;
  return base + ex;
}

template <int ESIZE, bool QUANT>
__global__ __launch_bounds__(kFusedThreads) void perm_fused_kernel(
    const void *__restrict__ xv, int T, int d, const int32_t *__restrict__ idx, int k, int E,
    int n_shared, int tpb, int cap, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ perm_src, int32_t *__restrict__ flat_to_row, void *__restrict__ x_perm,
    float *__restrict__ x_scale, int32_t *__restrict__ overflow,
    int32_t *__restrict__ n_overflow) {
  constexpr int NW = kFusedThreads / kWave;
  extern __shared__ int s_mem[];
  // bins: cp copies of [2][E] (entries before t0, entries from t0 on)
  const int cp = fused_copies(E);
  int *bins = s_mem;
  int *s_base = bins + cp * 2 * E;       // [E] entries of expert e before t0
  int *s_off = s_base + E;               // [E] offsets
  int *s_ovf = s_off + E;                // [E] overflow starts
  int *s_e = s_ovf + E;                  // [tpb * k] the workgroup's expert ids
  int *s_row = s_e + tpb * k;            // [tpb * k] their rows
  __shared__ int s_wave[NW];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * tpb;
  const int t1 = min(t0 + tpb, T);
  const int nent = (t1 - t0) * k;
  const int nall = T * k, nbefore = t0 * k;
  for (int i = tid; i < cp * 2 * E; i += kFusedThreads) bins[i] = 0;
  for (int i = tid; i < nent; i += kFusedThreads) s_e[i] = idx[(size_t)nbefore + i];
  __syncthreads();
  int *mb = bins + (tid % cp) * 2 * E;
  auto count = [&](int f, int e) {
    if (e >= 0 && e < E) atomicAdd(&mb[(f < nbefore ? 0 : E) + e], 1);
  };
  // histogram of all entries: 16-byte loads (four entries) when idx is
  // 16-byte aligned, up to sixteen of them in flight per thread
  int done = 0;
  if ((reinterpret_cast<uintptr_t>(idx) & 15) == 0) {
    const int ng = nall / 4;
    const int4 *idx4 = reinterpret_cast<const int4 *>(idx);
    for (int g0 = tid; g0 < ng; g0 += 16 * kFusedThreads) {
      int4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = idx4[min(g0 + u * kFusedThreads, ng - 1)];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int g = g0 + u * kFusedThreads;
        if (g < ng) {
          count(4 * g, v[u].x);
          count(4 * g + 1, v[u].y);
          count(4 * g + 2, v[u].z);
          count(4 * g + 3, v[u].w);
        }
      }
    }
    done = 4 * ng;
  }
  for (int f0 = done + tid; f0 < nall; f0 += 8 * kFusedThreads) {
    int ev[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) ev[u] = idx[min(f0 + u * kFusedThreads, nall - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (f0 + u * kFusedThreads < nall) count(f0 + u * kFusedThreads, ev[u]);
  }
  __syncthreads();
  // thread i owns experts [i * per, i * per + per): totals, kept and dropped
  const int per = (E + kFusedThreads - 1) / kFusedThreads;
  const int e_lo = min(E, tid * per), e_hi = min(E, e_lo + per);
  int kept_sum = 0, drop_sum = 0;
  for (int e = e_lo; e < e_hi; ++e) {
    int before = 0, after = 0;
    for (int w = 0; w < cp; ++w) {
      before += bins[w * 2 * E + e];
      after += bins[w * 2 * E + E + e];
    }
    const int total = before + after;
    s_base[e] = before;
    s_off[e] = total;  // the total, until the prefix below replaces it
    kept_sum += min(total, cap);
    drop_sum += total - min(total, cap);
  }
  int routed, dropped;
  int ko = fused_excl_scan(kept_sum, s_wave, &routed);
  int dro = fused_excl_scan(drop_sum, s_wave, &dropped);
  for (int e = e_lo; e < e_hi; ++e) {
    const int total = s_off[e], kept = min(total, cap);
    if (blockIdx.x == 0) {
      counts[e] = total;
      offsets[e] = ko;
    }
    s_off[e] = ko;
    s_ovf[e] = dro;
    ko += kept;
    dro += total - kept;
  }
  if (blockIdx.x == 0 && tid == 0) {
    offsets[E] = routed;
    for (int sh = 0; sh < n_shared; ++sh) offsets[E + sh + 1] = routed + (sh + 1) * T;
    if (n_overflow) *n_overflow = dropped;
  }
  __syncthreads();
  // the workgroup's own entries: rank = entries of the same expert before
  // t0, plus those before it in flat order inside the workgroup
  const size_t shared_base = (size_t)routed;
  for (int i = tid; i < (t1 - t0) * n_shared; i += kFusedThreads) {
    const int sh = i / (t1 - t0), t = t0 + i % (t1 - t0);
    flat_to_row[(size_t)T * k + (size_t)sh * T + t] = (int32_t)(shared_base + (size_t)sh * T + t);
  }
  for (int i = tid; i < nent; i += kFusedThreads) {
    const int e = s_e[i];
    const size_t f = (size_t)nbefore + i;
    int row = -1;
    if (e >= 0 && e < E) {
      int r = s_base[e];
      for (int j = 0; j < i; ++j) r += s_e[j] == e;
      if (r < cap) {
        row = s_off[e] + r;
        perm_src[row] = (int32_t)f;
      } else if (overflow) {
        overflow[s_ovf[e] + (r - cap)] = (int32_t)f;
      }
    }
    flat_to_row[f] = row;
    s_row[i] = row;
  }
  __syncthreads();
  copy_rows<ESIZE, QUANT>(xv, T, d, k, n_shared, t0, t1, s_row, shared_base, x_perm, x_scale);
}

// Library-owned scratch of moe_permute_noalloc (the per-block counts and
// overflow starts that moe_permute keeps in its workspace), one copy per GPU
// the library runs on, held until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the
// symbol): permute_noalloc_scratch looks up its device address.
static __device__ __align__(256) unsigned char scratch[MOE_PERMUTE_NOALLOC_SCRATCH_BYTES];

}  // namespace

// Device address of `scratch` on the current device.  The first call on a
// device asks the runtime (hipGetSymbolAddress, with that device current)
// and keeps the address per device; later calls reuse it.  No allocation.
hipError_t permute_noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void *> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    void *p = cache[dev].load(std::memory_order_acquire);
    if (p != nullptr) {
      *ptr = p;
      return hipSuccess;
    }
  }
  void *p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (cached) cache[dev].store(p, std::memory_order_release);
  *ptr = p;
  return hipSuccess;
}

size_t permute_ws_bytes(int T, int k, int E) {
  (void)k;
  if (T <= 0) return 0;
  const size_t nblk = ((size_t)T + kBlk - 1) / kBlk;
  return (nblk + 1) * (size_t)E * sizeof(int32_t);  // block counts, then overflow starts
}

namespace {
hipError_t launch_scatter(const void *x, int x_dt, int T, int d, const int32_t *topk_idx, int k,
                          int E, int n_shared, int capacity, int out_dt, void *x_perm,
                          float *x_perm_scale, int32_t *offsets, int32_t *perm_src,
                          int32_t *flat_to_row, int32_t *overflow, int32_t *blk,
                          int32_t *ovf_start, hipStream_t s);
}  // namespace

hipError_t launch_permute(const void *x, int x_dt, int T, int d, const int32_t *topk_idx, int k,
                          int E, int n_shared, int capacity, int out_dt, void *x_perm,
                          float *x_perm_scale, int32_t *counts, int32_t *offsets,
                          int32_t *perm_src, int32_t *flat_to_row, int32_t *overflow,
                          int32_t *n_overflow, void *ws, hipStream_t s) {
  if ((long long)T * k <= kFusedMaxEntries && out_dt != MOE_E4M3) {
    // tokens per workgroup: 16 once there are 256 workgroups' worth, fewer
    // below (one per workgroup under 512 tokens)
    const int tpb = max(1, min(16, T / 256));
    const dim3 grid((T + tpb - 1) / tpb), block(kFusedThreads);
    const size_t lds = sizeof(int) * ((size_t)fused_copies(E) * 2 * E + 3 * (size_t)E +
                                      2 * (size_t)tpb * k);
#define MOE_FUSED(ES)                                                                        \
  hipLaunchKernelGGL((perm_fused_kernel<ES, false>), grid, block, lds, s, x, T, d, topk_idx, k, \
                     E, n_shared, tpb, capacity, counts, offsets, perm_src, flat_to_row, x_perm, \
                     x_perm_scale, overflow, n_overflow)
    if (x_dt == MOE_BF16) MOE_FUSED(2);
    else MOE_FUSED(4);
#undef MOE_FUSED
    return hipGetLastError();
  }
  const int nblk = (T + kBlk - 1) / kBlk;
  int32_t *blk = static_cast<int32_t *>(ws);
  int32_t *ovf_start = blk + (size_t)nblk * E;
  const size_t rank_lds = sizeof(unsigned long long) * 4 * (size_t)E;
  if (k <= 2)
    hipLaunchKernelGGL(perm_rank_kernel<2>, dim3((nblk + 3) / 4), dim3(256), rank_lds, s,
                       topk_idx, T, k, E, nblk, blk, flat_to_row);
  else if (k <= 8)
    hipLaunchKernelGGL(perm_rank_kernel<8>, dim3((nblk + 3) / 4), dim3(256), rank_lds, s,
                       topk_idx, T, k, E, nblk, blk, flat_to_row);
  else
    hipLaunchKernelGGL(perm_rank_kernel<MOE_MAX_TOPK>, dim3((nblk + 3) / 4), dim3(256), rank_lds,
                       s, topk_idx, T, k, E, nblk, blk, flat_to_row);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, s, T, E, n_shared, nblk, capacity,
                     blk, counts, offsets, ovf_start, n_overflow);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_scatter(x, x_dt, T, d, topk_idx, k, E, n_shared, capacity, out_dt, x_perm,
                        x_perm_scale, offsets, perm_src, flat_to_row, overflow, blk, ovf_start, s);
}

namespace {

hipError_t launch_scatter(const void *x, int x_dt, int T, int d, const int32_t *topk_idx, int k,
                          int E, int n_shared, int capacity, int out_dt, void *x_perm,
                          float *x_perm_scale, int32_t *offsets, int32_t *perm_src,
                          int32_t *flat_to_row, int32_t *overflow, int32_t *blk,
                          int32_t *ovf_start, hipStream_t s) {
  const int tpb = T >= 1024 ? 4 : 1;  // tokens per scatter workgroup
  const dim3 grid((T + tpb - 1) / tpb), block(256);
  const size_t lds = sizeof(int) * (size_t)tpb * k;
  const bool quant = out_dt == MOE_E4M3;
#define MOE_SCATTER(ES, Q)                                                                  \
  hipLaunchKernelGGL((perm_scatter_kernel<ES, Q>), grid, block, lds, s, x, T, d, topk_idx, k, E, \
                     n_shared, tpb, blk, offsets, perm_src, flat_to_row, x_perm, x_perm_scale,  \
                     capacity, ovf_start, overflow)
  if (x_dt == MOE_BF16) {
    if (quant) MOE_SCATTER(2, true);
    else MOE_SCATTER(2, false);
  } else {
    if (quant) MOE_SCATTER(4, true);
    else MOE_SCATTER(4, false);
  }
#undef MOE_SCATTER
  return hipGetLastError();
}

}  // namespace

