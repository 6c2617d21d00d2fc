// route.hip -- router scoring, softmax and top-k selection.
//
// "DeepGEMM walkthrough" §2.1: p = Softmax(W_r x); keep the k highest
// scoring experts; the same p weights the combine.  "Dense GEMM to TP MoE"
// §4.2: the router is a linear layer with weight [num_experts][hidden_dim].
// "MoE in practice" §3.2 fuses the logits with the softmax and moves top-k to
// the GPU.
//
// E <= 32: one launch (route_small_bf16_lds for bf16 with d % 64 == 0,
// route_small_bf16 for other d, route_small_f32), scoring, softmax and
// top-k of 16 tokens per workgroup, no workspace.
// E > 32: two launches,
//   logits   a split-K GEMM x [T][d] . w_router[E][d]^T on the matrix cores
//            writing fp32 partial logits part[s][t][e] to the workspace
//            (route_logits_split: 128 tokens x 256 experts per workgroup
//            over one slice of the d axis, operands staged through a
//            three-slot LDS ring by LDS-direct loads; d % 64 != 0 and fp32
//            inputs take the register-staged route_logits_bf16 and the
//            per-thread route_logits_f32);
//   select   a wave per token (route_select_wave): the slices added in
//            slice order (deterministic), + bias, export, softmax, k rounds
//            of a wave-wide argmax on (logit descending, index ascending).
// Every path can also write, per block of 16 consecutive tokens, the sum of
// the softmax probabilities of each expert (prob_sums [ceil(T/16)][E]): the
// router statistics take their mean gate probabilities from it.
#include "moe_internal.h"

namespace {

using namespace moe;

constexpr int kThreads = 256;  // 4 waves
constexpr int RT = 128;        // tokens per logits tile (register-staged kernel)
constexpr int RK = 64;         // columns per K step
constexpr int RP = RK / 8;     // 16-byte pieces per tile row
constexpr int kTargetWG = 512; // two workgroups per CU
constexpr int kSumBlock = 16;  // tokens per probability-sum block (and per one-launch workgroup)

// piece p of row r is stored at slot p ^ (r & 7): eight consecutive rows of
// one piece (one fragment read phase) land in eight distinct bank groups
__device__ __forceinline__ int rswz(int r, int p) { return p ^ (r & 7); }

__host__ __device__ inline int route_eb(int E) { return E <= 32 ? 32 : (E <= 64 ? 64 : 128); }

// number of d-slices of the register-staged kernel: grow while the grid is
// below two workgroups per CU and slices keep at least four K steps on
// average; then drop the slices that equal steps per slice leave empty
inline int route_splits(int T, int d, int E) {
  const long long tiles = (long long)((T + RT - 1) / RT) * ((E + route_eb(E) - 1) / route_eb(E));
  const int kt = (d + RK - 1) / RK;
  int S = 1;
  while (tiles * S < kTargetWG && 2 * S * 4 <= kt) S *= 2;
  const int ks = (kt + S - 1) / S;
  return (kt + ks - 1) / ks;
}

template <int EB>
__global__ __launch_bounds__(kThreads, 2) void route_logits_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, int T, int d, int E,
    int ks_per_slice, float *__restrict__ part) {
  constexpr int NB = EB / 32;                   // 32-expert blocks per wave
  constexpr int LA = RT * RP / kThreads;        // A pieces per thread per step (4)
  constexpr int LB = (EB * RP + kThreads - 1) / kThreads;  // B pieces per thread (1, 2, 4)
  __shared__ u32x4 sA[2][RT * RP];
  __shared__ u32x4 sB[2][EB * RP];

  const int t0 = blockIdx.x * RT, e0 = blockIdx.y * EB, sl = blockIdx.z;
  const int kt_all = (d + RK - 1) / RK;
  const int kb = sl * ks_per_slice, ke = min(kt_all, kb + ks_per_slice);
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;

  u32x4 ra[LA], rb[LB];
  auto load = [&](int kt) {
    const int k0 = kt * RK;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int q = i * kThreads + tid, r = q / RP, c = k0 + (q % RP) * 8;
      const int t = t0 + r;
      ra[i] = (t < T && c < d) ? *reinterpret_cast<const u32x4 *>(x + (size_t)t * d + c)
                               : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int q = i * kThreads + tid, r = q / RP, c = k0 + (q % RP) * 8;
      const int e = e0 + r;
      rb[i] = (q < EB * RP && e < E && c < d)
                  ? *reinterpret_cast<const u32x4 *>(wr + (size_t)e * d + c)
                  : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int q = i * kThreads + tid, r = q / RP;
      sA[buf][r * RP + rswz(r, q % RP)] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int q = i * kThreads + tid, r = q / RP;
      if (q < EB * RP) sB[buf][r * RP + rswz(r, q % RP)] = rb[i];
    }
  };

  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x16{};
  const int fr = lane & 31, fh = lane >> 5;
  const int ar = wv * 32 + fr;  // this lane's token row in the tile

  if (kb < ke) {
    load(kb);
    store(0);
    __syncthreads();
    for (int kt = kb; kt < ke; ++kt) {
      const int cur = (kt - kb) & 1;
      if (kt + 1 < ke) load(kt + 1);
#pragma unroll
      for (int s = 0; s < RK / 16; ++s) {
        const int pc = s * 2 + fh;
        const bf16x8 a = __builtin_bit_cast(bf16x8, sA[cur][ar * RP + rswz(ar, pc)]);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int br = b * 32 + fr;
          const bf16x8 bv = __builtin_bit_cast(bf16x8, sB[cur][br * RP + rswz(br, pc)]);
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc[b], 0, 0, 0);
        }
      }
      if (kt + 1 < ke) store(cur ^ 1);
      __syncthreads();
    }
  }

  // 32x32 accumulator layout: lane holds column (expert) lane%32, register r
  // holds row (token) 8*(r/4) + 4*(lane/32) + r%4
  float *out = part + (size_t)sl * T * E;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int e = e0 + b * 32 + fr;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + wv * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
      if (t < T && e < E) out[(size_t)t * E + e] = acc[b][r];
    }
  }
}

// fp32 inputs: one thread per (token, expert) dot product, sequential in c
__global__ __launch_bounds__(kThreads) void route_logits_f32(const float *__restrict__ x,
                                                             const float *__restrict__ wr,
                                                             int T, int d, int E,
                                                             float *__restrict__ part) {
  const long long p = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (p >= (long long)T * E) return;
  const int t = (int)(p / E), e = (int)(p % E);
  const float *xr = x + (size_t)t * d;
  const float *wrow = wr + (size_t)e * d;
  float acc = 0.f;
  for (int c = 0; c < d; ++c) acc = fmaf(xr[c], wrow[c], acc);
  part[p] = acc;
}

// Segment all-reductions over aligned groups of W lanes (W = 2 ... 64).
// Step s pairs every lane with one partner in the other half of its
// 2^(s+1)-lane block: s = 0, 1 swap neighbours and pairs (DPP quad_perm),
// s = 2, 3 mirror within 8 and 16 lanes (DPP row_half_mirror, row_mirror),
// s = 4, 5 exchange with lane ^ 16 and lane ^ 32 (LDS permute).  Every
// step is an exchange, so all lanes of a segment end with the same value
// (also for sums: each pair adds the same two numbers).
template <int S>
__device__ __forceinline__ int seg_partner(int v) {
  if constexpr (S == 0) return __builtin_amdgcn_update_dpp(0, v, 0xb1, 0xf, 0xf, false);
  else if constexpr (S == 1) return __builtin_amdgcn_update_dpp(0, v, 0x4e, 0xf, 0xf, false);
  else if constexpr (S == 2) return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, false);
  else if constexpr (S == 3) return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, false);
  else if constexpr (S == 4) return __shfl_xor(v, 16, kWave);
  else return __shfl_xor(v, 32, kWave);
}
template <int S>
__device__ __forceinline__ float seg_partner(float v) {
  return __builtin_bit_cast(float, seg_partner<S>(__builtin_bit_cast(int, v)));
}

template <int W, int S = 0>
__device__ __forceinline__ float seg_max(float v) {
  if constexpr ((2 << S) > W) return v;
  else return seg_max<W, S + 1>(fmaxf(v, seg_partner<S>(v)));
}
template <int W, int S = 0>
__device__ __forceinline__ float seg_sum(float v) {
  if constexpr ((2 << S) > W) return v;
  else return seg_sum<W, S + 1>(v + seg_partner<S>(v));
}
// argmax on the key (value descending, index ascending)
template <int W, int S = 0>
__device__ __forceinline__ void seg_argmax(float &bv, int &be) {
  if constexpr ((2 << S) <= W) {
    const float ov = seg_partner<S>(bv);
    const int oe = seg_partner<S>(be);
    if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    seg_argmax<W, S + 1>(bv, be);
  }
}


// ---------------------------------------------------------------------------
// E > 32, bf16, d % 64 == 0: split-K logits on the matrix cores.
//
// A workgroup (8 waves, one per CU: the ring takes 144 KB of LDS) owns 128
// tokens x 256 experts over one slice of the d axis.  Stages of 64 columns
// (128-byte row pieces, whole cache lines) move HBM/L2 -> LDS with
// global_load_lds_dwordx4 through a ring of three slots (stage s + 2 is
// issued while stage s is multiplied), each wave waits only for its own
// loads and the waves meet at a plain s_barrier.  Piece p of row r sits at
// slot p ^ ((r >> 1) & 7), so the fragment reads (32 rows x one piece) hit
// distinct banks.  Waves form a 2 x 4 grid of 64 x 64 outputs
// (v_mfma_f32_32x32x16_bf16, 2 x 2 blocks).  Rows past T and experts past E
// are loaded clamped and never stored.  The slice's fp32 partial logits go
// to part[slice][t][e].  Against the register-staged 128 x 128 kernel this
// reads x and w_router from L2 once per 256 experts and 128 tokens and keeps
// two stages in flight.
constexpr int LT = 128, LE = 256, LK = 64;
constexpr int LNW = 8, LTH = LNW * kWave;
constexpr int LWT = LT / 64, LWE = LE / 64;        // wave grid (tokens x experts), 64 x 64 each
constexpr int LSA = LT * 8, LSB = LE * 8;          // 16-byte slots of an A / B stage
constexpr int LIA = LSA / LTH, LIB = LSB / LTH;    // LDS-direct loads per thread and stage
constexpr int kSplitTargetWG = 256;                // one workgroup per CU
static_assert(LWT * LWE == LNW, "the waves must tile the workgroup's outputs");

__device__ __forceinline__ int lswz(int row, int p) { return p ^ ((row >> 1) & 7); }

// slices of the split kernel: double while the grid stays within one
// workgroup per CU and slices keep at least four stages
inline int route_split_slices(int T, int d, int E) {
  const long long tiles = (long long)((T + LT - 1) / LT) * ((E + LE - 1) / LE);
  const int nst = d / LK;
  int S = 1;
  while (tiles * S * 2 <= kSplitTargetWG && nst / (S * 2) >= 4) S *= 2;
  const int sps = (nst + S - 1) / S;
  return (nst + sps - 1) / sps;
}

__global__ __launch_bounds__(LTH, 1) void route_logits_split(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr, int T, int d, int E, int sps,
    float *__restrict__ part) {
  __shared__ u32x4 sA0[LSA], sA1[LSA], sA2[LSA];
  __shared__ u32x4 sB0[LSB], sB1[LSB], sB2[LSB];
  const int t0 = blockIdx.x * LT, e0 = blockIdx.y * LE, sl = blockIdx.z;
  const int kb = sl * sps;
  const int ns = min(d / LK, kb + sps) - kb;  // stages of this slice (>= 1)
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  const int wm = wv / LWE, wn = wv % LWE;
  // LDS-direct sources: wave wv fills slots [wv * S / LNW, +S / LNW) of each
  // stage, 64 per instruction; slot q holds piece lswz(q / 8, q % 8) of row q / 8
  const uint16_t *ga[LIA];
  const uint16_t *gb[LIB];
#pragma unroll
  for (int i = 0; i < LIA; ++i) {
    const int q = wv * (LSA / LNW) + i * kWave + lane, r = q / 8;
    ga[i] = x + (size_t)min(t0 + r, T - 1) * d + (size_t)kb * LK + lswz(r, q % 8) * 8;
  }
#pragma unroll
  for (int i = 0; i < LIB; ++i) {
    const int q = wv * (LSB / LNW) + i * kWave + lane, r = q / 8;
    gb[i] = wr + (size_t)min(e0 + r, E - 1) * d + (size_t)kb * LK + lswz(r, q % 8) * 8;
  }
  const int da = wv * (LSA / LNW), db = wv * (LSB / LNW);
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const int fr = lane & 31, fh = lane >> 5;

#define MOE_RISSUE(SA, SB, ST)                                                                 \
  _Pragma("unroll") for (int i = 0; i < LIA; ++i)                                             \
    __builtin_amdgcn_global_load_lds((const void *)(ga[i] + (size_t)(ST) * LK),               \
                                     (lds_void *)((SA) + da + i * kWave), 16, 0, 0);          \
  _Pragma("unroll") for (int i = 0; i < LIB; ++i)                                             \
    __builtin_amdgcn_global_load_lds((const void *)(gb[i] + (size_t)(ST) * LK),               \
                                     (lds_void *)((SB) + db + i * kWave), 16, 0, 0);
#define MOE_RCOMPUTE(SA, SB)                                                                   \
  _Pragma("unroll") for (int ks = 0; ks < LK / 16; ++ks) {                                    \
    const int pc = ks * 2 + fh;                                                               \
    bf16x8 a[2], b[2];                                                                        \
    _Pragma("unroll") for (int mi = 0; mi < 2; ++mi) {                                        \
      const int r = wm * 64 + mi * 32 + fr;                                                   \
      a[mi] = __builtin_bit_cast(bf16x8, (SA)[r * 8 + lswz(r, pc)]);                          \
    }                                                                                         \
    _Pragma("unroll") for (int nb = 0; nb < 2; ++nb) {                                        \
      const int r = wn * 64 + nb * 32 + fr;                                                   \
      b[nb] = __builtin_bit_cast(bf16x8, (SB)[r * 8 + lswz(r, pc)]);                          \
    }                                                                                         \
    _Pragma("unroll") for (int mi = 0; mi < 2; ++mi)                                          \
      _Pragma("unroll") for (int nb = 0; nb < 2; ++nb)                                        \
        acc[mi][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[nb], acc[mi][nb], 0, 0, 0); \
  }
// stage s in slot s % 3: wait for this wave's loads of stage s (those of
// stage s + 1 may stay in flight) and for its own LDS reads (the compiler
// may sink stage s - 1's last multiplies below the barrier, with their reads
// still queued), meet (every wave is then past stage s - 1, whose slot is
// free), refill that slot with stage s + 2 (past the end the last stage
// again, into a slot nobody reads, so the counts never change), multiply
#define MOE_RSTAGE(CA, CB, NA, NB, S)                                                          \
  wait_vmcnt_lgkm0<LIA + LIB>();                                                              \
  stage_barrier();                                                                            \
  MOE_RISSUE(NA, NB, min((S) + 2, ns - 1))                                                    \
  MOE_RCOMPUTE(CA, CB)

  MOE_RISSUE(sA0, sB0, 0)
  MOE_RISSUE(sA1, sB1, min(1, ns - 1))
  int s = 0;
  for (; s + 3 <= ns; s += 3) {
    MOE_RSTAGE(sA0, sB0, sA2, sB2, s)
    MOE_RSTAGE(sA1, sB1, sA0, sB0, s + 1)
    MOE_RSTAGE(sA2, sB2, sA1, sB1, s + 2)
  }
  if (s < ns) {
    MOE_RSTAGE(sA0, sB0, sA2, sB2, s)
  }
  if (s + 1 < ns) {
    MOE_RSTAGE(sA1, sB1, sA0, sB0, s + 1)
  }
  wait_vmcnt<0>();  // no LDS-direct load may still be landing when the workgroup ends
#undef MOE_RSTAGE
#undef MOE_RCOMPUTE
#undef MOE_RISSUE

  // 32x32 accumulator layout: lane holds column (expert) lane % 32, register
  // r holds row (token) 8 (r / 4) + 4 (lane / 32) + r % 4
  float *out = part + (size_t)sl * T * E;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int e = e0 + wn * 64 + nb * 32 + fr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
        if (t < T && e < E) out[(size_t)t * E + e] = acc[mi][nb][r];
      }
    }
}


// Softmax and top-k of one token held by a segment of W lanes, segment
// lane e holding the logit v of expert e (ok: a real expert of a real
// token).  Max-subtracted softmax over the segment, then k rounds of argmax
// on (logit descending, index ascending); segment lane j < k keeps the j-th
// choice in *idx / *w (renormalised over the k choices with renorm).
// Returns the lane's own softmax probability (0 when !ok).
template <int W>
__device__ __forceinline__ float select_segment(float v, bool ok, int e, int k, int renorm,
                                                int *idx, float *w) {
  v = ok ? v : -INFINITY;
  const float mx = seg_max<W>(v);
  const float ex = ok ? expf(v - mx) : 0.f;
  const float z = seg_sum<W>(ex);
  bool taken = false;
  float my_w = 0.f;
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    float bv = (ok && !taken) ? v : -INFINITY;
    int be = (ok && !taken) ? e : 0x7fffffff;
    seg_argmax<W>(bv, be);
    if (be == e) taken = true;
    if (e == j) {
      my_idx = be;
      my_w = expf(bv - mx) / z;
    }
  }
  if (renorm) {
    float sw = e < k ? my_w : 0.f;
    sw = seg_sum<W>(sw);
    my_w = my_w / sw;
  }
  *idx = my_idx;
  *w = my_w;
  return ok ? ex / z : 0.f;
}

// The end of the one-launch bf16 routes: the eight waves' 16 x EC partial
// logits (acc, 16x16 MFMA layout) added in wave order through LDS, then one
// token per ES-lane segment selects, and the 16 tokens' probability sums
// are written per expert.  Called by all 512 threads.
template <int NB, int ES>
__device__ __forceinline__ void small_finish(const f32x4 (&acc)[NB], const float *__restrict__ bias,
                                             int T, int E, int k, int renorm,
                                             float *__restrict__ logits_out,
                                             int32_t *__restrict__ topk_idx,
                                             float *__restrict__ topk_w,
                                             float *__restrict__ prob_sums) {
  constexpr int NW = 8, EC = NB * 16;
  __shared__ float s_acc[NW][kSumBlock][EC + 1];
  __shared__ float s_p[kSumBlock][EC + 1];
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  const int t0 = blockIdx.x * kSumBlock;
  const int r = lane & 15, q = lane >> 4;
  // 16x16 accumulator layout: lane holds column (expert) lane % 16 and rows
  // (tokens) 4 (lane / 16) + i in register i
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_acc[wv][4 * q + i][b * 16 + r] = acc[b][i];
  __syncthreads();
  {
    const int tt = threadIdx.x / 32, e = threadIdx.x % 32;  // 512 threads = 16 tokens x 32
    if (e < EC) {
      float v = s_acc[0][tt][e];
#pragma unroll
      for (int w = 1; w < NW; ++w) v += s_acc[w][tt][e];
      s_acc[0][tt][e] = v;
    }
  }
  __syncthreads();
  constexpr int TPW = kWave / ES;          // tokens per wave in the selection
  constexpr int SW = kSumBlock / TPW;      // waves that select
  if (wv < SW) {
    const int i = wv * TPW + lane / ES, e = lane % ES, t = t0 + i;
    const bool ok = t < T && e < E;
    float v = 0.f;
    if (ok) {
      v = s_acc[0][i][e];
      if (bias) v += bias[e];
      if (logits_out) logits_out[(size_t)t * E + e] = v;
    }
    int my_idx;
    float my_w;
    const float p = select_segment<ES>(v, ok, e, k, renorm, &my_idx, &my_w);
    if (t < T && e < k) {
      topk_idx[(size_t)t * k + e] = my_idx;
      topk_w[(size_t)t * k + e] = my_w;
    }
    s_p[i][e] = p;
  }
  if (prob_sums) {
    __syncthreads();
    if ((int)threadIdx.x < E) {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < kSumBlock; ++i) sum += s_p[i][threadIdx.x];
      prob_sums[(size_t)blockIdx.x * E + threadIdx.x] = sum;
    }
  }
}

// ---------------------------------------------------------------------------
// E <= 32, bf16: one launch.  A workgroup (8 waves) owns 16 tokens.  The
// logits are a 16 x EC matrix product on the matrix cores
// (v_mfma_f32_16x16x32_bf16, tokens as rows, NB blocks of 16 experts as
// columns, EC = 16 NB): the waves split the d axis in 32-column steps (wave
// w takes steps w, w + 8, ...) and load both operands straight into
// registers (lane l: row l % 16, columns 8 (l / 16) .. + 8 of the step, 16
// bytes), eight steps' loads issued before their MFMAs, with clamped
// addresses and masked values (lanes of padding experts load nothing); the
// matrix cores do the reduction over d that a lane-parallel dot product
// would need shuffles for.  The eight waves' partial products are added in
// wave order through LDS; then one token per ES-lane segment (ES = E rounded
// up to 8, 16 or 32) takes the softmax and top-k, and the probability sums
// of the 16 tokens are written per expert.  Measured on the Mixtral shapes
// against a one-launch kernel of bf16 dot products per lane and a 63-step
// butterfly reduce-scatter per wave (8 tokens per workgroup): the same time
// (12.4 against 12.2 us), with fewer instructions and no shuffles.
template <int NB, int ES>
__global__ __launch_bounds__(512) void route_small_bf16(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const float *__restrict__ bias, int T, int d, int E, int k, int renorm,
    float *__restrict__ logits_out, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    float *__restrict__ prob_sums) {
  constexpr int NW = 8, EC = NB * 16, U = 8;
  static_assert(ES <= EC, "segment wider than the computed columns");
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  const int t0 = blockIdx.x * kSumBlock;
  const int r = lane & 15, q = lane >> 4;
  const int nsteps = (d + 31) / 32;
  const bool a_ok = t0 + r < T;
  const uint16_t *xa = x + (size_t)min(t0 + r, T - 1) * d;
  const uint16_t *wb[NB];
  bool b_ok[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int e = b * 16 + r;
    b_ok[b] = e < E;
    wb[b] = wr + (size_t)min(e, E - 1) * d;
  }
  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{};
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  for (int s0 = wv; s0 < nsteps; s0 += NW * U) {
    u32x4 av[U], bv[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int cc = min((s0 + u * NW) * 32 + q * 8, d - 8);
      av[u] = *reinterpret_cast<const u32x4 *>(xa + cc);
      // lanes of the padding columns (e >= E) load nothing: with E = 8 that
      // halves the router-weight requests (Mixtral shapes: 15 -> 14 us)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        bv[u][b] = zero4;
        if (b_ok[b]) bv[u][b] = *reinterpret_cast<const u32x4 *>(wb[b] + cc);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = (s0 + u * NW) * 32 + q * 8 < d;
      const bf16x8 a = __builtin_bit_cast(bf16x8, (in && a_ok) ? av[u] : zero4);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const bf16x8 w = __builtin_bit_cast(bf16x8, (in && b_ok[b]) ? bv[u][b] : zero4);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w, acc[b], 0, 0, 0);
      }
    }
  }
  small_finish<NB, ES>(acc, bias, T, E, k, renorm, logits_out, topk_idx, topk_w, prob_sums);
}

// E <= 32, bf16, d % 64 == 0: the same product with x staged through LDS.
// Wave w takes the 64-column chunks w, w + 8, ... of the 16 token rows and
// moves each by two LDS-direct loads of whole 128-byte row pieces (piece p
// of row r at slot p ^ ((r >> 1) & 7), so the fragment reads hit distinct
// banks) into its own part of LDS, eight chunks per round (all of a wave's
// chunks up to d = 4096); the router rows go straight to registers as
// above.  A wave waits for all of its round's loads, then multiplies; it
// reads only what it loaded itself, so no workgroup barrier is needed.
// Measured against the register-staged kernel, one process, by events in
// the layer: Mixtral shapes 17.8 -> 17.5 us, decode size 13.7 -> 13.0 us.
constexpr int kRouteChunkRound = 8;  // chunks per round of a wave
template <int NB, int ES>
__global__ __launch_bounds__(512) void route_small_bf16_lds(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const float *__restrict__ bias, int T, int d, int E, int k, int renorm,
    float *__restrict__ logits_out, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    float *__restrict__ prob_sums) {
  constexpr int NW = 8, CR = kRouteChunkRound;
  static_assert(ES <= NB * 16, "segment wider than the computed columns");
  __shared__ u32x4 s_x[NW][CR][16 * 8];  // per wave: CR chunks of 16 rows x 8 pieces
  const int lane = lane_id(), wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int t0 = blockIdx.x * kSumBlock;
  const int r = lane & 15, q = lane >> 4;
  const int nch = d / 64;
  const int mine = nch > wv ? (nch - wv + NW - 1) / NW : 0;  // chunks of this wave
  // LDS-direct sources: lane j of load h (0, 1) fills slot j of rows
  // 8 h .. 8 h + 7: row 8 h + j / 8, piece (j % 8) ^ ((row >> 1) & 7)
  const uint16_t *xs[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 8 * h + (lane >> 3);
    xs[h] = x + (size_t)min(t0 + row, T - 1) * d + (((lane & 7) ^ ((row >> 1) & 7)) * 8);
  }
  const uint16_t *wb[NB];
  bool b_ok[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int e = b * 16 + r;
    b_ok[b] = e < E;
    wb[b] = wr + (size_t)min(e, E - 1) * d;
  }
  const bool a_ok = t0 + r < T;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{};
  for (int j0 = 0; j0 < mine; j0 += CR) {
    // a round always loads CR chunks (past the wave's last chunk it loads
    // that one again and does not multiply it), so the loads stay unrolled
    // into registers
    u32x4 bv[CR][2][NB];
#pragma unroll
    for (int i = 0; i < CR; ++i) {
      const int c = wv + NW * min(j0 + i, mine - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        __builtin_amdgcn_global_load_lds((const void *)(xs[h] + (size_t)c * 64),
                                         (lds_void *)(&s_x[wv][i][h * 64]), 16, 0, 0);
      // lanes of the padding experts (e >= E) load nothing
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          bv[i][st][b] = zero4;
          if (b_ok[b])
            bv[i][st][b] = *reinterpret_cast<const u32x4 *>(wb[b] + (size_t)c * 64 + st * 32 + q * 8);
        }
    }
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");  // no LDS read moves above the wait
#pragma unroll
    for (int i = 0; i < CR; ++i) {
      if (j0 + i >= mine) continue;  // wave-uniform
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int p = st * 4 + q;
        const bf16x8 a =
            __builtin_bit_cast(bf16x8, a_ok ? s_x[wv][i][r * 8 + (p ^ ((r >> 1) & 7))] : zero4);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bv[i][st][b]),
                                                          acc[b], 0, 0, 0);
      }
    }
    // every fragment read of this round is complete before the next round's
    // loads rewrite the slots
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  small_finish<NB, ES>(acc, bias, T, E, k, renorm, logits_out, topk_idx, topk_w, prob_sums);
}

// E <= 32, fp32: one launch.  A workgroup of 16 ES threads owns 16 tokens;
// thread (i, e) = (tid / ES, tid % ES) accumulates the dot product of token
// i and expert e over d in order (16-byte loads), then the ES lanes of a
// token select as above.
template <int ES>
__global__ __launch_bounds__(kSumBlock * ES) void route_small_f32(
    const float *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    int T, int d, int E, int k, int renorm, float *__restrict__ logits_out,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, float *__restrict__ prob_sums) {
  __shared__ float s_p[kSumBlock][ES + 1];
  const int i = threadIdx.x / ES, e = threadIdx.x % ES;
  const int t = blockIdx.x * kSumBlock + i;
  const bool ok = t < T && e < E;
  const float4 *xr = reinterpret_cast<const float4 *>(x + (size_t)min(t, T - 1) * d);
  const float4 *wrow = reinterpret_cast<const float4 *>(wr + (size_t)min(e, E - 1) * d);
  float acc = 0.f;
#pragma unroll 4
  for (int c = 0; c < d / 4; ++c) {
    const float4 a = xr[c], b = wrow[c];
    acc = fmaf(a.x, b.x, acc);
    acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc);
    acc = fmaf(a.w, b.w, acc);
  }
  float v = acc;
  if (ok) {
    if (bias) v += bias[e];
    if (logits_out) logits_out[(size_t)t * E + e] = v;
  }
  int my_idx;
  float my_w;
  const float p = select_segment<ES>(v, ok, e, k, renorm, &my_idx, &my_w);
  if (t < T && e < k) {
    topk_idx[(size_t)t * k + e] = my_idx;
    topk_w[(size_t)t * k + e] = my_w;
  }
  if (prob_sums) {
    s_p[i][e] = p;
    __syncthreads();
    if ((int)threadIdx.x < E) {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < kSumBlock; ++j) sum += s_p[j][threadIdx.x];
      prob_sums[(size_t)blockIdx.x * E + threadIdx.x] = sum;
    }
  }
}

// Whole-wave maximum and sum, returned to every lane: an inclusive DPP scan
// (row_shr 1, 2, 4, 8 inside each 16-lane row, then row_bcast15 and
// row_bcast31 across the rows) leaves the total in lane 63, which is read
// back as a scalar -- no LDS round trip.  A lane without a source in a step
// contributes the identity.  Must be called by a whole wave.
#define MOE_DPP_F(v, id, ctrl, rmask)                                                   \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, (id)),  \
                                                        __builtin_bit_cast(int, (v)),   \
                                                        ctrl, rmask, 0xf, false))
__device__ __forceinline__ float wave_allmax(float v) {
  const float n = -INFINITY;
  v = fmaxf(v, MOE_DPP_F(v, n, 0x111, 0xf));  // row_shr:1
  v = fmaxf(v, MOE_DPP_F(v, n, 0x112, 0xf));  // row_shr:2
  v = fmaxf(v, MOE_DPP_F(v, n, 0x114, 0xf));  // row_shr:4
  v = fmaxf(v, MOE_DPP_F(v, n, 0x118, 0xf));  // row_shr:8
  v = fmaxf(v, MOE_DPP_F(v, n, 0x142, 0xa));  // row_bcast:15
  v = fmaxf(v, MOE_DPP_F(v, n, 0x143, 0xc));  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kWave - 1));
}
__device__ __forceinline__ float wave_allsum(float v) {
  v += MOE_DPP_F(v, 0.f, 0x111, 0xf);
  v += MOE_DPP_F(v, 0.f, 0x112, 0xf);
  v += MOE_DPP_F(v, 0.f, 0x114, 0xf);
  v += MOE_DPP_F(v, 0.f, 0x118, 0xf);
  v += MOE_DPP_F(v, 0.f, 0x142, 0xa);
  v += MOE_DPP_F(v, 0.f, 0x143, 0xc);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kWave - 1));
}
#undef MOE_DPP_F

// ---------------------------------------------------------------------------
// Selection from S slices of partial logits (or from given logits, S = 1):
// 16 tokens per workgroup of 16 waves, a wave per token (8 waves of two
// tokens each when NPER = 16), lane l holding the NPER consecutive experts
// l NPER .. l NPER + NPER - 1 (16-byte loads when VEC).  A wave issues the
// loads of up to 8 slices (32 values a lane) together, adds them in slice
// order (deterministic), adds the bias, exports, and selects with wave-wide
// reductions.  The probability sums of the 16 tokens are added over the
// waves in token order.  (Four waves of four tokens each, loads of four
// tokens in flight per wave: 32 us on the DeepSeek shapes; a wave per token:
// 16.7 us.)
// tokens a wave takes one after the other (two when a lane holds 16 experts,
// so that 256 registers are left to a lane)
__host__ __device__ constexpr int sel_tpw(int nper) { return nper >= 16 ? 2 : 1; }

template <int NPER, bool VEC>
__global__ __launch_bounds__(kSumBlock / sel_tpw(NPER) * kWave) void route_select_wave(
    const float *__restrict__ part, int S, const float *__restrict__ bias, int T, int E, int k,
    int renorm, float *__restrict__ logits_out, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, float *__restrict__ prob_sums) {
  constexpr int CH = NPER <= 4 ? 8 : 32 / NPER;  // slices loaded together (<= 32 values)
  extern __shared__ float s_ps[];  // [16][E] when prob_sums is given
  constexpr int TPW = sel_tpw(NPER), NWV = kSumBlock / TPW;
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  const int e0 = lane * NPER;
  for (int tw = 0; tw < TPW; ++tw) {
  const int ti = wv * TPW + tw;  // token of the block
  const int t = blockIdx.x * kSumBlock + ti;
  const bool tok = t < T;  // no early exit: the reductions need every lane
  const size_t tcl = (size_t)min(t, T - 1);
  float v[NPER];
  for (int s0 = 0; s0 < S; s0 += CH) {
    float q[CH][NPER];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const size_t rowb = ((size_t)min(s0 + j, S - 1) * T + tcl) * E;
      if constexpr (VEC) {
#pragma unroll
        for (int m = 0; m < NPER / 4; ++m) {
          const float4 f4 = *reinterpret_cast<const float4 *>(part + rowb + min(e0 + 4 * m, E - 4));
          q[j][4 * m] = f4.x;
          q[j][4 * m + 1] = f4.y;
          q[j][4 * m + 2] = f4.z;
          q[j][4 * m + 3] = f4.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < NPER; ++i) q[j][i] = part[rowb + min(e0 + i, E - 1)];
      }
    }
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (s0 + j < S) v[i] = (s0 + j == 0) ? q[j][i] : v[i] + q[j][i];
  }
  bool ok[NPER];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = e0 + i;
    ok[i] = tok && e < E;
    if (ok[i]) {
      if (bias) v[i] += bias[e];
      if (logits_out) logits_out[(size_t)t * E + e] = v[i];
    } else {
      v[i] = -INFINITY;
    }
    mx = fmaxf(mx, v[i]);
  }
  mx = wave_allmax(mx);
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < NPER; ++i)
    if (ok[i]) z += expf(v[i] - mx);
  z = wave_allsum(z);
  // k rounds: every lane offers its best expert not yet taken (ascending
  // index with a strict >, so its lowest index among equal logits), the
  // wave takes the largest offer and, among equal offers, the lowest lane:
  // a lane's experts are contiguous, so that is the lowest expert index.
  // Round j's logit and expert end up in lane j.
  uint32_t taken = 0;
  float my_v = -INFINITY;
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      if (ok[i] && !((taken >> i) & 1u) && (bi < 0 || v[i] > bv)) {
        bv = v[i];
        bi = i;
      }
    }
    const float m = wave_allmax(bv);
    const unsigned long long offers = __ballot(bi >= 0 && bv == m);
    // no offer at all only in a wave past the last token (nothing is stored)
    const int wl = offers ? __builtin_ctzll(offers) : 0;
    const int we = __builtin_amdgcn_readlane(e0 + bi, wl);
    if (offers && lane == wl) taken |= 1u << bi;
    if (lane == j) {
      my_v = m;
      my_idx = we;
    }
  }
  float my_w = lane < k ? expf(my_v - mx) / z : 0.f;
  if (renorm) my_w = my_w / wave_allsum(my_w);
  if (tok && lane < k) {
    topk_idx[(size_t)t * k + lane] = my_idx;
    topk_w[(size_t)t * k + lane] = my_w;
  }
  if (prob_sums) {
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (e0 + i < E) s_ps[ti * E + e0 + i] = ok[i] ? expf(v[i] - mx) / z : 0.f;
  }
  }  // tokens of the wave
  if (prob_sums) {
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += NWV * kWave) {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < kSumBlock; ++i) sum += s_ps[i * E + e];
      prob_sums[(size_t)blockIdx.x * E + e] = sum;
    }
  }
}

template <int NPER>
void launch_select_n(const float *part, int S, const float *bias, int T, int E, int k,
                     int renorm, float *logits_out, int32_t *topk_idx, float *topk_w,
                     float *prob_sums, hipStream_t s) {
  const dim3 grid((T + kSumBlock - 1) / kSumBlock), block(kSumBlock / sel_tpw(NPER) * kWave);
  const size_t lds = prob_sums ? sizeof(float) * kSumBlock * (size_t)E : 0;
  if constexpr (NPER % 4 == 0) {
    if (E % 4 == 0) {
      hipLaunchKernelGGL((route_select_wave<NPER, true>), grid, block, lds, s, part, S, bias, T,
                         E, k, renorm, logits_out, topk_idx, topk_w, prob_sums);
      return;
    }
  }
  hipLaunchKernelGGL((route_select_wave<NPER, false>), grid, block, lds, s, part, S, bias, T, E,
                     k, renorm, logits_out, topk_idx, topk_w, prob_sums);
}

void launch_select(const float *part, int S, const float *bias, int T, int E, int k, int renorm,
                   float *logits_out, int32_t *topk_idx, float *topk_w, float *prob_sums,
                   hipStream_t s) {
#define MOE_SEL(NP) \
  launch_select_n<NP>(part, S, bias, T, E, k, renorm, logits_out, topk_idx, topk_w, prob_sums, s)
  if (E <= 64) MOE_SEL(1);
  else if (E <= 128) MOE_SEL(2);
  else if (E <= 256) MOE_SEL(4);
  else if (E <= 512) MOE_SEL(8);
  else MOE_SEL(16);
#undef MOE_SEL
}

}  // namespace

size_t route_ws_bytes(int T, int d, int E) {
  if (E <= 32) return 0;  // one-launch paths
  const int S = d % LK == 0 ? route_split_slices(T, d, E) : route_splits(T, d, E);
  return sizeof(float) * (size_t)S * (size_t)T * (size_t)E;
}

hipError_t launch_route(const void *x, const void *w_router, int dt, const float *bias, int T,
                        int d, int E, int k, unsigned flags, float *logits, int32_t *topk_idx,
                        float *topk_w, float *prob_sums, float *ws, hipStream_t s) {
  const int renorm = (flags & MOE_ROUTE_RENORM) ? 1 : 0;
  if (flags & MOE_ROUTE_FROM_LOGITS) {
    launch_select(logits, 1, nullptr, T, E, k, renorm, nullptr, topk_idx, topk_w, prob_sums, s);
    return hipGetLastError();
  }
  const unsigned nblk = (unsigned)((T + kSumBlock - 1) / kSumBlock);
  if (E <= 32) {
    const int es = E <= 8 ? 8 : (E <= 16 ? 16 : 32);
    if (dt == MOE_BF16) {
      const uint16_t *xb = static_cast<const uint16_t *>(x);
      const uint16_t *wb = static_cast<const uint16_t *>(w_router);
#define MOE_SMALL(NB, ES)                                                                    \
  if (d % 64 == 0)                                                                           \
    hipLaunchKernelGGL((route_small_bf16_lds<NB, ES>), dim3(nblk), dim3(512), 0, s, xb, wb,   \
                       bias, T, d, E, k, renorm, logits, topk_idx, topk_w, prob_sums);       \
  else                                                                                       \
    hipLaunchKernelGGL((route_small_bf16<NB, ES>), dim3(nblk), dim3(512), 0, s, xb, wb, bias, \
                       T, d, E, k, renorm, logits, topk_idx, topk_w, prob_sums)
      if (es == 8) MOE_SMALL(1, 8);
      else if (es == 16) MOE_SMALL(1, 16);
      else MOE_SMALL(2, 32);
#undef MOE_SMALL
    } else {
      const float *xf = static_cast<const float *>(x);
      const float *wf = static_cast<const float *>(w_router);
#define MOE_SMALL(ES)                                                                          \
  hipLaunchKernelGGL((route_small_f32<ES>), dim3(nblk), dim3(kSumBlock * ES), 0, s, xf, wf, bias, \
                     T, d, E, k, renorm, logits, topk_idx, topk_w, prob_sums)
      if (es == 8) MOE_SMALL(8);
      else if (es == 16) MOE_SMALL(16);
      else MOE_SMALL(32);
#undef MOE_SMALL
    }
    return hipGetLastError();
  }
  int S = 1;
  const dim3 block(kThreads);
  if (dt == MOE_BF16) {
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    const uint16_t *wb = static_cast<const uint16_t *>(w_router);
    if (d % LK == 0) {
      S = route_split_slices(T, d, E);
      const int nst = d / LK, sps = (nst + S - 1) / S;
      const dim3 grid((T + LT - 1) / LT, (E + LE - 1) / LE, S);
      hipLaunchKernelGGL(route_logits_split, grid, dim3(LTH), 0, s, xb, wb, T, d, E, sps, ws);
    } else {
      S = route_splits(T, d, E);
      const int eb = route_eb(E);
      const int kt = (d + RK - 1) / RK;
      const dim3 grid((T + RT - 1) / RT, (E + eb - 1) / eb, S);
      const int ks = (kt + S - 1) / S;
      if (eb == 32)
        hipLaunchKernelGGL(route_logits_bf16<32>, grid, block, 0, s, xb, wb, T, d, E, ks, ws);
      else if (eb == 64)
        hipLaunchKernelGGL(route_logits_bf16<64>, grid, block, 0, s, xb, wb, T, d, E, ks, ws);
      else
        hipLaunchKernelGGL(route_logits_bf16<128>, grid, block, 0, s, xb, wb, T, d, E, ks, ws);
    }
  } else {
    const long long n = (long long)T * E;
    hipLaunchKernelGGL(route_logits_f32, dim3((unsigned)((n + kThreads - 1) / kThreads)), block,
                       0, s, static_cast<const float *>(x), static_cast<const float *>(w_router),
                       T, d, E, ws);
  }
  launch_select(ws, S, bias, T, E, k, renorm, logits, topk_idx, topk_w, prob_sums, s);
  return hipGetLastError();
}
