// route.hip -- router scoring, softmax and top-k selection in one launch.
//
// "DeepGEMM walkthrough" §2.1: p = Softmax(W_r x); keep the k highest
// scoring experts; the same p weights the combine.  "Dense GEMM to TP MoE"
// §4.2: the router is a linear layer with weight [num_experts][hidden_dim].
//
// E <= 32 with bf16 inputs: one launch (route_fused_small below; the
// logits are a few dot products per token, so the partial-logit round trip
// would dominate).  Otherwise two launches:
//   logits   a split-K GEMM x [T][d] . w_router[E][d]^T on the matrix cores
//            (v_mfma_f32_32x32x16_bf16): a workgroup (4 waves) owns 128
//            tokens x EB experts (EB = 32, 64 or 128) over one slice of the
//            d axis and writes fp32 partial logits part[s][t][e] to the
//            workspace.  Tiles are staged through LDS 64 columns at a time,
//            double buffered through registers; tokens, experts and columns
//            past the end read as zero.  Split-K gives enough workgroups to
//            fill the chip when T/128 x E/EB alone would not, and 128 x 128
//            tiles keep the re-reads of x and w_router from L2 low.  fp32
//            inputs (small configurations) take a plain per-thread dot
//            product with one slice.
//   select   one token per segment of lanes (the next power of two >= E,
//            at most a wave): sum of the partials in slice order
//            (deterministic; eight slices' loads in flight at once) plus the
//            bias, export of the logits, segment max, sum of exp, then k
//            rounds of a segment-wide argmax with the key (logit descending,
//            index ascending).
#include "moe_internal.h"

namespace {

using namespace moe;

constexpr int kThreads = 256;  // 4 waves
constexpr int RT = 128;        // tokens per logits tile
constexpr int RK = 64;         // columns per K step
constexpr int RP = RK / 8;     // 16-byte pieces per tile row
constexpr int kTargetWG = 512; // two workgroups per CU

// piece p of row r is stored at slot p ^ (r & 7): eight consecutive rows of
// one piece (one fragment read phase) land in eight distinct bank groups
__device__ __forceinline__ int rswz(int r, int p) { return p ^ (r & 7); }

__host__ __device__ inline int route_eb(int E) { return E <= 32 ? 32 : (E <= 64 ? 64 : 128); }

// number of d-slices: grow while the grid is below two workgroups per CU and
// slices keep at least four K steps on average; then drop the slices that
// equal steps per slice leave empty
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

// One token per segment of W lanes (W = 8 ... 64, so 64 / W tokens per
// wave when E <= 32); a lane holds NPER = ceil(E / W) experts, e = lane + W i.
// The S partials of a value are loaded eight slices at a time, all issued
// before the first is used, and added in slice order.  Segment-wide max,
// sum of exp and k rounds of argmax use xor shuffles inside the segment.
template <int W, int NPER>
__global__ __launch_bounds__(kThreads) void route_select(
    const float *__restrict__ part, int S, const float *__restrict__ bias, int T, int E, int k,
    int renorm, float *__restrict__ logits_out, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w) {
  constexpr int TPW = kWave / W;  // tokens per wave
  const int lane = lane_id(), wv = threadIdx.x / kWave, sl_lane = lane % W;
  const int t = (blockIdx.x * (kThreads / kWave) + wv) * TPW + lane / W;
  const bool tok = t < T;  // no early return: the shuffles need every lane
  bool ok[NPER];
  size_t base[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = sl_lane + i * W;
    ok[i] = tok && e < E;
    base[i] = (size_t)(tok ? t : 0) * E + (e < E ? e : 0);
  }
  float v[NPER];
  constexpr int CH = 8;  // slices loaded per round
  for (int s0 = 0; s0 < S; s0 += CH) {
    float q[CH][NPER];
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        q[j][i] = (s0 + j < S && ok[i]) ? part[(size_t)(s0 + j) * T * E + base[i]] : 0.f;
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        if (s0 + j < S) v[i] = (s0 + j == 0) ? q[j][i] : v[i] + q[j][i];
  }
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = sl_lane + i * W;
    if (ok[i]) {
      if (bias) v[i] += bias[e];
      if (logits_out) logits_out[base[i]] = v[i];
    } else {
      v[i] = -INFINITY;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NPER; ++i) mx = fmaxf(mx, v[i]);
  mx = seg_max<W>(mx);
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < NPER; ++i)
    if (ok[i]) z += expf(v[i] - mx);
  z = seg_sum<W>(z);

  uint32_t taken = 0;
  float my_w = 0.f;
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    // best untaken candidate held by this lane
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      const int e = sl_lane + i * W;
      if (ok[i] && !((taken >> i) & 1u)) {
        if (v[i] > bv || (v[i] == bv && e < be)) { bv = v[i]; be = e; }
      }
    }
    // segment-wide argmax on (value desc, index asc)
    seg_argmax<W>(bv, be);
    if (be != 0x7fffffff && (be % W) == sl_lane) taken |= 1u << (be / W);
    if (sl_lane == j) {
      my_idx = be;
      my_w = expf(bv - mx) / z;
    }
  }
  if (renorm) {
    float sw = sl_lane < k ? my_w : 0.f;
    sw = seg_sum<W>(sw);
    my_w = my_w / sw;
  }
  if (tok && sl_lane < k) {
    topk_idx[(size_t)t * k + sl_lane] = my_idx;
    topk_w[(size_t)t * k + sl_lane] = my_w;
  }
}

// Small E (<= 32, bf16): scoring, softmax and top-k in one launch, no
// workspace.  A workgroup takes TPW = 64 / EP tokens (EP = E rounded up to
// 8, 16 or 32) and its four waves split the d axis; a lane accumulates the
// bf16 dot products (v_dot2c_f32_bf16) of every (token, expert) pair over
// its 16-byte column chunks, with the token and weight chunks of a step all
// loaded before use.  A butterfly reduce-scatter over the wave (each value
// added in exactly one lane, fixed pairing) leaves lane l with value l =
// token l / EP, expert l % EP; the four waves' values are added in wave
// order through LDS, and wave 0 finishes like the select kernel with one
// token per EP-lane segment.  Measured on the Mixtral shapes: 13.9 us;
// eight waves 17.6 us (each wave pays the reduce-scatter); two chunks per
// step 15.1 us (201 registers, lower occupancy).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int EP>
__global__ __launch_bounds__(kThreads) void route_fused_small(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const float *__restrict__ bias, int T, int d, int E, int k, int renorm,
    float *__restrict__ logits_out, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w) {
  constexpr int TPW = kWave / EP;  // tokens per workgroup
  __shared__ float s_red[kThreads / kWave][kWave];
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  const int t0 = blockIdx.x * TPW;
  const int nch = d / 8;  // 16-byte chunks per row
  const int c_lo = wv * nch / 4, c_hi = (wv + 1) * nch / 4;
  float a[kWave];  // [t][e] partial dot products
#pragma unroll
  for (int i = 0; i < kWave; ++i) a[i] = 0.f;
  for (int c = c_lo + lane; c < c_hi; c += kWave) {
    // the 16-byte chunks go through plain arrays of dwords: bit-casting a
    // subscripted vector element (v[j]) to bf16x2 compiles to element 0
    // for every j with this toolchain
    unsigned xs[TPW][4], ws[EP][4];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const u32x4 v = t0 + t < T ? *reinterpret_cast<const u32x4 *>(x + (size_t)(t0 + t) * d + c * 8)
                                 : u32x4{0u, 0u, 0u, 0u};
      xs[t][0] = v.x; xs[t][1] = v.y; xs[t][2] = v.z; xs[t][3] = v.w;
    }
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      const u32x4 v = e < E ? *reinterpret_cast<const u32x4 *>(wr + (size_t)e * d + c * 8)
                            : u32x4{0u, 0u, 0u, 0u};
      ws[e][0] = v.x; ws[e][1] = v.y; ws[e][2] = v.z; ws[e][3] = v.w;
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int e = 0; e < EP; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          a[t * EP + e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xs[t][j]),
                                                          __builtin_bit_cast(bf16x2, ws[e][j]),
                                                          a[t * EP + e], false);
  }
  // reduce-scatter: at offset o a lane keeps the half of its values whose
  // index has bit o equal to its own and adds the partner's copy of them
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const bool hi = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < o; ++i) {
      const float send = hi ? a[i] : a[o + i];
      const float keep = hi ? a[o + i] : a[i];
      a[i] = keep + __shfl_xor(send, o, kWave);
    }
  }
  s_red[wv][lane] = a[0];
  __syncthreads();
  if (wv != 0) return;
  float v = ((s_red[0][lane] + s_red[1][lane]) + s_red[2][lane]) + s_red[3][lane];
  const int e = lane % EP, t = t0 + lane / EP;
  const bool ok = t < T && e < E;
  if (ok) {
    if (bias) v += bias[e];
    if (logits_out) logits_out[(size_t)t * E + e] = v;
  } else {
    v = -INFINITY;
  }
  float mx = v;
  mx = seg_max<EP>(mx);
  float z = ok ? expf(v - mx) : 0.f;
  z = seg_sum<EP>(z);
  bool taken = false;
  float my_w = 0.f;
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    float bv = (ok && !taken) ? v : -INFINITY;
    int be = (ok && !taken) ? e : 0x7fffffff;
    seg_argmax<EP>(bv, be);
    if (be == e) taken = true;
    if (e == j) {
      my_idx = be;
      my_w = expf(bv - mx) / z;
    }
  }
  if (renorm) {
    float sw = e < k ? my_w : 0.f;
    sw = seg_sum<EP>(sw);
    my_w = my_w / sw;
  }
  if (t < T && e < k) {
    topk_idx[(size_t)t * k + e] = my_idx;
    topk_w[(size_t)t * k + e] = my_w;
  }
}

template <int W, int NPER>
void launch_select_t(const float *part, int S, const float *bias, int T, int E, int k, int renorm,
                     float *logits_out, int32_t *topk_idx, float *topk_w, hipStream_t s) {
  constexpr int TPB = (kThreads / kWave) * (kWave / W);  // tokens per workgroup
  hipLaunchKernelGGL((route_select<W, NPER>), dim3((T + TPB - 1) / TPB), dim3(kThreads), 0, s,
                     part, S, bias, T, E, k, renorm, logits_out, topk_idx, topk_w);
}

// segment width: the next power of two >= E up to 64, then NPER = E / 64
void launch_select(const float *part, int S, const float *bias, int T, int E, int k, int renorm,
                   float *logits_out, int32_t *topk_idx, float *topk_w, hipStream_t s) {
#define MOE_SEL(W, NP) \
  launch_select_t<W, NP>(part, S, bias, T, E, k, renorm, logits_out, topk_idx, topk_w, s)
  if (E <= 8) MOE_SEL(8, 1);
  else if (E <= 16) MOE_SEL(16, 1);
  else if (E <= 32) MOE_SEL(32, 1);
  else if (E <= 64) MOE_SEL(64, 1);
  else if (E <= 128) MOE_SEL(64, 2);
  else if (E <= 256) MOE_SEL(64, 4);
  else if (E <= 512) MOE_SEL(64, 8);
  else MOE_SEL(64, 16);
#undef MOE_SEL
}

}  // namespace

size_t route_ws_bytes(int T, int d, int E) {
  return sizeof(float) * (size_t)route_splits(T, d, E) * (size_t)T * (size_t)E;
}

hipError_t launch_route(const void *x, const void *w_router, int dt, const float *bias, int T,
                        int d, int E, int k, unsigned flags, float *logits, int32_t *topk_idx,
                        float *topk_w, float *ws, hipStream_t s) {
  const int renorm = (flags & MOE_ROUTE_RENORM) ? 1 : 0;
  const dim3 block(kThreads);
  if (flags & MOE_ROUTE_FROM_LOGITS) {
    launch_select(logits, 1, nullptr, T, E, k, renorm, nullptr, topk_idx, topk_w, s);
    return hipGetLastError();
  }
  if (dt == MOE_BF16 && E <= 32) {
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    const uint16_t *wb = static_cast<const uint16_t *>(w_router);
    if (E <= 8)
      hipLaunchKernelGGL(route_fused_small<8>, dim3((T + 7) / 8), block, 0, s, xb, wb, bias, T, d,
                         E, k, renorm, logits, topk_idx, topk_w);
    else if (E <= 16)
      hipLaunchKernelGGL(route_fused_small<16>, dim3((T + 3) / 4), block, 0, s, xb, wb, bias, T, d,
                         E, k, renorm, logits, topk_idx, topk_w);
    else
      hipLaunchKernelGGL(route_fused_small<32>, dim3((T + 1) / 2), block, 0, s, xb, wb, bias, T, d,
                         E, k, renorm, logits, topk_idx, topk_w);
    return hipGetLastError();
  }
  int S = 1;
  if (dt == MOE_BF16) {
    S = route_splits(T, d, E);
    const int eb = route_eb(E);
    const int kt = (d + RK - 1) / RK;
    const dim3 grid((T + RT - 1) / RT, (E + eb - 1) / eb, S);
    const int ks = (kt + S - 1) / S;
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    const uint16_t *wb = static_cast<const uint16_t *>(w_router);
    if (eb == 32)
      hipLaunchKernelGGL(route_logits_bf16<32>, grid, block, 0, s, xb, wb, T, d, E, ks, ws);
    else if (eb == 64)
      hipLaunchKernelGGL(route_logits_bf16<64>, grid, block, 0, s, xb, wb, T, d, E, ks, ws);
    else
      hipLaunchKernelGGL(route_logits_bf16<128>, grid, block, 0, s, xb, wb, T, d, E, ks, ws);
  } else {
    const long long n = (long long)T * E;
    hipLaunchKernelGGL(route_logits_f32, dim3((unsigned)((n + kThreads - 1) / kThreads)), block,
                       0, s, static_cast<const float *>(x), static_cast<const float *>(w_router),
                       T, d, E, ws);
  }
  launch_select(ws, S, bias, T, E, k, renorm, logits, topk_idx, topk_w, s);
  return hipGetLastError();
}
