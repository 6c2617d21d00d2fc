// route.hip -- router scoring, softmax and top-k selection in one launch.
//
// "DeepGEMM walkthrough" §2.1: p = Softmax(W_r x); keep the k highest
// scoring experts; the same p weights the combine.  "Dense GEMM to TP MoE"
// §4.2: the router is a linear layer with weight [num_experts][hidden_dim].
//
// One workgroup (4 waves) scores 16 tokens against all E experts:
//   phase 1  logits.  bf16: MFMA v_mfma_f32_16x16x32_bf16, expert blocks of
//            16, the K loop split across the 4 waves in 32-wide chunks; each
//            wave leaves its partial sums in LDS and they are added in wave
//            order (deterministic).  fp32: one thread per (token, expert)
//            dot product.
//   phase 2  one wave per token: logits (+bias) to registers (E/64 per lane),
//            wave max, wave sum of exp, then k rounds of a wave-wide argmax
//            with the key (logit descending, index ascending).
#include "moe_internal.h"

namespace {

using namespace moe;

constexpr int kTok = 16;       // tokens per workgroup
constexpr int kThreads = 256;  // 4 waves
constexpr int kEChunk = 256;   // experts scored per pass of phase 1
constexpr int kMaxPerLane = MOE_MAX_EXPERTS / kWave;  // 16

// LDS layout (dynamic): part[4][kTok][ec + 4] partial logits of one expert
// chunk (ec = experts per chunk, a multiple of 16, at most kEChunk), then
// s_logit[kTok][E] final logits.
__host__ __device__ inline int route_chunk(int E) { return min((E + 15) / 16 * 16, kEChunk); }

__device__ __forceinline__ float &part_at(float *part, int ec, int w, int ti, int e) {
  return part[(w * kTok + ti) * (ec + 4) + e];
}

// phase 1, bf16: partial logits of 16 tokens x one expert chunk into
// part[wave][tok][e].  Expert rows >= E and tokens >= T read as zero.
__device__ void logits_bf16_chunk(const uint16_t *__restrict__ x,
                                  const uint16_t *__restrict__ wr, int T, int d, int E,
                                  int t0, int e0, float *part, int ec) {
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  const int nblk = min((E - e0 + 15) / 16, ec / 16);
  f32x4 acc[kEChunk / 16];
#pragma unroll
  for (int b = 0; b < kEChunk / 16; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int r = lane & 15;         // token / expert row inside a 16-block
  const int kofs = (lane >> 4) * 8;  // 8 consecutive k per lane
  const int tok = t0 + r;
  const int nchunk = (d + 31) / 32;
#pragma unroll 2
  for (int c = wv; c < nchunk; c += 4) {
    const int k = c * 32 + kofs;
    bf16x8 a;
    if (tok < T && k < d)
      a = *reinterpret_cast<const bf16x8 *>(x + (size_t)tok * d + k);
    else
      a = bf16x8{};
#pragma unroll
    for (int b = 0; b < kEChunk / 16; ++b) {
      if (b < nblk) {
        const int e = e0 + b * 16 + r;
        bf16x8 bv;
        if (e < E && k < d)
          bv = *reinterpret_cast<const bf16x8 *>(wr + (size_t)e * d + k);
        else
          bv = bf16x8{};
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc[b], 0, 0, 0);
      }
    }
  }
  // 16x16 output block: lane holds column (expert) lane%16 and rows
  // (tokens) 4*(lane/16) + i
#pragma unroll
  for (int b = 0; b < kEChunk / 16; ++b) {
    if (b < nblk) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        part_at(part, ec, wv, (lane >> 4) * 4 + i, b * 16 + (lane & 15)) = acc[b][i];
    }
  }
}

// phase 1, fp32: one thread per (token, expert) dot product, sequential in c.
__device__ void logits_f32_chunk(const float *__restrict__ x, const float *__restrict__ wr,
                                 int T, int d, int E, int t0, int e0, float *part, int ec) {
  const int ne = min(E - e0, ec);
  for (int p = threadIdx.x; p < kTok * ne; p += kThreads) {
    const int ti = p / ne, ei = p % ne;
    const int t = t0 + ti, e = e0 + ei;
    float acc = 0.f;
    if (t < T) {
      const float *xr = x + (size_t)t * d;
      const float *wrow = wr + (size_t)e * d;
      for (int c = 0; c < d; ++c) acc = fmaf(xr[c], wrow[c], acc);
    }
    part_at(part, ec, 0, ti, ei) = acc;
    part_at(part, ec, 1, ti, ei) = 0.f;
    part_at(part, ec, 2, ti, ei) = 0.f;
    part_at(part, ec, 3, ti, ei) = 0.f;
  }
}

template <bool BF16, bool FROM_LOGITS>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const void *__restrict__ xv, const void *__restrict__ wrv, const float *__restrict__ bias,
    int T, int d, int E, int k, int renorm, const float *__restrict__ logits_in,
    float *__restrict__ logits_out, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w) {
  extern __shared__ float smem[];
  const int ec = route_chunk(E);
  float *part = smem;
  float *s_logit = smem + 4 * kTok * (ec + 4);

  const int t0 = blockIdx.x * kTok;
  const int lane = lane_id(), wv = threadIdx.x / kWave;

  if (!FROM_LOGITS) {
    for (int e0 = 0; e0 < E; e0 += kEChunk) {
      if (BF16)
        logits_bf16_chunk(static_cast<const uint16_t *>(xv), static_cast<const uint16_t *>(wrv),
                          T, d, E, t0, e0, part, ec);
      else
        logits_f32_chunk(static_cast<const float *>(xv), static_cast<const float *>(wrv), T, d,
                         E, t0, e0, part, ec);
      __syncthreads();
      const int ne = min(E - e0, ec);
      for (int p = threadIdx.x; p < kTok * ne; p += kThreads) {
        const int ti = p / ne, ei = p % ne;
        float v = part_at(part, ec, 0, ti, ei);
        v += part_at(part, ec, 1, ti, ei);
        v += part_at(part, ec, 2, ti, ei);
        v += part_at(part, ec, 3, ti, ei);
        if (bias) v += bias[e0 + ei];
        s_logit[ti * E + e0 + ei] = v;
      }
      __syncthreads();
    }
  }

  // phase 2: one wave per token
  for (int ti = wv; ti < kTok; ti += 4) {
    const int t = t0 + ti;
    if (t >= T) break;
    float v[kMaxPerLane];
    int nper = (E + kWave - 1) / kWave;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + i * kWave;
      float val = -INFINITY;
      if (i < nper && e < E) {
        if (FROM_LOGITS)
          val = logits_in[(size_t)t * E + e];
        else {
          val = s_logit[ti * E + e];
          if (logits_out) logits_out[(size_t)t * E + e] = val;
        }
      }
      v[i] = val;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) mx = fmaxf(mx, v[i]);
    mx = wave_max(mx);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + i * kWave;
      if (i < nper && e < E) z += expf(v[i] - mx);
    }
    z = wave_sum(z);

    uint32_t taken = 0;
    float my_w = 0.f;
    int my_idx = 0;
    for (int j = 0; j < k; ++j) {
      // best untaken candidate held by this lane
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + i * kWave;
        if (i < nper && e < E && !((taken >> i) & 1u)) {
          if (v[i] > bv || (v[i] == bv && e < be)) { bv = v[i]; be = e; }
        }
      }
      // wave-wide argmax on (value desc, index asc)
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oe = __shfl_xor(be, o, kWave);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
      if (lane == j) {
        my_idx = be;
        my_w = expf(bv - mx) / z;
      }
    }
    if (renorm) {
      const float s = wave_sum(lane < k ? my_w : 0.f);
      my_w = my_w / s;
    }
    if (lane < k) {
      topk_idx[(size_t)t * k + lane] = my_idx;
      topk_w[(size_t)t * k + lane] = my_w;
    }
  }
}

}  // namespace

hipError_t launch_route(const void *x, const void *w_router, int dt, const float *bias, int T,
                        int d, int E, int k, unsigned flags, float *logits, int32_t *topk_idx,
                        float *topk_w, hipStream_t s) {
  const dim3 grid((T + kTok - 1) / kTok), block(kThreads);
  const int renorm = (flags & MOE_ROUTE_RENORM) ? 1 : 0;
  const size_t lds = sizeof(float) * (size_t)(4 * kTok * (route_chunk(E) + 4) + kTok * E);
  if (flags & MOE_ROUTE_FROM_LOGITS) {
    hipLaunchKernelGGL((route_kernel<true, true>), grid, block, 0, s, x, w_router, bias, T, d, E,
                       k, renorm, logits, nullptr, topk_idx, topk_w);
  } else if (dt == MOE_BF16) {
    hipLaunchKernelGGL((route_kernel<true, false>), grid, block, lds, s, x, w_router, bias, T, d,
                       E, k, renorm, nullptr, logits, topk_idx, topk_w);
  } else {
    hipLaunchKernelGGL((route_kernel<false, false>), grid, block, lds, s, x, w_router, bias, T,
                       d, E, k, renorm, nullptr, logits, topk_idx, topk_w);
  }
  return hipGetLastError();
}
