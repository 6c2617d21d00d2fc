// router_stats.hip -- load-balance statistics of one routing decision,
// forward only.
//
// "DeepGEMM walkthrough" §2.2: L_aux = alpha * E * sum_i f_i * P_i, with f_i
// the share of routed tokens that went to expert i and P_i its mean gate
// probability (here f_i = counts_i / (T*k), so sum f = 1 and a uniform
// router gives alpha); "Dense GEMM to TP MoE" §5.1: max/mean of the expert
// token counts (above 3 is a severe imbalance); "DeepSeek MoE evolution"
// §2.3: entropy -sum q_i log2(q_i + 1e-8) of the count distribution q.
//
// Two launches, no atomics (the results are bit-identical run to run):
//   partial  one workgroup per 16 tokens: the softmax maximum and
//            normaliser of each token (as the router takes them; several
//            tokens per wave when E <= 64), then per expert the sum of
//            p[t][e] over the block's tokens, split over token slices that
//            are added in a fixed order, into the workspace [block][E];
//   final    one workgroup: P_e = (sum over blocks, split over up to 1024/E
//            threads per expert and recombined in a fixed order) / T, f_e,
//            and the three scalars through fixed-order block reductions.
#include "moe_internal.h"

namespace {

using namespace moe;

constexpr int kRB = 16;         // tokens per partial block (256 blocks at T = 4096)
constexpr int kThreads = 256;   // 4 waves
constexpr int kMaxPerLane = MOE_MAX_EXPERTS / kWave;

// max / sum over aligned segments of S lanes (S a power of two <= 64)
template <int S>
__device__ __forceinline__ float seg_max(float v) {
#pragma unroll
  for (int o = S / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
template <int S>
__device__ __forceinline__ float seg_sum(float v) {
#pragma unroll
  for (int o = S / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Softmax maximum and normaliser of the block's tokens.  S <= 64: a token
// per S-lane segment (64/S tokens per wave and pass); S == 0: a wave per
// token, E/64 values per lane (E > 64).
template <int S>
__device__ __forceinline__ void block_softmax_norms(const float *__restrict__ logits, int t0,
                                                    int nt, int E, float *s_mx, float *s_z) {
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  constexpr int NW = kThreads / kWave;
  if constexpr (S > 0) {
    constexpr int TPW = kWave / S;  // tokens per wave and pass
    const int e = lane % S;
    for (int base = wv * TPW; base < nt; base += NW * TPW) {
      const int i = base + lane / S;
      const bool ok = i < nt && e < E;
      const float v = ok ? logits[(size_t)(t0 + i) * E + e] : -INFINITY;
      const float mx = seg_max<S>(v);
      const float z = seg_sum<S>(ok ? expf(v - mx) : 0.f);
      if (e == 0 && i < nt) {
        s_mx[i] = mx;
        s_z[i] = z;
      }
    }
  } else {
    const int nper = (E + kWave - 1) / kWave;
    for (int i = wv; i < nt; i += NW) {
      const float *l = logits + (size_t)(t0 + i) * E;
      float v[kMaxPerLane];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j) {
        const int e = lane + j * kWave;
        v[j] = (j < nper && e < E) ? l[e] : -INFINITY;
        mx = fmaxf(mx, v[j]);
      }
      mx = wave_max(mx);
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j) {
        const int e = lane + j * kWave;
        if (j < nper && e < E) z += expf(v[j] - mx);
      }
      z = wave_sum(z);
      if (lane == 0) {
        s_mx[i] = mx;
        s_z[i] = z;
      }
    }
  }
}

template <int S>
__global__ __launch_bounds__(kThreads) void stats_partial_kernel(const float *__restrict__ logits,
                                                                 int T, int E,
                                                                 float *__restrict__ part) {
  __shared__ float s_mx[kRB], s_z[kRB];
  __shared__ float s_part[kThreads];
  const int t0 = blockIdx.x * kRB;
  const int nt = min(kRB, T - t0);
  block_softmax_norms<S>(logits, t0, nt, E, s_mx, s_z);
  __syncthreads();
  // sum_t p[t][e] over the block: thread (slice, e) takes tokens slice,
  // slice + NS, ... in order; the NS slice sums are then added in order
  const int tid = threadIdx.x;
  const int NS = E < kThreads ? kThreads / E : 1;  // token slices
  for (int e0 = 0; e0 < E; e0 += kThreads) {
    const int e = e0 + tid % E, sl = tid / E;
    float acc = 0.f;
    if (sl < NS && e < E)
      for (int i = sl; i < nt; i += NS)
        acc += expf(logits[(size_t)(t0 + i) * E + e] - s_mx[i]) / s_z[i];
    if (NS > 1) {
      s_part[tid] = acc;
      __syncthreads();
      if (tid < E) {
        float sum = 0.f;
        for (int j = 0; j < NS; ++j) sum += s_part[j * E + tid];
        part[(size_t)blockIdx.x * E + tid] = sum;
      }
      __syncthreads();
    } else if (sl < NS && e < E) {  // one slice: threads past E have nothing
      part[(size_t)blockIdx.x * E + e] = acc;
    }
  }
}

// sum (or max) over the 1024 threads in a fixed order; every thread gets it
__device__ __forceinline__ float block_reduce(float v, bool is_max, float *s_wave) {
  const int lane = lane_id(), wv = threadIdx.x / kWave;
  v = is_max ? wave_max(v) : wave_sum(v);
  if (lane == 0) s_wave[wv] = v;
  __syncthreads();
  float r = is_max ? -INFINITY : 0.f;
  for (int w = 0; w < 16; ++w) r = is_max ? fmaxf(r, s_wave[w]) : r + s_wave[w];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(1024) void stats_final_kernel(const float *__restrict__ part, int nblk,
                                                           const int32_t *__restrict__ counts,
                                                           int T, int E, int k, float alpha,
                                                           float *__restrict__ f,
                                                           float *__restrict__ P,
                                                           float *__restrict__ summary) {
  __shared__ float s_wave[16];
  __shared__ float s_part[1024];
  // R threads per expert: thread (r, e) sums blocks r, r + R, ... in order
  // (eight loads in flight), then thread r = 0 adds the R sums in r order
  const int R = max(1, min(1024 / E, nblk));
  {
    const int ee = threadIdx.x % E, r = threadIdx.x / E;
    if (r < R && (int)threadIdx.x < R * E) {
      float acc = 0.f;
      for (int b0 = r; b0 < nblk; b0 += 8 * R) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int b = b0 + i * R;
          v[i] = b < nblk ? part[(size_t)b * E + ee] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += v[i];
      }
      s_part[r * E + ee] = acc;
    }
  }
  __syncthreads();
  const int e = threadIdx.x;
  float p = 0.f, fe = 0.f, c = 0.f;
  if (e < E) {
    for (int r = 0; r < R; ++r) p += s_part[r * E + e];
    p /= (float)T;
    c = (float)counts[e];
    fe = c / ((float)T * (float)k);
    P[e] = p;
    f[e] = fe;
  }
  const float dot = block_reduce(fe * p, false, s_wave);
  const float total = block_reduce(c, false, s_wave);
  const float cmax = block_reduce(c, true, s_wave);
  const float q = (e < E && total > 0.f) ? c / total : 0.f;
  const float ent = block_reduce(e < E ? -q * log2f(q + 1e-8f) : 0.f, false, s_wave);
  if (e == 0) {
    summary[0] = alpha * (float)E * dot;
    summary[1] = total > 0.f ? cmax / (total / (float)E) : 0.f;
    summary[2] = ent;
  }
}

}  // namespace

size_t router_stats_ws_bytes(int T, int E) {
  return sizeof(float) * (size_t)((T + kRB - 1) / kRB) * (size_t)E;
}

hipError_t launch_router_stats(const float *logits, const int32_t *counts, int T, int E, int k,
                               float alpha, float *f, float *P, float *summary, float *ws,
                               hipStream_t s) {
  const int nblk = (T + kRB - 1) / kRB;
  const dim3 g(nblk), b(kThreads);
  if (E <= 8) hipLaunchKernelGGL(stats_partial_kernel<8>, g, b, 0, s, logits, T, E, ws);
  else if (E <= 16) hipLaunchKernelGGL(stats_partial_kernel<16>, g, b, 0, s, logits, T, E, ws);
  else if (E <= 32) hipLaunchKernelGGL(stats_partial_kernel<32>, g, b, 0, s, logits, T, E, ws);
  else if (E <= 64) hipLaunchKernelGGL(stats_partial_kernel<64>, g, b, 0, s, logits, T, E, ws);
  else hipLaunchKernelGGL(stats_partial_kernel<0>, g, b, 0, s, logits, T, E, ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(1024), 0, s, ws, nblk, counts, T, E, k,
                     alpha, f, P, summary);
  return hipGetLastError();
}
