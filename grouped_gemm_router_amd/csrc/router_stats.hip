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
// One launch, one workgroup, no atomics (bit-identical run to run).  The
// router's selection already computes every token's softmax, and writes the
// per-expert sum of the probabilities of each block of 16 tokens
// (prob_sums); this kernel adds the blocks (split over up to 1024/E threads
// per expert, recombined in a fixed order) into P_e = sum / T, forms f_e,
// and the three scalars through fixed-order block reductions.
#include "moe_internal.h"

namespace {

using namespace moe;

constexpr int kRB = 16;  // tokens per probability-sum block (as the router writes them)

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

hipError_t launch_router_stats(const float *prob_sums, const int32_t *counts, int T, int E, int k,
                               float alpha, float *f, float *P, float *summary, hipStream_t s) {
  const int nblk = (T + kRB - 1) / kRB;
  hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(1024), 0, s, prob_sums, nblk, counts, T, E,
                     k, alpha, f, P, summary);
  return hipGetLastError();
}
