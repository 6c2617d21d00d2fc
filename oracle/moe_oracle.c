/*
 * moe_oracle.c -- plain, slow CPU oracle for the MoE expert-layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that tests/, the smoke check and the CPU
 * baseline leg of the benchmark can compare the HIP library against an
 * obviously correct computation.  It shares no code, table or helper with the
 * HIP kernels.
 *
 * Everything floating point is done in double precision, in the order the
 * definitions below state, with no blocking or fusion.  Page citations name
 * the source page by its short title:
 *   "DeepGEMM walkthrough"  = the MegaMoE maths / DeepGEMM source walk-through
 *                             page (2kiu.com news 6052262)
 *   "Dense GEMM to TP MoE"  = the grouped-GEMM / TP-MoE page (2kiu.com news
 *                             6174947)
 *
 * Parity status of each function is listed in its comment ("pinned by ...").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_E4M3 2

/* ------------------------------------------------------------------------ */
/* element access                                                            */
/* ------------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double elem(const void *p, int dt, int64_t i) {
  if (dt == ORC_F32) return (double)((const float *)p)[i];
  return bf16_bits_to_double(((const uint16_t *)p)[i]);
}

static float elem_f32(const void *p, int dt, int64_t i) {
  return (float)elem(p, dt, i); /* exact for both fp32 and bf16 */
}

/* ------------------------------------------------------------------------ */
/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no infinities, */
/* S.1111.111 is NaN, largest finite magnitude 448.                          */
/* ------------------------------------------------------------------------ */

/* Value of a code, read straight from the format definition. */
double orc_e4m3_value(uint8_t q) {
  int sign = q >> 7;
  int e = (q >> 3) & 15;
  int m = q & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, 1 - 7); /* subnormal: 0.m x 2^(1-bias) */
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7); /* normal: 1.m x 2^(e-bias) */
  return sign ? -v : v;
}

/*
 * Round a binary32 value to the nearest finite E4M3 code, ties to the code
 * with an even mantissa (round-half-to-even), saturating to +-448.  The sign
 * bit of the input is kept, so values that round to zero give +0 or -0.
 * Method: binary search over the 127 non-negative finite code values, which
 * increase with the code; then compare the two neighbours.
 */
uint8_t orc_e4m3_round(float y) {
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs((double)y);
  int lo = 0, hi = 126; /* code 126 = 0x7E = 448 */
  if (isnan(y)) return 0x7F;
  if (a >= orc_e4m3_value(126)) return sign | 126;
  /* invariant: value(lo) <= a < value(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (orc_e4m3_value((uint8_t)mid) <= a)
      lo = mid;
    else
      hi = mid;
  }
  {
    double dlo = a - orc_e4m3_value((uint8_t)lo);
    double dhi = orc_e4m3_value((uint8_t)hi) - a;
    int c;
    if (dlo < dhi)
      c = lo;
    else if (dhi < dlo)
      c = hi;
    else
      c = (lo % 2 == 0) ? lo : hi; /* tie: even mantissa LSB */
    return sign | (uint8_t)c;
  }
}

/*
 * Block quantisation (DeepGEMM walkthrough, §2.3 and §5.1: per-token,
 * per-group or per-block scale factors so that outliers do not ruin a whole
 * tensor).  v is a dense R x C binary32 matrix cut into br x bc blocks (the
 * last block in each direction may be short).  For every block:
 *   s = absmax(block) / 448  (binary32; s = 1 when the block is all zero)
 *   q = E4M3 round of (v / s), binary32 IEEE division, saturating
 * so that v ~ q * s.  s is stored row-major [ceil(R/br)][ceil(C/bc)].
 * Pinned by: exhaustive code-point / midpoint tests and the library cast
 * (tests/test_oracle_fp8.py).
 */
static void quant_one_block(const float *v, int64_t C, int64_t r0, int64_t r1,
                            int64_t c0, int64_t c1, uint8_t *q, float *s_out) {
  float amax = 0.0f, sc;
  for (int64_t r = r0; r < r1; ++r)
    for (int64_t c = c0; c < c1; ++c) {
      float a = fabsf(v[r * C + c]);
      if (a > amax) amax = a;
    }
  sc = amax > 0.0f ? amax / 448.0f : 1.0f;
  *s_out = sc;
  for (int64_t r = r0; r < r1; ++r)
    for (int64_t c = c0; c < c1; ++c) {
      float t = v[r * C + c] / sc;
      q[r * C + c] = orc_e4m3_round(t);
    }
}

void orc_quant_blocks(const float *v, int64_t R, int64_t C, int br, int bc,
                      uint8_t *q, float *s) {
  int64_t nbr = (R + br - 1) / br, nbc = (C + bc - 1) / bc;
#pragma omp parallel for schedule(dynamic)
  for (int64_t b = 0; b < nbr * nbc; ++b) {
    int64_t rb = b / nbc, cb = b % nbc;
    int64_t r0 = rb * br, c0 = cb * bc;
    int64_t r1 = r0 + br < R ? r0 + br : R, c1 = c0 + bc < C ? c0 + bc : C;
    quant_one_block(v, C, r0, r1, c0, c1, q, &s[rb * nbc + cb]);
  }
}

/* ------------------------------------------------------------------------ */
/* Router (DeepGEMM walkthrough §2.1: p = Softmax(W_r x); keep the k highest */
/* scoring experts; Dense GEMM to TP MoE §4.2: the router is a linear layer  */
/* with weight [num_experts][hidden_dim], then softmax, then top-k).         */
/* ------------------------------------------------------------------------ */

/*
 * logits[t][e] = sum_c x[t][c] * w_r[e][c] (+ bias[e]) in fp64.
 * absdot[t][e] = sum_c |x[t][c] * w_r[e][c]| (for rounding-error bounds).
 * Pinned by: numpy fp64 matmul on random inputs.
 */
void orc_router_logits(const void *x, const void *w_r, int dt,
                       const float *bias, int64_t T, int64_t d, int64_t E,
                       double *logits, double *absdot) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0, aacc = 0.0;
      for (int64_t c = 0; c < d; ++c) {
        double p = elem(x, dt, t * d + c) * elem(w_r, dt, e * d + c);
        acc += p;
        aacc += fabs(p);
      }
      if (bias) acc += (double)bias[e];
      logits[t * E + e] = acc;
      if (absdot) absdot[t * E + e] = aacc;
    }
}

/*
 * Selection and gate weights from binary32 logits.
 *   idx[t][j]: the k experts with the largest logit, in the order
 *              (logit descending, expert index ascending); equal logits
 *              (including -0 vs +0) go to the lower expert index.
 *   w[t][j]  = p[idx[t][j]], p = softmax over all E experts, computed in fp64
 *              as exp(l - max l) / sum exp(l - max l).
 *   renorm   : w[t][j] /= sum_j w[t][j] (softmax restricted to the top-k).
 * Selection is done by k passes of "largest not yet taken" with a strict
 * comparison, which keeps the first (lowest) index among equal values.
 * Pinned by: brute force sorted() on tiny inputs, closed forms (equal
 * logits -> 1/E; E = 2 -> logistic function).
 */
void orc_topk(const float *logits, int64_t T, int E, int k, int renorm,
              int32_t *idx, double *w) {
#pragma omp parallel
  {
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
      const float *l = logits + t * E;
      double mx = -INFINITY, z = 0.0, wsum = 0.0;
      memset(taken, 0, (size_t)E);
      for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
          if (taken[e]) continue;
          if (best < 0 || l[e] > l[best]) best = e;
        }
        taken[best] = 1;
        idx[t * k + j] = best;
      }
      for (int e = 0; e < E; ++e)
        if ((double)l[e] > mx) mx = (double)l[e];
      for (int e = 0; e < E; ++e) z += exp((double)l[e] - mx);
      for (int j = 0; j < k; ++j) {
        w[t * k + j] = exp((double)l[idx[t * k + j]] - mx) / z;
        wsum += w[t * k + j];
      }
      if (renorm)
        for (int j = 0; j < k; ++j) w[t * k + j] /= wsum;
    }
    free(taken);
  }
}

/* ------------------------------------------------------------------------ */
/* Histogram, offsets and the expert-contiguous permutation                  */
/* (Dense GEMM to TP MoE §2.2 data flow steps 3-4 and §4.2: bincount, then    */
/* offsets = cumsum(counts) - counts; scatter tokens by those offsets).       */
/* ------------------------------------------------------------------------ */

/*
 * counts[e] = number of (t, j) with idx[t][j] == e.
 * offsets[0] = 0, offsets[g+1] = offsets[g] + size of group g, where groups
 * 0..E-1 are the routed experts and groups E..E+n_shared-1 are shared
 * experts holding all T tokens each.  Returns -1 on an out-of-range index.
 * Pinned by: numpy bincount + cumsum.
 */
int orc_counts_offsets(const int32_t *idx, int64_t T, int k, int E,
                       int n_shared, int32_t *counts, int32_t *offsets) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < T * k; ++f) {
    if (idx[f] < 0 || idx[f] >= E) return -1;
    counts[idx[f]] += 1;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  for (int s = 0; s < n_shared; ++s)
    offsets[E + s + 1] = offsets[E + s] + (int32_t)T;
  return 0;
}

/*
 * Stable counting sort of the flat indices f = t*k + j by key idx[f]:
 *   perm_src[offsets[e] + r] = the r-th flat index (ascending) with key e,
 *   flat_to_row[f]           = the row f lands on (inverse permutation).
 * Pinned by: numpy argsort(kind="stable").
 */
void orc_permutation(const int32_t *idx, int64_t T, int k, int E,
                     const int32_t *offsets, int32_t *perm_src,
                     int32_t *flat_to_row) {
  int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  for (int e = 0; e < E; ++e) fill[e] = offsets[e];
  for (int64_t f = 0; f < T * k; ++f) {
    int32_t r = fill[idx[f]]++;
    perm_src[r] = (int32_t)f;
    flat_to_row[f] = r;
  }
  free(fill);
}

/*
 * Capacity-limited permutation ("Dense GEMM to TP MoE" §5.1: at inference a
 * capacity factor caps how many tokens each expert takes and the excess
 * goes down a fallback path; "DeepSeek MoE evolution" §3.2 on the cap as a
 * bound on the tokens one expert takes in one forward pass).  Reading: the
 * cap is an integer number of rows per expert; an expert keeps its first
 * `capacity` routed entries in flat order f = t*k + j and drops the rest.
 *   counts[e]       = routed entries of expert e (before the cap)
 *   offsets         = exclusive prefix of min(counts[e], capacity), then
 *                     n_shared groups of T rows
 *   perm_src, flat_to_row as in orc_permutation for kept entries;
 *   flat_to_row[f]  = -1 for a dropped entry;
 *   flat_to_row[T*k + s*T + t] = offsets[E] + s*T + t (shared rows)
 *   overflow        = dropped flat indices, expert by expert, each
 *                     expert's in ascending f, starting at the exclusive
 *                     prefix of max(counts[e] - capacity, 0)
 *   returns the number of dropped entries (-1 for an index outside [0, E)).
 * Pinned by: numpy stable argsort grouped by expert and sliced at the cap;
 * capacity >= max count reproduces orc_permutation.
 */
int64_t orc_capacity_permutation(const int32_t *idx, int64_t T, int k, int E, int n_shared,
                                 int64_t capacity, int32_t *counts, int32_t *offsets,
                                 int32_t *perm_src, int32_t *flat_to_row, int32_t *overflow) {
  if (E <= 0 || capacity < 0) return -1;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t f = 0; f < T * k; ++f) {
    if (idx[f] < 0 || idx[f] >= E) return -1;
    counts[idx[f]] += 1;
  }
  int64_t *ov_start = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
  int64_t *seen = (int64_t *)calloc((size_t)E, sizeof(int64_t));
  int64_t n_over = 0;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) {
    int64_t kept = counts[e] < capacity ? counts[e] : capacity;
    offsets[e + 1] = offsets[e] + (int32_t)kept;
    ov_start[e] = n_over;
    n_over += counts[e] - kept;
  }
  for (int s = 0; s < n_shared; ++s) offsets[E + s + 1] = offsets[E + s] + (int32_t)T;
  for (int64_t f = 0; f < T * k; ++f) {
    int e = idx[f];
    int64_t r = seen[e]++;
    if (r < capacity) {
      int32_t row = offsets[e] + (int32_t)r;
      perm_src[row] = (int32_t)f;
      flat_to_row[f] = row;
    } else {
      flat_to_row[f] = -1;
      overflow[ov_start[e] + (r - capacity)] = (int32_t)f;
    }
  }
  for (int s = 0; s < n_shared; ++s)
    for (int64_t t = 0; t < T; ++t)
      flat_to_row[T * k + s * T + t] = offsets[E] + (int32_t)(s * T + t);
  free(ov_start);
  free(seen);
  return n_over;
}

/*
 * Router statistics for load balancing, forward only.
 *   p[t][e] = softmax over all E of the binary32 logits (fp64, max-subtracted,
 *             as in orc_topk)
 *   P[e]    = (1/T) sum_t p[t][e]       mean gate probability
 *   f[e]    = counts[e] / (T*k)         share of the routed entries
 *   aux     = alpha * E * sum_e f[e] P[e]
 *             ("DeepGEMM walkthrough" §2.2; reading: f is the share of the
 *             T*k routed entries, so sum f = 1 and a uniform router gives
 *             aux = alpha whatever E and k are)
 *   max_over_mean = max_e counts[e] / (sum_e counts[e] / E)
 *             ("Dense GEMM to TP MoE" §5.1: above 3 is a severe imbalance)
 *   entropy = -sum_e q[e] log2(q[e] + 1e-8), q = counts / sum counts
 *             ("DeepSeek MoE evolution" §2.3, in bits)
 * summary = {aux, max_over_mean, entropy}.
 * Pinned by: closed forms (equal logits -> P = 1/E; uniform counts ->
 * max/mean 1, entropy log2 E; one expert -> entropy 0, max/mean E) and scipy
 * softmax + numpy on random inputs.
 */
void orc_router_stats(const float *logits, int64_t T, int E, const int32_t *counts, int k,
                      double alpha, double *f, double *P, double *summary) {
  for (int e = 0; e < E; ++e) P[e] = 0.0;
  double *p = (double *)malloc(sizeof(double) * (size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    const float *l = logits + t * E;
    double mx = l[0];
    for (int e = 1; e < E; ++e)
      if (l[e] > mx) mx = l[e];
    double z = 0.0;
    for (int e = 0; e < E; ++e) {
      p[e] = exp((double)l[e] - mx);
      z += p[e];
    }
    for (int e = 0; e < E; ++e) P[e] += p[e] / z;
  }
  free(p);
  double total = 0.0, cmax = 0.0;
  for (int e = 0; e < E; ++e) {
    P[e] /= (double)T;
    f[e] = (double)counts[e] / ((double)T * (double)k);
    total += counts[e];
    if (counts[e] > cmax) cmax = counts[e];
  }
  double dot = 0.0, ent = 0.0;
  for (int e = 0; e < E; ++e) {
    dot += f[e] * P[e];
    double q = total > 0 ? counts[e] / total : 0.0;
    ent -= q * log2(q + 1e-8);
  }
  summary[0] = alpha * E * dot;
  summary[1] = total > 0 ? cmax / (total / E) : 0.0;
  summary[2] = ent;
}

/*
 * Gathers the permuted activation rows x_perm[r] for the rows listed in
 * row_list: row r < T*k copies x[perm_src[r] / k]; a shared-expert row
 * r = T*k + s*T + t copies x[t].  Rows are copied byte for byte.
 */
void orc_permute_rows(const void *x, int64_t elem_bytes, int64_t T, int64_t d,
                      int k, const int32_t *perm_src, const int64_t *row_list,
                      int64_t nrow, void *out) {
  int64_t rb = elem_bytes * d;
  for (int64_t i = 0; i < nrow; ++i) {
    int64_t r = row_list[i], t;
    if (r < T * k)
      t = perm_src[r] / k;
    else
      t = (r - T * k) % T;
    memcpy((char *)out + i * rb, (const char *)x + t * rb, (size_t)rb);
  }
}

/* ------------------------------------------------------------------------ */
/* Grouped GEMM (DeepGEMM walkthrough §4.3; Dense GEMM to TP MoE §2.1-2.2):  */
/* group g owns rows offsets[g] .. offsets[g+1]-1 of A and multiplies them  */
/* by its own weight B[g] ([N][K], output x input).                          */
/* ------------------------------------------------------------------------ */

static int group_of_row(const int32_t *offsets, int G, int64_t r) {
  for (int g = 0; g < G; ++g)
    if (r >= offsets[g] && r < offsets[g + 1]) return g;
  return -1;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * For each listed row r of group g:
 *   c[n] = sum_k A[r][k] * B[g][n][k]                        (epi = 0)
 *   c[n] = silu(sum_k A[r][k] B[g][n][k]) * sum_k A[r][k] B2[g][n][k]
 *                                                           (epi = 1)
 * in fp64.  Rows outside every group give NaN.
 * Pinned by: numpy fp64 matmul per group (G = 1 is a plain GEMM).
 */
void orc_gemm_rows(const void *A, int adt, const void *B, const void *B2,
                   int bdt, const int32_t *offsets, int G, int64_t N,
                   int64_t K, int epi, const int64_t *row_list, int64_t nrow,
                   double *out) {
#pragma omp parallel for schedule(dynamic)
  for (int64_t i = 0; i < nrow; ++i) {
    int64_t r = row_list[i];
    int g = group_of_row(offsets, G, r);
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0, acc2 = 0.0;
      if (g < 0) {
        out[i * N + n] = NAN;
        continue;
      }
      for (int64_t kk = 0; kk < K; ++kk) {
        double a = elem(A, adt, r * K + kk);
        acc += a * elem(B, bdt, ((int64_t)g * N + n) * K + kk);
        if (epi) acc2 += a * elem(B2, bdt, ((int64_t)g * N + n) * K + kk);
      }
      out[i * N + n] = epi ? silu(acc) * acc2 : acc;
    }
  }
}

/*
 * FP8 block-scaled variant (DeepGEMM walkthrough §2.3: C is approximately
 * the product of the dequantised operands; §5.1: scales per token / group /
 * block, fp32 accumulation).  The stored scales are dequantisation
 * multipliers: A[r][k] ~ Aq[r][k] * As[r][k/128] and
 * B[g][n][k] ~ Bq[g][n][k] * Bs[g][n/128][k/128].  Written out as the plain
 * product of the dequantised matrices, in fp64.
 * Pinned by: numpy fp64 matmul of the dequantised matrices.
 */
void orc_gemm_fp8_rows(const uint8_t *Aq, const float *As, const uint8_t *Bq,
                       const float *Bs, const uint8_t *B2q, const float *B2s,
                       const int32_t *offsets, int G, int64_t N, int64_t K,
                       int epi, const int64_t *row_list, int64_t nrow,
                       double *out) {
  int64_t kb = K / 128, nb = N / 128;
#pragma omp parallel for schedule(dynamic)
  for (int64_t i = 0; i < nrow; ++i) {
    int64_t r = row_list[i];
    int g = group_of_row(offsets, G, r);
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0, acc2 = 0.0;
      if (g < 0) {
        out[i * N + n] = NAN;
        continue;
      }
      for (int64_t kk = 0; kk < K; ++kk) {
        double a = orc_e4m3_value(Aq[r * K + kk]) * (double)As[r * kb + kk / 128];
        int64_t bi = ((int64_t)g * N + n) * K + kk;
        int64_t si = ((int64_t)g * nb + n / 128) * kb + kk / 128;
        acc += a * orc_e4m3_value(Bq[bi]) * (double)Bs[si];
        if (epi) acc2 += a * orc_e4m3_value(B2q[bi]) * (double)B2s[si];
      }
      out[i * N + n] = epi ? silu(acc) * acc2 : acc;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* The whole layer, one token at a time                                      */
/* (DeepGEMM walkthrough §2.1: y = E_shared(x) + sum over the top-k experts  */
/* of p_i * E_i(x); Dense GEMM to TP MoE §2.2: each expert is an up and a    */
/* down projection; the activation between them is SwiGLU, h = silu(x Wg) * */
/* (x Wu), y = h Wd).                                                         */
/* ------------------------------------------------------------------------ */

typedef struct {
  int mode;          /* ORC_F32 / ORC_BF16: weights in that type;
                        ORC_E4M3: E4M3 codes + fp32 block scales */
  int x_dt;          /* ORC_F32 or ORC_BF16 */
  int64_t T, d, dff;
  int E, k, n_shared;
  const void *x;     /* [T][d] */
  /* per group g < E + n_shared (routed experts first, then shared):
     gate/up [dff][d], down [d][dff]; NULL for groups never used */
  const void *const *wg;
  const void *const *wu;
  const void *const *wd;
  /* ORC_E4M3 only: 128x128 block scales [dff/128][d/128] (gate/up) and
     [d/128][dff/128] (down) */
  const float *const *sg;
  const float *const *su;
  const float *const *sd;
} orc_layer_t;

/*
 * One expert FFN on one input vector xin[d] (already dequantised in fp8
 * mode), result added as  out += scale * FFN_g(xin).  fp8 mode also
 * quantises h the way the down-projection input is quantised: h is rounded
 * to binary32 and cut into 1 x 128 groups with s = absmax / 448.
 */
static void expert_ffn_acc(const orc_layer_t *L, int g, const double *xin,
                           double scale, double *h, float *h32,
                           uint8_t *hq, double *out) {
  int64_t d = L->d, dff = L->dff;
  for (int64_t n = 0; n < dff; ++n) {
    double a = 0.0, b = 0.0;
    for (int64_t c = 0; c < d; ++c) {
      double wgv, wuv;
      if (L->mode == ORC_E4M3) {
        int64_t si = (n / 128) * (d / 128) + c / 128;
        wgv = orc_e4m3_value(((const uint8_t *)L->wg[g])[n * d + c]) *
              (double)L->sg[g][si];
        wuv = orc_e4m3_value(((const uint8_t *)L->wu[g])[n * d + c]) *
              (double)L->su[g][si];
      } else {
        wgv = elem(L->wg[g], L->mode, n * d + c);
        wuv = elem(L->wu[g], L->mode, n * d + c);
      }
      a += xin[c] * wgv;
      b += xin[c] * wuv;
    }
    h[n] = silu(a) * b;
  }
  if (L->mode == ORC_E4M3) {
    float hs[1];
    for (int64_t n0 = 0; n0 < dff; n0 += 128) {
      for (int64_t n = n0; n < n0 + 128; ++n) h32[n] = (float)h[n];
      quant_one_block(h32 + n0, 128, 0, 1, 0, 128, hq + n0, hs);
      for (int64_t n = n0; n < n0 + 128; ++n)
        h[n] = orc_e4m3_value(hq[n]) * (double)hs[0];
    }
  }
  for (int64_t c = 0; c < d; ++c) {
    double o = 0.0;
    for (int64_t n = 0; n < dff; ++n) {
      double wdv;
      if (L->mode == ORC_E4M3)
        wdv = orc_e4m3_value(((const uint8_t *)L->wd[g])[c * dff + n]) *
              (double)L->sd[g][(c / 128) * (dff / 128) + n / 128];
      else
        wdv = elem(L->wd[g], L->mode, c * dff + n);
      o += h[n] * wdv;
    }
    out[c] += scale * o;
  }
}

/*
 * Layer output for the listed tokens, given the routing decision
 * (idx[T][k], w[T][k]).  Per token t:
 *   xin = x[t]            (fp8 mode: dequantised 1x128-group E4M3 of x[t])
 *   y[t] = sum_j w[t][j] * FFN_{idx[t][j]}(xin) + sum_s FFN_{E+s}(xin)
 * all in fp64, j ascending.  Returns -1 if a needed weight pointer is NULL.
 * Pinned by: the dense all-experts-masked brute force in numpy and the
 * hand-worked two-expert case.
 */
int orc_moe_tokens(const orc_layer_t *L, const int32_t *idx, const double *w,
                   const int64_t *tok, int64_t ntok, double *out) {
  int bad = 0;
  for (int64_t i = 0; i < ntok; ++i) {
    for (int j = 0; j < L->k; ++j) {
      int g = idx[tok[i] * L->k + j];
      if (!L->wg[g] || !L->wu[g] || !L->wd[g]) bad = 1;
    }
    for (int s = 0; s < L->n_shared; ++s)
      if (!L->wg[L->E + s]) bad = 1;
  }
  if (bad) return -1;
#pragma omp parallel
  {
    int64_t d = L->d, dff = L->dff;
    double *xin = (double *)malloc(sizeof(double) * (size_t)d);
    double *h = (double *)malloc(sizeof(double) * (size_t)dff);
    float *h32 = (float *)malloc(sizeof(float) * (size_t)(dff > d ? dff : d));
    uint8_t *hq = (uint8_t *)malloc((size_t)(dff > d ? dff : d));
    float *xs = (float *)malloc(sizeof(float) * (size_t)(d / 128 + 1));
#pragma omp for schedule(dynamic)
    for (int64_t i = 0; i < ntok; ++i) {
      int64_t t = tok[i];
      double *y = out + i * d;
      for (int64_t c = 0; c < d; ++c) y[c] = 0.0;
      if (L->mode == ORC_E4M3) {
        for (int64_t c = 0; c < d; ++c) h32[c] = elem_f32(L->x, L->x_dt, t * d + c);
        for (int64_t c0 = 0; c0 < d; c0 += 128)
          quant_one_block(h32, d, 0, 1, c0, c0 + 128 < d ? c0 + 128 : d, hq,
                          &xs[c0 / 128]);
        for (int64_t c = 0; c < d; ++c)
          xin[c] = orc_e4m3_value(hq[c]) * (double)xs[c / 128];
      } else {
        for (int64_t c = 0; c < d; ++c) xin[c] = elem(L->x, L->x_dt, t * d + c);
      }
      for (int j = 0; j < L->k; ++j)
        expert_ffn_acc(L, idx[t * L->k + j], xin, w[t * L->k + j], h, h32 + 0,
                       hq, y);
      for (int s = 0; s < L->n_shared; ++s)
        expert_ffn_acc(L, L->E + s, xin, 1.0, h, h32, hq, y);
    }
    free(xin);
    free(h);
    free(h32);
    free(hq);
    free(xs);
  }
  return 0;
}

/*
 * Combine step on its own (Dense GEMM to TP MoE §2.2 step 6: gather the
 * expert outputs back to token order, multiply by the gate weight, sum):
 *   out[t][c] = sum_j w[t][j] * Y[flat_to_row[t*k+j]][c]
 *               + sum_s Y[T*k + s*T + t][c]
 * in fp64, j ascending.  Pinned by: numpy fancy indexing + einsum.
 */
void orc_combine(const void *Y, int ydt, const int32_t *flat_to_row,
                 const float *w, int64_t T, int k, int64_t d, int n_shared,
                 double *out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j)
        acc += (double)w[t * k + j] *
               elem(Y, ydt, (int64_t)flat_to_row[t * k + j] * d + c);
      for (int s = 0; s < n_shared; ++s)
        acc += elem(Y, ydt, (T * k + s * T + t) * d + c);
      out[t * d + c] = acc;
    }
}
