/*
 * moe.h -- C ABI of libmoe.so: the forward pass of a Mixture-of-Experts
 * expert layer on one AMD Instinct MI355X (gfx950), as hand-written HIP
 * kernels.
 *
 * The layer (source pages, by short title):
 *   "DeepGEMM walkthrough" -- the MegaMoE maths / DeepGEMM source
 *       walk-through page: §2.1 gives the router p = Softmax(W_r x), the
 *       top-k selection and y = E_shared(x) + sum_{i in top-k} p_i E_i(x);
 *       §2.3 gives the FP8 form C ~ (A_q / scale_A)(B_q / scale_B) scale_C;
 *       §4.3 the grouped GEMM over an expert-contiguous layout; §5.1-5.3
 *       scales, double buffering and ragged tails.
 *   "Dense GEMM to TP MoE" -- the grouped-GEMM / tensor-parallel MoE page:
 *       §2.2 gives the six-step data flow (score, top-k, per-expert count and
 *       prefix sum, scatter, grouped GEMM, gather + gate weight + sum);
 *       §2.3 the grouped_gemm(A_ptrs, B_ptrs, C_ptrs, expert_sizes, N, K,
 *       workspace, stream) call and the rule that expert sizes stay on the
 *       GPU; §4.2 the router and offset computation; §5.3-5.4 workspace
 *       sizing and GPU-built pointer arrays.
 *
 * One forward pass is five calls on one stream, with no host round trip:
 *   moe_route -> moe_permute -> moe_grouped_gemm(_fp8) (gate/up, SwiGLU)
 *             -> moe_grouped_gemm(_fp8) (down) -> moe_combine
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers to dense row-major arrays with
 *     no strides, 16-byte aligned (one exception: the grouped GEMMs' weights
 *     may have a row pitch ldb >= K).  The caller allocates and frees every
 *     buffer; the library never allocates, frees, synchronises or copies
 *     device data to the host.
 *   - Every call only enqueues kernels on `stream` (a hipStream_t; NULL is
 *     the null stream) and returns; results are ready when the stream is.
 *   - Sizes are checked on the host before anything is launched; a failed
 *     check returns a status and launches nothing.  T == 0 is a no-op.
 *   - Per-expert row counts exist only in the device array `offsets`; the
 *     host passes only sizes it already knows (T, k, E, rows = T*k +
 *     n_shared*T).
 *   - Weights are stored [group][out][in] (the F.linear orientation), so a
 *     GEMM computes C[r][n] = sum_k A[r][k] * B[g][n][k].  Routed experts are
 *     groups 0..E-1; shared experts are groups E..E+n_shared-1.
 *   - Kernels are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,     /* bad argument: null/misaligned pointer, size out of range */
  MOE_ERR_UNSUPPORTED = 2, /* valid but not implemented (dtype combination, shape) */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than the size query returned */
  MOE_ERR_LAUNCH = 4       /* the HIP runtime refused a kernel launch */
} moe_status_t;

typedef enum {
  MOE_F32 = 0,  /* IEEE binary32 */
  MOE_BF16 = 1, /* bfloat16 */
  MOE_E4M3 = 2  /* OCP FP8 E4M3FN: bias 7, no infinities, max 448 */
} moe_dtype_t;

typedef enum {
  MOE_EPI_NONE = 0,  /* C = A B^T */
  MOE_EPI_SWIGLU = 1 /* C = silu(A B^T) * (A B2^T), silu(z) = z / (1 + e^-z) */
} moe_epilogue_t;

typedef void *moe_stream_t; /* a hipStream_t */

/* moe_route flags */
#define MOE_ROUTE_RENORM 1u      /* w[t][j] /= sum_j w[t][j] (softmax over the k selected logits) */
#define MOE_ROUTE_FROM_LOGITS 2u /* `logits` is an input; x, w_router and logit_bias are ignored */

/* Library limits (checked on the host). */
#define MOE_MAX_EXPERTS 1024 /* E */
#define MOE_MAX_TOPK 32      /* k */
#define MOE_MAX_GROUPS 1040  /* G = E + n_shared in a grouped GEMM */

/* Static text for a status code (never NULL). */
const char *moe_status_string(moe_status_t status);

/* ABI version of this header; bumped on any incompatible change. */
int moe_abi_version(void);

/*
 * Router scoring and top-k selection ("DeepGEMM walkthrough" §2.1; "Dense
 * GEMM to TP MoE" §2.2 steps 1-2 and §4.2).
 *
 *   logits[t][e] = sum_c x[t][c] * w_router[e][c] + logit_bias[e]
 *                  (fp32 accumulation; bias optional)
 *   topk_idx[t][j] = the k experts with the largest logits, ordered by
 *                  (logit descending, expert index ascending): equal logits
 *                  (including -0 and +0) go to the lower index
 *   topk_w[t][j]   = p[topk_idx[t][j]], p = softmax(logits[t][.]) over all E
 *                  experts (max-subtracted, fp32); with MOE_ROUTE_RENORM
 *                  divided by sum_j topk_w[t][j]
 *
 * x [T][d] and w_router [E][d] are both of type `dt` (MOE_F32 or MOE_BF16).
 * logit_bias [E] fp32 or NULL.  logits [T][E] fp32: written if non-NULL; with
 * MOE_ROUTE_FROM_LOGITS it is read instead (and must be non-NULL).
 * topk_idx [T][k] int32, topk_w [T][k] fp32 are written.
 * prob_sums [ceil(T/16)][E] fp32 or NULL: if given, prob_sums[b][e] = the sum
 * over tokens t = 16 b .. min(16 b + 15, T - 1) of p_t[e] (the softmax over
 * all E, before any renormalisation), summed in a fixed order; it feeds
 * moe_router_stats.
 * ws (device, 4-byte aligned) holds the fp32 partial logits of the d-axis
 * slices; it must hold moe_route_workspace_size(T, d, E) bytes (else
 * MOE_ERR_WORKSPACE).  With MOE_ROUTE_FROM_LOGITS it is unused (may be NULL,
 * ws_bytes 0).
 * Requires 1 <= k <= min(E, MOE_MAX_TOPK), E <= MOE_MAX_EXPERTS, d % 8 == 0.
 * Non-finite logits are a caller error (selection is then unspecified).
 */
moe_status_t moe_route(const void *x, const void *w_router, moe_dtype_t dt,
                       const float *logit_bias, int T, int d, int E, int k,
                       unsigned flags, float *logits, int32_t *topk_idx,
                       float *topk_w, float *prob_sums, void *ws, size_t ws_bytes,
                       moe_stream_t stream);

/* Bytes of device workspace moe_route needs for these sizes (the router's
 * split-K partial logits: at most a small multiple of T * E * 4; 0 for
 * E <= 32, which routes in one launch). */
size_t moe_route_workspace_size(int T, int d, int E);

/* Bytes of device workspace moe_permute needs for these sizes. */
size_t moe_permute_workspace_size(int T, int k, int E);

/*
 * Per-expert histogram, exclusive prefix sum and stable scatter of tokens
 * into expert-contiguous order ("Dense GEMM to TP MoE" §2.2 steps 3-4, §4.2;
 * "DeepGEMM walkthrough" §4.3 on the contiguous per-expert layout).
 *
 *   counts[e]   = #{(t, j) : topk_idx[t][j] == e}                 [E]
 *   offsets[g]  = exclusive prefix sum of the group sizes          [E+n_shared+1]
 *                 (routed experts first, then n_shared groups of T rows each)
 *   perm_src[offsets[e] + r] = the r-th flat index f = t*k + j (ascending)
 *                 whose expert is e (a stable counting sort)       [T*k]
 *   flat_to_row[f] = the row that flat index f lands on, and
 *   flat_to_row[T*k + s*T + t] = the row of token t in shared group s
 *                 (= offsets[E] + s*T + t)             [T*k + n_shared*T]
 *   x_perm[row]  = x[perm_src[row] / k] for routed rows, and
 *   x_perm[offsets[E] + s*T + t] = x[t] for the shared groups
 *                                                    [T*k + n_shared*T][d]
 *
 * out_dt == x_dt copies rows bit for bit.  out_dt == MOE_E4M3 (x_dt F32 or
 * BF16) quantises every row in 1 x 128 groups ("DeepGEMM walkthrough" §2.3:
 * per-token, per-group scales): s = absmax / 448 (1 if the group is all
 * zero), q = E4M3 round-to-nearest-even of (x / s) with IEEE fp32 division,
 * saturating at +-448; x_perm_scale receives s group-major, [d/128][rows]
 * (scale of row r, group c at c * rows + r; rows = T*k + n_shared*T, so one
 * column group's scales are contiguous for the GEMM's K loop); d % 128 == 0
 * required.  Otherwise x_perm_scale must be NULL.
 * Each token's k experts must be distinct (top-k output always is).  An
 * entry of topk_idx outside [0, E) is dropped: it is counted nowhere, its
 * flat_to_row is -1 and no row is written for it; the rows stay compact
 * (offsets[E] is then below T*k).  Requires d % 8 == 0.
 * ws must hold moe_permute_workspace_size(T, k, E) bytes (else
 * MOE_ERR_WORKSPACE).  It holds per-block counts when the call runs as
 * three launches (T*k above 32768 entries, or E4M3 rows); a call of at most
 * 32768 entries with bf16 / fp32 rows runs as one launch and leaves ws
 * untouched.  Either way the results are the same, bit for bit.
 */
moe_status_t moe_permute(const void *x, moe_dtype_t x_dt, int T, int d,
                         const int32_t *topk_idx, int k, int E, int n_shared,
                         moe_dtype_t out_dt, void *x_perm, float *x_perm_scale,
                         int32_t *counts, int32_t *offsets, int32_t *perm_src,
                         int32_t *flat_to_row, void *ws, size_t ws_bytes,
                         moe_stream_t stream);

/* Bytes of the static device scratch moe_permute_noalloc uses. */
#define MOE_PERMUTE_NOALLOC_SCRATCH_BYTES (1u << 20)

/*
 * moe_permute without a workspace argument, for callers that cannot
 * allocate device memory at call time: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments (minus
 * ws / ws_bytes), same results, same kernels as moe_permute.
 * The per-block counts that moe_permute keeps in its workspace (three-launch
 * sizes) live instead in a library-owned static device array of
 * MOE_PERMUTE_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held until the
 * process ends; this call itself calls no allocator.  Sizes whose moe_permute_workspace_size(T, k, E) exceeds that
 * limit return MOE_ERR_WORKSPACE and launch nothing (the limit allows, e.g.,
 * T up to 65472 at E = 256 and T up to 16320 at E = 1024).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (the kernels write every value they read, so nothing needs
 * clearing between calls): two calls that can run at the same time on one
 * GPU (different streams, no ordering between them) race and give wrong
 * results.  Order them, e.g. on one stream.
 */
moe_status_t moe_permute_noalloc(const void *x, moe_dtype_t x_dt, int T, int d,
                                 const int32_t *topk_idx, int k, int E, int n_shared,
                                 moe_dtype_t out_dt, void *x_perm, float *x_perm_scale,
                                 int32_t *counts, int32_t *offsets, int32_t *perm_src,
                                 int32_t *flat_to_row, moe_stream_t stream);

/*
 * moe_permute with a per-expert capacity ("Dense GEMM to TP MoE" §5.1: at
 * inference a capacity factor caps the tokens each expert takes and the
 * excess goes to a fallback path; "DeepSeek MoE evolution" §3.2).
 * Expert e keeps its first `capacity` routed entries in flat order
 * f = t*k + j (the ones a stable sort puts first) and drops the rest:
 *   counts[e]     = routed entries of expert e (before the cap)
 *   offsets       = exclusive prefix of min(counts[e], capacity), then the
 *                   n_shared groups of T rows (rows stay compact)
 *   flat_to_row[f] = -1 for a dropped entry (moe_combine skips it, so the
 *                   token gets only its kept experts and the shared ones)
 *   overflow      = the dropped flat indices, expert by expert (ascending f
 *                   within an expert), [T*k] capacity, or NULL
 *   *n_overflow   = number of dropped entries, or NULL
 * Everything else as moe_permute (same workspace).  capacity >= 0; a
 * capacity of at least T gives exactly moe_permute's result.
 */
moe_status_t moe_permute_capped(const void *x, moe_dtype_t x_dt, int T, int d,
                                const int32_t *topk_idx, int k, int E, int n_shared,
                                int capacity, moe_dtype_t out_dt, void *x_perm,
                                float *x_perm_scale, int32_t *counts, int32_t *offsets,
                                int32_t *perm_src, int32_t *flat_to_row, int32_t *overflow,
                                int32_t *n_overflow, void *ws, size_t ws_bytes,
                                moe_stream_t stream);

/*
 * Load-balance statistics of one routing decision, forward only.
 *   P[e] = (1/T) sum_t softmax(logits[t][.])[e]   mean gate probability [E]
 *   f[e] = counts[e] / (T*k)                      share of routed entries [E]
 *   summary[0] = alpha * E * sum_e f[e] P[e]       aux load-balance loss
 *                ("DeepGEMM walkthrough" §2.2)
 *   summary[1] = max_e counts[e] / mean_e counts[e]
 *                ("Dense GEMM to TP MoE" §5.1: above 3 is severe)
 *   summary[2] = -sum_e q[e] log2(q[e] + 1e-8), q = counts / sum counts
 *                (routing entropy in bits, "DeepSeek MoE evolution" §2.3)
 * prob_sums [ceil(T/16)][E] fp32 is moe_route's per-block sums of the
 * softmax probabilities (the router computes every p_t already, so no pass
 * over the logits is needed), counts [E] int32 is moe_permute's; all fp32
 * outputs on the device.  One launch; sums in a fixed order
 * (deterministic).  Counts are exact up to 2^24 in the fp32 arithmetic.
 */
moe_status_t moe_router_stats(const float *prob_sums, const int32_t *counts, int T, int E,
                              int k, float alpha, float *f, float *P, float *summary,
                              moe_stream_t stream);

/*
 * Grouped GEMM over ragged groups in one launch ("DeepGEMM walkthrough"
 * §4.3; "Dense GEMM to TP MoE" §2.1, §2.3).  Group g owns rows
 * offsets[g] .. offsets[g+1]-1 of A (device array, read by the kernel's own
 * tile scheduler -- the group sizes never reach the host):
 *   C[r][n] = sum_k A[r][k] * B[g][n][k]                       (MOE_EPI_NONE)
 *   C[r][n] = silu(sum_k A[r][k] B[g][n][k]) * sum_k A[r][k] B2[g][n][k]
 *                                                             (MOE_EPI_SWIGLU)
 * A [rows][K], B and B2 [G][N][ldb] of type ab_dt (MOE_F32 or MOE_BF16),
 * of whose rows the first K elements are used (B[g][n][k] is element
 * (g N + n) ldb + k), accumulation in fp32, C [rows][N] of type c_dt
 * (MOE_F32 or MOE_BF16).  ldb == 0 means K; otherwise ldb >= K with ldb
 * times the element size a multiple of 16 bytes, else MOE_ERR_INVALID.
 * Padding matters when a weight row is a power-of-two number of bytes and
 * the weights stream from HBM: the pieces a tile reads at one K offset then
 * fall on few memory channels (measured with 256 bytes of padding, the GEMM
 * alone: decode-size gate/up with 8 KB rows -20 %, DeepSeek-shape down with
 * 4 KB rows -8 %).
 * B2 must be NULL unless epi == MOE_EPI_SWIGLU.  Rows of C outside every
 * group are not written.  offsets values are clamped to [0, rows] and read
 * as their running maximum (group g owns rows [o_g, o_{g+1}) with o_g the
 * largest clamped offset up to g), so a bad offsets array gives wrong
 * results but no out-of-bounds access, in C and in the workspace.
 * Requires K % 8 == 0, 1 <= G <= MOE_MAX_GROUPS.
 *
 * ws (device, 16-byte aligned, caller-owned scratch) lets the bf16 path cut
 * the last, partial round of output tiles along K over the idle compute
 * units; the K-slices are added in a fixed order by a second kernel, so the
 * result is deterministic for a given device and offsets (it may differ in
 * the last bits from the ws == NULL result).  ws == NULL with ws_bytes == 0
 * runs without the split.  Otherwise ws_bytes must be at least
 * moe_grouped_gemm_workspace_size(G, rows, N, K, ab_dt, epi) (else
 * MOE_ERR_WORKSPACE); a size of 0 means the shape never splits and ws is
 * not touched.  Calls that share one ws must be ordered (same stream).
 */
moe_status_t moe_grouped_gemm(const void *A, const void *B, const void *B2,
                              moe_dtype_t ab_dt, void *C, moe_dtype_t c_dt,
                              const int32_t *offsets, int G, int rows, int N,
                              int K, int ldb, moe_epilogue_t epi, void *ws,
                              size_t ws_bytes, moe_stream_t stream);

/* Workspace bytes moe_grouped_gemm may use for this shape on the current
 * device (it depends on the device's compute-unit count); 0 for shapes and
 * dtypes that never split, and for invalid arguments. */
size_t moe_grouped_gemm_workspace_size(int G, int rows, int N, int K,
                                       moe_dtype_t ab_dt, moe_epilogue_t epi);

/*
 * FP8 block-scaled grouped GEMM ("DeepGEMM walkthrough" §2.3 and §5.1).
 * The stored scales are dequantisation multipliers (the reciprocal of the
 * page's scale_A / scale_B; scale_C = 1):
 *   A[r][k]    ~ A_q[r][k] * A_scale[k/128][r]          A_scale [K/128][rows]
 *   B[g][n][k] ~ B_q[g][n][k] * B_scale[g][n/128][k/128]
 *                                                  B_scale [G][N/128][K/128]
 *   C = A B^T (or the SwiGLU form with B2) computed as
 *       sum_kb A_scale[kb][r] B_scale[g][n/128][kb] * (sum_{k in kb} A_q B_q)
 *   with fp32 accumulation.
 * c_dt == MOE_BF16 writes bf16.  c_dt == MOE_E4M3 quantises each output row
 * in 1 x 128 groups with the scale absmax / 448, as moe_permute does (the
 * values are multiplied by the reciprocal of the scale, so a code can differ
 * from a division's in the last rounding), and writes C_scale
 * [N/128][rows] (group-major, like A_scale, so it feeds the next GEMM);
 * C_scale must be NULL otherwise.
 * B_q and B2_q rows sit ldb bytes apart (B_q[g][n][k] at (g N + n) ldb + k;
 * ldb == 0 means K; otherwise ldb >= K and ldb % 16 == 0, else
 * MOE_ERR_INVALID; padding as for moe_grouped_gemm); the scales stay dense.
 * Requires N % 128 == 0 and K % 128 == 0.
 */
moe_status_t moe_grouped_gemm_fp8(const uint8_t *A_q, const float *A_scale,
                                  const uint8_t *B_q, const float *B_scale,
                                  const uint8_t *B2_q, const float *B2_scale,
                                  void *C, moe_dtype_t c_dt, float *C_scale,
                                  const int32_t *offsets, int G, int rows,
                                  int N, int K, int ldb, moe_epilogue_t epi,
                                  moe_stream_t stream);

/*
 * Gather back to token order, weight by the gate and sum ("Dense GEMM to TP
 * MoE" §2.2 step 6; "DeepGEMM walkthrough" §2.1, shared expert weight 1):
 *   out[t][c] = sum_{j=0}^{k-1} topk_w[t][j] * Y[flat_to_row[t*k+j]][c]
 *               + sum_s Y[flat_to_row[T*k + s*T + t]][c]
 * fp32 sum in ascending j, then the shared rows; flat_to_row
 * [T*k + n_shared*T] is the array moe_permute wrote.  Y [T*k + n_shared*T][d]
 * of type y_dt, out [T][d] of type out_dt (MOE_F32 or MOE_BF16 each).  A
 * flat_to_row entry < 0 (a dropped entry) contributes nothing.
 * Requires d % 8 == 0.
 */
moe_status_t moe_combine(const void *Y, moe_dtype_t y_dt,
                         const int32_t *flat_to_row, const float *topk_w,
                         int T, int k, int d, int n_shared, void *out,
                         moe_dtype_t out_dt, moe_stream_t stream);

/*
 * Block FP8 quantisation of a matrix, for preparing expert weights
 * ("DeepGEMM walkthrough" §2.3, §5.1: per-block scales):
 *   src [R][C] (MOE_F32 or MOE_BF16) cut into block_rows x block_cols blocks,
 *   s = absmax(block) / 448 (1 for an all-zero block),
 *   q = E4M3 round-to-nearest-even of (src / s), fp32 IEEE division,
 *       saturating at +-448.
 * q [R][C] uint8, scale [R/block_rows][C/block_cols] fp32.  Requires
 * block_rows in {1, 128}, block_cols == 128, R % block_rows == 0,
 * C % 128 == 0.
 */
moe_status_t moe_quantize_fp8(const void *src, moe_dtype_t src_dt, int R,
                              int C, int block_rows, int block_cols,
                              uint8_t *q, float *scale, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
