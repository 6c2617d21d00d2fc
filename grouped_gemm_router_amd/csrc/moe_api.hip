// moe_api.hip -- the extern "C" entry points of libmoe.so (declared and
// documented in include/moe.h).  Each entry point checks its arguments on
// the host, returns a status without launching anything if they are bad,
// and otherwise enqueues the kernels on the caller's stream.  Nothing here
// allocates, frees, synchronises or reads device memory.
#include <stdint.h>

#include <atomic>

#include "moe_internal.h"

namespace {

constexpr int kAbiVersion = 8;

bool aligned16(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool opt_aligned4(const void *p) { return !p || (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool is_act(moe_dtype_t d) { return d == MOE_F32 || d == MOE_BF16; }

moe_status_t launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

hipStream_t as_stream(moe_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// Compute units of the current device (0 if it cannot be queried), cached
// per device: a host attribute, no device access.
int current_device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    const int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (cached) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

extern "C" {

const char *moe_status_string(moe_status_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype combination or shape";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int moe_abi_version(void) { return kAbiVersion; }

size_t moe_route_workspace_size(int T, int d, int E) {
  if (T < 0 || d < 1 || E < 1) return 0;
  return route_ws_bytes(T, d, E);
}

moe_status_t moe_route(const void *x, const void *w_router, moe_dtype_t dt,
                       const float *logit_bias, int T, int d, int E, int k, unsigned flags,
                       float *logits, int32_t *topk_idx, float *topk_w, float *prob_sums,
                       void *ws, size_t ws_bytes, moe_stream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (flags & ~(MOE_ROUTE_RENORM | MOE_ROUTE_FROM_LOGITS)) return MOE_ERR_INVALID;
  if (!aligned4(topk_idx) || !aligned4(topk_w) || !opt_aligned4(prob_sums))
    return MOE_ERR_INVALID;
  const bool from_logits = (flags & MOE_ROUTE_FROM_LOGITS) != 0;
  if (from_logits) {
    if (!aligned4(logits)) return MOE_ERR_INVALID;
  } else {
    if (!is_act(dt)) return MOE_ERR_UNSUPPORTED;
    if (d < 8 || d % 8 != 0) return MOE_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_INVALID;
    if (!opt_aligned4(logits) || !opt_aligned4(logit_bias)) return MOE_ERR_INVALID;
    const size_t need = route_ws_bytes(T, d, E);
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (need > 0 && !aligned4(ws)) return MOE_ERR_INVALID;
  }
  if (T == 0) return MOE_OK;
  return launched(launch_route(x, w_router, dt, logit_bias, T, d, E, k, flags, logits, topk_idx,
                               topk_w, prob_sums, static_cast<float *>(ws), as_stream(stream)));
}

size_t moe_permute_workspace_size(int T, int k, int E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  return permute_ws_bytes(T, k, E);
}

namespace {

moe_status_t permute_checked(const void *x, moe_dtype_t x_dt, int T, int d,
                             const int32_t *topk_idx, int k, int E, int n_shared, int capacity,
                             moe_dtype_t out_dt, void *x_perm, float *x_perm_scale,
                             int32_t *counts, int32_t *offsets, int32_t *perm_src,
                             int32_t *flat_to_row, int32_t *overflow, int32_t *n_overflow,
                             void *ws, size_t ws_bytes, bool static_scratch,
                             moe_stream_t stream) {
  if (T < 0 || d < 8 || E < 1 || k < 1 || k > E || n_shared < 0 || capacity < 0)
    return MOE_ERR_INVALID;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || n_shared > 8) return MOE_ERR_UNSUPPORTED;
  if (!is_act(x_dt)) return MOE_ERR_UNSUPPORTED;
  if (d % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * (k + n_shared) > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (out_dt == MOE_E4M3) {
    if (d % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if (!aligned4(x_perm_scale)) return MOE_ERR_INVALID;
  } else {
    if (out_dt != x_dt) return MOE_ERR_UNSUPPORTED;
    if (x_perm_scale) return MOE_ERR_INVALID;
  }
  if (!aligned16(x) || !aligned16(x_perm) || !aligned4(topk_idx) || !aligned4(counts) ||
      !aligned4(offsets) || !aligned4(perm_src) || !aligned4(flat_to_row) ||
      !opt_aligned4(overflow) || !opt_aligned4(n_overflow))
    return MOE_ERR_INVALID;
  const size_t need = permute_ws_bytes(T, k, E);
  if (static_scratch) {  // moe_permute_noalloc: the library's static scratch
    if (need > MOE_PERMUTE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    if (T == 0) return MOE_OK;
    if (permute_noalloc_scratch(&ws) != hipSuccess) return MOE_ERR_LAUNCH;
  } else {
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (need > 0 && !aligned4(ws)) return MOE_ERR_INVALID;
  }
  if (T == 0) return MOE_OK;
  return launched(launch_permute(x, x_dt, T, d, topk_idx, k, E, n_shared, capacity, out_dt,
                                 x_perm, x_perm_scale, counts, offsets, perm_src, flat_to_row,
                                 overflow, n_overflow, ws, as_stream(stream)));
}

}  // namespace

moe_status_t moe_permute(const void *x, moe_dtype_t x_dt, int T, int d, const int32_t *topk_idx,
                         int k, int E, int n_shared, moe_dtype_t out_dt, void *x_perm,
                         float *x_perm_scale, int32_t *counts, int32_t *offsets,
                         int32_t *perm_src, int32_t *flat_to_row, void *ws, size_t ws_bytes,
                         moe_stream_t stream) {
  return permute_checked(x, x_dt, T, d, topk_idx, k, E, n_shared, INT32_MAX, out_dt, x_perm,
                         x_perm_scale, counts, offsets, perm_src, flat_to_row, nullptr, nullptr,
                         ws, ws_bytes, false, stream);
}

moe_status_t moe_permute_noalloc(const void *x, moe_dtype_t x_dt, int T, int d,
                                 const int32_t *topk_idx, int k, int E, int n_shared,
                                 moe_dtype_t out_dt, void *x_perm, float *x_perm_scale,
                                 int32_t *counts, int32_t *offsets, int32_t *perm_src,
                                 int32_t *flat_to_row, moe_stream_t stream) {
  return permute_checked(x, x_dt, T, d, topk_idx, k, E, n_shared, INT32_MAX, out_dt, x_perm,
                         x_perm_scale, counts, offsets, perm_src, flat_to_row, nullptr, nullptr,
                         nullptr, 0, true, stream);
}

moe_status_t moe_permute_capped(const void *x, moe_dtype_t x_dt, int T, int d,
                                const int32_t *topk_idx, int k, int E, int n_shared,
                                int capacity, moe_dtype_t out_dt, void *x_perm,
                                float *x_perm_scale, int32_t *counts, int32_t *offsets,
                                int32_t *perm_src, int32_t *flat_to_row, int32_t *overflow,
                                int32_t *n_overflow, void *ws, size_t ws_bytes,
                                moe_stream_t stream) {
  return permute_checked(x, x_dt, T, d, topk_idx, k, E, n_shared, capacity, out_dt, x_perm,
                         x_perm_scale, counts, offsets, perm_src, flat_to_row, overflow,
                         n_overflow, ws, ws_bytes, false, stream);
}

moe_status_t moe_router_stats(const float *prob_sums, const int32_t *counts, int T, int E, int k,
                              float alpha, float *f, float *P, float *summary,
                              moe_stream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (!aligned4(prob_sums) || !aligned4(counts) || !aligned4(f) || !aligned4(P) ||
      !aligned4(summary))
    return MOE_ERR_INVALID;
  if (T == 0) return MOE_OK;
  return launched(launch_router_stats(prob_sums, counts, T, E, k, alpha, f, P, summary,
                                      as_stream(stream)));
}

size_t moe_grouped_gemm_workspace_size(int G, int rows, int N, int K, moe_dtype_t ab_dt,
                                       moe_epilogue_t epi) {
  if (G < 1 || G > MOE_MAX_GROUPS || rows < 0 || N < 1 || K < 1) return 0;
  if (ab_dt != MOE_BF16 || (epi != MOE_EPI_NONE && epi != MOE_EPI_SWIGLU)) return 0;
  return gemm_bf16_split_ws_bytes(G, rows, N, K, epi, current_device_cus());
}

moe_status_t moe_grouped_gemm(const void *A, const void *B, const void *B2, moe_dtype_t ab_dt,
                              void *C, moe_dtype_t c_dt, const int32_t *offsets, int G, int rows,
                              int N, int K, int ldb, moe_epilogue_t epi, void *ws,
                              size_t ws_bytes, moe_stream_t stream) {
  if (G < 1 || rows < 0 || N < 1 || K < 1) return MOE_ERR_INVALID;
  if (ldb == 0) ldb = K;
  if (ldb < K) return MOE_ERR_INVALID;
  if (G > MOE_MAX_GROUPS) return MOE_ERR_UNSUPPORTED;
  if (epi != MOE_EPI_NONE && epi != MOE_EPI_SWIGLU) return MOE_ERR_INVALID;
  if (!is_act(ab_dt) || !is_act(c_dt)) return MOE_ERR_UNSUPPORTED;
  if (K % 8 != 0) return MOE_ERR_UNSUPPORTED;
  // weight rows start on 16-byte boundaries like the matrices themselves
  if ((long long)ldb * (ab_dt == MOE_BF16 ? 2 : 4) % 16 != 0) return MOE_ERR_INVALID;
  if (!aligned16(A) || !aligned16(B) || !aligned4(C) || !aligned4(offsets)) return MOE_ERR_INVALID;
  if (epi == MOE_EPI_SWIGLU ? !aligned16(B2) : B2 != nullptr) return MOE_ERR_INVALID;
  if ((long long)G * N * ldb >= (1ll << 40)) return MOE_ERR_UNSUPPORTED;
  if (ws == nullptr && ws_bytes != 0) return MOE_ERR_INVALID;
  // the MFMA kernel writes C in 16-byte row pieces
  const bool mfma = ab_dt == MOE_BF16 && gemm_bf16_mfma_supports(N, K, epi) && aligned16(C);
  void *split_ws = nullptr;
  int cus = 0;
  if (ws != nullptr && mfma) {
    cus = current_device_cus();
    const size_t need = gemm_bf16_split_ws_bytes(G, rows, N, K, epi, cus);
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (need > 0) {
      if (!aligned16(ws)) return MOE_ERR_INVALID;
      split_ws = ws;
    }
  }
  if (rows == 0) return MOE_OK;
  const hipStream_t s = as_stream(stream);
  if (mfma)
    return launched(launch_gemm_bf16_mfma(A, B, B2, C, c_dt, offsets, G, rows, N, K, ldb, epi,
                                          split_ws, cus, s));
  return launched(
      launch_gemm_simple(A, B, B2, ab_dt, C, c_dt, offsets, G, rows, N, K, ldb, epi, s));
}

moe_status_t moe_grouped_gemm_fp8(const uint8_t *A_q, const float *A_scale, const uint8_t *B_q,
                                  const float *B_scale, const uint8_t *B2_q,
                                  const float *B2_scale, void *C, moe_dtype_t c_dt,
                                  float *C_scale, const int32_t *offsets, int G, int rows, int N,
                                  int K, int ldb, moe_epilogue_t epi, moe_stream_t stream) {
  if (G < 1 || rows < 0 || N < 1 || K < 1) return MOE_ERR_INVALID;
  if (G > MOE_MAX_GROUPS) return MOE_ERR_UNSUPPORTED;
  if (epi != MOE_EPI_NONE && epi != MOE_EPI_SWIGLU) return MOE_ERR_INVALID;
  if (N % 128 != 0 || K % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (ldb == 0) ldb = K;
  if (ldb < K || ldb % 16 != 0) return MOE_ERR_INVALID;
  if (c_dt != MOE_BF16 && c_dt != MOE_E4M3) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(A_q) || !aligned4(A_scale) || !aligned16(B_q) || !aligned4(B_scale) ||
      !aligned4(C) || !aligned4(offsets))
    return MOE_ERR_INVALID;
  if (epi == MOE_EPI_SWIGLU) {
    if (!aligned16(B2_q) || !aligned4(B2_scale)) return MOE_ERR_INVALID;
  } else if (B2_q || B2_scale) {
    return MOE_ERR_INVALID;
  }
  if (c_dt == MOE_E4M3 ? !aligned4(C_scale) : C_scale != nullptr) return MOE_ERR_INVALID;
  if ((long long)G * N * ldb >= (1ll << 40)) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (gemm_fp8_ring_supports(rows, N, K, ldb))
    return launched(launch_gemm_fp8_ring(A_q, A_scale, B_q, B_scale, B2_q, B2_scale, C, c_dt,
                                         C_scale, offsets, G, rows, N, K, ldb, epi,
                                         as_stream(stream)));
  return launched(launch_gemm_fp8(A_q, A_scale, B_q, B_scale, B2_q, B2_scale, C, c_dt, C_scale,
                                  offsets, G, rows, N, K, ldb, epi, as_stream(stream)));
}

moe_status_t moe_combine(const void *Y, moe_dtype_t y_dt, const int32_t *flat_to_row,
                         const float *topk_w, int T, int k, int d, int n_shared, void *out,
                         moe_dtype_t out_dt, moe_stream_t stream) {
  if (T < 0 || k < 1 || d < 8 || n_shared < 0) return MOE_ERR_INVALID;
  if (k > MOE_MAX_TOPK || n_shared > 8) return MOE_ERR_UNSUPPORTED;
  if (!is_act(y_dt) || !is_act(out_dt)) return MOE_ERR_UNSUPPORTED;
  if (d % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(Y) || !aligned16(out) || !aligned4(flat_to_row) || !aligned4(topk_w))
    return MOE_ERR_INVALID;
  if (T == 0) return MOE_OK;
  return launched(launch_combine(Y, y_dt, flat_to_row, topk_w, T, k, d, n_shared, out, out_dt,
                                 as_stream(stream)));
}

moe_status_t moe_quantize_fp8(const void *src, moe_dtype_t src_dt, int R, int C, int block_rows,
                              int block_cols, uint8_t *q, float *scale, moe_stream_t stream) {
  if (R < 0 || C < 0) return MOE_ERR_INVALID;
  if (!is_act(src_dt)) return MOE_ERR_UNSUPPORTED;
  if ((block_rows != 1 && block_rows != 128) || block_cols != 128) return MOE_ERR_UNSUPPORTED;
  if (R % block_rows != 0 || C % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(src) || !aligned16(q) || !aligned4(scale)) return MOE_ERR_INVALID;
  if ((long long)(R / block_rows) * (C / 128) > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (R == 0 || C == 0) return MOE_OK;
  return launched(launch_quantize_fp8(src, src_dt, R, C, block_rows, block_cols, q, scale,
                                      as_stream(stream)));
}

}  // extern "C"
