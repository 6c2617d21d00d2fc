"""ctypes binding of libmoe.so with the same names as the C ABI (include/moe.h).

Argument marshalling only: sizes are read off the tensors, pointers and the
current HIP stream are handed to the library, and a non-OK status raises
``MoEError``.  Every step runs in the library's HIP kernels; there is no
fallback of any kind.  Importing this module loads the library and raises if
it has not been built (``python -m grouped_gemm_router_amd.build``).
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH = range(5)
MOE_F32, MOE_BF16, MOE_E4M3 = 0, 1, 2
MOE_EPI_NONE, MOE_EPI_SWIGLU = 0, 1
MOE_ROUTE_RENORM, MOE_ROUTE_FROM_LOGITS = 1, 2
ABI_VERSION = 8

EXPORTS = ["moe_status_string", "moe_abi_version", "moe_route_workspace_size", "moe_route",
           "moe_permute_workspace_size", "moe_permute_capped", "moe_router_stats",
           "moe_permute", "moe_permute_noalloc", "moe_grouped_gemm_workspace_size",
           "moe_grouped_gemm",
           "moe_grouped_gemm_fp8", "moe_combine",
           "moe_quantize_fp8"]


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (fn, status_string(status), status))


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libmoe.so is not built at %s; run `python -m "
                          "grouped_gemm_router_amd.build`" % _LIB_PATH)
    lib = C.CDLL(_LIB_PATH)
    vp, i32, u32, sz = C.c_void_p, C.c_int, C.c_uint, C.c_size_t
    lib.moe_status_string.restype = C.c_char_p
    lib.moe_status_string.argtypes = [i32]
    lib.moe_abi_version.restype = i32
    lib.moe_abi_version.argtypes = []
    lib.moe_route.restype = i32
    lib.moe_route_workspace_size.restype = sz
    lib.moe_route_workspace_size.argtypes = [i32, i32, i32]
    lib.moe_route.argtypes = [vp, vp, i32, vp, i32, i32, i32, i32, u32, vp, vp, vp, vp, vp, sz,
                              vp]
    lib.moe_permute_workspace_size.restype = sz
    lib.moe_permute_workspace_size.argtypes = [i32, i32, i32]
    lib.moe_permute.restype = i32
    lib.moe_permute.argtypes = [vp, i32, i32, i32, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                vp, vp, sz, vp]
    lib.moe_permute_noalloc.restype = i32
    lib.moe_permute_noalloc.argtypes = [vp, i32, i32, i32, vp, i32, i32, i32, i32, vp, vp, vp,
                                        vp, vp, vp, vp]
    lib.moe_permute_capped.restype = i32
    lib.moe_permute_capped.argtypes = [vp, i32, i32, i32, vp, i32, i32, i32, i32, i32, vp, vp, vp,
                                       vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_router_stats.restype = i32
    lib.moe_router_stats.argtypes = [vp, vp, i32, i32, i32, C.c_float, vp, vp, vp, vp]
    lib.moe_grouped_gemm_workspace_size.restype = sz
    lib.moe_grouped_gemm_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.moe_grouped_gemm.restype = i32
    lib.moe_grouped_gemm.argtypes = [vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, i32,
                                     vp, sz, vp]
    lib.moe_grouped_gemm_fp8.restype = i32
    lib.moe_grouped_gemm_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32,
                                         i32, i32, i32, vp]
    lib.moe_combine.restype = i32
    lib.moe_combine.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, i32, vp]
    lib.moe_quantize_fp8.restype = i32
    lib.moe_quantize_fp8.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp]
    if lib.moe_abi_version() != ABI_VERSION:
        raise ImportError("libmoe.so ABI version %d, binding expects %d"
                          % (lib.moe_abi_version(), ABI_VERSION))
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.moe_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoEError(fn, status)


_defer = threading.local()


def _deferring() -> bool:
    return getattr(_defer, "on", False)


def _invoke(fn: str, cfn, *args):
    """Call the library entry cfn with marshalled args and check the status;
    inside deferred(), return that call as a thunk instead of making it."""
    if _deferring():
        def call():
            status = cfn(*args)
            if status != MOE_OK:
                raise MoEError(fn, status)
        call.entry = fn
        return call
    _check(fn, cfn(*args))
    return None


def deferred(entry, *args, **kwargs):
    """entry(*args, **kwargs) -- one of the entry points below -- with its
    arguments checked and marshalled now, as a thunk that makes the library
    call (same pointers, sizes and stream: the current stream now, if none is
    given) each time it is called.  The thunk holds the argument tensors.
    For callers that launch the same call many times: the per-call host cost
    is then one ctypes call.  Every buffer must be passed explicitly."""
    _defer.on = True
    try:
        call = entry(*args, **kwargs)
    finally:
        _defer.on = False
    if getattr(call, "entry", None) is None:
        raise TypeError("%s is not a library call entry point" % getattr(entry, "__name__", entry))

    def thunk():
        call()
    thunk.args = (args, kwargs)  # the argument tensors live as long as the thunk
    return thunk


def _ptr(t) -> C.c_void_p:
    if t is None:
        return C.c_void_p(0)
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor, got %r" % type(t))
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return C.c_void_p(t.data_ptr())


def _weights(B, B2=None):
    """(pointer of B, pointer of B2, row pitch in elements) of [G][N][K]
    weights whose rows may sit further apart than K (a view of [G][N][ldb]
    storage, ldb >= K); B2, when given, must have the same shape and strides."""
    if not isinstance(B, torch.Tensor) or B.dim() != 3:
        raise TypeError("weights must be a [G][N][K] torch.Tensor")
    G, N, K = B.shape
    ldb = B.stride(1)
    if B.stride(2) != 1 or ldb < K or B.stride(0) != N * ldb:
        raise ValueError("weights must be [G][N][K] rows of unit stride, %s given" % (B.stride(),))
    if B2 is not None and (B2.shape != B.shape or B2.stride() != B.stride()):
        raise ValueError("B2 must have B's shape and strides")
    p2 = C.c_void_p(0) if B2 is None else C.c_void_p(B2.data_ptr())
    return C.c_void_p(B.data_ptr()), p2, ldb


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MOE_E4M3
    raise TypeError("unsupported dtype %s" % t.dtype)


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ----------------------------------------------------------------------------

def moe_route_workspace_size(T: int, d: int, E: int) -> int:
    return int(lib.moe_route_workspace_size(T, d, E))


PROB_SUM_BLOCK = 16  # tokens per block of moe_route's probability sums


def prob_sum_blocks(T: int) -> int:
    return (T + PROB_SUM_BLOCK - 1) // PROB_SUM_BLOCK


def moe_route(x, w_router, topk_idx, topk_w, *, logits=None, logit_bias=None, flags=0,
              prob_sums=None, ws=None, stream=None):
    """Router scoring + top-k.  x [T][d], w_router [E][d] (fp32 or bf16);
    topk_idx [T][k] int32 and topk_w [T][k] fp32 are written; logits [T][E]
    fp32 is written if given (read instead with MOE_ROUTE_FROM_LOGITS);
    prob_sums [ceil(T/16)][E] fp32, if given, receives per-block sums of the
    softmax probabilities (for moe_router_stats).  ws: device workspace of
    moe_route_workspace_size(T, d, E) bytes; when None, one is allocated here
    for this call."""
    T, k = topk_idx.shape
    if flags & MOE_ROUTE_FROM_LOGITS:
        E = logits.shape[1]
        d, dt = 8, MOE_BF16
        ws_bytes = 0
    else:
        d = x.shape[1]
        E = w_router.shape[0]
        dt = _dt(x)
        if ws is None:
            if _deferring():
                raise ValueError("moe_route under deferred() needs its workspace passed")
            ws = torch.empty(max(moe_route_workspace_size(T, d, E), 4), dtype=torch.uint8,
                             device=topk_idx.device)
        ws_bytes = ws.numel() * ws.element_size()
    if prob_sums is not None and tuple(prob_sums.shape) != (prob_sum_blocks(T), E):
        raise ValueError("prob_sums must be [ceil(T/16)][E] = [%d][%d]" % (prob_sum_blocks(T), E))
    return _invoke("moe_route", lib.moe_route,
                   _ptr(x), _ptr(w_router), dt, _ptr(logit_bias), T, d, E, k, flags, _ptr(logits),
                   _ptr(topk_idx), _ptr(topk_w), _ptr(prob_sums), _ptr(ws), ws_bytes,
                   _stream(stream))


def moe_permute_workspace_size(T: int, k: int, E: int) -> int:
    return int(lib.moe_permute_workspace_size(T, k, E))


def moe_permute(x, topk_idx, E, n_shared, x_perm, counts, offsets, perm_src, flat_to_row, ws, *,
                x_perm_scale=None, stream=None):
    """Histogram + offsets + stable scatter.  x_perm's dtype selects the
    output: same as x (bit copy) or uint8 (E4M3 with 1x128 scales)."""
    T, d = x.shape
    k = topk_idx.shape[1]
    out_dt = _dt(x_perm)
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    return _invoke("moe_permute", lib.moe_permute,
                   _ptr(x), _dt(x), T, d, _ptr(topk_idx), k, E, n_shared, out_dt, _ptr(x_perm),
                   _ptr(x_perm_scale), _ptr(counts), _ptr(offsets), _ptr(perm_src),
                   _ptr(flat_to_row), _ptr(ws), ws_bytes, _stream(stream))


PERMUTE_NOALLOC_SCRATCH_BYTES = 1 << 20


def moe_permute_noalloc(x, topk_idx, E, n_shared, x_perm, counts, offsets, perm_src,
                        flat_to_row, *, x_perm_scale=None, stream=None):
    """moe_permute without a workspace: the library's static device scratch
    (PERMUTE_NOALLOC_SCRATCH_BYTES per GPU) holds the per-block counts, so
    the call allocates nothing.  Calls that overlap on one GPU race."""
    T, d = x.shape
    k = topk_idx.shape[1]
    return _invoke("moe_permute_noalloc", lib.moe_permute_noalloc,
                   _ptr(x), _dt(x), T, d, _ptr(topk_idx), k, E, n_shared, _dt(x_perm),
                   _ptr(x_perm), _ptr(x_perm_scale), _ptr(counts), _ptr(offsets), _ptr(perm_src),
                   _ptr(flat_to_row), _stream(stream))


def moe_permute_capped(x, topk_idx, E, n_shared, capacity, x_perm, counts, offsets, perm_src,
                       flat_to_row, ws, *, overflow=None, n_overflow=None, x_perm_scale=None,
                       stream=None):
    """moe_permute with each expert capped at `capacity` rows; dropped
    entries get flat_to_row -1 and are listed in `overflow` (expert by
    expert), their number in n_overflow[0]."""
    T, d = x.shape
    k = topk_idx.shape[1]
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    return _invoke("moe_permute_capped", lib.moe_permute_capped,
                   _ptr(x), _dt(x), T, d, _ptr(topk_idx), k, E, n_shared, int(capacity),
                   _dt(x_perm), _ptr(x_perm), _ptr(x_perm_scale), _ptr(counts), _ptr(offsets),
                   _ptr(perm_src), _ptr(flat_to_row), _ptr(overflow), _ptr(n_overflow), _ptr(ws),
                   ws_bytes, _stream(stream))


def moe_router_stats(prob_sums, counts, T, k, alpha, f, P, summary, *, stream=None):
    """Load-balance statistics from moe_route's probability sums
    [ceil(T/16)][E] and moe_permute's counts [E]: f [E], P [E], summary [3] =
    (aux loss, max/mean count, entropy in bits)."""
    E = prob_sums.shape[1]
    if prob_sums.shape[0] != prob_sum_blocks(T):
        raise ValueError("prob_sums must have ceil(T/16) = %d rows" % prob_sum_blocks(T))
    return _invoke("moe_router_stats", lib.moe_router_stats,
                   _ptr(prob_sums), _ptr(counts), T, E, k, float(alpha), _ptr(f), _ptr(P),
                   _ptr(summary), _stream(stream))


def moe_grouped_gemm_workspace_size(G: int, rows: int, N: int, K: int, dtype, epi: int) -> int:
    """Bytes of the tail-split workspace moe_grouped_gemm may use on the
    current device (0: this shape never splits)."""
    dt = dtype if isinstance(dtype, int) else _dt(torch.empty(0, dtype=dtype))
    return int(lib.moe_grouped_gemm_workspace_size(G, rows, N, K, dt, epi))


def moe_grouped_gemm(A, B, C_out, offsets, *, B2=None, epi=MOE_EPI_NONE, ws=None, stream=None):
    """C[r] = A[r] B[g]^T for rows r of group g (offsets on the device).
    ws: moe_grouped_gemm_workspace_size bytes of device scratch that lets the
    last, partial round of tiles be cut along K; None runs without it."""
    rows, K = A.shape
    G, N, K2 = B.shape
    if K2 != K:
        raise ValueError("A is [rows][%d] but B is [G][N][%d]" % (K, K2))
    if offsets.numel() != G + 1:
        raise ValueError("offsets must have G + 1 = %d entries" % (G + 1))
    pb, pb2, ldb = _weights(B, B2)
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    return _invoke("moe_grouped_gemm", lib.moe_grouped_gemm,
                   _ptr(A), pb, pb2, _dt(A), _ptr(C_out), _dt(C_out), _ptr(offsets), G, rows, N,
                   K, ldb, epi, _ptr(ws), ws_bytes, _stream(stream))


def moe_grouped_gemm_fp8(A_q, A_scale, B_q, B_scale, C_out, offsets, *, B2_q=None,
                         B2_scale=None, C_scale=None, epi=MOE_EPI_NONE, stream=None):
    rows, K = A_q.shape
    G, N, K2 = B_q.shape
    if K2 != K:
        raise ValueError("A_q is [rows][%d] but B_q is [G][N][%d]" % (K, K2))
    if offsets.numel() != G + 1:
        raise ValueError("offsets must have G + 1 = %d entries" % (G + 1))
    pb, pb2, ldb = _weights(B_q, B2_q)
    c_dt = MOE_E4M3 if C_out.dtype in (torch.uint8, torch.float8_e4m3fn) else _dt(C_out)
    return _invoke("moe_grouped_gemm_fp8", lib.moe_grouped_gemm_fp8,
                   _ptr(A_q), _ptr(A_scale), pb, _ptr(B_scale), pb2, _ptr(B2_scale), _ptr(C_out),
                   c_dt, _ptr(C_scale), _ptr(offsets), G, rows, N, K, ldb, epi, _stream(stream))


def moe_combine(Y, flat_to_row, topk_w, out, *, n_shared=0, stream=None):
    T, k = topk_w.shape
    d = Y.shape[1]
    return _invoke("moe_combine", lib.moe_combine,
                   _ptr(Y), _dt(Y), _ptr(flat_to_row), _ptr(topk_w), T, k, d, n_shared, _ptr(out),
                   _dt(out), _stream(stream))


def moe_quantize_fp8(src, q, scale, *, block_rows=128, block_cols=128, stream=None):
    R, Cn = src.shape
    return _invoke("moe_quantize_fp8", lib.moe_quantize_fp8,
                   _ptr(src), _dt(src), R, Cn, block_rows, block_cols, _ptr(q), _ptr(scale),
                   _stream(stream))
