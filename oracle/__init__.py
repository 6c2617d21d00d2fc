"""CPU oracle for the MoE expert-layer forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and the two share no code.

The arithmetic lives in ``moe_oracle.c`` (plain loops, fp64, OpenMP over
tokens); this module only builds it with gcc, loads it with ctypes and
marshals numpy arrays.  Every function documents the page passage it follows
in the C source.  Functions without an independent pin would say
"parity unpinned"; every function here is pinned by a test under
``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, E4M3 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-D_DEFAULT_SOURCE", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = C.CDLL(_LIB)
        _declare(_lib)
    return _lib


class LayerDesc(C.Structure):
    _fields_ = [
        ("mode", C.c_int), ("x_dt", C.c_int),
        ("T", C.c_int64), ("d", C.c_int64), ("dff", C.c_int64),
        ("E", C.c_int), ("k", C.c_int), ("n_shared", C.c_int),
        ("x", C.c_void_p),
        ("wg", C.POINTER(C.c_void_p)), ("wu", C.POINTER(C.c_void_p)),
        ("wd", C.POINTER(C.c_void_p)),
        ("sg", C.POINTER(C.c_void_p)), ("su", C.POINTER(C.c_void_p)),
        ("sd", C.POINTER(C.c_void_p)),
    ]


def _declare(L):
    vp, i64, i32, f64p = C.c_void_p, C.c_int64, C.c_int, C.c_void_p
    L.orc_e4m3_value.restype = C.c_double
    L.orc_e4m3_value.argtypes = [C.c_uint8]
    L.orc_e4m3_round.restype = C.c_uint8
    L.orc_e4m3_round.argtypes = [C.c_float]
    L.orc_quant_blocks.restype = None
    L.orc_quant_blocks.argtypes = [vp, i64, i64, i32, i32, vp, vp]
    L.orc_router_logits.restype = None
    L.orc_router_logits.argtypes = [vp, vp, i32, vp, i64, i64, i64, f64p, f64p]
    L.orc_topk.restype = None
    L.orc_topk.argtypes = [vp, i64, i32, i32, i32, vp, vp]
    L.orc_counts_offsets.restype = C.c_int
    L.orc_counts_offsets.argtypes = [vp, i64, i32, i32, i32, vp, vp]
    L.orc_permutation.restype = None
    L.orc_permutation.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    L.orc_capacity_permutation.restype = C.c_int64
    L.orc_capacity_permutation.argtypes = [vp, i64, i32, i32, i32, i64, vp, vp, vp, vp, vp]
    L.orc_router_stats.restype = None
    L.orc_router_stats.argtypes = [vp, i64, i32, vp, i32, C.c_double, vp, vp, vp]
    L.orc_permute_rows.restype = None
    L.orc_permute_rows.argtypes = [vp, i64, i64, i64, i32, vp, vp, i64, vp]
    L.orc_gemm_rows.restype = None
    L.orc_gemm_rows.argtypes = [vp, i32, vp, vp, i32, vp, i32, i64, i64, i32,
                                vp, i64, vp]
    L.orc_gemm_fp8_rows.restype = None
    L.orc_gemm_fp8_rows.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i64,
                                    i32, vp, i64, vp]
    L.orc_moe_tokens.restype = C.c_int
    L.orc_moe_tokens.argtypes = [C.POINTER(LayerDesc), vp, vp, vp, i64, vp]
    L.orc_combine.restype = None
    L.orc_combine.argtypes = [vp, i32, vp, vp, i64, i32, i64, i32, vp]


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a) -> C.c_void_p:
    return C.c_void_p(0 if a is None else a.ctypes.data)


def _dt_of(a: np.ndarray) -> int:
    """fp32 arrays are binary32; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle takes float32 or bf16 bit patterns (uint16), got %s" % a.dtype)


# ----------------------------------------------------------------------------
# FP8 (E4M3FN)
# ----------------------------------------------------------------------------

def e4m3_value(q: int) -> float:
    return lib().orc_e4m3_value(int(q))


def e4m3_decode(q: np.ndarray) -> np.ndarray:
    """Vectorised decode via the oracle's per-code values (table of 256)."""
    table = np.array([lib().orc_e4m3_value(i) for i in range(256)], dtype=np.float64)
    return table[np.asarray(q, dtype=np.uint8)]


def e4m3_round(y: float) -> int:
    return int(lib().orc_e4m3_round(float(y)))


def quant_blocks(v: np.ndarray, br: int, bc: int):
    """Block-quantise a 2-D float32 matrix: returns (codes uint8, scales f32)."""
    v = _c(v, np.float32)
    R, Cn = v.shape
    q = np.empty((R, Cn), dtype=np.uint8)
    s = np.empty(((R + br - 1) // br, (Cn + bc - 1) // bc), dtype=np.float32)
    lib().orc_quant_blocks(_p(v), R, Cn, br, bc, _p(q), _p(s))
    return q, s


# ----------------------------------------------------------------------------
# router, selection, histogram, permutation
# ----------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_r: np.ndarray, bias=None):
    """fp64 logits [T][E] and the matching sum of |products| [T][E]."""
    x = np.ascontiguousarray(x)
    w_r = np.ascontiguousarray(w_r)
    dt = _dt_of(x)
    assert _dt_of(w_r) == dt
    T, d = x.shape
    E = w_r.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    lg = np.empty((T, E), dtype=np.float64)
    ad = np.empty((T, E), dtype=np.float64)
    lib().orc_router_logits(_p(x), _p(w_r), dt, _p(b), T, d, E, _p(lg), _p(ad))
    return lg, ad


def topk(logits32: np.ndarray, k: int, renorm: bool = False):
    """Selection from binary32 logits: (idx int32 [T][k], w fp64 [T][k])."""
    lg = _c(logits32, np.float32)
    T, E = lg.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().orc_topk(_p(lg), T, E, k, int(renorm), _p(idx), _p(w))
    return idx, w


def counts_offsets(idx: np.ndarray, E: int, n_shared: int = 0):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + n_shared + 1, dtype=np.int32)
    rc = lib().orc_counts_offsets(_p(idx), T, k, E, n_shared, _p(counts), _p(offsets))
    if rc != 0:
        raise ValueError("expert index out of range")
    return counts, offsets


def permutation(idx: np.ndarray, E: int, offsets: np.ndarray):
    idx = _c(idx, np.int32)
    offsets = _c(offsets, np.int32)
    T, k = idx.shape
    perm_src = np.empty(T * k, dtype=np.int32)
    f2r = np.empty(T * k, dtype=np.int32)
    lib().orc_permutation(_p(idx), T, k, E, _p(offsets), _p(perm_src), _p(f2r))
    return perm_src, f2r


def capacity_permutation(idx: np.ndarray, E: int, capacity: int, n_shared: int = 0):
    """(counts, offsets, perm_src [kept rows], flat_to_row [T*k + n_shared*T],
    overflow [dropped]) with each expert capped at `capacity` rows."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + n_shared + 1, dtype=np.int32)
    perm_src = np.full(T * k, -1, dtype=np.int32)
    f2r = np.empty(T * k + n_shared * T, dtype=np.int32)
    overflow = np.full(T * k, -1, dtype=np.int32)
    n = lib().orc_capacity_permutation(_p(idx), T, k, E, n_shared, int(capacity), _p(counts),
                                       _p(offsets), _p(perm_src), _p(f2r), _p(overflow))
    if n < 0:
        raise ValueError("expert index out of range")
    return counts, offsets, perm_src[: offsets[E]], f2r, overflow[:n]


def router_stats(logits32: np.ndarray, counts: np.ndarray, k: int, alpha: float):
    """(f [E], P [E], aux, max_over_mean, entropy) in fp64."""
    lg = _c(logits32, np.float32)
    T, E = lg.shape
    counts = _c(counts, np.int32)
    f = np.empty(E, dtype=np.float64)
    P = np.empty(E, dtype=np.float64)
    summ = np.empty(3, dtype=np.float64)
    lib().orc_router_stats(_p(lg), T, E, _p(counts), k, float(alpha), _p(f), _p(P), _p(summ))
    return f, P, float(summ[0]), float(summ[1]), float(summ[2])


def permute_rows(x: np.ndarray, k: int, perm_src: np.ndarray, rows: np.ndarray):
    """Byte copies of x_perm for the listed rows."""
    x = np.ascontiguousarray(x)
    T, d = x.shape
    rows = _c(rows, np.int64)
    perm_src = _c(perm_src, np.int32)
    out = np.empty((len(rows), d), dtype=x.dtype)
    lib().orc_permute_rows(_p(x), x.dtype.itemsize, T, d, k, _p(perm_src),
                           _p(rows), len(rows), _p(out))
    return out


# ----------------------------------------------------------------------------
# grouped GEMM and combine
# ----------------------------------------------------------------------------

def gemm_rows(A, B, offsets, rows, B2=None, swiglu=False):
    """fp64 grouped GEMM for the listed rows: out [len(rows)][N]."""
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    G, N, K = B.shape
    assert A.shape[1] == K
    if swiglu:
        B2 = np.ascontiguousarray(B2)
        assert B2.shape == B.shape and _dt_of(B2) == _dt_of(B)
    offsets = _c(offsets, np.int32)
    rows = _c(rows, np.int64)
    out = np.empty((len(rows), N), dtype=np.float64)
    lib().orc_gemm_rows(_p(A), _dt_of(A), _p(B), _p(B2 if swiglu else None), _dt_of(B),
                        _p(offsets), G, N, K, int(swiglu), _p(rows), len(rows), _p(out))
    return out


def gemm_fp8_rows(Aq, As, Bq, Bs, offsets, rows, B2q=None, B2s=None, swiglu=False):
    Aq, As, Bq, Bs = (_c(Aq, np.uint8), _c(As, np.float32), _c(Bq, np.uint8),
                      _c(Bs, np.float32))
    G, N, K = Bq.shape
    if swiglu:
        B2q, B2s = _c(B2q, np.uint8), _c(B2s, np.float32)
    offsets = _c(offsets, np.int32)
    rows = _c(rows, np.int64)
    out = np.empty((len(rows), N), dtype=np.float64)
    lib().orc_gemm_fp8_rows(_p(Aq), _p(As), _p(Bq), _p(Bs),
                            _p(B2q if swiglu else None), _p(B2s if swiglu else None),
                            _p(offsets), G, N, K, int(swiglu), _p(rows), len(rows), _p(out))
    return out


def combine(Y, flat_to_row, w, T: int, k: int, n_shared: int = 0):
    Y = np.ascontiguousarray(Y)
    d = Y.shape[1]
    f2r = _c(flat_to_row, np.int32)
    w = _c(w, np.float32)
    out = np.empty((T, d), dtype=np.float64)
    lib().orc_combine(_p(Y), _dt_of(Y), _p(f2r), _p(w), T, k, d, n_shared, _p(out))
    return out


# ----------------------------------------------------------------------------
# the whole layer, token by token
# ----------------------------------------------------------------------------

class Layer:
    """Holds numpy views of one layer's inputs for ``moe_tokens``.

    mode: F32 / BF16 (weights in that type, given as float32 or uint16 bf16
    bit patterns) or E4M3 (weights given as uint8 codes + float32 128x128
    block scales).  Groups 0..E-1 are routed experts, E..E+n_shared-1 shared.
    ``wg``, ``wu``, ``wd`` are lists with one entry per group (None for a
    group that is never needed).
    """

    def __init__(self, x, E, k, n_shared, wg, wu, wd, mode=None, sg=None, su=None, sd=None):
        self.x = np.ascontiguousarray(x)
        self.T, self.d = self.x.shape
        self.E, self.k, self.n_shared = E, k, n_shared
        G = E + n_shared
        assert len(wg) == len(wu) == len(wd) == G
        first = next(a for a in wg if a is not None)
        self.dff = first.shape[0]
        if mode is None:
            mode = _dt_of(first)
        self.mode = mode
        self._keep = []

        def arr(lst, dtype=None):
            ptrs = (C.c_void_p * G)()
            for g, a in enumerate(lst):
                if a is None:
                    ptrs[g] = None
                else:
                    a = np.ascontiguousarray(a) if dtype is None else _c(a, dtype)
                    self._keep.append(a)
                    ptrs[g] = a.ctypes.data
            self._keep.append(ptrs)
            return ptrs

        if mode == E4M3:
            self._wg, self._wu, self._wd = arr(wg, np.uint8), arr(wu, np.uint8), arr(wd, np.uint8)
            self._sg, self._su, self._sd = (arr(sg, np.float32), arr(su, np.float32),
                                            arr(sd, np.float32))
        else:
            self._wg, self._wu, self._wd = arr(wg), arr(wu), arr(wd)
            null = (C.c_void_p * G)()
            self._keep.append(null)
            self._sg = self._su = self._sd = null

    def tokens(self, idx, w, tok):
        """fp64 layer output [len(tok)][d] for the listed tokens."""
        desc = LayerDesc(self.mode, _dt_of(self.x), self.T, self.d, self.dff,
                         self.E, self.k, self.n_shared, self.x.ctypes.data,
                         self._wg, self._wu, self._wd, self._sg, self._su, self._sd)
        idx = _c(idx, np.int32)
        w = _c(w, np.float64)
        tok = _c(tok, np.int64)
        out = np.empty((len(tok), self.d), dtype=np.float64)
        rc = lib().orc_moe_tokens(C.byref(desc), _p(idx), _p(w), _p(tok), len(tok), _p(out))
        if rc != 0:
            raise ValueError("a group needed by the listed tokens has no weights")
        return out


def route(x, w_r, k, bias=None, renorm=False):
    """Oracle routing: fp64 logits -> binary32 -> selection + weights.

    Returns (idx, w, logits64, absdot).
    """
    lg, ad = router_logits(x, w_r, bias)
    idx, w = topk(lg.astype(np.float32), k, renorm)
    return idx, w, lg, ad
