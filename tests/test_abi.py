"""CPU checks of the C ABI: the library loads, exports every function that
include/moe.h declares, and the host-side argument checks return the
documented status without launching anything (no GPU is touched: every call
below fails validation, or is a documented no-op, before any launch)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "grouped_gemm_router_amd", "libmoe.so")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
F32, BF16, E4M3 = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from grouped_gemm_router_amd import build
        build.build()
    L = C.CDLL(LIB)
    vp, i32, u32, sz = C.c_void_p, C.c_int, C.c_uint, C.c_size_t
    L.moe_route.argtypes = [vp, vp, i32, vp, i32, i32, i32, i32, u32, vp, vp, vp, vp, vp, sz, vp]
    L.moe_route_workspace_size.restype = sz
    L.moe_route_workspace_size.argtypes = [i32, i32, i32]
    L.moe_permute_workspace_size.restype = sz
    L.moe_permute_workspace_size.argtypes = [i32, i32, i32]
    L.moe_permute.argtypes = [vp, i32, i32, i32, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                              vp, sz, vp]
    L.moe_grouped_gemm_workspace_size.restype = sz
    L.moe_grouped_gemm_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    L.moe_grouped_gemm.argtypes = [vp, vp, vp, i32, vp, i32, vp, i32, i32, i32, i32, i32, i32,
                                   vp, sz, vp]
    L.moe_grouped_gemm_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32,
                                       i32, i32, i32, vp]
    L.moe_combine.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, i32, vp]
    L.moe_quantize_fp8.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp]
    L.moe_permute_capped.argtypes = [vp, i32, i32, i32, vp, i32, i32, i32, i32, i32, vp, vp, vp,
                                     vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_router_stats.argtypes = [vp, vp, i32, i32, i32, C.c_float, vp, vp, vp, vp]
    L.moe_status_string.restype = C.c_char_p
    L.moe_status_string.argtypes = [i32]
    return L


P = C.c_void_p(0x10000)      # an aligned, never-dereferenced stand-in pointer
P2 = C.c_void_p(0x20000)
MIS = C.c_void_p(0x10002)    # misaligned
NUL = C.c_void_p(0)


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert len(names) == 14, names
    for n in names:
        assert hasattr(lib, n), "libmoe.so does not export %s" % n


def test_status_strings_and_version(lib):
    for s in range(5):
        assert lib.moe_status_string(s)
    assert lib.moe_abi_version() == 8


def test_route_validation(lib):
    big = 1 << 40
    # (..., topk_w, prob_sums, stream) with an ample workspace
    r = lambda *a: lib.moe_route(*a[:-2], a[-2], P2, big, a[-1])  # noqa: E731
    # k > E, k < 1, E > max, d % 8, dtype, null outputs, misaligned x
    assert r(P, P, BF16, NUL, 16, 64, 4, 5, 0, NUL, P, P, NUL, NUL) == INVALID
    assert r(P, P, BF16, NUL, 16, 64, 4, 0, 0, NUL, P, P, NUL, NUL) == INVALID
    assert r(P, P, BF16, NUL, 16, 64, 2000, 2, 0, NUL, P, P, NUL, NUL) == UNSUPPORTED
    assert r(P, P, BF16, NUL, 16, 60, 8, 2, 0, NUL, P, P, NUL, NUL) == UNSUPPORTED
    assert r(P, P, E4M3, NUL, 16, 64, 8, 2, 0, NUL, P, P, NUL, NUL) == UNSUPPORTED
    assert r(P, P, BF16, NUL, 16, 64, 8, 2, 0, NUL, NUL, P, NUL, NUL) == INVALID
    assert r(MIS, P, BF16, NUL, 16, 64, 8, 2, 0, NUL, P, P, NUL, NUL) == INVALID
    assert r(P, P, BF16, NUL, 16, 64, 8, 2, 0, NUL, P, P, MIS, NUL) == INVALID  # prob_sums
    assert r(P, P, BF16, NUL, 16, 64, 8, 2, 8, NUL, P, P, NUL, NUL) == INVALID  # unknown flag
    assert r(NUL, NUL, BF16, NUL, 16, 64, 8, 2, 2, NUL, P, P, NUL, NUL) == INVALID  # no logits
    assert r(P, P, BF16, NUL, -1, 64, 8, 2, 0, NUL, P, P, NUL, NUL) == INVALID
    assert r(P, P, BF16, NUL, 0, 64, 8, 2, 0, NUL, P, P, NUL, NUL) == OK  # T == 0: no-op


def test_route_workspace(lib):
    need = lib.moe_route_workspace_size(4096, 7168, 256)
    assert need >= 4096 * 256 * 4 and need % (4096 * 256 * 4) == 0
    assert lib.moe_route_workspace_size(-1, 64, 8) == 0
    assert lib.moe_route_workspace_size(4096, 4096, 8) == 0   # E <= 32: one launch, no workspace
    args = (P, P, BF16, NUL, 4096, 7168, 256, 8, 0, NUL, P, P, NUL)
    assert lib.moe_route(*args, P2, need - 1, NUL) == WORKSPACE
    assert lib.moe_route(*args, NUL, 0, NUL) == WORKSPACE
    assert lib.moe_route(*args, MIS, need, NUL) == INVALID
    # from-logits needs no workspace; with T == 0 nothing is launched
    assert lib.moe_route(NUL, NUL, BF16, NUL, 0, 8, 256, 8, 2, P, P, P, NUL, NUL, 0, NUL) == OK


def test_permute_validation_and_workspace(lib):
    ws = lib.moe_permute_workspace_size(4096, 8, 256)
    assert ws >= 64 * 256 * 4
    assert lib.moe_permute_workspace_size(-1, 2, 8) == 0
    p = lambda x_dt, T, d, k, E, ns, odt, scale, wsb: lib.moe_permute(  # noqa: E731
        P, x_dt, T, d, P, k, E, ns, odt, P, scale, P, P, P, P, P, wsb, NUL)
    assert p(BF16, 4096, 4096, 2, 8, 0, BF16, NUL, 0) == WORKSPACE
    # (a large enough workspace passes validation and would launch, so only
    # failing cases are exercised here)
    assert p(BF16, 64, 4096, 2, 8, 0, F32, NUL, 1 << 20) == UNSUPPORTED   # dtype change
    assert p(BF16, 64, 4100, 2, 8, 0, E4M3, P, 1 << 20) == UNSUPPORTED    # d % 128 for fp8
    assert p(BF16, 64, 4096, 2, 8, 0, E4M3, NUL, 1 << 20) == INVALID      # fp8 needs scales
    assert p(BF16, 64, 4096, 2, 8, 0, BF16, P, 1 << 20) == INVALID        # scales only for fp8
    assert p(BF16, 64, 4096, 9, 8, 0, BF16, NUL, 1 << 20) == INVALID      # k > E
    assert p(BF16, 0, 4096, 2, 8, 0, BF16, NUL, 0) == OK                  # T == 0


def test_permute_noalloc_validation(lib):
    """The allocation-free permute checks its arguments like moe_permute and
    refuses sizes whose per-block counts exceed its static scratch, before
    any launch (and before it looks up the scratch on a device)."""
    vp, i32 = C.c_void_p, C.c_int
    lib.moe_permute_noalloc.argtypes = [vp, i32, i32, i32, vp, i32, i32, i32, i32, vp, vp, vp, vp,
                                        vp, vp, vp]
    p = lambda T, d, k, E, odt=BF16, scale=NUL: lib.moe_permute_noalloc(  # noqa: E731
        P, BF16, T, d, P, k, E, 0, odt, P, scale, P, P, P, P, NUL)
    limit = 1 << 20
    assert lib.moe_permute_workspace_size(65472, 8, 256) <= limit
    assert lib.moe_permute_workspace_size(65536, 8, 256) > limit
    assert p(65536, 4096, 8, 256) == WORKSPACE
    assert p(16384, 4096, 8, 1024) == WORKSPACE
    assert p(64, 4096, 9, 8) == INVALID                 # k > E
    assert p(64, 4096, 2, 8, F32) == UNSUPPORTED        # dtype change
    assert p(64, 4096, 2, 8, E4M3, NUL) == INVALID      # fp8 needs scales
    assert p(0, 4096, 2, 8) == OK                       # T == 0: nothing launched


def test_permute_workspace_error_is_reported(lib):
    need = lib.moe_permute_workspace_size(1000, 2, 8)
    assert need > 0
    rc = lib.moe_permute(P, BF16, 1000, 64, P, 2, 8, 0, BF16, P, NUL, P, P, P, P, P, need - 1, NUL)
    assert rc == WORKSPACE


def test_gemm_validation(lib):
    g = lambda A, B, B2, dt, cdt, G, rows, N, K, epi, ldb=0: lib.moe_grouped_gemm(  # noqa: E731
        A, B, B2, dt, P, cdt, P, G, rows, N, K, ldb, epi, NUL, 0, NUL)
    assert g(P, P, NUL, BF16, BF16, 0, 10, 256, 64, 0) == INVALID        # G < 1
    assert g(P, P, NUL, BF16, BF16, 5000, 10, 256, 64, 0) == UNSUPPORTED  # G > max
    assert g(P, P, NUL, BF16, BF16, 2, 10, 256, 60, 0) == UNSUPPORTED    # K % 8
    assert g(P, P, NUL, E4M3, BF16, 2, 10, 256, 64, 0) == UNSUPPORTED    # fp8 via bf16 entry
    assert g(P, P, NUL, BF16, BF16, 2, 10, 256, 64, 1) == INVALID        # SwiGLU needs B2
    assert g(P, P, P2, BF16, BF16, 2, 10, 256, 64, 0) == INVALID         # B2 without SwiGLU
    assert g(P, P, NUL, BF16, BF16, 2, 10, 256, 64, 7) == INVALID        # bad epilogue
    assert g(MIS, P, NUL, BF16, BF16, 2, 10, 256, 64, 0) == INVALID
    assert g(P, P, NUL, BF16, BF16, 2, 0, 256, 64, 0) == OK              # no rows: no-op
    # weight row pitch: at least K, rows 16-byte aligned
    assert g(P, P, NUL, BF16, BF16, 2, 10, 256, 64, 0, 56) == INVALID    # ldb < K
    assert g(P, P, NUL, BF16, BF16, 2, 10, 256, 64, 0, -8) == INVALID
    assert g(P, P, NUL, BF16, BF16, 2, 10, 256, 64, 0, 68) == INVALID    # 136-byte rows
    assert g(P, P, NUL, F32, F32, 2, 10, 256, 64, 0, 66) == INVALID      # 264-byte rows
    assert g(P, P, NUL, BF16, BF16, 2, 0, 256, 64, 0, 72) == OK          # 144-byte rows
    assert g(P, P, NUL, F32, F32, 2, 0, 256, 64, 0, 68) == OK            # 272-byte rows
    # a workspace size without a workspace
    assert lib.moe_grouped_gemm(P, P, NUL, BF16, P, BF16, P, 2, 10, 256, 64, 0, 0, NUL, 64,
                                NUL) == INVALID


def test_gemm_workspace_size(lib):
    ws = lib.moe_grouped_gemm_workspace_size
    assert ws(0, 1024, 4096, 14336, BF16, 0) == 0        # invalid G
    assert ws(8, -1, 4096, 14336, BF16, 0) == 0          # invalid rows
    assert ws(8, 1024, 4096, 14336, F32, 0) == 0         # only the bf16 path splits
    assert ws(8, 1024, 4096, 14336, BF16, 5) == 0        # bad epilogue
    assert ws(8, 1024, 4096, 200, BF16, 0) == 0          # off the MFMA grid
    assert ws(8, 1024, 4096, 256, BF16, 0) == 0          # K too short to cut in two


def test_gemm_fp8_validation(lib):
    f = lambda N, K, cdt, cs, b2, b2s, epi, ldb=0, rows=10: lib.moe_grouped_gemm_fp8(  # noqa: E731
        P, P, P, P, b2, b2s, P, cdt, cs, P, 2, rows, N, K, ldb, epi, NUL)
    assert f(200, 256, BF16, NUL, NUL, NUL, 0) == UNSUPPORTED   # N % 128
    assert f(256, 200, BF16, NUL, NUL, NUL, 0) == UNSUPPORTED   # K % 128
    assert f(256, 256, F32, NUL, NUL, NUL, 0) == UNSUPPORTED    # output dtype
    assert f(256, 256, E4M3, NUL, NUL, NUL, 0) == INVALID       # fp8 output needs scales
    assert f(256, 256, BF16, P, NUL, NUL, 0) == INVALID         # scales only for fp8 output
    assert f(256, 256, BF16, NUL, NUL, NUL, 1) == INVALID       # SwiGLU needs B2
    assert f(256, 256, BF16, NUL, P, P, 0) == INVALID           # B2 without SwiGLU
    assert f(256, 256, BF16, NUL, NUL, NUL, 0, 128) == INVALID  # ldb < K
    assert f(256, 256, BF16, NUL, NUL, NUL, 0, 264) == INVALID  # rows not 16-byte aligned
    assert f(256, 256, BF16, NUL, NUL, NUL, 0, 512, 0) == OK    # padded rows, nothing to do


def test_combine_and_quant_validation(lib):
    c = lambda T, k, d, ns, ydt, odt: lib.moe_combine(  # noqa: E731
        P, ydt, P, P, T, k, d, ns, P, odt, NUL)
    assert c(16, 0, 64, 0, BF16, BF16) == INVALID
    assert c(16, 2, 60, 0, BF16, BF16) == UNSUPPORTED
    assert c(16, 2, 64, 0, E4M3, BF16) == UNSUPPORTED
    assert c(16, 40, 64, 0, BF16, BF16) == UNSUPPORTED
    assert c(0, 2, 64, 0, BF16, BF16) == OK
    q = lambda R, Cn, br, bc, dt: lib.moe_quantize_fp8(P, dt, R, Cn, br, bc, P, P, NUL)  # noqa: E731
    assert q(256, 256, 64, 128, F32) == UNSUPPORTED
    assert q(256, 256, 128, 64, F32) == UNSUPPORTED
    assert q(200, 256, 128, 128, F32) == UNSUPPORTED
    assert q(256, 200, 1, 128, F32) == UNSUPPORTED
    assert q(256, 256, 128, 128, E4M3) == UNSUPPORTED
    assert q(0, 256, 128, 128, F32) == OK


def test_permute_capped_validation(lib):
    need = lib.moe_permute_workspace_size(1000, 2, 8)
    c = lambda cap, ov, wsb: lib.moe_permute_capped(  # noqa: E731
        P, BF16, 1000, 64, P, 2, 8, 0, cap, BF16, P, NUL, P, P, P, P, ov, NUL, P2, wsb, NUL)
    assert c(-1, NUL, need) == INVALID          # negative capacity
    assert c(10, MIS, need) == INVALID          # misaligned overflow list
    assert c(10, NUL, need - 1) == WORKSPACE
    assert lib.moe_permute_capped(P, BF16, 0, 64, P, 2, 8, 0, 5, BF16, P, NUL, P, P, P, P, NUL,
                                  NUL, NUL, 0, NUL) == OK   # T == 0


def test_router_stats_validation(lib):
    s = lambda T, E, k, ps=P: lib.moe_router_stats(ps, P, T, E, k, 0.01, P, P, P, NUL)  # noqa: E731
    assert s(4096, 256, 0) == INVALID     # k < 1
    assert s(4096, 2000, 8) == UNSUPPORTED
    assert s(4096, 256, 8, MIS) == INVALID
    assert s(4096, 256, 8, NUL) == INVALID
    assert s(0, 256, 8) == OK             # T == 0: nothing launched


def test_padded_weights_layout():
    """Host logic of the layer's weight storage: rows of a power-of-two size
    of at least 4 KB get 256 bytes of padding (the GEMMs read the pitch from
    the view's strides), other rows stay contiguous; values are unchanged."""
    import torch
    from grouped_gemm_router_amd.layer import padded_weights
    cases = [((2, 3, 4096), torch.bfloat16, 4096 + 128),   # 8 KB rows
             ((2, 3, 2048), torch.bfloat16, 2048 + 128),   # 4 KB rows
             ((2, 3, 1024), torch.float32, 1024 + 64),     # 4 KB rows
             ((2, 3, 2048), torch.uint8, 2048),            # 2 KB rows: dense
             ((2, 3, 14336), torch.bfloat16, 14336),       # 28 KB: not a power of two
             ((2, 3, 7168), torch.bfloat16, 7168)]
    for shape, dt, ldb in cases:
        n = shape[0] * shape[1] * shape[2]
        w = torch.arange(n, dtype=torch.int32).remainder(251).to(dt).view(shape)
        p = padded_weights(w)
        assert p.shape == w.shape and p.stride() == (shape[1] * ldb, ldb, 1), (shape, dt)
        assert torch.equal(p, w)


def test_deferred_calls_marshal_now_and_call_later():
    """api.deferred checks and marshals an entry's arguments at once and
    returns a thunk that makes the library call each time it runs; here the
    call is one the library rejects on the host (k = 0) before any launch."""
    import torch
    from grouped_gemm_router_amd import api

    class Stream:
        cuda_stream = 0
    Y = torch.zeros((8, 64), dtype=torch.float32)
    flat = torch.zeros((0,), dtype=torch.int32)
    w = torch.zeros((4, 0), dtype=torch.float32)
    out = torch.zeros((4, 64), dtype=torch.float32)
    with pytest.raises(api.MoEError) as now:
        api.moe_combine(Y, flat, w, out, stream=Stream())
    thunk = api.deferred(api.moe_combine, Y, flat, w, out, stream=Stream())
    for _ in range(2):
        with pytest.raises(api.MoEError) as later:
            thunk()
        assert later.value.status == now.value.status == api.MOE_ERR_INVALID
    with pytest.raises(TypeError):   # not a library call
        api.deferred(api.moe_permute_workspace_size, 16, 2, 8)
    with pytest.raises(ValueError):  # array shapes are still checked when marshalling
        api.deferred(api.moe_grouped_gemm, torch.zeros((4, 64)), torch.zeros((2, 8, 32)),
                     torch.zeros((4, 8)), torch.zeros((3,), dtype=torch.int32), stream=Stream())
