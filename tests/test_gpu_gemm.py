"""GPU parity of moe_grouped_gemm (bf16 MFMA path and the fp32 / off-grid
vector path) against the oracle's fp64 grouped GEMM.

Tolerance, elementwise, derived from the arithmetic: fp32 accumulation of K
exact products errs by at most (K + 2) u sum_k |a_k b_k| (u = 2^-24); the
SwiGLU epilogue propagates that through silu(g) u (|silu'| <= 1.1) plus a few
fp32 roundings; storing to bf16 adds at most 2^-8 |y| (fp32: u |y|).

Small cases compare every row; the full Mixtral-shape gate/up and down GEMMs
(in the launch configuration the benchmark times) compare sampled rows from
every group.
"""
import numpy as np
import pytest
import torch

from grouped_gemm_router_amd import synth
from gpu_util import (DEV, U32, abs_operand, assert_within, np_of, offsets_from_sizes,
                      sample_rows, swiglu_bound)

pytestmark = pytest.mark.gpu


def api():
    from grouped_gemm_router_amd import api as a
    return a


def make(sizes, N, K, dt, seed, swiglu):
    offs = offsets_from_sizes(sizes)
    rows = int(offs[-1])
    G = len(sizes)
    A = synth.randn((max(rows, 1), K), 1.0, seed, DEV, dt)[:rows]
    B = synth.randn((G, N, K), 1.0 / np.sqrt(K), seed + 1, DEV, dt)
    B2 = synth.randn((G, N, K), 1.0 / np.sqrt(K), seed + 2, DEV, dt) if swiglu else None
    return A.contiguous(), B, B2, offs


def ref_and_bound(orc, An, Bn, B2n, offs, rows, swiglu, store_rel):
    K = An.shape[1]
    g = orc.gemm_rows(An, Bn, offs, rows)
    eg = (K + 2) * U32 * orc.gemm_rows(abs_operand(An), abs_operand(Bn), offs, rows)
    if not swiglu:
        return g, eg + (2 * U32 + store_rel) * np.abs(g)
    u = orc.gemm_rows(An, B2n, offs, rows)
    eu = (K + 2) * U32 * orc.gemm_rows(abs_operand(An), abs_operand(B2n), offs, rows)
    bound, h = swiglu_bound(g, u, eg, eu, store_rel)
    return h, bound


def gpu_gemm(A, B, B2, offs, out_dtype, swiglu):
    a = api()
    rows = A.shape[0]
    N = B.shape[1]
    C = torch.full((rows, N), float("nan"), dtype=out_dtype, device=DEV)
    a.moe_grouped_gemm(A, B, C, torch.from_numpy(offs).to(DEV), B2=B2,
                       epi=a.MOE_EPI_SWIGLU if swiglu else a.MOE_EPI_NONE)
    torch.cuda.synchronize()
    return C


# Group sizes chosen so that the last tile of a group takes each height the
# kernel picks from its row count (64, 128 or 256 rows) on both sides of
# every switch point: 64/65, 128/129, 256/257, 320 = 256 + 64, 384 = 256 + 128.
SIZES = [
    [0, 1, 127, 129, 255, 256, 257, 600],
    [1000],
    [3, 0, 0, 5],
    [256, 256],
    [64, 65, 128, 320, 384, 385, 63],
]


@pytest.mark.parametrize("sizes", SIZES)
@pytest.mark.parametrize("N,K,swiglu", [(256, 128, False), (512, 384, False), (128, 256, True),
                                        (384, 128, True), (256, 64, False), (128, 192, True)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_bf16_all_rows(orc, sizes, N, K, swiglu, out):
    A, B, B2, offs = make(sizes, N, K, torch.bfloat16, 100 + N + K, swiglu)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    C = gpu_gemm(A, B, B2, offs, odt, swiglu)
    ref, bound = ref_and_bound(orc, np_of(A), np_of(B), None if B2 is None else np_of(B2), offs,
                               np.arange(A.shape[0]), swiglu, 2.0 ** -8 if out == "bf16" else U32)
    assert_within(C.float().cpu().numpy(), ref, bound)


# fp32 operands: N % 32 == 0 takes the fp32 matrix cores (32 x 32 tiles, K
# in chunks of 64 with a zero-padded tail: K = 40, 128, 200, 256), other N the
# vector-ALU kernel (N = 100, 72)
@pytest.mark.parametrize("sizes", [[0, 5, 64, 65, 1], [200], [31, 32, 33]])
@pytest.mark.parametrize("N,K,swiglu", [(256, 128, True), (128, 256, False), (100, 40, False),
                                        (72, 24, True), (64, 40, False), (96, 200, True)])
def test_fp32_vector_path(orc, sizes, N, K, swiglu):
    A, B, B2, offs = make(sizes, N, K, torch.float32, 200 + N, swiglu)
    C = gpu_gemm(A, B, B2, offs, torch.float32, swiglu)
    ref, bound = ref_and_bound(orc, np_of(A), np_of(B), None if B2 is None else np_of(B2), offs,
                               np.arange(A.shape[0]), swiglu, U32)
    assert_within(C.cpu().numpy(), ref, bound)


def test_bf16_off_grid_shape_uses_vector_path(orc):
    A, B, B2, offs = make([7, 70], 200, 40, torch.bfloat16, 7, False)
    C = gpu_gemm(A, B, B2, offs, torch.bfloat16, False)
    ref, bound = ref_and_bound(orc, np_of(A), np_of(B), None, offs, np.arange(A.shape[0]), False,
                               2.0 ** -8)
    assert_within(C.float().cpu().numpy(), ref, bound)


def pad_rows(B, pad):
    """B [G][N][K] as a view of [G][N][K + pad] storage whose pad columns
    hold NaN: a kernel that read past the first K elements of a row would
    carry the NaN into its output."""
    if B is None:
        return None
    G, N, K = B.shape
    store = torch.full((G, N, K + pad), float("nan"), dtype=B.dtype, device=B.device)
    store[:, :, :K] = B
    return store[:, :, :K]


# Weight rows further apart than K (the row pitch ldb the C ABI takes from the
# view's strides): every kernel path -- bf16 matrix cores, fp32 matrix cores,
# the vector-ALU kernel -- with pads of one 16-byte piece up to 256 bytes.
@pytest.mark.parametrize("dt,N,K,swiglu,pad", [
    ("bf16", 256, 128, False, 8), ("bf16", 256, 128, False, 128), ("bf16", 128, 256, True, 64),
    ("bf16", 384, 128, True, 128), ("bf16", 200, 40, False, 8),
    ("f32", 128, 256, False, 4), ("f32", 256, 128, True, 64), ("f32", 100, 40, False, 4),
    ("f32", 72, 24, True, 12)])
def test_padded_weight_rows(orc, dt, N, K, swiglu, pad):
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    A, B, B2, offs = make([0, 1, 127, 129, 257, 64], N, K, tdt, 300 + N + pad, swiglu)
    Bp, B2p = pad_rows(B, pad), pad_rows(B2, pad)
    assert Bp.stride(1) == K + pad
    C = gpu_gemm(A, Bp, B2p, offs, tdt, swiglu)
    ref, bound = ref_and_bound(orc, np_of(A), np_of(B), None if B2 is None else np_of(B2), offs,
                               np.arange(A.shape[0]), swiglu, 2.0 ** -8 if dt == "bf16" else U32)
    assert_within(C.float().cpu().numpy(), ref, bound)
    # the same bits as with contiguous weights: the pitch changes addresses only
    C0 = gpu_gemm(A, B, B2, offs, tdt, swiglu)
    bits = torch.int16 if dt == "bf16" else torch.int32
    assert torch.equal(C.view(bits), C0.view(bits))


def test_weight_views_that_are_not_row_pitched_are_refused():
    a = api()
    A, B, B2, offs = make([10], 256, 64, torch.bfloat16, 5, False)
    C = torch.empty((10, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):  # columns of a transposed matrix
        a.moe_grouped_gemm(A, B.transpose(1, 2).contiguous().transpose(1, 2), C,
                           torch.from_numpy(offs).to(DEV))
    with pytest.raises(ValueError):  # B2 with another pitch than B
        a.moe_grouped_gemm(A, pad_rows(B, 8), C, torch.from_numpy(offs).to(DEV),
                           B2=pad_rows(B, 16), epi=a.MOE_EPI_SWIGLU)


def test_rows_outside_groups_untouched():
    A, B, B2, offs = make([10, 20], 256, 64, torch.bfloat16, 9, False)
    a = api()
    C = torch.full((A.shape[0], 256), 7.0, dtype=torch.bfloat16, device=DEV)
    offs2 = offs.copy()
    offs2[-1] = 25   # last group shortened: rows 25..29 belong to no group
    a.moe_grouped_gemm(A, B, C, torch.from_numpy(offs2).to(DEV))
    torch.cuda.synchronize()
    assert (C[25:].float() == 7.0).all()


def many_group_sizes(G, seed):
    """G groups, most of them empty or a few rows, with one of every tile
    height (64, 128, 256 and a 256 + 1 split) among them."""
    rng = np.random.default_rng(seed)
    sizes = rng.integers(0, 4, G)
    sizes[rng.permutation(G)[:4]] = [300, 129, 64, 257]
    return sizes


# Group counts that give the scheduler's lanes runs of different lengths:
# 65 (runs of 2, the last lane's cut short), 129 (runs of 3) and the
# 1040-group limit (runs of 17, the longest).  K = 128 runs the MFMA kernel,
# K = 64 the vector path.
@pytest.mark.parametrize("G", [65, 129, 1040])
@pytest.mark.parametrize("K", [128, 64])
@pytest.mark.parametrize("swiglu", [False, True])
def test_many_groups_all_rows(orc, G, K, swiglu):
    sizes = many_group_sizes(G, 800 + G)
    N = 128 if swiglu else 256
    A, B, B2, offs = make(sizes, N, K, torch.bfloat16, 810 + G + K, swiglu)
    C = gpu_gemm(A, B, B2, offs, torch.bfloat16, swiglu)
    ref, bound = ref_and_bound(orc, np_of(A), np_of(B), None if B2 is None else np_of(B2), offs,
                               np.arange(A.shape[0]), swiglu, 2.0 ** -8)
    assert_within(C.float().cpu().numpy(), ref, bound)


def _sampled_check(orc, A, B, B2, offs, C, swiglu, per_group=4):
    rows = sample_rows(offs, per_group=per_group, seed=1)
    An = np_of(A[torch.from_numpy(rows).to(DEV)])
    got = C[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    ref = np.empty_like(got, dtype=np.float64)
    bound = np.empty_like(got, dtype=np.float64)
    groups = np.searchsorted(offs, rows, side="right") - 1
    for g in np.unique(groups):
        sel = np.where(groups == g)[0]
        Bg = np_of(B[g:g + 1])
        B2g = np_of(B2[g:g + 1]) if swiglu else None
        ref[sel], bound[sel] = ref_and_bound(orc, An[sel], Bg, B2g,
                                             np.array([0, len(sel)], np.int32),
                                             np.arange(len(sel)), swiglu, 2.0 ** -8)
    assert_within(got, ref, bound)


def mixtral_sizes():
    idx = synth.random_selection(4096, 8, 2, s=77).numpy()
    return np.bincount(idx.ravel(), minlength=8)


def test_mixtral_gate_up_full_size_sampled(orc):
    sizes = mixtral_sizes()
    A, B, B2, offs = make(sizes, 14336, 4096, torch.bfloat16, 300, True)
    C = gpu_gemm(A, B, B2, offs, torch.bfloat16, True)
    _sampled_check(orc, A, B, B2, offs, C, True, per_group=2)


def test_mixtral_down_full_size_sampled(orc):
    sizes = mixtral_sizes()
    A, B, _, offs = make(sizes, 4096, 14336, torch.bfloat16, 400, False)
    C = gpu_gemm(A, B, None, offs, torch.bfloat16, False)
    _sampled_check(orc, A, B, None, offs, C, False, per_group=2)


def test_deepseek_shaped_groups_sampled(orc):
    """257 groups of ~128 rows (256 routed experts at T=4096, k=8, plus a
    4096-row shared group): most tiles are the 128- or 256-row kind; K as
    the DeepSeek gate/up, N cut to 256 to keep the weights small."""
    rng = np.random.default_rng(11)
    sizes = np.concatenate([rng.integers(98, 166, 256), [4096]])
    A, B, B2, offs = make(sizes, 256, 7168, torch.bfloat16, 500, True)
    C = gpu_gemm(A, B, B2, offs, torch.bfloat16, True)
    _sampled_check(orc, A, B, B2, offs, C, True, per_group=2)


def test_decode_shaped_groups_all_rows(orc):
    """Skewed decode: 256 rows over 8 experts, every tile 64 or 128 rows."""
    sizes = [89, 55, 41, 27, 19, 12, 9, 4]
    A, B, _, offs = make(sizes, 512, 1024, torch.bfloat16, 600, False)
    C = gpu_gemm(A, B, None, offs, torch.bfloat16, False)
    ref, bound = ref_and_bound(orc, np_of(A), np_of(B), None, offs, np.arange(A.shape[0]), False,
                               2.0 ** -8)
    assert_within(C.float().cpu().numpy(), ref, bound)


def test_gemm_is_deterministic():
    A, B, B2, offs = make([300, 700, 0, 1024], 1024, 512, torch.bfloat16, 5, True)
    c1 = gpu_gemm(A, B, B2, offs, torch.bfloat16, True)
    c2 = gpu_gemm(A, B, B2, offs, torch.bfloat16, True)
    assert torch.equal(c1, c2)
