"""GPU parity of moe_grouped_gemm with a workspace: the last, partial round
of output tiles is cut along K into S slices whose fp32 partial tiles a
second kernel adds in slice order.

Each case is chosen (for the device's compute-unit count) so that the split
really happens -- the workspace header the kernel writes (n_split, S) is
checked against the documented plan -- and the split tiles cover every tile
height (64, 128, 256 rows), ragged group ends, both epilogues and both
output types.  Results are compared with the oracle's fp64 grouped GEMM to
the same arithmetic bound as the unsplit kernel (adding S fp32 partials in
order is still one fp32 sum of the K products, in another order), and split
runs must be bit-identical run to run.
"""
import math

import numpy as np
import pytest
import torch

from gpu_util import DEV, U32, assert_within, np_of
from test_gpu_gemm import _sampled_check, api, make, mixtral_sizes, ref_and_bound

pytestmark = pytest.mark.gpu

SPLIT_MAX, MIN_STEPS, BK, BM = 8, 32, 32, 256


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def expected_plan(sizes, nt, K, n_cu):
    """(n_split, S) of the documented plan: split only when the last round
    holds at most half as many tiles as there are CUs; S the largest power
    of two <= 8 with S * rem <= CUs, K/32 a multiple of 4 S and at least 32
    K-steps per slice."""
    tiles = sum(math.ceil(int(m) / BM) for m in sizes) * nt
    rem = tiles % n_cu
    if rem == 0 or 2 * rem > n_cu:
        return 0, 1
    KT = K // BK
    S = SPLIT_MAX
    while S > 1 and (S * rem > n_cu or KT % (4 * S) or KT // S < MIN_STEPS):
        S //= 2
    return (rem if S > 1 else 0), S


def run(A, B, B2, offs, out_dtype, swiglu, ws):
    a = api()
    rows, N = A.shape[0], B.shape[1]
    C = torch.full((rows, N), float("nan"), dtype=out_dtype, device=DEV)
    a.moe_grouped_gemm(A, B, C, torch.from_numpy(offs).to(DEV), B2=B2,
                       epi=a.MOE_EPI_SWIGLU if swiglu else a.MOE_EPI_NONE, ws=ws)
    torch.cuda.synchronize()
    return C


def workspace(A, B, swiglu):
    a = api()
    G, N, K = B.shape
    n = a.moe_grouped_gemm_workspace_size(G, A.shape[0], N, K, torch.bfloat16,
                                          a.MOE_EPI_SWIGLU if swiglu else a.MOE_EPI_NONE)
    assert n > 0
    return torch.full((n,), 0xAB, dtype=torch.uint8, device=DEV)


def header(ws):
    h = ws[:8].view(torch.int32).cpu().tolist()
    return h[0], h[1]


# (sizes, N, K, swiglu): the last round is every tile, so every tile is
# split; tile heights 64 (37, 65, ..), 128 (100, 129), 256 (300 -> 256 + 64)
CASES = [
    ([300, 37, 400, 129], 256, 4096, False),       # 6 tiles, S = 4
    ([65, 200, 0, 129, 257], 128, 4096, True),     # 5 tiles, S = 4
    ([100], 256, 8192, False),                     # 1 tile, S = 8
    ([500, 64], 256, 2048, False),                 # 3 tiles, S = 2
    ([1, 255, 3], 256, 2048, True),                # SwiGLU, nt = 2: 6 tiles, S = 2
]


@pytest.mark.parametrize("sizes,N,K,swiglu", CASES)
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_split_all_rows(orc, sizes, N, K, swiglu, out):
    A, B, B2, offs = make(sizes, N, K, torch.bfloat16, 700 + K + N, swiglu)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    ws = workspace(A, B, swiglu)
    C = run(A, B, B2, offs, odt, swiglu, ws)
    nt = N // 128 if swiglu else N // 256
    n_split, S = expected_plan(sizes, nt, K, cus())
    assert n_split > 0
    assert header(ws) == (n_split, S)
    ref, bound = ref_and_bound(orc, np_of(A), np_of(B), None if B2 is None else np_of(B2), offs,
                               np.arange(A.shape[0]), swiglu, 2.0 ** -8 if out == "bf16" else U32)
    assert_within(C.float().cpu().numpy(), ref, bound)
    # deterministic: the slices are always added in the same order
    C2 = run(A, B, B2, offs, odt, swiglu, ws)
    bits = torch.int16 if odt == torch.bfloat16 else torch.int32
    assert torch.equal(C.view(bits), C2.view(bits))


def test_full_last_round_is_not_split():
    """More than half the CUs busy in the last round: no split, and the
    result is bit-identical to the call without a workspace."""
    n_cu = cus()
    nt = n_cu // 16 + 1                    # 8 row tiles x nt > n_cu / 2 tiles
    sizes = [256] * 8
    N, K = 256 * nt, 2048
    assert expected_plan(sizes, nt, K, n_cu) == (0, 1)
    A, B, _, offs = make(sizes, N, K, torch.bfloat16, 801, False)
    ws = workspace(A, B, False)
    c_ws = run(A, B, None, offs, torch.bfloat16, False, ws)
    c_no = run(A, B, None, offs, torch.bfloat16, False, None)
    assert header(ws) == (0, 1)
    assert torch.equal(c_ws.view(torch.int16), c_no.view(torch.int16))


def test_workspace_too_small_is_reported():
    a = api()
    A, B, _, offs = make([300], 256, 4096, torch.bfloat16, 802, False)
    need = a.moe_grouped_gemm_workspace_size(1, A.shape[0], 256, 4096, torch.bfloat16,
                                             a.MOE_EPI_NONE)
    small = torch.empty((need - 16,), dtype=torch.uint8, device=DEV)
    C = torch.empty((A.shape[0], 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(a.MoEError) as e:
        a.moe_grouped_gemm(A, B, C, torch.from_numpy(offs).to(DEV), ws=small)
    assert e.value.status == a.MOE_ERR_WORKSPACE
    # short K: the shape never splits and needs no workspace
    assert a.moe_grouped_gemm_workspace_size(1, 300, 256, 256, torch.bfloat16,
                                             a.MOE_EPI_NONE) == 0


def test_mixtral_down_split_sampled(orc):
    """The full Mixtral-shape down GEMM as the layer launches it (with a
    workspace): with ~4.3 row tiles per expert and 16 column tiles the last
    round is a small remainder, which is split; sampled rows of every group,
    including the last group's final rows (they sit in the split tiles)."""
    sizes = mixtral_sizes()
    A, B, _, offs = make(sizes, 4096, 14336, torch.bfloat16, 400, False)
    ws = workspace(A, B, False)
    C = run(A, B, None, offs, torch.bfloat16, False, ws)
    n_split, S = expected_plan(sizes, 16, 14336, cus())
    assert header(ws) == (n_split, S)
    _sampled_check(orc, A, B, None, offs, C, False, per_group=2)
    last = int(offs[-1])
    n = 70                                      # the last group's final rows
    ref, bound = ref_and_bound(orc, np_of(A[last - n:last]), np_of(B[-1:]), None,
                               np.array([0, n], np.int32), np.arange(n), False, 2.0 ** -8)
    assert_within(C[last - n:last].float().cpu().numpy(), ref, bound)


def test_decode_gate_up_split_sampled(orc):
    """Decode-size gate/up (256 rows over 8 experts, d 4096, d_ff 14336):
    896 tiles of 64 rows, the last 128 split in two."""
    sizes = [89, 55, 41, 27, 19, 12, 9, 4]
    A, B, B2, offs = make(sizes, 14336, 4096, torch.bfloat16, 803, True)
    ws = workspace(A, B, True)
    C = run(A, B, B2, offs, torch.bfloat16, True, ws)
    n_split, S = expected_plan(sizes, 112, 4096, cus())
    assert header(ws) == (n_split, S)
    _sampled_check(orc, A, B, B2, offs, C, True, per_group=2)


@pytest.mark.parametrize("sizes,N,K,swiglu,pad", [
    ([89, 55, 41, 27, 19, 12, 9, 4], 14336, 4096, True, 128),   # decode gate/up, as the layer
    ([300, 37, 400, 129], 256, 4096, False, 8),                  # every tile split, S = 4
])
def test_split_with_padded_weight_rows(orc, sizes, N, K, swiglu, pad):
    """Split tiles with weight rows further apart than K (the layer stores
    8 KB weight rows with 256 bytes of padding); the pad columns hold NaN,
    so any read past a row's K elements would show in the output, and the
    result must be bit-identical to the one with contiguous weights."""
    from test_gpu_gemm import pad_rows
    A, B, B2, offs = make(sizes, N, K, torch.bfloat16, 805 + pad, swiglu)
    ws = workspace(A, B, swiglu)
    C = run(A, pad_rows(B, pad), pad_rows(B2, pad), offs, torch.bfloat16, swiglu, ws)
    nt = N // 128 if swiglu else N // 256
    assert header(ws) == expected_plan(sizes, nt, K, cus())
    _sampled_check(orc, A, B, B2, offs, C, swiglu, per_group=2)
    C0 = run(A, B, B2, offs, torch.bfloat16, swiglu, ws)
    assert torch.equal(C.view(torch.int16), C0.view(torch.int16))


def test_non_monotone_offsets_stay_in_bounds(orc):
    """Offsets that go down are a caller error; the scheduler reads each
    clamped offset as the largest one up to its group, so the groups never
    hold more than `rows` rows and the tile count stays within the bound the
    workspace is sized for.  Here [0, 1024, 0, 1024, 0, 1024, 0] read as
    independent ranges would make 12 row tiles against a host bound of 10 and
    place split partials past the workspace; read as a running maximum it is
    group 0 with all 1024 rows and five empty groups.  A guard region after
    the workspace must come back untouched and every row must be group 0's
    product."""
    a = api()
    rows, N, K, G = 1024, 256, 8192, 6
    offs = np.array([0, 1024, 0, 1024, 0, 1024, 0], dtype=np.int32)
    A, B, _, _ = make([rows] + [0] * (G - 1), N, K, torch.bfloat16, 804, False)
    need = a.moe_grouped_gemm_workspace_size(G, rows, N, K, torch.bfloat16, a.MOE_EPI_NONE)
    guard = 1 << 20
    buf = torch.full((need + guard,), 0xAB, dtype=torch.uint8, device=DEV)
    C = run(A, B, None, offs, torch.bfloat16, False, buf[:need])
    assert header(buf) == expected_plan([rows] + [0] * (G - 1), 1, K, cus())
    assert bool((buf[need:] == 0xAB).all()), "the kernel wrote past its workspace"
    ref, bound = ref_and_bound(orc, np_of(A), np_of(B[:1]), None,
                               np.array([0, rows], np.int32), np.arange(rows), False, 2.0 ** -8)
    assert_within(C.float().cpu().numpy(), ref, bound)
