"""GPU parity of moe_permute against the oracle: counts, offsets, perm_src,
flat_to_row and the permuted rows bit-exact (bf16 / fp32 copies), and the
E4M3 codes and 1 x 128 scales bit-exact against the oracle's quantiser."""
import numpy as np
import pytest
import torch

from grouped_gemm_router_amd import synth
from gpu_util import DEV, np_of

pytestmark = pytest.mark.gpu


def api():
    from grouped_gemm_router_amd import api as a
    return a


def run_permute(x, idx, E, ns, fp8=False):
    a = api()
    T, d = x.shape
    k = idx.shape[1]
    rows = T * k + ns * T
    out_dtype = torch.uint8 if fp8 else x.dtype
    x_perm = torch.full((rows, d), 0, dtype=out_dtype, device=DEV)
    scale = torch.zeros((d // 128, rows), dtype=torch.float32, device=DEV) if fp8 else None
    counts = torch.empty((E,), dtype=torch.int32, device=DEV)
    offsets = torch.empty((E + ns + 1,), dtype=torch.int32, device=DEV)
    perm_src = torch.empty((T * k,), dtype=torch.int32, device=DEV)
    f2r = torch.empty((T * k + ns * T,), dtype=torch.int32, device=DEV)
    ws = torch.empty((max(a.moe_permute_workspace_size(T, k, E), 16),), dtype=torch.uint8,
                     device=DEV)
    a.moe_permute(x, idx, E, ns, x_perm, counts, offsets, perm_src, f2r, ws,
                  x_perm_scale=scale)
    torch.cuda.synchronize()
    # scales come back group-major [d/128][rows]; hand them out row-major
    scale = scale.t().contiguous() if fp8 else None
    return x_perm, scale, counts, offsets, perm_src, f2r


CASES = [  # T, E, k, ns, d, weights
    (1, 1, 1, 0, 64, None),
    (63, 8, 2, 0, 128, None),
    (64, 8, 2, 1, 128, None),
    (4096, 8, 2, 0, 256, None),
    (1000, 256, 8, 1, 128, None),
    (777, 16, 16, 0, 64, None),
    (300, 64, 4, 2, 64, "skew"),
    (130, 32, 2, 0, 64, "empty"),
    (5000, 1024, 32, 0, 8, None),
    # one launch up to T k = 32768 entries: a ragged last workgroup; the
    # limit (the DeepSeek routing shape)
    (4097, 8, 2, 0, 64, None),
    (4096, 256, 8, 1, 64, None),
    # past the limit, three launches (rank, scan, scatter): one entry past
    # it, with a ragged 65th block of tokens
    (4097, 256, 8, 1, 64, None),
    (2049, 64, 16, 0, 64, None),
    (20000, 8, 2, 0, 64, "skew"),
]


def weights_for(kind, E):
    if kind == "skew":
        return 1.0 / (1.0 + np.arange(E)) ** 1.2
    if kind == "empty":
        w = np.full(E, 1e-12)
        w[[0, 5, 6, 31]] = [1, 2, 3, 4]
        return w
    return None


@pytest.mark.parametrize("T,E,k,ns,d,kind", CASES)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_permute_bit_exact(orc, T, E, k, ns, d, kind, dt):
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    x = synth.randn((T, d), 1.0, 21 + T, DEV, tdt)
    idx_cpu = synth.random_selection(T, E, k, s=31 + T + E, weights=weights_for(kind, E))
    idx = idx_cpu.to(DEV)
    x_perm, _, counts, offsets, perm_src, f2r = run_permute(x, idx, E, ns)
    ridx = idx_cpu.numpy()
    rc, ro = orc.counts_offsets(ridx, E, ns)
    rp, rf = orc.permutation(ridx, E, ro)
    np.testing.assert_array_equal(counts.cpu().numpy(), rc)
    np.testing.assert_array_equal(offsets.cpu().numpy(), ro)
    np.testing.assert_array_equal(perm_src.cpu().numpy(), rp)
    f = f2r.cpu().numpy()
    np.testing.assert_array_equal(f[: T * k], rf)
    # shared-expert rows follow the routed rows, token order
    for s in range(ns):
        np.testing.assert_array_equal(f[T * k + s * T: T * k + (s + 1) * T],
                                      T * k + s * T + np.arange(T))
    rows = np.arange(T * k + ns * T)
    ref = orc.permute_rows(np_of(x), k, rp, rows)
    np.testing.assert_array_equal(np_of(x_perm), ref)


# E4M3 rows take the three launches at every size; the DeepSeek routing
# shape (T k = 32768) and one token past it are among the cases
@pytest.mark.parametrize("T,E,k,ns,d", [(70, 8, 2, 0, 256), (300, 256, 8, 1, 512),
                                        (4096, 8, 2, 0, 128), (5, 3, 3, 2, 1024),
                                        (4096, 256, 8, 1, 256), (4097, 256, 8, 1, 256),
                                        (9000, 8, 4, 1, 128)])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_permute_fp8_quantisation_bit_exact(orc, T, E, k, ns, d, dt):
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    x = synth.randn((T, d), 3.0, 41 + T, DEV, tdt)
    if T > 3:
        x[1].zero_()         # an all-zero token: scale 1, codes 0
        x[2, :128].mul_(1e-30 if dt == "f32" else 1e-20)  # tiny values: subnormal codes
    idx_cpu = synth.random_selection(T, E, k, s=51 + T)
    x_perm, scale, _, _, perm_src, _ = run_permute(x, idx_cpu.to(DEV), E, ns, fp8=True)
    xf = x.float().cpu().numpy()
    qref, sref = orc.quant_blocks(xf, 1, 128)        # per token, 1 x 128 groups
    rp = perm_src.cpu().numpy()
    src_tok = np.concatenate([rp // k, np.tile(np.arange(T), ns)])
    np.testing.assert_array_equal(x_perm.cpu().numpy(), qref[src_tok])
    np.testing.assert_array_equal(scale.cpu().numpy(), sref[src_tok])


@pytest.mark.parametrize("T,E,k", [(300, 8, 2), (999, 64, 8), (4097, 256, 8)])
def test_index_array_without_16_byte_alignment(T, E, k):
    """topk_idx at a 4-byte but not 16-byte aligned address (the one-launch
    path then reads it entry by entry) gives the same result as an aligned
    copy, bit for bit."""
    x = synth.randn((T, 128), 1.0, 5 + T, DEV, torch.bfloat16)
    idx = synth.random_selection(T, E, k, s=6 + T).to(DEV)
    buf = torch.empty((T * k + 4,), dtype=torch.int32, device=DEV)
    odd = buf[1: 1 + T * k].view(T, k)
    odd.copy_(idx)
    assert odd.data_ptr() % 16 == 4
    ref = run_permute(x, idx, E, 1)
    got = run_permute(x, odd, E, 1)
    for u, v in zip(ref, got):
        if u is not None:
            assert torch.equal(u, v)


def test_dropped_entries_stay_in_bounds(orc):
    """Expert ids outside [0, E) are dropped: not counted, flat_to_row -1,
    rows compact; the remaining entries are still a stable sort."""
    T, E, k, d = 200, 8, 2, 64
    idx_cpu = synth.random_selection(T, E, k, s=3)
    idx_np = idx_cpu.numpy().copy()
    idx_np[::7, 1] = -1
    idx_np[::11, 0] = E + 3
    x = synth.randn((T, d), 1.0, 4, DEV, torch.bfloat16)
    x_perm, _, counts, offsets, perm_src, f2r = run_permute(
        x, torch.from_numpy(idx_np).to(DEV), E, 1)
    valid = (idx_np >= 0) & (idx_np < E)
    flat = idx_np.ravel()
    np.testing.assert_array_equal(counts.cpu().numpy(),
                                  np.bincount(flat[valid.ravel()], minlength=E))
    n = int(valid.sum())
    o = offsets.cpu().numpy()
    assert o[E] == n and o[E + 1] == n + T
    f = f2r.cpu().numpy()
    assert (f[: T * k][~valid.ravel()] == -1).all()
    order = np.argsort(np.where(valid.ravel(), flat, E), kind="stable")[:n]
    np.testing.assert_array_equal(perm_src.cpu().numpy()[:n], order)
    np.testing.assert_array_equal(f[T * k:], n + np.arange(T))


def test_permute_is_deterministic():
    T, E, k, d = 4096, 256, 8, 256
    x = synth.randn((T, d), 1.0, 8, DEV, torch.bfloat16)
    idx = synth.random_selection(T, E, k, s=9).to(DEV)
    r1 = run_permute(x, idx, E, 1)
    r2 = run_permute(x, idx, E, 1)
    for u, v in zip(r1, r2):
        if u is not None:
            assert torch.equal(u, v)


def run_permute_capped(x, idx, E, ns, cap, fp8=False):
    a = api()
    T, d = x.shape
    k = idx.shape[1]
    rows = T * k + ns * T
    x_perm = torch.full((rows, d), 0, dtype=torch.uint8 if fp8 else x.dtype, device=DEV)
    scale = torch.zeros((d // 128, rows), dtype=torch.float32, device=DEV) if fp8 else None
    counts = torch.empty((E,), dtype=torch.int32, device=DEV)
    offsets = torch.empty((E + ns + 1,), dtype=torch.int32, device=DEV)
    perm_src = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    f2r = torch.empty((T * k + ns * T,), dtype=torch.int32, device=DEV)
    overflow = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    n_over = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty((max(a.moe_permute_workspace_size(T, k, E), 16),), dtype=torch.uint8,
                     device=DEV)
    a.moe_permute_capped(x, idx, E, ns, cap, x_perm, counts, offsets, perm_src, f2r, ws,
                         overflow=overflow, n_overflow=n_over, x_perm_scale=scale)
    torch.cuda.synchronize()
    if fp8:
        scale = scale.t().contiguous()
    return x_perm, scale, counts, offsets, perm_src, f2r, overflow, n_over


CAPPED = [  # T, E, k, ns, d, kind, capacity
    (300, 8, 2, 0, 128, "skew", 40),
    (300, 8, 2, 1, 128, None, 75),
    (4096, 8, 2, 0, 64, "skew", 1024),        # capacity factor 1.0 at T*k/E = 1024
    (1000, 256, 8, 1, 128, None, 20),
    (777, 16, 16, 0, 64, None, 0),            # everything routed is dropped
    (130, 32, 2, 2, 64, "empty", 5),
    (200, 8, 2, 0, 64, None, 200),            # cap >= T: the drop-less result
    (20000, 8, 2, 0, 64, "skew", 4000),       # three launches
    (4097, 256, 8, 1, 64, None, 100),         # three launches, ragged last block
]


@pytest.mark.parametrize("T,E,k,ns,d,kind,cap", CAPPED)
def test_permute_capped_bit_exact(orc, T, E, k, ns, d, kind, cap):
    x = synth.randn((T, d), 1.0, 61 + T, DEV, torch.bfloat16)
    idx_cpu = synth.random_selection(T, E, k, s=71 + T + E, weights=weights_for(kind, E))
    x_perm, _, counts, offsets, perm_src, f2r, overflow, n_over = run_permute_capped(
        x, idx_cpu.to(DEV), E, ns, cap)
    rc, ro, rp, rf, rov = orc.capacity_permutation(idx_cpu.numpy(), E, cap, ns)
    np.testing.assert_array_equal(counts.cpu().numpy(), rc)
    np.testing.assert_array_equal(offsets.cpu().numpy(), ro)
    n_kept = int(ro[E])
    ps = perm_src.cpu().numpy()
    np.testing.assert_array_equal(ps[:n_kept], rp)
    assert (ps[n_kept:] == -7).all()              # nothing written past the kept rows
    np.testing.assert_array_equal(f2r.cpu().numpy(), rf)
    assert int(n_over.cpu()[0]) == len(rov)
    ov = overflow.cpu().numpy()
    np.testing.assert_array_equal(ov[:len(rov)], rov)
    assert (ov[len(rov):] == -7).all()
    # kept rows and shared rows hold their tokens, bit for bit
    src = np.concatenate([rp // k, np.tile(np.arange(T), ns)])
    xp = np_of(x_perm)
    np.testing.assert_array_equal(xp[: n_kept + ns * T], np_of(x)[src])
    if cap >= T:
        # the drop-less entry point gives the same rows
        dp, _, _, doff, dps, df2r = run_permute(x, idx_cpu.to(DEV), E, ns)
        np.testing.assert_array_equal(doff.cpu().numpy(), ro)
        np.testing.assert_array_equal(np_of(dp), xp)


def test_permute_capped_fp8_rows(orc):
    T, E, k, ns, d, cap = 500, 16, 4, 1, 256, 60
    x = synth.randn((T, d), 2.0, 81, DEV, torch.bfloat16)
    idx_cpu = synth.random_selection(T, E, k, s=82, weights=weights_for("skew", E))
    x_perm, scale, *_ = run_permute_capped(x, idx_cpu.to(DEV), E, ns, cap, fp8=True)
    _, ro, rp, _, _ = orc.capacity_permutation(idx_cpu.numpy(), E, cap, ns)
    qref, sref = orc.quant_blocks(x.float().cpu().numpy(), 1, 128)
    src = np.concatenate([rp // k, np.tile(np.arange(T), ns)])
    n = int(ro[E]) + ns * T
    np.testing.assert_array_equal(x_perm.cpu().numpy()[:n], qref[src])
    np.testing.assert_array_equal(scale.cpu().numpy()[:n], sref[src])
