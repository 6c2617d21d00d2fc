"""Pins for the oracle's grouped GEMM (bf16/fp32 and FP8 block-scaled) and
combine, against numpy fp64 matmuls of the same operands."""
import numpy as np
import pytest
import torch

from grouped_gemm_router_amd import synth
from test_oracle_route import bf16_bits, bits_to_f64


def silu(z):
    return z / (1.0 + np.exp(-z))


def offsets_from_sizes(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("epi", [False, True])
def test_grouped_gemm_matches_per_group_matmul(orc, dt, epi):
    rng = np.random.default_rng(4)
    sizes = [0, 1, 127, 129, 3]
    G, N, K = len(sizes), 24, 40
    offsets = offsets_from_sizes(sizes)
    rows = int(offsets[-1])
    A = rng.standard_normal((rows, K)).astype(np.float32)
    B = (rng.standard_normal((G, N, K)) / np.sqrt(K)).astype(np.float32)
    B2 = (rng.standard_normal((G, N, K)) / np.sqrt(K)).astype(np.float32)
    if dt == "bf16":
        A, B, B2 = bf16_bits(A), bf16_bits(B), bf16_bits(B2)
        Af, Bf, B2f = bits_to_f64(A), bits_to_f64(B), bits_to_f64(B2)
    else:
        Af, Bf, B2f = A.astype(np.float64), B.astype(np.float64), B2.astype(np.float64)
    out = orc.gemm_rows(A, B, offsets, np.arange(rows), B2=B2, swiglu=epi)
    for g in range(G):
        a = Af[offsets[g]:offsets[g + 1]]
        ref = a @ Bf[g].T
        if epi:
            ref = silu(ref) * (a @ B2f[g].T)
        np.testing.assert_allclose(out[offsets[g]:offsets[g + 1]], ref, rtol=1e-12, atol=1e-12)


def test_single_group_is_plain_gemm(orc):
    rng = np.random.default_rng(8)
    A = rng.standard_normal((9, 16)).astype(np.float32)
    B = rng.standard_normal((1, 5, 16)).astype(np.float32)
    out = orc.gemm_rows(A, B, np.array([0, 9], np.int32), np.arange(9))
    np.testing.assert_allclose(out, A.astype(np.float64) @ B[0].T.astype(np.float64), rtol=1e-12)


def torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


@pytest.mark.parametrize("epi", [False, True])
def test_fp8_grouped_gemm_is_dequantised_product(orc, epi):
    sizes = [2, 0, 5, 1]
    G, N, K = len(sizes), 256, 384
    offsets = offsets_from_sizes(sizes)
    rows = int(offsets[-1])
    Aq = synth.random_e4m3_codes((rows, K), 1).numpy()
    As = synth.random_scales((rows, K // 128), 2).numpy()
    Bq = synth.random_e4m3_codes((G, N, K), 3).numpy()
    Bs = synth.random_scales((G, N // 128, K // 128), 4).numpy()
    B2q = synth.random_e4m3_codes((G, N, K), 5).numpy()
    B2s = synth.random_scales((G, N // 128, K // 128), 6).numpy()
    out = orc.gemm_fp8_rows(Aq, As, Bq, Bs, offsets, np.arange(rows), B2q, B2s, swiglu=epi)
    Ad = torch_decode(Aq) * np.repeat(As.astype(np.float64), 128, axis=1)
    for g in range(G):
        sB = np.repeat(np.repeat(Bs[g].astype(np.float64), 128, 0), 128, 1)
        sB2 = np.repeat(np.repeat(B2s[g].astype(np.float64), 128, 0), 128, 1)
        a = Ad[offsets[g]:offsets[g + 1]]
        ref = a @ (torch_decode(Bq[g]) * sB).T
        if epi:
            ref = silu(ref) * (a @ (torch_decode(B2q[g]) * sB2).T)
        np.testing.assert_allclose(out[offsets[g]:offsets[g + 1]], ref, rtol=1e-11, atol=1e-9)


@pytest.mark.parametrize("ns", [0, 1])
def test_combine_matches_numpy(orc, ns):
    rng = np.random.default_rng(12)
    T, E, k, d = 30, 6, 3, 20
    idx = synth.random_selection(T, E, k, s=1).numpy()
    counts, offsets = orc.counts_offsets(idx, E, ns)
    _, f2r = orc.permutation(idx, E, offsets)
    rows = T * k + ns * T
    Y = rng.standard_normal((rows, d)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    out = orc.combine(Y, f2r, w, T, k, ns)
    Yf = Y.astype(np.float64)
    ref = (w.astype(np.float64)[:, :, None] * Yf[f2r.reshape(T, k)]).sum(axis=1)
    if ns:
        ref = ref + Yf[T * k:]
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)
