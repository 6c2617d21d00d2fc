"""GPU parity of moe_router_stats against the oracle's fp64 statistics.

The statistics take their mean gate probabilities from moe_route's
per-16-token probability sums (here produced from given logits with
MOE_ROUTE_FROM_LOGITS, or by the layer's own route), and the counts from the
permutation.

Tolerances from the fp32 arithmetic (u = 2^-24): each softmax term errs by
at most about (E + 30) u relative (max-subtracted exp of an argument below
~20 in magnitude, a normaliser summed over E terms, one division), and P
adds at most 64 + nblk more roundings of sums of positive terms (16 terms
per block, the blocks, the division by T): |P - P_ref| <= (E + 100 + nblk)
u P_ref, nblk = ceil(T / 16).  f is one division (2 u).  aux adds E + 3
roundings of positive terms.  max/mean is two roundings.  The entropy is a
sum of E terms q log2 q, each within a few ulp of its (at most ~log2(T k))
magnitude: |H - H_ref| <= 8 (E + 8) u (1 + log2(T k)).
"""
import numpy as np
import pytest
import torch

from grouped_gemm_router_amd import synth
from gpu_util import DEV

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def api():
    from grouped_gemm_router_amd import api as a
    return a


def gpu_stats(logits, counts, k, alpha):
    """moe_route from the given logits (probability sums only), then
    moe_router_stats."""
    a = api()
    T, E = logits.shape
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    ps = torch.full((a.prob_sum_blocks(T), E), float("nan"), dtype=torch.float32, device=DEV)
    a.moe_route(None, None, idx, w, logits=logits, flags=a.MOE_ROUTE_FROM_LOGITS, prob_sums=ps)
    f = torch.empty((E,), dtype=torch.float32, device=DEV)
    P = torch.empty_like(f)
    summ = torch.empty((3,), dtype=torch.float32, device=DEV)
    a.moe_router_stats(ps, counts, T, k, alpha, f, P, summ)
    torch.cuda.synchronize()
    return f.cpu().numpy(), P.cpu().numpy(), summ.cpu().numpy()


def check(orc, lg32, counts, k, alpha):
    T, E = lg32.shape
    f, P, s = gpu_stats(torch.from_numpy(lg32).to(DEV), torch.from_numpy(counts).to(DEV), k,
                        alpha)
    rf, rP, raux, rmm, rent = orc.router_stats(lg32, counts, k, alpha)
    nblk = (T + 15) // 16
    tolP = (E + 100 + nblk) * U
    assert (np.abs(P - rP) <= tolP * rP + 1e-30).all(), np.abs(P / rP - 1).max()
    np.testing.assert_allclose(f, rf, rtol=2 * U, atol=0)
    assert abs(s[0] - raux) <= (tolP + (E + 3) * U) * abs(raux) + 1e-30
    assert abs(s[1] - rmm) <= 4 * U * rmm
    assert abs(s[2] - rent) <= 8 * (E + 8) * U * (1 + np.log2(T * k))
    return s


# E covers every code path: segments of 8/16/32/64 lanes (E <= 64, also
# non-powers of two), several token slices (E < 256), one slice with idle
# threads (128 < E < 256), and experts looped over (E > 256)
@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (300, 32, 4), (4096, 8, 2), (777, 256, 8),
                                   (64, 1000, 16), (130, 3, 2), (200, 12, 3), (500, 50, 4),
                                   (129, 200, 8), (1000, 64, 6)])
def test_router_stats_random(orc, T, E, k):
    rng = np.random.default_rng(T + E)
    lg = (rng.standard_normal((T, E)) * 1.5).astype(np.float32)
    idx = synth.random_selection(T, E, k, s=T * 3 + E).numpy()
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    check(orc, lg, counts, k, 0.01)


def test_router_stats_closed_forms(orc):
    T, E, k = 128, 16, 2
    lg = np.zeros((T, E), np.float32)
    counts = np.full(E, T * k // E, np.int32)
    s = check(orc, lg, counts, k, 0.02)
    assert abs(s[0] - 0.02) < 1e-7 and s[1] == 1.0
    counts = np.zeros(E, np.int32)
    counts[3] = T * k
    s = check(orc, lg, counts, k, 0.02)
    assert s[1] == E and abs(s[2]) < 1e-6


@pytest.mark.parametrize("name", ["mixtral_bf16", "skew_bf16", "deepseek_bf16"])
def test_router_stats_of_the_layer(orc, name):
    """The statistics of a full-size routing decision, from the probability
    sums the layer's route wrote and its counts, against the oracle on the
    layer's logits; the skewed workload must show its imbalance."""
    from test_gpu_layer import build_layer
    cfg = synth.CONFIGS[name]
    layer, x, *_ = build_layer(cfg)
    layer(x)
    st = layer.router_stats(alpha=0.01)
    torch.cuda.synchronize()
    lg = layer.logits.cpu().numpy()
    counts = layer.counts.cpu().numpy()
    rf, rP, raux, rmm, rent = orc.router_stats(lg, counts, cfg.k, 0.01)
    T, E = lg.shape
    tolP = (E + 100 + (T + 15) // 16) * U
    P = st["P"].cpu().numpy()
    assert (np.abs(P - rP) <= tolP * rP + 1e-30).all(), np.abs(P / rP - 1).max()
    np.testing.assert_allclose(st["f"].cpu().numpy(), rf, rtol=2 * U, atol=0)
    assert abs(float(st["aux_loss"]) - raux) <= (tolP + (E + 3) * U) * abs(raux)
    s = [float(st["aux_loss"]), float(st["max_over_mean"]), float(st["entropy_bits"])]
    assert abs(s[1] - rmm) <= 4 * U * rmm
    assert abs(s[2] - rent) <= 8 * (E + 8) * U * (1 + np.log2(T * cfg.k))
    if name == "skew_bf16":
        assert s[1] > 2.0
    else:
        assert s[1] < 1.5
