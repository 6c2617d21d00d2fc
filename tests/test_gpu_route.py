"""GPU parity of moe_route against the oracle.

* From given fp32 logits (MOE_ROUTE_FROM_LOGITS): indices bit-exact, weights
  within 1e-6, for random logits and logits full of exact ties.
* Full scoring: logits within the fp32 accumulation bound of the oracle's
  fp64 logits (d u sum |x w|, u = 2^-24).  Selection: a token whose oracle
  ordering of its top k + 1 logits has every gap wider than twice the
  largest deviation of that token's GPU logits from the exact ones has one
  correct answer, which must be matched exactly; otherwise several answers
  are correct and the GPU's must be one of them (each selected logit within
  twice that deviation of the oracle's j-th largest).
"""
import numpy as np
import pytest
import torch

from grouped_gemm_router_amd import synth
from gpu_util import DEV, np_of

pytestmark = pytest.mark.gpu


def api():
    from grouped_gemm_router_amd import api as a
    return a


def run_from_logits(lg: np.ndarray, k: int, renorm=False):
    a = api()
    T, E = lg.shape
    logits = torch.from_numpy(lg).to(DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    flags = a.MOE_ROUTE_FROM_LOGITS | (a.MOE_ROUTE_RENORM if renorm else 0)
    ps = torch.full((a.prob_sum_blocks(T), E), float("nan"), dtype=torch.float32, device=DEV)
    a.moe_route(None, None, idx, w, logits=logits, flags=flags, prob_sums=ps)
    torch.cuda.synchronize()
    check_prob_sums(ps, lg)
    return idx.cpu().numpy(), w.cpu().numpy()


# every select path: one expert per lane (E <= 64), two, four (E <= 256,
# with 16-byte loads when E % 4 == 0 and without: E = 201), eight and
# sixteen; E = 1024 and k = 32 are the library's limits
@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (37, 8, 2), (300, 8, 2), (129, 256, 8),
                                   (64, 32, 32), (50, 1000, 32), (33, 65, 3), (45, 201, 7),
                                   (70, 400, 9), (20, 1024, 32)])
@pytest.mark.parametrize("renorm", [False, True])
def test_from_logits_random(orc, T, E, k, renorm):
    rng = np.random.default_rng(T * 1000 + E + k)
    lg = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    idx, w = run_from_logits(lg, k, renorm)
    ridx, rw = orc.topk(lg, k, renorm)
    np.testing.assert_array_equal(idx, ridx)
    np.testing.assert_allclose(w, rw, atol=1e-6, rtol=0)


@pytest.mark.parametrize("E,k", [(8, 2), (256, 8), (16, 16), (70, 5)])
def test_from_logits_exact_ties(orc, E, k):
    rng = np.random.default_rng(E + k)
    pool = np.array([-2.0, -0.0, 0.0, 0.5, 0.5, 1.25], dtype=np.float32)
    lg = rng.choice(pool, size=(200, E)).astype(np.float32)
    lg[0, :] = 0.0
    lg[1, :] = -0.0
    lg[2, ::2] = -0.0
    idx, w = run_from_logits(lg, k)
    ridx, rw = orc.topk(lg, k)
    np.testing.assert_array_equal(idx, ridx)
    np.testing.assert_allclose(w, rw, atol=1e-6, rtol=0)


def check_prob_sums(ps, lg32):
    """Per-16-token sums of the softmax probabilities against fp64 sums of the
    softmax of the same fp32 logits: each term within ~(E + 30) u relative
    (exp, the normaliser over E terms, one division), 16 more roundings of
    the positive partial sums."""
    T, E = lg32.shape
    l64 = lg32.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    nb = (T + 15) // 16
    pad = np.zeros((nb * 16, E))
    pad[:T] = p
    ref = pad.reshape(nb, 16, E).sum(axis=1)
    got = ps.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    assert (np.abs(got - ref) <= (E + 50) * 2.0 ** -24 * ref + 1e-30).all(), \
        np.abs(got / np.maximum(ref, 1e-300) - 1).max()


def check_selection(idx, lg_ref, bound, k):
    """idx (GPU) against the oracle's fp64 logits with per-token error bound."""
    T, E = lg_ref.shape
    l32 = lg_ref.astype(np.float32).astype(np.float64)
    n_ambig = 0
    for t in range(T):
        order = np.lexsort((np.arange(E), -l32[t]))
        top = order[: min(k + 1, E)]
        gaps = np.abs(np.diff(l32[t, top]))
        sel = idx[t]
        assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < E
        if gaps.size == 0 or gaps.min() > 2 * bound[t] + 1e-7:
            np.testing.assert_array_equal(sel, order[:k], err_msg="token %d" % t)
        else:
            n_ambig += 1
            np.testing.assert_allclose(lg_ref[t, sel], lg_ref[t, order[:k]],
                                       atol=2 * bound[t] + 1e-6)
    return n_ambig


@pytest.mark.parametrize("dt,T,d,E,k,bias", [
    ("f32", 256, 128, 8, 2, False),
    ("bf16", 300, 4096, 8, 2, False),
    ("bf16", 200, 4096, 8, 2, True),
    ("bf16", 96, 7168, 256, 8, False),
    ("bf16", 40, 256, 1000, 4, False),
    ("bf16", 17, 64, 3, 3, False),
    # column tail inside a K step (1000 = 15 x 64 + 40), expert tiles of
    # 128 with a ragged last one, several d-slices
    ("bf16", 130, 1000, 100, 6, True),
    # 64-expert tiles, three token tiles with a ragged tail, d-slices of
    # unequal step counts
    ("bf16", 257, 2056, 48, 4, False),
    # one-launch path for E <= 32: 16-lane segments, 25 column chunks split
    # unevenly over the four waves, ragged token tail
    ("bf16", 129, 200, 16, 4, True),
    # 32-lane segments (E = 30 leaves two idle lanes per token)
    ("bf16", 65, 512, 30, 5, False),
    # E < 8 in 8-lane segments, d = 2048 (one chunk per lane and wave)
    ("bf16", 9, 2048, 5, 2, True),
    # d % 64 == 0 stages x through LDS: one 64-column chunk (seven waves
    # idle), nine chunks over eight waves, two rounds of eight chunks per
    # wave (d = 8192) with 8-, 16- and 32-lane segments
    ("bf16", 33, 64, 8, 2, False),
    ("bf16", 50, 576, 16, 3, True),
    ("bf16", 70, 8192, 8, 2, False),
    ("bf16", 40, 8192, 32, 8, True),
    # split-K MFMA logits (d % 64 == 0): 48 experts of a 256-wide tile, three
    # token tiles with a ragged tail; two expert tiles, the second ragged
    ("bf16", 257, 2048, 48, 4, False),
    ("bf16", 200, 512, 300, 6, True),
    # one-launch fp32 path with 16- and 32-lane segments
    ("f32", 100, 64, 16, 3, True),
    ("f32", 33, 256, 20, 4, False),
])
def test_scoring_and_selection(orc, dt, T, d, E, k, bias):
    a = api()
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    x = synth.randn((T, d), 1.0, 11 + T, DEV, tdt)
    wr = synth.randn((E, d), 0.02 if d >= 1024 else 0.3, 12 + E, DEV, tdt)
    b = synth.randn((E,), 0.5, 13, DEV) if bias else None
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    ps = torch.full((a.prob_sum_blocks(T), E), float("nan"), dtype=torch.float32, device=DEV)
    a.moe_route(x, wr, idx, w, logits=logits, logit_bias=b, prob_sums=ps)
    torch.cuda.synchronize()
    check_prob_sums(ps, logits.cpu().numpy())
    lg_ref, absdot = orc.router_logits(np_of(x), np_of(wr), None if b is None else np_of(b))
    got = logits.cpu().numpy().astype(np.float64)
    # fp32 accumulation of exact products: |err| <= d * 2^-24 * sum|x w| (+ bias rounding)
    bound_el = d * 2.0 ** -24 * absdot + 1e-6 * np.abs(lg_ref)
    assert (np.abs(got - lg_ref) <= bound_el + 1e-7).all()
    dev_max = np.abs(got - lg_ref).max(axis=1)
    bound = bound_el.max(axis=1)
    gi = idx.cpu().numpy()
    # given the GPU's own fp32 logits, the selection is exact (ties to the
    # lower index) and the weights are their softmax
    ridx, rw = orc.topk(logits.cpu().numpy(), k)
    np.testing.assert_array_equal(gi, ridx)
    np.testing.assert_allclose(w.cpu().numpy(), rw, atol=1e-6, rtol=1e-5)
    n_ambig = check_selection(gi, lg_ref, dev_max, k)
    assert n_ambig <= max(2, T // 50)
    # weights: softmax of the oracle logits at the GPU's selection
    l64 = lg_ref.astype(np.float32).astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ref_w = np.take_along_axis(p, gi.astype(np.int64), axis=1)
    tol = 1e-6 + 4 * bound[:, None] * ref_w
    assert (np.abs(w.cpu().numpy() - ref_w) <= tol).all()


def test_route_is_deterministic():
    a = api()
    T, d, E, k = 512, 7168, 256, 8
    x = synth.randn((T, d), 1.0, 5, DEV, torch.bfloat16)
    wr = synth.randn((E, d), 0.02, 6, DEV, torch.bfloat16)
    outs = []
    for _ in range(2):
        lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
        idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, k), dtype=torch.float32, device=DEV)
        a.moe_route(x, wr, idx, w, logits=lg)
        outs.append((lg.cpu(), idx.cpu(), w.cpu()))
    for u, v in zip(*outs):
        assert torch.equal(u, v)


@pytest.mark.parametrize("T,d,E,k", [(300, 4096, 8, 2), (77, 1024, 32, 6), (1000, 7168, 256, 8)])
def test_renorm_without_logits_matches_logits_run(orc, T, d, E, k):
    """Both routing paths (one launch for E <= 32, split-K above): no logits
    output and renormalised weights give the same experts as a run that
    exports the logits, and weights that are the oracle's renormalised
    softmax of those logits."""
    a = api()
    x = synth.randn((T, d), 1.0, 31 + T, DEV, torch.bfloat16)
    wr = synth.randn((E, d), 0.02, 32 + E, DEV, torch.bfloat16)
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    idx1 = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w1 = torch.empty((T, k), dtype=torch.float32, device=DEV)
    a.moe_route(x, wr, idx1, w1, logits=lg)
    idx2 = torch.empty_like(idx1)
    w2 = torch.empty_like(w1)
    a.moe_route(x, wr, idx2, w2, flags=a.MOE_ROUTE_RENORM)
    torch.cuda.synchronize()
    assert torch.equal(idx1, idx2)
    ridx, rw = orc.topk(lg.cpu().numpy(), k, renorm=True)
    np.testing.assert_array_equal(idx2.cpu().numpy(), ridx)
    np.testing.assert_allclose(w2.cpu().numpy(), rw, atol=1e-6, rtol=1e-5)
