"""Pins of the oracle's capacity-limited permutation and router statistics
against definitions it does not share code with: numpy's stable argsort
sliced at the cap, the drop-less permutation, scipy's softmax and entropy,
and closed forms."""
import numpy as np
import pytest
import scipy.special
import scipy.stats

from grouped_gemm_router_amd import synth


def expected_capacity(idx, E, cap, ns):
    T, k = idx.shape
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    kept_c = np.minimum(counts, cap)
    offsets = np.concatenate([[0], np.cumsum(kept_c), np.cumsum(kept_c)[-1] + T * np.arange(1, ns + 1)])
    perm, over = [], []
    f2r = np.full(T * k + ns * T, -1, dtype=np.int64)
    for e in range(E):
        fe = order[flat[order] == e]
        perm.append(fe[:cap])
        over.append(fe[cap:])
        f2r[fe[:cap]] = offsets[e] + np.arange(len(fe[:cap]))
    f2r[T * k:] = offsets[E] + np.arange(ns * T)
    return counts, offsets, np.concatenate(perm), f2r, np.concatenate(over)


@pytest.mark.parametrize("T,E,k,ns", [(300, 8, 2, 0), (257, 64, 6, 1), (64, 16, 4, 2), (1, 4, 2, 0)])
@pytest.mark.parametrize("cap", [0, 1, 7, 40])
def test_capacity_permutation_is_sliced_stable_sort(orc, T, E, k, ns, cap):
    idx = synth.random_selection(T, E, k, s=T + E + cap).numpy()
    got = orc.capacity_permutation(idx, E, cap, ns)
    exp = expected_capacity(idx, E, cap, ns)
    for g, x in zip(got, exp):
        np.testing.assert_array_equal(g, x)


def test_capacity_at_or_above_max_count_is_dropless(orc):
    idx = synth.random_selection(500, 16, 4, s=3).numpy()
    counts, offs = orc.counts_offsets(idx, 16, 1)
    perm, f2r = orc.permutation(idx, 16, offs)
    c2, o2, p2, f2, ov = orc.capacity_permutation(idx, 16, int(counts.max()), 1)
    np.testing.assert_array_equal(c2, counts)
    np.testing.assert_array_equal(o2, offs)
    np.testing.assert_array_equal(p2, perm)
    np.testing.assert_array_equal(f2[:500 * 4], f2r)
    assert len(ov) == 0


def test_capacity_zero_drops_every_routed_entry(orc):
    idx = synth.random_selection(50, 8, 2, s=9).numpy()
    c, o, p, f2r, ov = orc.capacity_permutation(idx, 8, 0, 1)
    assert (o[:9] == 0).all() and o[9] == 50 and len(p) == 0
    assert (f2r[:100] == -1).all() and (f2r[100:] == np.arange(50)).all()
    assert sorted(ov.tolist()) == list(range(100))


def test_router_stats_closed_forms(orc):
    T, E, k = 64, 16, 2
    lg = np.zeros((T, E), np.float32)           # equal logits: P = 1/E
    counts = np.full(E, T * k // E, np.int32)   # uniform load
    f, P, aux, mm, ent = orc.router_stats(lg, counts, k, 0.01)
    np.testing.assert_allclose(P, 1.0 / E, rtol=1e-14)
    np.testing.assert_allclose(f, 1.0 / E, rtol=1e-14)
    assert abs(aux - 0.01) < 1e-15           # alpha * E * E * (1/E)(1/E)
    assert mm == 1.0
    assert abs(ent - np.log2(E)) < 1e-6      # the page's +1e-8 moves it by < E 1e-8 / ln 2
    one = np.zeros(E, np.int32)
    one[5] = T * k
    _, _, _, mm1, ent1 = orc.router_stats(lg, one, k, 0.01)
    assert mm1 == E and abs(ent1) < 1e-7


def test_router_stats_against_scipy(orc):
    rng = np.random.default_rng(4)
    T, E, k = 300, 32, 4
    lg = (rng.standard_normal((T, E)) * 1.7).astype(np.float32)
    idx = synth.random_selection(T, E, k, s=5).numpy()
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    f, P, aux, mm, ent = orc.router_stats(lg, counts, k, 0.003)
    P_ref = scipy.special.softmax(lg.astype(np.float64), axis=1).mean(axis=0)
    f_ref = counts / (T * k)
    np.testing.assert_allclose(P, P_ref, rtol=1e-12)
    np.testing.assert_allclose(f, f_ref, rtol=1e-15)
    assert abs(aux - 0.003 * E * np.dot(f_ref, P_ref)) < 1e-14
    assert abs(mm - counts.max() / counts.mean()) < 1e-14
    # the page's +1e-8 inside log2 lowers each term by q log2(1 + 1e-8/q) <= 1e-8 / ln 2
    d = scipy.stats.entropy(counts / counts.sum(), base=2) - ent
    assert 0 <= d <= E * 1e-8 / np.log(2) + 1e-12
