"""Pins for the oracle's histogram, offsets, permutation and row gather."""
import numpy as np
import pytest

from grouped_gemm_router_amd import synth


@pytest.mark.parametrize("T,E,k,ns", [(1, 1, 1, 0), (64, 8, 2, 0), (100, 256, 8, 1),
                                      (333, 7, 3, 2), (0, 4, 2, 1)])
def test_counts_offsets_match_bincount_cumsum(orc, T, E, k, ns):
    idx = synth.random_selection(T, E, k, s=T * 7 + E).numpy()
    counts, offsets = orc.counts_offsets(idx, E, ns)
    ref = np.bincount(idx.ravel(), minlength=E)
    np.testing.assert_array_equal(counts, ref)
    # exclusive prefix sum (cumsum - counts), then the shared segments of T rows
    np.testing.assert_array_equal(offsets[:E], np.cumsum(ref) - ref)
    assert offsets[E] == T * k == counts.sum()
    for s in range(ns):
        assert offsets[E + s + 1] - offsets[E + s] == T


def test_counts_rejects_out_of_range(orc):
    idx = np.array([[0, 4]], dtype=np.int32)
    with pytest.raises(ValueError):
        orc.counts_offsets(idx, 4)


@pytest.mark.parametrize("T,E,k", [(50, 8, 2), (257, 256, 8), (64, 3, 3), (10, 1, 1)])
def test_permutation_is_stable_sort(orc, T, E, k):
    idx = synth.random_selection(T, E, k, s=99 + T).numpy()
    counts, offsets = orc.counts_offsets(idx, E)
    perm_src, f2r = orc.permutation(idx, E, offsets)
    ref = np.argsort(idx.ravel(), kind="stable")
    np.testing.assert_array_equal(perm_src, ref)
    np.testing.assert_array_equal(f2r[perm_src], np.arange(T * k))
    # every token exactly k times, each row inside its expert's segment
    toks = perm_src // k
    assert (np.bincount(toks, minlength=T) == k).all()
    for e in range(E):
        seg = perm_src[offsets[e]:offsets[e] + counts[e]]
        assert (idx.ravel()[seg] == e).all()
        assert (np.diff(seg // k) > 0).all()  # ascending tokens, no repeats


def test_permutation_skewed_and_empty_experts(orc):
    T, E, k = 300, 16, 2
    w = np.zeros(E)
    w[[1, 3, 4]] = [10.0, 1.0, 0.5]
    w[w == 0] = 1e-9
    idx = synth.random_selection(T, E, k, s=5, weights=w).numpy()
    counts, offsets = orc.counts_offsets(idx, E)
    assert (counts == 0).sum() > 0
    perm_src, f2r = orc.permutation(idx, E, offsets)
    np.testing.assert_array_equal(perm_src, np.argsort(idx.ravel(), kind="stable"))


def test_permute_rows_copies_bytes(orc):
    rng = np.random.default_rng(2)
    T, d, E, k, ns = 40, 24, 5, 2, 1
    x = rng.integers(0, 65535, size=(T, d), dtype=np.uint16)
    idx = synth.random_selection(T, E, k, s=3).numpy()
    counts, offsets = orc.counts_offsets(idx, E, ns)
    perm_src, _ = orc.permutation(idx, E, offsets)
    rows = np.arange(T * k + ns * T)
    xp = orc.permute_rows(x, k, perm_src, rows)
    for r in range(T * k):
        np.testing.assert_array_equal(xp[r], x[perm_src[r] // k])
    np.testing.assert_array_equal(xp[T * k:], x)
