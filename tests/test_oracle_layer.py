"""Pins for the oracle's whole-layer, token-by-token computation.

* against a dense all-experts-masked brute force in numpy (every expert run on
  every token, masked by the selection and weighted by the probabilities);
* against degenerate cases with a closed form (one expert = dense SwiGLU FFN;
  identical experts = sum of weights times one FFN);
* against a hand-worked two-expert top-1 batch of four tokens (the debugging
  recipe of the "Dense GEMM to TP MoE" page, §4.3);
* FP8 mode against numpy with quantisation done by torch's float8 cast;
* and the routing invariants: counts sum to T*k, offsets are the exclusive
  prefix sum, every token appears k times, weights are the selected softmax
  probabilities.
"""
import math

import numpy as np
import pytest
import torch

from test_oracle_route import bf16_bits, bits_to_f64


def silu(z):
    return z / (1.0 + np.exp(-z))


def make_layer(rng, T, d, dff, E, k, ns, dt="f32", skew=False):
    x = rng.standard_normal((T, d)).astype(np.float32)
    wr = (rng.standard_normal((E, d)) * 0.5).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.3).astype(np.float32) if skew else None
    G = E + ns
    wg = (rng.standard_normal((G, dff, d)) / np.sqrt(d)).astype(np.float32)
    wu = (rng.standard_normal((G, dff, d)) / np.sqrt(d)).astype(np.float32)
    wd = (rng.standard_normal((G, d, dff)) / np.sqrt(dff)).astype(np.float32)
    if dt == "bf16":
        x, wr, wg, wu, wd = (bf16_bits(a) for a in (x, wr, wg, wu, wd))
    return x, wr, bias, wg, wu, wd


def as_f64(a):
    return bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def dense_masked(x, wr, bias, wg, wu, wd, k, ns):
    X = as_f64(x)
    lg = X @ as_f64(wr).T
    if bias is not None:
        lg = lg + bias.astype(np.float64)
    l32 = lg.astype(np.float32)
    T, E = l32.shape
    mask = np.zeros((T, E))
    for t in range(T):
        order = np.lexsort((np.arange(E), -l32[t].astype(np.float64)))
        mask[t, order[:k]] = 1.0
    l64 = l32.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    G = E + ns
    Y_all = np.stack([(silu(X @ as_f64(wg[g]).T) * (X @ as_f64(wu[g]).T)) @ as_f64(wd[g]).T
                      for g in range(G)])
    y = np.einsum("te,etc->tc", mask * p, Y_all[:E])
    for s in range(ns):
        y = y + Y_all[E + s]
    return y, mask, p


def oracle_layer(orc, x, wr, bias, wg, wu, wd, k, ns, tok=None):
    E = wr.shape[0]
    idx, w, lg, _ = orc.route(x, wr, k, bias)
    L = orc.Layer(x, E, k, ns, list(wg), list(wu), list(wd))
    if tok is None:
        tok = np.arange(x.shape[0])
    return L.tokens(idx, w, tok), idx, w


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("E,k,ns,skew", [(8, 2, 0, False), (6, 3, 1, True), (4, 4, 2, False),
                                         (1, 1, 0, False)])
def test_layer_matches_dense_masked_brute_force(orc, dt, E, k, ns, skew):
    rng = np.random.default_rng(E * 10 + k)
    x, wr, bias, wg, wu, wd = make_layer(rng, 23, 16, 12, E, k, ns, dt, skew)
    out, idx, w = oracle_layer(orc, x, wr, bias, wg, wu, wd, k, ns)
    ref, mask, p = dense_masked(x, wr, bias, wg, wu, wd, k, ns)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # routing invariants
    counts, offsets = orc.counts_offsets(idx, E, ns)
    assert counts.sum() == x.shape[0] * k and offsets[E] == x.shape[0] * k
    np.testing.assert_array_equal(offsets[:E], np.cumsum(counts) - counts)
    np.testing.assert_array_equal(mask.sum(axis=1), k)
    for t in range(x.shape[0]):
        assert mask[t, idx[t]].all()
        np.testing.assert_allclose(w[t], p[t, idx[t]], rtol=1e-14)
    perm_src, _ = orc.permutation(idx, E, offsets)
    assert (np.bincount(perm_src // k, minlength=x.shape[0]) == k).all()


def test_subset_of_tokens_matches_full_run(orc):
    rng = np.random.default_rng(77)
    x, wr, bias, wg, wu, wd = make_layer(rng, 40, 16, 8, 5, 2, 1)
    full, idx, w = oracle_layer(orc, x, wr, bias, wg, wu, wd, 2, 1)
    tok = np.array([39, 0, 17])
    part, _, _ = oracle_layer(orc, x, wr, bias, wg, wu, wd, 2, 1, tok=tok)
    np.testing.assert_array_equal(part, full[tok])


def test_single_expert_is_dense_swiglu(orc):
    rng = np.random.default_rng(21)
    x, wr, bias, wg, wu, wd = make_layer(rng, 11, 8, 6, 1, 1, 0)
    out, idx, w = oracle_layer(orc, x, wr, bias, wg, wu, wd, 1, 0)
    assert (idx == 0).all() and (w == 1.0).all()
    X = x.astype(np.float64)
    ref = (silu(X @ wg[0].T.astype(np.float64)) * (X @ wu[0].T.astype(np.float64))) \
        @ wd[0].T.astype(np.float64)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_identical_experts_scale_by_weight_sum(orc):
    rng = np.random.default_rng(22)
    x, wr, bias, wg, wu, wd = make_layer(rng, 9, 8, 6, 4, 3, 0)
    wg[:] = wg[0]
    wu[:] = wu[0]
    wd[:] = wd[0]
    out, idx, w = oracle_layer(orc, x, wr, bias, wg, wu, wd, 3, 0)
    X = x.astype(np.float64)
    ffn = (silu(X @ wg[0].T.astype(np.float64)) * (X @ wu[0].T.astype(np.float64))) \
        @ wd[0].T.astype(np.float64)
    np.testing.assert_allclose(out, w.sum(axis=1, keepdims=True) * ffn, rtol=1e-12, atol=1e-13)


def test_hand_worked_two_experts_top1(orc):
    """Two experts, top-1, four tokens, d = 2, d_ff = 1, worked by hand.

    Router W_r = I, so the logits are the tokens themselves.
    Expert 0: g = x0 + x1, u = 2 x0, out = h * [1, -1].
    Expert 1: g = x1,      u = x0 + x1, out = h * [0.5, 0.5].
    """
    x = np.array([[1, 0], [0, 1], [2, -1], [0, 0]], dtype=np.float32)
    wr = np.eye(2, dtype=np.float32)
    wg = np.array([[[1, 1]], [[0, 1]]], dtype=np.float32)
    wu = np.array([[[2, 0]], [[1, 1]]], dtype=np.float32)
    wd = np.array([[[1], [-1]], [[0.5], [0.5]]], dtype=np.float32)
    out, idx, w = oracle_layer(orc, x, wr, None, wg, wu, wd, 1, 0)
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))  # noqa: E731
    silu1 = 1.0 * sig(1.0)
    # token 0: logits (1, 0) -> expert 0, p = sig(1); g = 1, u = 2
    # token 1: logits (0, 1) -> expert 1, p = sig(1); g = 1, u = 1
    # token 2: logits (2, -1) -> expert 0, p = sig(3); g = 1, u = 4
    # token 3: logits (0, 0) tie -> expert 0, p = 1/2; g = 0 -> h = 0
    assert list(idx[:, 0]) == [0, 1, 0, 0]
    np.testing.assert_allclose(w[:, 0], [sig(1.0), sig(1.0), sig(3.0), 0.5], rtol=1e-15)
    expect = np.array([
        [sig(1.0) * 2 * silu1, -sig(1.0) * 2 * silu1],
        [sig(1.0) * 0.5 * silu1, sig(1.0) * 0.5 * silu1],
        [sig(3.0) * 4 * silu1, -sig(3.0) * 4 * silu1],
        [0.0, 0.0],
    ])
    np.testing.assert_allclose(out, expect, rtol=1e-14, atol=1e-15)
    # renormalised top-1 gives the expert output itself
    idx_r, w_r, _, _ = orc.route(x, wr, 1, None, renorm=True)
    assert (w_r == 1.0).all()


# ----------------------------------------------------------------------------
# FP8 mode
# ----------------------------------------------------------------------------

def torch_quant(v, br, bc):
    """Block quantisation written with torch's float8 cast (the pin)."""
    v = np.asarray(v, dtype=np.float32)
    R, C = v.shape
    q = np.empty((R, C), dtype=np.uint8)
    s = np.empty((R // br, C // bc), dtype=np.float32)
    for rb in range(R // br):
        for cb in range(C // bc):
            blk = v[rb * br:(rb + 1) * br, cb * bc:(cb + 1) * bc]
            amax = np.float32(np.abs(blk).max())
            sc = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
            s[rb, cb] = sc
            quot = torch.from_numpy((blk / sc).astype(np.float32))
            q[rb * br:(rb + 1) * br, cb * bc:(cb + 1) * bc] = \
                quot.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, s


def deq(q, s, br, bc):
    vals = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn)
    vals = vals.to(torch.float32).numpy().astype(np.float64)
    return vals * np.repeat(np.repeat(s.astype(np.float64), br, 0), bc, 1)


@pytest.mark.parametrize("x_dt", ["f32", "bf16"])
def test_fp8_layer_matches_torch_quantised_reference(orc, x_dt):
    rng = np.random.default_rng(31)
    T, d, dff, E, k, ns = 6, 256, 384, 3, 2, 1
    G = E + ns
    x, wr, bias, wg, wu, wd = make_layer(rng, T, d, dff, E, k, ns, "f32")
    if x_dt == "bf16":
        x, wr = bf16_bits(x), bf16_bits(wr)
    idx, w, _, _ = orc.route(x, wr, k, None)
    # the oracle quantises the fp32 weights itself
    qg = [orc.quant_blocks(wg[g], 128, 128) for g in range(G)]
    qu = [orc.quant_blocks(wu[g], 128, 128) for g in range(G)]
    qd = [orc.quant_blocks(wd[g], 128, 128) for g in range(G)]
    L = orc.Layer(x, E, k, ns, [a[0] for a in qg], [a[0] for a in qu], [a[0] for a in qd],
                  mode=orc.E4M3, sg=[a[1] for a in qg], su=[a[1] for a in qu],
                  sd=[a[1] for a in qd])
    out = L.tokens(idx, w, np.arange(T))
    # reference with torch casts
    X32 = as_f64(x).astype(np.float32)
    Wg = [deq(*torch_quant(wg[g], 128, 128), 128, 128) for g in range(G)]
    Wu = [deq(*torch_quant(wu[g], 128, 128), 128, 128) for g in range(G)]
    Wd = [deq(*torch_quant(wd[g], 128, 128), 128, 128) for g in range(G)]
    ref = np.zeros((T, d))
    for t in range(T):
        xh = deq(*torch_quant(X32[t:t + 1], 1, 128), 1, 128)[0]

        def ffn(g):
            h = silu(Wg[g] @ xh) * (Wu[g] @ xh)
            hh = deq(*torch_quant(h.astype(np.float32)[None, :], 1, 128), 1, 128)[0]
            return Wd[g] @ hh
        for j in range(k):
            ref[t] += w[t, j] * ffn(idx[t, j])
        for s in range(ns):
            ref[t] += ffn(E + s)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-11)


def test_bf16_expert_outputs_cannot_meet_the_bf16_bar(orc):
    """Why the bf16 layers keep the expert outputs Y in fp32 until the
    combine.  On the small Mixtral-shape layer of the GPU layer tests
    (T 512, d 512, d_ff 1024, 8 experts top-2, the synthetic recipe), the
    roundings alone -- no GEMM error at all -- cost, against the fp64 layer:
      * Y rounded to bf16, combined in fp32 in j order, out rounded to bf16:
        more than the 2e-2 x RMS bar;
      * Y kept in fp32, the same combine and final rounding: well inside it.
    The outputs are heavy-tailed (max |y| ~ 6 RMS), and one bf16 rounding of
    an output near 6 RMS can already cost up to 2^-8 x 6 RMS ~ 0.023 RMS.
    Rounding by torch's float32 -> bfloat16 cast (round to nearest even)."""
    from grouped_gemm_router_amd import synth
    cfg = synth.scaled(synth.CONFIGS["mixtral_bf16"], name="mixtral_small", T=512, d=512,
                       dff=1024)

    def bits(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    def to_bf16(a):
        return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()

    x, wr = synth.gen_x(cfg, "cpu"), synth.gen_router(cfg, "cpu")
    wg, wu, wd = synth.gen_experts(cfg, "cpu")
    xs = bits(x)
    idx, w, _, _ = orc.route(xs, bits(wr), cfg.k)
    L = orc.Layer(xs, cfg.E, cfg.k, 0, [bits(a) for a in wg], [bits(a) for a in wu],
                  [bits(a) for a in wd])
    tok = np.arange(cfg.T)
    Y = []   # each selected expert's output for every token, fp64
    for j in range(cfg.k):
        unit = np.zeros_like(w)
        unit[:, j] = 1.0
        Y.append(L.tokens(idx, unit, tok))
    y = sum(w[:, j:j + 1] * Y[j] for j in range(cfg.k))
    np.testing.assert_allclose(y, L.tokens(idx, w, tok), rtol=1e-12, atol=1e-12)
    scale = np.sqrt(np.mean(y * y))

    def combine(Ys):
        acc = np.zeros(y.shape, np.float32)
        for j in range(cfg.k):
            acc = np.float32(acc + w[:, j:j + 1].astype(np.float32) * Ys[j])
        return to_bf16(acc).astype(np.float64)

    err_f32 = np.abs(combine([np.float32(v) for v in Y]) - y).max() / scale
    err_bf16 = np.abs(combine([to_bf16(v) for v in Y]) - y).max() / scale
    assert np.abs(y).max() / scale > 5.0
    assert err_bf16 > 2e-2, err_bf16
    assert err_f32 < 0.6 * 2e-2, err_f32
