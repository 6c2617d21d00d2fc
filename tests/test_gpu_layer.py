"""End-to-end parity of the MoE layer (route -> permute -> grouped GEMMs ->
combine, all through libmoe.so) against the oracle's token-by-token layer.

Routing, for every compared token:
  * the GPU logits lie within the fp32 accumulation bound of the oracle's
    fp64 logits;
  * given the GPU's own fp32 logits, the oracle's top-k returns exactly the
    GPU's indices (ties to the lower index) and weights within 1e-6;
  * against the oracle's own logits the GPU's selection is the oracle's for
    every token whose top-(k+1) logits are separated by more than twice that
    token's logit deviation, and a valid choice otherwise (several
    selections are correct for such near ties).
Outputs, for every compared token (near ties included), against the
oracle's layer evaluated at the GPU's selection with the oracle's softmax
weights of those logits: fp32 layer max |y - y_ref| <= 1e-4 max(|y_ref|,
RMS); bf16 layers <= 2e-2 RMS(y_ref); FP8 layer <= 5e-2 RMS(y_ref).

Small shapes compare every token; the five full-size workloads compare a
sample of tokens in the exact configuration the benchmark runs.
"""
import numpy as np
import pytest
import torch

from grouped_gemm_router_amd import synth
from gpu_util import DEV, assert_bf16_close, assert_f32_close, np_of, rms
from test_gpu_route import check_selection

pytestmark = pytest.mark.gpu


def build_layer(cfg, renorm=False, capacity_factor=None):
    from grouped_gemm_router_amd.layer import MoELayer
    x = synth.gen_x(cfg, DEV)
    wr = synth.gen_router(cfg, DEV)
    bias = synth.gen_bias(cfg, DEV)
    wg, wu, wd = synth.gen_experts(cfg, DEV)
    layer = MoELayer(wr, wg, wu, wd, cfg.k, n_shared=cfg.n_shared, bias=bias,
                     fp8=cfg.dtype == "fp8", renorm=renorm, capacity_factor=capacity_factor)
    return layer, x, wr, bias, (wg, wu, wd)


def oracle_layer(orc, cfg, xs, weights, groups):
    """The oracle's layer over the token rows xs (numpy, the oracle's
    convention) with the weights of the listed groups (all shared groups are
    added); its token i is row i of xs."""
    wg, wu, wd = weights
    G = cfg.G
    need = set(int(g) for g in groups) | set(range(cfg.E, G))
    lists = {n: [None] * G for n in ("g", "u", "d", "sg", "su", "sd")}
    for g in sorted(need):
        if cfg.dtype == "fp8":
            for key, wt in (("g", wg), ("u", wu), ("d", wd)):
                q, s = orc.quant_blocks(wt[g].float().cpu().numpy(), 128, 128)
                lists[key][g], lists["s" + key][g] = q, s
        else:
            lists["g"][g], lists["u"][g], lists["d"][g] = np_of(wg[g]), np_of(wu[g]), np_of(wd[g])
    mode = orc.E4M3 if cfg.dtype == "fp8" else None
    return orc.Layer(xs, cfg.E, cfg.k, cfg.n_shared, lists["g"], lists["u"], lists["d"],
                     mode=mode, sg=lists["sg"], su=lists["su"], sd=lists["sd"])


def check_routing(orc, cfg, layer, x, wr, bias, tokens, renorm=False):
    """The routing checks above; returns the GPU's selection of the tokens
    and the oracle's weights for it (softmax of the GPU's fp32 logits)."""
    _, _, lg, ad = orc.route(np_of(x)[tokens], np_of(wr), cfg.k,
                             None if bias is None else np_of(bias), renorm)
    gidx = layer.topk_idx.cpu().numpy()[tokens]
    gw = layer.topk_w.cpu().numpy()[tokens]
    glg32 = layer.logits.cpu().numpy()[tokens]
    glg = glg32.astype(np.float64)
    assert (np.abs(glg - lg) <= cfg.d * 2.0 ** -24 * ad + 1e-6 * np.abs(lg) + 1e-7).all()
    ridx, rw = orc.topk(glg32, cfg.k, renorm)
    np.testing.assert_array_equal(gidx, ridx)
    np.testing.assert_allclose(gw, rw, atol=1e-6, rtol=0)
    check_selection(gidx, lg, np.abs(glg - lg).max(axis=1), cfg.k)
    return gidx, rw


def assert_layer_close(cfg, got, ref):
    if cfg.dtype == "f32":
        assert_f32_close(got, ref)
    elif cfg.dtype == "fp8":
        err = np.abs(got - ref).max()
        assert err <= 5e-2 * rms(ref), "fp8 layer: max err %.3e vs RMS %.3e" % (err, rms(ref))
    else:
        assert_bf16_close(got, ref)


def compare_layer(orc, cfg, tokens, renorm=False):
    layer, x, wr, bias, weights = build_layer(cfg, renorm)
    out = layer(x)
    torch.cuda.synchronize()
    gidx, rw = check_routing(orc, cfg, layer, x, wr, bias, tokens, renorm)
    L = oracle_layer(orc, cfg, np_of(x)[tokens], weights, np.unique(gidx))
    ref = L.tokens(np.ascontiguousarray(gidx), rw, np.arange(len(tokens)))
    assert_layer_close(cfg, out.float().cpu().numpy()[tokens], ref)
    return layer, out


SMALL = [
    synth.CONFIGS["tiny_f32"],
    synth.scaled(synth.CONFIGS["mixtral_bf16"], name="mixtral_small", T=512, d=512, dff=1024),
    synth.scaled(synth.CONFIGS["skew_bf16"], name="skew_small", T=512, d=512, dff=1024),
    synth.scaled(synth.CONFIGS["deepseek_bf16"], name="deepseek_small", T=300, d=512, dff=256,
                 E=64, k=6),
    synth.scaled(synth.CONFIGS["deepseek_fp8"], name="fp8_small", T=300, d=512, dff=256, E=32,
                 k=4),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_layer_small_every_token(orc, cfg):
    compare_layer(orc, cfg, np.arange(cfg.T))


DEGENERATE = [
    # one token; seven tokens (a ragged 16-token routing block) with every
    # expert taking every token (k = E) and a shared expert; one expert
    synth.scaled(synth.CONFIGS["mixtral_bf16"], name="one_token", T=1, d=256, dff=512),
    synth.scaled(synth.CONFIGS["deepseek_bf16"], name="k_equals_e", T=7, d=256, dff=256, E=4,
                 k=4),
    synth.scaled(synth.CONFIGS["mixtral_bf16"], name="one_expert", T=33, d=256, dff=512, E=1,
                 k=1),
    synth.scaled(synth.CONFIGS["tiny_f32"], name="f32_one_token", T=1),
]


@pytest.mark.parametrize("cfg", DEGENERATE, ids=[c.name for c in DEGENERATE])
def test_layer_degenerate_shapes(orc, cfg):
    compare_layer(orc, cfg, np.arange(cfg.T))


def test_layer_renormalised_gate(orc):
    cfg = synth.scaled(synth.CONFIGS["mixtral_bf16"], name="renorm", T=256, d=256, dff=512)
    compare_layer(orc, cfg, np.arange(cfg.T), renorm=True)


FULL = ["mixtral_bf16", "skew_bf16", "skew_decode_bf16", "deepseek_bf16", "deepseek_fp8"]


@pytest.mark.parametrize("name", FULL)
def test_layer_full_size_sampled_tokens(orc, name):
    cfg = synth.CONFIGS[name]
    rng = np.random.default_rng(5)
    n = 8 if cfg.T > 1000 else 6
    tokens = np.unique(np.concatenate([[0, cfg.T - 1], rng.integers(0, cfg.T, n)]))
    layer, out = compare_layer(orc, cfg, tokens)
    # whole-layer invariants on every token
    counts = layer.counts.cpu().numpy()
    offs = layer.offsets.cpu().numpy()
    assert counts.sum() == cfg.T * cfg.k and offs[cfg.E] == cfg.T * cfg.k
    np.testing.assert_array_equal(offs[:cfg.E], np.cumsum(counts) - counts)
    assert torch.isfinite(out.float()).all()


def test_layer_is_deterministic():
    cfg = synth.scaled(synth.CONFIGS["deepseek_bf16"], name="det", T=512, d=1024, dff=512, E=32)
    layer, x, _, _, _ = build_layer(cfg)
    o1 = layer(x).clone()
    o2 = layer(x).clone()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("cfg_name,cf", [("skew_bf16", 0.5), ("skew_bf16", 1.25),
                                         ("deepseek_bf16", 1.0)])
def test_layer_with_capacity_factor(orc, cfg_name, cf):
    """Each expert keeps ceil(cf T k / E) rows (first in flat order); a
    dropped (token, expert) pair contributes nothing.  The oracle output is
    the token loop with the dropped pairs' weights set to zero, the drop
    pattern taken from the oracle's capacity permutation of the selection
    (whose flat_to_row must equal the GPU's exactly)."""
    base = synth.CONFIGS[cfg_name]
    if cfg_name == "skew_bf16":
        cfg = synth.scaled(base, name="cap", T=512, d=512, dff=1024)
    else:
        cfg = synth.scaled(base, name="cap_ds", T=300, d=512, dff=256, E=64, k=6)
    layer, x, wr, bias, weights = build_layer(cfg, capacity_factor=cf)
    out = layer(x)
    torch.cuda.synchronize()
    cap = layer.capacity(cfg.T)
    tokens = np.arange(cfg.T)
    gidx, rw = check_routing(orc, cfg, layer, x, wr, bias, tokens)
    _, _, _, f2r, ov = orc.capacity_permutation(gidx, cfg.E, cap, cfg.n_shared)
    kept = (f2r[: cfg.T * cfg.k] >= 0).reshape(cfg.T, cfg.k)
    n_drop = int(layer.n_overflow.cpu()[0])
    assert n_drop == len(ov)
    if cf < 1.0:
        assert n_drop > 0
    np.testing.assert_array_equal(layer.flat_to_row.cpu().numpy(), f2r)
    # oracle layer with the dropped pairs zero-weighted
    L = oracle_layer(orc, cfg, np_of(x), weights, np.unique(gidx))
    ref = L.tokens(gidx, np.where(kept, rw, 0.0), tokens)
    ref_all = L.tokens(gidx, rw, tokens)          # the drop-less layer
    got = out.float().cpu().numpy()
    # Dropping zeroes terms, it does not change the arithmetic of the kept
    # ones: the error scale is that of the drop-less layer, so the bf16 bar
    # (2e-2 x RMS) is taken on the drop-less reference output (the capped
    # output's own RMS shrinks with every dropped pair).  The premise,
    # token by token: a token that dropped nothing has exactly the drop-less
    # reference and stays within the drop-less bar; a token that dropped
    # pairs is within the same bar.
    scale = rms(ref_all)
    dropped = ~kept.all(axis=1)
    np.testing.assert_array_equal(ref[~dropped], ref_all[~dropped])
    err = np.abs(got - ref).max(axis=1)
    assert err[~dropped].max() <= 2e-2 * scale, \
        "tokens without drops: max err %.3e vs 2e-2 x RMS %.3e" % (err[~dropped].max(), scale)
    if dropped.any():
        assert err[dropped].max() <= 2e-2 * scale, \
            "tokens with drops: max err %.3e vs 2e-2 x RMS %.3e" % (err[dropped].max(), scale)


@pytest.mark.parametrize("name", ["tiny_f32", "deepseek_small"])
def test_graph_replays_match_eager(name):
    """The five library calls captured in a HIP graph: every replay, with
    the program's own eager work and synchronisations in between (another
    eager forward into a second buffer, a torch op on x's copy), gives
    bit-identical outputs to the eager forward."""
    cfg = synth.CONFIGS[name] if name in synth.CONFIGS else \
        next(c for c in SMALL if c.name == name)
    layer, x, *_ = build_layer(cfg)
    eager = layer(x).clone()
    out = torch.empty_like(eager)
    g = layer.capture(x, out)
    torch.cuda.synchronize()
    bits = torch.int32 if eager.dtype == torch.float32 else torch.int16
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(bits), eager.view(bits)), "replay %d differs" % rep
        other = layer(x)                      # eager work between replays
        y = (x.float() * 2.0).sum()
        torch.cuda.synchronize()
        assert torch.equal(other.view(bits), eager.view(bits)) and torch.isfinite(y)


def test_forward_keeps_and_refreshes_its_marshalled_calls():
    """forward() keeps its five marshalled calls while x, out, the stream and
    the buffers stay the same, and builds new ones when any changes: switching
    between inputs, output buffers and token counts must give the same bits as
    a fresh layer does for each input."""
    from grouped_gemm_router_amd.layer import MoELayer
    cfg = next(c for c in SMALL if c.name == "mixtral_small")
    layer, x, wr, bias, (wg, wu, wd) = build_layer(cfg)
    x2 = synth.randn(tuple(x.shape), 1.0, 4242, DEV, x.dtype)
    x3 = x2[: cfg.T // 2 + 5].contiguous()          # another token count: new buffers

    def fresh(inp):
        f = MoELayer(wr, wg, wu, wd, cfg.k, n_shared=cfg.n_shared, bias=bias)
        return f(inp).clone()
    want = {id(t): fresh(t) for t in (x, x2, x3)}
    bits = torch.int16
    buf = torch.empty_like(want[id(x)])
    for t in (x, x2, x, x3, x2, x, x3):
        got = layer(t).clone()
        assert torch.equal(got.view(bits), want[id(t)].view(bits))
        if t.shape[0] == cfg.T:                     # the same call into a caller's buffer
            layer(t, out=buf)
            torch.cuda.synchronize()
            assert torch.equal(buf.view(bits), want[id(t)].view(bits))
