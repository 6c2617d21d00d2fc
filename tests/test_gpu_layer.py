"""End-to-end parity of the MoE layer (route -> permute -> grouped GEMMs ->
combine, all through libmoe.so) against the oracle's token-by-token layer.

Routing: the GPU logits must lie within the fp32 accumulation bound of the
oracle's fp64 logits; the oracle selects from its own logits rounded to
fp32; the GPU's selection must equal it for every token whose top-(k+1)
logits are separated by more than twice the largest deviation of that
token's GPU logits, and be a valid choice otherwise (those few tokens are
then left out of the output comparison -- several selections are correct
there).
Outputs: fp32 layer max |y - y_ref| <= 1e-4 max(|y_ref|, RMS); bf16 layers
<= 2e-2 RMS(y_ref); FP8 layer <= 5e-2 RMS(y_ref).

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


def oracle_layer_for(orc, cfg, x, wr, bias, weights, tokens, renorm=False):
    """Oracle routing + outputs for the listed tokens (needed groups only)."""
    wg, wu, wd = weights
    xs = np_of(x)
    idx, w, lg, ad = orc.route(xs[tokens], np_of(wr), cfg.k,
                               None if bias is None else np_of(bias), renorm)
    G = cfg.G
    need = set(np.unique(idx).tolist()) | set(range(cfg.E, G))
    lists = {n: [None] * G for n in ("g", "u", "d", "sg", "su", "sd")}
    for g in sorted(need):
        if cfg.dtype == "fp8":
            for key, wt in (("g", wg), ("u", wu), ("d", wd)):
                q, s = orc.quant_blocks(wt[g].float().cpu().numpy(), 128, 128)
                lists[key][g], lists["s" + key][g] = q, s
        else:
            lists["g"][g], lists["u"][g], lists["d"][g] = np_of(wg[g]), np_of(wu[g]), np_of(wd[g])
    mode = orc.E4M3 if cfg.dtype == "fp8" else None
    L = orc.Layer(xs[tokens], cfg.E, cfg.k, cfg.n_shared, lists["g"], lists["u"], lists["d"],
                  mode=mode, sg=lists["sg"], su=lists["su"], sd=lists["sd"])
    out = L.tokens(idx, w, np.arange(len(tokens)))
    return out, idx, w, lg, ad


def compare_layer(orc, cfg, tokens, renorm=False):
    layer, x, wr, bias, weights = build_layer(cfg, renorm)
    out = layer(x)
    torch.cuda.synchronize()
    ref, ridx, rw, lg, ad = oracle_layer_for(orc, cfg, x, wr, bias, weights, tokens, renorm)
    gidx = layer.topk_idx.cpu().numpy()[tokens]
    glg = layer.logits.cpu().numpy().astype(np.float64)[tokens]
    assert (np.abs(glg - lg) <= cfg.d * 2.0 ** -24 * ad + 1e-6 * np.abs(lg) + 1e-7).all()
    check_selection(gidx, lg, np.abs(glg - lg).max(axis=1), cfg.k)
    same = (gidx == ridx).all(axis=1)
    assert same.mean() >= 0.9, "routing differs on %d of %d tokens" % ((~same).sum(), len(same))
    got = out.float().cpu().numpy()[tokens][same]
    ref = ref[same]
    if cfg.dtype == "f32":
        assert_f32_close(got, ref)
    elif cfg.dtype == "fp8":
        err = np.abs(got - ref).max()
        assert err <= 5e-2 * rms(ref), "fp8 layer: max err %.3e vs RMS %.3e" % (err, rms(ref))
    else:
        assert_bf16_close(got, ref)
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
    gidx = layer.topk_idx.cpu().numpy()
    tokens = np.arange(cfg.T)
    ref_all, ridx, rw, lg, _ = oracle_layer_for(orc, cfg, x, wr, bias, weights, tokens)
    same = (gidx == ridx).all(axis=1)
    assert same.mean() >= 0.9
    _, _, _, f2r, ov = orc.capacity_permutation(gidx, cfg.E, cap, cfg.n_shared)
    kept = (f2r[: cfg.T * cfg.k] >= 0).reshape(cfg.T, cfg.k)
    n_drop = int(layer.n_overflow.cpu()[0])
    assert n_drop == len(ov)
    if cf < 1.0:
        assert n_drop > 0
    np.testing.assert_array_equal(layer.flat_to_row.cpu().numpy(), f2r)
    # oracle layer with the dropped pairs zero-weighted
    wg, wu, wd = weights
    G = cfg.G
    need = set(np.unique(gidx).tolist()) | set(range(cfg.E, G))
    lists = {n: [None] * G for n in ("g", "u", "d")}
    for g in sorted(need):
        lists["g"][g], lists["u"][g], lists["d"][g] = np_of(wg[g]), np_of(wu[g]), np_of(wd[g])
    L = orc.Layer(np_of(x), cfg.E, cfg.k, cfg.n_shared, lists["g"], lists["u"], lists["d"])
    ref = L.tokens(gidx, np.where(kept, rw, 0.0), tokens)
    got = out.float().cpu().numpy()
    # Dropping zeroes terms, it does not change the arithmetic of the kept
    # ones: the error scale is that of the drop-less layer, so the bf16 bar
    # (2e-2 x RMS) is taken on the drop-less reference output (the capped
    # output's own RMS shrinks with every dropped pair).
    scale = rms(L.tokens(gidx, rw, tokens)[same])
    err = np.abs(got[same] - ref[same]).max()
    assert err <= 2e-2 * scale, "capped layer: max err %.3e vs 2e-2 x RMS %.3e" % (err, scale)
