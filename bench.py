"""Benchmark: one step = one MoE expert-layer forward (route -> permute ->
grouped GEMM gate/up + SwiGLU -> grouped GEMM down -> combine) through
libmoe.so on one MI355X, over seeded synthetic inputs already resident in
HBM.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]
                    [--no-configs] [--no-extras]

Headline workload: the Mixtral-shape bf16 layer (T=4096, d=4096, E=8, top-2,
SwiGLU d_ff=14336).  `value` is layer tokens/s over K timed steps (HIP events
around the whole loop, nothing else recorded inside it), after W warm-up
steps.  Per-kernel times come from a pass of K steps before those, with HIP
events on the launch stream around every call.  The grouped-GEMM TFLOP/s and fraction of the bf16 MFMA
peak ride along, and `configs` repeats the measurement (fewer steps) for the
other workloads, each also as HIP-graph replays of the five calls
(`ms_per_step_graph`: the launch-bound workloads are set by the host-side
cost of five calls, which a replay removes).  HBM fractions divide the
algorithmic bytes of each step
(bf16 expert outputs Y, as the method stores them) by the kernel time; the
bf16 layers keep Y in fp32, whose extra bytes are reported next to them as
`impl_bytes` / `hbm_frac_impl_bytes`.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "grouped-GEMM TFLOP/s (% MFMA peak) + MoE-layer tokens/s per config"
PEAK = {"bf16": 2516.6, "f32": 157.3, "fp8": 5033.2}  # dense MFMA TFLOP/s, MI355X
HBM_PEAK_GBS = 8000.0
STEP_NAMES = ["route", "permute", "gemm_gate_up", "gemm_down", "combine"]
# the workloads of the `configs` block, in this order
CONFIG_ORDER = ["tiny_f32", "mixtral_bf16", "skew_bf16", "skew_decode_bf16", "deepseek_bf16",
                "deepseek_fp8"]



def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="mixtral_bf16")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-configs", action="store_true",
                   help="measure only --config (no `configs` block)")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the routing variants timed outside the layer step")
    p.add_argument("--config-steps", type=int, default=10,
                   help="timed steps of each workload of the `configs` block")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (counter calibration)")
    return p.parse_args()


def step_bytes_flops(cfg, counts, logits_exported=False):
    """Per step: (algorithmic bytes, implementation bytes, flops) of one
    launch.  Algorithmic bytes count every input once, every output once and
    each active expert's weights once, with the method's own storage types
    (bf16 H and Y; E4M3 + fp32 scales in the FP8 layer); the bf16 copy of the
    shared expert's rows is not algorithmic (the rows are x itself).
    Implementation bytes differ where this implementation moves more: the
    bf16 layers store Y in fp32, and the permutation writes the shared rows."""
    es = 4 if cfg.dtype == "f32" else 2
    T, d, E, k, dff, ns = cfg.T, cfg.d, cfg.E, cfg.k, cfg.dff, cfg.n_shared
    rows = cfg.rows
    routed = T * k
    active = int((counts > 0).sum()) + ns
    fp8 = cfg.dtype == "fp8"
    w_es = 1 if fp8 else es
    act_es = 1 if fp8 else es
    maps = T * k * 4 * 4  # topk ids read, perm_src / flat_to_row written, ranks
    out = {}
    rb = T * d * es + E * d * es + T * k * 8 + (T * E * 4 if logits_exported else 0)
    out["route"] = (rb, rb, 2.0 * T * E * d)
    perm_rows = rows if fp8 else routed  # shared rows: quantised (FP8) or x itself
    pb = T * d * es + perm_rows * d * act_es + maps + (rows * (d // 128) * 4 if fp8 else 0)
    out["permute"] = (pb, T * d * es + rows * d * act_es + maps
                      + (rows * (d // 128) * 4 if fp8 else 0), 0.0)
    wsc = (active * 2 * (dff // 128) * (d // 128) * 4) if fp8 else 0
    xsc = rows * (d // 128) * 4 if fp8 else 0     # the activations' 1 x 128 scales
    hsc = rows * (dff // 128) * 4 if fp8 else 0
    gb = rows * d * act_es + xsc + active * 2 * dff * d * w_es + wsc + rows * dff * act_es + hsc
    out["gemm_gate_up"] = (gb, gb, 2.0 * rows * d * 2 * dff)
    y_alg = es                       # Y as the method stores it (bf16; fp32 layer: fp32)
    y_impl = es if fp8 or es == 4 else 4   # the bf16 layers keep Y in fp32
    db = rows * dff * act_es + hsc + active * d * dff * w_es + wsc // 2
    out["gemm_down"] = (db + rows * d * y_alg, db + rows * d * y_impl, 2.0 * rows * dff * d)
    cb = T * d * es + T * k * 4 + (T * k + ns * T) * 4  # out, gate weights, flat_to_row
    out["combine"] = (rows * d * y_alg + cb, rows * d * y_impl + cb, 0.0)
    return out


def load_traffic(kernel, cfg_name):
    """Counter-measured HBM bytes per launch of a kernel (FETCH_SIZE +
    WRITE_SIZE, scaled by a plain copy), if taken on the current source."""
    from grouped_gemm_router_amd.profiling import source_hash
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, cfg_name))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def timed(fn, reps, stream):
    """Average ms of fn over reps launches, HIP events on the launch stream."""
    import torch
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def extras(cfg, layer, x, reps, stream):
    """The routing variants outside the layer step, timed on their own:
    the router statistics of this routing decision, and the permutation with
    a capacity factor of 1.0 (ceil(T k / E) rows per expert)."""
    import torch
    from grouped_gemm_router_amd import api
    T, E, k, d = cfg.T, cfg.E, cfg.k, cfg.d
    dev = x.device
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    ps = torch.empty((api.prob_sum_blocks(T), E), dtype=torch.float32, device=dev)
    api.moe_route(x, layer.w_router, idx, w, logit_bias=layer.bias, prob_sums=ps)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    f = torch.empty((E,), dtype=torch.float32, device=dev)
    P = torch.empty_like(f)
    summ = torch.empty((3,), dtype=torch.float32, device=dev)
    out = {}
    # permutation under a capacity factor of 1.0
    cap = -(-T * k // E)
    ov = torch.empty((T * k,), dtype=torch.int32, device=dev)
    nov = torch.empty((1,), dtype=torch.int32, device=dev)
    run = lambda: api.moe_permute_capped(x, idx, E, layer.n_shared, cap, layer.x_perm, counts,  # noqa: E731
                                         layer.offsets, layer.perm_src, layer.flat_to_row,
                                         layer.ws, overflow=ov, n_overflow=nov,
                                         x_perm_scale=layer.x_scale)
    ms = timed(run, reps, stream)
    kept = int(layer.offsets[E].item())
    es = 4 if cfg.dtype == "f32" else 2
    oes = 1 if cfg.dtype == "fp8" else es
    by = T * d * es + (kept + layer.n_shared * T) * d * oes + T * k * 4 * 4
    out["permute_capped_cf1"] = {"ms": round(ms, 5), "capacity": cap,
                                 "dropped": int(nov.item()), "GB/s": round(by / ms / 1e6, 1),
                                 "hbm_frac": round(by / ms / 1e6 / HBM_PEAK_GBS, 4)}
    # router statistics (reads the route's probability sums and the counts)
    run = lambda: api.moe_router_stats(ps, counts, T, k, 0.01, f, P, summ)  # noqa: E731
    ms = timed(run, reps, stream)
    by = ps.numel() * 4 + E * 4 * 3 + 12
    s = summ.cpu().tolist()
    out["router_stats"] = {"ms": round(ms, 5), "GB/s": round(by / ms / 1e6, 1),
                           "hbm_frac": round(by / ms / 1e6 / HBM_PEAK_GBS, 4),
                           "aux_loss_alpha_0.01": round(s[0], 6),
                           "max_over_mean": round(s[1], 4), "entropy_bits": round(s[2], 4)}
    return out


def cpu_baseline(cfg, layer, x, wr, bias, weights, target_s):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np
    import torch

    import oracle as orc

    def host(t):
        t = t.detach().contiguous().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    xs = host(x)
    wg, wu, wd = weights
    G = cfg.G
    if cfg.dtype == "fp8":
        qs = [[orc.quant_blocks(w[g].float().cpu().numpy(), 128, 128) for g in range(G)]
              for w in (wg, wu, wd)]
        L = orc.Layer(xs, cfg.E, cfg.k, cfg.n_shared, [q for q, _ in qs[0]], [q for q, _ in qs[1]],
                      [q for q, _ in qs[2]], mode=orc.E4M3, sg=[s for _, s in qs[0]],
                      su=[s for _, s in qs[1]], sd=[s for _, s in qs[2]])
    else:
        L = orc.Layer(xs, cfg.E, cfg.k, cfg.n_shared, [host(w) for w in wg],
                      [host(w) for w in wu], [host(w) for w in wd])
    b = None if bias is None else host(bias)
    t0 = time.perf_counter()
    idx, w, _, _ = orc.route(xs, host(wr), cfg.k, b)
    _, offs = orc.counts_offsets(idx, cfg.E, cfg.n_shared)
    orc.permutation(idx, cfg.E, offs)
    t_route = time.perf_counter() - t0
    n = 16
    t0 = time.perf_counter()
    L.tokens(idx, w, np.arange(n))
    t_first = time.perf_counter() - t0
    more = int(min(cfg.T - n, max(0, (target_s - t_first) / max(t_first / n, 1e-6))))
    t0 = time.perf_counter()
    if more > 0:
        L.tokens(idx, w, np.arange(n, n + more))
    t_more = time.perf_counter() - t0
    ntok = n + more
    per_token = t_route / cfg.T + (t_first + t_more) / ntok
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "routing + histogram + permutation of all %d tokens (%.2f s), expert FFN "
                      "+ combine of the first %d tokens (%.2f s), fp64, OpenMP over tokens"
                      % (cfg.T, t_route, ntok, t_first + t_more)}


def build_layer(cfg, dev):
    import torch

    from grouped_gemm_router_amd import synth
    from grouped_gemm_router_amd.layer import MoELayer
    x = synth.gen_x(cfg, dev)
    wr = synth.gen_router(cfg, dev)
    bias = synth.gen_bias(cfg, dev)
    weights = synth.gen_experts(cfg, dev)
    layer = MoELayer(wr, *weights, cfg.k, n_shared=cfg.n_shared, bias=bias,
                     fp8=cfg.dtype == "fp8", keep_logits=False, keep_prob_sums=False)
    layer.alloc(cfg.T)
    out = torch.empty((cfg.T, cfg.d), dtype=layer.out_dtype, device=dev)
    return layer, x, wr, bias, weights, out


def measure(cfg, layer, x, out, warmup, K, stream):
    """(ms per layer step, {step: ms per call}): one untimed step (the first
    launch of each kernel in a process also loads its code), K steps with
    events around every call (on the stream the library launches on), then
    `warmup` untimed steps, then the K timed steps with events only around
    the whole loop."""
    import numpy as np
    import torch
    steps = layer.steps(x, out)
    for _, fn in steps:
        fn()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in steps] for _ in range(K)]
    for i in range(K):
        for j, (_, fn) in enumerate(steps):
            ev[i][j][0].record(stream)
            fn()
            ev[i][j][1].record(stream)
    torch.cuda.synchronize()
    per = {name: float(np.mean([ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(K)]))
           for j, (name, _) in enumerate(steps)}
    for _ in range(warmup):
        for _, fn in steps:
            fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(K):
        for _, fn in steps:
            fn()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / K
    return ms_step, per


def kernel_table(cfg, per, counts):
    bf = step_bytes_flops(cfg, counts)
    peak = PEAK[cfg.dtype]
    kernels = {}
    for name in STEP_NAMES:
        alg, impl, fl = bf[name]
        t = per[name] * 1e-3
        kr = {"ms": round(per[name], 5), "alg_bytes": alg, "GB/s": round(alg / t / 1e9, 1),
              "hbm_frac": round(alg / t / 1e9 / HBM_PEAK_GBS, 4)}
        if impl != alg:
            kr["impl_bytes"] = impl
            kr["hbm_frac_impl_bytes"] = round(impl / t / 1e9 / HBM_PEAK_GBS, 4)
        if fl:
            kr["TFLOP/s"] = round(fl / t / 1e12, 2)
            kr["mfma_frac"] = round(fl / t / 1e12 / peak, 4)
        kernels[name] = kr
    return kernels, bf


def measure_graph(layer, x, out, K, stream):
    """(ms per layer step when the five calls replay as one HIP graph, ms per
    eager step timed right after it): the two loops alternate twice and each
    keeps its faster pass, so a clock that drifts between them does not
    decide the comparison."""
    import torch
    g = layer.capture(x, out)
    for _ in range(3):
        g.replay()
    steps = layer.steps(x, out)
    torch.cuda.synchronize()

    def timed(run):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(K):
            run()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / K

    def eager():
        for _, fn in steps:
            fn()
    best_g, best_e = float("inf"), float("inf")
    for _ in range(2):
        best_g = min(best_g, timed(g.replay))
        best_e = min(best_e, timed(eager))
    del g
    return best_g, best_e


def config_summary(cfg, ms_step, per, counts, ms_graph=None, ms_eager_adjacent=None):
    kernels, _ = kernel_table(cfg, per, counts)
    gemm_ms = per["gemm_gate_up"] + per["gemm_down"]
    tf = cfg.gemm_flops() / (gemm_ms * 1e-3) / 1e12
    return {"ms_per_step": round(ms_step, 5), "tokens_per_s": round(cfg.T / (ms_step * 1e-3), 1),
            "grouped_gemm_tflops": round(tf, 2),
            "grouped_gemm_frac_mfma_peak": round(tf / PEAK[cfg.dtype], 4),
            "peak_tflops": PEAK[cfg.dtype],
            "rows_per_expert_max_over_mean": round(float(counts.max() / counts.mean()), 3),
            "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 5),
            "tokens_per_s_graph": None if ms_graph is None else round(cfg.T / (ms_graph * 1e-3), 1),
            # eager steps timed alternately with the graph replays
            "ms_per_step_eager_beside_graph": (None if ms_eager_adjacent is None
                                               else round(ms_eager_adjacent, 5)),
            "kernels": {n: {kk: v for kk, v in r.items()
                            if kk in ("ms", "hbm_frac", "hbm_frac_impl_bytes", "mfma_frac")}
                        for n, r in kernels.items()}}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: it measures the MoE layer on a single "
              "MI355X (no collectives); got --gpus %d / WORLD_SIZE %d" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import torch

    from grouped_gemm_router_amd import synth

    cfg = synth.CONFIGS[args.config]
    dev = "cuda"
    stream = torch.cuda.current_stream()
    layer, x, wr, bias, weights, out = build_layer(cfg, dev)
    K = args.steps
    extra = None if args.no_extras else extras(cfg, layer, x, K, stream)
    ms_step, per = measure(cfg, layer, x, out, args.warmup, K, stream)

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    counts = layer.counts.cpu().numpy()
    kernels, bf = kernel_table(cfg, per, counts)
    gemm_ms = per["gemm_gate_up"] + per["gemm_down"]
    gemm_tflops = cfg.gemm_flops() / (gemm_ms * 1e-3) / 1e12
    peak = PEAK[cfg.dtype]
    # dominant kernel: gate/up GEMM.  MFMA-bound when its flops need longer at
    # peak than its bytes at HBM peak, else HBM-bound.
    by, _, fl = bf["gemm_gate_up"]
    t = per["gemm_gate_up"] * 1e-3
    mfma_bound = fl / (peak * 1e12) >= by / (HBM_PEAK_GBS * 1e9)
    traffic = load_traffic("gemm_gate_up", cfg.name)
    if mfma_bound:
        roof = {"kernel": "gemm_gate_up", "bound": "mfma", "achieved": round(fl / t / 1e12, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(fl / t / 1e12 / peak, 4),
                "traffic": traffic}
    else:
        roof = {"kernel": "gemm_gate_up", "bound": "hbm", "achieved": round(by / t / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4), "traffic": traffic}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, layer, x, wr, bias, weights, args.cpu_seconds)

    configs = None
    if not args.no_configs:
        ms_g, ms_e = measure_graph(layer, x, out, args.config_steps, stream)
        configs = {cfg.name: config_summary(cfg, ms_step, per, counts, ms_g, ms_e)}
        del layer, x, wr, bias, weights, out
        torch.cuda.empty_cache()
        for name in CONFIG_ORDER:
            if name == cfg.name:
                continue
            c = synth.CONFIGS[name]
            L, xx, _, _, _, oo = build_layer(c, dev)
            ms_c, per_c = measure(c, L, xx, oo, 3, args.config_steps, stream)
            ms_g, ms_e = measure_graph(L, xx, oo, args.config_steps, stream)
            configs[name] = config_summary(c, ms_c, per_c, L.counts.cpu().numpy(), ms_g, ms_e)
            del L, xx, oo
            torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": round(cfg.T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "fp8": "e4m3"}[cfg.dtype],
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) router, N(0,1/sqrt(fan_in)) "
                "experts)",
        "config": {"workload": cfg.name, **cfg.describe(),
                   "rows_per_expert_max_over_mean": round(float(counts.max() / counts.mean()), 3)},
        "grouped_gemm_tflops": round(gemm_tflops, 2),
        "grouped_gemm_frac_mfma_peak": round(gemm_tflops / peak, 4),
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": cpu,
        "configs": configs,
        "extras": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
