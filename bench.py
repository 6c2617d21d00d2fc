"""Benchmark: one step = one MoE expert-layer forward (route -> permute ->
grouped GEMM gate/up + SwiGLU -> grouped GEMM down -> combine) through
libmoe.so on one MI355X, over seeded synthetic inputs already resident in
HBM.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

Default workload: the Mixtral-shape bf16 layer (T=4096, d=4096, E=8, top-2,
SwiGLU d_ff=14336).  `value` is layer tokens/s; the grouped-GEMM TFLOP/s and
fraction of bf16 MFMA peak ride along.  Per-kernel times come from HIP events
recorded on the launch stream around every call of every timed step.
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



def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="mixtral_bf16")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (counter calibration)")
    return p.parse_args()


def step_bytes_flops(cfg, counts):
    """Algorithmic bytes and flops per launch of each step."""
    es = 4 if cfg.dtype == "f32" else 2
    T, d, E, k, dff, ns = cfg.T, cfg.d, cfg.E, cfg.k, cfg.dff, cfg.n_shared
    rows = cfg.rows
    active = int((counts > 0).sum()) + ns
    w_es = 1 if cfg.dtype == "fp8" else es
    act_es = 1 if cfg.dtype == "fp8" else es
    out = {}
    out["route"] = (T * d * es + E * d * es + T * E * 4 + T * k * 8, 2.0 * T * E * d)
    out["permute"] = (T * d * es + rows * d * act_es + T * k * 4 * 4
                      + (rows * (d // 128) * 4 if cfg.dtype == "fp8" else 0), 0.0)
    wsc = (active * 2 * (dff // 128) * (d // 128) * 4) if cfg.dtype == "fp8" else 0
    out["gemm_gate_up"] = (rows * d * act_es + active * 2 * dff * d * w_es + wsc
                           + rows * dff * act_es, 2.0 * rows * d * 2 * dff)
    y_es = 2 if cfg.dtype == "fp8" else 4  # Y is fp32 except in the FP8 layer
    out["gemm_down"] = (rows * dff * act_es + active * d * dff * w_es + wsc // 2
                        + rows * d * y_es, 2.0 * rows * dff * d)
    out["combine"] = (rows * d * y_es + T * d * es + T * k * 8, 0.0)
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
    lg = torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    api.moe_route(x, layer.w_router, idx, w, logits=lg, logit_bias=layer.bias)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    f = torch.empty((E,), dtype=torch.float32, device=dev)
    P = torch.empty_like(f)
    summ = torch.empty((3,), dtype=torch.float32, device=dev)
    sws = torch.empty((max(api.moe_router_stats_workspace_size(T, E), 4),), dtype=torch.uint8,
                      device=dev)
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
    # router statistics (reads the logits and the counts)
    run = lambda: api.moe_router_stats(lg, counts, k, 0.01, f, P, summ, ws=sws)  # noqa: E731
    ms = timed(run, reps, stream)
    by = T * E * 4 + E * 4 * 3 + 12
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


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: it measures the MoE layer on a single "
              "MI355X (no collectives); got --gpus %d / WORLD_SIZE %d" % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from grouped_gemm_router_amd import synth
    from grouped_gemm_router_amd.layer import MoELayer

    cfg = synth.CONFIGS[args.config]
    dev = "cuda"
    x = synth.gen_x(cfg, dev)
    wr = synth.gen_router(cfg, dev)
    bias = synth.gen_bias(cfg, dev)
    weights = synth.gen_experts(cfg, dev)
    layer = MoELayer(wr, *weights, cfg.k, n_shared=cfg.n_shared, bias=bias,
                     fp8=cfg.dtype == "fp8", keep_logits=False)
    layer.alloc(cfg.T)
    out = torch.empty((cfg.T, cfg.d), dtype=layer.out_dtype, device=dev)
    steps = layer.steps(x, out)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        for _, fn in steps:
            fn()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in steps] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        for j, (_, fn) in enumerate(steps):
            ev[i][j][0].record(stream)
            fn()
            ev[i][j][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / K
    per = {name: float(np.mean([ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(K)]))
           for j, (name, _) in enumerate(steps)}

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    counts = layer.counts.cpu().numpy()
    bf = step_bytes_flops(cfg, counts)
    gemm_ms = per["gemm_gate_up"] + per["gemm_down"]
    gemm_tflops = cfg.gemm_flops() / (gemm_ms * 1e-3) / 1e12
    peak = PEAK[cfg.dtype]
    kernels = {}
    for name in STEP_NAMES:
        by, fl = bf[name]
        t = per[name] * 1e-3
        kernels[name] = {"ms": round(per[name], 5), "GB/s": round(by / t / 1e9, 1),
                         "hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4)}
        if fl:
            kernels[name]["TFLOP/s"] = round(fl / t / 1e12, 2)
            kernels[name]["mfma_frac"] = round(fl / t / 1e12 / peak, 4)
    # dominant kernel: gate/up GEMM.  MFMA-bound when its flops need longer at
    # peak than its bytes at HBM peak, else HBM-bound.
    by, fl = bf["gemm_gate_up"]
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

    extra = extras(cfg, layer, x, K, stream)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, layer, x, wr, bias, weights, args.cpu_seconds)

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
        "extras": extra,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
