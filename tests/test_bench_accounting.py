"""CPU checks of the benchmark's algorithmic byte and flop counts (the
denominators of every roofline fraction it prints), against the per-step
figures worked out from the layer's shapes: GEMM flops count real rows
only, bytes count every input and output once and each active expert's
weights once, in the method's storage types (bf16 H and Y; E4M3 with fp32
scales in the FP8 layer)."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from grouped_gemm_router_amd import synth  # noqa: E402


def counts_of(cfg, active=None):
    c = np.full(cfg.E, cfg.T * cfg.k // cfg.E, dtype=np.int64)
    if active is not None:
        c[active:] = 0
    return c


def test_mixtral_gemm_flops_and_bytes():
    cfg = synth.CONFIGS["mixtral_bf16"]
    bf = bench.step_bytes_flops(cfg, counts_of(cfg))
    rows = 4096 * 2
    assert bf["gemm_gate_up"][2] == pytest.approx(1.924e12, rel=1e-3)   # 2 x 8192 x 4096 x 28672
    assert bf["gemm_down"][2] == pytest.approx(0.962e12, rel=1e-3)
    a = rows * 4096 * 2
    w = 8 * 2 * 14336 * 4096 * 2                                        # 1.88 GB of gate/up weights
    h = rows * 14336 * 2
    assert bf["gemm_gate_up"][0] == a + w + h
    # down: H in, the down weights, Y out in bf16 (the method's type); the
    # implementation's fp32 Y is the second figure
    wd = 8 * 4096 * 14336 * 2
    assert bf["gemm_down"][0] == h + wd + rows * 4096 * 2
    assert bf["gemm_down"][1] == h + wd + rows * 4096 * 4
    # route: x and the router weights in, the selection out
    assert bf["route"][0] == 4096 * 4096 * 2 + 8 * 4096 * 2 + 4096 * 2 * 8
    # combine: Y in (bf16), out, the gate weights and flat_to_row
    assert bf["combine"][0] == rows * 4096 * 2 + 4096 * 4096 * 2 + 4096 * 2 * 4 + rows * 4


def test_deepseek_counts_active_experts_and_the_shared_one():
    cfg = synth.CONFIGS["deepseek_bf16"]
    full = bench.step_bytes_flops(cfg, counts_of(cfg))
    rows = 4096 * 8 + 4096
    assert full["gemm_gate_up"][2] == pytest.approx(2.165e12, rel=1e-3)
    assert full["gemm_down"][2] == pytest.approx(1.082e12, rel=1e-3)
    wg = 257 * 2 * 2048 * 7168 * 2                                      # 15.1 GB
    assert full["gemm_gate_up"][0] == rows * 7168 * 2 + wg + rows * 2048 * 2
    # an expert with no rows contributes no weight bytes
    half = bench.step_bytes_flops(cfg, counts_of(cfg, active=128))
    assert full["gemm_gate_up"][0] - half["gemm_gate_up"][0] == 128 * 2 * 2048 * 7168 * 2


def test_fp8_weights_and_scales():
    cfg = synth.CONFIGS["deepseek_fp8"]
    bf = bench.step_bytes_flops(cfg, counts_of(cfg))
    rows = 4096 * 8 + 4096
    wg = 257 * 2 * 2048 * 7168                                          # E4M3
    wsc = 257 * 2 * (2048 // 128) * (7168 // 128) * 4                   # 128 x 128 block scales
    a = rows * 7168 + rows * (7168 // 128) * 4                          # codes + 1 x 128 scales
    assert bf["gemm_gate_up"][0] == a + wg + wsc + rows * 2048 + rows * (2048 // 128) * 4
    wd = 257 * 7168 * 2048
    # both GEMMs' weights with their scales: 11.32 GB + 2.7 MB
    assert wg + wd == pytest.approx(11.32e9, rel=1e-3)
    assert wsc * 3 // 2 == pytest.approx(2.7e6, rel=0.05)
