"""GPU parity of moe_combine against the oracle's fp64 gather-weight-sum.

Tolerance, elementwise: fp32 accumulation of the k + n_shared terms errs by
at most (k + n_shared + 1) u sum_j |w_j Y_j| (u = 2^-24), plus one rounding
of the stored output (bf16: 2^-8 |y|; fp32: u |y|).
"""
import numpy as np
import pytest
import torch

from grouped_gemm_router_amd import synth
from gpu_util import DEV, U32, abs_operand, assert_within, np_of

pytestmark = pytest.mark.gpu


def api():
    from grouped_gemm_router_amd import api as a
    return a


@pytest.mark.parametrize("T,E,k,ns,d", [(1, 1, 1, 0, 8), (256, 8, 2, 0, 128), (300, 256, 8, 1, 7168),
                                        (77, 16, 4, 2, 64), (4096, 8, 2, 0, 4096)])
@pytest.mark.parametrize("ydt,odt", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")])
def test_combine(orc, T, E, k, ns, d, ydt, odt):
    a = api()
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
    idx = synth.random_selection(T, E, k, s=T + E).numpy()
    _, offs = orc.counts_offsets(idx, E, ns)
    _, f2r = orc.permutation(idx, E, offs)
    rows = T * k + ns * T
    f2r_full = np.concatenate([f2r, T * k + np.arange(ns * T)]).astype(np.int32)
    Y = synth.randn((rows, d), 1.0, 3 + d, DEV, tdt[ydt])
    w = synth.random_gate_weights(T, k, 4 + T).to(DEV)
    out = torch.full((T, d), float("nan"), dtype=tdt[odt], device=DEV)
    a.moe_combine(Y, torch.from_numpy(f2r_full).to(DEV), w, out, n_shared=ns)
    torch.cuda.synchronize()
    ref = orc.combine(np_of(Y), f2r, np_of(w), T, k, ns)
    absum = orc.combine(abs_operand(np_of(Y)), f2r, np_of(w), T, k, ns)
    store = 2.0 ** -8 if odt == "bf16" else U32
    bound = (k + ns + 1) * U32 * absum + store * np.abs(ref)
    assert_within(out.float().cpu().numpy(), ref, bound)


def test_combine_skips_dropped_entries(orc):
    a = api()
    T, k, d = 10, 2, 64
    Y = synth.randn((T * k, d), 1.0, 1, DEV, torch.float32)
    f2r = np.arange(T * k, dtype=np.int32)
    f2r[3] = -1
    w = torch.ones((T, k), dtype=torch.float32, device=DEV)
    out = torch.empty((T, d), dtype=torch.float32, device=DEV)
    a.moe_combine(Y, torch.from_numpy(f2r).to(DEV), w, out)
    torch.cuda.synchronize()
    Yn = Y.cpu().numpy()
    np.testing.assert_allclose(out[1].cpu().numpy(), Yn[2], rtol=1e-6)   # token 1 lost j = 1
    np.testing.assert_allclose(out[0].cpu().numpy(), Yn[0] + Yn[1], rtol=1e-6)
