"""Seeded synthetic inputs and workload shapes for the MoE expert layer.

This module only draws random numbers and names shapes.  It holds none of the
layer's arithmetic (no routing, no permutation, no GEMM, no quantisation), so
both the HIP path and the CPU oracle may take their inputs from it.  It
imports torch only; it does not load the HIP library.

Recipe:

* Every tensor is drawn with ``torch.randn`` / ``torch.rand`` from its own
  ``torch.Generator`` seeded with ``seed(cfg_id, tensor, group, matrix)``;
  draws are fp32 and then rounded (round-to-nearest-even) to the layer dtype.
  The same seed on the same device type always gives the same tensor, so any
  single expert can be regenerated on its own.
* x ~ N(0, 1); router W_r [E][d] ~ N(0, 0.02); W_gate, W_up [dff][d] ~
  N(0, 1/sqrt(d)); W_down [d][dff] ~ N(0, 1/sqrt(dff)) (second argument is
  the standard deviation; fan_in is the input width of each matrix).
* Skewed routing adds a per-expert logit bias b_e = -lam * s * ln(1 + r_e)
  with s = 1.2 (a Zipf exponent) and r a seeded random ranking of the
  experts, so expert popularity falls off like a Zipf law.  lam = 1.15 puts
  the hottest expert near 3x the mean load for the 8-expert top-2 shape (the
  most a top-2 of 8 layer can reach is 4x).
* The decode-size skewed case uses the first 128 tokens of the skewed
  4096-token draw with the same router, bias and experts.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

# tensor ids inside a config
X, ROUTER, EXPERT, SHARED, RANK, AUX = 1, 2, 3, 4, 5, 6
# matrix ids inside an expert
GATE, UP, DOWN = 0, 1, 2

ZIPF_S = 1.2
SKEW_LAMBDA = 1.15


@dataclass(frozen=True)
class MoEConfig:
    name: str
    cfg_id: int
    T: int
    d: int
    E: int
    k: int
    dff: int
    n_shared: int = 0
    dtype: str = "bf16"  # "f32" | "bf16" | "fp8" (fp8 = E4M3 expert GEMMs)
    skew: bool = False
    t_source: int = 0    # draw x with this many rows and keep the first T

    @property
    def G(self) -> int:
        return self.E + self.n_shared

    @property
    def rows(self) -> int:
        return self.T * self.k + self.n_shared * self.T

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def gemm_flops(self) -> float:
        """Algorithmic FLOPs of the two grouped GEMMs (real rows only)."""
        return 2.0 * self.rows * self.d * 2 * self.dff + 2.0 * self.rows * self.dff * self.d

    def describe(self) -> dict:
        return {"T": self.T, "d_model": self.d, "experts": self.E, "top_k": self.k,
                "d_ff": self.dff, "shared_experts": self.n_shared, "dtype": self.dtype,
                "skew": self.skew}


CONFIGS = {
    c.name: c
    for c in [
        MoEConfig("tiny_f32", 1, T=256, d=128, E=8, k=2, dff=256, dtype="f32"),
        MoEConfig("mixtral_bf16", 2, T=4096, d=4096, E=8, k=2, dff=14336),
        MoEConfig("skew_bf16", 3, T=4096, d=4096, E=8, k=2, dff=14336, skew=True),
        MoEConfig("skew_decode_bf16", 3, T=128, d=4096, E=8, k=2, dff=14336, skew=True,
                  t_source=4096),
        MoEConfig("deepseek_bf16", 5, T=4096, d=7168, E=256, k=8, dff=2048, n_shared=1),
        MoEConfig("deepseek_fp8", 6, T=4096, d=7168, E=256, k=8, dff=2048, n_shared=1,
                  dtype="fp8"),
    ]
}


def scaled(cfg: MoEConfig, **kw) -> MoEConfig:
    """A copy of a config with some sizes replaced (for small parity cases)."""
    d = dict(cfg.__dict__)
    d.update(kw)
    return MoEConfig(**d)


def seed(cfg_id: int, tensor: int, group: int = 0, matrix: int = 0) -> int:
    return ((cfg_id * 16 + tensor) * 4096 + group) * 4 + matrix


def generator(s: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def randn(shape, std: float, s: int, device, dtype=torch.float32) -> torch.Tensor:
    t = torch.randn(shape, generator=generator(s, device), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def to_bf16_bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (for the oracle)."""
    return t.contiguous().view(torch.int16).cpu().numpy().view("uint16")


# ----------------------------------------------------------------------------
# layer inputs
# ----------------------------------------------------------------------------

def gen_x(cfg: MoEConfig, device) -> torch.Tensor:
    n = max(cfg.T, cfg.t_source)
    x = randn((n, cfg.d), 1.0, seed(cfg.cfg_id, X), device, cfg.torch_dtype)
    return x[: cfg.T].contiguous()


def gen_router(cfg: MoEConfig, device) -> torch.Tensor:
    return randn((cfg.E, cfg.d), 0.02, seed(cfg.cfg_id, ROUTER), device, cfg.torch_dtype)


def gen_bias(cfg: MoEConfig, device):
    """Zipf-shaped logit bias for the skewed configs (None otherwise)."""
    if not cfg.skew:
        return None
    g = generator(seed(cfg.cfg_id, RANK), "cpu")
    rank = torch.randperm(cfg.E, generator=g)
    b = torch.tensor([-SKEW_LAMBDA * ZIPF_S * math.log(1.0 + float(r)) for r in rank],
                     dtype=torch.float32)
    return b.to(device)


def gen_expert(cfg: MoEConfig, group: int, matrix: int, device, dtype=None) -> torch.Tensor:
    """One expert matrix in F.linear orientation ([out][in]).

    Groups 0..E-1 are routed experts, E.. are shared experts.  Returned in
    ``dtype`` (default: the layer dtype; fp32 draws for fp8 layers, which each
    side quantises itself).
    """
    if dtype is None:
        dtype = torch.float32 if cfg.dtype in ("f32", "fp8") else torch.bfloat16
    tensor = EXPERT if group < cfg.E else SHARED
    gi = group if group < cfg.E else group - cfg.E
    if matrix in (GATE, UP):
        shape, std = (cfg.dff, cfg.d), 1.0 / math.sqrt(cfg.d)
    else:
        shape, std = (cfg.d, cfg.dff), 1.0 / math.sqrt(cfg.dff)
    return randn(shape, std, seed(cfg.cfg_id, tensor, gi, matrix), device, dtype)


def gen_experts(cfg: MoEConfig, device, dtype=None):
    """All expert weights stacked: (W_gate [G][dff][d], W_up, W_down [G][d][dff])."""
    if dtype is None:
        dtype = torch.float32 if cfg.dtype in ("f32", "fp8") else torch.bfloat16
    G = cfg.G
    wg = torch.empty((G, cfg.dff, cfg.d), dtype=dtype, device=device)
    wu = torch.empty((G, cfg.dff, cfg.d), dtype=dtype, device=device)
    wd = torch.empty((G, cfg.d, cfg.dff), dtype=dtype, device=device)
    for g in range(G):
        wg[g] = gen_expert(cfg, g, GATE, device, dtype)
        wu[g] = gen_expert(cfg, g, UP, device, dtype)
        wd[g] = gen_expert(cfg, g, DOWN, device, dtype)
    return wg, wu, wd


# ----------------------------------------------------------------------------
# stand-alone kernel inputs (structurally valid routing decisions etc.)
# ----------------------------------------------------------------------------

def random_selection(T: int, E: int, k: int, s: int, device="cpu", weights=None):
    """A random routing decision: k distinct experts per token, int32 [T][k].

    Drawn by weighted sampling without replacement (Efraimidis-Spirakis keys
    u^(1/w)); uniform when ``weights`` is None.  This only produces a valid
    input for the permutation and combine steps; it is not the router.
    """
    u = torch.rand((T, E), generator=generator(s, "cpu"), dtype=torch.float64)
    if weights is not None:
        w = torch.as_tensor(weights, dtype=torch.float64)
        u = u.clamp_min(1e-300).log() / w  # log of u^(1/w), same order
    order = torch.argsort(u, dim=1, descending=True, stable=True)
    return order[:, :k].to(torch.int32).contiguous().to(device)


def random_gate_weights(T: int, k: int, s: int, device="cpu") -> torch.Tensor:
    return torch.rand((T, k), generator=generator(s, "cpu"), dtype=torch.float32).to(device)


def random_e4m3_codes(shape, s: int, device="cpu") -> torch.Tensor:
    """Random finite E4M3 codes (uint8), never the NaN codes 0x7F / 0xFF."""
    c = torch.randint(0, 254, shape, generator=generator(s, "cpu"), dtype=torch.int32)
    c = torch.where(c >= 0x7F, c + 1, c)  # skip 0x7F; 0xFF is out of range
    return c.to(torch.uint8).to(device)


def random_scales(shape, s: int, device="cpu", lo=0.25, hi=4.0) -> torch.Tensor:
    u = torch.rand(shape, generator=generator(s, "cpu"), dtype=torch.float32)
    return (lo * (hi / lo) ** u).to(device)
