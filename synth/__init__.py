"""Seeded synthetic inputs for the MoE layer, shared by the tests, the benchmark and
the smoke check.

This module holds none of the method's arithmetic: it draws random numbers and
converts them to bf16 with torch's own conversion.  Host tensors come from numpy
PCG64 streams keyed (config, tensor id, expert); large device tensors come from a
torch device generator seeded from the same key, so nothing of that size ever
crosses PCIe.  Either way the same key gives the same bytes on every run.

Workload recipes (shapes and distributions of the pages' workloads; the pages'
datasets and checkpoints are not available, these stand in for them):

* tiny     E=8,   H=256,  I=128,  k=2, T=64,    r=8   router R~N(0,0.02), logits = fl32(X R^T)
* glm      E=256, H=6144, I=2048, k=8, T=16384, r=64  logits ~U(0,1)
* qwen     E=128, H=2048, I=768,  k=8, T=8192,  r=64  logits ~U(0,1), W4A4
* glm_nf4  glm with NF4 weights; logits = -1.1 ln(rank_e) + Gumbel, 16 experts masked to -inf
* skew     logits ~U(0,1) with +1 on expert 0 for the first 23% of the tokens (one
           expert with about twice the rows of the others; a parity-test recipe)
* balanced logits 1 on experts (k t + j) mod E, j < k, and 0 elsewhere: every expert gets
           exactly T k / E rows when E divides T k (a reference routing for timing)
* weights  ~N(0,0.02) with a Bernoulli(0.001) outlier mask multiplied by 20
  (the quantizer workload; tiny uses no outliers), LoRA A, B ~N(0,0.01),
  activations and output gradients ~N(0,1).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# tensor ids of the seed keys
T_X, T_ROUTER, T_LOGITS, T_WGU, T_WDN, T_AGU, T_BGU, T_ADN, T_BDN, T_DOUT, T_MISC = range(11)


@dataclass(frozen=True)
class Shape:
    name: str
    E: int
    H: int
    I: int
    k: int
    T: int
    r: int
    act_quant: bool = False
    fmt: str = "nvfp4"
    logits: str = "uniform"      # "router" | "uniform" | "zipf" | "skew" | "balanced"
    outliers: bool = True
    seed: int = 0
    weight_seed: int = -1          # -1: same as seed
    shared_a: bool = False         # one LoRA-A for all experts: A_gu [r, H], A_dn [r, I]

    @property
    def wseed(self) -> int:
        return self.seed if self.weight_seed < 0 else self.weight_seed

    @property
    def R(self) -> int:
        return self.T * self.k


TINY = Shape("tiny", E=8, H=256, I=128, k=2, T=64, r=8, logits="router", outliers=False, seed=1)
GLM = Shape("glm", E=256, H=6144, I=2048, k=8, T=16384, r=64, seed=4, weight_seed=2)
QWEN = Shape("qwen", E=128, H=2048, I=768, k=8, T=8192, r=64, act_quant=True, seed=3)
GLM_NF4 = Shape("glm_nf4", E=256, H=6144, I=2048, k=8, T=16384, r=64, fmt="nf4", logits="zipf", seed=5,
                weight_seed=2)
SHAPES = {s.name: s for s in (TINY, GLM, QWEN, GLM_NF4)}


def _torch():
    import torch
    return torch


def _rng(*key):
    return np.random.default_rng([int(v) for v in key])


def _dev_gen(device, *key):
    torch = _torch()
    g = torch.Generator(device=device)
    s = 0
    for v in key:
        s = (s * 1_000_003 + int(v) + 1) % (2 ** 62)
    g.manual_seed(s)
    return g


def to_bf16_host(a: np.ndarray):
    """float32 numpy -> torch.bfloat16 CPU tensor (torch's round to nearest even)."""
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def normal(shape, std, key, device="cpu", outliers=False):
    """bf16 tensor of N(0, std^2) draws (times 20 where a Bernoulli(0.001) mask hits)."""
    torch = _torch()
    if device == "cpu":
        rng = _rng(*key)
        a = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
        if outliers:
            m = rng.random(size=shape, dtype=np.float32) < np.float32(0.001)
            a = np.where(m, a * np.float32(20.0), a).astype(np.float32)
        return to_bf16_host(a)
    g = _dev_gen(device, *key)
    a = torch.randn(shape, generator=g, device=device, dtype=torch.float32).mul_(std)
    if outliers:
        m = torch.rand(shape, generator=g, device=device, dtype=torch.float32) < 0.001
        a = torch.where(m, a * 20.0, a)
    return a.to(torch.bfloat16)


def normal_stack(E, rows, cols, std, key, device="cpu", outliers=False):
    """[E, rows, cols] bf16, one stream per expert (so any expert can be regenerated alone)."""
    torch = _torch()
    out = torch.empty((E, rows, cols), dtype=torch.bfloat16, device=device)
    for e in range(E):
        out[e] = normal((rows, cols), std, key + (e,), device=device, outliers=outliers)
    return out


def logits(shape: Shape, x=None, router=None, device="cpu"):
    """fp32 router logits [T, E] for the shape's recipe."""
    torch = _torch()
    T, E = shape.T, shape.E
    key = (shape.seed, T_LOGITS)
    if shape.logits == "router":
        # fl32(X R^T) accumulated in float64 on the host
        xf = x.float().cpu().numpy().astype(np.float64)
        rf = router.float().cpu().numpy().astype(np.float64)
        lg = torch.from_numpy((xf @ rf.T).astype(np.float32))
        return lg.to(device)
    if shape.logits == "uniform":
        if device == "cpu":
            return torch.from_numpy(_rng(*key).random((T, E), dtype=np.float32))
        g = _dev_gen(device, *key)
        return torch.rand((T, E), generator=g, device=device, dtype=torch.float32)
    if shape.logits == "balanced":
        torch_ = _torch()
        e = (shape.k * torch_.arange(T)[:, None] + torch_.arange(shape.k)[None, :]) % E
        lg = torch_.zeros((T, E), dtype=torch_.float32)
        lg.scatter_(1, e, 1.0)
        return lg.to(device)
    if shape.logits == "skew":
        lg = _rng(*key).random((T, E), dtype=np.float32)
        lg[: (23 * T + 99) // 100, 0] += np.float32(1.0)
        return torch.from_numpy(lg).to(device)
    # Zipf(1.1)-skewed: -1.1 ln(rank_e) + Gumbel(0,1); the 16 least popular masked out
    rng = _rng(*key)
    rank = rng.permutation(E) + 1
    bias = (-1.1 * np.log(rank.astype(np.float64))).astype(np.float32)
    gum = rng.gumbel(size=(T, E)).astype(np.float32)
    lg = (bias[None, :] + gum).astype(np.float32)
    lg[:, rank > E - 16] = -np.inf
    return torch.from_numpy(lg).to(device)


@dataclass
class LayerInputs:
    shape: Shape
    x: object            # bf16 [T, H]
    logits: object       # f32 [T, E]
    w_gu: object         # bf16 [E, 2I, H]
    w_dn: object         # bf16 [E, H, I]
    A_gu: object         # bf16 [E, r, H] ([r, H] when shared)
    B_gu: object         # bf16 [E, 2I, r]
    A_dn: object         # bf16 [E, r, I] ([r, I] when shared)
    B_dn: object         # bf16 [E, H, r]
    dout: object         # bf16 [T, H]
    router: object = None


def layer_inputs(shape: Shape, device="cpu", with_weights=True) -> LayerInputs:
    s = shape
    sd = s.seed
    x = normal((s.T, s.H), 1.0, (sd, T_X), device=device)
    router = None
    if s.logits == "router":
        router = normal((s.E, s.H), 0.02, (sd, T_ROUTER), device="cpu")
    lg = logits(s, x=x, router=router, device=device)
    if with_weights:
        ws = s.wseed
        wgu = normal_stack(s.E, 2 * s.I, s.H, 0.02, (ws, T_WGU), device, outliers=s.outliers)
        wdn = normal_stack(s.E, s.H, s.I, 0.02, (ws, T_WDN), device, outliers=s.outliers)
    else:
        wgu = wdn = None
    if s.r:
        ea = () if s.shared_a else (s.E,)
        agu = normal(ea + (s.r, s.H), 0.01, (sd, T_AGU), device=device)
        bgu = normal((s.E, 2 * s.I, s.r), 0.01, (sd, T_BGU), device=device)
        adn = normal(ea + (s.r, s.I), 0.01, (sd, T_ADN), device=device)
        bdn = normal((s.E, s.H, s.r), 0.01, (sd, T_BDN), device=device)
    else:
        agu = bgu = adn = bdn = None
    dout = normal((s.T, s.H), 1.0, (sd, T_DOUT), device=device)
    return LayerInputs(s, x, lg, wgu, wdn, agu, bgu, adn, bdn, dout, router)


def quantizer_stacks(device="cuda", E=256, H=6144, I=2048, seed=2):
    """The quantizer workload: gate_up [E, 2I, H] and down [E, H, I], N(0,0.02) with outliers."""
    wgu = normal_stack(E, 2 * I, H, 0.02, (seed, T_WGU), device, outliers=True)
    wdn = normal_stack(E, H, I, 0.02, (seed, T_WDN), device, outliers=True)
    return wgu, wdn


def f32_numpy(t) -> np.ndarray:
    """Any torch tensor -> float32 numpy on the host (bf16 values convert exactly)."""
    return t.detach().float().cpu().numpy()
