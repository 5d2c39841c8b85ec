"""Seeded synthetic inputs for the GLA + SREM path.

This module is shared by the tests, the benchmark and the smoke check: the
same materialised tensors go to the HIP library and to the CPU oracle.  It
holds no arithmetic of the method itself (no recurrence, conv, remap or
normalisation): it only draws random numbers and shapes them.

Shapes follow the DiG latent grids: T = (I/p)^2 tokens for I = image/8 latent
side and patch p = 2 ("Scalable Diffusion Models with Transformers" notes,
3.1 Patchify, Eq. 2; DiG paper notes, 整体框架), i.e. a 16x16 grid at 256^2,
64x64 at 1024^2, 112x112 at 1792^2 and 128x128 at 2048^2.  The pages train on
ImageNet; no dataset, VAE or trained weight is available here, so seeded
Gaussian activations of those shapes stand in for the real ones.

Distributions:
  q, k, v         ~ N(0, 1) * qkv_scale          (bf16 or fp32)
  log_alpha       = logsigmoid(x) / 16,  x ~ N(gate_mu, 1)   (per key channel)
  conv weight w   = identity 3x3 (centre tap 1) [+ N(0, 0.01) perturbation]
  adaLN scale/shift ~ N(0, 0.1)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch
import torch.nn.functional as F

DIRS = ("l2r", "r2l", "t2b", "b2t")
DIR_CODE = {d: i for i, d in enumerate(DIRS)}


@dataclass(frozen=True)
class Config:
    key: str
    name: str
    B: int
    H: int
    gh: int
    gw: int
    d: int
    dtype: str            # "f32" or "bf16" for q, k, v, log_alpha
    qkv_scale: float
    gate_mu: float
    chunk: int
    dirs: tuple
    adaln: bool = False   # full token-mixer step: adaLN prologue on raw activations
    conv_perturb: float = 0.0
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return self.gh * self.gw

    @property
    def C(self) -> int:
        return self.H * self.d

    def direction(self, call_index: int) -> str:
        return self.dirs[call_index % len(self.dirs)]


CONFIGS = {
    "C0": Config("C0", "tiny-fp32-8x8", B=1, H=2, gh=8, gw=8, d=16, dtype="f32",
                 qkv_scale=1.0, gate_mu=0.0, chunk=16, dirs=("l2r",), seed=1000),
    "C1": Config("C1", "dig-s2-256px", B=32, H=6, gh=16, gw=16, d=64, dtype="bf16",
                 qkv_scale=1.0 / math.sqrt(64), gate_mu=0.0, chunk=64, dirs=DIRS, seed=1001),
    "C2": Config("C2", "dig-xl2-1024px", B=8, H=16, gh=64, gw=64, d=72, dtype="bf16",
                 qkv_scale=1.0 / math.sqrt(72), gate_mu=2.0, chunk=64, dirs=DIRS,
                 conv_perturb=0.01, seed=1002),
    "C3": Config("C3", "dig-s2-1792px", B=4, H=6, gh=112, gw=112, d=64, dtype="bf16",
                 qkv_scale=1.0 / math.sqrt(64), gate_mu=0.0, chunk=64, dirs=("t2b", "b2t"), seed=1003),
    "C4": Config("C4", "dig-xl2-2048px-mixer-step", B=1, H=16, gh=128, gw=128, d=72, dtype="bf16",
                 qkv_scale=1.0 / math.sqrt(72), gate_mu=2.0, chunk=64, dirs=DIRS, adaln=True,
                 conv_perturb=0.01, seed=1004),
    # DiG-B/2 at 512^2 (32x32 latent-patch grid).  The pages give the B model's
    # depth only; its width is read as 12 heads of 64 channels (hidden 768),
    # between S (6 x 64) and XL (16 x 72), and the image side as 512, between
    # the S (256) and XL (1024) workloads; the gates as S's.
    "CB": Config("CB", "dig-b2-512px", B=16, H=12, gh=32, gw=32, d=64, dtype="bf16",
                 qkv_scale=1.0 / math.sqrt(64), gate_mu=0.0, chunk=64, dirs=DIRS, seed=1005),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gate_from_normal(x: torch.Tensor) -> torch.Tensor:
    """log alpha = logsigmoid(x) / 16: the synthetic forget-gate recipe (alpha = sigmoid(x)^(1/16))."""
    return F.logsigmoid(x) / 16.0


def conv_weight(C: int, perturb: float, gen: torch.Generator | None, device="cpu") -> torch.Tensor:
    """[C, 3, 3] fp32: identity 3x3 (centre 1, rest 0), plus N(0, perturb) if perturb > 0."""
    w = torch.zeros(C, 3, 3, dtype=torch.float32, device=device)
    w[:, 1, 1] = 1.0
    if perturb > 0:
        w += torch.randn(C, 3, 3, generator=gen, dtype=torch.float32, device=device) * perturb
    return w


def gla_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16", seed: int = 0,
               qkv_scale: float = 1.0, gate_mu: float = 0.0, gate_div: float = 16.0) -> dict:
    """Generic seeded q, k, v, log_alpha in canonical [B, T, H, d] layout (CPU tensors)."""
    gen = _gen(seed)
    td = torch_dtype(dtype)
    q = (torch.randn(B, T, H, dk, generator=gen) * qkv_scale).to(td)
    k = (torch.randn(B, T, H, dk, generator=gen) * qkv_scale).to(td)
    v = (torch.randn(B, T, H, dv, generator=gen) * qkv_scale).to(td)
    x = torch.randn(B, T, H, dk, generator=gen) + gate_mu
    g = (F.logsigmoid(x) / gate_div).to(td)
    return {"q": q, "k": k, "v": v, "log_alpha": g}


def make_inputs(key: str, set_index: int = 0, device="cpu") -> dict:
    """Materialise the inputs of one named workload.

    Draw order: q (or raw x_q), k (x_k), v (x_v), gate x, then the full-step
    extras (adaLN scale, shift, conv-weight perturbation).  `set_index` > 0
    gives an independent set of the same shapes (rotating buffers).  With
    device="cuda" the draws come from the seeded device generator (a
    different, equally seeded stream; used for large benchmark sets).
    """
    cfg = CONFIGS[key]
    gen = _gen(cfg.seed + 7919 * set_index, device)
    B, T, H, d = cfg.B, cfg.T, cfg.H, cfg.d
    td = torch_dtype(cfg.dtype)
    out = {"cfg": cfg}
    if cfg.adaln:
        # raw activations [3, B, T, C] (x_q, x_k, x_v), modulated on the path
        xs = [torch.randn(B, T, H * d, generator=gen, device=device) for _ in range(3)]
        out["x_qkv"] = torch.stack(xs, 0).to(td)
    else:
        for n in ("q", "k", "v"):
            out[n] = torch.randn(B, T, H, d, generator=gen, device=device).mul_(cfg.qkv_scale).to(td)
    x = torch.randn(B, T, H, d, generator=gen, device=device).add_(cfg.gate_mu)
    out["log_alpha"] = gate_from_normal(x).to(td)
    if cfg.adaln:
        out["ada_scale"] = torch.randn(H * d, generator=gen, device=device) * 0.1
        out["ada_shift"] = torch.randn(H * d, generator=gen, device=device) * 0.1
        out["ada_out_scale"] = cfg.qkv_scale
    out["w"] = conv_weight(H * d, cfg.conv_perturb, gen, device)
    return out


def block_inputs(B: int, T: int, C: int, seed: int = 0, device="cpu", conv_perturb: float = 0.01) -> dict:
    """Seeded synthetic inputs and weights of one DiG block (no trained weights
    exist here): the residual stream x [B, T, C] ~ N(0, 1) (bf16), the
    conditioning c [B, C] ~ N(0, 1) (fp32), the linear weights ~ N(0, 1/fan_in)
    (bf16; the adaLN regression ~ N(0, 0.25/C) so that shifts, scales and gates
    stay O(0.5)), biases ~ N(0, 0.02^2) (fp32) and the conv near identity."""
    g = _gen(seed, device)

    def w(rows, cols, s=1.0):
        return (torch.randn(rows, cols, generator=g, device=device) * (s / math.sqrt(cols))).to(torch.bfloat16)

    def bias(n):
        return torch.randn(n, generator=g, device=device) * 0.02

    x = torch.randn(B, T, C, generator=g, device=device).to(torch.bfloat16)
    c = torch.randn(B, C, generator=g, device=device)
    out = {"x": x, "c": c,
           "w_ada": w(6 * C, C, 0.5), "b_ada": bias(6 * C),
           "w_in": w(4 * C, C), "b_in": bias(4 * C),
           "w_out": w(C, C), "b_out": bias(C),
           "w_ff1": w(4 * C, C), "b_ff1": bias(4 * C),
           "w_ff2": w(C, 4 * C), "b_ff2": bias(C)}
    out["w_conv"] = conv_weight(C, conv_perturb, g, device)
    return out
