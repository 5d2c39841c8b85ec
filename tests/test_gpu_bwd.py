"""GPU parity of the GLA backward (gla_bwd, through the C ABI) against the fp64
CPU oracle's reverse-mode derivative (oracle.gla_bwd, itself pinned by finite
differences and autograd in test_oracle_pins.py).

Same seeded tensors on both sides; bf16 inputs and gradient outputs, fp32
d log alpha and ds0.  Tolerance: normwise per (batch, head) slice, 2e-2 (as
the bf16 forward: bf16 operands, fp32 accumulation, and here also bf16 chunk
states), see helpers.py.
"""
import math

import numpy as np
import pytest
import torch

from gated_linear_attention_gla_amd import binding as dg
from gated_linear_attention_gla_amd import inputs as gen
from helpers import TOL_BF16, assert_o_close, assert_state_close, to_np

pytestmark = pytest.mark.gpu
DIRS = gen.DIRS
NAMES = ("dq", "dk", "dv", "dlog_alpha")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dg.lib()
    yield
    torch.cuda.synchronize()


def dev(t):
    return None if t is None else t.to("cuda")


def make_case(B, T, H, dk, dv, seed, gate_div=16.0, gate_mu=0.0, with_state=True):
    x = gen.gla_inputs(B, T, H, dk, dv, dtype="bf16", seed=seed, qkv_scale=1.0 / math.sqrt(dk),
                       gate_mu=gate_mu, gate_div=gate_div)
    g = torch.Generator().manual_seed(seed + 1000)
    x["do"] = torch.randn(B, T, H, dv, generator=g).to(torch.bfloat16)
    x["dsf"] = torch.randn(B, H, dk, dv, generator=g) * 0.5 if with_state else None
    x["s0"] = torch.randn(B, H, dk, dv, generator=g) * 0.5 if with_state else None
    return x


def run_bwd(x, grid, direction, chunk=0):
    out = dg.gla_bwd(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["log_alpha"]), grid, direction,
                     dev(x["do"]), chunk=chunk, s0=dev(x["s0"]), ds_final=dev(x["dsf"]))
    torch.cuda.synchronize()
    return tuple(t.cpu() for t in out)


def oracle_bwd(orc, x, grid, direction):
    f = lambda t: None if t is None else t.double().numpy()
    q, k, v, g, do, dsf, s0 = (x["q"], x["k"], x["v"], x["log_alpha"], x["do"], x["dsf"], x["s0"])
    return orc.gla_bwd(q, k, v, g, grid, direction, do, ds_final=f(dsf), s0=f(s0))


def check(got, ref, tag, x=None):
    """dq, dk, dv, ds0: normwise per slice (and per 64-token block).
    dlog_alpha is the chunk sum of q (.) dq - k (.) dk (plus the state term):
    its rounding is relative to those summands, which cancel where the true
    value vanishes (alpha -> 0 gives exactly 0), so its gated scale is the
    larger of |dlog_alpha| and |q (.) dq| per (batch, head) slice.  The error
    against |dlog_alpha| alone is printed beside it (not gated), so the gap
    between the two scales is visible in the test log."""
    for n, a, r in zip(NAMES[:3], got[:3], ref[:3]):
        assert_o_close(a, r, TOL_BF16, f"{tag} {n}")
    assert_state_close(got[4], ref[4], TOL_BF16, f"{tag} ds0")
    gq = to_np(x["q"])
    a, r = to_np(got[3]), ref[3]
    scale = np.maximum(np.max(np.abs(r), axis=(1, 3)), np.max(np.abs(gq * ref[0]), axis=(1, 3)))
    num = np.max(np.abs(a - r), axis=(1, 3))
    e = num / np.maximum(scale, 1e-30)
    e_self = num / np.maximum(np.max(np.abs(r), axis=(1, 3)), 1e-30)
    print(f"[dlog_alpha] {tag}: err/max(|dlog_alpha|, |q dq|) = {e.max():.3e}, "
          f"err/|dlog_alpha| = {e_self.max():.3e}", flush=True)
    assert np.all(np.isfinite(a)), f"{tag} dlog_alpha: non-finite"
    assert e.max() <= TOL_BF16, f"{tag} dlog_alpha: rel err {e.max():.3e} > {TOL_BF16:g}"


SHAPES = [
    # (B, H, gh, gw, dk, dv, chunk)
    (1, 2, 8, 8, 64, 64, 64),      # one chunk
    (2, 3, 11, 9, 72, 72, 64),     # 80-channel tiles, ragged second chunk
    (1, 2, 10, 13, 32, 48, 32),    # dk != dv, ragged, 32-token chunks
    (1, 2, 9, 7, 128, 128, 32),    # 128 channels
    (1, 1, 12, 12, 96, 96, 0),     # 96 channels, automatic chunk (32)
    (1, 2, 6, 6, 16, 16, 16),      # 32-channel tiles, 16-token chunks
    (1, 2, 5, 9, 72, 72, 16),      # ragged 16-token chunks
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_shapes_vs_oracle(orc, shape):
    B, H, gh, gw, dk, dv, chunk = shape
    x = make_case(B, gh * gw, H, dk, dv, seed=40 + dk + gh)
    for d in DIRS:
        check(run_bwd(x, (gh, gw), d, chunk), oracle_bwd(orc, x, (gh, gw), d), f"{shape} {d}", x)


def test_bwd_without_state_and_final_gradient(orc):
    x = make_case(1, 80, 2, 64, 64, seed=51, with_state=False)
    got = run_bwd(x, (8, 10), "t2b")
    check(got, oracle_bwd(orc, x, (8, 10), "t2b"), "no s0/ds_final", x)


@pytest.mark.parametrize("case", ["all_zero_alpha", "mixed_extreme", "alpha_one", "long_memory"])
def test_bwd_gate_extremes(orc, case):
    """alpha -> 0, chunks mixing extreme and mild gates (the exact-exponent
    path), alpha == 1 and very slow decay."""
    gh, gw = 10, 16
    x = make_case(2, gh * gw, 2, 64, 64, seed=52)
    g = x["log_alpha"].float()
    if case == "all_zero_alpha":
        g = torch.full_like(g, -1e4)
    elif case == "mixed_extreme":
        g[:, 40:44] = -1e4
        g[:, 100, :, :8] = -300.0
    elif case == "alpha_one":
        g = torch.zeros_like(g)
    elif case == "long_memory":
        g = g / 64.0
    x["log_alpha"] = g.to(torch.bfloat16)
    for d in ("l2r", "b2t"):
        check(run_bwd(x, (gh, gw), d), oracle_bwd(orc, x, (gh, gw), d), f"{case} {d}", x)


def test_bwd_deterministic():
    x = make_case(2, 64 * 5, 4, 72, 72, seed=53)
    a = run_bwd(x, (16, 20), "r2l")
    b = run_bwd(x, (16, 20), "r2l")
    for u, w in zip(a, b):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u.view(torch.int32),
                           w.view(torch.int16) if w.dtype == torch.bfloat16 else w.view(torch.int32))


def test_bwd_gradient_of_forward_loss(orc):
    """gla_bwd's gradients against the change of the GPU forward's loss along a
    random direction (a directional derivative, independent of the oracle)."""
    gh, gw = 8, 12
    x = make_case(1, gh * gw, 2, 64, 64, seed=54)
    got = run_bwd(x, (gh, gw), "l2r")
    # L(q + e u) - L(q - e u) over 2e ~ <dq, u>, with the fp64 oracle forward (the GPU
    # forward's bf16 rounding would swamp a small step)
    u = torch.randn(x["q"].shape, generator=torch.Generator().manual_seed(9), dtype=torch.float64)
    eps = 1e-3
    f64 = lambda t: t.double().numpy()

    def loss(qv):
        o, sf = orc.gla_fwd(qv, f64(x["k"]), f64(x["v"]), f64(x["log_alpha"]), (gh, gw), "l2r", s0=f64(x["s0"]))
        return float(np.sum(o * f64(x["do"])) + np.sum(sf * f64(x["dsf"])))

    q0 = f64(x["q"])
    dd = (loss(q0 + eps * u.numpy()) - loss(q0 - eps * u.numpy())) / (2 * eps)
    gd = float(np.sum(got[0].double().numpy() * u.numpy()))
    assert abs(gd - dd) <= 2e-2 * max(abs(dd), 1e-6), (gd, dd)


def _full_bwd(orc, key, directions):
    """A named workload at full size, every (batch, head) unit compared."""
    cfg = gen.CONFIGS[key]
    x = gen.make_inputs(key)
    g = torch.Generator().manual_seed(cfg.seed + 77)
    x["do"] = torch.randn(cfg.B, cfg.T, cfg.H, cfg.d, generator=g).to(torch.bfloat16)
    x["dsf"] = None
    x["s0"] = None
    for d in directions:
        got = run_bwd(x, (cfg.gh, cfg.gw), d, chunk=cfg.chunk)
        check(got, oracle_bwd(orc, x, (cfg.gh, cfg.gw), d), f"{key} {d}", x)


def test_bwd_c1_full(orc):
    _full_bwd(orc, "C1", DIRS)


def test_bwd_c2_full(orc):
    _full_bwd(orc, "C2", DIRS)


def test_bwd_c4_shape_full(orc):
    """The 2048-pixel shape (B = 1, H = 16, 128 x 128 tokens, d = 72, long-memory
    gates): 16 scans of 256 chunks each, so the scans are the longest the
    workloads have and every workgroup of the persistent chunk kernel runs a
    long run of chunks; every unit compared, with s0 and dS_final."""
    x = make_case(1, 128 * 128, 16, 72, 72, seed=88, gate_mu=2.0)
    for d in ("l2r", "b2t"):
        check(run_bwd(x, (128, 128), d), oracle_bwd(orc, x, (128, 128), d), f"C4 shape {d}", x)
