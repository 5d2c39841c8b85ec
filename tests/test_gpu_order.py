"""GPU parity of the table scan orders: gla_fwd_ordered, gla_bwd_ordered and
dig_gather_rows through the C ABI, against the fp64 oracle's table path
(oracle.gla_fwd / gla_bwd with `order`, pinned in test_oracle_orders.py).

The GPU side takes its tables from gated_linear_attention_gla_amd.scan_orders,
the oracle side builds its own (oracle.zigzag_order); both are checked
against the same hand-listed orders on the CPU.  Tolerances as for the
grid orders (helpers.py); the table of a grid order reproduces that
direction bit for bit, and so does the left-to-right scan of the arranged
sequence.
"""
import math

import numpy as np
import pytest
import torch

from gated_linear_attention_gla_amd import binding as dg
from gated_linear_attention_gla_amd import inputs as gen
from gated_linear_attention_gla_amd import scan_orders as so
from helpers import TOL_BF16, TOL_F32, assert_o_close, assert_state_close
from test_gpu_bwd import check as check_bwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dg.lib()
    yield
    torch.cuda.synchronize()


def dev(t):
    return None if t is None else t.to("cuda")


def table(order):
    return so.to_device(order, "cuda")


def fwd(x, order=None, grid=None, direction=None, chunk=0, s0=None):
    o, sf = dg.gla_fwd(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["log_alpha"]), grid, direction,
                       chunk=chunk, s0=dev(s0), order=None if order is None else table(order))
    torch.cuda.synchronize()
    return o.cpu(), sf.cpu()


def bitwise(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("case", [
    # (B, H, gh, gw, d, dtype, chunk)
    (2, 3, 11, 9, 72, "bf16", 64),
    (1, 8, 64, 64, 64, "bf16", 64),     # eight segments per scan (look-back)
    (6, 16, 32, 32, 64, "bf16", 32),    # the two-segment split
    (2, 2, 10, 20, 32, "bf16", 128),    # 128-token chunks, ragged tail
    (8, 16, 32, 32, 32, "bf16", 128),   # 128-token chunks, the two-segment split
    (1, 2, 8, 8, 16, "f32", 16),
], ids=lambda c: "x".join(map(str, c)))
def test_fwd_table_of_a_grid_order_is_that_direction(case):
    B, H, gh, gw, d, dt, chunk = case
    x = gen.gla_inputs(B, gh * gw, H, d, d, dtype=dt, seed=60 + d, qkv_scale=1 / math.sqrt(d))
    s0 = torch.randn(B, H, d, d, generator=torch.Generator().manual_seed(6)) * 0.5
    for direction in gen.DIRS:
        a = fwd(x, grid=(gh, gw), direction=direction, chunk=chunk, s0=s0)
        b = fwd(x, order=so.grid_order(direction, gh, gw), chunk=chunk, s0=s0)
        assert bitwise(a[0], b[0]) and bitwise(a[1], b[1]), direction


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_fwd_zigzag_vs_oracle(orc, dt):
    B, H, gh, gw, d = (2, 2, 10, 13, 64) if dt == "bf16" else (1, 2, 6, 7, 16)
    x = gen.gla_inputs(B, gh * gw, H, d, d, dtype=dt, seed=61, qkv_scale=1 / math.sqrt(d))
    s0 = torch.randn(B, H, d, d, generator=torch.Generator().manual_seed(7)) * 0.5
    tol = TOL_BF16 if dt == "bf16" else TOL_F32
    for j in range(8):
        o, sf = fwd(x, order=so.zigzag(j, gh, gw), s0=s0)
        ro, rs = orc.gla_fwd(x["q"], x["k"], x["v"], x["log_alpha"], None, None, s0=s0.double().numpy(),
                             order=orc.zigzag_order(j, gh, gw))
        assert_o_close(o, ro, tol, f"zigzag S_{j} o")
        assert_state_close(sf, rs, tol, f"zigzag S_{j} s_final")


def test_fwd_random_permutation_segmented_vs_oracle(orc):
    """A random order through the segmented scan (several workgroups per
    scan, look-back), every head."""
    B, H, gh, gw, d = 1, 8, 48, 48, 64
    T = gh * gw
    x = gen.gla_inputs(B, T, H, d, d, seed=62, qkv_scale=1 / 8)
    perm = np.random.default_rng(62).permutation(T)
    o, sf = fwd(x, order=perm)
    ro, rs = orc.gla_fwd(x["q"], x["k"], x["v"], x["log_alpha"], None, None, order=perm)
    assert_o_close(o, ro, TOL_BF16, "random order o")
    assert_state_close(sf, rs, TOL_BF16, "random order s_final")


def test_fwd_random_permutation_chunk128_vs_oracle(orc):
    """A random order with 128-token chunks (32-channel heads) through the
    eight-segment look-back."""
    B, H, gh, gw, d = 1, 2, 64, 64, 32
    T = gh * gw
    x = gen.gla_inputs(B, T, H, d, d, seed=63, qkv_scale=0.17)
    perm = np.random.default_rng(63).permutation(T)
    o, sf = fwd(x, order=perm, chunk=128)
    ro, rs = orc.gla_fwd(x["q"], x["k"], x["v"], x["log_alpha"], None, None, order=perm)
    assert_o_close(o, ro, TOL_BF16, "random order o")
    assert_state_close(sf, rs, TOL_BF16, "random order s_final")


def _gather(t, order):
    """[B, T, H, d] -> arranged in `order`, through dig_gather_rows on the GPU."""
    B, T, H, d = t.shape
    y = dg.gather_rows(t.reshape(B, T, H * d).to("cuda").contiguous(), table(order))
    return y.reshape(B, T, H, d)


def test_fwd_table_is_the_arranged_l2r_scan():
    B, H, gh, gw, d = 2, 4, 16, 20, 64
    T = gh * gw
    x = gen.gla_inputs(B, T, H, d, d, seed=63, qkv_scale=1 / 8)
    order = so.zigzag(4, gh, gw)
    o1, s1 = fwd(x, order=order)
    xa = {n: _gather(x[n], order) for n in ("q", "k", "v", "log_alpha")}
    o2, s2 = dg.gla_fwd(xa["q"], xa["k"], xa["v"], xa["log_alpha"], (1, T), "l2r")
    torch.cuda.synchronize()
    assert bitwise(o1, o2.cpu()) and bitwise(s1, s2.cpu())


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gather_rows_exact(dtype):
    B, T, C = 3, 77, 48
    x = torch.randn(B, T, C, generator=torch.Generator().manual_seed(64)).to(dtype)
    order = so.zigzag(2, 7, 11)
    y = dg.gather_rows(x.to("cuda"), table(order)).cpu()
    assert torch.equal(y, x[:, torch.as_tensor(order.astype(np.int64))])
    back = dg.gather_rows(y.to("cuda"), table(so.inverse(order))).cpu()
    assert torch.equal(back, x)
    bad = order.copy()
    bad[5], bad[9] = -1, T
    z = dg.gather_rows(x.to("cuda"), table(bad)).cpu()
    assert torch.all(z[:, 5] == 0) and torch.all(z[:, 9] == 0)
    keep = [p for p in range(T) if p not in (5, 9)]
    assert torch.equal(z[:, keep], x[:, torch.as_tensor(order.astype(np.int64))][:, keep])


# ------------------------------------------------------------------ backward

def bwd_case(B, T, H, d, seed):
    x = gen.gla_inputs(B, T, H, d, d, dtype="bf16", seed=seed, qkv_scale=1.0 / math.sqrt(d))
    g = torch.Generator().manual_seed(seed + 1000)
    x["do"] = torch.randn(B, T, H, d, generator=g).to(torch.bfloat16)
    x["dsf"] = torch.randn(B, H, d, d, generator=g) * 0.5
    x["s0"] = torch.randn(B, H, d, d, generator=g) * 0.5
    return x


def bwd(x, order=None, grid=None, direction=None, chunk=0):
    out = dg.gla_bwd(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["log_alpha"]), grid, direction, dev(x["do"]),
                     chunk=chunk, s0=dev(x["s0"]), ds_final=dev(x["dsf"]),
                     order=None if order is None else table(order))
    torch.cuda.synchronize()
    return tuple(t.cpu() for t in out)


def test_bwd_table_of_a_grid_order_is_that_direction():
    gh, gw = 11, 9
    x = bwd_case(2, gh * gw, 3, 72, seed=65)
    for direction in gen.DIRS:
        a = bwd(x, grid=(gh, gw), direction=direction)
        b = bwd(x, order=so.grid_order(direction, gh, gw))
        for u, w in zip(a, b):
            assert bitwise(u, w), direction


def _oracle_bwd(orc, x, order):
    f = lambda t: None if t is None else t.double().numpy()
    return orc.gla_bwd(x["q"], x["k"], x["v"], x["log_alpha"], None, None, x["do"], ds_final=f(x["dsf"]),
                       s0=f(x["s0"]), order=order)


@pytest.mark.parametrize("j", [0, 3, 5, 6])
def test_bwd_zigzag_vs_oracle(orc, j):
    gh, gw = 10, 13
    x = bwd_case(1, gh * gw, 2, 64, seed=66 + j)
    got = bwd(x, order=so.zigzag(j, gh, gw))
    check_bwd(got, _oracle_bwd(orc, x, orc.zigzag_order(j, gh, gw)), f"zigzag S_{j}", x)


def test_bwd_random_permutation_several_chunks_per_workgroup(orc):
    """Enough chunks that every workgroup of the persistent chunk kernel runs
    several (its table entries are loaded one chunk ahead)."""
    B, H, gh, gw, d = 8, 8, 32, 32, 64
    T = gh * gw
    x = bwd_case(B, T, H, d, seed=70)
    perm = np.random.default_rng(70).permutation(T)
    got = bwd(x, order=perm)
    check_bwd(got, _oracle_bwd(orc, x, perm), "random order", x)


def test_c2_zigzag_full(orc):
    """The C2 workload (DiG-XL/2 at 1024 px) over zigzag scans, forward and
    backward, every (batch, head) unit."""
    cfg = gen.CONFIGS["C2"]
    x = gen.make_inputs("C2")
    o, sf = fwd(x, order=so.zigzag(1, cfg.gh, cfg.gw), chunk=cfg.chunk)
    ro, rs = orc.gla_fwd(x["q"], x["k"], x["v"], x["log_alpha"], None, None,
                         order=orc.zigzag_order(1, cfg.gh, cfg.gw))
    assert_o_close(o, ro, TOL_BF16, "C2 zigzag o")
    assert_state_close(sf, rs, TOL_BF16, "C2 zigzag s")
    g = torch.Generator().manual_seed(cfg.seed + 77)
    x["do"] = torch.randn(cfg.B, cfg.T, cfg.H, cfg.d, generator=g).to(torch.bfloat16)
    x["dsf"] = None
    x["s0"] = None
    got = bwd(x, order=so.zigzag(6, cfg.gh, cfg.gw), chunk=cfg.chunk)
    check_bwd(got, _oracle_bwd(orc, x, orc.zigzag_order(6, cfg.gh, cfg.gw)), "C2 zigzag bwd", x)
