"""GPU parity of the DiG block forward (dig_block_fwd, through the C ABI)
against the fp64 oracle (oracle.block_fwd, pinned in test_oracle_block.py).

The GPU rounds every intermediate to bf16 (the modulated rows, the four
projections, the GLA output, the out-projection, the residual after the
mixer, the FFN's hidden layer and output, the residual after the FFN) with
fp32 accumulation inside each product, so about eight bf16 roundings
(2^-9 relative each) stand between input and output: the block output is
compared element by element at 2e-2 of its largest magnitude per batch
element (max|y - ref| / max|ref|, as the bf16 GLA), and its update y - x,
which carries all of that rounding, at 4e-2 of the update's largest
magnitude.  Zero adaLN weights with the identity conv give the identity map
exactly.
"""
import numpy as np
import pytest
import torch

from gated_linear_attention_gla_amd import binding as dg
from gated_linear_attention_gla_amd import inputs as gen

pytestmark = pytest.mark.gpu
TOL_Y, TOL_UPDATE = 2e-2, 4e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dg.lib()
    yield
    torch.cuda.synchronize()


def _run(x, grid, direction, H):
    w = {n: x[n].to("cuda").contiguous() for n in dg.BLOCK_WEIGHTS}
    y = dg.block_fwd(x["x"].to("cuda"), x["c"].to("cuda"), w, grid, direction, H)
    torch.cuda.synchronize()
    return y.cpu()


def _check(y, ref, x, what):
    y = y.double().numpy()
    x0 = x["x"].double().numpy()
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    for b in range(y.shape[0]):
        err = np.abs(y[b] - ref[b])
        e = err.max() / np.abs(ref[b]).max()
        u = err.max() / np.abs(ref[b] - x0[b]).max()
        assert e <= TOL_Y, f"{what} b={b}: y rel err {e:.3e}"
        assert u <= TOL_UPDATE, f"{what} b={b}: update rel err {u:.3e}"


@pytest.mark.parametrize("shape", [(2, 8, 8, 128, 2), (1, 11, 9, 144, 2), (2, 6, 10, 256, 4), (1, 6, 7, 256, 2),
                                   (2, 4, 5, 16, 2), (17, 4, 5, 16, 2)],
                         ids=lambda s: "x".join(map(str, s)))
def test_block_vs_oracle(orc, shape):
    """Small shapes in all four directions: ragged chunks, 72-channel heads,
    128-channel heads (32-token chunks) and 8-channel heads; with 17 batch
    elements the conditioning product (17 rows) runs on the MFMA tile with
    fp32 output instead of the few-row kernel."""
    B, gh, gw, C, H = shape
    x = gen.block_inputs(B, gh * gw, C, seed=80 + C)
    w = {n: x[n] for n in orc.BLOCK_WEIGHTS}
    for d in gen.DIRS:
        _check(_run(x, (gh, gw), d, H), orc.block_fwd(x["x"], x["c"], w, (gh, gw), d, H=H), x, f"{shape} {d}")


def test_block_adaln_zero_is_identity():
    x = gen.block_inputs(2, 64, 128, seed=81, conv_perturb=0.0)
    x["w_ada"].zero_()
    x["b_ada"].zero_()
    for d in gen.DIRS:
        assert torch.equal(_run(x, (8, 8), d, 2), x["x"]), d


def test_block_c2_shape(orc):
    """The DiG-XL/2 block at 1024 px (B=8, 64x64 tokens, C=1152, 16 heads):
    the GPU and the oracle over the whole batch."""
    B, gh, gw, C, H = 8, 64, 64, 1152, 16
    x = gen.block_inputs(B, gh * gw, C, seed=82)
    y = _run(x, (gh, gw), "t2b", H)
    w = {n: x[n] for n in orc.BLOCK_WEIGHTS}
    _check(y, orc.block_fwd(x["x"], x["c"], w, (gh, gw), "t2b", H=H), x, "C2 block")


@pytest.mark.parametrize("shape", [(300, 200, 256), (256, 256, 64), (1, 8, 8), (777, 136, 1160),
                                   (4096, 1152, 1152), (513, 4608, 72), (32768, 1152, 8), (8, 6912, 1152),
                                   (16, 40, 4608), (17, 264, 16)],
                         ids=lambda s: "x".join(map(str, s)))
def test_linear_vs_fp64(shape):
    """dig_linear (the block's products, no epilogue) against an fp64
    product of the same bf16 operands, element by element: ragged M, N and
    K tails, a single row, both feature-tile widths, K of one step, and the
    few-row kernel (M <= 16: the conditioning product's shape)."""
    M, N, K = shape
    g = torch.Generator().manual_seed(83 + M + N + K)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16)
    w = (torch.randn(N, K, generator=g) / np.sqrt(K)).to(torch.bfloat16)
    y = dg.linear(x.to("cuda"), w.to("cuda")).cpu().double()
    ref = x.double() @ w.double().T
    # fp32 accumulation of bf16 products, then one bf16 rounding (2^-9 of |y|)
    err = (y - ref).abs()
    bound = 2.0 ** -8 * ref.abs() + 1e-5 * (x.double().abs() @ w.double().abs().T)
    assert bool((err <= bound).all()), float((err - bound).max())


def test_block_workspace_reused_across_shapes(orc):
    """One workspace, filled with a byte pattern first, serves two shapes in
    turn (A, B, A): the GLA's counters sit at a shape-dependent offset inside
    it, and every result still matches the oracle."""
    xa = gen.block_inputs(2, 8 * 12, 128, seed=84)
    xb = gen.block_inputs(1, 11 * 9, 144, seed=85)
    n = max(dg.lib().dig_block_workspace_size(2, 96, 128, 2), dg.lib().dig_block_workspace_size(1, 99, 144, 2))
    ws = torch.full((int(n),), 0x5A, dtype=torch.uint8, device="cuda")
    assert ws.data_ptr() % 256 == 0

    def run(x, grid, d):
        w = {k: x[k].to("cuda").contiguous() for k in dg.BLOCK_WEIGHTS}
        y = dg.block_fwd(x["x"].to("cuda"), x["c"].to("cuda"), w, grid, d, 2, workspace=ws)
        torch.cuda.synchronize()
        return y.cpu()

    for x, grid, d in ((xa, (8, 12), "r2l"), (xb, (11, 9), "t2b"), (xa, (8, 12), "b2t")):
        w = {k: x[k] for k in orc.BLOCK_WEIGHTS}
        _check(run(x, grid, d), orc.block_fwd(x["x"], x["c"], w, grid, d, H=2), x, f"reused workspace {grid} {d}")
