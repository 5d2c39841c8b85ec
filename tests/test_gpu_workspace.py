"""gla_fwd's workspace on the GPU: a workspace that was never zero-filled,
reuse across calls and shapes, and replays of a captured graph.

The forward's workspace holds cyclic ticket counters, launch-tagged flags and
the published segment states.  These tests fill it with a byte pattern
before the first call, reuse it across shapes and directions, and capture the
call into a graph whose replays see new inputs, each time comparing every
output with the fp64 oracle (2e-2 normwise, helpers.py) and checking that no
wait between workgroups gave up (gla_fwd_workspace_status).
"""
import numpy as np
import pytest
import torch

from gated_linear_attention_gla_amd import binding as dg
from gated_linear_attention_gla_amd import inputs as gen
from helpers import TOL_BF16, assert_o_close, assert_state_close

pytestmark = pytest.mark.gpu

# (B, H, gh, gw, d): two segments per scan (the pipelined split) and eight
# segments per scan (the look-back over published aggregates)
SEGMENTED = [(6, 16, 32, 32, 64), (1, 8, 64, 64, 72)]
# one segment per scan (192 scans of 4 chunks): the work comes from the
# launch index and the kernel touches no workspace word
SINGLE = (16, 12, 16, 16, 64)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dg.lib()
    yield
    torch.cuda.synchronize()


def _inputs(shape, seed):
    B, H, gh, gw, d = shape
    return gen.gla_inputs(B, gh * gw, H, d, d, dtype="bf16", seed=seed, qkv_scale=1 / np.sqrt(d))


def _check(orc, x, o, sf, grid, direction, what):
    ro, rs = orc.gla_fwd(x["q"], x["k"], x["v"], x["log_alpha"], grid, direction)
    assert_o_close(o.cpu(), ro, TOL_BF16, f"{what} o")
    assert_state_close(sf.cpu(), rs, TOL_BF16, f"{what} s_final")


def test_workspace_not_zero_filled(orc):
    """A workspace holding 0x5A bytes (ticket counters far above the grid,
    flags of no epoch, a non-zero error word) serves both segmented layouts
    in turn, twice each, with every output right.  The error word is part of
    the header the pattern filled, so the first status check reports it (and
    clears it); after that every call must leave it clear."""
    n = max(dg.workspace_bytes(dg.DIG_BF16, s[0], s[2] * s[3], s[1], s[4], s[4]) for s in SEGMENTED)
    ws = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    assert ws.data_ptr() % 256 == 0
    for i, (shape, direction) in enumerate([(SEGMENTED[0], "l2r"), (SEGMENTED[1], "b2t"),
                                            (SEGMENTED[0], "t2b"), (SEGMENTED[1], "r2l"), (SINGLE, "b2t")]):
        x = _inputs(shape, 90 + i)
        grid = (shape[2], shape[3])
        xd = {k: x[k].to("cuda") for k in ("q", "k", "v", "log_alpha")}
        print(f"[ws] call {i}: shape {shape} {direction}", flush=True)
        o, sf = dg.gla_fwd(xd["q"], xd["k"], xd["v"], xd["log_alpha"], grid, direction, workspace=ws)
        torch.cuda.synchronize()
        _check(orc, x, o, sf, grid, direction, f"call {i} {shape} {direction}")
        if i == 0:
            with pytest.raises(dg.DigError, match="0x5a5a5a5a"):
                dg.workspace_status(ws)
        dg.workspace_status(ws)


@pytest.mark.parametrize("shape", SEGMENTED + [SINGLE], ids=lambda s: "x".join(map(str, s)))
def test_graph_replays_see_new_inputs(orc, shape):
    """gla_fwd captured into a graph: every replay carries the same launch
    tag, so the flags of the previous replay must not read as published.
    Each replay gets new inputs; eager calls on the same workspace run in
    between; every replay is compared with the oracle."""
    B, H, gh, gw, d = shape
    T, grid, direction = gh * gw, (gh, gw), "t2b"
    dev = torch.device("cuda")
    x0 = _inputs(shape, 100)
    xd = {k: x0[k].to(dev).clone() for k in ("q", "k", "v", "log_alpha")}
    o = torch.empty(B, T, H, d, dtype=torch.bfloat16, device=dev)
    sf = torch.empty(B, H, d, d, dtype=torch.float32, device=dev)
    ws = torch.zeros(dg.workspace_bytes(dg.DIG_BF16, B, T, H, d, d), dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dg.gla_fwd(xd["q"], xd["k"], xd["v"], xd["log_alpha"], grid, direction, out=o, s_final=sf, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dg.gla_fwd(xd["q"], xd["k"], xd["v"], xd["log_alpha"], grid, direction, out=o, s_final=sf, workspace=ws)
    torch.cuda.synchronize()
    for r in range(4):
        x = _inputs(shape, 101 + r)
        for k in xd:
            xd[k].copy_(x[k].to(dev))
        torch.cuda.synchronize()
        print(f"[graph] {shape} replay {r}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        _check(orc, x, o, sf, grid, direction, f"replay {r}")
        # eager work on the same workspace between replays (new launch tags)
        oe, sfe = dg.gla_fwd(xd["q"], xd["k"], xd["v"], xd["log_alpha"], grid, "l2r", workspace=ws)
        torch.cuda.synchronize()
        _check(orc, x, oe, sfe, grid, "l2r", f"eager after replay {r}")
    dg.workspace_status(ws)
