"""gla_fwd_noalloc (the allocation-free entry point, through the C ABI)
against gla_fwd with a workspace of its own: two calls in a row, the second
with a smaller input, each bitwise equal to gla_fwd and within 2e-2 of the
fp64 oracle (helpers.py), plus an input too large for the fixed scratch,
rejected with DIG_EWORKSPACE and nothing queued."""
import ctypes

import numpy as np
import pytest
import torch

from gated_linear_attention_gla_amd import binding as dg
from gated_linear_attention_gla_amd import inputs as gen
from helpers import TOL_BF16, assert_o_close, assert_state_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dg.lib()
    yield
    torch.cuda.synchronize()


def _bitwise(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


# (B, H, gh, gw, d, direction): the DiG-XL/2 workload at 1024 px (two
# segments per scan), then a smaller one with eight segments per scan, then
# one segment per scan
CALLS = [(8, 16, 64, 64, 72, "t2b"), (1, 8, 64, 64, 72, "b2t"), (32, 6, 16, 16, 64, "r2l")]


def test_noalloc_matches_gla_fwd_on_consecutive_calls(orc):
    dev = torch.device("cuda")
    for i, (B, H, gh, gw, d, direction) in enumerate(CALLS):
        T = gh * gw
        x = gen.gla_inputs(B, T, H, d, d, dtype="bf16", seed=110 + i, qkv_scale=1 / np.sqrt(d),
                           gate_mu=2.0 if d == 72 else 0.0)
        xd = {k: x[k].to(dev) for k in ("q", "k", "v", "log_alpha")}
        o = torch.empty(B, T, H, d, dtype=torch.bfloat16, device=dev)
        sf = torch.empty(B, H, d, d, dtype=torch.float32, device=dev)
        print(f"[noalloc] call {i}: B={B} H={H} {gh}x{gw} d={d} {direction}", flush=True)
        dg.gla_fwd_noalloc(xd["q"], xd["k"], xd["v"], xd["log_alpha"], (gh, gw), direction, out=o, s_final=sf)
        ws = torch.zeros(dg.workspace_bytes(dg.DIG_BF16, B, T, H, d, d), dtype=torch.uint8, device=dev)
        o2, sf2 = dg.gla_fwd(xd["q"], xd["k"], xd["v"], xd["log_alpha"], (gh, gw), direction, workspace=ws)
        torch.cuda.synchronize()
        assert _bitwise(o, o2) and _bitwise(sf, sf2), f"call {i}: gla_fwd_noalloc differs from gla_fwd"
        ro, rs = orc.gla_fwd(x["q"], x["k"], x["v"], x["log_alpha"], (gh, gw), direction)
        assert_o_close(o.cpu(), ro, TOL_BF16, f"call {i} o")
        assert_state_close(sf.cpu(), rs, TOL_BF16, f"call {i} s_final")


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """Sixteen scans of 128 channels over 128 x 128 tokens, each split into
    sixteen segments whose published 128 x 128 fp32 aggregates need more
    workspace than the fixed 16 MiB scratch holds: refused before any
    launch (the pointers are never dereferenced)."""
    L = dg.lib()
    B, H, T, d = 1, 16, 128 * 128, 128
    assert L.gla_fwd_workspace_size(dg.DIG_BF16, B, T, H, d, d, 0) > (16 << 20)
    p = ctypes.c_void_p(1 << 12)
    rc = L.gla_fwd_noalloc(p, p, p, p, dg.DIG_BF16, T * H * d, H * d, d, T * H * d, H * d, d,
                           B, T, H, d, d, 128, 128, 0, 0, None, ctypes.c_void_p(1 << 13), T * H * d, H * d, d,
                           None, None)
    assert rc == -2, rc
    assert b"scratch" in L.dig_last_error()
