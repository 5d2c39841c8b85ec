"""C-ABI contract tests that need no GPU: the library loads, exports every
function include/dig_gla.h declares, and rejects invalid arguments with
DIG_EINVAL and a message before making any HIP call."""
import ctypes
import os
import re

import pytest

from gated_linear_attention_gla_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", txt, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    return binding.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert {"gla_fwd", "gla_fwd_workspace_size", "srem_dwconv", "srem_remap", "dig_adaln_modulate",
            "dig_last_error", "dig_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_version(L):
    assert b"gfx950" in L.dig_version()


def _gla(L, **kw):
    a = dict(q=16, k=32, v=48, g=64, dtype=1, qk=(4096 * 8 * 8, 64, 8), vs=(4096 * 8 * 8, 64, 8),
             B=1, T=64, H=8, dk=8, dv=8, gh=8, gw=8, dir=0, chunk=0, s0=None, o=128,
             os=(4096 * 8 * 8, 64, 8), sf=None, ws=None, wsb=0)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.gla_fwd(p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), a["dtype"], *a["qk"], *a["vs"],
                     a["B"], a["T"], a["H"], a["dk"], a["dv"], a["gh"], a["gw"], a["dir"], a["chunk"],
                     p(a["s0"]), p(a["o"]), *a["os"], p(a["sf"]), p(a["ws"]), a["wsb"], None)


@pytest.mark.parametrize("bad", [
    dict(q=None), dict(o=None), dict(B=0), dict(T=-1), dict(dk=0), dict(dv=136),
    dict(gh=7), dict(dir=4), dict(dtype=7), dict(chunk=48), dict(dk=12, dv=12),
    dict(q=18), dict(qk=(4096 * 64, 60, 8)), dict(o=16), dict(dtype=0, chunk=256),
    dict(qk=(-8, 64, 8)), dict(dk=128, dv=128, chunk=64), dict(dk=40, dv=40, chunk=128),
])
def test_gla_rejects_bad_arguments(L, bad):
    rc = _gla(L, **bad)
    assert rc == -1
    assert len(L.dig_last_error()) > 0


def test_workspace_size_rejects_bad_sizes(L):
    assert L.gla_fwd_workspace_size(1, 1, 64, 8, 12, 12, 0) == ctypes.c_size_t(-1).value
    assert L.gla_fwd_workspace_size(0, 1, 64, 8, 16, 16, 0) == 0
    # automatic chunk for 128 channels is 32 (64-token chunks are limited to 96 channels)
    assert L.gla_fwd_workspace_size(1, 1, 64, 8, 128, 128, 0) != ctypes.c_size_t(-1).value
    assert L.gla_fwd_workspace_size(1, 1, 64, 8, 128, 128, 64) == ctypes.c_size_t(-1).value


def _conv(L, **kw):
    a = dict(x=16, dtype=1, B=1, T=64, C=64, xs=(4096, 64), w=32, gh=8, gw=8, dir=0, y=48, ys=(4096, 64))
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.srem_dwconv(p(a["x"]), a["dtype"], a["B"], a["T"], a["C"], *a["xs"], p(a["w"]), a["gh"],
                         a["gw"], a["dir"], p(a["y"]), *a["ys"], None)


@pytest.mark.parametrize("bad", [dict(x=None), dict(w=None), dict(C=12), dict(gh=3), dict(dir=-1),
                                 dict(xs=(4096, 8)), dict(y=16), dict(x=24), dict(dtype=3)])
def test_dwconv_rejects_bad_arguments(L, bad):
    assert _conv(L, **bad) == -1
    assert len(L.dig_last_error()) > 0


@pytest.mark.parametrize("bad", [dict(C=10), dict(frm=5), dict(gh=5), dict(x=None), dict(y=16)])
def test_remap_rejects_bad_arguments(L, bad):
    a = dict(x=16, dtype=1, B=1, T=64, C=64, gh=8, gw=8, frm=0, to=2, y=48)
    a.update(bad)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    assert L.srem_remap(p(a["x"]), a["dtype"], a["B"], a["T"], a["C"], a["gh"], a["gw"], a["frm"], a["to"],
                        p(a["y"]), None) == -1


@pytest.mark.parametrize("bad", [dict(N=0), dict(C=12), dict(C=16392), dict(xs=8), dict(eps=-1.0),
                                 dict(scale=None)])
def test_adaln_rejects_bad_arguments(L, bad):
    a = dict(x=16, dtype=1, N=4, C=64, xs=64, scale=32, shift=48, eps=1e-6, os=1.0, y=64, ys=64)
    a.update(bad)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    assert L.dig_adaln_modulate(p(a["x"]), a["dtype"], a["N"], a["C"], a["xs"], p(a["scale"]), p(a["shift"]),
                                a["eps"], a["os"], p(a["y"]), a["ys"], None) == -1


def test_binding_raises_on_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(binding.DigError):
        binding.lib()


def _bwd(L, **kw):
    a = dict(q=16, k=32, v=48, g=64, dtype=1, qk=(4096 * 8 * 8, 64, 8), vs=(4096 * 8 * 8, 64, 8),
             B=1, T=64, H=8, dk=8, dv=8, gh=8, gw=8, dir=0, chunk=0, s0=None, do=80,
             dos=(4096 * 8 * 8, 64, 8), dsf=None, dq=96, dk_=112, dv_=128, dg=144, ds0=None, ws=None, wsb=0)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.gla_bwd(p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), a["dtype"], *a["qk"], *a["vs"],
                     a["B"], a["T"], a["H"], a["dk"], a["dv"], a["gh"], a["gw"], a["dir"], a["chunk"],
                     p(a["s0"]), p(a["do"]), *a["dos"], p(a["dsf"]), p(a["dq"]), p(a["dk_"]), p(a["dv_"]),
                     p(a["dg"]), p(a["ds0"]), p(a["ws"]), a["wsb"], None)


@pytest.mark.parametrize("bad", [
    dict(q=None), dict(do=None), dict(dq=None), dict(dg=None), dict(dtype=0), dict(B=0), dict(dk=0),
    dict(dv=136), dict(dk=12, dv=12), dict(gh=7), dict(dir=4), dict(chunk=48), dict(dk=96, dv=96, chunk=64),
    dict(q=18), dict(do=88), dict(dos=(4096 * 64, 60, 8)), dict(qk=(-8, 64, 8)), dict(dq=16),
    # d log alpha of one batch (T * H * dk fp32) would span 2 GiB
    dict(T=65536, gh=256, gw=256, H=64, dk=128, dv=128, qk=(65536 * 128, 128, 8), vs=(65536 * 128, 128, 8),
         dos=(65536 * 128, 128, 8)),
])
def test_bwd_rejects_bad_arguments(L, bad):
    rc = _bwd(L, **bad)
    assert rc == binding.DIG_EINVAL if hasattr(binding, "DIG_EINVAL") else rc == -1, bad
    assert L.dig_last_error()


def test_bwd_workspace_size(L):
    n = L.gla_bwd_workspace_size(1, 8, 4096, 16, 72, 72, 0)
    assert n == 2 * 8 * 16 * 64 * 80 * 80 * 2          # two bf16 [units][chunks][80][80] state sets
    assert L.gla_bwd_workspace_size(0, 8, 4096, 16, 72, 72, 0) == ctypes.c_size_t(-1).value


def _block(L, **kw):
    a = dict(x=256, c=512, w=[768 + 256 * i for i in range(10)], w_conv=4096, B=1, T=64, C=128, H=2, gh=8, gw=8,
             dir=0, y=8192)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    w = [p(v) for v in a["w"]]
    return L.dig_block_fwd(p(a["x"]), p(a["c"]), *w, p(a["w_conv"]), a["B"], a["T"], a["C"], a["H"], a["gh"],
                           a["gw"], a["dir"], p(a["y"]), None, 0, None)


@pytest.mark.parametrize("bad", [
    dict(x=None), dict(c=None), dict(y=None), dict(w_conv=None), dict(w=[768] * 9 + [None]), dict(B=0),
    dict(C=130), dict(H=3), dict(C=136, H=1), dict(C=24, H=2), dict(C=16392, H=2), dict(gh=7), dict(dir=4),
    dict(x=264), dict(y=256),
    dict(w=[768 + 256 * i for i in range(3)] + [1032] + [768 + 256 * i for i in range(4, 10)]),   # b_in misaligned
    dict(B=64, T=4096, gh=64, gw=64, C=1024, H=8),                                                 # B*T*4C >= 2^30
])
def test_block_rejects_bad_arguments(L, bad):
    """Checked before any device query: nulls, head size (C/H a multiple of
    8, at most 128), C <= 16384, the grid, the direction, alignment of the
    bf16 tensors and of b_in/b_out/b_ff1/b_ff2, y aliasing x, the product size."""
    assert _block(L, **bad) == -1, bad
    assert L.dig_last_error()


@pytest.mark.parametrize("bad", [dict(x=None), dict(M=0), dict(K=-1), dict(x=264), dict(y=256), dict(y=512),
                                 dict(K=12), dict(N=12), dict(M=1 << 27), dict(N=1 << 27)])
def test_linear_rejects_bad_arguments(L, bad):
    """Checked before any device query: nulls, sizes (K and N multiples of 8,
    M*K and N*K below 2^30), 16-byte alignment, y aliasing an input.  The
    product needs no workspace."""
    assert L.dig_linear_workspace_size() == 0
    a = dict(x=256, w=512, y=768, M=4, N=8, K=16, ws=None, wsb=0)
    a.update(bad)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    rc = L.dig_linear(p(a["x"]), p(a["w"]), p(a["y"]), a["M"], a["N"], a["K"], p(a["ws"]), a["wsb"], None)
    assert rc in (-1, -2), bad
    assert L.dig_last_error()


def test_workspace_status_rejects_missing_workspace(L):
    assert L.gla_fwd_workspace_status(None, 0, None) == -1
    assert b"workspace" in L.dig_last_error()
    assert L.gla_fwd_workspace_status(ctypes.c_void_p(256), 16, None) == -1
