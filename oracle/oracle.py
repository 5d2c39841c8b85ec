"""Python entry to the fp64 CPU oracle in ``gla_oracle.c``.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``.  The product package never imports
it, and it never imports the product package.

The arithmetic lives in ``gla_oracle.c`` (plain loops, fp64).  This module only
builds that file with gcc, converts arrays to contiguous float64 numpy arrays
and calls it through ctypes.  See the C file for the definitions and the
passages of the pages each one follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

DIRS = {"l2r": 0, "r2l": 1, "t2b": 2, "b2t": 3}


def build(force: bool = False) -> str:
    """Compile gla_oracle.c into liboracle.so (gcc -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Werror",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            d, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
            lib.oracle_gla_fwd.argtypes = [d, d, d, d, i64, i64, i64, i64, i64, i64, i64, i32, d, d, d, i32]
            lib.oracle_gla_fwd.restype = i32
            lib.oracle_gla_bwd.argtypes = [d, d, d, d, i64, i64, i64, i64, i64, i64, i64, i32, d, d, d,
                                           d, d, d, d, d, i32]
            lib.oracle_gla_bwd.restype = i32
            lib.oracle_gla_fwd_order.argtypes = [d, d, d, d, i64, i64, i64, i64, i64, d, d, d, d, i32]
            lib.oracle_gla_fwd_order.restype = i32
            lib.oracle_gla_bwd_order.argtypes = [d, d, d, d, i64, i64, i64, i64, i64, d, d, d, d,
                                                 d, d, d, d, d, i32]
            lib.oracle_gla_bwd_order.restype = i32
            lib.oracle_srem_dwconv.argtypes = [d, i64, i64, i64, d, i64, i64, i32, d, i32]
            lib.oracle_srem_dwconv.restype = i32
            lib.oracle_remap.argtypes = [d, i64, i64, i64, i64, i32, i32, d]
            lib.oracle_remap.restype = i32
            lib.oracle_adaln_modulate.argtypes = [d, i64, i64, d, d, ctypes.c_double, ctypes.c_double, d, i32]
            lib.oracle_adaln_modulate.restype = i32
            lib.oracle_scan_perm.argtypes = [i32, i64, i64, d]
            lib.oracle_scan_perm.restype = i32
            lib.oracle_max_threads.argtypes = []
            lib.oracle_max_threads.restype = i32
            _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    """Contiguous float64 copy/view of a numpy array or CPU torch tensor (exact for bf16/fp32)."""
    if hasattr(a, "detach"):  # torch tensor: bf16 has no numpy dtype, widen in torch first
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dir(d) -> int:
    return DIRS[d] if isinstance(d, str) else int(d)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def scan_perm(direction, gh: int, gw: int) -> np.ndarray:
    """perm[p] = canonical (row-major) grid index visited at scan position p."""
    out = np.empty(gh * gw, dtype=np.int64)
    rc = _load().oracle_scan_perm(_dir(direction), gh, gw, _ptr(out))
    if rc != 0:
        raise ValueError("bad direction")
    return out


def zigzag_order(j: int, gh: int, gw: int) -> np.ndarray:
    """ZigMa's snake scan S_j (ZigMa notes, 关键设计 / Zigzag 扫描方案): lines
    (rows for j < 4, columns for j >= 4) walked one after the other, each in
    the direction opposite to the one before, starting at corner j % 4 =
    top-left, top-right, bottom-left, bottom-right.  Written out as walks."""
    if not 0 <= j < 8:
        raise ValueError("zigzag scheme must be in [0, 8)")
    columns, corner = j >= 4, j % 4
    from_bottom, from_right = corner >= 2, corner % 2 == 1
    out = []
    if not columns:
        rows = range(gh - 1, -1, -1) if from_bottom else range(gh)
        rightward = not from_right
        for r in rows:
            cols = range(gw) if rightward else range(gw - 1, -1, -1)
            out += [r * gw + c for c in cols]
            rightward = not rightward
    else:
        cols = range(gw - 1, -1, -1) if from_right else range(gw)
        downward = not from_bottom
        for c in cols:
            rows = range(gh) if downward else range(gh - 1, -1, -1)
            out += [r * gw + c for r in rows]
            downward = not downward
    return np.array(out, dtype=np.int64)


def _order_arg(order, T):
    o = np.ascontiguousarray(np.asarray(order), dtype=np.int64)
    if o.shape != (T,):
        raise ValueError("order must have T entries")
    return o


def gla_fwd(q, k, v, log_alpha, grid, direction, s0=None, nthreads: int = 0, order=None):
    """Token-by-token fp64 GLA forward.

    q, k, log_alpha: [B, T, H, dk]; v: [B, T, H, dv]; canonical token order.
    order: optional table (order[p] = canonical token at scan position p, a
    permutation) used instead of (grid, direction).
    Returns (o_scan [B, T, H, dv] in scan order, s_final [B, H, dk, dv]).
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(log_alpha)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != (B, T, H):
        raise ValueError("shape mismatch")
    o = np.empty((B, T, H, dv), dtype=np.float64)
    sf = np.empty((B, H, dk, dv), dtype=np.float64)
    s0a = None if s0 is None else _f64(s0)
    if s0a is not None and s0a.shape != (B, H, dk, dv):
        raise ValueError("s0 shape")
    if order is not None:
        ordv = _order_arg(order, T)
        rc = _load().oracle_gla_fwd_order(_ptr(q), _ptr(k), _ptr(v), _ptr(g), B, T, H, dk, dv, _ptr(ordv),
                                          None if s0a is None else _ptr(s0a), _ptr(o), _ptr(sf), int(nthreads))
    else:
        gh, gw = grid
        rc = _load().oracle_gla_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), B, T, H, dk, dv, gh, gw,
                                    _dir(direction), None if s0a is None else _ptr(s0a),
                                    _ptr(o), _ptr(sf), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gla_fwd rejected its arguments")
    return o, sf


def gla_bwd(q, k, v, log_alpha, grid, direction, do_scan, ds_final=None, s0=None, nthreads: int = 0,
            order=None):
    """Token-by-token fp64 GLA backward (reverse-mode derivative of gla_fwd).

    do_scan [B, T, H, dv] in scan order (the gradient of o), ds_final
    [B, H, dk, dv] or None.  Returns (dq, dk, dv, dlog_alpha, ds0) with dq, dk,
    dlog_alpha [B, T, H, dk] and dv [B, T, H, dv] in canonical token order and
    ds0 [B, H, dk, dv].
    """
    q, k, v, g, dO = _f64(q), _f64(k), _f64(v), _f64(log_alpha), _f64(do_scan)
    B, T, H, dk = q.shape
    dv = v.shape[3]
    if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != (B, T, H) or dO.shape != v.shape:
        raise ValueError("shape mismatch")
    s0a = None if s0 is None else _f64(s0)
    dsf = None if ds_final is None else _f64(ds_final)
    for a in (s0a, dsf):
        if a is not None and a.shape != (B, H, dk, dv):
            raise ValueError("state shape")
    dq, dkk, dg = (np.empty((B, T, H, dk)) for _ in range(3))
    dvv = np.empty((B, T, H, dv))
    ds0 = np.empty((B, H, dk, dv))
    if order is not None:
        ordv = _order_arg(order, T)
        rc = _load().oracle_gla_bwd_order(_ptr(q), _ptr(k), _ptr(v), _ptr(g), B, T, H, dk, dv, _ptr(ordv),
                                          None if s0a is None else _ptr(s0a), _ptr(dO),
                                          None if dsf is None else _ptr(dsf), _ptr(dq), _ptr(dkk), _ptr(dvv),
                                          _ptr(dg), _ptr(ds0), int(nthreads))
    else:
        rc = _load().oracle_gla_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), B, T, H, dk, dv, grid[0], grid[1],
                                    _dir(direction), None if s0a is None else _ptr(s0a), _ptr(dO),
                                    None if dsf is None else _ptr(dsf), _ptr(dq), _ptr(dkk), _ptr(dvv),
                                    _ptr(dg), _ptr(ds0), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gla_bwd rejected its arguments")
    return dq, dkk, dvv, dg, ds0


def srem_dwconv(x_scan, w, grid, direction, nthreads: int = 0):
    """x_scan [B, T, C] in scan order, w [C, 3, 3] -> y [B, T, C] canonical order."""
    x, wf = _f64(x_scan), _f64(w)
    B, T, C = x.shape
    if wf.shape != (C, 3, 3):
        raise ValueError("w shape")
    y = np.empty_like(x)
    rc = _load().oracle_srem_dwconv(_ptr(x), B, T, C, _ptr(wf), grid[0], grid[1],
                                    _dir(direction), _ptr(y), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_srem_dwconv rejected its arguments")
    return y


def remap(x, grid, src, dst):
    """x [B, T, C] in scan order `src` -> y in scan order `dst` (exact permutation)."""
    xf = _f64(x)
    B, T, C = xf.shape
    y = np.empty_like(xf)
    rc = _load().oracle_remap(_ptr(xf), B, C, grid[0], grid[1], _dir(src), _dir(dst), _ptr(y))
    if rc != 0:
        raise ValueError("oracle_remap rejected its arguments")
    return y


def adaln_modulate(x, scale, shift, eps: float = 1e-6, out_scale: float = 1.0, nthreads: int = 0):
    """x [..., C] -> LN over C, then * (1 + scale) + shift, then * out_scale."""
    xf = _f64(x)
    C = xf.shape[-1]
    N = xf.size // C
    sc, sh = _f64(scale).reshape(C), _f64(shift).reshape(C)
    y = np.empty_like(xf)
    rc = _load().oracle_adaln_modulate(_ptr(xf), N, C, _ptr(sc), _ptr(sh), float(eps),
                                       float(out_scale), _ptr(y), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_adaln_modulate rejected its arguments")
    return y


BLOCK_WEIGHTS = ("w_ada", "b_ada", "w_in", "b_in", "w_out", "b_out", "w_ff1", "b_ff1", "w_ff2", "b_ff2", "w_conv")


def block_fwd(x, c, w, grid, direction, H: int, nthreads: int = 0):
    """One DiG block forward in fp64, the steps in the order the pages give
    them (DiG notes, 关键设计 / DiG Block设计; adaLN-Zero from DiT notes, 3.2):

      (1) conditioning c -> SiLU -> linear -> six vectors per batch element:
          shift, scale, gate of the mixer branch, then of the FFN branch;
      (2) x -> LN (no affine, eps 1e-6) -> (1 + scale) * . + shift -> the q, k,
          v, gate projections -> GLA over the block's scan direction (q scaled
          by 1/sqrt(d), log gate = logsigmoid(u) / 16) -> out projection ->
          added to x times the gate, back in canonical token order;
      (3) the same adaLN -> FFN (C -> 4C, tanh GELU, 4C -> C) -> gated residual;
      (4) the tokens in the scan order of the direction, as that scan's 2-D
          frame, through the 3x3 depthwise conv, stored in canonical order.

    x [B, T, C] (canonical), c [B, C]; w: dict of the weights in
    BLOCK_WEIGHTS (PyTorch Linear layout [out, in]).  Returns y [B, T, C]."""
    x = _f64(x)
    c = _f64(c)
    W = {n: _f64(w[n]) for n in BLOCK_WEIGHTS}
    B, T, C = x.shape
    d = C // H
    gh, gw = grid
    # (1) adaLN-Zero parameters
    silu = c / (1.0 + np.exp(-c))
    ada = silu @ W["w_ada"].T + W["b_ada"]                              # [B, 6C]
    s1, a1, g1, s2, a2, g2 = (ada[:, i * C:(i + 1) * C][:, None, :] for i in range(6))

    def ln(z):
        mu = z.mean(axis=-1, keepdims=True)
        var = ((z - mu) ** 2).mean(axis=-1, keepdims=True)
        return (z - mu) / np.sqrt(var + 1e-6)

    # (2) token mixer
    h = ln(x) * (1.0 + a1) + s1
    qkvu = h @ W["w_in"].T + W["b_in"]                                 # [B, T, 4C]
    q, k, v, u = (qkvu[..., i * C:(i + 1) * C].reshape(B, T, H, d) for i in range(4))
    q = q / np.sqrt(d)
    log_alpha = (np.minimum(u, 0.0) - np.log1p(np.exp(-np.abs(u)))) / 16.0
    o, _ = gla_fwd(q, k, v, log_alpha, grid, direction, nthreads=nthreads)   # scan order
    o2 = o.reshape(B, T, C) @ W["w_out"].T + W["b_out"]
    perm = scan_perm(direction, gh, gw)                                # perm[p] = canonical token
    o2c = np.empty_like(o2)
    o2c[:, perm] = o2
    x1 = x + g1 * o2c
    # (3) FFN
    h2 = ln(x1) * (1.0 + a2) + s2
    z = h2 @ W["w_ff1"].T + W["b_ff1"]
    z = 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))
    x2 = x1 + g2 * (z @ W["w_ff2"].T + W["b_ff2"])
    # (4) SREM conv in the scan frame of the direction
    return srem_dwconv(x2[:, perm], W["w_conv"], grid, direction, nthreads=nthreads)
