"""Thin ctypes binding over libdig_gla.so (include/dig_gla.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback of any kind: if the library is missing or a call fails,
an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdig_gla.so")

DIG_F32, DIG_BF16 = 0, 1
DIRS = {"l2r": 0, "r2l": 1, "t2b": 2, "b2t": 3}
_lock = threading.Lock()
_lib = None
_ws_cache: dict = {}


class DigError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libdig_gla.so (built in-tree); raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise DigError(f"{LIB_PATH} is missing: build it with "
                               "`python -m gated_linear_attention_gla_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            p, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
            L.gla_fwd.argtypes = [p, p, p, p, i32, i64, i64, i64, i64, i64, i64,
                                  i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                  p, p, i64, i64, i64, p, p, sz, p]
            L.gla_fwd.restype = i32
            L.gla_fwd_ordered.argtypes = [p, p, p, p, i32, i64, i64, i64, i64, i64, i64,
                                          i32, i32, i32, i32, i32, p, i32,
                                          p, p, i64, i64, i64, p, p, sz, p]
            L.gla_fwd_ordered.restype = i32
            L.gla_fwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
            L.gla_fwd_workspace_size.restype = sz
            L.gla_fwd_noalloc.argtypes = [p, p, p, p, i32, i64, i64, i64, i64, i64, i64,
                                          i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                          p, p, i64, i64, i64, p, p]
            L.gla_fwd_noalloc.restype = i32
            L.gla_fwd_workspace_status.argtypes = [p, sz, p]
            L.gla_fwd_workspace_status.restype = i32
            L.gla_bwd.argtypes = [p, p, p, p, i32, i64, i64, i64, i64, i64, i64,
                                  i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                  p, p, i64, i64, i64, p, p, p, p, p, p, p, sz, p]
            L.gla_bwd.restype = i32
            L.gla_bwd_ordered.argtypes = [p, p, p, p, i32, i64, i64, i64, i64, i64, i64,
                                          i32, i32, i32, i32, i32, p, i32,
                                          p, p, i64, i64, i64, p, p, p, p, p, p, p, sz, p]
            L.gla_bwd_ordered.restype = i32
            L.dig_gather_rows.argtypes = [p, i32, i32, i32, i32, p, p, p]
            L.dig_gather_rows.restype = i32
            L.dig_linear_workspace_size.argtypes = []
            L.dig_linear_workspace_size.restype = sz
            L.dig_linear.argtypes = [p, p, p, i32, i32, i32, p, sz, p]
            L.dig_linear.restype = i32
            L.dig_block_workspace_size.argtypes = [i32, i32, i32, i32]
            L.dig_block_workspace_size.restype = sz
            L.dig_block_fwd.argtypes = [p] * 13 + [i32] * 7 + [p, p, sz, p]
            L.dig_block_fwd.restype = i32
            L.gla_bwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
            L.gla_bwd_workspace_size.restype = sz
            L.srem_dwconv.argtypes = [p, i32, i32, i32, i32, i64, i64, p, i32, i32, i32, p, i64, i64, p]
            L.srem_dwconv.restype = i32
            L.srem_remap.argtypes = [p, i32, i32, i32, i32, i32, i32, i32, i32, p, p]
            L.srem_remap.restype = i32
            L.dig_adaln_modulate.argtypes = [p, i32, i64, i32, i64, p, p, f32, f32, p, i64, p]
            L.dig_adaln_modulate.restype = i32
            L.dig_last_error.argtypes = []
            L.dig_last_error.restype = ctypes.c_char_p
            L.dig_version.argtypes = []
            L.dig_version.restype = ctypes.c_char_p
            _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        msg = lib().dig_last_error().decode(errors="replace")
        raise DigError(f"{what} failed ({rc}): {msg}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DIG_BF16
    if t.dtype == torch.float32:
        return DIG_F32
    raise DigError(f"unsupported dtype {t.dtype}")


def _dir(d) -> int:
    return DIRS[d] if isinstance(d, str) else int(d)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _order(order, T: int, device: torch.device):
    """A scan-order table for the *_ordered calls: int32 [T], contiguous, on `device`."""
    if order.dtype != torch.int32 or tuple(order.shape) != (T,) or not order.is_contiguous() \
            or order.device != device:
        raise DigError(f"order must be a contiguous int32 [{T}] tensor on {device}")
    return order


def workspace_bytes(dtype_code: int, B: int, T: int, H: int, dk: int, dv: int, chunk: int = 0) -> int:
    n = lib().gla_fwd_workspace_size(dtype_code, B, T, H, dk, dv, chunk)
    if n == ctypes.c_size_t(-1).value:
        raise DigError("gla_fwd_workspace_size: invalid sizes: " + lib().dig_last_error().decode())
    return int(n)


def get_workspace(device: torch.device, nbytes: int, key: str = "fwd") -> torch.Tensor | None:
    """A cached, zero-initialised workspace of at least nbytes for `device` and its current
    stream (grown on demand).  Calls in flight at the same time must not share a workspace,
    so the cache is per stream; gla_fwd's (which keeps flags across calls) and gla_bwd's
    are separate buffers."""
    if nbytes == 0:
        return None
    key = (key, device.type, device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def gla_fwd(q, k, v, log_alpha, grid, direction, chunk: int = 0, s0=None, out=None,
            s_final: bool | torch.Tensor = True, workspace=None, order=None):
    """GLA forward over one scan direction.

    q, k, log_alpha: [B, T, H, dk]; v: [B, T, H, dv]; canonical token order,
    innermost dim contiguous, all on one GPU, same dtype (bf16 or fp32).
    order: optional int32 [T] device table (scan position -> canonical token,
    see scan_orders.py); when given, grid and direction are not used
    (gla_fwd_ordered).
    Returns (o [B, T, H, dv] in SCAN order, s_final [B, H, dk, dv] fp32 or None).
    """
    B, T, H, dk = q.shape
    dv = v.shape[3]
    if k.shape != q.shape or log_alpha.shape != q.shape or tuple(v.shape[:3]) != (B, T, H):
        raise DigError("gla_fwd: shape mismatch")
    for t in (q, k, v, log_alpha):
        if t.stride(3) != 1 or t.dtype != q.dtype or t.device != q.device:
            raise DigError("gla_fwd: tensors must share dtype/device and have a contiguous last dim")
    if k.stride() != q.stride() or log_alpha.stride() != q.stride():
        raise DigError("gla_fwd: q, k, log_alpha must share strides")
    dc = _dtype_code(q)
    dev = q.device
    if out is None:
        out = torch.empty(B, T, H, dv, dtype=q.dtype, device=dev)
    sf = None
    if isinstance(s_final, torch.Tensor):
        sf = s_final
    elif s_final:
        sf = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    if s0 is not None:
        if s0.dtype != torch.float32 or tuple(s0.shape) != (B, H, dk, dv) or not s0.is_contiguous():
            raise DigError("gla_fwd: s0 must be contiguous fp32 [B, H, dk, dv]")
    if workspace is None:
        workspace = get_workspace(dev, workspace_bytes(dc, B, T, H, dk, dv, chunk))
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if order is not None:
        rc = lib().gla_fwd_ordered(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), dc,
                                   q.stride(0), q.stride(1), q.stride(2), v.stride(0), v.stride(1), v.stride(2),
                                   B, T, H, dk, dv, _ptr(_order(order, T, dev)), chunk,
                                   _ptr(s0), _ptr(out), out.stride(0), out.stride(1), out.stride(2),
                                   _ptr(sf), _ptr(workspace), wsb, _stream(dev))
        _check(rc, "gla_fwd_ordered")
        return out, sf
    gh, gw = grid
    rc = lib().gla_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), dc,
                       q.stride(0), q.stride(1), q.stride(2), v.stride(0), v.stride(1), v.stride(2),
                       B, T, H, dk, dv, gh, gw, _dir(direction), chunk,
                       _ptr(s0), _ptr(out), out.stride(0), out.stride(1), out.stride(2),
                       _ptr(sf), _ptr(workspace), wsb, _stream(dev))
    _check(rc, "gla_fwd")
    return out, sf


def gla_fwd_noalloc(q, k, v, log_alpha, grid, direction, chunk: int = 0, s0=None, out=None, s_final=None):
    """gla_fwd through the allocation-free entry point (its workspace is the
    library's fixed per-GPU scratch).  out and s_final must be given
    (preallocated): this wrapper allocates nothing either."""
    B, T, H, dk = q.shape
    dv = v.shape[3]
    if out is None:
        raise DigError("gla_fwd_noalloc: out must be preallocated")
    if k.shape != q.shape or log_alpha.shape != q.shape or tuple(v.shape[:3]) != (B, T, H):
        raise DigError("gla_fwd_noalloc: shape mismatch")
    if k.stride() != q.stride() or log_alpha.stride() != q.stride():
        raise DigError("gla_fwd_noalloc: q, k, log_alpha must share strides")
    gh, gw = grid
    rc = lib().gla_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _dtype_code(q),
                               q.stride(0), q.stride(1), q.stride(2), v.stride(0), v.stride(1), v.stride(2),
                               B, T, H, dk, dv, gh, gw, _dir(direction), chunk,
                               _ptr(s0), _ptr(out), out.stride(0), out.stride(1), out.stride(2),
                               _ptr(s_final), _stream(q.device))
    _check(rc, "gla_fwd_noalloc")
    return out, s_final


def workspace_status(workspace) -> None:
    """Synchronise the current stream and raise DigError if a gla_fwd call that used
    `workspace` had a wait between workgroups give up (gla_fwd_workspace_status)."""
    rc = lib().gla_fwd_workspace_status(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                        _stream(workspace.device))
    _check(rc, "gla_fwd_workspace_status")


def gla_bwd(q, k, v, log_alpha, grid, direction, d_o, chunk: int = 0, s0=None, ds_final=None,
            need_ds0: bool = True, workspace=None, order=None):
    """Gradients of gla_fwd (bf16): d_o [B, T, H, dv] in SCAN order (the
    gradient of o), ds_final fp32 [B, H, dk, dv] or None (zero).  order: as
    for gla_fwd (gla_bwd_ordered).

    Returns (dq, dk, dv, dlog_alpha, ds0): dq, dk bf16 [B, T, H, dk], dv bf16
    [B, T, H, dv], dlog_alpha fp32 [B, T, H, dk], all canonical token order;
    ds0 fp32 [B, H, dk, dv] (None when need_ds0 is False).
    """
    B, T, H, dk = q.shape
    dv = v.shape[3]
    if k.shape != q.shape or log_alpha.shape != q.shape or tuple(v.shape[:3]) != (B, T, H):
        raise DigError("gla_bwd: shape mismatch")
    if tuple(d_o.shape) != (B, T, H, dv):
        raise DigError("gla_bwd: d_o must be [B, T, H, dv]")
    for t in (q, k, v, log_alpha, d_o):
        if t.stride(3) != 1 or t.dtype != torch.bfloat16 or t.device != q.device:
            raise DigError("gla_bwd: bf16 tensors on one device with a contiguous last dim")
    if k.stride() != q.stride() or log_alpha.stride() != q.stride():
        raise DigError("gla_bwd: q, k, log_alpha must share strides")
    dev = q.device
    for name, t in (("s0", s0), ("ds_final", ds_final)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (B, H, dk, dv) or not t.is_contiguous()):
            raise DigError(f"gla_bwd: {name} must be contiguous fp32 [B, H, dk, dv]")
    dq = torch.empty(B, T, H, dk, dtype=torch.bfloat16, device=dev)
    dk_ = torch.empty(B, T, H, dk, dtype=torch.bfloat16, device=dev)
    dv_ = torch.empty(B, T, H, dv, dtype=torch.bfloat16, device=dev)
    dg = torch.empty(B, T, H, dk, dtype=torch.float32, device=dev)
    ds0 = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev) if need_ds0 else None
    if workspace is None:
        n = lib().gla_bwd_workspace_size(DIG_BF16, B, T, H, dk, dv, chunk)
        if n == ctypes.c_size_t(-1).value:
            raise DigError("gla_bwd: invalid sizes: " + lib().dig_last_error().decode(errors="replace"))
        workspace = get_workspace(dev, n, key="bwd")
    wsb = workspace.numel() * workspace.element_size()
    if order is not None:
        rc = lib().gla_bwd_ordered(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), DIG_BF16,
                                   q.stride(0), q.stride(1), q.stride(2), v.stride(0), v.stride(1), v.stride(2),
                                   B, T, H, dk, dv, _ptr(_order(order, T, dev)), chunk, _ptr(s0),
                                   _ptr(d_o), d_o.stride(0), d_o.stride(1), d_o.stride(2), _ptr(ds_final),
                                   _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(ds0), _ptr(workspace), wsb,
                                   _stream(dev))
        _check(rc, "gla_bwd_ordered")
        return dq, dk_, dv_, dg, ds0
    rc = lib().gla_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), DIG_BF16,
                       q.stride(0), q.stride(1), q.stride(2), v.stride(0), v.stride(1), v.stride(2),
                       B, T, H, dk, dv, grid[0], grid[1], _dir(direction), chunk, _ptr(s0),
                       _ptr(d_o), d_o.stride(0), d_o.stride(1), d_o.stride(2), _ptr(ds_final),
                       _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(ds0), _ptr(workspace), wsb,
                       _stream(dev))
    _check(rc, "gla_bwd")
    return dq, dk_, dv_, dg, ds0


def srem_dwconv(x_scan, w, grid, direction, out=None):
    """x_scan [B, T, C] (scan order of `direction`), w fp32 [C, 3, 3] -> y [B, T, C] canonical order."""
    B, T, C = x_scan.shape
    if x_scan.stride(2) != 1:
        raise DigError("srem_dwconv: channels must be contiguous")
    if w.dtype != torch.float32 or tuple(w.shape) != (C, 3, 3) or not w.is_contiguous():
        raise DigError("srem_dwconv: w must be contiguous fp32 [C, 3, 3]")
    if out is None:
        out = torch.empty(B, T, C, dtype=x_scan.dtype, device=x_scan.device)
    rc = lib().srem_dwconv(_ptr(x_scan), _dtype_code(x_scan), B, T, C, x_scan.stride(0), x_scan.stride(1),
                           _ptr(w), grid[0], grid[1], _dir(direction), _ptr(out), out.stride(0),
                           out.stride(1), _stream(x_scan.device))
    _check(rc, "srem_dwconv")
    return out


def srem_remap(x, grid, src, dst, out=None):
    """Contiguous x [B, T, C] in scan order `src` -> y in scan order `dst`."""
    B, T, C = x.shape
    if not x.is_contiguous():
        raise DigError("srem_remap: x must be contiguous")
    if out is None:
        out = torch.empty_like(x)
    rc = lib().srem_remap(_ptr(x), _dtype_code(x), B, T, C, grid[0], grid[1], _dir(src), _dir(dst),
                          _ptr(out), _stream(x.device))
    _check(rc, "srem_remap")
    return out


def gather_rows(x, index, out=None):
    """Contiguous x [B, T, C] -> y with y[:, p] = x[:, index[p]] (index int32 [T] on the device;
    an entry outside [0, T) gives a zero row)."""
    B, T, C = x.shape
    if not x.is_contiguous():
        raise DigError("gather_rows: x must be contiguous")
    if out is None:
        out = torch.empty_like(x)
    rc = lib().dig_gather_rows(_ptr(x), _dtype_code(x), B, T, C, _ptr(_order(index, T, x.device)), _ptr(out),
                               _stream(x.device))
    _check(rc, "dig_gather_rows")
    return out


BLOCK_WEIGHTS = ("w_ada", "b_ada", "w_in", "b_in", "w_out", "b_out", "w_ff1", "b_ff1", "w_ff2", "b_ff2", "w_conv")


def linear(x, w, out=None, workspace=None):
    """y = x w^T for bf16 x [M, K] and w [N, K] (rows contiguous), y [M, N] bf16 (fp32 accumulation)."""
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16 \
            or not x.is_contiguous() or not w.is_contiguous():
        raise DigError("linear: contiguous bf16 x [M, K] and w [N, K] needed")
    if out is None:
        out = torch.empty(M, N, dtype=torch.bfloat16, device=x.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().dig_linear(_ptr(x), _ptr(w), _ptr(out), M, N, K, _ptr(workspace), wsb, _stream(x.device))
    _check(rc, "dig_linear")
    return out


def block_fwd(x, c, weights: dict, grid, direction, H: int, out=None, workspace=None):
    """One DiG block forward (dig_block_fwd): x bf16 [B, T, C] canonical, c fp32 [B, C], weights
    a dict with the keys of BLOCK_WEIGHTS (bf16 w_*, fp32 b_* and w_conv).  Returns y [B, T, C]."""
    B, T, C = x.shape
    if x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise DigError("block_fwd: x must be contiguous bf16 [B, T, C]")
    if c.dtype != torch.float32 or tuple(c.shape) != (B, C) or not c.is_contiguous():
        raise DigError("block_fwd: c must be contiguous fp32 [B, C]")
    shapes = {"w_ada": (6 * C, C), "b_ada": (6 * C,), "w_in": (4 * C, C), "b_in": (4 * C,), "w_out": (C, C),
              "b_out": (C,), "w_ff1": (4 * C, C), "b_ff1": (4 * C,), "w_ff2": (C, 4 * C), "b_ff2": (C,),
              "w_conv": (C, 3, 3)}
    for n in BLOCK_WEIGHTS:
        t = weights[n]
        want = torch.bfloat16 if n.startswith("w_") and n != "w_conv" else torch.float32
        if t.dtype != want or tuple(t.shape) != shapes[n] or not t.is_contiguous() or t.device != x.device:
            raise DigError(f"block_fwd: {n} must be contiguous {want} {shapes[n]} on {x.device}")
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        n = lib().dig_block_workspace_size(B, T, C, H)
        if n == ctypes.c_size_t(-1).value:
            raise DigError("block_fwd: invalid sizes")
        workspace = get_workspace(x.device, int(n), key="block")
    rc = lib().dig_block_fwd(_ptr(x), _ptr(c), *[_ptr(weights[n]) for n in BLOCK_WEIGHTS], B, T, C, H, grid[0],
                             grid[1], _dir(direction), _ptr(out), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(x.device))
    _check(rc, "dig_block_fwd")
    return out


def adaln_modulate(x, scale, shift, eps: float = 1e-6, out_scale: float = 1.0, out=None):
    """x [..., C] (rows contiguous) -> LN over C, * (1 + scale) + shift, * out_scale."""
    C = x.shape[-1]
    if not x.is_contiguous():
        raise DigError("adaln_modulate: x must be contiguous")
    N = x.numel() // C
    if out is None:
        out = torch.empty_like(x)
    for t in (scale, shift):
        if t.dtype != torch.float32 or t.numel() != C or not t.is_contiguous():
            raise DigError("adaln_modulate: scale/shift must be contiguous fp32 [C]")
    rc = lib().dig_adaln_modulate(_ptr(x), _dtype_code(x), N, C, C, _ptr(scale), _ptr(shift),
                                  float(eps), float(out_scale), _ptr(out), C, _stream(x.device))
    _check(rc, "dig_adaln_modulate")
    return out


def version() -> str:
    return lib().dig_version().decode()
