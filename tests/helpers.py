"""Comparison helpers for GPU-vs-oracle parity tests.

Tolerances: the fp32 path must match the fp64 oracle within 1e-4 and the bf16
path (bf16 inputs, fp32 state/accumulation) within 2e-2, as max relative
error measured normwise: max|gpu - ref| / max|ref| over each (batch, head)
slice of o, each (batch, head) state, and each (batch, channel) of a conv
output.  o (and any [B, T, H, d] tensor) is also gated per 64-token block of
each (batch, head) slice -- a scan chunk when the tensor is in scan order --
so an error in a stretch whose values are small (the start of a scan, where
the state is still building up) cannot hide behind the slice's maximum.
Elementwise relative error is undefined where a sum cancels to ~0, so it is
not gated.
"""
from __future__ import annotations

import numpy as np
import torch

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
BLOCK_TOKENS = 64


def to_np(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").double().numpy()
    return np.asarray(t, dtype=np.float64)


def normwise_by(gpu, ref, axes_keep) -> np.ndarray:
    """max|g-r| / max|r| reduced over every axis not in axes_keep."""
    g, r = to_np(gpu), to_np(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    red = tuple(i for i in range(g.ndim) if i not in axes_keep)
    num = np.max(np.abs(g - r), axis=red)
    den = np.maximum(np.max(np.abs(r), axis=red), 1e-30)
    return num / den


def normwise_token_blocks(gpu, ref, block=BLOCK_TOKENS) -> np.ndarray:
    """[B, T, H, d] -> max|g-r| / max|r| per (batch, block of `block` tokens, head);
    the last block holds the ragged tail."""
    g, r = to_np(gpu), to_np(ref)
    assert g.shape == r.shape and g.ndim == 4, (g.shape, r.shape)
    B, T, H, _ = g.shape
    nb = -(-T // block)
    pad = nb * block - T
    d = np.abs(g - r)
    a = np.abs(r)
    if pad:
        d = np.concatenate([d, np.zeros((B, pad) + d.shape[2:])], axis=1)
        a = np.concatenate([a, np.zeros((B, pad) + a.shape[2:])], axis=1)
    num = d.reshape(B, nb, block, H, -1).max(axis=(2, 4))
    den = np.maximum(a.reshape(B, nb, block, H, -1).max(axis=(2, 4)), 1e-30)
    return num / den


def assert_o_close(o_gpu, o_ref, tol, what="o", block=BLOCK_TOKENS):
    """o: [B, T, H, dv] -> per (b, h) and per (b, 64-token block, h)."""
    assert np.all(np.isfinite(to_np(o_gpu))), f"{what}: non-finite GPU values"
    e = normwise_by(o_gpu, o_ref, (0, 2))
    assert e.max() <= tol, f"{what}: normwise rel err {e.max():.3e} > {tol:g}"
    eb = normwise_token_blocks(o_gpu, o_ref, block)
    if eb.max() > tol:
        b, c, h = np.unravel_index(np.argmax(eb), eb.shape)
        raise AssertionError(f"{what}: rel err {eb.max():.3e} > {tol:g} in the {block}-token block {c} "
                             f"of (batch {b}, head {h})")
    return float(max(e.max(), eb.max()))


def assert_state_close(s_gpu, s_ref, tol, what="s_final"):
    """s: [B, H, dk, dv] -> per (b, h)."""
    e = normwise_by(s_gpu, s_ref, (0, 1))
    assert e.max() <= tol, f"{what}: normwise rel err {e.max():.3e} > {tol:g}"
    return float(e.max())


def assert_conv_close(y_gpu, y_ref, tol, what="y"):
    """y: [B, T, C] -> per (b, channel)."""
    e = normwise_by(y_gpu, y_ref, (0, 2))
    assert e.max() <= tol, f"{what}: normwise rel err {e.max():.3e} > {tol:g}"
    return float(e.max())
