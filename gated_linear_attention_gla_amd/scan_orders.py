"""Scan-order tables for gla_fwd_ordered / gla_bwd_ordered / gather_rows.

A table is int32 [T] with table[p] = the canonical (row-major, n = r*gw + c)
index of the token visited at scan position p.

* grid_order: the four orders of DiG's SREM (DiG notes, 关键设计 / SREM):
  rows left to right, its reversal, columns top to bottom, its reversal --
  the orders gla_fwd takes as `dir`.
* zigzag: ZigMa's snake scans (ZigMa notes, 关键设计 / Zigzag 扫描方案): each
  row (or column) is walked in the direction opposite to the one before, so
  consecutive tokens are always grid neighbours.  The notes give eight
  schemes S_0..S_7 over the horizontal/vertical directions and start points
  without listing them; read here as the two orientations times the four
  start corners: j // 4 = 0 rows / 1 columns, j % 4 = start at top-left,
  top-right, bottom-left, bottom-right.
* inverse: the table that arranges a scan-ordered tensor back to canonical
  order (for gather_rows).
"""
from __future__ import annotations

import numpy as np
import torch

DIRS = ("l2r", "r2l", "t2b", "b2t")


def grid_order(direction: str, gh: int, gw: int) -> np.ndarray:
    """Table of one of the four grid orders (the kernels' built-in directions)."""
    n = np.arange(gh * gw, dtype=np.int64).reshape(gh, gw)
    d = DIRS.index(direction) if isinstance(direction, str) else int(direction)
    seq = n.T.reshape(-1) if d >= 2 else n.reshape(-1)      # column-major walk for t2b / b2t
    if d & 1:
        seq = seq[::-1]
    return np.ascontiguousarray(seq, dtype=np.int32)


def zigzag(j: int, gh: int, gw: int) -> np.ndarray:
    """Snake scan S_j, j in [0, 8) (see the module docstring for the reading)."""
    if not 0 <= j < 8:
        raise ValueError("zigzag scheme must be in [0, 8)")
    n = np.arange(gh * gw, dtype=np.int64).reshape(gh, gw)
    columns, corner = j // 4, j % 4
    g = n.T if columns else n                       # lines = rows (or columns) in the walk's frame
    # start corner: flip the frame so the walk starts at its top-left
    first_line_last = corner >= 2                   # start at the bottom (rows) / the bottom end (columns)
    first_pos_last = corner % 2 == 1                # start at the right (rows) / the right line (columns)
    if columns:
        first_line_last, first_pos_last = first_pos_last, first_line_last
    if first_line_last:
        g = g[::-1]
    if first_pos_last:
        g = g[:, ::-1]
    g = g.copy()
    g[1::2] = g[1::2, ::-1]                         # every second line walked backwards
    return np.ascontiguousarray(g.reshape(-1), dtype=np.int32)


def inverse(order) -> np.ndarray:
    """inv[order[p]] = p."""
    order = np.asarray(order)
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size, dtype=order.dtype)
    return inv


def to_device(order, device) -> torch.Tensor:
    return torch.as_tensor(np.asarray(order, dtype=np.int32)).to(device).contiguous()
