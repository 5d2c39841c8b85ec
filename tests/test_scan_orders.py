"""The product-side scan-order tables (gated_linear_attention_gla_amd.scan_orders)
against the hand-listed orders (CPU)."""
import json
import os

import numpy as np

from gated_linear_attention_gla_amd import scan_orders as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_zigzag_tables_match_hand_listed_orders():
    g = _golden("zigzag_orders_2x3.json")
    gh, gw = g["grid"]
    for j, order in g["orders"].items():
        t = so.zigzag(int(j), gh, gw)
        assert t.dtype == np.int32 and t.tolist() == order, j


def test_grid_order_tables_match_hand_listed_orders():
    g = _golden("scan_orders_2x3.json")
    gh, gw = g["grid"]
    for d, order in g["perm"].items():
        assert so.grid_order(d, gh, gw).tolist() == order, d


def test_inverse():
    for order in (so.zigzag(3, 5, 7), so.grid_order("b2t", 4, 6)):
        inv = so.inverse(order)
        assert np.array_equal(inv[order], np.arange(order.size))
        assert np.array_equal(order[inv], np.arange(order.size))
