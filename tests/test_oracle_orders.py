"""Pins of the oracle's table scan orders (CPU): ZigMa's zigzag scans against
hand-listed orders, their defining property, and the table path of the
forward/backward oracle against its grid-order path, against the L->R scan
of the arranged sequence, and against finite differences."""
import json
import os

import numpy as np
import pytest

from test_oracle_pins import _bwd_case, _rand, _relerr

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_golden_zigzag_orders(orc):
    g = _golden("zigzag_orders_2x3.json")
    gh, gw = g["grid"]
    for j, order in g["orders"].items():
        assert orc.zigzag_order(int(j), gh, gw).tolist() == order, j


@pytest.mark.parametrize("grid", [(2, 3), (3, 3), (4, 5), (5, 2), (1, 4), (6, 1)])
def test_zigzag_is_a_neighbour_walk(orc, grid):
    """The property the scans are defined by: a permutation of the grid in
    which every two consecutive tokens are grid neighbours."""
    gh, gw = grid
    seen = set()
    for j in range(8):
        o = orc.zigzag_order(j, gh, gw)
        assert sorted(o.tolist()) == list(range(gh * gw)), j
        r, c = np.divmod(o, gw)
        assert np.all(np.abs(np.diff(r)) + np.abs(np.diff(c)) == 1), (j, o)
        seen.add(tuple(o.tolist()))
    if gh >= 2 and gw >= 2:
        assert len(seen) == 8


def test_order_table_of_a_grid_order_is_that_direction(orc):
    x = _rand(2, 12, 2, 3, 4, seed=31, gate_div=2.0)
    s0 = np.random.default_rng(31).standard_normal((2, 2, 3, 4))
    for d in ("l2r", "r2l", "t2b", "b2t"):
        a = orc.gla_fwd(x["q"], x["k"], x["v"], x["log_alpha"], (3, 4), d, s0=s0)
        b = orc.gla_fwd(x["q"], x["k"], x["v"], x["log_alpha"], (3, 4), d, s0=s0, order=orc.scan_perm(d, 3, 4))
        for u, w in zip(a, b):
            np.testing.assert_array_equal(u, w)


def _arranged(x, order):
    """The sequence in scan order, as canonical inputs of a 1 x T grid."""
    return {n: (x[n][:, order] if n in ("q", "k", "v", "log_alpha") else x[n]) for n in x}


def test_order_table_is_the_arranged_l2r_scan(orc):
    """gla over table `order` == gla over the arranged sequence x[:, order]
    scanned left to right (ZigMa's arrange -> scan; the output stays in scan
    order)."""
    gh, gw = 3, 4
    x = _rand(1, 12, 2, 3, 2, seed=32, gate_div=2.0)
    for order in (orc.zigzag_order(5, gh, gw), np.random.default_rng(3).permutation(12)):
        o1, s1 = orc.gla_fwd(x["q"], x["k"], x["v"], x["log_alpha"], (gh, gw), "l2r", order=order)
        xa = _arranged(x, order)
        o2, s2 = orc.gla_fwd(xa["q"], xa["k"], xa["v"], xa["log_alpha"], (1, 12), "l2r")
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(s1, s2)


def test_order_table_backward_is_the_arranged_l2r_backward(orc):
    gh, gw = 2, 3
    x = _bwd_case(33, gh=gh, gw=gw)
    order = orc.zigzag_order(6, gh, gw)
    g1 = orc.gla_bwd(x["q"], x["k"], x["v"], x["log_alpha"], (gh, gw), "l2r", x["do"], ds_final=x["dsf"],
                     s0=x["s0"], order=order)
    xa = _arranged(x, order)
    g2 = orc.gla_bwd(xa["q"], xa["k"], xa["v"], xa["log_alpha"], (1, 6), "l2r", x["do"], ds_final=x["dsf"],
                     s0=x["s0"])
    for u, w in zip(g1[:4], g2[:4]):               # canonical token order[p] <- arranged position p
        np.testing.assert_array_equal(u[:, order], w)
    np.testing.assert_array_equal(g1[4], g2[4])


def test_order_table_backward_finite_differences(orc):
    gh, gw = 2, 3
    x = _bwd_case(34, gh=gh, gw=gw)
    order = orc.zigzag_order(7, gh, gw)
    got = orc.gla_bwd(x["q"], x["k"], x["v"], x["log_alpha"], (gh, gw), "l2r", x["do"], ds_final=x["dsf"],
                      s0=x["s0"], order=order)

    def loss():
        o, sf = orc.gla_fwd(x["q"], x["k"], x["v"], x["log_alpha"], (gh, gw), "l2r", s0=x["s0"], order=order)
        return float(np.sum(o * x["do"]) + np.sum(sf * x["dsf"]))

    h = 1e-6
    for name, grad in (("q", got[0]), ("k", got[1]), ("v", got[2]), ("log_alpha", got[3])):
        fd = np.empty_like(grad)
        for idx in np.ndindex(grad.shape):
            base = x[name][idx]
            x[name][idx] = base + h
            lp = loss()
            x[name][idx] = base - h
            lm = loss()
            x[name][idx] = base
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8, err_msg=name)


def test_order_pin_rejects_the_inverse_table(orc):
    """A table read the other way round (position of token n instead of the
    token at position p) must fail the arranged-scan pin."""
    gh, gw = 3, 4
    x = _rand(1, 12, 1, 3, 2, seed=35, gate_div=2.0)
    order = orc.zigzag_order(5, gh, gw)
    inv = np.empty_like(order)
    inv[order] = np.arange(12)
    assert not np.array_equal(inv, order)
    o_wrong, _ = orc.gla_fwd(x["q"], x["k"], x["v"], x["log_alpha"], (gh, gw), "l2r", order=inv)
    xa = _arranged(x, order)
    o_ref, _ = orc.gla_fwd(xa["q"], xa["k"], xa["v"], xa["log_alpha"], (1, 12), "l2r")
    assert _relerr(o_wrong, o_ref) > 1e-3


def test_order_table_must_be_a_permutation(orc):
    x = _rand(1, 6, 1, 2, 2, seed=36)
    for bad in ([0, 1, 2, 3, 4, 4], [0, 1, 2, 3, 4, 6], [0, 1, 2, 3, 4]):
        with pytest.raises(ValueError):
            orc.gla_fwd(x["q"], x["k"], x["v"], x["log_alpha"], (2, 3), "l2r", order=bad)
