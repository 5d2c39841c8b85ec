"""Pins of the fp64 DiG-block oracle (oracle.block_fwd), CPU.

Each test isolates one branch of the block by choosing weights, and checks
it against something other than the oracle's own code: the adaLN-Zero
identity the pages state (zero-initialised gates and the identity-initialised
conv leave the block an identity map), closed forms for the gate and bias
paths, and library routines (torch's SiLU, linear, layer_norm, tanh GELU) for
single steps, with the already-pinned GLA and conv oracles for the rest."""
import numpy as np
import torch
import torch.nn.functional as F

from gated_linear_attention_gla_amd import inputs as gen


def _case(B=2, gh=3, gw=4, C=32, seed=0):
    x = gen.block_inputs(B, gh * gw, C, seed=seed)
    w = {n: x[n].double().numpy().copy() for n in ("w_ada", "b_ada", "w_in", "b_in", "w_out", "b_out", "w_ff1",
                                                    "b_ff1", "w_ff2", "b_ff2", "w_conv")}
    return x["x"].double().numpy(), x["c"].double().numpy(), w


def _identity_conv(w):
    w["w_conv"][:] = 0.0
    w["w_conv"][:, 1, 1] = 1.0


def test_adaln_zero_block_is_the_identity(orc):
    """DiT notes 3.2 (adaLN-Zero: gates regressed as zero make each residual
    branch the identity) and DiG notes, SREM (the conv starts as identity)."""
    x, c, w = _case(seed=1)
    w["w_ada"][:] = 0.0
    w["b_ada"][:] = 0.0
    _identity_conv(w)
    for d in ("l2r", "r2l", "t2b", "b2t"):
        y = orc.block_fwd(x, c, w, (3, 4), d, H=2)
        np.testing.assert_array_equal(y, x)


def test_gates_and_biases_closed_form(orc):
    """Zero projections leave only the biases: the mixer adds g1 * b_out, the
    FFN g2 * b_ff2 (GELU(0) = 0)."""
    x, c, w = _case(seed=2)
    C = x.shape[2]
    w["w_ada"][:] = 0.0
    for n in ("w_out", "w_ff1", "b_ff1"):
        w[n][:] = 0.0
    _identity_conv(w)
    g1, g2 = w["b_ada"][2 * C:3 * C], w["b_ada"][5 * C:6 * C]
    y = orc.block_fwd(x, c, w, (3, 4), "b2t", H=2)
    np.testing.assert_allclose(y, x + g1 * w["b_out"] + g2 * w["b_ff2"], rtol=0, atol=1e-14)


def test_conditioning_regression(orc):
    """The mixer gate regressed from c: with the mixer's output the constant 1
    (zero out-projection, b_out = 1) and the FFN silenced, y - x is the gate
    SiLU(c) W^T + b of the regression's third block (torch's silu and linear)."""
    x, c, w = _case(seed=3)
    C = x.shape[2]
    w["w_out"][:] = 0.0
    w["b_out"][:] = 1.0
    w["w_ada"][5 * C:] = 0.0
    w["b_ada"][5 * C:] = 0.0
    _identity_conv(w)
    y = orc.block_fwd(x, c, w, (3, 4), "l2r", H=2)
    ada = F.linear(F.silu(torch.tensor(c)), torch.tensor(w["w_ada"]), torch.tensor(w["b_ada"])).numpy()
    np.testing.assert_allclose(y - x, np.broadcast_to(ada[:, None, 2 * C:3 * C], x.shape), rtol=1e-12, atol=1e-12)


def test_mixer_plumbing(orc):
    """q = k = v = LN(x) and u = 0 (log gate logsigmoid(0) / 16), identity
    out-projection and unit mixer gate: y - x is the pinned GLA oracle on those
    inputs, brought back to canonical order; the FFN is silenced."""
    B, gh, gw, C, H = 2, 3, 4, 16, 2
    T, d = gh * gw, C // H
    x, c, w = _case(B, gh, gw, C, seed=4)
    eye = np.eye(C)
    w["w_ada"][:] = 0.0
    w["b_ada"][:] = 0.0
    w["b_ada"][2 * C:3 * C] = 1.0                      # mixer gate 1, FFN gate 0
    w["w_in"][:] = np.concatenate([eye, eye, eye, 0 * eye])
    w["b_in"][:] = 0.0
    w["w_out"][:] = eye
    w["b_out"][:] = 0.0
    _identity_conv(w)
    for direction in ("r2l", "t2b"):
        y = orc.block_fwd(x, c, w, (gh, gw), direction, H=H)
        h = F.layer_norm(torch.tensor(x), (C,), eps=1e-6).numpy().reshape(B, T, H, d)
        la = np.full_like(h, -np.log(2.0) / 16.0)
        o, _ = orc.gla_fwd(h / np.sqrt(d), h, h, la, (gh, gw), direction)
        oc = np.empty((B, T, C))
        oc[:, orc.scan_perm(direction, gh, gw)] = o.reshape(B, T, C)
        np.testing.assert_allclose(y - x, oc, rtol=1e-10, atol=1e-12)


def test_mixer_log_gate(orc):
    """The gate projection taken as u = LN(x) (not 0, where logsigmoid(u) and
    logsigmoid(-u) agree): y - x is the pinned GLA oracle with log alpha =
    logsigmoid(u) / 16 from torch's logsigmoid; the FFN is silenced."""
    B, gh, gw, C, H = 2, 3, 4, 16, 2
    T, d = gh * gw, C // H
    x, c, w = _case(B, gh, gw, C, seed=7)
    eye = np.eye(C)
    w["w_ada"][:] = 0.0
    w["b_ada"][:] = 0.0
    w["b_ada"][2 * C:3 * C] = 1.0
    w["w_in"][:] = np.concatenate([eye, eye, eye, eye])
    w["b_in"][:] = 0.0
    w["w_out"][:] = eye
    w["b_out"][:] = 0.0
    _identity_conv(w)
    for direction in ("l2r", "b2t"):
        y = orc.block_fwd(x, c, w, (gh, gw), direction, H=H)
        ht = F.layer_norm(torch.tensor(x), (C,), eps=1e-6)
        h = ht.numpy().reshape(B, T, H, d)
        la = (F.logsigmoid(ht) / 16.0).numpy().reshape(B, T, H, d)
        o, _ = orc.gla_fwd(h / np.sqrt(d), h, h, la, (gh, gw), direction)
        oc = np.empty((B, T, C))
        oc[:, orc.scan_perm(direction, gh, gw)] = o.reshape(B, T, C)
        np.testing.assert_allclose(y - x, oc, rtol=1e-10, atol=1e-12)


def test_ffn_branch(orc):
    """With the mixer gate zero and the FFN gate one, y - x is the FFN of the
    modulated LN(x) (torch's layer_norm, linear and tanh GELU)."""
    x, c, w = _case(seed=5)
    C = x.shape[2]
    w["w_ada"][:] = 0.0
    w["b_ada"][:] = 0.0
    w["b_ada"][3 * C:4 * C] = 0.3                      # FFN shift
    w["b_ada"][4 * C:5 * C] = -0.2                     # FFN scale
    w["b_ada"][5 * C:6 * C] = 1.0                      # FFN gate
    _identity_conv(w)
    y = orc.block_fwd(x, c, w, (3, 4), "l2r", H=2)
    t = lambda a: torch.tensor(a)
    h2 = F.layer_norm(t(x), (C,), eps=1e-6) * (1 - 0.2) + 0.3
    f = F.linear(F.gelu(F.linear(h2, t(w["w_ff1"]), t(w["b_ff1"])), approximate="tanh"), t(w["w_ff2"]),
                 t(w["b_ff2"])).numpy()
    np.testing.assert_allclose(y - x, f, rtol=1e-10, atol=1e-12)


def test_conv_step(orc):
    """All gates zero: y is the pinned conv oracle applied to x in the scan
    order of the direction."""
    x, c, w = _case(seed=6)
    w["w_ada"][:] = 0.0
    w["b_ada"][:] = 0.0
    for direction in ("l2r", "b2t"):
        y = orc.block_fwd(x, c, w, (3, 4), direction, H=2)
        ref = orc.srem_dwconv(x[:, orc.scan_perm(direction, 3, 4)], w["w_conv"], (3, 4), direction)
        np.testing.assert_array_equal(y, ref)
