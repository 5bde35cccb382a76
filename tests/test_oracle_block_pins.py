"""Pins for the fp64 oracle of the operators around attention (oracle/block_ops.py).

Closed forms, invariants, library routines and brute force, chosen so that a
plausible slip (sample instead of population variance, eps outside the root,
scale instead of 1 + scale, gate applied to x, gate and up halves swapped,
sigmoid instead of SiLU) fails at least one of them.
"""
import math

import numpy as np
import torch
from scipy.special import expit

from oracle import block_ops as O
from oracle import brute as B
from synth import make_block_inputs

rng = np.random.default_rng(4321)
EPS = 1e-6


# ----------------------------------------------------------------------------- LayerNorm + modulation
def test_constant_row_gives_shift():
    d = 64
    shift = rng.standard_normal(d)
    scale = rng.standard_normal(d)
    x = np.full((3, d), 7.25)
    np.testing.assert_array_equal(O.adaln_modulate(x, shift, scale, EPS), np.broadcast_to(shift, (3, d)))


def test_two_valued_row_closed_form():
    a, b, d = 3.0, -1.0, 10
    x = np.array([[a] * (d // 2) + [b] * (d // 2)])
    half = (a - b) / 2
    want = np.array([half] * (d // 2) + [-half] * (d // 2)) / math.sqrt(half * half + EPS)
    np.testing.assert_allclose(O.layer_norm(x, EPS)[0], want, rtol=1e-15)
    # eps inside the root, added to the variance: tiny spread against eps
    s = 1e-4
    y = O.layer_norm(np.array([[s, -s]]), EPS)[0]
    np.testing.assert_allclose(y, [s / math.sqrt(s * s + EPS), -s / math.sqrt(s * s + EPS)], rtol=1e-14)


def test_moments_population_variance():
    x = rng.standard_normal((16, 5376)) * rng.uniform(0.01, 20, (16, 1)) + rng.uniform(-50, 50, (16, 1))
    y = O.layer_norm(x, EPS)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose((y ** 2).mean(axis=1), var / (var + EPS), rtol=1e-12)


def test_modulation_uses_one_plus_scale():
    x = rng.standard_normal((4, 32))
    shift = rng.standard_normal(32)
    h = O.adaln_modulate(x, shift, np.full(32, -1.0), EPS)
    np.testing.assert_array_equal(h, np.broadcast_to(shift, h.shape))
    h0 = O.adaln_modulate(x, np.zeros(32), np.zeros(32), EPS)
    np.testing.assert_allclose(h0, O.layer_norm(x, EPS), rtol=0, atol=0)


def test_shift_invariance_and_library_layer_norm():
    x = rng.standard_normal((8, 5376)) * 3 + 1
    shift, scale = rng.standard_normal(5376), rng.standard_normal(5376)
    h = O.adaln_modulate(x, shift, scale, EPS)
    np.testing.assert_allclose(O.adaln_modulate(x + 123.0, shift, scale, EPS), h, rtol=1e-9, atol=1e-9)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (5376,), eps=EPS).numpy() * (1 + scale) + shift
    np.testing.assert_allclose(h, ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- gated residual
def test_gated_residual_special_cases():
    x, y = rng.standard_normal((3, 48)), rng.standard_normal((3, 48))
    np.testing.assert_array_equal(O.gated_residual(x, y, np.zeros(48)), x)
    np.testing.assert_array_equal(O.gated_residual(x, -x, np.ones(48)), np.zeros((3, 48)))
    g = rng.standard_normal(48)
    np.testing.assert_allclose(O.gated_residual(x, y, 2 * g) - x, 2 * (O.gated_residual(x, y, g) - x), rtol=1e-12, atol=1e-14)
    # the gate multiplies the branch, not the stream
    np.testing.assert_array_equal(O.gated_residual(np.zeros((1, 48)), y[:1], g), g * y[:1])


def test_fused_residual_then_update():
    x = rng.standard_normal((2, 64))
    shift, scale = rng.standard_normal(64), rng.standard_normal(64)
    r, h = O.gated_residual_adaln(x, -x, np.ones(64), shift, scale, EPS)
    np.testing.assert_array_equal(r, 0.0)
    np.testing.assert_array_equal(h, np.broadcast_to(shift, h.shape))   # LN of a zero row is 0
    y, g = rng.standard_normal((2, 64)), rng.standard_normal(64)
    r, h = O.gated_residual_adaln(x, y, g, shift, scale, EPS)
    np.testing.assert_allclose(h, O.adaln_modulate(x + g * y, shift, scale, EPS), rtol=1e-15, atol=1e-15)


# ----------------------------------------------------------------------------- SiLU / SwiGLU
def test_silu_identities():
    z = np.concatenate([rng.standard_normal(1000) * 5, [0.0, 1e-300, -30.0, 30.0, -800.0, 800.0]])
    s = O.silu(z)
    assert O.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(s - O.silu(-z), z, rtol=1e-13, atol=1e-13)      # silu(z) - silu(-z) = z
    np.testing.assert_allclose(s, z * expit(z), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([-800.0]))[0] == 0.0 and O.silu(np.array([800.0]))[0] == 800.0
    np.testing.assert_allclose(s, torch.nn.functional.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300)


def test_swiglu_halves():
    f = 40
    g = rng.standard_normal((3, f)) * 3
    u = rng.standard_normal((3, f))
    out = O.swiglu(np.concatenate([g, u], axis=1))
    np.testing.assert_allclose(out, g * expit(g) * u, rtol=1e-14)
    # the gate half goes through SiLU, the up half does not
    big = O.swiglu(np.concatenate([np.full((1, f), 50.0), u[:1]], axis=1))
    np.testing.assert_allclose(big, 50.0 * u[:1], rtol=1e-15)
    assert np.all(O.swiglu(np.concatenate([np.zeros((1, f)), u[:1]], axis=1)) == 0.0)
    assert np.all(O.swiglu(np.concatenate([g[:1], np.zeros((1, f))], axis=1)) == 0.0)


# ----------------------------------------------------------------------------- brute force
def test_brute_force_tiny_workload():
    x = make_block_inputs("b_tiny")
    X, Y, GU = np.asarray(x.x, np.float64), np.asarray(x.y, np.float64), np.asarray(x.gate_up, np.float64)
    h = O.adaln_modulate(X, x.shift, x.scale, EPS)
    np.testing.assert_allclose(h, B.adaln_modulate(X.tolist(), x.shift, x.scale, EPS), rtol=1e-12, atol=1e-12)
    r, h2 = O.gated_residual_adaln(X, Y, x.gate, x.shift, x.scale, EPS)
    rb = B.gated_residual(X.tolist(), Y.tolist(), x.gate)
    np.testing.assert_allclose(r, rb, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(h2, B.adaln_modulate(rb, x.shift, x.scale, EPS), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.swiglu(GU), B.swiglu(GU.tolist()), rtol=1e-13, atol=1e-15)


def test_block_inputs_reproducible_and_shaped():
    a, b = make_block_inputs("b_odd"), make_block_inputs("b_odd", threads=1)
    assert a.x.shape == (19, 1032) and a.gate_up.shape == (19, 1552)
    for t in ("x", "y", "gate_up"):
        np.testing.assert_array_equal(getattr(a, t).bits, getattr(b, t).bits)
    np.testing.assert_array_equal(a.gate, b.gate)
    big = np.asarray(a.x)[:, ::128]
    assert np.abs(big).max() > 8.0          # the wide channels are there
