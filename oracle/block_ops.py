"""fp64 reference for the elementwise operators around attention in the DiT block.

TEST INFRASTRUCTURE ONLY.  This is the slow, plain CPU definition the HIP
kernels are checked against.  Only the tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import it; the product path never
does.

Source: the H3 SGLang report (CocoLoop), fused-operator paragraph in the section
on the three stacked acceleration tiers -- the AdaLN update, the gated residual
path and the SwiGLU activation are fused kernels that leave every result
unchanged; H3-Image spec table, "DiT" row -- hidden 5376, FFN 14336.  The pages
name the operators but not their formulas; the readings are:

1. AdaLN update: LayerNorm over the hidden channels of each token, without
   affine parameters, population variance, eps inside the square root; then
   h = LN(x) * (1 + scale) + shift with per-channel shift and scale vectors
   (the adaptive-LayerNorm modulation of diffusion transformers).
2. Gated residual: r = x + gate * y, gate a per-channel vector, y the output of
   the attention or FFN branch.
3. Gated residual followed by the next AdaLN update, as one operator: the
   update normalises the exact sum r (not a rounded copy of it).
4. SwiGLU: the FFN's fused up projection yields [tokens][2 F]; the first F
   columns are the gate g, the last F the up projection u;
   out = silu(g) * u with silu(z) = z / (1 + exp(-z)).

Everything is float64 on the exact input values.
"""
from __future__ import annotations

import numpy as np


def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) over the last axis; mean and variance are population moments."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def adaln_modulate(x, shift, scale, eps: float = 1e-6) -> np.ndarray:
    """h = LN(x) * (1 + scale) + shift (reading 1)."""
    shift = np.asarray(shift, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    return layer_norm(x, eps) * (1.0 + scale) + shift


def gated_residual(x, y, gate) -> np.ndarray:
    """r = x + gate * y (reading 2)."""
    return np.asarray(x, dtype=np.float64) + np.asarray(gate, dtype=np.float64) * np.asarray(y, dtype=np.float64)


def gated_residual_adaln(x, y, gate, shift, scale, eps: float = 1e-6):
    """(r, h): the gated residual and the AdaLN update of the exact r (reading 3)."""
    r = gated_residual(x, y, gate)
    return r, adaln_modulate(r, shift, scale, eps)


def silu(z) -> np.ndarray:
    """z / (1 + exp(-z)); exp overflows to inf for very negative z, giving -0."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(gate_up) -> np.ndarray:
    """silu(g) * u for gate_up = [g | u] along the last axis (reading 4)."""
    gu = np.asarray(gate_up, dtype=np.float64)
    f = gu.shape[-1] // 2
    return silu(gu[..., :f]) * gu[..., f:]
