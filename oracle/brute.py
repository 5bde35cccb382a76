"""Brute-force attention in pure Python (no numpy, no BLAS) for tiny grids.

TEST INFRASTRUCTURE ONLY (see oracle/attention.py).  Written independently of
oracle/attention.py, straight from the definition, one scalar at a time, so the
vectorised oracle can be checked against it.
"""
from __future__ import annotations

import math


# channel widths of the t, h, w rotation chunks: equal thirds at 96, (44, 42, 42) at 128
_WIDTHS = {96: (32, 32, 32), 128: (44, 42, 42)}


def _normalise_rotate(vec, weight, t, h, w, theta, eps):
    d = len(vec)
    ms = sum(x * x for x in vec) / d
    inv = 1.0 / math.sqrt(ms + eps)
    xn = [vec[c] * weight[c] * inv for c in range(d)]
    out = list(xn)
    start = 0
    for pos, width in zip((t, h, w), _WIDTHS[d]):
        for i in range(width // 2):
            e = start + 2 * i
            ang = pos * theta ** (-(2.0 * i) / width)
            co, si = math.cos(ang), math.sin(ang)
            out[e] = xn[e] * co - xn[e + 1] * si
            out[e + 1] = xn[e] * si + xn[e + 1] * co
        start += width
    return out


def attention(Q, K, V, wq, wk, T, H, W, theta=1e4, eps=1e-6, mask=None, block=128):
    """O[n][head][c] as nested lists; Q/K/V given as nested [N][heads][96] sequences."""
    N = T * H * W
    heads = len(Q[0])
    d = len(Q[0][0])
    wq = [float(x) for x in wq]
    wk = [float(x) for x in wk]
    pos = [((n // (H * W)), (n // W) % H, n % W) for n in range(N)]
    out = [[[0.0] * d for _ in range(heads)] for _ in range(N)]
    for hd in range(heads):
        qs = [_normalise_rotate([float(x) for x in Q[n][hd]], wq, *pos[n], theta, eps) for n in range(N)]
        ks = [_normalise_rotate([float(x) for x in K[n][hd]], wk, *pos[n], theta, eps) for n in range(N)]
        for i in range(N):
            keys = [j for j in range(N)
                    if mask is None or mask[hd][i // block][j // block]]
            if not keys:
                continue
            lg = [sum(qs[i][c] * ks[j][c] for c in range(d)) / math.sqrt(d) for j in keys]
            top = max(lg)
            ex = [math.exp(x - top) for x in lg]
            tot = sum(ex)
            for c in range(d):
                out[i][hd][c] = sum(ex[a] * float(V[j][hd][c]) for a, j in enumerate(keys)) / tot
    return out


def attention_joint(Q, K, V, wq, wk, q_pos, k_pos, theta=1e4, eps=1e-6):
    """Joint attention with explicit positions, as nested lists: Q [Nq][heads][96] at q_pos [Nq][3],
    K, V [Nkv][heads][96] at k_pos [Nkv][3]; every query sees every key."""
    heads = len(Q[0])
    d = len(Q[0][0])
    wq = [float(x) for x in wq]
    wk = [float(x) for x in wk]
    out = [[[0.0] * d for _ in range(heads)] for _ in range(len(Q))]
    for hd in range(heads):
        qs = [_normalise_rotate([float(x) for x in Q[i][hd]], wq, *[int(p) for p in q_pos[i]], theta, eps)
              for i in range(len(Q))]
        ks = [_normalise_rotate([float(x) for x in K[j][hd]], wk, *[int(p) for p in k_pos[j]], theta, eps)
              for j in range(len(K))]
        for i in range(len(Q)):
            lg = [sum(qs[i][c] * ks[j][c] for c in range(d)) / math.sqrt(d) for j in range(len(K))]
            top = max(lg)
            ex = [math.exp(x - top) for x in lg]
            tot = sum(ex)
            for c in range(d):
                out[i][hd][c] = sum(ex[j] * float(V[j][hd][c]) for j in range(len(K))) / tot
    return out


# ----------------------------------------------------------------------------
# Operators around attention, one scalar at a time (checks oracle/block_ops.py).
# ----------------------------------------------------------------------------

def adaln_modulate(rows, shift, scale, eps=1e-6):
    """LayerNorm without affine parameters, then * (1 + scale) + shift, per row of a nested list."""
    out = []
    for row in rows:
        d = len(row)
        mean = 0.0
        for v in row:
            mean += float(v)
        mean /= d
        var = 0.0
        for v in row:
            var += (float(v) - mean) ** 2
        var /= d
        inv = 1.0 / math.sqrt(var + eps)
        out.append([(float(row[c]) - mean) * inv * (1.0 + float(scale[c])) + float(shift[c]) for c in range(d)])
    return out


def gated_residual(rows_x, rows_y, gate):
    return [[float(x[c]) + float(gate[c]) * float(y[c]) for c in range(len(x))] for x, y in zip(rows_x, rows_y)]


def swiglu(rows):
    """First half of each row is the gate, second half the up projection."""
    out = []
    for row in rows:
        f = len(row) // 2
        res = []
        for c in range(f):
            g = float(row[c])
            sig = 1.0 / (1.0 + math.exp(-g)) if g > -700.0 else 0.0
            res.append(g * sig * float(row[f + c]))
        out.append(res)
    return out
