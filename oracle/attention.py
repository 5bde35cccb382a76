"""fp64 reference for QK-RMSNorm + 3D RoPE + bidirectional softmax attention.

TEST INFRASTRUCTURE ONLY.  This is the slow, plain CPU definition the HIP
kernels are checked against.  Only the tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import it; the product path never
does.

What is computed (sources: the H3 SGLang report (CocoLoop), section on the
three stacked acceleration tiers -- the fused-operator paragraph names
"QK-RMSNorm with 3D-RoPE" ahead of attention and the limits section says the
attention is long and non-causal; H3-Image spec table, "DiT" row -- 56 heads,
hidden 5376, 3D multimodal RoPE):

1. token n of a T x H x W grid sits at t = n // (H W), h = (n // W) mod H,
   w = n mod W  (row-major flattening; reading).
2. RMSNorm over the d channels of each (token, head) (d = 96; 128 for the
   head-dim-128 instantiation), weights w_q / w_k shared by all heads, eps
   inside the square root (reading: textbook form).
3. 3D RoPE: at d = 96 channels [0,32) rotate with t, [32,64) with h, [64,96)
   with w; at d = 128 the chunks are [0,44), [44,86), [86,128) (reading, see
   ROPE_SPLITS).  Inside a chunk of width c the pairs are (2i, 2i+1), angle
   pos * theta^(-2i/c) (reading: RoFormer form with the chunk width as the
   denominator).  V is neither normalised nor rotated.
4. O = softmax(Q^ K^T / sqrt(d)) V over all keys (non-causal).
5. block-sparse: keys outside the kept 128-token KV blocks of the query's
   block are excluded and the softmax renormalises over the kept keys; a
   query block with no kept block gets O = 0.
6. joint attention (``attention_joint``): queries and keys are separate token
   sets, each token with an explicit integer (t, h, w) position -- the
   single-stream DiT with 3D multimodal RoPE over text, reference-image and
   target tokens (H3-Image spec table, "DiT" and reference-image rows).
   Steps 2-4 are unchanged; only the positions come from the caller.

Everything is float64 on the exact input values.  BLAS matmuls serve as steps;
there is no blocking or online softmax here.
"""
from __future__ import annotations

import math

import numpy as np

D = 96          # head dim: 5376 hidden / 56 heads
AXIS = 32       # channels per RoPE axis (t, h, w) at head dim 96
PAIRS = AXIS // 2

# Channels given to the t, h and w axes.  Head dim 96: three equal chunks of 32.  Head dim 128 (the
# SubBlock precondition in the limits section of the H3 SGLang report): the pages give no split; the
# nearest-equal split into even widths is taken, the remainder going to the first axis: 44, 42, 42.
# Each axis rotates its own pairs (2i, 2i+1) with frequencies theta^(-2i/width).
ROPE_SPLITS = {96: (32, 32, 32), 128: (44, 42, 42)}


def rope_split(d: int):
    """Channel widths of the t, h, w RoPE chunks for head dim d."""
    if d not in ROPE_SPLITS:
        raise ValueError(f"no RoPE split defined for head dim {d}")
    return ROPE_SPLITS[d]


def positions(T: int, H: int, W: int, rows=None):
    """(t, h, w) integer grid coordinates of the given token indices."""
    n = np.arange(T * H * W, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    return n // (H * W), (n // W) % H, n % W


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x * w / sqrt(mean(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * np.asarray(w, dtype=np.float64) / np.sqrt(ms + eps)


def rope_frequencies(theta: float, width: int = AXIS) -> np.ndarray:
    """theta^(-2i/width) for the width/2 pairs of one axis chunk."""
    return float(theta) ** (-2.0 * np.arange(width // 2) / width)


def rope_3d(x: np.ndarray, pt, ph, pw, theta: float) -> np.ndarray:
    """Rotate the (2i, 2i+1) pairs of the t, h and w chunks of x [rows, ..., d] (split by rope_split(d))."""
    x = np.asarray(x, dtype=np.float64)
    y = np.empty_like(x)
    extra = (None,) * (x.ndim - 2)
    o = 0
    for a, (pos, width) in enumerate(zip((pt, ph, pw), rope_split(x.shape[-1]))):
        freq = rope_frequencies(theta, width)
        ang = np.asarray(pos, dtype=np.float64)[:, None] * freq[None, :]     # [rows, width/2]
        c = np.cos(ang)[(slice(None),) + extra + (slice(None),)]
        s = np.sin(ang)[(slice(None),) + extra + (slice(None),)]
        e = x[..., o:o + width:2]
        f = x[..., o + 1:o + width:2]
        y[..., o:o + width:2] = e * c - f * s
        y[..., o + 1:o + width:2] = e * s + f * c
        o += width
    return y


def prepare(x, w, T, H, W, theta, eps, rows=None) -> np.ndarray:
    """RMSNorm then 3D RoPE of x [rows, d] (one head) at the given token indices."""
    pt, ph, pw = positions(T, H, W, rows)
    return rope_3d(rms_norm(x, w, eps), pt, ph, pw, theta)


def _head_slice(X, rows, head):
    if rows is None:
        return np.asarray(X[:, head, :], dtype=np.float64)
    return np.asarray(X[np.asarray(rows), head, :], dtype=np.float64)


def _allowed(mask_h: np.ndarray, rows: np.ndarray, N: int, block: int) -> np.ndarray:
    """[len(rows), N] boolean: key n is in a kept KV block of the row's query block."""
    qb = rows // block
    kb = np.arange(N) // block
    return mask_h[qb][:, kb].astype(bool)


def logits(Q, K, wq, wk, T, H, W, head, rows=None, theta=1e4, eps=1e-6) -> np.ndarray:
    """L = Q^ K^T / sqrt(d) for one head, [len(rows), N]."""
    N = T * H * W
    rows = np.arange(N) if rows is None else np.asarray(rows)
    qh = prepare(_head_slice(Q, rows, head), wq, T, H, W, theta, eps, rows)
    kh = prepare(_head_slice(K, None, head), wk, T, H, W, theta, eps)
    return qh @ kh.T / math.sqrt(qh.shape[-1])


def softmax_rows(L: np.ndarray, allowed: np.ndarray | None = None) -> np.ndarray:
    """Row softmax; excluded entries get probability 0; a row with nothing allowed is all 0."""
    L = np.array(L, dtype=np.float64)
    if allowed is not None:
        L[~allowed] = -np.inf
    m = np.max(L, axis=1, keepdims=True)
    empty = ~np.isfinite(m[:, 0])
    m[empty] = 0.0
    P = np.exp(L - m)
    s = P.sum(axis=1, keepdims=True)
    s[empty] = 1.0
    return P / s


def attention(Q, K, V, wq, wk, T, H, W, theta=1e4, eps=1e-6, heads=None, rows=None,
              mask=None, block=128, chunk=256) -> np.ndarray:
    """O for the selected query rows and heads: float64 [len(rows), len(heads), d].

    Q, K, V are indexable as [N, heads, d] (numpy arrays or synth.BF16Tensor), d = 96 or 128;
    mask (optional) is uint8 [heads, nb, nb] with 1 = KV block kept.
    """
    N = T * H * W
    nheads = Q.shape[1]
    D = Q.shape[2]
    heads = list(range(nheads)) if heads is None else list(heads)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), len(heads), D), dtype=np.float64)
    for hi, hd in enumerate(heads):
        kh = prepare(_head_slice(K, None, hd), wk, T, H, W, theta, eps)
        vh = _head_slice(V, None, hd)
        for r0 in range(0, len(rows), chunk):
            rr = rows[r0:r0 + chunk]
            qh = prepare(_head_slice(Q, rr, hd), wq, T, H, W, theta, eps, rr)
            L = qh @ kh.T / math.sqrt(D)
            allowed = None if mask is None else _allowed(np.asarray(mask[hd]), rr, N, block)
            P = softmax_rows(L, allowed)
            out[r0:r0 + chunk, hi, :] = P @ vh
    return out


def prepare_at(x, w, pos, theta, eps) -> np.ndarray:
    """RMSNorm then 3D RoPE of x [rows, d] (one head) at explicit positions pos [rows, 3]."""
    pos = np.asarray(pos, dtype=np.int64)
    return rope_3d(rms_norm(x, w, eps), pos[:, 0], pos[:, 1], pos[:, 2], theta)


def attention_joint(Q, K, V, wq, wk, q_pos, k_pos, theta=1e4, eps=1e-6, heads=None, rows=None,
                    chunk=256) -> np.ndarray:
    """Joint attention: O for the selected query rows and heads, float64 [len(rows), len(heads), d].

    Q is indexable as [Nq, heads, d] at q_pos [Nq, 3]; K, V as [Nkv, heads, d] at k_pos [Nkv, 3].
    Every query attends to every key (non-causal), softmax scale 1/sqrt(d).
    """
    Nq = Q.shape[0]
    nheads = Q.shape[1]
    D = Q.shape[2]
    q_pos = np.asarray(q_pos)
    k_pos = np.asarray(k_pos)
    heads = list(range(nheads)) if heads is None else list(heads)
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), len(heads), D), dtype=np.float64)
    for hi, hd in enumerate(heads):
        kh = prepare_at(_head_slice(K, None, hd), wk, k_pos, theta, eps)
        vh = _head_slice(V, None, hd)
        for r0 in range(0, len(rows), chunk):
            rr = rows[r0:r0 + chunk]
            qh = prepare_at(_head_slice(Q, rr, hd), wq, q_pos[rr], theta, eps)
            out[r0:r0 + chunk, hi, :] = softmax_rows(qh @ kh.T / math.sqrt(D)) @ vh
    return out
