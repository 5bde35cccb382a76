"""Block router of the block-sparse attention mode, as an exact fp32 specification.

TEST INFRASTRUCTURE ONLY (see oracle/attention.py for who may import it).

Source: the H3 SGLang report (CocoLoop), SubBlock-Sparse-Attention paragraph in
the section on the three acceleration tiers: a block-wise sparse router prunes
the KV blocks that take part in attention, at sparsity 0.75 or 0.80.  The page
gives no formula; the reading used here (each item is a reading where the page
is silent):

* blocks are 128 consecutive tokens of the flattened grid, for queries and
  keys alike; the last block holds the remainder;
* the router pools the post-RMSNorm, post-RoPE q and k (the vectors attention
  itself uses) by their mean over each block, in fp32;
* block score s_ij = dot(qbar_i, kbar_j) with no 1/sqrt(d) (rank-invariant);
* every query block keeps its own (diagonal) KV block: s_ii = +inf;
* keep = nb - floor(sparsity * nb + 1e-9), clamped to [1, nb]; the kept set
  is the first `keep` blocks under (score descending, block index ascending).

To make the mask reproducible bit for bit, every arithmetic step has a fixed
fp32 order (below).  ``route_mask`` evaluates it in float64 and rounds to fp32
after every single operation; for +, -, *, / and sqrt that equals IEEE fp32
because float64 carries more than 2*24+2 bits (double rounding is innocuous --
S. Figueroa, "When is double rounding innocuous?", 1995).
``route_mask_f32`` is a second, independent evaluation in numpy float32
arithmetic; the two must agree bitwise.

  R0 c[a][p][i] = fl(cos(p * theta^(-2i/w_a))), s likewise, w_a the channel width of axis a
     (32 each at head dim d = 96; 44, 42, 42 at d = 128, see attention.ROPE_SPLITS); angle in
     fp64, cos/sin from the C library (Python's math module).
  R1 ss = 0; for c in 0..d-1: ss = fl(ss + fl(x_c * x_c))
     ms = fl(ss / d); r = fl(1 / fl(sqrt(fl(ms + eps))))
  R2 xh_c = fl(fl(x_c * r) * w_c)
     y_e = fl(fl(xh_e * c) - fl(xh_f * s)); y_f = fl(fl(xh_e * s) + fl(xh_f * c))
  R3 acc = 0; for tokens n of block b ascending: acc = fl(acc + y_c[n])
     mean = fl(acc / count_b)
  R4 acc = 0; for c in 0..d-1: acc = fl(acc + fl(qbar_i,c * kbar_j,c)); s_ii = +inf
  R5 top-`keep` selection under (score desc, j asc); -0.0 == +0.0.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import rope_split


def keep_count(nb: int, sparsity: float) -> int:
    """Number of KV blocks kept per query block: nb - floor(s*nb + 1e-9), clamped to [1, nb].

    ``sparsity`` is taken at float32 precision (the value a caller passes across the C ABI).
    """
    s = float(np.float32(sparsity))
    k = nb - int(math.floor(s * nb + 1e-9))
    return max(1, min(nb, k))


def rope_tables_f32(T: int, H: int, W: int, theta: float, split=(32, 32, 32)):
    """R0: fp32 cos/sin tables per axis, [T|H|W][width/2] each, returned as float64 arrays."""
    th = float(np.float32(theta))
    out = []
    for npos, width in zip((T, H, W), split):
        pairs = width // 2
        c = np.empty((npos, pairs), dtype=np.float64)
        s = np.empty((npos, pairs), dtype=np.float64)
        for i in range(pairs):
            inv = th ** (-2 * i / width)
            for p in range(npos):
                ang = p * inv
                c[p, i] = float(np.float32(math.cos(ang)))
                s[p, i] = float(np.float32(math.sin(ang)))
        out.append((c, s))
    return out


def _fl(x):
    """Round float64 values to the nearest float32 (ties to even), kept as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _positions(T, H, W):
    n = np.arange(T * H * W, dtype=np.int64)
    return n // (H * W), (n // W) % H, n % W


def _prepare_f64r(x, w, tabs, T, H, W, eps):
    """R1 + R2 for one head: x [N, d] -> y [N, d] (fp32 values in float64)."""
    x = np.asarray(x, dtype=np.float64)
    N, D = x.shape
    ss = np.zeros(N)
    for c in range(D):
        ss = _fl(ss + _fl(x[:, c] * x[:, c]))
    ms = _fl(ss / float(D))
    r = _fl(1.0 / _fl(np.sqrt(_fl(ms + float(np.float32(eps))))))
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    xh = _fl(_fl(x * r[:, None]) * w[None, :])
    y = np.empty_like(xh)
    pos = _positions(T, H, W)
    o = 0
    for a, width in enumerate(rope_split(D)):
        c = tabs[a][0][pos[a]]   # [N, width/2]
        s = tabs[a][1][pos[a]]
        e = xh[:, o:o + width:2]
        f = xh[:, o + 1:o + width:2]
        y[:, o:o + width:2] = _fl(_fl(e * c) - _fl(f * s))
        y[:, o + 1:o + width:2] = _fl(_fl(e * s) + _fl(f * c))
        o += width
    return y


def _pool_f64r(y, block):
    """R3: sequential fp32 block sums, then division by the true token count."""
    N, D = y.shape
    nb = -(-N // block)
    pad = nb * block - N
    yp = np.concatenate([y, np.zeros((pad, D))]) if pad else y
    yb = yp.reshape(nb, block, D)
    count = np.full(nb, float(block))
    count[-1] = N - (nb - 1) * block
    acc = np.zeros((nb, D))
    for p in range(block):
        live = (p < count)[:, None]
        acc = np.where(live, _fl(acc + yb[:, p, :]), acc)
    return _fl(acc / count[:, None])


def _scores_f64r(qbar, kbar):
    """R4: sequential fp32 dot products, diagonal forced to +inf."""
    nb, D = qbar.shape
    acc = np.zeros((nb, nb))
    for c in range(D):
        acc = _fl(acc + _fl(qbar[:, c][:, None] * kbar[:, c][None, :]))
    np.fill_diagonal(acc, np.inf)
    return acc


def select_topk(scores: np.ndarray, keep: int) -> np.ndarray:
    """R5: uint8 [nb, nb] mask of the first `keep` blocks per row under (score desc, j asc)."""
    nb = scores.shape[0]
    s = np.where(scores == 0.0, 0.0, scores)            # -0.0 ranks as +0.0
    rows = np.repeat(np.arange(nb), nb)
    cols = np.tile(np.arange(nb), nb)
    order = np.lexsort((cols, -s.reshape(-1), rows))     # primary: row, then -score, then j
    rank = np.empty(nb * nb, dtype=np.int64)
    rank[order] = np.tile(np.arange(nb), nb)
    return (rank.reshape(nb, nb) < keep).astype(np.uint8)


def route_scores(Q, K, wq, wk, T, H, W, theta=1e4, eps=1e-6, block=128, heads=None):
    """R0-R4 per head: list of fp32-exact score matrices [nb, nb] (float64 holding fp32 values)."""
    tabs = rope_tables_f32(T, H, W, theta, rope_split(Q.shape[2]))
    nheads = Q.shape[1]
    heads = range(nheads) if heads is None else heads
    out = []
    for hd in heads:
        yq = _prepare_f64r(Q[:, hd, :], wq, tabs, T, H, W, eps)
        yk = _prepare_f64r(K[:, hd, :], wk, tabs, T, H, W, eps)
        out.append(_scores_f64r(_pool_f64r(yq, block), _pool_f64r(yk, block)))
    return out


def route_mask(Q, K, wq, wk, T, H, W, sparsity, theta=1e4, eps=1e-6, block=128, heads=None):
    """Kept-block mask uint8 [heads, nb, nb] of the fp32 router specification."""
    N = T * H * W
    nb = -(-N // block)
    keep = keep_count(nb, sparsity)
    sc = route_scores(Q, K, wq, wk, T, H, W, theta, eps, block, heads)
    return np.stack([select_topk(s, keep) for s in sc])


# ----------------------------------------------------------------------------
# Independent second evaluation in numpy float32 arithmetic (cross-check).
# ----------------------------------------------------------------------------

def route_scores_f32(Q, K, wq, wk, T, H, W, theta=1e4, eps=1e-6, block=128, heads=None):
    """R0-R4 with float32 numpy operations (each op rounds to fp32; no fusion)."""
    f = np.float32
    N = T * H * W
    nb = -(-N // block)
    D = Q.shape[2]
    split = rope_split(D)
    th = float(np.float32(theta))
    tabs = []
    for npos, width in zip((T, H, W), split):
        pairs = width // 2
        c = np.array([[math.cos(p * th ** (-2 * i / width)) for i in range(pairs)] for p in range(npos)],
                     dtype=np.float32).reshape(npos, pairs)
        s = np.array([[math.sin(p * th ** (-2 * i / width)) for i in range(pairs)] for p in range(npos)],
                     dtype=np.float32).reshape(npos, pairs)
        tabs.append((c, s))
    pos = _positions(T, H, W)
    eps32 = f(eps)
    out = []
    nheads = Q.shape[1]
    heads = range(nheads) if heads is None else heads

    def prep(x, w):
        x = np.asarray(x, dtype=np.float32)
        ss = np.zeros(N, dtype=np.float32)
        for c in range(D):
            ss = ss + x[:, c] * x[:, c]
        ms = ss / f(D)
        r = f(1.0) / np.sqrt(ms + eps32)
        xh = (x * r[:, None]) * np.asarray(w, dtype=np.float32)[None, :]
        y = np.empty_like(xh)
        off = 0
        for a, width in enumerate(split):
            c = tabs[a][0][pos[a]]
            s = tabs[a][1][pos[a]]
            e = xh[:, off:off + width:2]
            o = xh[:, off + 1:off + width:2]
            y[:, off:off + width:2] = e * c - o * s
            y[:, off + 1:off + width:2] = e * s + o * c
            off += width
        return y

    def pool(y):
        acc = np.zeros((nb, D), dtype=np.float32)
        blocks = np.arange(nb)
        for p in range(block):
            n = blocks * block + p
            live = n < N
            acc[live] = acc[live] + y[n[live]]
        count = np.minimum(N - blocks * block, block).astype(np.float32)
        return acc / count[:, None]

    for hd in heads:
        qb = pool(prep(Q[:, hd, :], wq))
        kb = pool(prep(K[:, hd, :], wk))
        acc = np.zeros((nb, nb), dtype=np.float32)
        for c in range(D):
            acc = acc + qb[:, c][:, None] * kb[:, c][None, :]
        np.fill_diagonal(acc, np.float32(np.inf))
        out.append(acc)
    return out


# ----------------------------------------------------------------------------
# Exact (float64, no rounding) scores -- used to pin the meaning of the router.
# ----------------------------------------------------------------------------

def route_scores_exact(Q, K, wq, wk, T, H, W, theta=1e4, eps=1e-6, block=128, head=0):
    """qbar_i . kbar_j in float64 from the float64 RMSNorm+RoPE (no fp32 rounding, no diagonal)."""
    from .attention import prepare
    N = T * H * W
    nb = -(-N // block)
    q = prepare(np.asarray(Q[:, head, :], np.float64), wq, T, H, W, theta, eps)
    k = prepare(np.asarray(K[:, head, :], np.float64), wk, T, H, W, theta, eps)
    qb = np.stack([q[b * block:min(N, (b + 1) * block)].mean(axis=0) for b in range(nb)])
    kb = np.stack([k[b * block:min(N, (b + 1) * block)].mean(axis=0) for b in range(nb)])
    return qb @ kb.T
