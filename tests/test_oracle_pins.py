"""Pins for the fp64 oracle: closed forms, invariants, special cases and brute force.

Each test is chosen so that a plausible slip in oracle/ (a dropped term, a wrong
sign, index or axis, a transposed operand, eps outside the root, sum instead of
mean, a wrong frequency denominator) makes at least one of them fail.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import brute as B
from oracle import router as R
from synth import custom_workload, make_inputs, make_joint_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng(1234)


# ----------------------------------------------------------------------------- RMSNorm
def test_rmsnorm_rms_closed_form():
    x = rng0.standard_normal((64, 96)) * rng0.uniform(1e-4, 30.0, (64, 1))
    w = 1.0 + 0.1 * rng0.standard_normal(96)
    eps = 1e-6
    y = A.rms_norm(x, w, eps)
    ms = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean((y / w) ** 2, axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)
    # direction of each row is that of x * w
    cos = np.sum(y * (x * w), axis=1) / (np.linalg.norm(y, axis=1) * np.linalg.norm(x * w, axis=1))
    np.testing.assert_allclose(cos, 1.0, rtol=1e-13)


def test_rmsnorm_eps_inside_root_and_mean():
    x = np.full((1, 96), 1e-5)
    y = A.rms_norm(x, np.ones(96), 1e-6)
    np.testing.assert_allclose(y, 1e-5 / math.sqrt(1e-10 + 1e-6), rtol=1e-14)
    y1 = A.rms_norm(np.ones((1, 96)), np.full(96, 2.0), 0.0)
    np.testing.assert_allclose(y1, 2.0, rtol=1e-15)       # mean (not sum) of squares
    assert np.all(A.rms_norm(np.zeros((2, 96)), np.ones(96), 1e-6) == 0.0)


# ----------------------------------------------------------------------------- 3D RoPE
def test_token_flattening():
    T, H, W = 3, 5, 7
    t, h, w = A.positions(T, H, W)
    for n in [0, 1, 6, 7, 34, 35, 104]:
        assert (t[n] * H + h[n]) * W + w[n] == n
    assert (t[35], h[35], w[35]) == (1, 0, 0)
    assert (t[8], h[8], w[8]) == (0, 1, 1)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_rope_worked_rotation(axis):
    """Unit vector on the first channel of an axis chunk rotates by pos * 1 rad, counter-clockwise;
    pair 8 has frequency 10000^(-16/32) = 0.01 exactly; other axes' channels stay put."""
    p = 3
    pos = [np.array([0]), np.array([0]), np.array([0])]
    pos[axis] = np.array([p])
    x = np.zeros((1, 96))
    x[0, 32 * axis] = 1.0
    x[0, 32 * axis + 17] = 2.0          # odd member of pair 8
    other = 32 * ((axis + 1) % 3) + 5
    x[0, other] = 0.7
    y = A.rope_3d(x, *pos, theta=10000.0)
    e = 32 * axis
    assert y[0, e] == pytest.approx(math.cos(p), abs=1e-15)
    assert y[0, e + 1] == pytest.approx(math.sin(p), abs=1e-15)
    assert y[0, e + 16] == pytest.approx(-2.0 * math.sin(0.01 * p), abs=1e-15)
    assert y[0, e + 17] == pytest.approx(2.0 * math.cos(0.01 * p), abs=1e-15)
    assert y[0, other] == 0.7
    np.testing.assert_array_equal(np.delete(y[0], [e, e + 1, e + 16, e + 17, other]), 0.0)


def test_rope_identity_at_origin_and_pair_norms():
    x = rng0.standard_normal((40, 3, 96))
    z = np.zeros(40, dtype=np.int64)
    np.testing.assert_array_equal(A.rope_3d(x, z, z, z, 1e4), x)
    pt, ph, pw = (rng0.integers(0, 60, 40) for _ in range(3))
    y = A.rope_3d(x, pt, ph, pw, 1e4)
    nx = np.hypot(x[..., 0::2], x[..., 1::2])
    ny = np.hypot(y[..., 0::2], y[..., 1::2])
    np.testing.assert_allclose(ny, nx, rtol=1e-14)


def test_rope_relative_position():
    """<R_p a, R_p' b> depends only on p' - p: shifting every position leaves the logits unchanged."""
    a = rng0.standard_normal((30, 96))
    b = rng0.standard_normal((30, 96))
    pa = [rng0.integers(0, 50, 30) for _ in range(3)]
    pb = [rng0.integers(0, 50, 30) for _ in range(3)]
    l0 = np.sum(A.rope_3d(a, *pa, 1e4) * A.rope_3d(b, *pb, 1e4), axis=1)
    sh = [7, 3, 11]
    l1 = np.sum(A.rope_3d(a, *[p + s for p, s in zip(pa, sh)], 1e4)
                * A.rope_3d(b, *[p + s for p, s in zip(pb, sh)], 1e4), axis=1)
    np.testing.assert_allclose(l1, l0, rtol=1e-11, atol=1e-11)


# ----------------------------------------------------------------------------- attention
def _tiny():
    return make_inputs("tiny")


def test_brute_force_tiny_fp32_draw():
    x = _tiny()
    wl = x.workload
    o = A.attention(x.q32, x.k32, x.v32, x.wq, x.wk, wl.T, wl.H, wl.W)
    ob = np.array(B.attention(x.q32.tolist(), x.k32.tolist(), x.v32.tolist(), x.wq, x.wk, wl.T, wl.H, wl.W))
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)


@pytest.mark.slow
def test_brute_force_s1_bf16_inputs():
    x = make_inputs("s1")
    wl = x.workload
    q, k, v = (np.asarray(t) for t in (x.q, x.k, x.v))
    o = A.attention(q, k, v, x.wq, x.wk, wl.T, wl.H, wl.W, chunk=64)
    ob = np.array(B.attention(q.tolist(), k.tolist(), v.tolist(), x.wq, x.wk, wl.T, wl.H, wl.W))
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)


def test_probability_rows_sum_to_one():
    x = make_inputs("s2")
    wl = x.workload
    for hd in range(wl.heads):
        L = A.logits(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, hd)
        P = A.softmax_rows(L)
        assert np.all(P >= 0)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-13)


def test_two_token_closed_form():
    """Grid 1x1x2; q, k nonzero only on channel 0 (t-chunk, t=0 for both) so RoPE is inert."""
    wq = 1.0 + 0.1 * rng0.standard_normal(96)
    wk = 1.0 + 0.1 * rng0.standard_normal(96)
    Q = np.zeros((2, 1, 96)); K = np.zeros((2, 1, 96)); V = rng0.standard_normal((2, 1, 96))
    Q[0, 0, 0] = 1.0; Q[1, 0, 0] = -2.0
    K[0, 0, 0] = 3.0; K[1, 0, 0] = -1.0
    eps = 1e-6
    o = A.attention(Q, K, V, wq, wk, 1, 1, 2, eps=eps)
    for i, qv in enumerate([1.0, -2.0]):
        qh = qv * wq[0] / math.sqrt(qv * qv / 96 + eps)
        k0 = 3.0 * wk[0] / math.sqrt(9.0 / 96 + eps)
        k1 = -1.0 * wk[0] / math.sqrt(1.0 / 96 + eps)
        l0, l1 = qh * k0 / math.sqrt(96), qh * k1 / math.sqrt(96)
        p0 = 1.0 / (1.0 + math.exp(l1 - l0))
        np.testing.assert_allclose(o[i, 0], p0 * V[0, 0] + (1 - p0) * V[1, 0], rtol=1e-13, atol=1e-14)


def test_special_cases():
    rng = np.random.default_rng(5)
    w = 1 + 0.1 * rng.standard_normal(96)
    # single token: O = V
    V1 = rng.standard_normal((1, 2, 96))
    o = A.attention(rng.standard_normal((1, 2, 96)), rng.standard_normal((1, 2, 96)), V1, w, w, 1, 1, 1)
    np.testing.assert_array_equal(o, V1)
    # zero queries: all logits 0, O = mean of V over keys
    T, H, W = 2, 3, 5
    N = T * H * W
    V = rng.standard_normal((N, 2, 96))
    o = A.attention(np.zeros((N, 2, 96)), rng.standard_normal((N, 2, 96)), V, w, w, T, H, W)
    np.testing.assert_allclose(o, np.broadcast_to(V.mean(axis=0), o.shape), rtol=1e-13, atol=1e-14)
    # constant V: O = V
    Vc = np.broadcast_to(rng.standard_normal((1, 2, 96)), (N, 2, 96))
    o = A.attention(rng.standard_normal((N, 2, 96)), rng.standard_normal((N, 2, 96)), Vc, w, w, T, H, W)
    np.testing.assert_allclose(o, np.broadcast_to(Vc[0], o.shape), rtol=1e-13)


def test_sampled_rows_equal_full():
    x = make_inputs("s3")
    wl = x.workload
    full = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W)
    rows = np.array([0, 1, 127, 128, 500, 959])
    part = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, rows=rows, heads=[2, 0])
    np.testing.assert_allclose(part, full[rows][:, [2, 0]], rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------- block-sparse
def test_sparse_all_kept_equals_dense_and_row_wise():
    x = make_inputs("s3")
    wl = x.workload
    nb = wl.nb
    dense = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W)
    ones = np.ones((wl.heads, nb, nb), np.uint8)
    sp = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, mask=ones)
    np.testing.assert_allclose(sp, dense, rtol=0, atol=1e-13)
    # random mask, but row 3 fully kept: block 3's rows equal dense
    m = (np.random.default_rng(3).random((wl.heads, nb, nb)) < 0.4).astype(np.uint8)
    m[:, np.arange(nb), np.arange(nb)] = 1
    m[:, 3, :] = 1
    sp = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, mask=m)
    np.testing.assert_allclose(sp[384:512], dense[384:512], rtol=0, atol=1e-13)
    assert np.max(np.abs(sp[:128] - dense[:128])) > 1e-3


def test_sparse_zero_query_mean_over_kept_and_empty_row():
    x = make_inputs("s3")
    wl = x.workload
    N, nb = wl.N, wl.nb
    m = (np.random.default_rng(4).random((wl.heads, nb, nb)) < 0.5).astype(np.uint8)
    m[1, 2, :] = 0                                   # head 1, query block 2 keeps nothing
    V = np.asarray(x.v).astype(np.float64)
    o = A.attention(np.zeros_like(V), x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, mask=m)
    kb = np.arange(N) // 128
    for hd in range(wl.heads):
        for i in range(nb):
            rows = slice(i * 128, min(N, (i + 1) * 128))
            keep = m[hd, i][kb].astype(bool)
            if keep.any():
                np.testing.assert_allclose(o[rows, hd], np.broadcast_to(V[keep, hd].mean(axis=0), o[rows, hd].shape),
                                           rtol=1e-12, atol=1e-13)
            else:
                assert np.all(o[rows, hd] == 0.0)


def test_sparse_brute_force():
    wl = custom_workload(1, 10, 20, 2, seed=21)        # N = 200: blocks of 128 and 72
    x = make_inputs(wl)
    q, k, v = (np.asarray(t) for t in (x.q, x.k, x.v))
    m = np.array([[[1, 0], [1, 1]], [[0, 1], [0, 0]]], np.uint8)
    o = A.attention(q, k, v, x.wq, x.wk, 1, 10, 20, mask=m)
    sub = list(range(0, 200, 9))
    ob = np.array(B.attention(q.tolist(), k.tolist(), v.tolist(), x.wq, x.wk, 1, 10, 20, mask=m.tolist()))
    np.testing.assert_allclose(o[sub], ob[sub], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- router
def test_keep_count_golden():
    g = json.load(open(os.path.join(GOLD, "keep_counts.json")))
    for c in g["cases"]:
        T, H, W = c["grid"]
        N = T * H * W
        assert N == c["N"]
        nb = -(-N // 128)
        assert nb == c["nb"] and N - (nb - 1) * 128 == c["tail"]
        assert R.keep_count(nb, c["sparsity"]) == c["keep"]


def test_model_shape_golden():
    g = json.load(open(os.path.join(GOLD, "model_shape.json")))
    assert g["hidden"] // g["heads"] == g["head_dim"] == A.D
    assert A.rope_split(A.D) == (g["rope_axis_dim"],) * g["rope_axes"]
    assert g["rope_axes"] * g["rope_axis_dim"] == A.D and A.AXIS == g["rope_axis_dim"]


@pytest.mark.parametrize("name", ["s1", "s3", "s1_128"])
def test_router_score_is_mean_block_logit(name):
    """Bilinearity: qbar_i . kbar_j / sqrt(d) equals the mean logit of block pair (i, j), ragged tail included."""
    x = make_inputs(name)
    wl = x.workload
    N, nb = wl.N, wl.nb
    for hd in range(wl.heads):
        s = R.route_scores_exact(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, head=hd)
        L = A.logits(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, hd)
        for i in range(nb):
            for j in range(nb):
                blk = L[i * 128:min(N, (i + 1) * 128), j * 128:min(N, (j + 1) * 128)]
                assert s[i, j] / math.sqrt(wl.head_dim) == pytest.approx(blk.mean(), rel=1e-11, abs=1e-13)


def test_router_fp32_spec_close_to_exact():
    x = make_inputs("s4")
    wl = x.workload
    sc = R.route_scores(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W)
    for hd in range(wl.heads):
        ex = R.route_scores_exact(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, head=hd)
        f = sc[hd].copy()
        np.fill_diagonal(f, 0.0)
        np.fill_diagonal(ex, 0.0)
        assert np.max(np.abs(f - ex)) <= 1e-5 * np.max(np.abs(ex))


@pytest.mark.parametrize("name", ["s1", "s2", "s3", "s4", "s3_128"])
def test_router_two_fp32_evaluations_bitwise(name):
    x = make_inputs(name)
    wl = x.workload
    a = R.route_scores(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W)
    b = R.route_scores_f32(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W)
    for sa, sb in zip(a, b):
        assert sb.dtype == np.float32
        np.testing.assert_array_equal(sa.astype(np.float32).view(np.uint32), sb.view(np.uint32))


def test_router_zero_query_closed_form_and_ties():
    """Q = 0 -> every score is 0 -> row i keeps i plus the keep-1 lowest other indices."""
    wl = custom_workload(3, 16, 32, 2, seed=8)        # N = 1536, nb = 12
    x = make_inputs(wl)
    nb = wl.nb
    Z = np.zeros(x.q.shape, np.float32)
    for s in [0.0, 0.5, 0.75, 0.8, 0.99]:
        keep = R.keep_count(nb, s)
        m = R.route_mask(Z, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, s)
        for i in range(nb):
            want = {i} | set([j for j in range(nb) if j != i][:keep - 1])
            assert set(np.nonzero(m[0, i])[0]) == want and set(np.nonzero(m[1, i])[0]) == want


def test_router_rows_keep_exactly_k_with_diagonal():
    x = make_inputs("s4")
    wl = x.workload
    for s in [0.5, 0.75, 0.8]:
        m = R.route_mask(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, s)
        keep = R.keep_count(wl.nb, s)
        assert m.shape == (wl.heads, wl.nb, wl.nb)
        assert np.all(m.sum(axis=2) == keep)
        assert np.all(m[:, np.arange(wl.nb), np.arange(wl.nb)] == 1)


def test_select_topk_order():
    s = np.array([[np.inf, 1.0, -0.0, 0.0, 1.0, 2.0],
                  [3.0, np.inf, 3.0, -1.0, 0.0, -0.0],
                  [0.0, -0.0, np.inf, 0.0, 5.0, 5.0]] + [[0.0] * 6] * 3)
    m = R.select_topk(s, 3)
    assert list(np.nonzero(m[0])[0]) == [0, 1, 5]        # 1.0 ties at j=1 and j=4: j=1 wins
    assert list(np.nonzero(m[1])[0]) == [0, 1, 2]
    assert list(np.nonzero(m[2])[0]) == [2, 4, 5]
    m = R.select_topk(s, 5)
    assert list(np.nonzero(m[1])[0]) == [0, 1, 2, 4, 5]     # -0.0 ties +0.0, lower index first


def test_router_fp32_mask_differs_from_exact_only_at_near_ties():
    x = make_inputs("s4")
    wl = x.workload
    keep = R.keep_count(wl.nb, 0.75)
    m32 = R.route_mask(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, 0.75)
    for hd in range(wl.heads):
        ex = R.route_scores_exact(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, head=hd)
        np.fill_diagonal(ex, np.inf)
        m64 = R.select_topk(ex, keep)
        for i in np.nonzero(np.any(m64 != m32[hd], axis=1))[0]:
            row = np.sort(ex[i][np.isfinite(ex[i])])[::-1]
            gap = row[keep - 2] - row[keep - 1]
            assert gap <= 1e-5 * np.max(np.abs(row))


# ------------------------------------------------------------------------------------ joint attention
def test_joint_with_grid_positions_equals_grid_oracle():
    """Joint attention whose tokens sit at their grid positions is the grid layer itself."""
    x = make_inputs("s1")
    wl = x.workload
    pos = np.stack(A.positions(wl.T, wl.H, wl.W), axis=1)
    got = A.attention_joint(x.q, x.k, x.v, x.wq, x.wk, pos, pos, wl.theta, wl.eps)
    ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, wl.theta, wl.eps)
    assert np.max(np.abs(got - ref)) <= 1e-13


def test_joint_shift_of_all_positions_changes_nothing():
    """RoPE rotations compose: shifting every query and key coordinate by the same per-axis offset
    leaves all logits, hence O, unchanged."""
    x = make_joint_inputs("j_small")
    wl = x.workload
    rows = np.arange(0, wl.Nq, 37)
    ref = A.attention_joint(x.q, x.k, x.v, x.wq, x.wk, x.q_pos, x.k_pos, wl.theta, wl.eps, rows=rows)
    off = np.array([7, 3, 11])
    got = A.attention_joint(x.q, x.k, x.v, x.wq, x.wk, x.q_pos + off, x.k_pos + off, wl.theta, wl.eps,
                            rows=rows)
    assert np.max(np.abs(got - ref)) <= 1e-12
    # a shift of the keys alone does change the result (positions do enter)
    moved = A.attention_joint(x.q, x.k, x.v, x.wq, x.wk, x.q_pos, x.k_pos + off, wl.theta, wl.eps, rows=rows)
    assert np.max(np.abs(moved - ref)) > 1e-3


def test_joint_brute_force_tiny():
    x = make_joint_inputs("j_tiny")
    wl = x.workload
    q, k, v = np.asarray(x.q, np.float64), np.asarray(x.k, np.float64), np.asarray(x.v, np.float64)
    ref = np.array(B.attention_joint(q.tolist(), k.tolist(), v.tolist(), x.wq, x.wk, x.q_pos.tolist(),
                                         x.k_pos.tolist(), wl.theta, wl.eps))
    got = A.attention_joint(x.q, x.k, x.v, x.wq, x.wk, x.q_pos, x.k_pos, wl.theta, wl.eps)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_joint_brute_force_queries_shorter_than_keys():
    x = make_joint_inputs("j_small")
    wl = x.workload
    qi = np.array([0, 1, 300, wl.Nq - 1])          # a few queries against all 1314 keys, one head
    q = np.asarray(x.q, np.float64)[qi][:, :1]
    k, v = np.asarray(x.k, np.float64)[:, :1], np.asarray(x.v, np.float64)[:, :1]
    ref = np.array(B.attention_joint(q.tolist(), k.tolist(), v.tolist(), x.wq, x.wk, x.q_pos[qi].tolist(),
                                         x.k_pos.tolist(), wl.theta, wl.eps))
    got = A.attention_joint(x.q, x.k, x.v, x.wq, x.wk, x.q_pos, x.k_pos, wl.theta, wl.eps, heads=[0], rows=qi)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_joint_single_key_gives_v():
    x = make_joint_inputs("j_tiny")
    wl = x.workload
    got = A.attention_joint(x.q, x.k[3:4], x.v[3:4], x.wq, x.wk, x.q_pos, x.k_pos[3:4], wl.theta, wl.eps)
    assert np.array_equal(got, np.broadcast_to(np.asarray(x.v[3:4], np.float64), got.shape))


# ----------------------------------------------------------------------------- head dim 128
SPLIT128 = ((0, 44), (44, 42), (86, 42))          # (first channel, width) of the t, h, w chunks


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_rope128_worked_rotation(axis):
    """d = 128: pair 0 of an axis chunk turns by pos rad; pair i of a chunk of width c turns by
    pos * 10000^(-2i/c): 0.01 for (c, i) = (44, 11), 10^(-4/3) for (42, 7); other chunks stay put."""
    p = 5
    start, width = SPLIT128[axis]
    i2, f2 = (11, 0.01) if width == 44 else (7, 10.0 ** (-4.0 / 3.0))
    pos = [np.array([0]), np.array([0]), np.array([0])]
    pos[axis] = np.array([p])
    x = np.zeros((1, 128))
    x[0, start] = 1.0
    x[0, start + 2 * i2 + 1] = 2.0                       # odd member of pair i2
    other = SPLIT128[(axis + 1) % 3][0] + 3
    x[0, other] = 0.7
    y = A.rope_3d(x, *pos, theta=10000.0)
    assert y[0, start] == pytest.approx(math.cos(p), abs=1e-15)
    assert y[0, start + 1] == pytest.approx(math.sin(p), abs=1e-15)
    assert y[0, start + 2 * i2] == pytest.approx(-2.0 * math.sin(f2 * p), abs=1e-14)
    assert y[0, start + 2 * i2 + 1] == pytest.approx(2.0 * math.cos(f2 * p), abs=1e-14)
    assert y[0, other] == 0.7
    np.testing.assert_array_equal(np.delete(y[0], [start, start + 1, start + 2 * i2, start + 2 * i2 + 1, other]), 0.0)


def test_rope128_chunk_boundaries():
    """A position on one axis moves exactly that axis's channels: [0,44) t, [44,86) h, [86,128) w."""
    x = np.ones((1, 128))
    for axis, (start, width) in enumerate(SPLIT128):
        pos = [np.array([0]), np.array([0]), np.array([0])]
        pos[axis] = np.array([9])
        moved = np.nonzero(A.rope_3d(x, *pos, 1e4)[0] != 1.0)[0]
        assert moved.min() == start and moved.max() == start + width - 1


def test_rope128_norms_and_relative_position():
    a = rng0.standard_normal((30, 128))
    b = rng0.standard_normal((30, 128))
    pa = [rng0.integers(0, 50, 30) for _ in range(3)]
    pb = [rng0.integers(0, 50, 30) for _ in range(3)]
    ya = A.rope_3d(a, *pa, 1e4)
    np.testing.assert_allclose(np.hypot(ya[:, 0::2], ya[:, 1::2]), np.hypot(a[:, 0::2], a[:, 1::2]), rtol=1e-14)
    l0 = np.sum(ya * A.rope_3d(b, *pb, 1e4), axis=1)
    sh = [4, 13, 2]
    l1 = np.sum(A.rope_3d(a, *[p + q for p, q in zip(pa, sh)], 1e4)
                * A.rope_3d(b, *[p + q for p, q in zip(pb, sh)], 1e4), axis=1)
    np.testing.assert_allclose(l1, l0, rtol=1e-11, atol=1e-11)


def test_brute_force_head_dim_128():
    x = make_inputs("t128")
    wl = x.workload
    q, k, v = (np.asarray(t) for t in (x.q, x.k, x.v))
    o = A.attention(q, k, v, x.wq, x.wk, wl.T, wl.H, wl.W)
    ob = np.array(B.attention(q.tolist(), k.tolist(), v.tolist(), x.wq, x.wk, wl.T, wl.H, wl.W))
    assert o.shape == (32, 2, 128)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    # scale 1/sqrt(128): logits of a two-token grid with q = k = e_0 (t chunk, t = 0: no rotation)
    Q = np.zeros((2, 1, 128)); K = np.zeros((2, 1, 128)); V = rng0.standard_normal((2, 1, 128))
    Q[:, 0, 0] = 1.0; K[0, 0, 0] = 1.0; K[1, 0, 0] = -1.0
    ones = np.ones(128)
    o2 = A.attention(Q, K, V, ones, ones, 1, 1, 2, eps=0.0)
    g = math.sqrt(128.0)                                # |q^| = |k^| = sqrt(128) after the norm
    lg = np.array([g * g, -g * g]) / math.sqrt(128.0)
    p = np.exp(lg - lg.max()); p /= p.sum()
    np.testing.assert_allclose(o2[0, 0], p @ V[:, 0, :], rtol=1e-12)


def test_router_head_dim_128_sparse_brute_force():
    x = make_inputs("s1_128")
    wl = x.workload
    m = R.route_mask(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, 0.5)
    assert m.shape == (2, 2, 2) and np.all(m.sum(axis=2) == R.keep_count(2, 0.5))
    q, k, v = (np.asarray(t) for t in (x.q, x.k, x.v))
    rows = np.array([0, 5, 127, 128, 199])
    o = A.attention(q, k, v, x.wq, x.wk, wl.T, wl.H, wl.W, rows=rows, mask=m)
    ob = np.array(B.attention(q.tolist(), k.tolist(), v.tolist(), x.wq, x.wk, wl.T, wl.H, wl.W, mask=m.tolist()))
    np.testing.assert_allclose(o, ob[rows], rtol=0, atol=1e-12)
