"""GPU parity: the HIP path (called through the C ABI) against the fp64 oracle.

Tolerances: O within max-abs 2e-2 and relative L2 1e-2 of the oracle evaluated on
the same bf16 inputs; the router mask bit-exact; results bitwise reproducible.
"""
import numpy as np
import pytest
import torch

import image_diffusion_transformer_amd as dit
from oracle import attention as A
from oracle import router as R
from synth import WORKLOADS, custom_workload, f32_to_bf16_bits, make_inputs

from bounds import STATIC_LIMIT, UNSHIFTED_LIMIT, pair_bound, spike_to_bound

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
MAX_ABS, REL_L2 = 2e-2, 1e-2


def upload(x):
    def t(b):
        return torch.from_numpy(b.bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return (t(x.q), t(x.k), t(x.v), torch.from_numpy(x.wq).to(DEV), torch.from_numpy(x.wk).to(DEV))


def grid(wl):
    return (wl.T, wl.H, wl.W)


def as_np(o):
    return o.float().cpu().numpy()


def check_close(got, ref, what=""):
    err = np.abs(got.astype(np.float64) - ref)
    maxabs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30))
    print(f"{what}: max_abs={maxabs:.3e} rel_l2={rel:.3e}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert maxabs <= MAX_ABS, (what, maxabs)
    assert rel <= REL_L2, (what, rel)
    return maxabs, rel


def run_dense(x, **kw):
    q, k, v, wq, wk = upload(x)
    wl = x.workload
    o = dit.dit_attn_dense(q, k, v, wq, wk, grid(wl), wl.theta, wl.eps, **kw)
    torch.cuda.synchronize()
    return o


SMALL = ["tiny", "s1", "s2", "s3", "s4"]


@pytest.mark.parametrize("name", SMALL)
def test_dense_small_all_rows(name):
    x = make_inputs(name)
    wl = x.workload
    print(f"case dense {name} N={wl.N} heads={wl.heads}", flush=True)
    got = as_np(run_dense(x))
    ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, wl.theta, wl.eps)
    check_close(got, ref, f"dense {name}")


@pytest.mark.parametrize("T,H,W,heads", [(1, 1, 1, 1), (1, 1, 5, 2), (1, 16, 16, 1), (1, 1, 257, 3),
                                         (3, 7, 11, 5), (2, 9, 29, 56)])
def test_dense_edge_shapes(T, H, W, heads):
    wl = custom_workload(T, H, W, heads, seed=T * 1000 + H * 10 + W)
    x = make_inputs(wl)
    print(f"case dense edge {T}x{H}x{W} heads={heads}", flush=True)
    got = as_np(run_dense(x))
    ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, T, H, W)
    check_close(got, ref, f"dense {T}x{H}x{W}x{heads}")


def test_dense_single_token_is_v():
    wl = custom_workload(1, 1, 1, 4, seed=77)
    x = make_inputs(wl)
    got = run_dense(x)
    q, k, v, wq, wk = upload(x)
    assert torch.equal(got, v)


def test_dense_large_weights_and_theta():
    """Norm weights ~N(3, 0.5) push logits to |l| ~ 90.  The MFMA consumes bf16 q^ and k^, whose
    rounding moves a logit by up to about |l| * 2^-8, so only the relative L2 bound is asserted
    here (max-abs reaches ~0.1 at these logits); the standard-weight cases carry both bounds."""
    wl = custom_workload(2, 12, 20, 3, seed=31, theta=500.0, eps=1e-5)
    x = make_inputs(wl)
    x.wq = (3.0 + 0.5 * np.random.default_rng(1).standard_normal(96)).astype(np.float32)
    x.wk = (3.0 + 0.5 * np.random.default_rng(2).standard_normal(96)).astype(np.float32)
    got = as_np(run_dense(x))
    ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, wl.theta, wl.eps)
    err = np.abs(got - ref)
    rel = np.linalg.norm(err) / np.linalg.norm(ref)
    print(f"dense large weights: max_abs={err.max():.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(got)) and rel <= REL_L2


def aligned_keys(x, wl, qrows, krows, head):
    """Raw keys whose RMSNorm + RoPE output points along the normalised, rotated query of the same
    index: k = R(p_q - p_k)(w_q * q) / w_k, since rotations of one axis compose additively."""
    q = np.asarray(x.q[qrows, head, :], dtype=np.float64) * x.wq
    tq, hq, wq_ = A.positions(wl.T, wl.H, wl.W, qrows)
    tk, hk, wk_ = A.positions(wl.T, wl.H, wl.W, krows)
    u = A.rope_3d(q, tq - tk, hq - hk, wq_ - wk_, wl.theta)
    return f32_to_bf16_bits((u / x.wk).astype(np.float32))


def static_shift_bound(wq, wk, d=96):
    """The kernels' test for the softmax mode, restated: the base-2 logit bound
    log2(e) sqrt(d) max_i u_i v_i (u_i, v_i the larger |weight| of channel pair i of w_q, w_k), with
    the kernels' 2% margin; up to 48 the static kernel takes exp2 of the logits, up to 80 it subtracts the
    constant bound - 48 first, past 80 the running-maximum kernel runs."""
    return pair_bound(wq, wk, d)


@pytest.mark.parametrize("weights", ["standard", "shifted", "online"])
def test_dense_running_max_rescale(weights):
    """Queries 0..63 meet keys aligned with them (logit ~ sqrt(96) ~ 9.4) only in the second tile,
    well above every earlier block max (~3).  With one query weight (channel 0) raised to a logit bound of
    90, past the static limit, the running-max kernel runs, and the block sums of p pass 2^8 there, so its
    max must move, rescaling O and the row sum.  With standard weights the static kernel runs the same
    case, and with that channel at 4 (bound between 48 and 80) the static kernel with its constant shift."""
    wl = custom_workload(1, 5, 40, 2, seed=41, smooth=False)        # N = 200: keys 136..199 aligned
    x = make_inputs(wl)
    N = wl.N
    if weights == "shifted":
        x.wq = x.wq.copy()
        x.wq[0] = 4.0
        assert UNSHIFTED_LIMIT < static_shift_bound(x.wq, x.wk) <= STATIC_LIMIT
    for hd in range(wl.heads):
        x.k.bits[N - 64:, hd, :] = aligned_keys(x, wl, np.arange(64), np.arange(N - 64, N), hd)
    if weights == "online":
        # raised after the keys are aligned (with the standard weights): the late logits stay near 9 instead of
        # growing with the raised channel, where bf16 q^ and k^ would carry about 2.5e-2 of error into O
        x.wq = spike_to_bound(x.wq, x.wk, 96, 0)
        assert static_shift_bound(x.wq, x.wk) > STATIC_LIMIT
    elif weights == "standard":
        assert static_shift_bound(x.wq, x.wk) <= UNSHIFTED_LIMIT
    L = A.logits(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, 0, rows=np.arange(64))
    assert np.all(L[np.arange(64), N - 64 + np.arange(64)] - L[:, :N - 64].max(axis=1) > 8 / np.log2(np.e))
    got = as_np(run_dense(x))
    ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W)
    check_close(got, ref, f"dense late max ({weights} weights)")


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_non_finite_norm_weight_gives_non_finite_rows_not_garbage(bad):
    """A NaN or infinite norm weight has no logit bound, so the running-maximum kernel takes the call (the static
    one returns at once).  Every q^ then carries a non-finite channel, every logit is NaN and so is every O
    element in the fp64 oracle too: the call completes and writes NaN everywhere, dense and block-sparse."""
    x = make_inputs("s3")
    wl = x.workload
    q, k, v, wq, wk = upload(x)
    wq[5] = bad
    with np.errstate(invalid="ignore"):
        ref = A.attention(x.q, x.k, x.v, np.where(np.arange(96) == 5, np.float32(bad), x.wq), x.wk, wl.T, wl.H,
                          wl.W, wl.theta, wl.eps, heads=[0], rows=np.arange(64))
    assert np.all(np.isnan(ref))
    o = dit.dit_attn_dense(q, k, v, wq, wk, grid(wl))
    ones = torch.ones((wl.heads, wl.nb, wl.nb), dtype=torch.uint8, device=DEV)
    os_ = dit.dit_attn_block_sparse(q, k, v, wq, wk, grid(wl), ones)
    torch.cuda.synchronize()
    assert bool(torch.isnan(o).all()) and bool(torch.isnan(os_).all())


def test_dense_deterministic():
    x = make_inputs("s4")
    a = run_dense(x)
    b = run_dense(x)
    assert torch.equal(a, b)


# ---------------------------------------------------------------------------------------------- router
@pytest.mark.parametrize("name", ["s1", "s2", "s3", "s4"])
@pytest.mark.parametrize("sparsity", [0.0, 0.5, 0.75, 0.8])
def test_route_mask_bit_exact_small(name, sparsity):
    x = make_inputs(name)
    wl = x.workload
    q, k, v, wq, wk = upload(x)
    print(f"case route {name} s={sparsity}", flush=True)
    m = dit.dit_attn_route(q, k, wq, wk, grid(wl), sparsity, wl.theta, wl.eps)
    torch.cuda.synchronize()
    ref = R.route_mask(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, sparsity, wl.theta, wl.eps)
    got = m.cpu().numpy()
    assert got.shape == ref.shape
    bad = np.argwhere(np.any(got != ref, axis=2))
    assert bad.size == 0, f"mismatched (head, row) pairs: {bad[:10].tolist()}"


def test_route_ties_and_zero_queries():
    wl = custom_workload(3, 16, 32, 2, seed=8)
    x = make_inputs(wl)
    q, k, v, wq, wk = upload(x)
    z = torch.zeros_like(q)
    m = dit.dit_attn_route(z, k, wq, wk, grid(wl), 0.75).cpu().numpy()
    ref = R.route_mask(np.zeros(x.q.shape, np.float32), x.k, x.wq, x.wk, wl.T, wl.H, wl.W, 0.75)
    np.testing.assert_array_equal(m, ref)


# ---------------------------------------------------------------------------------------------- sparse
@pytest.mark.parametrize("name", ["s1", "s3", "s4"])
@pytest.mark.parametrize("sparsity", [0.5, 0.75])
def test_block_sparse_on_oracle_mask(name, sparsity):
    x = make_inputs(name)
    wl = x.workload
    mask = R.route_mask(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, sparsity, wl.theta, wl.eps)
    q, k, v, wq, wk = upload(x)
    print(f"case sparse {name} s={sparsity}", flush=True)
    o = dit.dit_attn_block_sparse(q, k, v, wq, wk, grid(wl), torch.from_numpy(mask).to(DEV), wl.theta, wl.eps)
    torch.cuda.synchronize()
    ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, wl.theta, wl.eps, mask=mask)
    check_close(as_np(o), ref, f"sparse {name} s={sparsity}")


def test_block_sparse_all_ones_equals_dense_bitwise():
    x = make_inputs("s4")
    wl = x.workload
    q, k, v, wq, wk = upload(x)
    ones = torch.ones((wl.heads, wl.nb, wl.nb), dtype=torch.uint8, device=DEV)
    a = dit.dit_attn_dense(q, k, v, wq, wk, grid(wl))
    b = dit.dit_attn_block_sparse(q, k, v, wq, wk, grid(wl), ones)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_block_sparse_random_mask_with_empty_rows():
    x = make_inputs("s4")
    wl = x.workload
    rng = np.random.default_rng(9)
    mask = (rng.random((wl.heads, wl.nb, wl.nb)) < 0.3).astype(np.uint8)
    mask[0, 5, :] = 0
    mask[1, wl.nb - 1, :] = 0
    mask[1, 0, :] = 1
    q, k, v, wq, wk = upload(x)
    o = dit.dit_attn_block_sparse(q, k, v, wq, wk, grid(wl), torch.from_numpy(mask).to(DEV))
    torch.cuda.synchronize()
    got = as_np(o)
    ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, mask=mask)
    check_close(got, ref, "sparse random mask")
    assert np.all(got[5 * 128:6 * 128, 0] == 0)
    assert np.all(got[(wl.nb - 1) * 128:, 1] == 0)


@pytest.mark.parametrize("name", ["s4", "s4_128"])
def test_block_sparse_rows_do_not_depend_on_other_rows(name):
    """Which router blocks share a query tile is chosen from the whole mask, but each block's output
    must depend only on its own row of the mask: the same block run alone is bitwise equal."""
    x = make_inputs(name)
    wl = x.workload
    mask = R.route_mask(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, 0.75, wl.theta, wl.eps)
    q, k, v, wq, wk = upload(x)
    full = dit.dit_attn_block_sparse(q, k, v, wq, wk, grid(wl), torch.from_numpy(mask).to(DEV), wl.theta, wl.eps)
    for i in (0, 17, wl.nb - 1):
        alone = np.zeros_like(mask)
        alone[:, i] = mask[:, i]
        o = dit.dit_attn_block_sparse(q, k, v, wq, wk, grid(wl), torch.from_numpy(alone).to(DEV), wl.theta, wl.eps)
        torch.cuda.synchronize()
        rows = slice(i * 128, min((i + 1) * 128, wl.N))
        assert torch.equal(o[rows], full[rows]), f"block {i}"
        others = np.ones(wl.N, bool)
        others[rows] = False
        assert torch.count_nonzero(o[torch.from_numpy(others).to(DEV)]) == 0


def test_route_then_sparse_pipeline():
    x = make_inputs("s4")
    wl = x.workload
    q, k, v, wq, wk = upload(x)
    ws = dit.workspace_for(q, grid(wl))
    m = dit.dit_attn_route(q, k, wq, wk, grid(wl), 0.75, workspace=ws)
    o = dit.dit_attn_block_sparse(q, k, v, wq, wk, grid(wl), m, workspace=ws)
    torch.cuda.synchronize()
    mask = R.route_mask(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, 0.75)
    np.testing.assert_array_equal(m.cpu().numpy(), mask)
    ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, mask=mask)
    check_close(as_np(o), ref, "route+sparse")


@pytest.mark.parametrize("bound", [47.0, 79.0])
@pytest.mark.parametrize("sparse", [False, True])
def test_static_rows_whose_logits_are_all_very_negative(sparse, bound):
    """Every key anti-aligned with every query, with logits near -bound in base 2, on a ragged grid
    (500 tokens, so the last KV tile has 12 keys past the grid), under weights that still select the
    static kernel: at a bound of 47 without a shift (row sums about 500 * 2^-46), at 79 with the shift of
    31 (p about 2^-109, the low end of the range the shift guarantees normal).  Keys past the grid must be
    masked out.  If they were counted with p = 1 and their count subtracted at the end, the row sum would
    vanish next to that count in fp32 and O would drop to zero.  q and k put all their energy on the
    lowest-frequency RoPE pair of each axis, whose rotation over the grid is below 0.01 rad."""
    T, H, W, d = 1, 10, 50, 96
    N = T * H * W
    c = np.sqrt(bound / (np.log2(np.e) * np.sqrt(d) * 1.02))
    w = np.full(d, c, dtype=np.float32)
    edge = UNSHIFTED_LIMIT if bound < UNSHIFTED_LIMIT else STATIC_LIMIT
    assert bound - 0.5 < static_shift_bound(w, w) <= edge
    x = np.zeros((N, 1, d), dtype=np.float32)
    x[:, 0, [30, 62, 94]] = 1.0
    rng = np.random.default_rng(11)
    v = rng.standard_normal((N, 1, d)).astype(np.float32)
    qb, kb, vb = f32_to_bf16_bits(x), f32_to_bf16_bits(-x), f32_to_bf16_bits(v)

    def t(bits):
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)

    wt = torch.from_numpy(w).to(DEV)
    if sparse:
        nb = -(-N // 128)
        mask = np.ones((1, nb, nb), dtype=np.uint8)
        o = dit.dit_attn_block_sparse(t(qb), t(kb), t(vb), wt, wt, (T, H, W), torch.from_numpy(mask).to(DEV))
    else:
        o = dit.dit_attn_dense(t(qb), t(kb), t(vb), wt, wt, (T, H, W))
    torch.cuda.synchronize()
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    L = A.logits(f(qb), f(kb), w, w, T, H, W, 0)
    assert L.max() * np.log2(np.e) < -(bound - 2)             # every logit far below zero
    ref = A.attention(f(qb), f(kb), f(vb), w, w, T, H, W)
    assert np.abs(ref[:, 0] - f(vb)[:, 0].mean(axis=0)).max() < 0.05   # nearly uniform weights
    check_close(as_np(o), ref, f"all logits very negative, {'sparse' if sparse else 'dense'}")
