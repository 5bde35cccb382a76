"""GPU parity on seeded random configurations: grid shapes from 1 token up to a few thousand, 1-4 heads,
head dims 96 and 128, two RoPE bases, and all four attention calls (dense, block-sparse on a random mask,
router then block-sparse, joint with random positions and Nq != Nkv), each against the fp64 oracle on
every row.  Cases 16-23 set one random channel of w_q to 4, which takes the pairwise logit bound past 48
(the static mode then shifts its exponent by a constant); cases 24-31 raise one random channel of w_q until
the bound is 90, past the static limit of 80, so the same calls run the running-maximum kernels.  Tolerances
as everywhere: O within max-abs 2e-2 and relative L2 1e-2, masks bit-exact."""
import numpy as np
import pytest
import torch

import image_diffusion_transformer_amd as dit
from oracle import attention as A
from oracle import router as R
from synth import bf16_bits_to_f32, custom_workload, f32_to_bf16_bits, make_inputs

from bounds import STATIC_LIMIT, UNSHIFTED_LIMIT, pair_bound, spike_to_bound

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
MAX_ABS, REL_L2 = 2e-2, 1e-2
MODES = ("dense", "sparse", "route_sparse", "joint")
CASES = 32
BIG_FROM = 16            # cases 16-23: one w_q channel at 4 (shifted static softmax)
ONLINE_FROM = 24         # cases 24-31: one w_q channel raised to a bound of 90 (running-maximum softmax)


def check_close(got, ref, what):
    err = np.abs(got.astype(np.float64) - ref)
    maxabs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30))
    print(f"{what}: max_abs={maxabs:.3e} rel_l2={rel:.3e}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert maxabs <= MAX_ABS and rel <= REL_L2, (what, maxabs, rel)


def t16(bits):
    return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)


def spiked(wq, wk, d, big, online):
    """w_q with channel `big` at 4 (bound between 48 and 80) or raised to a bound of 90; the kernel the bound
    selects is asserted."""
    if online:
        w = spike_to_bound(wq, wk, d, big)
        assert pair_bound(w, wk, d) > STATIC_LIMIT
    else:
        w = np.array(wq, dtype=np.float32, copy=True)
        w[big] = 4.0
        assert UNSHIFTED_LIMIT < pair_bound(w, wk, d) <= STATIC_LIMIT
    return w


def config(i):
    rng = np.random.default_rng(5000 + i)
    mode = MODES[i % 4]
    d = (96, 128)[(i // 4) % 2]
    while True:
        T, H, W = int(rng.integers(1, 5)), int(rng.integers(1, 25)), int(rng.integers(1, 49))
        if T * H * W <= 4000:
            break
    heads = int(rng.integers(1, 5))
    theta = float(rng.choice([1e4, 500.0]))
    return rng, mode, d, (T, H, W), heads, theta


@pytest.mark.parametrize("i", range(CASES))
def test_random_configuration(i):
    rng, mode, d, (T, H, W), heads, theta = config(i)
    big = int(rng.integers(0, d)) if i >= BIG_FROM else None
    online = i >= ONLINE_FROM
    what = (f"case {i}: {mode} d={d} grid={T}x{H}x{W} heads={heads} theta={theta:g} big w_q channel {big}"
            + (" (running max)" if online else ""))
    print(what, flush=True)
    if mode == "joint":
        nq, nk, max_pos = int(rng.integers(1, 600)), int(rng.integers(1, 1500)), int(rng.integers(1, 65))
        q = f32_to_bf16_bits(rng.standard_normal((nq, heads, d)).astype(np.float32))
        k = f32_to_bf16_bits(rng.standard_normal((nk, heads, d)).astype(np.float32))
        v = f32_to_bf16_bits(rng.standard_normal((nk, heads, d)).astype(np.float32))
        qp = rng.integers(0, max_pos, (nq, 3)).astype(np.int32)
        kp = rng.integers(0, max_pos, (nk, 3)).astype(np.int32)
        wq = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
        wk = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
        if big is not None:
            wq = spiked(wq, wk, d, big, online)
        else:
            assert pair_bound(wq, wk, d) <= UNSHIFTED_LIMIT
        o = dit.dit_attn_joint(t16(q), t16(k), t16(v), torch.from_numpy(wq).to(DEV), torch.from_numpy(wk).to(DEV),
                               torch.from_numpy(qp).to(DEV), torch.from_numpy(kp).to(DEV), max_pos, theta)
        torch.cuda.synchronize()
        ref = A.attention_joint(bf16_bits_to_f32(q), bf16_bits_to_f32(k), bf16_bits_to_f32(v), wq, wk, qp, kp,
                                theta)
        check_close(o.float().cpu().numpy(), ref, what + f" nq={nq} nk={nk} max_pos={max_pos}")
        return
    wl = custom_workload(T, H, W, heads, seed=6000 + i, head_dim=d, theta=theta)
    x = make_inputs(wl)
    if big is not None:
        x.wq = spiked(x.wq, x.wk, d, big, online)
    else:
        assert pair_bound(x.wq, x.wk, d) <= UNSHIFTED_LIMIT
    q, k, v = t16(x.q.bits), t16(x.k.bits), t16(x.v.bits)
    wq, wk = torch.from_numpy(x.wq).to(DEV), torch.from_numpy(x.wk).to(DEV)
    g = (T, H, W)
    mask = None
    if mode == "dense":
        o = dit.dit_attn_dense(q, k, v, wq, wk, g, theta, wl.eps)
    elif mode == "sparse":
        mask = (rng.random((heads, wl.nb, wl.nb)) < rng.uniform(0.1, 0.9)).astype(np.uint8)
        if rng.random() < 0.5:
            mask[:, np.arange(wl.nb), np.arange(wl.nb)] = 1
        mask[0, int(rng.integers(0, wl.nb))] = 0                   # one query block keeps nothing
        o = dit.dit_attn_block_sparse(q, k, v, wq, wk, g, torch.from_numpy(mask).to(DEV), theta, wl.eps)
    else:
        sparsity = float(rng.choice([0.5, 0.75, 0.8]))
        m = dit.dit_attn_route(q, k, wq, wk, g, sparsity, theta, wl.eps)
        torch.cuda.synchronize()
        mask = R.route_mask(x.q, x.k, x.wq, x.wk, T, H, W, sparsity, theta, wl.eps)
        np.testing.assert_array_equal(m.cpu().numpy(), mask)
        o = dit.dit_attn_block_sparse(q, k, v, wq, wk, g, m, theta, wl.eps)
    torch.cuda.synchronize()
    ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, T, H, W, theta, wl.eps, mask=mask)
    check_close(o.float().cpu().numpy(), ref, what)
