"""The allocation-free dense entry point (dit_attn_dense_noalloc) against dit_attn_dense, through the C ABI.

Its scratch is the library's static per-GPU array, which keeps the previous call's contents.  So each case makes
two calls in a row: the first at the largest size the scratch holds (it fills the whole array), the second smaller
and with a ragged last block, which would read stale data wherever it failed to write its own.  Each output must
equal dit_attn_dense's bit for bit (the same kernels on the same inputs), and it is held to the oracle's bar
(max-abs 2e-2, relative L2 1e-2) on sampled rows.
"""
import numpy as np
import pytest
import torch

import image_diffusion_transformer_amd as dit
from oracle import attention as A
from synth import custom_workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
MAX_ABS, REL_L2 = 2e-2, 1e-2
TILE_BYTES = {96: 48 * 1024, 128: 64 * 1024}


def t16(b):
    return torch.from_numpy(b.bits.view(np.int16)).to(DEV).view(torch.bfloat16)


def upload(x):
    return (t16(x.q), t16(x.k), t16(x.v), torch.from_numpy(x.wq).to(DEV), torch.from_numpy(x.wk).to(DEV))


def scratch_need(T, H, W, heads, d):
    """Bytes the call needs: the RoPE table (rows T + H + W, 256-byte aligned) and heads x ceil(N/128) images."""
    rs = 32 if d == 96 else 44
    table = -(-((T + H + W) * rs * 4) // 256) * 256
    return table + heads * (-(-(T * H * W) // 128)) * TILE_BYTES[d]


# (largest grid first, then a smaller ragged one); both fit 64 MiB.  At head dim 96: 4 heads x 341 blocks =
# 1364 tile images of 48 KiB, 5.4 KB under the limit; at 128: 2 heads x 511 blocks = 1022 images of 64 KiB,
# 18 KB under it.
CASES = [
    (96, 1.0, (1, 128, 341), 4, (3, 10, 12), 3),
    (128, 1.5, (1, 128, 511), 2, (2, 11, 13), 2),
]


@pytest.mark.parametrize("d,scale,big,bheads,small,sheads", CASES, ids=["d96", "d128_scaled_weights"])
def test_noalloc_equals_dense_on_two_calls_in_a_row(d, scale, big, bheads, small, sheads):
    limit = dit.NOALLOC_SCRATCH_BYTES
    assert scratch_need(*big, bheads, d) <= limit < scratch_need(*big, bheads, d) + TILE_BYTES[d]
    calls = []
    for grid, heads, seed in ((big, bheads, 61), (small, sheads, 62)):
        wl = custom_workload(*grid, heads, seed=seed, head_dim=d, weight_scale=scale)
        x = make_inputs(wl)
        q, k, v, wq, wk = upload(x)
        o = torch.empty_like(q)
        print(f"case noalloc d={d} grid={grid} heads={heads} N={wl.N} scratch={scratch_need(*grid, heads, d)}",
              flush=True)
        dit.dit_attn_dense_noalloc(q, k, v, wq, wk, grid, wl.theta, wl.eps, o=o)
        calls.append((wl, x, (q, k, v, wq, wk), o))
    torch.cuda.synchronize()
    for wl, x, (q, k, v, wq, wk), o in calls:
        grid = (wl.T, wl.H, wl.W)
        ref = dit.dit_attn_dense(q, k, v, wq, wk, grid, wl.theta, wl.eps)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), f"noalloc differs from dense at {grid}"
        rows = np.unique(np.concatenate([np.arange(0, wl.N, max(1, wl.N // 300)), np.arange(wl.N - 70, wl.N)]))
        got = o[torch.from_numpy(rows).to(DEV)].float().cpu().numpy().astype(np.float64)
        exp = A.attention(x.q, x.k, x.v, x.wq, x.wk, *grid, wl.theta, wl.eps, rows=rows)
        err = np.abs(got - exp)
        rel = float(np.linalg.norm(err) / np.linalg.norm(exp))
        print(f"noalloc {grid}: max_abs={err.max():.3e} rel_l2={rel:.3e}", flush=True)
        assert np.all(np.isfinite(got)) and err.max() <= MAX_ABS and rel <= REL_L2


def test_noalloc_rejects_a_call_past_the_scratch():
    # 4 heads x 342 blocks at head dim 96: one tile image more than 64 MiB holds
    wl = custom_workload(1, 128, 342, 4, seed=63)
    x = make_inputs(wl)
    q, k, v, wq, wk = upload(x)
    with pytest.raises(dit.DitAttnError, match="static scratch"):
        dit.dit_attn_dense_noalloc(q, k, v, wq, wk, (wl.T, wl.H, wl.W), wl.theta, wl.eps)
