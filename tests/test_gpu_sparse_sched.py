"""GPU parity of the block-sparse schedule's less common paths, through the C ABI against the fp64
oracle (same tolerances as the other attention tests: max-abs 2e-2, relative L2 1e-2).

The schedule puts each 512-token query tile's four router blocks together greedily: the lowest block not
yet placed, then the block among the next 256 that overlaps the tile's kept union most.  When every one
of those 256 blocks is already placed, it takes the lowest free block anywhere; above 4096 blocks it
takes consecutive blocks.  The output must not depend on any of this; the running-max kernel must
handle the grouped tiles as the static-shift one does."""
import numpy as np
import pytest
import torch

import image_diffusion_transformer_amd as dit
from oracle import attention as A
from oracle import router as R
from synth import custom_workload, make_inputs

from bounds import STATIC_LIMIT, pair_bound, spike_to_bound

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
MAX_ABS, REL_L2 = 2e-2, 1e-2


def upload(x):
    def t(b):
        return torch.from_numpy(b.bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return t(x.q), t(x.k), t(x.v), torch.from_numpy(x.wq).to(DEV), torch.from_numpy(x.wk).to(DEV)


def check_close(got, ref, what):
    err = np.abs(got.astype(np.float64) - ref)
    maxabs = float(err.max())
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30))
    print(f"{what}: max_abs={maxabs:.3e} rel_l2={rel:.3e}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert maxabs <= MAX_ABS and rel <= REL_L2, (what, maxabs, rel)


def window_exhausting_mask(nb, low=85, seed=3):
    """A mask on which the greedy fills a tile's whole 256-block window before the tile is complete.

    Blocks 0..low-1 keep only their own column, so each is a tile's first block and no other low block
    overlaps it.  The next 3*low blocks keep every low column, so each of those tiles takes three of them,
    in order.  Block `low` keeps nothing: it becomes a first block only after all of them are placed,
    and by then its next 255 blocks are taken, it takes the 256th, and its last two come from outside
    the window."""
    m = np.zeros((nb, nb), np.uint8)
    m[np.arange(low), np.arange(low)] = 1
    m[low + 1:low + 1 + 3 * low, :low] = 1
    rng = np.random.default_rng(seed)
    rest = low + 1 + 3 * low
    m[rest:] = rng.random((nb - rest, nb)) < 0.2
    return m


def test_window_exhausted_fallback():
    wl = custom_workload(1, 200, 256, 1, seed=41)          # 51,200 tokens, 400 blocks
    assert wl.nb == 400
    x = make_inputs(wl)
    q, k, v, wq, wk = upload(x)
    mask = window_exhausting_mask(wl.nb)[None]
    g = (wl.T, wl.H, wl.W)
    print("case sparse window-exhausting mask, nb=400", flush=True)
    o = dit.dit_attn_block_sparse(q, k, v, wq, wk, g, torch.from_numpy(mask).to(DEV), wl.theta, wl.eps)
    torch.cuda.synchronize()
    blocks = [0, 84, 85, 86, 340, 341, 342, 343, 399]
    rows = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in blocks])
    got = o[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, wl.theta, wl.eps, rows=rows, mask=mask)
    check_close(got, ref, "window-exhausting mask")
    assert np.all(got[2 * 128:3 * 128] == 0)               # block 85 keeps nothing
    # the blocks the fallback placed give the same bits when run alone
    for b in (342, 343):
        alone = np.zeros_like(mask)
        alone[0, b] = mask[0, b]
        oa = dit.dit_attn_block_sparse(q, k, v, wq, wk, g, torch.from_numpy(alone).to(DEV), wl.theta, wl.eps)
        torch.cuda.synchronize()
        assert torch.equal(oa[b * 128:(b + 1) * 128], o[b * 128:(b + 1) * 128]), f"block {b}"


def test_consecutive_tiles_above_4096_blocks():
    wl = custom_workload(1, 640, 820, 1, seed=42)          # 524,800 tokens, 4100 blocks
    assert wl.nb == 4100
    x = make_inputs(wl)
    q, k, v, wq, wk = upload(x)
    rng = np.random.default_rng(43)
    mask = (rng.random((1, wl.nb, wl.nb)) < 0.03).astype(np.uint8)
    mask[0, np.arange(wl.nb), np.arange(wl.nb)] = 1
    mask[0, 7] = 0
    print("case sparse nb=4100 (consecutive tiles)", flush=True)
    o = dit.dit_attn_block_sparse(q, k, v, wq, wk, (wl.T, wl.H, wl.W), torch.from_numpy(mask).to(DEV),
                                  wl.theta, wl.eps)
    torch.cuda.synchronize()
    blocks = [0, 7, 2049, 4096, 4099]
    rows = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in blocks])
    got = o[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, wl.theta, wl.eps, rows=rows, mask=mask)
    check_close(got, ref, "sparse nb=4100")
    assert np.all(got[128:256] == 0)


@pytest.mark.parametrize("name", ["s4", "s4_128"])
def test_block_sparse_online_softmax_weights(name):
    """Norm weights whose logit bound (90) exceeds the static limit: the running-max kernel runs on the
    grouped tiles (ragged last block included), router mask from the oracle."""
    x = make_inputs(name)
    wl = x.workload
    wq = spike_to_bound(x.wq, x.wk, wl.head_dim, 5)
    assert pair_bound(wq, x.wk, wl.head_dim) > STATIC_LIMIT
    mask = R.route_mask(x.q, x.k, wq, x.wk, wl.T, wl.H, wl.W, 0.75, wl.theta, wl.eps)
    q, k, v, _, wk = upload(x)
    print(f"case sparse online {name}", flush=True)
    o = dit.dit_attn_block_sparse(q, k, v, torch.from_numpy(wq).to(DEV), wk, (wl.T, wl.H, wl.W),
                                  torch.from_numpy(mask).to(DEV), wl.theta, wl.eps)
    torch.cuda.synchronize()
    ref = A.attention(x.q, x.k, x.v, wq, x.wk, wl.T, wl.H, wl.W, wl.theta, wl.eps, mask=mask)
    check_close(o.float().cpu().numpy(), ref, f"sparse online {name}")


@pytest.mark.parametrize("H,nb", [(513, 513), (1024, 1024)])
def test_segment_boundaries(H, nb):
    """Router blocks are grouped in independent segments of 512: 513 blocks leave a segment of one block
    (a tile with three empty slots), 1024 give two full segments."""
    wl = custom_workload(1, H, 128, 2, seed=44)
    assert wl.nb == nb
    x = make_inputs(wl)
    q, k, v, wq, wk = upload(x)
    mask = R.route_mask(x.q, x.k, x.wq, x.wk, wl.T, wl.H, wl.W, 0.75, wl.theta, wl.eps)
    print(f"case sparse segments nb={nb}", flush=True)
    o = dit.dit_attn_block_sparse(q, k, v, wq, wk, (wl.T, wl.H, wl.W), torch.from_numpy(mask).to(DEV),
                                  wl.theta, wl.eps)
    torch.cuda.synchronize()
    blocks = [0, 255, 510, 511, 512, nb - 1]
    rows = np.concatenate([np.arange(b * 128, (b + 1) * 128) for b in sorted(set(blocks))])
    got = o[torch.from_numpy(rows).to(DEV)].float().cpu().numpy()
    ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, wl.theta, wl.eps, rows=rows, mask=mask)
    check_close(got, ref, f"sparse segments nb={nb}")


@pytest.mark.parametrize("d", [96, 128])
@pytest.mark.parametrize("T,H,W,heads", [(1, 1, 1, 1), (1, 1, 5, 2), (1, 1, 257, 3), (3, 7, 11, 5)])
def test_block_sparse_edge_shapes(T, H, W, heads, d):
    """A single token, one short block, a ragged third block, several heads: random masks with an empty
    row in head 0 (that block's output must be exactly 0) and rows kept in full elsewhere."""
    wl = custom_workload(T, H, W, heads, seed=7 * T + H + W, head_dim=d)
    x = make_inputs(wl)
    q, k, v, wq, wk = upload(x)
    rng = np.random.default_rng(T * 100 + W)
    mask = (rng.random((heads, wl.nb, wl.nb)) < 0.5).astype(np.uint8)
    mask[:, np.arange(wl.nb), np.arange(wl.nb)] = 1
    if wl.nb > 1:
        mask[0, 0] = 0
    print(f"case sparse edge {T}x{H}x{W} heads={heads} d={d}", flush=True)
    o = dit.dit_attn_block_sparse(q, k, v, wq, wk, (T, H, W), torch.from_numpy(mask).to(DEV), wl.theta, wl.eps)
    torch.cuda.synchronize()
    assert o.shape == (wl.N, heads, d)
    got = o.float().cpu().numpy()
    ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, T, H, W, wl.theta, wl.eps, mask=mask)
    check_close(got, ref, f"sparse edge {T}x{H}x{W}x{heads} d={d}")
    if wl.nb > 1:
        assert np.all(got[:128, 0] == 0)
