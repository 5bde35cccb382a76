"""Dense calls whose last round of workgroups is partly filled split those query tiles along the keys.

The query tiles run as 8 XCD runs of ceil(tiles / 8) each, 32 CUs per XCD and one workgroup per CU.  When a
run has at least 4 full rounds and a last round of rem < 32 tiles, and cutting each of those tiles into P
(2..4) key-range pieces saves at least 1% of the call, the pieces write fp32 partial results that a merge
kernel sums.  The rule is restated here to find the split tiles, which are then checked:
  * against the fp64 oracle (static and running-maximum softmax, head dim 96 and 128, and the full-size
    7-head share of the 5 s video layer, the sharded case the split is for);
  * against the block-sparse call with an all-ones mask, which never splits: every other tile bitwise equal,
    split tiles within the rounding of a different summation order;
  * for determinism: a repeated call and the reversed workgroup order give the same bits;
  * the joint call at grid positions makes the same split and equals the dense call bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import image_diffusion_transformer_amd as dit
from oracle import attention as A
from synth import custom_workload, make_inputs, make_joint_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
MAX_ABS, REL_L2 = 2e-2, 1e-2


def upload(x):
    def t(b):
        return torch.from_numpy(b.bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return (t(x.q), t(x.k), t(x.v), torch.from_numpy(x.wq).to(DEV), torch.from_numpy(x.wk).to(DEV))


def plan(total, nk):
    per = (total + 7) // 8
    rounds, rem = divmod(per, 32)
    if rounds < 4 or rem == 0 or (nk + 127) // 128 < 16:
        return per, per, 0, 1
    best, cost = 1, 1.0
    for p in range(2, 5):
        c = math.ceil(rem * p / 32) / p
        if c < cost - 1e-9:
            best, cost = p, c
    if (1 - cost) / (rounds + 1) < 0.01:
        return per, per, 0, 1
    return per, per - rem, rem, best


def query_tile(d):
    return 512 if d == 96 else 256


def split_tiles(wl):
    """(head, query tile) pairs the dense call splits, and the number of pieces."""
    bq = query_tile(wl.head_dim)
    nqt = -(-wl.N // bq)
    total = wl.heads * nqt
    per, main, rem, pieces = plan(total, wl.N)
    out = []
    for x in range(8):
        for t in range(rem):
            logical = x * per + main + t
            if logical < total:
                out.append(divmod(logical, nqt))
    return out, pieces


def rows_of(wl, qt):
    """First and last 128-query block of query tile qt (clipped to the grid)."""
    bq = query_tile(wl.head_dim)
    lo, hi = qt * bq, min(wl.N, (qt + 1) * bq)
    return np.unique(np.concatenate([np.arange(lo, min(hi, lo + 128)), np.arange(max(lo, hi - 128), hi)]))


@pytest.mark.parametrize("name,pieces", [("t9", 2), ("t9o", 2), ("t6_128", 4), ("t6_128o", 4), ("v5h7", 4)])
def test_split_tiles_match_the_oracle(name, pieces):
    x = make_inputs(name)
    wl = x.workload
    tiles, p = split_tiles(wl)
    assert p == pieces and len(tiles) > 0
    q, k, v, wq, wk = upload(x)
    o = dit.dit_attn_dense(q, k, v, wq, wk, (wl.T, wl.H, wl.W), wl.theta, wl.eps)
    torch.cuda.synchronize()
    split = set(tiles)
    nqt = -(-wl.N // query_tile(wl.head_dim))
    plain = next((h, t) for h in range(wl.heads) for t in range(nqt) if (h, t) not in split)
    for head, qt in [tiles[0], tiles[len(tiles) // 2], tiles[-1], plain]:
        rows = rows_of(wl, qt)
        ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, wl.theta, wl.eps, heads=[head], rows=rows)
        got = o[torch.from_numpy(rows).to(DEV), head].float().cpu().numpy().astype(np.float64)
        err = np.abs(got - ref[:, 0])
        rel = float(np.linalg.norm(err) / np.linalg.norm(ref))
        print(f"{name} head {head} tile {qt} ({'split' if (head, qt) in split else 'whole'}): "
              f"max_abs={err.max():.3e} rel_l2={rel:.3e}", flush=True)
        assert np.all(np.isfinite(got))
        assert err.max() <= MAX_ABS and rel <= REL_L2


@pytest.mark.parametrize("name", ["t9", "t6_128"])
def test_split_against_the_unsplit_block_sparse_path(name):
    x = make_inputs(name)
    wl = x.workload
    tiles, _ = split_tiles(wl)
    q, k, v, wq, wk = upload(x)
    g = (wl.T, wl.H, wl.W)
    dense = dit.dit_attn_dense(q, k, v, wq, wk, g, wl.theta, wl.eps)
    ones = torch.ones((wl.heads, wl.nb, wl.nb), dtype=torch.uint8, device=DEV)
    sparse = dit.dit_attn_block_sparse(q, k, v, wq, wk, g, ones, wl.theta, wl.eps)
    torch.cuda.synchronize()
    bq = query_tile(wl.head_dim)
    in_split = torch.zeros((wl.N, wl.heads), dtype=torch.bool, device=DEV)
    for head, qt in tiles:
        in_split[qt * bq:min(wl.N, (qt + 1) * bq), head] = True
    same = torch.eq(dense, sparse).all(dim=2)
    assert bool(same[~in_split].all()), "a tile that is not split differs from the unsplit path"
    diff = (dense.float() - sparse.float()).abs()[in_split]
    print(f"{name}: split tiles differ from the unsplit path in {int((diff > 0).sum())} of {diff.numel()} "
          f"elements, max {float(diff.max()):.3e}", flush=True)
    assert float(diff.max()) <= 2e-3


@pytest.mark.parametrize("name", ["t9", "t9o", "t6_128", "t6_128o"])
def test_split_is_deterministic_in_either_workgroup_order(name):
    x = make_inputs(name)
    wl = x.workload
    q, k, v, wq, wk = upload(x)
    g = (wl.T, wl.H, wl.W)
    a = dit.dit_attn_dense(q, k, v, wq, wk, g, wl.theta, wl.eps)
    b = dit.dit_attn_dense(q, k, v, wq, wk, g, wl.theta, wl.eps)
    try:
        dit.dit_attn_set_launch_order(1)
        c = dit.dit_attn_dense(q, k, v, wq, wk, g, wl.theta, wl.eps)
    finally:
        dit.dit_attn_set_launch_order(0)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_joint_at_grid_positions_splits_alike():
    x = make_inputs("t9")
    wl = x.workload
    q, k, v, wq, wk = upload(x)
    pos = torch.from_numpy(np.stack(A.positions(wl.T, wl.H, wl.W), axis=1).astype(np.int32)).to(DEV)
    a = dit.dit_attn_dense(q, k, v, wq, wk, (wl.T, wl.H, wl.W), wl.theta, wl.eps)
    b = dit.dit_attn_joint(q, k, v, wq, wk, pos, pos, int(pos.max()) + 1, wl.theta, wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_joint_with_more_keys_than_queries_splits_against_the_oracle():
    """Joint call, 65,536 target queries against 82,432 keys (text, one reference image, target), 9 heads:
    its split tiles cut the longer key range."""
    x = make_joint_inputs("j_ref9")
    wl = x.workload
    nqt = -(-wl.Nq // 512)
    total = wl.heads * nqt
    per, main, rem, pieces = plan(total, wl.Nkv)
    assert pieces == 2 and rem > 0
    t16 = lambda b: torch.from_numpy(b.bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    tpos = lambda p: torch.from_numpy(np.ascontiguousarray(p, dtype=np.int32)).to(DEV)
    o = dit.dit_attn_joint(t16(x.q), t16(x.k), t16(x.v), torch.from_numpy(x.wq).to(DEV),
                           torch.from_numpy(x.wk).to(DEV), tpos(x.q_pos), tpos(x.k_pos), x.max_pos, wl.theta, wl.eps)
    torch.cuda.synchronize()
    split = [divmod(x0 * per + main + t, nqt) for x0 in range(8) for t in range(rem) if x0 * per + main + t < total]
    for head, qt in [split[0], split[-1], (0, 0)]:
        rows = np.concatenate([np.arange(qt * 512, qt * 512 + 128), np.arange(qt * 512 + 384, qt * 512 + 512)])
        ref = A.attention_joint(x.q, x.k, x.v, x.wq, x.wk, x.q_pos, x.k_pos, wl.theta, wl.eps, heads=[head],
                                rows=rows)
        got = o[torch.from_numpy(rows).to(DEV), head].float().cpu().numpy().astype(np.float64)
        err = np.abs(got - ref[:, 0])
        rel = float(np.linalg.norm(err) / np.linalg.norm(ref))
        print(f"j_ref9 head {head} tile {qt}: max_abs={err.max():.3e} rel_l2={rel:.3e}", flush=True)
        assert np.all(np.isfinite(got)) and err.max() <= MAX_ABS and rel <= REL_L2


# Seeded shapes in the split regime with ragged last blocks, both head dims, 2-4 pieces; the last two with one
# large w_q channel, which sends them to the running-maximum kernels.
SHAPES = [(6, 84, 70, 12, 128, 0.0), (5, 79, 59, 16, 128, 0.0), (5, 92, 76, 23, 96, 0.0),
          (6, 79, 85, 14, 128, 6.0), (5, 92, 76, 23, 96, 6.0)]


@pytest.mark.parametrize("T,H,W,heads,d,spike", SHAPES)
def test_split_on_seeded_ragged_shapes(T, H, W, heads, d, spike):
    wl = custom_workload(T, H, W, heads, seed=50 + T + H + W + heads, smooth=True, head_dim=d, wq_spike=spike)
    print(f"case {wl.name} d={d} spike={spike}", flush=True)
    x = make_inputs(wl)
    tiles, p = split_tiles(wl)
    assert p > 1 and tiles
    q, k, v, wq, wk = upload(x)
    g = (wl.T, wl.H, wl.W)
    o = dit.dit_attn_dense(q, k, v, wq, wk, g, wl.theta, wl.eps)
    try:
        dit.dit_attn_set_launch_order(1)
        o_rev = dit.dit_attn_dense(q, k, v, wq, wk, g, wl.theta, wl.eps)
    finally:
        dit.dit_attn_set_launch_order(0)
    torch.cuda.synchronize()
    assert torch.equal(o, o_rev)
    bq = query_tile(d)
    nqt = -(-wl.N // bq)
    last = next(((h, t) for h, t in tiles if t == nqt - 1), (wl.heads - 1, nqt - 1))
    for head, qt in [tiles[0], tiles[-1], last]:
        rows = rows_of(wl, qt)
        ref = A.attention(x.q, x.k, x.v, x.wq, x.wk, wl.T, wl.H, wl.W, wl.theta, wl.eps, heads=[head], rows=rows)
        got = o[torch.from_numpy(rows).to(DEV), head].float().cpu().numpy().astype(np.float64)
        err = np.abs(got - ref[:, 0])
        rel = float(np.linalg.norm(err) / np.linalg.norm(ref))
        print(f"  head {head} tile {qt} ({'split' if (head, qt) in set(tiles) else 'whole'}): "
              f"max_abs={err.max():.3e} rel_l2={rel:.3e}", flush=True)
        assert np.all(np.isfinite(got)) and err.max() <= MAX_ABS and rel <= REL_L2
