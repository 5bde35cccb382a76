"""GPU parity of joint attention (explicit 3D positions, separate query and key token sets) against the
fp64 oracle, through the C ABI.  Same tolerances as the grid calls: max-abs 2e-2, relative L2 1e-2."""
import numpy as np
import pytest
import torch

import image_diffusion_transformer_amd as dit
from oracle import attention as A
from synth import WORKLOADS, make_inputs, make_joint_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
MAX_ABS, REL_L2 = 2e-2, 1e-2


def t16(b):
    return torch.from_numpy(b.bits.view(np.int16)).to(DEV).view(torch.bfloat16)


def tpos(p):
    return torch.from_numpy(np.ascontiguousarray(p, dtype=np.int32)).to(DEV)


def check(got, ref, what):
    err = np.abs(got.astype(np.float64) - ref)
    rel = float(np.linalg.norm(err) / np.linalg.norm(ref))
    print(f"{what}: max_abs={err.max():.3e} rel_l2={rel:.3e}", flush=True)
    assert np.all(np.isfinite(got)) and err.max() <= MAX_ABS and rel <= REL_L2, (what, err.max(), rel)


def run_joint(x, q_pos=None, k_pos=None, wq=None, wk=None):
    wl = x.workload
    wq = x.wq if wq is None else wq
    wk = x.wk if wk is None else wk
    o = dit.dit_attn_joint(t16(x.q), t16(x.k), t16(x.v), torch.from_numpy(wq).to(DEV), torch.from_numpy(wk).to(DEV),
                           tpos(x.q_pos if q_pos is None else q_pos), tpos(x.k_pos if k_pos is None else k_pos),
                           x.max_pos, wl.theta, wl.eps)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("name", ["j_tiny", "j_all", "j_small"])
def test_joint_small_all_rows(name):
    x = make_joint_inputs(name)
    wl = x.workload
    print(f"case joint {name} nq={wl.Nq} nk={wl.Nkv}", flush=True)
    got = run_joint(x).float().cpu().numpy()
    ref = A.attention_joint(x.q, x.k, x.v, x.wq, x.wk, x.q_pos, x.k_pos, wl.theta, wl.eps)
    check(got, ref, f"joint {name}")


def test_joint_at_grid_positions_equals_dense_bitwise():
    x = make_inputs("s4")
    wl = x.workload
    g = (wl.T, wl.H, wl.W)
    pos = np.stack(A.positions(wl.T, wl.H, wl.W), axis=1)
    q, k, v = t16(x.q), t16(x.k), t16(x.v)
    wq, wk = torch.from_numpy(x.wq).to(DEV), torch.from_numpy(x.wk).to(DEV)
    a = dit.dit_attn_dense(q, k, v, wq, wk, g)
    b = dit.dit_attn_joint(q, k, v, wq, wk, tpos(pos), tpos(pos), int(pos.max()) + 1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_joint_positions_out_of_range_are_clamped():
    x = make_joint_inputs("j_all")
    qp = x.q_pos.copy()
    kp = x.k_pos.copy()
    qp[::7, 0] = x.max_pos + 5          # clamped to max_pos - 1
    kp[::5, 2] = -3                     # clamped to 0
    a = run_joint(x, qp, kp)
    b = run_joint(x, np.clip(qp, 0, x.max_pos - 1), np.clip(kp, 0, x.max_pos - 1))
    assert torch.equal(a, b)


def test_joint_single_query_and_ragged_keys():
    x = make_joint_inputs("j_small")
    wl = x.workload
    # one query against the first 131 keys (one full tile plus a ragged one)
    q, k, v = t16(x.q)[:1], t16(x.k)[:131], t16(x.v)[:131]
    o = dit.dit_attn_joint(q, k, v, torch.from_numpy(x.wq).to(DEV), torch.from_numpy(x.wk).to(DEV),
                           tpos(x.q_pos[:1]), tpos(x.k_pos[:131]), x.max_pos, wl.theta, wl.eps)
    torch.cuda.synchronize()
    ref = A.attention_joint(x.q[:1], x.k[:131], x.v[:131], x.wq, x.wk, x.q_pos[:1], x.k_pos[:131], wl.theta, wl.eps)
    check(o.float().cpu().numpy(), ref, "joint nq=1 nk=131")


def test_joint_online_softmax_weights():
    """Norm weights whose logit bound exceeds the static-shift limit take the running-max kernel.  One
    large channel weight (4.0) lifts the bound log2(e) sqrt(96) max_i u_i v_i (u_i, v_i the larger
    |weight| of channel pair i of w_q, w_k) above 48 while the typical logit stays of the usual size."""
    x = make_joint_inputs("j_small")
    wl = x.workload
    wq = x.wq.copy()
    wq[5] = 4.0
    wk = x.wk
    got = run_joint(x, wq=wq, wk=wk).float().cpu().numpy()
    ref = A.attention_joint(x.q, x.k, x.v, wq, wk, x.q_pos, x.k_pos, wl.theta, wl.eps)
    check(got, ref, "joint online")


def test_joint_edit_two_references_full_size_sampled():
    x = make_joint_inputs("j_edit2")
    wl = x.workload
    print(f"case joint j_edit2 nq={wl.Nq} nk={wl.Nkv}", flush=True)
    o = run_joint(x)
    rows = np.concatenate([np.arange(0, 128), np.arange(30000, 30064), np.arange(wl.Nq - 96, wl.Nq)])
    heads = [0, 55]
    got = o[torch.from_numpy(rows).to(DEV)][:, heads].float().cpu().numpy()
    ref = A.attention_joint(x.q, x.k, x.v, x.wq, x.wk, x.q_pos, x.k_pos, wl.theta, wl.eps, heads=heads, rows=rows)
    check(got, ref, "joint j_edit2 sampled")
