"""GPU parity of the block router at large block counts: the whole mask bit-exact against the
fp32-specification oracle where the top-k kernel holds 64 keys per lane (2048 < nb <= 4096) and
where the router scores and selects one row per workgroup instead (nb > 4096)."""
import numpy as np
import pytest
import torch

import image_diffusion_transformer_amd as dit
from oracle import router as R
from synth import custom_workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _upload(x):
    def t(b):
        return torch.from_numpy(b.bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return t(x.q), t(x.k), torch.from_numpy(x.wq).to(DEV), torch.from_numpy(x.wk).to(DEV)


@pytest.mark.parametrize("T,H,W,heads,nb", [
    (1, 500, 600, 2, 2344),    # 300,000 tokens, 96-token tail
    (1, 640, 820, 1, 4100),    # 524,800 tokens: past the register top-k
])
def test_route_mask_bit_exact_large_nb(T, H, W, heads, nb):
    wl = custom_workload(T, H, W, heads, seed=31)
    assert wl.nb == nb
    x = make_inputs(wl)
    q, k, wq, wk = _upload(x)
    print(f"case route large nb={nb} heads={heads}", flush=True)
    m = dit.dit_attn_route(q, k, wq, wk, (T, H, W), 0.75, wl.theta, wl.eps)
    torch.cuda.synchronize()
    got = m.cpu().numpy()
    ref = R.route_mask(x.q, x.k, x.wq, x.wk, T, H, W, 0.75, wl.theta, wl.eps)
    assert got.shape == ref.shape
    bad = np.argwhere(np.any(got != ref, axis=2))
    assert bad.size == 0, f"mismatched (head, row) pairs: {bad[:10].tolist()}"
