"""GPU parity of the operators around attention (AdaLN update, gated residual, SwiGLU),
called through the C ABI, against the fp64 oracle on the same bf16 inputs.

Tolerance, from the arithmetic: the kernels compute in float32 and round each output once to
bfloat16 (nearest even), an error of at most half a unit in the last place, i.e. 2^-8 |ref|;
float32 LayerNorm statistics over 5376 channels add well under 1e-4.  Every element must
satisfy |got - ref| <= 2^-8 |ref| + 1e-4.
"""
import numpy as np
import pytest
import torch

import image_diffusion_transformer_amd as dit
from oracle import block_ops as O
from synth import BLOCK_WORKLOADS, make_block_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
REL, ABS = 2.0 ** -8, 1e-4


def upload(x):
    def t(b):
        return torch.from_numpy(b.bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    v = lambda a: torch.from_numpy(a).to(DEV)
    return t(x.x), t(x.y), t(x.gate_up), v(x.gate), v(x.shift), v(x.scale)


def check(got, ref, what):
    got = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    bound = REL * np.abs(ref) + ABS
    worst = float((err / bound).max()) if err.size else 0.0
    print(f"{what}: max_abs={err.max():.3e} worst err/bound={worst:.3f}", flush=True)
    assert np.all(np.isfinite(got)), what
    assert worst <= 1.0, (what, worst)


@pytest.mark.parametrize("name", ["b_min", "b_tiny", "b_small", "b_mid", "b_odd", "b_wide"])
def test_block_ops_all_rows(name):
    x = make_block_inputs(name)
    wl = x.workload
    print(f"case block {name}", flush=True)
    X, Y, GU, gate, shift, scale = upload(x)
    h = dit.dit_adaln_modulate(X, shift, scale, wl.eps)
    xo, h2 = dit.dit_gated_residual(X, Y, gate, shift, scale, wl.eps)
    xr, none = dit.dit_gated_residual(X, Y, gate, modulate=False)
    out = dit.dit_swiglu(GU)
    torch.cuda.synchronize()
    assert none is None
    Xf, Yf, GUf = (np.asarray(a, np.float64) for a in (x.x, x.y, x.gate_up))
    check(h, O.adaln_modulate(Xf, x.shift, x.scale, wl.eps), f"{name} adaln")
    r, href = O.gated_residual_adaln(Xf, Yf, x.gate, x.shift, x.scale, wl.eps)
    check(xo, r, f"{name} residual")
    check(h2, href, f"{name} residual+adaln")
    assert torch.equal(xr, xo)                 # the residual does not depend on the modulation
    check(out, O.swiglu(GUf), f"{name} swiglu")


def test_in_place_residual_and_determinism():
    x = make_block_inputs("b_mid")
    wl = x.workload
    X, Y, GU, gate, shift, scale = upload(x)
    xo, h = dit.dit_gated_residual(X, Y, gate, shift, scale, wl.eps)
    xo_b, h_b = dit.dit_gated_residual(X, Y, gate, shift, scale, wl.eps)
    Xc = X.clone()
    xi, hi = dit.dit_gated_residual(Xc, Y, gate, shift, scale, wl.eps, x_out=Xc)
    o1, o2 = dit.dit_swiglu(GU), dit.dit_swiglu(GU)
    torch.cuda.synchronize()
    assert xi.data_ptr() == Xc.data_ptr()
    assert torch.equal(xo, xo_b) and torch.equal(h, h_b) and torch.equal(o1, o2)
    assert torch.equal(xi, xo) and torch.equal(hi, h)


def test_special_cases():
    x = make_block_inputs("b_small")
    wl = x.workload
    X, Y, GU, gate, shift, scale = upload(x)
    zero = torch.zeros_like(gate)
    xo, h = dit.dit_gated_residual(X, Y, zero, shift, scale, wl.eps)
    # gate 0: the stream passes through bit for bit; scale -1: every output is the shift
    h_shift = dit.dit_adaln_modulate(X, shift, torch.full_like(scale, -1.0), wl.eps)
    const = torch.full_like(X, 3.5)
    h_const = dit.dit_adaln_modulate(const, shift, scale, wl.eps)
    gu0 = GU.clone()
    gu0[:, : wl.ffn] = 0
    o0 = dit.dit_swiglu(gu0)
    big = GU.clone()
    big[:, : wl.ffn] = -200.0
    ob = dit.dit_swiglu(big)
    torch.cuda.synchronize()
    assert torch.equal(xo, X)
    want = shift.to(torch.bfloat16).expand_as(X)
    assert torch.equal(h_shift, want) and torch.equal(h_const, want)
    assert torch.count_nonzero(o0) == 0
    assert torch.all(ob.float().abs() < 1e-30)


def test_full_size_sampled_rows():
    x = make_block_inputs("b_v5")
    wl = x.workload
    print("case block b_v5", flush=True)
    X, Y, GU, gate, shift, scale = upload(x)
    h = dit.dit_adaln_modulate(X, shift, scale, wl.eps)
    xo, h2 = dit.dit_gated_residual(X, Y, gate, shift, scale, wl.eps)
    out = dit.dit_swiglu(GU)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, wl.tokens - 1], np.random.default_rng(7).integers(0, wl.tokens, 61)]))
    idx = torch.from_numpy(rows).to(DEV)
    Xf, Yf, GUf = (a[rows].astype(np.float64) for a in (x.x, x.y, x.gate_up))
    check(h[idx], O.adaln_modulate(Xf, x.shift, x.scale, wl.eps), "b_v5 adaln")
    r, href = O.gated_residual_adaln(Xf, Yf, x.gate, x.shift, x.scale, wl.eps)
    check(xo[idx], r, "b_v5 residual")
    check(h2[idx], href, "b_v5 residual+adaln")
    check(out[idx], O.swiglu(GUf), "b_v5 swiglu")
