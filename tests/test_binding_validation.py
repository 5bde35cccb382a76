"""The Python binding checks every tensor before it hands a raw pointer to the C ABI: dtype, shape,
contiguity and GPU memory (a host pointer or a strided view would otherwise be read as if it were a
contiguous device buffer).  These run on the CPU: each wrong property is reported before the device."""
import pytest
import torch

import image_diffusion_transformer_amd as dit

G = (2, 4, 4)                                   # N = 32 tokens
N, HEADS, D = 32, 2, 96


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def dense_args(**kw):
    a = dict(q=t(N, HEADS, D), k=t(N, HEADS, D), v=t(N, HEADS, D), wq=t(D, dtype=torch.float32),
             wk=t(D, dtype=torch.float32))
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,text", [
    (dict(), "GPU memory"),                                              # host tensors
    (dict(q=t(N, HEADS, D, dtype=torch.float32)), "bfloat16"),
    (dict(q=t(N + 1, HEADS, D)), "shape"),                               # N != T*H*W
    (dict(k=t(N, HEADS + 1, D)), "shape"),
    (dict(v=t(N, HEADS, D + 32)), "shape"),
    (dict(wq=t(D)), "float32"),
    (dict(wk=t(D + 1, dtype=torch.float32)), "shape"),
    (dict(q=t(N, D, HEADS).transpose(1, 2)), "contiguous"),
])
def test_dense_operands(kw, text):
    a = dense_args(**kw)
    with pytest.raises(ValueError, match=text):
        dit.dit_attn_dense(a["q"], a["k"], a["v"], a["wq"], a["wk"], G)


def test_sparse_mask_and_route_mask():
    a = dense_args()
    with pytest.raises(ValueError, match="mask"):
        dit.dit_attn_block_sparse(a["q"], a["k"], a["v"], a["wq"], a["wk"], G, t(HEADS, 2, 2, dtype=torch.uint8))
    with pytest.raises(ValueError, match="uint8"):
        dit.dit_attn_block_sparse(a["q"], a["k"], a["v"], a["wq"], a["wk"], G, t(HEADS, 1, 1))
    with pytest.raises(ValueError, match="mask"):
        dit.dit_attn_route(a["q"], a["k"], a["wq"], a["wk"], G, 0.5, mask=t(HEADS, 1, 2, dtype=torch.uint8))


def test_joint_operands():
    q, k, v = t(5, HEADS, D), t(7, HEADS, D), t(7, HEADS, D)
    w = t(D, dtype=torch.float32)
    qp, kp = t(5, 3, dtype=torch.int32), t(7, 3, dtype=torch.int32)
    with pytest.raises(ValueError, match="int32"):
        dit.dit_attn_joint(q, k, v, w, w, t(5, 3, dtype=torch.int64), kp, 4)
    with pytest.raises(ValueError, match="shape"):
        dit.dit_attn_joint(q, k, v, w, w, qp, t(6, 3, dtype=torch.int32), 4)
    with pytest.raises(ValueError, match="shape"):
        dit.dit_attn_joint(q, k, t(8, HEADS, D), w, w, qp, kp, 4)
    with pytest.raises(ValueError, match="GPU memory"):
        dit.dit_attn_joint(q, k, v, w, w, qp, kp, 4)


def test_block_operator_operands():
    x, y = t(3, 64), t(3, 64)
    vec = t(64, dtype=torch.float32)
    with pytest.raises(ValueError, match="shape"):
        dit.dit_gated_residual(x, t(3, 72), vec, vec, vec)
    with pytest.raises(ValueError, match="float32"):
        dit.dit_adaln_modulate(x, t(64), vec)
    with pytest.raises(ValueError, match="even width"):
        dit.dit_swiglu(t(3, 65))
    with pytest.raises(ValueError, match="GPU memory"):
        dit.dit_swiglu(t(3, 64))
    with pytest.raises(ValueError, match="GPU memory"):
        dit.dit_gated_residual(x, y, vec, modulate=False)
