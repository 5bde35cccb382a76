"""ctypes binding of libditattn.so: the C entry points under the same names.

Argument marshalling only -- every step of the path runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  Importing this
module does not load the library; the first call does, and raises if it has not
been built (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libditattn.so")
HEAD_DIM = 96
BLOCK = 128

DIT_OK, DIT_ERR_INVALID_ARG, DIT_ERR_UNSUPPORTED, DIT_ERR_WORKSPACE, DIT_ERR_HIP = range(5)
STATUS_NAMES = {0: "DIT_OK", 1: "DIT_ERR_INVALID_ARG", 2: "DIT_ERR_UNSUPPORTED",
                3: "DIT_ERR_WORKSPACE", 4: "DIT_ERR_HIP"}

EXPORTS = ("dit_attn_workspace_bytes", "dit_attn_keep_count", "dit_attn_dense", "dit_attn_route",
           "dit_attn_block_sparse", "dit_attn_joint_workspace_bytes", "dit_attn_joint", "dit_attn_last_error",
           "dit_adaln_modulate", "dit_gated_residual", "dit_swiglu")

_lib = None
_lock = threading.Lock()


class DitAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libditattn.so and declare the C signatures (idempotent)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run image_diffusion_transformer_amd.build.build() first")
        lib = ctypes.CDLL(path)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.dit_attn_workspace_bytes.argtypes = [i, i, i, i, i, i]
        lib.dit_attn_workspace_bytes.restype = sz
        lib.dit_attn_keep_count.argtypes = [i, f]
        lib.dit_attn_keep_count.restype = i
        lib.dit_attn_dense.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, f, vp, vp, sz, vp]
        lib.dit_attn_dense.restype = i
        lib.dit_attn_route.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, f, f, i, vp, vp, sz, vp]
        lib.dit_attn_route.restype = i
        lib.dit_attn_block_sparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, f, i, vp, vp, vp, sz, vp]
        lib.dit_attn_block_sparse.restype = i
        lib.dit_attn_joint_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.dit_attn_joint_workspace_bytes.restype = sz
        lib.dit_attn_joint.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, f, vp, vp, sz, vp]
        lib.dit_attn_joint.restype = i
        ll = ctypes.c_longlong
        lib.dit_adaln_modulate.argtypes = [vp, vp, vp, ll, i, f, vp, vp]
        lib.dit_adaln_modulate.restype = i
        lib.dit_gated_residual.argtypes = [vp, vp, vp, vp, vp, ll, i, f, vp, vp, vp]
        lib.dit_gated_residual.restype = i
        lib.dit_swiglu.argtypes = [vp, ll, i, vp, vp]
        lib.dit_swiglu.restype = i
        lib.dit_attn_last_error.argtypes = []
        lib.dit_attn_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _check(status: int) -> None:
    if status != DIT_OK:
        raise DitAttnError(status, load_library().dit_attn_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _shape(q, grid):
    T, H, W = (int(x) for x in grid)
    if q.dim() != 3:
        raise ValueError("q must be [N, heads, head_dim]")
    return T, H, W, int(q.shape[1]), int(q.shape[2])


def dit_attn_workspace_bytes(T: int, H: int, W: int, heads: int, head_dim: int = HEAD_DIM, block: int = BLOCK) -> int:
    return int(load_library().dit_attn_workspace_bytes(T, H, W, heads, head_dim, block))


def dit_attn_keep_count(nb: int, sparsity: float) -> int:
    return int(load_library().dit_attn_keep_count(nb, sparsity))


def workspace_for(q, grid, device=None) -> torch.Tensor:
    """Allocate a workspace tensor large enough for every entry point at this shape."""
    T, H, W, heads, d = _shape(q, grid)
    n = dit_attn_workspace_bytes(T, H, W, heads, d, BLOCK)
    if n == 0:
        raise DitAttnError(DIT_ERR_INVALID_ARG, "invalid shape for workspace sizing")
    return torch.empty(n, dtype=torch.uint8, device=device or q.device)


def dit_attn_dense(q, k, v, wq, wk, grid, rope_theta=10000.0, eps=1e-6, o=None, workspace=None, stream=None):
    """O = attention(RoPE(RMSNorm(q)), RoPE(RMSNorm(k)), v); q, k, v bf16 [N, heads, 96] on the GPU."""
    T, H, W, heads, d = _shape(q, grid)
    if o is None:
        o = torch.empty_like(q)
    if workspace is None:
        workspace = workspace_for(q, grid)
    _check(load_library().dit_attn_dense(_ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk), T, H, W, heads, d,
                                          rope_theta, eps, _ptr(o), _ptr(workspace), workspace.numel(),
                                          _stream(stream)))
    return o


def dit_attn_route(q, k, wq, wk, grid, sparsity, rope_theta=10000.0, eps=1e-6, block=BLOCK, mask=None,
                   workspace=None, stream=None):
    """Kept-block mask uint8 [heads, nb, nb] of the block router."""
    T, H, W, heads, d = _shape(q, grid)
    nb = -(-(T * H * W) // block)
    if mask is None:
        mask = torch.empty((heads, nb, nb), dtype=torch.uint8, device=q.device)
    if workspace is None:
        workspace = workspace_for(q, grid)
    _check(load_library().dit_attn_route(_ptr(q), _ptr(k), _ptr(wq), _ptr(wk), T, H, W, heads, d, rope_theta, eps,
                                          sparsity, block, _ptr(mask), _ptr(workspace), workspace.numel(),
                                          _stream(stream)))
    return mask


def dit_attn_block_sparse(q, k, v, wq, wk, grid, mask, rope_theta=10000.0, eps=1e-6, block=BLOCK, o=None,
                          workspace=None, stream=None):
    """Attention restricted to the kept KV blocks of `mask` (uint8 [heads, nb, nb])."""
    T, H, W, heads, d = _shape(q, grid)
    if o is None:
        o = torch.empty_like(q)
    if workspace is None:
        workspace = workspace_for(q, grid)
    _check(load_library().dit_attn_block_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk), T, H, W, heads, d,
                                                 rope_theta, eps, block, _ptr(mask), _ptr(o), _ptr(workspace),
                                                 workspace.numel(), _stream(stream)))
    return o


def dit_attn_joint_workspace_bytes(nq: int, nk: int, heads: int, head_dim: int = HEAD_DIM, max_pos: int = 1) -> int:
    return int(load_library().dit_attn_joint_workspace_bytes(nq, nk, heads, head_dim, max_pos))


def dit_attn_joint(q, k, v, wq, wk, q_pos, k_pos, max_pos, rope_theta=10000.0, eps=1e-6, o=None, workspace=None,
                   stream=None):
    """Joint attention: q bf16 [nq, heads, 96] at q_pos int32 [nq, 3], k / v bf16 [nk, heads, 96] at k_pos
    int32 [nk, 3] (t, h, w positions, each coordinate < max_pos); writes o [nq, heads, 96]."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q and k must be [tokens, heads, head_dim]")
    nq, heads, d = (int(x) for x in q.shape)
    nk = int(k.shape[0])
    if tuple(q_pos.shape) != (nq, 3) or tuple(k_pos.shape) != (nk, 3):
        raise ValueError("q_pos must be [nq, 3] and k_pos [nk, 3]")
    if q_pos.dtype != torch.int32 or k_pos.dtype != torch.int32:
        raise ValueError("positions must be int32")
    if o is None:
        o = torch.empty_like(q)
    if workspace is None:
        n = dit_attn_joint_workspace_bytes(nq, nk, heads, d, int(max_pos))
        if n == 0:
            raise DitAttnError(DIT_ERR_INVALID_ARG, "invalid sizes for joint workspace sizing")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    _check(load_library().dit_attn_joint(_ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk), _ptr(q_pos), _ptr(k_pos),
                                          nq, nk, heads, d, int(max_pos), rope_theta, eps, _ptr(o), _ptr(workspace),
                                          workspace.numel(), _stream(stream)))
    return o


def _rows(x, name):
    if x.dim() != 2 or x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bf16 [tokens, width] tensor")
    return int(x.shape[0]), int(x.shape[1])


def dit_adaln_modulate(x, shift, scale, eps=1e-6, h=None, stream=None):
    """AdaLN update: h = LayerNorm(x) * (1 + scale) + shift; x bf16 [tokens, hidden], shift / scale fp32 [hidden]."""
    tokens, hidden = _rows(x, "x")
    if h is None:
        h = torch.empty_like(x)
    _check(load_library().dit_adaln_modulate(_ptr(x), _ptr(shift), _ptr(scale), tokens, hidden, eps, _ptr(h),
                                             _stream(stream)))
    return h


def dit_gated_residual(x, y, gate, shift=None, scale=None, eps=1e-6, x_out=None, h=None, modulate=True, stream=None):
    """x_out = x + gate * y and, if ``modulate``, h = LayerNorm(x_out) * (1 + scale) + shift from the float32 sum.
    Returns (x_out, h); h is None without modulation.  x_out may be x (in-place)."""
    tokens, hidden = _rows(x, "x")
    if x_out is None:
        x_out = torch.empty_like(x)
    if modulate and h is None:
        h = torch.empty_like(x)
    if not modulate:
        h = None
    _check(load_library().dit_gated_residual(_ptr(x), _ptr(y), _ptr(gate), _ptr(shift), _ptr(scale), tokens, hidden,
                                             eps, _ptr(x_out), _ptr(h), _stream(stream)))
    return x_out, h


def dit_swiglu(gate_up, out=None, stream=None):
    """out = silu(g) * u for gate_up = [g | u], bf16 [tokens, 2 ffn] -> [tokens, ffn]."""
    tokens, width = _rows(gate_up, "gate_up")
    ffn = width // 2
    if out is None:
        out = torch.empty((tokens, ffn), dtype=gate_up.dtype, device=gate_up.device)
    _check(load_library().dit_swiglu(_ptr(gate_up), tokens, ffn, _ptr(out), _stream(stream)))
    return out


def dit_attn_last_error() -> str:
    return load_library().dit_attn_last_error().decode()
