"""ctypes binding of libditattn.so: the C entry points under the same names.

Argument marshalling only -- every step of the path runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  Importing this
module does not load the library; the first call does, and raises if it has not
been built (there is no fallback).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libditattn.so")
HEAD_DIM = 96
BLOCK = 128

DIT_OK, DIT_ERR_INVALID_ARG, DIT_ERR_UNSUPPORTED, DIT_ERR_WORKSPACE, DIT_ERR_HIP, DIT_ERR_HOST = range(6)
STATUS_NAMES = {0: "DIT_OK", 1: "DIT_ERR_INVALID_ARG", 2: "DIT_ERR_UNSUPPORTED",
                3: "DIT_ERR_WORKSPACE", 4: "DIT_ERR_HIP", 5: "DIT_ERR_HOST"}

EXPORTS = ("dit_attn_workspace_bytes", "dit_attn_keep_count", "dit_attn_dense", "dit_attn_route",
           "dit_attn_block_sparse", "dit_attn_joint_workspace_bytes", "dit_attn_joint", "dit_attn_dense_noalloc",
           "dit_attn_set_launch_order",
           "dit_attn_last_error", "dit_adaln_modulate", "dit_gated_residual", "dit_swiglu")

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
        lib.dit_attn_workspace_bytes.argtypes = [i, i, i, i, i, i, f]
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
        lib.dit_attn_dense_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, f, vp, vp]
        lib.dit_attn_dense_noalloc.restype = i
        lib.dit_attn_set_launch_order.argtypes = [i]
        lib.dit_attn_set_launch_order.restype = i
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


def _on_stream(stream):
    """Context in which a call allocates its temporaries (workspace, o, mask): on the stream the call runs on.
    torch's caching allocator then hands that memory to other work on that stream only, which runs after the
    call's kernels; allocated on another stream, a temporary freed at return could be reused while the
    kernels still read or write it."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _dev(t, name, dtype, shape=None):
    """t as the C ABI reads it: a contiguous tensor of this dtype and shape (None: any size).  Where it lives
    is checked by _on once every operand has passed this."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and (t.dim() != len(shape) or
                              any(s is not None and int(a) != int(s) for a, s in zip(t.shape, shape))):
        want = tuple("*" if s is None else s for s in shape)
        raise ValueError(f"{name} must have shape {want} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on(device, **tensors):
    """Every operand in GPU memory, on one device: the library takes raw device pointers."""
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be in GPU memory (got {t.device})")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, the other operands on {device}")


def _shape(q, grid):
    T, H, W = (int(x) for x in grid)
    _dev(q, "q", torch.bfloat16, (T * H * W, None, None))
    return T, H, W, int(q.shape[1]), int(q.shape[2])


def _attn_operands(q, k, v, wq, wk, N, heads, d, nk=None):
    """Checks q [N, heads, d], k and v [nk, heads, d] (v may be None) bf16 and wq, wk fp32 [d]."""
    nk = N if nk is None else nk
    _dev(q, "q", torch.bfloat16, (N, heads, d))
    _dev(k, "k", torch.bfloat16, (nk, heads, d))
    if v is not None:
        _dev(v, "v", torch.bfloat16, (nk, heads, d))
    _dev(wq, "wq", torch.float32, (d,))
    _dev(wk, "wk", torch.float32, (d,))


def _workspace(ws):
    return _dev(ws, "workspace", torch.uint8, (None,))


def dit_attn_workspace_bytes(T: int, H: int, W: int, heads: int, head_dim: int = HEAD_DIM, block: int = BLOCK,
                             sparsity: float = 0.0) -> int:
    return int(load_library().dit_attn_workspace_bytes(T, H, W, heads, head_dim, block, sparsity))


def dit_attn_keep_count(nb: int, sparsity: float) -> int:
    return int(load_library().dit_attn_keep_count(nb, sparsity))


def workspace_for(q, grid, device=None, sparsity: float = 0.0) -> torch.Tensor:
    """Allocate a workspace tensor large enough for every entry point at this shape (on the current stream)."""
    T, H, W, heads, d = _shape(q, grid)
    n = dit_attn_workspace_bytes(T, H, W, heads, d, BLOCK, sparsity)
    if n == 0:
        raise DitAttnError(DIT_ERR_INVALID_ARG, "invalid shape or sparsity for workspace sizing")
    return torch.empty(n, dtype=torch.uint8, device=device or q.device)


def dit_attn_dense(q, k, v, wq, wk, grid, rope_theta=10000.0, eps=1e-6, o=None, workspace=None, stream=None):
    """O = attention(RoPE(RMSNorm(q)), RoPE(RMSNorm(k)), v); q, k, v bf16 [N, heads, 96] on the GPU."""
    T, H, W, heads, d = _shape(q, grid)
    _attn_operands(q, k, v, wq, wk, T * H * W, heads, d)
    with _on_stream(stream):
        if o is None:
            o = torch.empty_like(q)
        if workspace is None:
            workspace = workspace_for(q, grid)
    _dev(o, "o", torch.bfloat16, tuple(q.shape))
    _workspace(workspace)
    _on(q.device, q=q, k=k, v=v, wq=wq, wk=wk, o=o, workspace=workspace)
    _check(load_library().dit_attn_dense(_ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk), T, H, W, heads, d,
                                          rope_theta, eps, _ptr(o), _ptr(workspace), workspace.numel(),
                                          _stream(stream)))
    return o


def dit_attn_route(q, k, wq, wk, grid, sparsity, rope_theta=10000.0, eps=1e-6, block=BLOCK, mask=None,
                   workspace=None, stream=None):
    """Kept-block mask uint8 [heads, nb, nb] of the block router."""
    T, H, W, heads, d = _shape(q, grid)
    _attn_operands(q, k, None, wq, wk, T * H * W, heads, d)
    nb = -(-(T * H * W) // block)
    with _on_stream(stream):
        if mask is None:
            mask = torch.empty((heads, nb, nb), dtype=torch.uint8, device=q.device)
        if workspace is None:
            workspace = workspace_for(q, grid, sparsity=sparsity)
    _dev(mask, "mask", torch.uint8, (heads, nb, nb))
    _workspace(workspace)
    _on(q.device, q=q, k=k, wq=wq, wk=wk, mask=mask, workspace=workspace)
    _check(load_library().dit_attn_route(_ptr(q), _ptr(k), _ptr(wq), _ptr(wk), T, H, W, heads, d, rope_theta, eps,
                                          sparsity, block, _ptr(mask), _ptr(workspace), workspace.numel(),
                                          _stream(stream)))
    return mask


def dit_attn_block_sparse(q, k, v, wq, wk, grid, mask, rope_theta=10000.0, eps=1e-6, block=BLOCK, o=None,
                          workspace=None, stream=None):
    """Attention restricted to the kept KV blocks of `mask` (uint8 [heads, nb, nb])."""
    T, H, W, heads, d = _shape(q, grid)
    _attn_operands(q, k, v, wq, wk, T * H * W, heads, d)
    nb = -(-(T * H * W) // block)
    _dev(mask, "mask", torch.uint8, (heads, nb, nb))
    with _on_stream(stream):
        if o is None:
            o = torch.empty_like(q)
        if workspace is None:
            workspace = workspace_for(q, grid)
    _dev(o, "o", torch.bfloat16, tuple(q.shape))
    _workspace(workspace)
    _on(q.device, q=q, k=k, v=v, wq=wq, wk=wk, mask=mask, o=o, workspace=workspace)
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
    _dev(q, "q", torch.bfloat16, (None, None, None))
    _dev(k, "k", torch.bfloat16, (None, None, None))
    nq, heads, d = (int(x) for x in q.shape)
    nk = int(k.shape[0])
    _attn_operands(q, k, v, wq, wk, nq, heads, d, nk)
    _dev(q_pos, "q_pos", torch.int32, (nq, 3))
    _dev(k_pos, "k_pos", torch.int32, (nk, 3))
    with _on_stream(stream):
        if o is None:
            o = torch.empty_like(q)
        if workspace is None:
            n = dit_attn_joint_workspace_bytes(nq, nk, heads, d, int(max_pos))
            if n == 0:
                raise DitAttnError(DIT_ERR_INVALID_ARG, "invalid sizes for joint workspace sizing")
            workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    _dev(o, "o", torch.bfloat16, tuple(q.shape))
    _workspace(workspace)
    _on(q.device, q=q, k=k, v=v, wq=wq, wk=wk, q_pos=q_pos, k_pos=k_pos, o=o, workspace=workspace)
    _check(load_library().dit_attn_joint(_ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk), _ptr(q_pos), _ptr(k_pos),
                                          nq, nk, heads, d, int(max_pos), rope_theta, eps, _ptr(o), _ptr(workspace),
                                          workspace.numel(), _stream(stream)))
    return o


def _rows(x, name):
    _dev(x, name, torch.bfloat16, (None, None))
    return int(x.shape[0]), int(x.shape[1])


def _vec(t, name, hidden):
    return _dev(t, name, torch.float32, (hidden,))


def dit_adaln_modulate(x, shift, scale, eps=1e-6, h=None, stream=None):
    """AdaLN update: h = LayerNorm(x) * (1 + scale) + shift; x bf16 [tokens, hidden], shift / scale fp32 [hidden]."""
    tokens, hidden = _rows(x, "x")
    _vec(shift, "shift", hidden)
    _vec(scale, "scale", hidden)
    if h is None:
        with _on_stream(stream):
            h = torch.empty_like(x)
    _dev(h, "h", torch.bfloat16, (tokens, hidden))
    _on(x.device, x=x, shift=shift, scale=scale, h=h)
    _check(load_library().dit_adaln_modulate(_ptr(x), _ptr(shift), _ptr(scale), tokens, hidden, eps, _ptr(h),
                                             _stream(stream)))
    return h


def dit_gated_residual(x, y, gate, shift=None, scale=None, eps=1e-6, x_out=None, h=None, modulate=True, stream=None):
    """x_out = x + gate * y and, if ``modulate``, h = LayerNorm(x_out) * (1 + scale) + shift from the float32 sum.
    Returns (x_out, h); h is None without modulation.  x_out may be x (in-place)."""
    tokens, hidden = _rows(x, "x")
    _dev(y, "y", torch.bfloat16, (tokens, hidden))
    _vec(gate, "gate", hidden)
    if modulate:
        _vec(shift, "shift", hidden)
        _vec(scale, "scale", hidden)
    with _on_stream(stream):
        if x_out is None:
            x_out = torch.empty_like(x)
        if modulate and h is None:
            h = torch.empty_like(x)
    _dev(x_out, "x_out", torch.bfloat16, (tokens, hidden))
    if not modulate:
        h = None
    else:
        _dev(h, "h", torch.bfloat16, (tokens, hidden))
    _on(x.device, x=x, y=y, gate=gate, shift=shift if modulate else None, scale=scale if modulate else None,
        x_out=x_out, h=h)
    _check(load_library().dit_gated_residual(_ptr(x), _ptr(y), _ptr(gate), _ptr(shift), _ptr(scale), tokens, hidden,
                                             eps, _ptr(x_out), _ptr(h), _stream(stream)))
    return x_out, h


def dit_swiglu(gate_up, out=None, stream=None):
    """out = silu(g) * u for gate_up = [g | u], bf16 [tokens, 2 ffn] -> [tokens, ffn]."""
    tokens, width = _rows(gate_up, "gate_up")
    if width % 2:
        raise ValueError(f"gate_up must hold the gate and up halves: even width (got {width})")
    ffn = width // 2
    if out is None:
        with _on_stream(stream):
            out = torch.empty((tokens, ffn), dtype=gate_up.dtype, device=gate_up.device)
    _dev(out, "out", torch.bfloat16, (tokens, ffn))
    _on(gate_up.device, gate_up=gate_up, out=out)
    _check(load_library().dit_swiglu(_ptr(gate_up), tokens, ffn, _ptr(out), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def dit_attn_dense_noalloc(q, k, v, wq, wk, grid, rope_theta=10000.0, eps=1e-6, o=None, stream=None):
    """dit_attn_dense without a workspace: its scratch is the library's static 64 MiB per-GPU array, so the C call
    allocates no device memory (pass ``o`` too and nothing is allocated at all).  Calls that overlap in time on
    one GPU race on that scratch."""
    T, H, W, heads, d = _shape(q, grid)
    _attn_operands(q, k, v, wq, wk, T * H * W, heads, d)
    if o is None:
        with _on_stream(stream):
            o = torch.empty_like(q)
    _dev(o, "o", torch.bfloat16, tuple(q.shape))
    _on(q.device, q=q, k=k, v=v, wq=wq, wk=wk, o=o)
    _check(load_library().dit_attn_dense_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk), T, H, W, heads, d,
                                                  rope_theta, eps, _ptr(o), _stream(stream)))
    return o


def dit_attn_set_launch_order(order: int) -> None:
    """Diagnostic: 0 = the tuned workgroup order of the attention calls, 1 = reversed (no result may change)."""
    _check(load_library().dit_attn_set_launch_order(int(order)))


def dit_attn_last_error() -> str:
    return load_library().dit_attn_last_error().decode()
