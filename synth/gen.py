"""Seeded synthetic inputs for one DiT self-attention layer.

This module only draws and rounds numbers; it holds none of the attention
arithmetic.  Both the HIP path (through the tests and the bench) and the fp64
oracle consume what it returns, so they always see bit-identical inputs.

Workloads (token grids and head shape of MiniMax H3 / H3-Image, whose DiT has
56 heads over a 5376-wide hidden state, i.e. head dim 96 -- H3-Image model
table, "DiT" row; 1344x768 / 24 FPS / 5 s and 10 s clips from the H3 SGLang
report's test setup):

* Q, K, V: i.i.d. N(0, 1) in float32, then rounded to bfloat16 (RNE).
* video grids add a smooth, position-dependent component so the block router
  has structure to find: three random low-frequency sinusoids over (t, h, w),
  each with amplitude 0.5 and a random sign per (tensor, head, channel).
* RMSNorm weights: 1 + 0.1 * N(0, 1), float32, one vector of 96 per Q and K (1.75 times that for
  the workloads that exercise the running-maximum softmax).

Generation is chunked over tokens; every chunk draws from its own
``SeedSequence([seed, tensor, chunk])`` stream, so results do not depend on
the number of worker threads.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 96
CHUNK_TOKENS = 2048


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    W: int
    heads: int
    seed: int
    smooth: bool
    mode: str = "dense"          # "dense" or "sparse"
    sparsity: float = 0.0
    block: int = 128
    theta: float = 10000.0
    eps: float = 1e-6
    fp32_inputs: bool = False    # the tiny grid also keeps its float32 draw
    head_dim: int = HEAD_DIM     # 96 (the model's); 128 for the head-dim-128 instantiation
    weight_scale: float = 1.0    # RMSNorm weights are weight_scale * (1 + 0.1 N(0, 1))
    wq_spike: float = 0.0        # if nonzero, w_q channel 0 is set to this value (one large channel)
    notes: str = field(default="", compare=False)

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def nb(self) -> int:
        return -(-self.N // self.block)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny", 2, 4, 4, 2, seed=0, smooth=False, fp32_inputs=True,
                 notes="2x4x4 grid, 2 heads, float32 N(0,1) draw"),
        Workload("image", 1, 256, 256, 56, seed=1, smooth=False,
                 notes="H3-Image-like 1x256x256 token grid, dense"),
        Workload("v5", 31, 48, 84, 56, seed=2, smooth=True,
                 notes="5 s 1344x768 video token grid (124,992 tokens), dense"),
        Workload("v5s", 31, 48, 84, 56, seed=2, smooth=True, mode="sparse", sparsity=0.75,
                 notes="same tensors as v5, block-sparse at sparsity 0.75"),
        Workload("v10s", 61, 48, 84, 56, seed=3, smooth=True, mode="sparse", sparsity=0.80,
                 notes="10 s 1344x768 video token grid (245,952 tokens), sparsity 0.80"),
        Workload("v10d", 61, 48, 84, 56, seed=3, smooth=True,
                 notes="10 s video grid, dense"),
        Workload("v5h7", 31, 48, 84, 7, seed=2, smooth=True,
                 notes="5 s video grid with 7 heads: one GPU's share of the layer when its 56 heads are "
                       "split over 8 GPUs (sequence-parallel attention resharded by head)"),
        # small grids for element-by-element parity: several tiles plus ragged tails
        Workload("s1", 2, 10, 10, 2, seed=10, smooth=True, notes="N=200 (tail 72)"),
        Workload("s2", 3, 16, 16, 3, seed=11, smooth=True, notes="N=768 (6 full blocks)"),
        Workload("s3", 4, 12, 20, 4, seed=12, smooth=True, notes="N=960 (tail 64)"),
        Workload("s4", 5, 24, 40, 2, seed=13, smooth=True, notes="N=4800 (tail 64), 38 blocks"),
        Workload("s4s", 5, 24, 40, 2, seed=13, smooth=True, mode="sparse", sparsity=0.75,
                 notes="s4's tensors, block-sparse at sparsity 0.75"),
        # head dim 128 (42 heads x 128 = the same 5376 hidden width)
        Workload("t128", 2, 4, 4, 2, seed=30, smooth=False, head_dim=128, notes="2x4x4 grid, head dim 128"),
        Workload("s1_128", 2, 10, 10, 2, seed=31, smooth=True, head_dim=128, notes="N=200 (tail 72), head dim 128"),
        Workload("s3_128", 4, 12, 20, 3, seed=32, smooth=True, head_dim=128, notes="N=960 (tail 64), head dim 128"),
        Workload("s4_128", 5, 24, 40, 2, seed=33, smooth=True, head_dim=128, notes="N=4800, 38 blocks, head dim 128"),
        Workload("v5d128", 31, 48, 84, 42, seed=34, smooth=True, head_dim=128,
                 notes="5 s video grid, 42 heads x 128 (hidden 5376), dense"),
        Workload("v5s128", 31, 48, 84, 42, seed=34, smooth=True, head_dim=128, mode="sparse", sparsity=0.75,
                 notes="same tensors as v5d128, block-sparse at sparsity 0.75"),
        # head counts whose last round of dense workgroups is partly filled (the kernels split its query tiles
        # along the keys): 9 x 128 query tiles of 512 at head dim 96, 6 x 200 tiles of 256 at head dim 128
        Workload("t9", 1, 256, 256, 9, seed=40, smooth=False,
                 notes="1x256x256 grid, 9 heads: 144 tiles per XCD run, 16 of them in a split last round"),
        Workload("t9o", 1, 256, 256, 9, seed=40, smooth=False, wq_spike=6.0,
                 notes="t9's tensors with w_q channel 0 at 6 (running-maximum kernels)"),
        Workload("t6_128", 1, 200, 256, 6, seed=41, smooth=False, head_dim=128,
                 notes="1x200x256 grid, 6 heads x 128: 150 tiles per XCD run, 22 of them split"),
        Workload("t6_128o", 1, 200, 256, 6, seed=41, smooth=False, head_dim=128, wq_spike=6.0,
                 notes="t6_128's tensors with w_q channel 0 at 6 (running-maximum kernels)"),
        # norm weights 1.75 times as large: the logit bound (59.6 in base 2) is past what exp2 takes without
        # a shift, so the static mode subtracts a constant (bound - 48) from every logit
        Workload("v5w", 31, 48, 84, 56, seed=2, smooth=True, weight_scale=1.75,
                 notes="same tensors as v5, norm weights 1.75(1 + 0.1 N(0,1)), dense"),
        Workload("v5sw", 31, 48, 84, 56, seed=2, smooth=True, weight_scale=1.75, mode="sparse", sparsity=0.75,
                 notes="same tensors as v5, norm weights 1.75(1 + 0.1 N(0,1)), block-sparse at sparsity 0.75"),
        # w_q channel 0 at 6: the pairwise logit bound (about 90 in base 2) is past the static mode's limit of 80,
        # so the running-maximum kernels run, while the logits themselves stay moderate
        Workload("v5o", 31, 48, 84, 56, seed=2, smooth=True, wq_spike=6.0,
                 notes="same tensors as v5, w_q channel 0 at 6, dense"),
        Workload("v5so", 31, 48, 84, 56, seed=2, smooth=True, wq_spike=6.0, mode="sparse", sparsity=0.75,
                 notes="same tensors as v5, w_q channel 0 at 6, block-sparse at sparsity 0.75"),
    ]
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class BF16Tensor:
    """A [N, heads, 96] bfloat16 tensor held as uint16 bits; slicing returns exact float32."""

    def __init__(self, bits: np.ndarray):
        self.bits = bits

    @property
    def shape(self):
        return self.bits.shape

    def __getitem__(self, idx):
        return bf16_bits_to_f32(self.bits[idx])

    def __array__(self, dtype=None, copy=None):
        a = bf16_bits_to_f32(self.bits)
        return a if dtype is None else a.astype(dtype)


@dataclass
class Inputs:
    workload: Workload
    q: BF16Tensor
    k: BF16Tensor
    v: BF16Tensor
    wq: np.ndarray                 # float32 [96]
    wk: np.ndarray                 # float32 [96]
    q32: np.ndarray | None = None  # float32 draw before rounding (tiny grid only)
    k32: np.ndarray | None = None
    v32: np.ndarray | None = None


def _smooth_params(seed: int, heads: int, d: int = HEAD_DIM):
    """Frequencies, phases and per-(tensor, head, channel) signs of the three sinusoids."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    freqs, phases = [], []
    for _ in range(3):
        while True:
            f = g.integers(0, 3, size=3)
            if f.any():
                break
        freqs.append(f)
        phases.append(g.uniform(0.0, 2.0 * math.pi))
    signs = g.choice(np.array([-1.0, 1.0]), size=(3, heads, d, 3))  # [tensor, head, c, m]
    return np.array(freqs, dtype=np.float64), np.array(phases), signs


def _weights(seed: int, d: int = HEAD_DIM, scale: float = 1.0):
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    wq = (scale * (1.0 + 0.1 * g.standard_normal(d))).astype(np.float32)
    wk = (scale * (1.0 + 0.1 * g.standard_normal(d))).astype(np.float32)
    return wq, wk


def norm_weights(wl: Workload | str) -> tuple[np.ndarray, np.ndarray]:
    """The workload's RMSNorm weights (w_q, w_k), float32 [head_dim] each, without drawing Q/K/V."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    wq, wk = _weights(wl.seed, wl.head_dim, wl.weight_scale)
    if wl.wq_spike:
        wq = wq.copy()
        wq[0] = np.float32(wl.wq_spike)
    return wq, wk


def _fill_chunk(wl: Workload, tensor: int, chunk: int, smooth, out_bits, out_f32):
    n0 = chunk * CHUNK_TOKENS
    n1 = min(wl.N, n0 + CHUNK_TOKENS)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, tensor, chunk])))
    d = wl.head_dim
    x = g.standard_normal((n1 - n0, wl.heads, d), dtype=np.float32)
    if smooth is not None:
        freqs, phases, signs = smooth
        n = np.arange(n0, n1)
        t = n // (wl.H * wl.W)
        h = (n // wl.W) % wl.H
        w = n % wl.W
        arg = (freqs[:, 0:1] * (t / wl.T) + freqs[:, 1:2] * (h / wl.H)
               + freqs[:, 2:3] * (w / wl.W))                      # [3, n]
        F = np.sin(2.0 * math.pi * arg + phases[:, None])           # [3, n]
        s = signs[tensor].reshape(wl.heads * d, 3)                  # [heads*d, 3]
        add = 0.5 * (F.T @ s.T)                                     # [n, heads*d]
        x += add.reshape(n1 - n0, wl.heads, d).astype(np.float32)
    out_bits[n0:n1] = f32_to_bf16_bits(x)
    if out_f32 is not None:
        out_f32[n0:n1] = x


def make_inputs(wl: Workload | str, threads: int | None = None) -> Inputs:
    """Draw the seeded inputs of a workload (host memory)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    d = wl.head_dim
    smooth = _smooth_params(wl.seed, wl.heads, d) if wl.smooth else None
    nchunks = -(-wl.N // CHUNK_TOKENS)
    bits = [np.empty((wl.N, wl.heads, d), dtype=np.uint16) for _ in range(3)]
    f32 = ([np.empty((wl.N, wl.heads, d), dtype=np.float32) for _ in range(3)]
           if wl.fp32_inputs else [None] * 3)
    jobs = [(t, c) for t in range(3) for c in range(nchunks)]
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if len(jobs) == 1 or threads <= 1:
        for t, c in jobs:
            _fill_chunk(wl, t, c, smooth, bits[t], f32[t])
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda tc: _fill_chunk(wl, tc[0], tc[1], smooth, bits[tc[0]], f32[tc[0]]), jobs))
    wq, wk = norm_weights(wl)
    return Inputs(wl, BF16Tensor(bits[0]), BF16Tensor(bits[1]), BF16Tensor(bits[2]), wq, wk,
                  *f32)


def custom_workload(T, H, W, heads, seed, smooth=True, **kw) -> Workload:
    return Workload(f"custom_{T}x{H}x{W}x{heads}_s{seed}", T, H, W, heads, seed, smooth, **kw)
