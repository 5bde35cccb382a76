"""Seeded synthetic inputs for the operators around attention in the DiT block.

This module only draws and rounds numbers; it holds none of the operators'
arithmetic.  Shapes follow the H3-Image spec table ("DiT" row: hidden 5376,
FFN 14336); token counts follow the attention workloads (124,992 tokens for the
5 s 1344x768 clip).

* x (residual stream), bf16 [tokens][hidden]: N(0, 1) * s_c + o_c with a
  per-channel offset o_c ~ 2 N(0, 1) and a per-channel spread s_c that is 1,
  except 8 for every 128th channel (a few large channels, as residual streams
  of large transformers carry them), so the LayerNorm's mean and variance are
  far from 0 and 1.
* y (branch output), bf16 [tokens][hidden]: N(0, 1).
* gate, shift, scale (modulation vectors), float32 [hidden]: 0.5 N(0, 1) each.
* gate_up (fused FFN up projection), bf16 [tokens][2 ffn]: 2 N(0, 1), so the
  SiLU sees its whole curved range.

Every tensor is drawn in token chunks, each chunk from its own
``SeedSequence([seed, tensor, chunk])`` stream.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .gen import BF16Tensor, f32_to_bf16_bits

BLOCK_CHUNK = 256


@dataclass(frozen=True)
class BlockWorkload:
    name: str
    tokens: int
    hidden: int
    ffn: int
    seed: int
    eps: float = 1e-6
    notes: str = field(default="", compare=False)


BLOCK_WORKLOADS = {
    w.name: w for w in [
        BlockWorkload("b_tiny", 5, 64, 40, seed=40, notes="5 tokens, hidden 64, FFN 40"),
        BlockWorkload("b_small", 37, 5376, 14336, seed=41, notes="37 tokens at the model's hidden and FFN widths"),
        BlockWorkload("b_mid", 1000, 5376, 14336, seed=42, notes="1000 tokens, several waves per CU"),
        BlockWorkload("b_odd", 19, 1032, 776, seed=43,
                      notes="hidden 1032 and FFN 776: widths that are multiples of 8 but not of 64"),
        BlockWorkload("b_wide", 29, 8184, 16400, seed=45,
                      notes="hidden 8184 (16 vectors per lane, last one ragged) and FFN 16400 (two "
                            "workgroups per row)"),
        BlockWorkload("b_min", 1, 8, 8, seed=46, notes="one token, hidden 8, FFN 8: one vector per row"),
        BlockWorkload("b_v5", 124992, 5376, 14336, seed=44,
                      notes="124,992 tokens (5 s 1344x768 clip) at hidden 5376, FFN 14336"),
    ]
}


@dataclass
class BlockInputs:
    workload: BlockWorkload
    x: BF16Tensor          # [tokens][hidden]
    y: BF16Tensor          # [tokens][hidden]
    gate_up: BF16Tensor    # [tokens][2 ffn]
    gate: np.ndarray       # float32 [hidden]
    shift: np.ndarray
    scale: np.ndarray


def _vectors(wl: BlockWorkload):
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 100])))
    gate = (0.5 * g.standard_normal(wl.hidden)).astype(np.float32)
    shift = (0.5 * g.standard_normal(wl.hidden)).astype(np.float32)
    scale = (0.5 * g.standard_normal(wl.hidden)).astype(np.float32)
    offset = (2.0 * g.standard_normal(wl.hidden)).astype(np.float32)
    spread = np.ones(wl.hidden, dtype=np.float32)
    spread[::128] = 8.0
    return gate, shift, scale, offset, spread


def _fill(wl, tensor, chunk, out, offset, spread):
    n0 = chunk * BLOCK_CHUNK
    n1 = min(wl.tokens, n0 + BLOCK_CHUNK)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, tensor, chunk])))
    z = g.standard_normal((n1 - n0, out.shape[1]), dtype=np.float32)
    if tensor == 0:
        z = z * spread + offset
    elif tensor == 2:
        z = z * np.float32(2.0)
    out[n0:n1] = f32_to_bf16_bits(z)


def make_block_inputs(wl: BlockWorkload | str, threads: int | None = None) -> BlockInputs:
    """Draw the seeded inputs of a block-operator workload (host memory)."""
    if isinstance(wl, str):
        wl = BLOCK_WORKLOADS[wl]
    gate, shift, scale, offset, spread = _vectors(wl)
    bits = [np.empty((wl.tokens, wl.hidden), dtype=np.uint16),
            np.empty((wl.tokens, wl.hidden), dtype=np.uint16),
            np.empty((wl.tokens, 2 * wl.ffn), dtype=np.uint16)]
    nchunks = -(-wl.tokens // BLOCK_CHUNK)
    jobs = [(t, c) for t in range(3) for c in range(nchunks)]
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    run = lambda tc: _fill(wl, tc[0], tc[1], bits[tc[0]], offset, spread)
    if len(jobs) <= 3 or threads <= 1:
        for tc in jobs:
            run(tc)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, jobs))
    return BlockInputs(wl, BF16Tensor(bits[0]), BF16Tensor(bits[1]), BF16Tensor(bits[2]), gate, shift, scale)
