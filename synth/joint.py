"""Seeded synthetic inputs for joint attention over text, reference-image and target tokens.

The DiT of H3-Image is a single-stream transformer with 3D multimodal RoPE that takes up to 16
reference images (H3-Image spec table, "DiT" and reference-image rows); with more reference
images the keys and values grow (same page, optimisation-focus row).  The pages give no token
layout, so these inputs use one (a reading, stated in the design notes):

* one sequence: text tokens, then each reference image, then the target frames;
* text token i sits at (i, i, i); reference image r at (n_text + r, h, w); target frame t at
  (n_text + n_refs + t, h, w);
* keys and values cover the whole sequence; queries cover either the whole sequence or only
  the target tokens (the KV of the conditioning tokens is then longer than Q).

Like ``synth.gen`` this module only draws and rounds numbers and lays out integer positions.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .gen import HEAD_DIM, BF16Tensor, f32_to_bf16_bits


@dataclass(frozen=True)
class JointWorkload:
    name: str
    n_text: int
    refs: tuple            # ((H, W), ...) one per reference image
    target: tuple          # (T, H, W)
    heads: int
    seed: int
    queries: str = "target"      # "target" or "all"
    theta: float = 10000.0
    eps: float = 1e-6
    head_dim: int = HEAD_DIM     # 96 (the model's) or 128
    notes: str = field(default="", compare=False)

    @property
    def n_ref_tokens(self) -> int:
        return sum(h * w for h, w in self.refs)

    @property
    def n_target(self) -> int:
        T, H, W = self.target
        return T * H * W

    @property
    def Nkv(self) -> int:
        return self.n_text + self.n_ref_tokens + self.n_target

    @property
    def Nq(self) -> int:
        return self.n_target if self.queries == "target" else self.Nkv


JOINT_WORKLOADS = {
    w.name: w for w in [
        JointWorkload("j_tiny", 7, ((3, 4),), (2, 3, 4), 2, seed=20, queries="all",
                      notes="43 tokens, all of them queries"),
        JointWorkload("j_small", 50, ((16, 16), (12, 20)), (3, 16, 16), 3, seed=21,
                      notes="Nkv = 50 + 256 + 240 + 768 = 1314, queries = 768 target tokens"),
        JointWorkload("j_all", 33, ((8, 8),), (2, 12, 10), 2, seed=22, queries="all",
                      notes="Nkv = Nq = 33 + 64 + 240 = 337"),
        JointWorkload("j_small128", 50, ((16, 16), (12, 20)), (3, 16, 16), 3, seed=24, head_dim=128,
                      notes="j_small's sequence at head dim 128"),
        JointWorkload("j_edit2", 512, ((256, 256), (256, 256)), (1, 256, 256), 56, seed=23,
                      notes="image edit with 2 reference images: 197,120 keys, 65,536 target queries"),
        JointWorkload("j_ref9", 512, ((128, 128),), (1, 256, 256), 9, seed=25,
                      notes="one reference image, 9 heads: 82,432 keys, 65,536 target queries; 144 query tiles "
                            "per XCD run, so the dense tail split applies"),
    ]
}


@dataclass
class JointInputs:
    workload: JointWorkload
    q: BF16Tensor          # [Nq, heads, 96]
    k: BF16Tensor          # [Nkv, heads, 96]
    v: BF16Tensor
    q_pos: np.ndarray      # int32 [Nq, 3]: (t, h, w)
    k_pos: np.ndarray      # int32 [Nkv, 3]
    max_pos: int           # every coordinate is < max_pos
    wq: np.ndarray
    wk: np.ndarray


def sequence_positions(wl: JointWorkload) -> np.ndarray:
    """int32 [Nkv, 3] (t, h, w) of every token of the joint sequence, in sequence order."""
    parts = []
    i = np.arange(wl.n_text, dtype=np.int64)
    parts.append(np.stack([i, i, i], axis=1))
    for r, (H, W) in enumerate(wl.refs):
        hh, ww = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
        parts.append(np.stack([np.full(H * W, wl.n_text + r), hh.ravel(), ww.ravel()], axis=1))
    T, H, W = wl.target
    tt, hh, ww = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    parts.append(np.stack([wl.n_text + len(wl.refs) + tt.ravel(), hh.ravel(), ww.ravel()], axis=1))
    return np.concatenate(parts, axis=0).astype(np.int32)


def _draw(seed: int, tensor: int, shape) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1000 + tensor])))
    return g.standard_normal(shape, dtype=np.float32)


def make_joint_inputs(wl: JointWorkload | str) -> JointInputs:
    if isinstance(wl, str):
        wl = JOINT_WORKLOADS[wl]
    k_pos = sequence_positions(wl)
    q_pos = k_pos[wl.Nkv - wl.Nq:] if wl.queries == "target" else k_pos
    d = wl.head_dim
    q = f32_to_bf16_bits(_draw(wl.seed, 0, (wl.Nq, wl.heads, d)))
    k = f32_to_bf16_bits(_draw(wl.seed, 1, (wl.Nkv, wl.heads, d)))
    v = f32_to_bf16_bits(_draw(wl.seed, 2, (wl.Nkv, wl.heads, d)))
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 7])))
    wq = (1.0 + 0.1 * g.standard_normal(d)).astype(np.float32)
    wk = (1.0 + 0.1 * g.standard_normal(d)).astype(np.float32)
    max_pos = int(k_pos.max()) + 1
    return JointInputs(wl, BF16Tensor(q), BF16Tensor(k), BF16Tensor(v), np.ascontiguousarray(q_pos),
                       np.ascontiguousarray(k_pos), max_pos, wq, wk)
