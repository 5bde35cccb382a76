/*
 * dit_block.h -- C ABI of the fused elementwise operators around attention in
 * the MiniMax H3 / H3-Image DiT block, on MI355X (gfx950).
 *
 * Sources (pages as titled; sections named on each page):
 *  - H3 SGLang report (CocoLoop, "MiniMax-H3 in SGLang-Diffusion on 8x H200"),
 *    fused-operator paragraph in the section on the three stacked acceleration
 *    tiers: the AdaLN update, the gated residual path and the SwiGLU activation
 *    run as fused kernels that cut activation traffic through device memory and
 *    change no result.
 *  - H3-Image spec table (52hbtv.com), "DiT" row: hidden 5376, FFN 14336.
 *
 * The pages give the operators' names, not their formulas.  The forms used here:
 *  - AdaLN update: LayerNorm over the `hidden` channels of one token, without
 *    affine parameters, population variance, eps inside the square root, then
 *    h = LN(x) * (1 + scale) + shift with per-channel vectors shift, scale.
 *  - Gated residual: r = x + gate * y with a per-channel gate vector.
 *  - SwiGLU: gate_up [tokens][2 ffn] holds the gate g in columns [0, ffn) and the
 *    up projection u in [ffn, 2 ffn); out = silu(g) * u, silu(z) = z / (1 + e^-z).
 *
 * Conventions
 *  - Activations (x, y, x_out, h, gate_up, out) are bfloat16, row-major, device
 *    memory, 16-byte aligned.  Modulation vectors (gate, shift, scale) are
 *    float32 [hidden], device memory, 16-byte aligned.
 *  - Arithmetic is float32; each output is rounded once to bfloat16 (nearest,
 *    ties to even).  The LayerNorm of the fused operator normalises the float32
 *    sum r, not its rounded copy.
 *  - hidden and ffn must be multiples of 8; hidden <= 8192.  tokens may be 0
 *    (nothing is queued).
 *  - Calls are asynchronous on `hip_stream` (NULL = the null stream), allocate
 *    nothing, and validate every argument on the host before queuing work; on
 *    error dit_attn_last_error() (dit_attn.h) describes the problem.
 *  - Status codes are those of dit_attn.h.
 */
#ifndef DIT_BLOCK_H
#define DIT_BLOCK_H

#include "dit_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* AdaLN update: h = LN(x) * (1 + scale) + shift.
 * x, h: [tokens][hidden]; h must not overlap x. */
dit_status dit_adaln_modulate(const void* x, const float* shift, const float* scale,
                              long long tokens, int hidden, float eps,
                              void* h, void* hip_stream);

/* Gated residual, optionally followed by the next AdaLN update, in one pass:
 * x_out = x + gate * y; if h is not NULL, also h = LN(x + gate * y) * (1 + scale) + shift.
 * x, y, x_out, h: [tokens][hidden].  x_out may be x itself (in-place update of the
 * residual stream) but must not partly overlap x or y; h must not overlap any of them.
 * shift and scale are read only when h is not NULL. */
dit_status dit_gated_residual(const void* x, const void* y, const float* gate,
                              const float* shift, const float* scale,
                              long long tokens, int hidden, float eps,
                              void* x_out, void* h, void* hip_stream);

/* SwiGLU: out[n][c] = silu(gate_up[n][c]) * gate_up[n][ffn + c].
 * gate_up: [tokens][2 ffn]; out: [tokens][ffn], not overlapping gate_up. */
dit_status dit_swiglu(const void* gate_up, long long tokens, int ffn, void* out, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* DIT_BLOCK_H */
