/*
 * dit_attn.h -- C ABI of the MI355X (gfx950) DiT self-attention hot path.
 *
 * One DiT self-attention layer of MiniMax H3 / H3-Image inference: per-head
 * QK-RMSNorm and 3D (t, h, w) RoPE applied to Q and K as they are loaded, then
 * bidirectional (non-causal) softmax attention over the whole token grid, with
 * an optional block-sparse mode driven by a block router.
 *
 * Sources (pages as titled; sections named on each page):
 *  - H3 SGLang report (CocoLoop, "MiniMax-H3 in SGLang-Diffusion on 8x H200"),
 *    section on the three stacked acceleration tiers: the fused-operator paragraph
 *    names QK-RMSNorm with 3D RoPE; the SubBlock-Sparse-Attention paragraph
 *    describes a block-wise router that prunes KV blocks at sparsity 0.75 / 0.80;
 *    the limits section restricts that mode to long, non-causal BF16 attention.
 *  - H3-Image spec table (52hbtv.com), "DiT" row: 56 heads, hidden 5376
 *    (head dim 96), 3D multimodal RoPE.
 *
 * Conventions shared by every entry point
 *  - N = T * H * W tokens; token n sits at t = n / (H*W), h = (n / W) % H,
 *    w = n % W (row-major flattening of the grid).
 *  - q, k, v, o: bfloat16, shape [N][heads][head_dim], contiguous, device memory.
 *  - wq, wk: float32 [head_dim] RMSNorm weights, shared by all heads, device memory.
 *  - RMSNorm: x * w / sqrt(mean_c(x_c^2) + eps) over the head_dim channels of
 *    one (token, head).  RoPE: at head_dim 96 channels [0,32) rotate with t,
 *    [32,64) with h, [64,96) with w; at head_dim 128 (the SubBlock precondition in
 *    the report's limits section; the pages give no split, the nearest-equal even
 *    one is used) [0,44) with t, [44,86) with h, [86,128) with w.  Within a chunk
 *    of width c the pairs are (2i, 2i+1) at angle pos * rope_theta^(-2i/c); the
 *    pair (a, b) becomes (a cos - b sin, a sin + b cos).  V is untouched.
 *  - Attention: O = softmax(Q^ K^T / sqrt(head_dim)) V, every query sees every key.
 *  - head_dim must be 96 or 128, block 128 and heads at most 65535
 *    (DIT_ERR_UNSUPPORTED otherwise).
 *  - All pointers are owned by the caller.  The library allocates no device
 *    memory; scratch space comes from `workspace` (see dit_attn_workspace_bytes).
 *  - Every call is asynchronous on `hip_stream` (a hipStream_t; NULL means the
 *    null stream) and returns as soon as its work is queued.  Nothing is
 *    synchronised, printed or thrown across the ABI.
 *  - Arguments are validated on the host before anything is queued; on error
 *    no work is queued and dit_attn_last_error() describes the problem.
 *  - Every buffer a call writes (o, route's mask, the workspace) must not
 *    overlap any other buffer of the call (DIT_ERR_INVALID_ARG, checked on the
 *    host over the bytes the call reads or writes); read-only inputs (q, k, v,
 *    weights, positions, block_sparse's mask) may share memory with each other.
 *    Calls that share a workspace must be ordered on one stream.
 *  - Nothing is thrown across the ABI: a host-side failure (out of host memory
 *    for the RoPE table) returns DIT_ERR_HOST.
 */
#ifndef DIT_ATTN_H
#define DIT_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DIT_OK = 0,
  DIT_ERR_INVALID_ARG = 1, /* null pointer, bad size, non-finite theta/eps, sparsity outside [0,1) */
  DIT_ERR_UNSUPPORTED = 2, /* head_dim not 96/128, block != 128, grid too large for one call  */
  DIT_ERR_WORKSPACE = 3,   /* workspace missing or smaller than dit_attn_workspace_bytes()    */
  DIT_ERR_HIP = 4,         /* a HIP runtime call failed; the HIP error string is in last_error */
  DIT_ERR_HOST = 5         /* host-side failure (out of host memory); nothing was queued       */
} dit_status;

/* Bytes of device workspace that dense, route and block_sparse need for this
 * shape (enough for any of the three; about 2 * N * heads * head_dim * 2 bytes
 * for the K^/V fragment images plus the largest of the router's share, the
 * block-sparse schedule's (iteration lists and their slot flags, grouping table,
 * the mask packed to bits) and, for a dense call that splits its last round of
 * query tiles, the pieces' fp32 partial results).  `sparsity` is the router's (checked to lie in [0, 1)); the
 * size does not depend on it, since block_sparse accepts any mask.
 * Returns 0 if the shape or the sparsity is invalid. */
size_t dit_attn_workspace_bytes(int T, int H, int W, int heads, int head_dim, int block, float sparsity);

/* Number of KV blocks each query block keeps at `sparsity`:
 * nb - floor(sparsity * nb + 1e-9), clamped to [1, nb], where nb = ceil(N / block).
 * Returns -1 for invalid arguments. */
int dit_attn_keep_count(int nb, float sparsity);

/* Dense attention.  Writes o [N][heads][head_dim] bf16.
 * Kernels on `hip_stream`: a prepass that RMS-normalises and rotates every
 * K row once and writes K^ (bf16) and V into the workspace as MFMA operand
 * fragments, then the attention kernel: RMSNorm + RoPE of Q on load,
 * S = Q^K^T with bf16 MFMA (fp32 accumulate), softmax in fp32 (base 2),
 * O += P V with bf16 MFMA (P rounded to bf16), O / rowsum rounded to bf16.
 * Large calls whose query tiles leave the last round of workgroups part-empty
 * (at least 4 full rounds of 256 tiles, at least 16 key tiles of 128, and the
 * split saving at least 1% of the call) cut each of those last tiles along the
 * keys into 2-4 pieces: the pieces write unnormalised fp32 partials into the
 * workspace and a third kernel sums them in piece order and normalises.  Those tiles then differ from an
 * unsplit evaluation only by the order of the fp32 sums.  The result is the same
 * bits on every call. */
dit_status dit_attn_dense(const void* q, const void* k, const void* v,
                          const float* wq, const float* wk,
                          int T, int H, int W, int heads, int head_dim,
                          float rope_theta, float eps,
                          void* o,
                          void* workspace, size_t workspace_bytes, void* hip_stream);

/* Block router.  Writes mask [heads][nb][nb] uint8 (1 = KV block j kept for
 * query block i), nb = ceil(N / block), the last block holding the remainder.
 * Per (head, block) it mean-pools the post-RMSNorm, post-RoPE q and k in fp32,
 * scores block pairs by their dot product, forces the diagonal to +inf and keeps
 * the dit_attn_keep_count(nb, sparsity) highest-scoring KV blocks per query block,
 * lower index first on equal scores.  Every fp32 operation is done in one fixed
 * order with IEEE round-to-nearest and no fused multiply-add, so the mask is
 * reproducible bit for bit (sequential channel sums, sequential token sums,
 * correctly rounded division and square root, host-computed cos/sin tables). */
dit_status dit_attn_route(const void* q, const void* k,
                          const float* wq, const float* wk,
                          int T, int H, int W, int heads, int head_dim,
                          float rope_theta, float eps, float sparsity, int block,
                          unsigned char* mask,
                          void* workspace, size_t workspace_bytes, void* hip_stream);

/* Block-sparse attention restricted to the kept KV blocks of `mask`
 * ([heads][nb][nb] uint8, any 0/1 content, e.g. from dit_attn_route or another
 * source).  Keys of dropped blocks are never loaded; the softmax renormalises
 * over the kept keys.  A query block that keeps no KV block gets O = 0.
 * With an all-ones mask the result equals dit_attn_dense bit for bit, except on
 * the query tiles a dense call splits (see dit_attn_dense), where the two agree
 * up to the order of the fp32 sums. */
dit_status dit_attn_block_sparse(const void* q, const void* k, const void* v,
                                 const float* wq, const float* wk,
                                 int T, int H, int W, int heads, int head_dim,
                                 float rope_theta, float eps, int block,
                                 const unsigned char* mask,
                                 void* o,
                                 void* workspace, size_t workspace_bytes, void* hip_stream);

/* Bytes of device workspace dit_attn_joint needs for these sizes (0 if they are invalid). */
size_t dit_attn_joint_workspace_bytes(int nq, int nk, int heads, int head_dim, int max_pos);

/* Joint attention over one token sequence with explicit 3D positions: the
 * single-stream DiT of H3-Image (spec table, "DiT" row: 3D multimodal RoPE)
 * attends over text, reference-image (up to 16, reference-image row) and
 * target tokens together.
 *  - q: bf16 [nq][heads][head_dim] at positions q_pos: int32 [nq][3] (t, h, w);
 *    k, v: bf16 [nk][heads][head_dim] at positions k_pos: int32 [nk][3].
 *    nq and nk may differ (e.g. only the target tokens as queries against the
 *    whole sequence as keys).  All device memory, owned by the caller.
 *  - Positions are integers in [0, max_pos): every coordinate rotates its axis
 *    chunk by pos * rope_theta^(-2i/32), as in the grid calls.  Coordinates
 *    outside that range are clamped to it (no error is raised on the device).
 *  - RMSNorm, RoPE, softmax and the MFMA path are those of dit_attn_dense; every
 *    query attends to every key.  Writes o [nq][heads][head_dim] bf16.
 *  - Splits the last round of query tiles as dit_attn_dense does; with q = k =
 *    the grid tokens at their grid positions the result equals dit_attn_dense
 *    bit for bit. */
dit_status dit_attn_joint(const void* q, const void* k, const void* v,
                          const float* wq, const float* wk,
                          const int* q_pos, const int* k_pos,
                          int nq, int nk, int heads, int head_dim, int max_pos,
                          float rope_theta, float eps,
                          void* o,
                          void* workspace, size_t workspace_bytes, void* hip_stream);

/* Dense attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * dit_attn_dense without a workspace.  Its scratch (the RoPE table and the
 * K^/V fragment images) is a static device array of the library, one per GPU,
 * of DIT_ATTN_NOALLOC_SCRATCH_BYTES (64 MiB), held from the call that first
 * uses it on a GPU until the process ends.  The call allocates no device
 * memory and calls no allocating routine.
 *  - Arguments, layouts and results as dit_attn_dense (the same kernels: the
 *    output equals dit_attn_dense's bit for bit).
 *  - Size limit: the RoPE table plus heads * ceil(N / 128) tile images
 *    (48 KiB each at head_dim 96, 64 KiB at 128) must fit the scratch; larger
 *    calls return DIT_ERR_UNSUPPORTED (at head_dim 96 about 1,360 tiles, e.g.
 *    56 heads x 3,072 tokens or 8 heads x 21,760 tokens).  Calls of this size
 *    are too small to split their last round of query tiles, so no partials
 *    are needed.
 *  - The current device must be the stream's device (DIT_ERR_INVALID_ARG).
 *  - All calls on one GPU share its scratch and it keeps the last call's
 *    contents (nothing in it needs to start at zero): calls that overlap in
 *    time on one GPU (different streams without ordering) race and give wrong
 *    results.  Order them on one stream. */
#define DIT_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dit_status dit_attn_dense_noalloc(const void* q, const void* k, const void* v,
                                  const float* wq, const float* wk,
                                  int T, int H, int W, int heads, int head_dim,
                                  float rope_theta, float eps,
                                  void* o, void* hip_stream);

/* Diagnostic: the order in which the workgroups of the attention calls (dense,
 * block_sparse, joint: the K^/V prepass and the attention kernel) take their
 * work.  0, the default, is the tuned order; 1 reverses it.  Every workgroup
 * writes outputs of its own and reads none another writes, so no result may
 * depend on the order: tests compare both orders bit for bit, which catches
 * races inside a workgroup (its LDS double buffer) that a change of timing
 * exposes.  Process-wide; applies to calls queued after it returns.
 * DIT_ERR_INVALID_ARG for any other value. */
dit_status dit_attn_set_launch_order(int order);

/* Text of the last error on the calling thread ("" if the last call succeeded).
 * Valid until the next call on the same thread. */
const char* dit_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DIT_ATTN_H */
