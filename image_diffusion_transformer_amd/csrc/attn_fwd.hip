// Fused QK-RMSNorm + 3D RoPE + flash-style bidirectional attention for gfx950.
//
// What is computed: the H3 SGLang report (CocoLoop), section on the three
// acceleration tiers, names QK-RMSNorm with 3D RoPE fused ahead of a long,
// non-causal attention; its SubBlock-Sparse-Attention paragraph prunes whole KV
// blocks.  Head shape (56 heads x 96) from the H3-Image spec table, DiT row; the
// same kernels are instantiated for head dim 128, the SubBlock precondition named
// in that report's limits section.
//
// Design (the same kernels serve dense and block-sparse):
//  * A bandwidth-bound prepass normalises and rotates every K row once per layer
//    and writes K^ and V, per (head, 128-key tile), as an image of MFMA operand
//    fragments (64 lanes x 16 bytes each; 48 KB at head dim 96, 64 KB at 128).
//    The attention kernel then stages a KV tile with plain global->LDS copies and
//    no vector ALU work, which leaves the VALU to the softmax.
//  * Attention work is split per (head, query tile of NW*QB*32 tokens); for dense
//    calls the launch index is remapped so the workgroups resident on one XCD walk
//    the same head's K/V and share its L2.  Block-sparse query tiles hold router
//    blocks grouped by the overlap of their kept sets (sparse_sched.hip).
//  * Each wave owns QB blocks of 32 queries (2 at head dim 96, 1 at 128, where
//    the Q fragments and O accumulators of two blocks would not fit the 256
//    registers of a wave).  Its Q rows are loaded once (two lanes per query, half
//    the channels each), RMS-normalised, rotated, scaled by log2(e)/sqrt(d) and
//    kept in registers as bf16 MFMA B operands.
//  * KV tiles are double-buffered in LDS: the next tile's fragment image is in
//    flight (global->LDS, no registers, issued as inline assembly so that the
//    fragment reads get graded LDS waits) while the current one is consumed.
//    Dense calls issue that copy in parts, one per 32-key sub-block, so its LDS
//    writes interleave with the fragment reads.  Block-sparse tiles take their KV
//    tile and slot flags from per-tile lists whose entries are loaded two visits
//    ahead.
//  * Dense calls whose last round of workgroups would leave CUs idle split those
//    query tiles along the keys into pieces with fp32 partial results, which a
//    merge kernel sums (tail_plan).
//  * S^T = K^ Q^T with v_mfma_f32_32x32x16_bf16 (keys on rows, queries on columns):
//    each lane holds one query column, so the softmax row statistics need only
//    in-lane reductions plus one permlane32 swap, and the S^T accumulator is
//    already the B operand of the next MFMA after bf16 packing.
//  * O^T += V^T P^T with the same MFMA, V^T fragments read from LDS with one
//    16-byte load per lane.
//  * Static-shift softmax when the QK-RMSNorm logit bound B allows it (B <= 80 in
//    base 2: p = exp2(S - c), c = max(0, B - 48) taken as the first S MFMA's
//    accumulator input, no running max); otherwise an online softmax in base 2 whose running max
//    m enters the same way (-m as the accumulator input) and only moves (and O, l
//    are rescaled) when a lane's block sum of p passes 2^8, so every p stays
//    <= 2^8 and the block max is computed only then; the final O / l is exact
//    for any stale max.
//  * Row sums accumulate the bf16-rounded probabilities (v_dot2_f32_bf16), the
//    same values the PV product uses.
#include "dit_internal.h"

// Every floating-point expression here is evaluated as written, without fused multiply-adds the compiler
// chooses by itself: the choice could differ between the unrolled copies of the same code (for example
// the two query blocks of a wave), and a query would then round differently depending on which wave and
// slot computes it.  Fused operations are written out (fmaf) where they are wanted.
#pragma clang fp contract(off)

namespace dit {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = kBlock;    // keys per KV tile (= router block)
constexpr float kSumLimit = 256.0f;  // 2^8: largest per-lane block sum of p before the running max moves

// Fragment image of one (head, 128-key tile), written by kv_prep_kernel: FRAGS fragments of 512 bf16
// (lane l owns elements 8l..8l+7).  With KS = d/16 channel steps and DB = d/32 channel blocks:
//   fragment kb*KS + ks      (K^, 0..4KS-1):  lane l holds K^[32kb + l%32][16ks + 8(l/32) + e], e = 0..7:
//                             the A operand of S^T for key sub-block kb, channel step ks.
//   fragment 4KS + (2kb+s)*DB + db (V^T):  lane l holds V[key][32db + l%32] for the keys
//                             32kb + 16s + 4(l/32) + {0, 1, 2, 3, 8, 9, 10, 11}: the A operand of
//                             O^T for channel block db, k-step s of sub-block kb.  That key order is
//                             the one in which the S^T accumulator holds the probabilities.
// Keys past the grid have zero K^ and V.  Head dim 96: 24 + 24 fragments (48 KB); 128: 32 + 32 (64 KB).
constexpr int kFrag = 512;

// Shape of the workgroups: waves and 32-query blocks per wave.
#ifndef DIT_D96_NW
#define DIT_D96_NW 8
#endif
#ifndef DIT_D96_QB
#define DIT_D96_QB 2
#endif
#ifndef DIT_D128_NW
#define DIT_D128_NW 8
#endif
#ifndef DIT_D128_QB
#define DIT_D128_QB 1
#endif

template <int D>
struct Head {
  static_assert(D == 96 || D == 128, "head dim");
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int VFRAG0 = 4 * KS;
  static constexpr int FRAGS = 4 * KS + 8 * DB;
  static constexpr int TILE = FRAGS * kFrag;         // bf16 elements of one tile image
  static constexpr int NW = D == 96 ? DIT_D96_NW : DIT_D128_NW;   // waves per workgroup
  static constexpr int QB = D == 96 ? DIT_D96_QB : DIT_D128_QB;   // 32-query blocks per wave
  static constexpr int BQ = NW * QB * 32;                // queries per workgroup
  static constexpr int RS = rope_row_floats(D);       // floats per RoPE table row
  static constexpr int PAIRS0 = rope_width(D, 0) / 2, PAIRS1 = rope_width(D, 1) / 2;
};

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, const FastDiv& f) {
  return (uint32_t)(((uint64_t)n * f.m) >> f.s);
}

__device__ __forceinline__ void grid_pos(uint32_t n, const GridDesc& g, int& t, int& h, int& w) {
  const uint32_t tt = fastdiv(n, g.div_hw);
  const uint32_t nw = fastdiv(n, g.div_w);
  t = (int)tt;
  h = (int)(nw - tt * (uint32_t)g.H);
  w = (int)(n - nw * (uint32_t)g.W);
}

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// x combined with the same register of lane (l ^ 32); both lanes get bit-identical results.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Rows of the RoPE table that rotate the three axis chunks of token n.  Grid tokens: rows t, T + h and
// T + H + w of the per-axis table.  Tokens with explicit (t, h, w) positions: the coordinates themselves,
// clamped to [0, max_pos), in the axis's section of max_pos rows (rope_sec; at head dim 96 the three
// axes share one section, their rows depending only on the position).
__device__ __forceinline__ void rope_rows(const AttnArgs& a, const int* pos, int n, int (&r)[3]) {
  if (pos != nullptr) {
#pragma unroll
    for (int i = 0; i < 3; ++i) r[i] = a.rope_sec[i] + min(max(pos[3 * (size_t)n + i], 0), a.max_pos - 1);
  } else {
    int t, h, w;
    grid_pos((uint32_t)n, a.g, t, h, w);
    r[0] = t;
    r[1] = a.g.T + h;
    r[2] = a.g.T + a.g.H + w;
  }
}

// RMS-normalise (scale r) and rotate 8 consecutive channels 8c..8c+7 held as bf16 in `raw`.  rows[a]
// points at the RoPE table row of axis a for this token (cos of pair i at i, sin at RS/2 + i).
template <int D>
__device__ __forceinline__ u32x4 norm_rope_chunk(u32x4 raw, float r, float scale, const float* const (&rows)[3],
                                                 int c, const float* wvec) {
  const f32x4 w0 = *(const f32x4*)(wvec + 8 * c);
  const f32x4 w1 = *(const f32x4*)(wvec + 8 * c + 4);
  const float wv[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
  float co[4], si[4];
  if constexpr (D == 96) {
    // 32-channel axis chunks: the vector's 4 pairs are pairs 4(c%4) .. 4(c%4)+3 of axis c/4
    const float* rp = rows[c >> 2];
    const f32x4 cv = *(const f32x4*)(rp + 4 * (c & 3));
    const f32x4 sv = *(const f32x4*)(rp + Head<D>::RS / 2 + 4 * (c & 3));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      co[e] = cv[e];
      si[e] = sv[e];
    }
  } else {
    // chunks of 44, 42, 42 channels: a vector may straddle two axes, so each pair finds its own
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = 4 * c + e;
      const int ax = (p >= Head<D>::PAIRS0) + (p >= Head<D>::PAIRS0 + Head<D>::PAIRS1);
      const int i = p - (ax == 0 ? 0 : (ax == 1 ? Head<D>::PAIRS0 : Head<D>::PAIRS0 + Head<D>::PAIRS1));
      const float* rp = ax == 0 ? rows[0] : (ax == 1 ? rows[1] : rows[2]);
      co[e] = rp[i];
      si[e] = rp[Head<D>::RS / 2 + i];
    }
  }
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float xe = bf_lo(raw[e]) * r * wv[2 * e];
    const float xf = bf_hi(raw[e]) * r * wv[2 * e + 1];
    const float ye = xe * co[e] - xf * si[e];
    const float yf = xe * si[e] + xf * co[e];
    out[e] = pack_bf16(ye * scale, yf * scale);
  }
  return out;
}

// Softmax modes.  QK-RMSNorm bounds every logit.  RoPE rotates each channel pair (2i, 2i+1) rigidly, so
// pair i of q^ . k^ is at most |a_i| |b_i|, with a_i the normalised q pair times its weights:
// |a_i| <= u_i |x_i|, u_i = max(|w_q,2i|, |w_q,2i+1|) (v_i likewise for k).  Summing and Cauchy-Schwarz
// over the pairs (|x| <= sqrt(d) after the norm): |q^ . k^| / sqrt(d) <= sqrt(d) max_i u_i v_i = B (in
// base-2 units), never looser than sqrt(d) max|w_q| max|w_k|.  When B <= kStaticBound, the static mode
// takes p = exp2(S - c) with the constant shift c = max(0, B - 48): every exponent lies in
// [48 - 2B, 48], so p is a normal bf16 / fp32 number, never overflowing (p <= 2^48) nor flushed
// (p >= 2^-112), for any input, and the shift cancels in O / rowsum.  The shift costs nothing: it is
// the accumulator input of each key sub-block's first S MFMA.  No running max, no subtraction, no
// rescale; the fp32 sums stay finite while N max|V| < 2^80.  Otherwise (B > kStaticBound, or NaN
// weights) the online (running-max) softmax runs.
enum SoftmaxMode { kStatic = 0, kOnline = 1 };
constexpr float kStaticBound = 80.0f;
constexpr float kUnshiftedBound = 48.0f;

// Shift of the static mode for these weights (0 while B <= 48).
template <int D>
__device__ __forceinline__ float logit_bound(const AttnArgs& a, int lane, bool& bad_out) {
  float m = 0.f;
  int bad = 0;                                     // a NaN weight sends the call to the online kernel
  for (int i = lane; i < D / 2; i += 64) {
    const float u = fmaxf(fabsf(a.wq[2 * i]), fabsf(a.wq[2 * i + 1]));
    const float v = fmaxf(fabsf(a.wk[2 * i]), fabsf(a.wk[2 * i + 1]));
    bad |= (a.wq[2 * i] != a.wq[2 * i]) | (a.wq[2 * i + 1] != a.wq[2 * i + 1]) |
           (a.wk[2 * i] != a.wk[2 * i]) | (a.wk[2 * i + 1] != a.wk[2 * i + 1]);
    m = fmaxf(m, u * v);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    m = fmaxf(m, __shfl_xor(m, o));
    bad |= __shfl_xor(bad, o);
  }
  // 1.02 covers the approximate reciprocal square root, the rotation and the bf16 rounding of q^, k^.
  const float sqrt_d = D == 96 ? 9.797958971132712f : 11.313708498984761f;
  bad_out = bad != 0;
  return 1.4426950408889634f * sqrt_d * m * 1.02f;
}

template <int D>
__device__ __forceinline__ bool static_bound_holds(const AttnArgs& a, int lane, float& shift) {
  bool bad;
  const float bound = logit_bound<D>(a, lane, bad);
  shift = fmaxf(bound - kUnshiftedBound, 0.0f);
  return !bad && bound <= kStaticBound;            // false for infinite weights too
}

// Query block (32 queries) of the workgroup's tile that block qb of a wave holds.  Dense: wave w holds
// blocks QB*w .. QB*w+QB-1.  Block-sparse (QB = 2): wave w holds part w%4 of router blocks 2(w/4) and
// 2(w/4)+1, so each router block's 128 queries are spread over all four SIMDs (waves w and w+4 share
// SIMD w%4) and a KV tile kept by few router blocks still keeps every SIMD busy.
template <int QB, bool SPARSE, int NW = 8>
__device__ __forceinline__ int query_block(int wave, int qb) {
  if constexpr (SPARSE && QB == 2 && NW == 8) {
    return 8 * (wave >> 2) + 4 * qb + (wave & 3);
  } else if constexpr (SPARSE && QB == 2) {
    // four waves: block qb of wave w is part w of router block qb
    return 4 * qb + wave;
  } else {
    // (block-sparse with one block per wave: waves 0-3 and 4-7 hold the two router blocks of the
    // 256-query tile, each spread over the four SIMDs already)
    return wave * QB + qb;
  }
}
// Router block (within the tile) of the wave's query block qb.
template <int QB, bool SPARSE, int NW = 8>
__device__ __forceinline__ int router_block(int wave, int qb) {
  return query_block<QB, SPARSE, NW>(wave, qb) >> 2;
}

// Token of the query that lane l32 holds in block qb of the wave.  Dense: the tile's consecutive
// tokens.  Block-sparse: slot s of the tile holds the router block that the grouping pass put there
// (a slot without one maps past the last query and is never loaded or stored).
template <int D, bool SPARSE>
__device__ __forceinline__ int query_token(const AttnArgs& a, int head, int qt, int wave, int qb, int l32) {
  constexpr int QB = Head<D>::QB, BQ = Head<D>::BQ;
  const int blk = query_block<QB, SPARSE, Head<D>::NW>(wave, qb);
  if constexpr (SPARSE) {
    const int rb = a.perm[((size_t)head * a.nqt + qt) * (BQ / BK) + (blk >> 2)];
    return rb < 0 ? a.nq : rb * BK + (blk & 3) * 32 + l32;
  } else {
    return qt * BQ + blk * 32 + l32;
  }
}

// Q fragments of the wave: load, RMSNorm, RoPE, scale by log2(e)/sqrt(d), pack to bf16 (once per query).
template <int D, int QB, int BQ, bool SPARSE>
__device__ __forceinline__ void load_q(const AttnArgs& a, int head, int qt, int wave, int lane,
                                       bf16x8 (&qf)[QB][Head<D>::KS]) {
  constexpr int KS = Head<D>::KS;
  const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int n = query_token<D, SPARSE>(a, head, qt, wave, qb, l32);
    const bool live = n < a.nq;
    u32x4 raw[KS];
    const size_t base = ((size_t)(live ? n : 0) * a.g.heads + head) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      raw[ks] = live ? *(const u32x4*)(a.q + base + 16 * ks + 8 * half) : u32x4{0, 0, 0, 0};
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf_lo(raw[ks][e]), hi = bf_hi(raw[ks][e]);
        ss += lo * lo + hi * hi;
      }
    ss = pair_sum(ss);
    const float r = live ? __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.eps) : 0.f;
    int rr[3] = {0, 0, 0};
    if (live) rope_rows(a, a.q_pos, n, rr);
    const float* const rows[3] = {a.rope + rr[0] * Head<D>::RS, a.rope + rr[1] * Head<D>::RS,
                                  a.rope + rr[2] * Head<D>::RS};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = 2 * ks + half;
      qf[qb][ks] = __builtin_bit_cast(bf16x8, norm_rope_chunk<D>(raw[ks], r, a.qscale, rows, c, a.wq));
    }
  }
}

// S^T - m for key sub-block kb (32 keys) against the wave's QB query blocks: KS K^ fragments, KS*QB MFMAs,
// the first of each query block accumulating onto negm[qb] (every element -m of the lane's query).
// QM: bit qb set = query block qb takes part (block-sparse tiles kept by only some of a wave's blocks).
template <int D, int QB, int QM = (1 << QB) - 1>
__device__ __forceinline__ void qk_block(const uint16_t* T_, int kb, int lane, const bf16x8 (&qf)[QB][Head<D>::KS],
                                         const f32x16 (&negm)[QB], f32x16 (&S)[QB]) {
  constexpr int KS = Head<D>::KS;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) S[qb] = negm[qb];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 ka = *(const bf16x8*)(T_ + (kb * KS + ks) * kFrag + lane * 8);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      if (((QM >> qb) & 1) != 0)
        S[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[qb][ks], S[qb], 0, 0, 0);
  }
  // A second reader of each -m block beside its MFMA: with the MFMA as the only one the compiler accumulates in
  // place and copies the block into S every sub-block (16 register moves) instead of reading it as a separate
  // accumulator input.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) asm volatile("" ::"v"(negm[qb]));
}

// O^T += V^T P^T for key sub-block kb: 2*DB V^T fragments, 2*DB*QB MFMAs.
template <int D, int QB, int QM = (1 << QB) - 1>
__device__ __forceinline__ void pv_block(const uint16_t* T_, int kb, int lane, const bf16x8 (&P)[QB][2],
                                         f32x16 (&acc)[QB][Head<D>::DB]) {
  constexpr int DB = Head<D>::DB;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 va = *(const bf16x8*)(T_ + (Head<D>::VFRAG0 + (2 * kb + s) * DB + db) * kFrag + lane * 8);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        if (((QM >> qb) & 1) != 0)
          acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, P[qb][s], acc[qb][db], 0, 0, 0);
    }
}

// Pack 16 probabilities of one query block as two bf16x8 PV operands and add their bf16 values to l.
__device__ __forceinline__ void pack_probs(const float (&p)[16], float& l, bf16x8 (&P)[2]) {
  // Packed pairs kept in scalar variables: bit-casting an element of a u32x4 to bf16x2
  // mis-selects the element in this toolchain (every dot2 then reads element 0).
  uint32_t w[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = pack_bf16(p[2 * e], p[2 * e + 1]);
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float ls = l;
#pragma unroll
  for (int e = 0; e < 8; ++e) ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), one, ls, false);
  l = ls;
  P[0] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
  P[1] = __builtin_bit_cast(bf16x8, u32x4{w[4], w[5], w[6], w[7]});
}

// Key k of register i in a lane's S^T fragment of sub-block kb: kb*32 + 8*(i/4) + 4*(lane/32) + i%4.
__device__ __forceinline__ bool key_live(int key0, int i, int half, int N) {
  return key0 + 8 * (i >> 2) + 4 * half + (i & 3) < N;
}

// Logits of keys past the grid (key index >= N, in the last, ragged tile) set to -inf: p = 0 there.
template <int QB>
__device__ __forceinline__ void mask_past_grid(f32x16 (&S)[QB], int key0, int N, int lane) {
  const int half = lane >> 5;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool live = key_live(key0, i, half, N);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) S[qb][i] = live ? S[qb][i] : -INFINITY;
  }
}

// Online (running-max) softmax of one sub-block.  S holds the logits less the lane's running max m (the
// accumulator input of the sub-block's first S MFMA was -m), so p = exp2(S) needs no subtraction; keys >= N get
// probability 0.  Every p is at most its lane's block sum, so while every sum of the wave stays within
// kSumLimit no p exceeds it and m needs no update.  lim holds the limit a lane's block sum is held to: kSumLimit
// once the lane has a running max, -1 before its first block with a live key (no sum passes it).  Only when some
// sum of the wave is past its limit, infinite or NaN is the block max computed: then m moves up to the block max
// (to it, for a first block), O and l are rescaled, p is redone with the extra subtraction and -m is written to
// negm for the next sub-blocks.  All query blocks are exponentiated first and checked with one branch.
// The running max lives only in negm (m = -negm[qb][0]), which gives the block a use besides the MFMA: with
// the MFMA as its only reader the compiler accumulates in place and copies the block into S every sub-block.
template <int DB, int QB, int QM = (1 << QB) - 1>
__device__ __forceinline__ void softmax_online(f32x16 (&S)[QB], bool ragged, int key0, int N, int lane,
                                               float (&lim)[QB], f32x16 (&negm)[QB], float (&l)[QB],
                                               f32x16 (&acc)[QB][DB], bf16x8 (&P)[QB][2]) {
  if (ragged) mask_past_grid<QB>(S, key0, N, lane);
  float lb[QB];
  bool over = false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (((QM >> qb) & 1) == 0) continue;
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(S[qb][i]);
    lb[qb] = 0.f;
    pack_probs(p, lb[qb], P[qb]);
    over = over || !(lb[qb] <= lim[qb]);
  }
  if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (((QM >> qb) & 1) == 0) continue;
      if (!__builtin_amdgcn_ballot_w64(!(lb[qb] <= lim[qb]))) continue;
      const bool has_max = lim[qb] >= 0.f;
      float mx = S[qb][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, S[qb][i]);
      mx = pair_max(mx);
      // raise of m: up to the block max (to it, for a lane without a max yet); none for a block of masked keys
      const bool live = mx > -INFINITY;
      const float d = live ? (has_max ? fmaxf(mx, 0.f) : mx) : 0.f;
      const float alpha = __builtin_amdgcn_exp2f(-d);
      l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[qb][db] *= alpha;
      const float mnew = d - negm[qb][0];
      lim[qb] = (has_max || live) ? kSumLimit : -1.f;
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(S[qb][i] - d);
      lb[qb] = 0.f;
      pack_probs(p, lb[qb], P[qb]);
#pragma unroll
      for (int i = 0; i < 16; ++i) negm[qb][i] = -mnew;
    }
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
    if ((QM >> qb) & 1) l[qb] += lb[qb];
}

// Static-shift softmax of one sub-block: p = exp2(S), S already holding the logits less the constant shift.
// The caller has masked keys past the grid to -inf.
template <int QB, int QM = (1 << QB) - 1>
__device__ __forceinline__ void softmax_static(const f32x16 (&S)[QB], float (&l)[QB], bf16x8 (&P)[QB][2]) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (((QM >> qb) & 1) == 0) continue;
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(S[qb][i]);
    pack_probs(p, l[qb], P[qb]);
  }
}

template <int D, int QB, int BQ, bool SPARSE>
__device__ __forceinline__ void store_o(const AttnArgs& a, int head, int qt, int wave, int lane,
                                        const f32x16 (&acc)[QB][Head<D>::DB], const float (&l)[QB]) {
  const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int n = query_token<D, SPARSE>(a, head, qt, wave, qb, l32);
    const float lt = pair_sum(l[qb]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    if (n < a.nq) {
      uint16_t* op = a.o + ((size_t)n * a.g.heads + head) * D;
#pragma unroll
      for (int db = 0; db < Head<D>::DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = db * 32 + 8 * j + 4 * half;
          u32x2 v;
          v[0] = pack_bf16(acc[qb][db][4 * j] * inv, acc[qb][db][4 * j + 1] * inv);
          v[1] = pack_bf16(acc[qb][db][4 * j + 2] * inv, acc[qb][db][4 * j + 3] * inv);
          *(u32x2*)(op + d) = v;
        }
    }
  }
}

// Partial result of a tail piece: per wave, query block and lane, its DB x 16 accumulators, its row sum
// and its running maximum (-inf before any key; 0 in the static mode, whose constant shift is the same for
// every piece), element-major so that each store is coalesced over the lanes.
template <int D>
constexpr int kPartialElems = Head<D>::DB * 16 + 2;

template <int D>
__device__ __forceinline__ void store_partial(const AttnArgs& a, int slot, int wave, int lane,
                                              const f32x16 (&acc)[Head<D>::QB][Head<D>::DB],
                                              const float (&l)[Head<D>::QB], const f32x16 (&negm)[Head<D>::QB],
                                              const float (&lim)[Head<D>::QB], bool online) {
  constexpr int QB = Head<D>::QB, DB = Head<D>::DB, NW = Head<D>::NW, E = kPartialElems<D>;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float* dst = a.partial + (((size_t)slot * NW + wave) * QB + qb) * E * 64 + lane;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[(db * 16 + i) * 64] = acc[qb][db][i];
    dst[(E - 2) * 64] = l[qb];
    dst[(E - 1) * 64] = online ? (lim[qb] >= 0.f ? -negm[qb][0] : -INFINITY) : 0.f;
  }
}

// Shared setup of both kernels: workgroup -> (head, query tile) with the XCD-aware order, tile list.
struct TileIter {
  int head, qt, ntiles;
  int k0;                       // dense: first KV tile (a tail piece starts inside the key range)
  int slot;                     // tail piece: index of its partial result
  const int* lst;               // block-sparse: visited KV tiles (plain indices below nb)
  const unsigned char* flg;     // block-sparse: slots of the query tile that keep each visited tile
  __device__ __forceinline__ int tile(int it, bool sparse) const { return sparse ? lst[it] : k0 + it; }
};

template <bool SPARSE, bool PIECE = false>
__device__ __forceinline__ bool tile_iter(const AttnArgs& a, TileIter& ti) {
  // Dense: XCD x (launch index mod 8) takes a contiguous run of (head, query tile) pairs, so the
  // workgroups resident on one XCD walk one head's K/V in step and share its L2.  The last tail_rem tiles
  // of each run may be split into key-range pieces (a kernel of their own, PIECE).  Block-sparse: the
  // tiles of a head visit different KV subsets and drift apart, so L2 sharing is weak; consecutive
  // launch indices keep the whole chip on about one head at a time instead, whose fragment image is
  // then re-read from the last-level cache rather than HBM (3% faster on the 10 s video layer).
  // The diagnostic reversed order (a.order) permutes the same work within each run.
  const int nt = (a.nk + BK - 1) / BK;
  int logical;
  ti.k0 = 0;
  ti.slot = 0;
  ti.ntiles = nt;
  if constexpr (SPARSE) {
    logical = (int)blockIdx.x;
    if (logical >= a.total) return false;
    if (a.order != 0) logical = a.total - 1 - logical;
  } else {
    const int x = (int)(blockIdx.x & 7), x0 = x * a.per_xcd;
    int j = (int)(blockIdx.x >> 3);
    if constexpr (!PIECE) {
      const int valid = min(a.main_per_xcd, a.total - x0);
      if (j >= valid) return false;
      if (a.order != 0) j = valid - 1 - j;
      logical = x0 + j;
    } else {
      int piece = j / a.tail_rem, t = j - piece * a.tail_rem;
      const int valid = min(a.tail_rem, a.total - x0 - a.main_per_xcd);
      if (piece >= a.tail_pieces || t >= valid) return false;
      if (a.order != 0) {
        t = valid - 1 - t;
        piece = a.tail_pieces - 1 - piece;
      }
      logical = x0 + a.main_per_xcd + t;
      ti.slot = (x * a.tail_rem + t) * a.tail_pieces + piece;
      ti.k0 = piece * nt / a.tail_pieces;
      ti.ntiles = (piece + 1) * nt / a.tail_pieces - ti.k0;
    }
  }
  ti.head = logical / a.nqt;
  ti.qt = logical - ti.head * a.nqt;
  if constexpr (SPARSE) {
    ti.ntiles = a.list_len[logical];
    ti.lst = a.list + (size_t)logical * a.nb;
    ti.flg = a.list_flags + (size_t)logical * a.nb;
  } else {
    ti.lst = nullptr;
    ti.flg = nullptr;
  }
  return true;
}

// ------------------------------------------------------------------------------------------------
// K^ / V fragment prepass: one workgroup per (128-key tile, head).  The tile's raw K and V rows are read
// with coalesced 16-byte loads into LDS; each K row is RMS-normalised and rotated (two threads per row,
// d/16 8-channel chunks each) and every fragment lane slot is written with one 16-byte store.
template <int D>
__global__ void __launch_bounds__(256) kv_prep_kernel(AttnArgs a) {
  constexpr int KS = Head<D>::KS, DB = Head<D>::DB, CH = D / 8;
  __shared__ __attribute__((aligned(16))) uint16_t rk[BK * D];
  __shared__ __attribute__((aligned(16))) uint16_t rv[BK * D];
  __shared__ __attribute__((aligned(16))) float sW[D];
  const int tile = a.order != 0 ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
  const int head = a.order != 0 ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y;
  const int tid = threadIdx.x, N = a.nk;
  if (tid < D) sW[tid] = a.wk[tid];
  for (int i = tid; i < BK * CH; i += 256) {
    const int row = i / CH, c = i - CH * row;
    const int n = tile * BK + row;
    u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
    if (n < N) {
      const size_t off = ((size_t)n * a.g.heads + head) * D + 8 * c;
      kx = *(const u32x4*)(a.k + off);
      vx = *(const u32x4*)(a.v + off);
    }
    *(u32x4*)(rk + row * D + 8 * c) = kx;
    *(u32x4*)(rv + row * D + 8 * c) = vx;
  }
  __syncthreads();
  uint16_t* img = a.kvf + ((size_t)head * a.nb + tile) * Head<D>::TILE;
  {
    const int kk = tid & (BK - 1), cg = tid >> 7;     // key row; chunks KS*cg .. KS*cg + KS-1
    const int n = tile * BK + kk;
    const bool live = n < N;
    const u32x4* row = (const u32x4*)(rk + kk * D);
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const u32x4 x = row[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf_lo(x[e]), hi = bf_hi(x[e]);
        ss += lo * lo + hi * hi;
      }
    }
    const float r = live ? __builtin_amdgcn_rsqf(ss * (1.0f / D) + a.eps) : 0.f;
    int rr[3] = {0, 0, 0};
    if (live) rope_rows(a, a.k_pos, n, rr);
    const float* const rows[3] = {a.rope + rr[0] * Head<D>::RS, a.rope + rr[1] * Head<D>::RS,
                                  a.rope + rr[2] * Head<D>::RS};
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const int c = KS * cg + j;                       // channels 8c .. 8c+7 = step c/2, lane half c%2
      const u32x4 y = norm_rope_chunk<D>(row[c], r, 1.0f, rows, c, sW);
      *(u32x4*)(img + ((kk >> 5) * KS + (c >> 1)) * kFrag + ((c & 1) * 32 + (kk & 31)) * 8) =
          live ? y : u32x4{0, 0, 0, 0};
    }
  }
  for (int i = tid; i < 8 * DB * 64; i += 256) {
    const int f = i >> 6, l = i & 63;                  // f = (2kb + s)*DB + db
    const int d = 32 * (f % DB) + (l & 31);
    const int key0 = 16 * (f / DB) + 4 * (l >> 5);
    uint32_t w[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const int key = key0 + 2 * e2 + (e2 >= 2 ? 4 : 0);
      w[e2] = (uint32_t)rv[key * D + d] | ((uint32_t)rv[(key + 1) * D + d] << 16);
    }
    *(u32x4*)(img + (Head<D>::VFRAG0 + f) * kFrag + l * 8) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// One 16-byte-per-lane global -> LDS copy issued as inline assembly: lane l reads the 16 bytes at
// src + voff_l (src a wave-uniform address in scalar registers, voff_l = 16 l) and writes LDS bytes
// [dst + 16 l, dst + 16 l + 16).  With the builtin, the compiler cannot order the copy against later LDS
// reads and waits for every outstanding read (lgkmcnt(0)) before each use; the assembly form has no
// register result, the copy only counts against vmcnt (waited for explicitly at the tile barrier), and the
// reads of the current stage get graded waits.  The memory clobber keeps LDS accesses on their side.  Both
// addresses are wave-uniform, so forming them takes scalar instructions only.
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t voff, __attribute__((address_space(3))) void* lds_dst) {
  const uint32_t base = (uint32_t)(uintptr_t)lds_dst;
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(src), "{m0}"(base) : "memory");
}

// This wave's share (fragments FPW*w .. FPW*w + FPW-1, FPW = FRAGS / 8) of one tile's fragment image,
// copied global -> LDS without passing through registers: lane l of each copy moves the 16 bytes of lane
// slot l.  src (the tile's image), wave and dst are wave-uniform; voff = 16 * lane.
template <int D>
__device__ __forceinline__ void dma_tile(const uint16_t* src, int wave, uint32_t voff, uint16_t* dst) {
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int FPW = Head<D>::FRAGS / Head<D>::NW;
  static_assert(FPW * Head<D>::NW == Head<D>::FRAGS, "fragments per wave");
#pragma unroll
  for (int c = 0; c < FPW; ++c) {
    const int f = FPW * wave + c;
    lds_copy16((const void*)(src + f * kFrag), voff, (lds_void*)(dst + f * kFrag));
  }
}

// The next tile's copy as the dense loop issues it: in BK/32 parts, one at the start of each sub-block of
// the current tile (fragments 2, 1, 2, 1 of the wave's 6 at head dim 96; 2 each at 128), so that its LDS writes
// interleave with the waves' fragment reads instead of arriving in one burst (1% faster on the dense layer;
// the block-sparse loop, whose visits are shorter, issues the whole copy at the top of the visit).
struct CopyJob {
  const uint16_t* src;      // the tile's fragment image (wave-uniform)
  uint16_t* dst;            // its LDS stage
  int wave;                 // wave index (scalar)
  uint32_t voff;            // 16 * lane
  bool on;                  // false: nothing to copy in the sub-blocks
};

template <int D>
__device__ __forceinline__ void dma_part(const CopyJob& cj, int kb) {
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int FPW = Head<D>::FRAGS / Head<D>::NW;
  constexpr int NP = BK / 32;
  const int lo = (kb * FPW + NP - 1) / NP, hi = ((kb + 1) * FPW + NP - 1) / NP;
  for (int c = lo; c < hi; ++c) {
    const int f = FPW * cj.wave + c;
    lds_copy16((const void*)(cj.src + f * kFrag), cj.voff, (lds_void*)(cj.dst + f * kFrag));
  }
}

// Barrier that publishes a tile.  Each wave first waits for its own global->LDS copies (vmcnt(0): the
// compiler does not relate these copies to later LDS reads and inserts no wait for them) and for its LDS
// accesses (lgkmcnt(0)); after the barrier every wave's copies have landed.  sched_barrier(0) and the
// empty asm statements keep the compiler from moving any instruction or memory access across.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------------------------------------------------------------------
// Attention kernels: 8 waves (2 per SIMD), QB blocks of 32 queries per wave.  Per KV tile: copy the next
// tile's fragment image into the other LDS stage (block-sparse: all at once at the top; dense: a part at the
// start of each sub-block), and per 32-key sub-block: S MFMAs, softmax, PV MFMAs.  One barrier per tile.  Block-sparse tiles are computed only for the query blocks whose
// router block keeps them (activity mask QM of the wave's blocks).
// S^T - c of sub-block kb with its first two K^ fragments already in registers (kp); negc holds -c in
// every element and is the accumulator input of the first MFMA.
template <int D, int QB, int QM>
__device__ __forceinline__ void qk_block_pre(const uint16_t* T_, int kb, int lane, const bf16x8 (&qf)[QB][Head<D>::KS],
                                             const bf16x8 (&kp)[2], const f32x16& negc, f32x16 (&S)[QB]) {
  constexpr int KS = Head<D>::KS;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) S[qb] = negc;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 ka = ks < 2 ? kp[ks] : *(const bf16x8*)(T_ + (kb * KS + ks) * kFrag + lane * 8);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      if (((QM >> qb) & 1) != 0)
        S[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[qb][ks], S[qb], 0, 0, 0);
  }
}

// Issue priority of the younger wave of each SIMD (waves 4-7 share SIMDs with waves 0-3, which the issue
// arbiter favours) raised for a tile's last sub-block, so it catches up with its partner before the tile
// barrier instead of finishing the tile alone.  Reset after the barrier.  Dense only: measured 0.9% faster on
// the dense layer and 0.7% slower on the block-sparse one.
__device__ __forceinline__ void raise_younger_wave(int kb, int wave) {
  if (kb == BK / 32 - 1 && wave >= 4) __builtin_amdgcn_s_setprio(1);
}

template <int D, int QB, int QM, int MODE>
__device__ __forceinline__ void tile_body(const uint16_t* T_, int lane, int wave, bool balance,
                                          const bf16x8 (&qf)[QB][Head<D>::KS],
                                          f32x16 (&acc)[QB][Head<D>::DB], float (&lim)[QB], f32x16 (&negm)[QB],
                                          float (&l)[QB], const f32x16& negc, bool ragged, int key0, int N,
                                          const CopyJob& cj) {
  constexpr int KS = Head<D>::KS;
  if constexpr (MODE == kStatic) {
    // The first two K^ fragments of each sub-block are read while the previous sub-block's S MFMAs
    // drain, so a sub-block's S MFMAs start without an LDS wait (measured 0.6% on the dense layer;
    // the online mode, with its longer softmax, was slower this way and keeps the plain order).
    bf16x8 kp[2];
    kp[0] = *(const bf16x8*)(T_ + 0 * kFrag + lane * 8);
    kp[1] = *(const bf16x8*)(T_ + 1 * kFrag + lane * 8);
    auto sub_block = [&](int kb) {
      if (balance) raise_younger_wave(kb, wave);
      // copy part: before the S MFMAs at head dim 96, after them at 128 (each measured the faster there)
      if (D == 96 && cj.on) dma_part<D>(cj, kb);
      f32x16 S[QB];
      qk_block_pre<D, QB, QM>(T_, kb, lane, qf, kp, negc, S);
      if (D == 128 && cj.on) dma_part<D>(cj, kb);
      const int nk = kb + 1 < BK / 32 ? kb + 1 : kb;   // the last sub-block re-reads its own (unused)
      kp[0] = *(const bf16x8*)(T_ + (nk * KS + 0) * kFrag + lane * 8);
      kp[1] = *(const bf16x8*)(T_ + (nk * KS + 1) * kFrag + lane * 8);
      __builtin_amdgcn_sched_barrier(0);
      // Keys past the grid are masked, not counted and taken off the row sum at the end: when every real
      // logit of a row is very negative, its sum would vanish next to that count in fp32.
      if (ragged) mask_past_grid<QB>(S, key0 + kb * 32, N, lane);
      bf16x8 P[QB][2];
      softmax_static<QB, QM>(S, l, P);
      pv_block<D, QB, QM>(T_, kb, lane, P, acc);
      asm volatile("" ::"v"(kp[0]), "v"(kp[1]));   // keeps the reads where they are issued
    };
    if (balance) {
      // Dense: the four sub-blocks unrolled (fragment offsets become immediates, no loop bookkeeping):
      // measured 0.9% faster on the dense layer.  The block-sparse variants keep the loop, whose unrolled
      // form spills registers at the loop boundary.
#pragma unroll
      for (int kb = 0; kb < BK / 32; ++kb) sub_block(kb);
    } else {
#pragma unroll 1
      for (int kb = 0; kb < BK / 32; ++kb) sub_block(kb);
    }
  } else {
#pragma unroll 1
    for (int kb = 0; kb < BK / 32; ++kb) {
      if (balance) raise_younger_wave(kb, wave);
      if (cj.on) dma_part<D>(cj, kb);
      f32x16 S[QB];
      qk_block<D, QB, QM>(T_, kb, lane, qf, negm, S);
      bf16x8 P[QB][2];
      softmax_online<Head<D>::DB, QB, QM>(S, ragged, key0 + kb * 32, N, lane, lim, negm, l, acc, P);
      pv_block<D, QB, QM>(T_, kb, lane, P, acc);
    }
  }
}

// Both modes mask keys past the grid (zero K^ and V) in the last, ragged KV tile only.
template <int D, bool SPARSE, int MODE, bool PIECE>
__device__ __forceinline__ void attn_kernel_body(const AttnArgs& a, uint16_t* sKV) {
  constexpr int QB = Head<D>::QB, BQ = Head<D>::BQ, TILE = Head<D>::TILE;
  constexpr int KS = Head<D>::KS, DB = Head<D>::DB;
  static_assert(BQ % BK == 0, "tile shape");
  TileIter ti;
  if (!tile_iter<SPARSE, PIECE>(a, ti)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // A scalar copy of the wave index for the tile copies, whose addresses are then scalar arithmetic.  (Used
  // everywhere, it costs the block-sparse kernel at head dim 96 register spills.)
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t voff = 16u * (uint32_t)lane;
  float shift;
  if (static_bound_holds<D>(a, lane, shift) != (MODE == kStatic)) return;   // the other kernel takes these weights
  f32x16 negc;
#pragma unroll
  for (int i = 0; i < 16; ++i) negc[i] = -shift;
  const int N = a.nk, nt = ti.ntiles;
  int rbit[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) rbit[qb] = router_block<QB, SPARSE, Head<D>::NW>(wave, qb);
  const uint16_t* img = a.kvf + (size_t)ti.head * a.nb * TILE;
  if (nt > 0) dma_tile<D>(img + (size_t)__builtin_amdgcn_readfirstlane(ti.tile(0, SPARSE)) * TILE, wave_s, voff, sKV);
  bf16x8 qf[QB][KS];
  load_q<D, QB, BQ, SPARSE>(a, ti.head, ti.qt, wave, lane, qf);
  // Finish Q here: left free, the compiler sinks the norm and rotation below the first tile barrier,
  // next to the loop, and carries the raw loads across it in scratch.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[qb][ks]));
  f32x16 acc[QB][DB];
  // Online mode: -m, the running max of the lane's query (0 and not yet set before its first block with a
  // live key), in every element of negm, the accumulator input of each sub-block's first S MFMA.
  float l[QB];
  float lim[QB];
  f32x16 negm[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    lim[qb] = -1.f;
    negm[qb] = f32x16{};
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = f32x16{};
  }
  // Block-sparse: the list entries (tile and slot flags) of the current and the next tile are carried in
  // registers, and those two tiles ahead are loaded at the top of each iteration; only the tile barrier's
  // vmcnt(0) waits for them, so no visit stalls on a list read before it can start the next copy and its
  // own MFMAs.  Tile indices and flags come from separate arrays: a copy address is formed from a plain
  // tile index, with no field to mask off.
  // List entries are the same in every lane; the loaded ones (in flight: vector registers) are made scalar one
  // visit before their use, which keeps the copy addressing and the activity mask scalar.
  int e_cur = 0, e_nxt = 0, f_cur = 0, f_nxt = 0;
  if constexpr (SPARSE) {
    e_cur = nt > 0 ? __builtin_amdgcn_readfirstlane(ti.lst[0]) : 0;
    e_nxt = nt > 1 ? ti.lst[1] : 0;
    f_cur = nt > 0 ? __builtin_amdgcn_readfirstlane(ti.flg[0]) : 0;
    f_nxt = nt > 1 ? ti.flg[1] : 0;
  }
  tile_barrier();
  for (int it = 0; it < nt; ++it) {
    int e_nn = 0, f_nn = 0;
    if constexpr (SPARSE) {
      e_nn = it + 2 < nt ? ti.lst[it + 2] : 0;
      f_nn = it + 2 < nt ? ti.flg[it + 2] : 0;
      e_nxt = __builtin_amdgcn_readfirstlane(e_nxt);   // loaded a visit ago
      f_nxt = __builtin_amdgcn_readfirstlane(f_nxt);
    }
    const int st = it & 1, tile = SPARSE ? e_cur : ti.k0 + it;
    CopyJob cj{img + (size_t)(SPARSE ? e_nxt : tile + 1) * TILE, sKV + (st ^ 1) * TILE, wave_s, voff, false};
    if (it + 1 < nt) {
      if constexpr (SPARSE)
        dma_tile<D>(cj.src, wave_s, voff, cj.dst);
      else
        cj.on = true;
    }
    const int flags = SPARSE ? f_cur : 0xff;
    int qm = 0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) qm |= ((flags >> rbit[qb]) & 1) << qb;
    const uint16_t* T_ = sKV + (st != 0 ? TILE : 0);     // a select, not a multiply by the stage
    const bool ragged = (tile + 1) * BK > N;
    if constexpr (SPARSE && QB == 2) {
      if (qm == 3)
        tile_body<D, QB, 3, MODE>(T_, lane, wave, false, qf, acc, lim, negm, l, negc, ragged, tile * BK, N, cj);
      else if (qm == 1)
        tile_body<D, QB, 1, MODE>(T_, lane, wave, false, qf, acc, lim, negm, l, negc, ragged, tile * BK, N, cj);
      else if (qm == 2)
        tile_body<D, QB, 2, MODE>(T_, lane, wave, false, qf, acc, lim, negm, l, negc, ragged, tile * BK, N, cj);
    } else if constexpr (SPARSE) {
      if (qm != 0) tile_body<D, QB, (1 << QB) - 1, MODE>(T_, lane, wave, false, qf, acc, lim, negm, l, negc, ragged, tile * BK, N, cj);
    } else {
      tile_body<D, QB, (1 << QB) - 1, MODE>(T_, lane, wave, true, qf, acc, lim, negm, l, negc, ragged, tile * BK,
                                            N, cj);
    }
    tile_barrier();
    if constexpr (!SPARSE) __builtin_amdgcn_s_setprio(0);
    e_cur = e_nxt;
    e_nxt = e_nn;
    f_cur = f_nxt;
    f_nxt = f_nn;
  }
  if constexpr (PIECE)
    store_partial<D>(a, ti.slot, wave, lane, acc, l, negm, lim, MODE == kOnline);
  else
    store_o<D, QB, BQ, SPARSE>(a, ti.head, ti.qt, wave, lane, acc, l);
}

template <int D, bool SPARSE, bool PIECE>
__global__ void __launch_bounds__(64 * Head<D>::NW) attn_static_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sKV[2 * Head<D>::TILE];
  attn_kernel_body<D, SPARSE, kStatic, PIECE>(a, sKV);
}

template <int D, bool SPARSE, bool PIECE>
__global__ void __launch_bounds__(64 * Head<D>::NW) attn_online_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sKV[2 * Head<D>::TILE];
  attn_kernel_body<D, SPARSE, kOnline, PIECE>(a, sKV);
}

// Merge of a split tile's pieces: per lane, the pieces' accumulators and row sums are rescaled to their
// largest running maximum (the static mode writes 0 for every piece: no rescale) and summed in piece
// order, then O is normalised and stored as by the unsplit kernels.
template <int D>
__global__ void __launch_bounds__(64 * Head<D>::NW) attn_merge_kernel(AttnArgs a) {
  constexpr int QB = Head<D>::QB, DB = Head<D>::DB, NW = Head<D>::NW, E = kPartialElems<D>;
  const int x = (int)(blockIdx.x & 7), t = (int)(blockIdx.x >> 3);
  const int x0 = x * a.per_xcd;
  if (t >= min(a.tail_rem, a.total - x0 - a.main_per_xcd)) return;
  const int logical = x0 + a.main_per_xcd + t;
  const int head = logical / a.nqt, qt = logical - head * a.nqt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot0 = (x * a.tail_rem + t) * a.tail_pieces;
  f32x16 acc[QB][DB];
  float l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float mx = -INFINITY;
    for (int p = 0; p < a.tail_pieces; ++p) {
      const float* src = a.partial + (((size_t)(slot0 + p) * NW + wave) * QB + qb) * E * 64 + lane;
      mx = fmaxf(mx, src[(E - 1) * 64]);
    }
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = f32x16{};
    if (mx == -INFINITY) continue;                 // no piece saw a key: O = 0, as unsplit
    for (int p = 0; p < a.tail_pieces; ++p) {
      const float* src = a.partial + (((size_t)(slot0 + p) * NW + wave) * QB + qb) * E * 64 + lane;
      const float m = src[(E - 1) * 64];
      if (m == -INFINITY) continue;
      const float f = __builtin_amdgcn_exp2f(m - mx);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[qb][db][i] += f * src[(db * 16 + i) * 64];
      l[qb] += f * src[(E - 2) * 64];
    }
  }
  store_o<D, QB, Head<D>::BQ, false>(a, head, qt, wave, lane, acc, l);
}

template <int D, bool SPARSE>
hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(kv_prep_kernel<D>, dim3(a.nb, a.g.heads), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 block(64 * Head<D>::NW);
  const int blocks = SPARSE ? a.per_xcd * 8 : a.main_per_xcd * 8;
  // Both softmax kernels are queued; each checks the weight bound itself and the one that does
  // not apply returns before touching any data.
  if (blocks > 0) {
    hipLaunchKernelGGL((attn_static_kernel<D, SPARSE, false>), dim3(blocks), block, 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((attn_online_kernel<D, SPARSE, false>), dim3(blocks), block, 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if constexpr (!SPARSE) {
    if (a.tail_pieces > 1) {
      const int pieces = 8 * a.tail_rem * a.tail_pieces;
      hipLaunchKernelGGL((attn_static_kernel<D, false, true>), dim3(pieces), block, 0, s, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL((attn_online_kernel<D, false, true>), dim3(pieces), block, 0, s, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL(attn_merge_kernel<D>, dim3(8 * a.tail_rem), block, 0, s, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

int attn_query_tile(int head_dim) { return head_dim == 128 ? Head<128>::BQ : Head<96>::BQ; }

size_t tail_partial_bytes(int head_dim) {
  return head_dim == 128 ? (size_t)Head<128>::NW * Head<128>::QB * kPartialElems<128> * 64 * sizeof(float)
                         : (size_t)Head<96>::NW * Head<96>::QB * kPartialElems<96> * 64 * sizeof(float);
}

TailPlan tail_plan(int total, int nk) {
  constexpr int kCusPerXcd = 32;
  TailPlan p;
  p.per_xcd = (total + 7) / 8;
  p.main_per_xcd = p.per_xcd;
  p.rem = 0;
  p.pieces = 1;
  const int rounds = p.per_xcd / kCusPerXcd, rem = p.per_xcd % kCusPerXcd;
  const int nt = (nk + BK - 1) / BK;
  // Small calls are left alone (their whole run is one or a few rounds), and so are key ranges too short
  // to split.
  if (rounds < 4 || rem == 0 || nt < 16) return p;
  // Last-round time, in units of one unsplit tile, with the rem tiles cut into P pieces: ceil(rem P / 32)
  // rounds of 1/P each.
  int best = 1;
  double best_cost = 1.0;
  for (int P = 2; P <= 4; ++P) {
    const double cost = (double)((rem * P + kCusPerXcd - 1) / kCusPerXcd) / P;
    if (cost < best_cost - 1e-9) {
      best = P;
      best_cost = cost;
    }
  }
  // worth it only if it saves at least 1% of the call
  if ((1.0 - best_cost) / (rounds + 1) < 0.01) return p;
  p.main_per_xcd = p.per_xcd - rem;
  p.rem = rem;
  p.pieces = best;
  return p;
}

hipError_t launch_attn_dense(const AttnArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? launch_attn<128, false>(a, s) : launch_attn<96, false>(a, s);
}
hipError_t launch_attn_sparse(const AttnArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? launch_attn<128, true>(a, s) : launch_attn<96, true>(a, s);
}

}  // namespace dit
