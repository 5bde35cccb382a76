// Fused QK-RMSNorm + 3D RoPE + flash-style bidirectional attention for gfx950.
//
// What is computed: the H3 SGLang report (CocoLoop), section on the three
// acceleration tiers, names QK-RMSNorm with 3D RoPE fused ahead of a long,
// non-causal attention; its SubBlock-Sparse-Attention paragraph prunes whole KV
// blocks.  Head shape (56 heads x 96) from the H3-Image spec table, DiT row.
//
// Design (one kernel for dense and block-sparse):
//  * Work is split per (head, query tile of NW*QB*32 tokens); the launch index is
//    remapped so the workgroups resident on one XCD walk the same head's K/V and
//    share its L2.
//  * Each wave owns QB blocks of 32 queries.  Its Q rows are loaded once (two
//    lanes per query, 48 channels each), RMS-normalised, rotated, scaled by
//    log2(e)/sqrt(96) and kept in registers as bf16 MFMA B operands.
//  * K/V stream through LDS in tiles of 128 keys, double-buffered: while a tile is
//    consumed, the next tile's raw rows are already in registers; K rows are then
//    RMS-normalised and rotated once per workgroup and written as bf16, V rows are
//    copied as they are.
//  * S^T = K^ Q^T with v_mfma_f32_32x32x16_bf16 (keys on rows, queries on columns):
//    each lane holds one query column, so the softmax row statistics need only
//    in-lane reductions plus one permlane32 swap, and the S^T accumulator is
//    already the B operand of the next MFMA after bf16 packing.
//  * O^T += V^T P^T with the same MFMA; V^T fragments come straight from the
//    row-major V tile through ds_read_b64_tr_b16 (transposing LDS reads).
//  * Online softmax in base 2 with a lazy rescale: the running max only moves
//    (and O, l are rescaled) when a block max exceeds it by more than 8, so
//    exp2 arguments stay <= 8; the final O / l is exact for any stale max.
//  * Row sums accumulate the bf16-rounded probabilities (v_dot2_f32_bf16), the
//    same values the PV product uses.
#include "dit_internal.h"

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
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int BK = kBlock;    // keys per KV tile (= router block)
constexpr int KROW = 104;     // bf16 per K^ row in LDS: 208 B (odd multiple of 16 B): conflict-free b128 reads
constexpr int VROW = 96;      // bf16 per V row in LDS: 192 B: conflict-free transposing reads
constexpr float kTau = 8.0f;  // lazy-rescale threshold, base-2 log units

// Kernel shape: kNW waves per workgroup, kQB blocks of 32 queries per wave.
#ifndef DIT_ATTN_NW
#define DIT_ATTN_NW 8
#endif
#ifndef DIT_ATTN_QB
#define DIT_ATTN_QB 2
#endif
constexpr int kNW = DIT_ATTN_NW;
constexpr int kQB = DIT_ATTN_QB;
constexpr int kBQ = kNW * kQB * 32;   // queries per workgroup

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

// Sum over groups of TPK adjacent lanes (TPK in {1, 2, 4}); every lane of a group gets the same bits.
template <int TPK>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (TPK >= 2) x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
  if constexpr (TPK >= 4) x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
  return x;
}

__device__ __forceinline__ int rope_row(const GridDesc& g, int axis, int t, int h, int w) {
  return axis == 0 ? t : (axis == 1 ? g.T + h : g.T + g.H + w);
}

// RMS-normalise (scale r) and rotate 8 consecutive channels 8c..8c+7 held as bf16 in `raw`.
__device__ __forceinline__ u32x4 norm_rope_chunk(u32x4 raw, float r, float scale, const float* rope_row_ptr,
                                                 int c, const float* wvec) {
  const f32x4 co = *(const f32x4*)(rope_row_ptr + 4 * (c & 3));
  const f32x4 si = *(const f32x4*)(rope_row_ptr + kPairs + 4 * (c & 3));
  const f32x4 w0 = *(const f32x4*)(wvec + 8 * c);
  const f32x4 w1 = *(const f32x4*)(wvec + 8 * c + 4);
  const float wv[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
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

template <int TPK, int CPT>
__device__ __forceinline__ void load_kv_raw(const AttnArgs& a, int head, int tile, int kk, int sub,
                                            u32x4 (&kr)[CPT], u32x4 (&vr)[CPT]) {
  const int n = tile * BK + kk;
  if (n < a.g.N) {
    const size_t base = ((size_t)n * a.g.heads + head) * kHeadDim;
    const u32x4* kp = (const u32x4*)(a.k + base);
    const u32x4* vp = (const u32x4*)(a.v + base);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      kr[j] = kp[sub + TPK * j];
      vr[j] = vp[sub + TPK * j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      kr[j] = u32x4{0, 0, 0, 0};
      vr[j] = u32x4{0, 0, 0, 0};
    }
  }
}

// Normalise + rotate this thread's K chunks and write K^ and V into one LDS stage.
template <int TPK, int CPT>
__device__ __forceinline__ void stage_kv(const AttnArgs& a, int tile, int kk, int sub,
                                         const u32x4 (&kr)[CPT], const u32x4 (&vr)[CPT],
                                         const float* wk, uint16_t* sK, uint16_t* sV) {
  const int n = tile * BK + kk;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bf_lo(kr[j][e]), hi = bf_hi(kr[j][e]);
      ss += lo * lo + hi * hi;
    }
  ss = group_sum<TPK>(ss);
  const bool live = n < a.g.N;
  const float r = live ? __builtin_amdgcn_rsqf(ss * (1.0f / kHeadDim) + a.eps) : 0.f;
  int t = 0, h = 0, w = 0;
  if (live) grid_pos((uint32_t)n, a.g, t, h, w);
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = sub + TPK * j;
    const float* rp = a.rope + rope_row(a.g, c >> 2, t, h, w) * kRopeRow;
    const u32x4 y = norm_rope_chunk(kr[j], r, 1.0f, rp, c, wk);
    *(u32x4*)(sK + kk * KROW + 8 * c) = live ? y : u32x4{0, 0, 0, 0};
    *(u32x4*)(sV + kk * VROW + 8 * c) = vr[j];
  }
}

// V^T fragment (A operand, 32 channels x 16 keys) for k-step s of key sub-block kb, channel block db.
// Lane group g = lane/16 covers channels d0..d0+15 of half hh = g/2; k-slots 0..3 of the half are keys
// base+0..3, k-slots 4..7 keys base+8..11 (matching where S^T keeps those keys).
__device__ __forceinline__ bf16x8 load_vt(const uint16_t* sV, int kb, int s, int db, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int d0 = db * 32 + 16 * (g & 1);
  const int key = kb * 32 + 16 * s + 4 * (g >> 1) + (i >> 2);
  const int col = d0 + 4 * (i & 3);
  const lds_s16x4* p0 = (const lds_s16x4*)(sV + key * VROW + col);
  const lds_s16x4* p1 = (const lds_s16x4*)(sV + (key + 8) * VROW + col);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Softmax modes.  QK-RMSNorm bounds every logit: |q^ . k^| / sqrt(96) <= sqrt(96) max|w_q| max|w_k|
// (RoPE preserves norms).  When that bound, in base-2 units, is at most kStaticBound, exp2(S) with
// no shift can neither overflow nor underflow for any input, and the shift cancels in O / rowsum:
// no running max, no subtraction, no rescale.  Otherwise the online (running-max) softmax runs.
enum SoftmaxMode { kStatic = 0, kOnline = 1 };
constexpr float kStaticBound = 48.0f;

__device__ __forceinline__ bool static_bound_holds(const AttnArgs& a, int lane) {
  float mq = 0.f, mk = 0.f;
  for (int i = lane; i < kHeadDim; i += 64) {
    mq = fmaxf(mq, fabsf(a.wq[i]));
    mk = fmaxf(mk, fabsf(a.wk[i]));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mq = fmaxf(mq, __shfl_xor(mq, o));
    mk = fmaxf(mk, __shfl_xor(mk, o));
  }
  // |q^|, |k^| <= sqrt(96) max|w| (RMS <= 1 after the norm); 1.02 covers rsq, rotation and bf16 rounding.
  const float bound = 1.4426950408889634f * 9.797958971132712f * mq * mk * 1.02f;
  return bound <= kStaticBound;   // false for NaN weights
}

template <int NW, int QB, bool SPARSE, int MODE>
__global__ void __launch_bounds__(NW * 64) attn_kernel(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int BQ = NW * QB * 32;
  constexpr int TPK = NT / BK;        // threads per key row while staging
  constexpr int CPT = 12 / TPK;       // 16-byte chunks per thread per tensor
  static_assert(TPK * BK == NT && CPT * TPK == 12, "staging layout");
  static_assert(BQ % BK == 0, "query tile must hold whole router blocks");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2 * BK * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2 * BK * VROW];
  // K's norm weights live in LDS: read once per tile there instead of being held in registers.
  __shared__ __attribute__((aligned(16))) float sWk[kHeadDim];

  const int logical = (int)(blockIdx.x & 7) * a.per_xcd + (int)(blockIdx.x >> 3);
  if (logical >= a.total) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Both softmax kernels are launched; the one whose mode does not apply exits here.
  if (static_bound_holds(a, lane) != (MODE == kStatic)) return;
  if (tid < kHeadDim) sWk[tid] = a.wk[tid];
  __syncthreads();
  const int head = logical / a.nqt;
  const int qt = logical - head * a.nqt;
  const int half = lane >> 5, l32 = lane & 31;
  const int N = a.g.N;
  const int rb = (wave * QB * 32) / BK;   // router block of this wave inside the query tile

  int ntiles;
  const int* lst = nullptr;
  if constexpr (SPARSE) {
    ntiles = a.list_len[logical];
    lst = a.list + (size_t)logical * a.nb;
  } else {
    ntiles = (N + BK - 1) / BK;
  }

  // ---- Q: load, RMSNorm, RoPE, scale, pack (once per query) ----
  bf16x8 qf[QB][6];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int n = qt * BQ + (wave * QB + qb) * 32 + l32;
    const bool live = n < N;
    u32x4 raw[6];
    const size_t base = ((size_t)(live ? n : 0) * a.g.heads + head) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks)
      raw[ks] = live ? *(const u32x4*)(a.q + base + 16 * ks + 8 * half) : u32x4{0, 0, 0, 0};
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf_lo(raw[ks][e]), hi = bf_hi(raw[ks][e]);
        ss += lo * lo + hi * hi;
      }
    ss = pair_sum(ss);
    const float r = live ? __builtin_amdgcn_rsqf(ss * (1.0f / kHeadDim) + a.eps) : 0.f;
    int t = 0, h = 0, w = 0;
    if (live) grid_pos((uint32_t)n, a.g, t, h, w);
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) {
      const int c = 2 * ks + half;
      const float* rp = a.rope + rope_row(a.g, ks >> 1, t, h, w) * kRopeRow;
      qf[qb][ks] = __builtin_bit_cast(bf16x8, norm_rope_chunk(raw[ks], r, a.qscale, rp, c, a.wq));
    }
  }

  f32x16 acc[QB][3];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -1e30f;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < 3; ++db) acc[qb][db] = f32x16{};
  }

  const int kk = tid / TPK, sub = tid % TPK;
  u32x4 kr[CPT], vr[CPT];
  if (ntiles > 0) {
    const int t0 = SPARSE ? (lst[0] & 0xffffff) : 0;
    load_kv_raw<TPK, CPT>(a, head, t0, kk, sub, kr, vr);
    stage_kv<TPK, CPT>(a, t0, kk, sub, kr, vr, sWk, sK, sV);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int st = it & 1;
    int tile = it, flags = 0xff;
    if constexpr (SPARSE) {
      const int e = lst[it];
      tile = e & 0xffffff;
      flags = e >> 24;
    }
    const bool has_next = it + 1 < ntiles;
    const int ntile = has_next ? (SPARSE ? (lst[it + 1] & 0xffffff) : it + 1) : 0;
    if (has_next) load_kv_raw<TPK, CPT>(a, head, ntile, kk, sub, kr, vr);

    if ((flags >> rb) & 1) {
      const uint16_t* K_ = sK + st * BK * KROW;
      const uint16_t* V_ = sV + st * BK * VROW;
      const bool ragged = (tile + 1) * BK > N;
#pragma unroll 1
      for (int kb = 0; kb < BK / 32; ++kb) {
        f32x16 S[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) S[qb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 6; ++ks) {
          const bf16x8 ka = *(const bf16x8*)(K_ + (kb * 32 + l32) * KROW + 16 * ks + 8 * half);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            S[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[qb][ks], S[qb], 0, 0, 0);
        }
        if (ragged) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = tile * BK + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
            if (key >= N)
#pragma unroll
              for (int qb = 0; qb < QB; ++qb) S[qb][i] = -INFINITY;
          }
        }
        bf16x8 P[QB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if constexpr (MODE == kOnline) {
            float mx = S[qb][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, S[qb][i]);
            mx = pair_max(mx);
            if (__builtin_amdgcn_ballot_w64(mx > m[qb] + kTau)) {
              const float mn = fmaxf(m[qb], mx);
              const float alpha = __builtin_amdgcn_exp2f(m[qb] - mn);
              l[qb] *= alpha;
#pragma unroll
              for (int db = 0; db < 3; ++db) acc[qb][db] *= alpha;
              m[qb] = mn;
            }
          }
          float p[16];
#pragma unroll
          for (int i = 0; i < 16; ++i)
            p[i] = __builtin_amdgcn_exp2f(MODE == kOnline ? S[qb][i] - m[qb] : S[qb][i]);
          // Packed pairs kept in scalar variables: bit-casting an element of a u32x4 to bf16x2
          // mis-selects the element in this toolchain (every dot2 then reads element 0).
          uint32_t w[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = pack_bf16(p[2 * e], p[2 * e + 1]);
          const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
          float ls = l[qb];
#pragma unroll
          for (int e = 0; e < 8; ++e) ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), one, ls, false);
          l[qb] = ls;
          P[qb][0] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
          P[qb][1] = __builtin_bit_cast(bf16x8, u32x4{w[4], w[5], w[6], w[7]});
        }
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int db = 0; db < 3; ++db) {
            const bf16x8 va = load_vt(V_, kb, s, db, lane);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, P[qb][s], acc[qb][db], 0, 0, 0);
          }
      }
    }
    if (has_next)
      stage_kv<TPK, CPT>(a, ntile, kk, sub, kr, vr, sWk, sK + (st ^ 1) * BK * KROW, sV + (st ^ 1) * BK * VROW);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, bf16 RNE ----
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int n = qt * BQ + (wave * QB + qb) * 32 + l32;
    const float lt = pair_sum(l[qb]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    if (n < N) {
      uint16_t* op = a.o + ((size_t)n * a.g.heads + head) * kHeadDim;
#pragma unroll
      for (int db = 0; db < 3; ++db)
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

// Block-sparse iteration lists: for each (head, query tile) the ascending KV blocks kept by any of the
// tile's router blocks, each tagged with which of them keep it (bit b = router block b of the tile).
__global__ void __launch_bounds__(256) compact_kernel(CompactArgs a) {
  __shared__ int wave_tot[4];
  const int tile = blockIdx.x;              // head * nqt + qt
  const int head = tile / a.nqt, qt = tile - head * a.nqt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int* out = a.list + (size_t)tile * a.nb;
  int base = 0;
  for (int j0 = 0; j0 < a.nb; j0 += 256) {
    const int j = j0 + threadIdx.x;
    int flags = 0;
    if (j < a.nb)
      for (int b = 0; b < a.group; ++b) {
        const int i = qt * a.group + b;
        if (i < a.nb && a.mask[((size_t)head * a.nb + i) * a.nb + j]) flags |= 1 << b;
      }
    const uint64_t bal = __builtin_amdgcn_ballot_w64(flags != 0);
    const int before = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wave_tot[w];
    if (flags) out[off + before] = j | (flags << 24);
    base += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.list_len[tile] = base;
}

template <bool SPARSE>
hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  const int blocks = a.per_xcd * 8;
  // Both softmax kernels are queued; each checks the weight bound itself and the one that does
  // not apply returns before touching any data.
  hipLaunchKernelGGL((attn_kernel<kNW, kQB, SPARSE, kStatic>), dim3(blocks), dim3(kNW * 64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_kernel<kNW, kQB, SPARSE, kOnline>), dim3(blocks), dim3(kNW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int attn_query_tile() { return kBQ; }

hipError_t launch_attn_dense(const AttnArgs& a, hipStream_t s) { return launch_attn<false>(a, s); }
hipError_t launch_attn_sparse(const AttnArgs& a, hipStream_t s) { return launch_attn<true>(a, s); }

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(compact_kernel, dim3(a.heads * a.nqt), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dit
