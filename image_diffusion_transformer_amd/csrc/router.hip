// Block router of the block-sparse mode (gfx950), reproducible bit for bit.
//
// Source: H3 SGLang report (CocoLoop), SubBlock-Sparse-Attention paragraph in the
// section on the three acceleration tiers -- a block-wise sparse router prunes the
// KV blocks taking part in attention, at sparsity 0.75 or 0.80.  Reading of the
// unspecified parts: 128-token blocks of the flattened grid; mean-pooled
// post-RMSNorm / post-RoPE q and k in fp32; score = dot(qbar_i, kbar_j); the
// diagonal block is always kept (score +inf); keep the top
// nb - floor(s*nb + 1e-9) blocks per query block, lower index first on ties.
//
// Every fp32 operation below runs in one fixed order with IEEE round-to-nearest:
// explicit __f*_rn intrinsics (plain IEEE operations), no contraction (this file is built with
// -ffp-contract=off), correctly rounded sqrt (__builtin_sqrtf: approximation plus an exact
// neighbour check) and division (the default IEEE division expansion), and cos/sin tables
// computed on the host.  The kernels:
//   route_pool:   per (block, head, tensor): 1 / sqrt(mean(x^2) + eps) per token (channel sum in
//                 order 0..95), then per channel pair: normalise, rotate and sum the block's tokens
//                 in ascending order, then divide by the token count
//   route_score:  per (head, 64 x 64 tile of block pairs): dot products (channel sum in order)
//                 written as order-preserving keys, the diagonal as +inf
//   route_topk:   per (head, query block): exact top-k of the key row by a bitwise search
//   route_select: the same scores and top-k in one workgroup per row, for grids with more
//                 blocks than the top-k kernel holds in registers
#include "dit_internal.h"

#pragma clang fp contract(off)

namespace dit {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// LDS row stride of a staged token row: d bf16 = d/2 words, padded by 4 (52 or 68 words) so that
// the 16-byte reads of consecutive rows by consecutive lanes cover all 64 banks without conflict.
template <int D>
constexpr int row_words() { return D / 2 + 4; }
constexpr int kPoolPart = 64;   // tokens staged at a time (half a block)

// One wave per (block, head, tensor), over the block's two halves in token order: stage the
// half's rows in LDS (coalesced 16-byte loads), compute each token's reciprocal RMS (sequential
// channel sum) and RoPE table rows, then let lane p < 48 walk the tokens in ascending order,
// normalising and rotating its channel pair and adding it to the running block sums.
template <int D>
__global__ void __launch_bounds__(64) route_pool_kernel(RouteArgs a) {
  constexpr int kRowWords = row_words<D>(), CH = D / 8, RS = rope_row_floats(D);
  constexpr int P0 = rope_width(D, 0) / 2, P1 = rope_width(D, 1) / 2;
  __shared__ __attribute__((aligned(16))) uint32_t xs[kPoolPart * kRowWords];
  __shared__ float rs[kPoolPart];
  __shared__ int rowoff[kPoolPart][3];   // float offsets of the t, h and w rows of the RoPE table
  const int b = blockIdx.x, head = blockIdx.y, tensor = blockIdx.z;
  const int lane = threadIdx.x;
  const uint16_t* X = tensor ? a.k : a.q;
  const int n0 = b * kBlock;
  const int cnt = min(kBlock, a.g.N - n0);
  const float* wv = tensor ? a.wk : a.wq;
  const int p = min(lane, D / 2 - 1);
  const float we = wv[2 * p], wf = wv[2 * p + 1];
  const int axis = (p >= P0) + (p >= P0 + P1);
  const int i = p - (axis == 0 ? 0 : (axis == 1 ? P0 : P0 + P1));
  float acc_e = 0.f, acc_f = 0.f;
  for (int m0 = 0; m0 < cnt; m0 += kPoolPart) {
    const int part_cnt = min(kPoolPart, cnt - m0);
    // Rows past the tail block's last token repeat that token; they are staged but never read.
    constexpr int kChunks = kPoolPart * CH / 64;   // 16-byte chunks per lane
    u32x4 v[kChunks];
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int c = lane + 64 * k, t = c / CH, part = c - CH * t;
      const int tl = min(t, part_cnt - 1);
      v[k] = *(const u32x4*)(X + ((size_t)(n0 + m0 + tl) * a.g.heads + head) * D + part * 8);
    }
    __syncthreads();   // the previous half's rows are no longer read
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int c = lane + 64 * k, t = c / CH, part = c - CH * t;
      *(u32x4*)(xs + t * kRowWords + part * 4) = v[k];
    }
    __syncthreads();
    if (lane < part_cnt) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const u32x4 x = *(const u32x4*)(xs + lane * kRowWords + 4 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = bf_lo(x[e]), hi = bf_hi(x[e]);
          ss = __fadd_rn(ss, __fmul_rn(lo, lo));
          ss = __fadd_rn(ss, __fmul_rn(hi, hi));
        }
      }
      const float ms = __fdiv_rn(ss, (float)D);
      rs[lane] = __fdiv_rn(1.0f, __builtin_sqrtf(__fadd_rn(ms, a.eps)));
      const int n = n0 + m0 + lane;
      const int t = n / (a.g.H * a.g.W), h = (n / a.g.W) % a.g.H, w = n % a.g.W;
      rowoff[lane][0] = t * RS;
      rowoff[lane][1] = (a.g.T + h) * RS;
      rowoff[lane][2] = (a.g.T + a.g.H + w) * RS;
    }
    __syncthreads();
#pragma unroll 8
    for (int n = 0; n < part_cnt; ++n) {
      const uint32_t x2 = xs[n * kRowWords + p];
      const float r = rs[n];
      const int ro = rowoff[n][axis];
      const float c = a.rope[ro + i];
      const float s = a.rope[ro + RS / 2 + i];
      const float xe = __fmul_rn(__fmul_rn(bf_lo(x2), r), we);
      const float xf = __fmul_rn(__fmul_rn(bf_hi(x2), r), wf);
      const float ye = __fsub_rn(__fmul_rn(xe, c), __fmul_rn(xf, s));
      const float yf = __fadd_rn(__fmul_rn(xe, s), __fmul_rn(xf, c));
      acc_e = __fadd_rn(acc_e, ye);
      acc_f = __fadd_rn(acc_f, yf);
    }
  }
  if (lane >= D / 2) return;
  const float fc = (float)cnt;
  float* out = a.pooled + (((size_t)tensor * a.g.heads + head) * a.nb + b) * D;
  out[2 * p] = __fdiv_rn(acc_e, fc);
  out[2 * p + 1] = __fdiv_rn(acc_f, fc);
}

// Order-preserving key: larger float -> larger unsigned; -0.0 maps with +0.0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int block_sum256(int v, int* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// Block scores of one head as order keys: a 64 x 64 tile of (query block, KV block) pairs per
// workgroup, the pooled vectors staged channel-major in LDS (row stride 65 words: conflict-free
// transposing stores).  Thread (ty, tx) owns rows ty + 16a and columns tx + 16b; every dot product
// runs over channels 0..95 in order.
constexpr int kScoreTile = 64;
constexpr int kTileStride = kScoreTile + 1;

template <int D>
__global__ void __launch_bounds__(256) route_score_kernel(RouteArgs a) {
  __shared__ float qs[D * kTileStride];
  __shared__ float ks[D * kTileStride];
  const int nb = a.nb;
  const int j0 = blockIdx.x * kScoreTile, i0 = blockIdx.y * kScoreTile, head = blockIdx.z;
  const int tid = threadIdx.x;
  const f32x4* qbar = (const f32x4*)(a.pooled + ((size_t)head * nb + i0) * D);
  const f32x4* kbar = (const f32x4*)(a.pooled + ((size_t)(a.g.heads + head) * nb + j0) * D);
  constexpr int kVec = kScoreTile * D / 4;
  for (int f = tid; f < kVec; f += 256) {
    const int row = f / (D / 4), c4 = f - row * (D / 4);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const f32x4 qv = i0 + row < nb ? qbar[f] : zero;
    const f32x4 kv = j0 + row < nb ? kbar[f] : zero;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qs[(4 * c4 + e) * kTileStride + row] = qv[e];
      ks[(4 * c4 + e) * kTileStride + row] = kv[e];
    }
  }
  __syncthreads();
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int z = 0; z < 4; ++z) acc[u][z] = 0.f;
#pragma unroll 4
  for (int c = 0; c < D; ++c) {
    float qv[4], kv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) qv[u] = qs[c * kTileStride + ty + 16 * u];
#pragma unroll
    for (int z = 0; z < 4; ++z) kv[z] = ks[c * kTileStride + tx + 16 * z];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int z = 0; z < 4; ++z) acc[u][z] = __fadd_rn(acc[u][z], __fmul_rn(qv[u], kv[z]));
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = i0 + ty + 16 * u;
    if (i >= nb) continue;
    uint32_t* dst = a.scores + ((size_t)head * nb + i) * nb;
#pragma unroll
    for (int z = 0; z < 4; ++z) {
      const int j = j0 + tx + 16 * z;
      if (j < nb) dst[j] = order_key(i == j ? INFINITY : acc[u][z]);
    }
  }
}

// Exact top-k of one score row per wave, R keys per lane (key j = 64m + lane in slot m; slots
// past nb hold 0, below every real key).  A bitwise search from the top bit finds the largest
// threshold that at least `keep` keys reach (wave ballots, no barriers); keys above it are kept,
// and keys equal to it are kept in index order until `keep` is reached.
template <int R>
__global__ void __launch_bounds__(256) route_topk_kernel(RouteArgs a) {
  const int nb = a.nb;
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);   // head * nb + i
  if (row >= (long long)a.g.heads * nb) return;
  const uint32_t* src = a.scores + row * nb;
  uint32_t key[R];
#pragma unroll
  for (int m = 0; m < R; ++m) {
    const int j = 64 * m + lane;
    key[m] = j < nb ? src[j] : 0u;
  }
  const int keep = a.keep;
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int m = 0; m < R; ++m) cnt += __popcll(__ballot(key[m] >= cand));
    if (cnt >= keep) thr = cand;
  }
  int gt = 0;
#pragma unroll
  for (int m = 0; m < R; ++m) gt += __popcll(__ballot(key[m] > thr));
  const int need = keep - gt;
  const unsigned long long below = (1ull << lane) - 1ull;
  int before = 0;
  unsigned char* mrow = a.mask + row * nb;
#pragma unroll
  for (int m = 0; m < R; ++m) {
    const unsigned long long eq = __ballot(key[m] == thr);
    const int rank = before + __popcll(eq & below);
    const bool kept = key[m] > thr || (key[m] == thr && rank < need);
    const int j = 64 * m + lane;
    if (j < nb) mrow[j] = kept ? 1 : 0;
    before += __popcll(eq);
  }
}

// Large-nb path (nb > route_topk_max_blocks()): one workgroup per score row, scores and order keys in LDS.
template <int D>
__global__ void __launch_bounds__(256) route_select_kernel(RouteArgs a) {
  extern __shared__ uint32_t keys[];   // [nb] scores, then order keys
  __shared__ float qrow[D];
  __shared__ int red[4];
  __shared__ int scan[256];
  const int nb = a.nb;
  const int row = blockIdx.x;          // head * nb + i
  const int head = row / nb, i = row - head * nb;
  const float* qbar = a.pooled + ((size_t)head * nb + i) * D;
  const float* kbar = a.pooled + ((size_t)(a.g.heads + head) * nb) * D;
  if (threadIdx.x < D) qrow[threadIdx.x] = qbar[threadIdx.x];
  __syncthreads();
  for (int j = threadIdx.x; j < nb; j += 256) {
    const f32x4* kv = (const f32x4*)(kbar + (size_t)j * D);
    float acc = 0.f;
    for (int c4 = 0; c4 < D / 4; ++c4) {
      const f32x4 k4 = kv[c4];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __fadd_rn(acc, __fmul_rn(qrow[4 * c4 + e], k4[e]));
    }
    keys[j] = order_key(j == i ? INFINITY : acc);
  }
  __syncthreads();

  // Each thread owns a contiguous run of columns so that index order is easy to scan.
  const int per = (nb + 255) / 256;
  const int j0 = min(nb, threadIdx.x * per), j1 = min(nb, j0 + per);
  const int keep = a.keep;
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int cnt = 0;
    for (int j = j0; j < j1; ++j) cnt += keys[j] >= cand;
    if (block_sum256(cnt, red) >= keep) thr = cand;
  }
  int gt = 0, eq = 0;
  for (int j = j0; j < j1; ++j) {
    gt += keys[j] > thr;
    eq += keys[j] == thr;
  }
  const int need = keep - block_sum256(gt, red);
  // exclusive scan of eq over threads (index order)
  scan[threadIdx.x] = eq;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = threadIdx.x >= o ? scan[threadIdx.x - o] : 0;
    __syncthreads();
    scan[threadIdx.x] += v;
    __syncthreads();
  }
  int before = scan[threadIdx.x] - eq;
  unsigned char* mrow = a.mask + (size_t)row * nb;
  for (int j = j0; j < j1; ++j) {
    const uint32_t kj = keys[j];
    unsigned char kept = 0;
    if (kj > thr) {
      kept = 1;
    } else if (kj == thr) {
      kept = before < need;
      ++before;
    }
    mrow[j] = kept;
  }
}


template <int D>
hipError_t launch_route_d(const RouteArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(route_pool_kernel<D>, dim3(a.nb, a.g.heads, 2), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.nb <= route_topk_max_blocks()) {
    const unsigned tiles = (unsigned)((a.nb + kScoreTile - 1) / kScoreTile);
    hipLaunchKernelGGL(route_score_kernel<D>, dim3(tiles, tiles, a.g.heads), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned rows = (unsigned)(((long long)a.g.heads * a.nb + 3) / 4);
    if (a.nb <= 1024)
      hipLaunchKernelGGL(route_topk_kernel<16>, dim3(rows), dim3(256), 0, s, a);
    else if (a.nb <= 2048)
      hipLaunchKernelGGL(route_topk_kernel<32>, dim3(rows), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(route_topk_kernel<64>, dim3(rows), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const size_t lds = (size_t)a.nb * sizeof(uint32_t);
  if (lds > 64 * 1024) {
    e = hipFuncSetAttribute((const void*)route_select_kernel<D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(route_select_kernel<D>, dim3(a.g.heads * a.nb), dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? launch_route_d<128>(a, s) : launch_route_d<96>(a, s);
}

}  // namespace dit
