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
// computed on the host.  The three kernels:
//   route_rms:    1 / sqrt(mean(x^2) + eps) per (tensor, token, head), channel sum in order 0..95
//   route_pool:   per (tensor, head, block, channel pair): normalise, rotate and sum the block's
//                 tokens in ascending order, then divide by the token count
//   route_select: per (head, query block): scores against every KV block (channel sum in order),
//                 then an exact top-k by a bitwise radix search on an order-preserving key
#include "dit_internal.h"

#pragma clang fp contract(off)

namespace dit {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__global__ void __launch_bounds__(256) route_rms_kernel(RouteArgs a) {
  const long long per = (long long)a.g.N * a.g.heads;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= 2 * per) return;
  const int tensor = idx >= per;
  const long long row = tensor ? idx - per : idx;
  const u32x4* x = (const u32x4*)((tensor ? a.k : a.q) + row * kHeadDim);
  float ss = 0.f;
  for (int j = 0; j < 12; ++j) {
    const u32x4 v = x[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bf_lo(v[e]), hi = bf_hi(v[e]);
      ss = __fadd_rn(ss, __fmul_rn(lo, lo));
      ss = __fadd_rn(ss, __fmul_rn(hi, hi));
    }
  }
  const float ms = __fdiv_rn(ss, (float)kHeadDim);
  a.r[idx] = __fdiv_rn(1.0f, __builtin_sqrtf(__fadd_rn(ms, a.eps)));
}

__global__ void __launch_bounds__(256) route_pool_kernel(RouteArgs a) {
  const int npair = kHeadDim / 2;
  const long long total = 2ll * a.g.heads * a.nb * npair;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int p = (int)(idx % npair);
  long long rest = idx / npair;
  const int b = (int)(rest % a.nb);
  rest /= a.nb;
  const int head = (int)(rest % a.g.heads);
  const int tensor = (int)(rest / a.g.heads);
  const uint16_t* X = tensor ? a.k : a.q;
  const float* R = a.r + (size_t)tensor * a.g.N * a.g.heads;
  const float* wv = tensor ? a.wk : a.wq;
  const float we = wv[2 * p], wf = wv[2 * p + 1];
  const int axis = p / kPairs, i = p % kPairs;
  const int n0 = b * kBlock;
  const int n1 = min(a.g.N, n0 + kBlock);
  int t = n0 / (a.g.H * a.g.W);
  int h = (n0 / a.g.W) % a.g.H;
  int w = n0 % a.g.W;
  float acc_e = 0.f, acc_f = 0.f;
  for (int n = n0; n < n1; ++n) {
    const size_t row = (size_t)n * a.g.heads + head;
    const uint32_t x2 = *(const uint32_t*)(X + row * kHeadDim + 2 * p);
    const float r = R[row];
    const int trow = axis == 0 ? t : (axis == 1 ? a.g.T + h : a.g.T + a.g.H + w);
    const float c = a.rope[trow * kRopeRow + i];
    const float s = a.rope[trow * kRopeRow + kPairs + i];
    const float xe = __fmul_rn(__fmul_rn(bf_lo(x2), r), we);
    const float xf = __fmul_rn(__fmul_rn(bf_hi(x2), r), wf);
    const float ye = __fsub_rn(__fmul_rn(xe, c), __fmul_rn(xf, s));
    const float yf = __fadd_rn(__fmul_rn(xe, s), __fmul_rn(xf, c));
    acc_e = __fadd_rn(acc_e, ye);
    acc_f = __fadd_rn(acc_f, yf);
    if (++w == a.g.W) {
      w = 0;
      if (++h == a.g.H) {
        h = 0;
        ++t;
      }
    }
  }
  const float cnt = (float)(n1 - n0);
  float* out = a.pooled + (((size_t)tensor * a.g.heads + head) * a.nb + b) * kHeadDim;
  out[2 * p] = __fdiv_rn(acc_e, cnt);
  out[2 * p + 1] = __fdiv_rn(acc_f, cnt);
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

__global__ void __launch_bounds__(256) route_select_kernel(RouteArgs a) {
  extern __shared__ uint32_t keys[];   // [nb] scores, then order keys
  __shared__ float qrow[kHeadDim];
  __shared__ int red[4];
  __shared__ int scan[256];
  const int nb = a.nb;
  const int row = blockIdx.x;          // head * nb + i
  const int head = row / nb, i = row - head * nb;
  const float* qbar = a.pooled + ((size_t)head * nb + i) * kHeadDim;
  const float* kbar = a.pooled + ((size_t)(a.g.heads + head) * nb) * kHeadDim;
  if (threadIdx.x < kHeadDim) qrow[threadIdx.x] = qbar[threadIdx.x];
  __syncthreads();
  for (int j = threadIdx.x; j < nb; j += 256) {
    const f32x4* kv = (const f32x4*)(kbar + (size_t)j * kHeadDim);
    float acc = 0.f;
    for (int c4 = 0; c4 < kHeadDim / 4; ++c4) {
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

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  const long long n1 = 2ll * a.g.N * a.g.heads;
  hipLaunchKernelGGL(route_rms_kernel, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n2 = 2ll * a.g.heads * a.nb * (kHeadDim / 2);
  hipLaunchKernelGGL(route_pool_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)a.nb * sizeof(uint32_t);
  if (lds > 64 * 1024) {
    e = hipFuncSetAttribute((const void*)route_select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(route_select_kernel, dim3(a.g.heads * a.nb), dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace dit
