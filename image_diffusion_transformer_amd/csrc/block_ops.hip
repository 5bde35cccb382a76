// Fused elementwise operators around attention in the DiT block (gfx950).
//
// Source: H3 SGLang report (CocoLoop), fused-operator paragraph in the section on the three
// acceleration tiers -- the AdaLN update, the gated residual path and the SwiGLU activation are
// fused kernels that cut activation traffic and change no result; H3-Image spec table, "DiT" row
// (hidden 5376, FFN 14336).  Forms: h = LayerNorm(x) * (1 + scale) + shift (no affine LayerNorm
// parameters, population variance, eps inside the root); r = x + gate * y; out = silu(g) * u over
// the two halves of the fused up projection.
//
// All three are HBM streams: each activation byte is read once and each output byte written once,
// with 16-byte accesses and float32 arithmetic in registers.
//   adaln_kernel<VPT, RESID, NORM>: one wave per token row; lane l holds the 8-channel vectors
//     l, l + 64, ... (VPT of them), packed.  The optional gated residual is formed in float32 and
//     written if asked; the LayerNorm takes the mean, then the centred second moment (no
//     E[x^2] - E[x]^2 cancellation), each by a 64-lane butterfly that leaves every lane with the
//     same bits, then normalises and modulates.
//   swiglu_kernel<U>: one workgroup per (token row, chunk of 256 U vectors); all loads of a thread
//     are issued before its first store.
#include "dit_internal.h"

namespace dit {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two floats to a bf16 pair (round to nearest, ties to even), low channel in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Activations are touched once: loads and stores carry the nontemporal hint (measured on MI355X:
// a 4 GiB read stream reaches 7.1 TB/s with it against 6.5 without; copies 5.56 against 5.34).
__device__ __forceinline__ u32x4 load_stream(const uint16_t* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}
__device__ __forceinline__ void store_stream(uint16_t* p, const u32x4 v) {
  __builtin_nontemporal_store(v, (u32x4*)p);
}

__device__ __forceinline__ void unpack8(const u32x4 v, float (&f)[8]) {
  f[0] = bf_lo(v.x); f[1] = bf_hi(v.x);
  f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
  f[4] = bf_lo(v.z); f[5] = bf_hi(v.z);
  f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 v;
  v.x = pack_bf16(f[0], f[1]);
  v.y = pack_bf16(f[2], f[3]);
  v.z = pack_bf16(f[4], f[5]);
  v.w = pack_bf16(f[6], f[7]);
  return v;
}

__device__ __forceinline__ void load8f(const float* p, float (&f)[8]) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Start of a pass over the packed row: the compiler may neither keep float32 copies of the row
// from an earlier pass nor hoist later LDS reads above this point (either would take registers
// that hold other waves' rows in flight).
// Returns the lane index as a value the compiler cannot see through, so that the pass recomputes
// its vector addresses (a few integer instructions) rather than holding them in registers.
template <int VPT, bool RESID>
__device__ __forceinline__ int pass_fence(u32x4 (&xv)[VPT], u32x4 (&yv)[VPT]) {
  __asm__ volatile("" ::: "memory");
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    __asm__ volatile("" : "+v"(xv[i]));
    if (RESID) __asm__ volatile("" : "+v"(yv[i]));
  }
  int lane = threadIdx.x & 63;
  __asm__ volatile("" : "+v"(lane));
  return lane;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Gated residual of one 8-channel vector from the packed row and the gate staged in LDS:
// r = x + gate * y (one fma per channel, so every pass rebuilds the same float32 r).
template <bool RESID>
__device__ __forceinline__ void resid8(const u32x4 xv, const u32x4 yv, const float* gate, float (&r)[8]) {
  unpack8(xv, r);
  if (RESID) {
    float y[8], g[8];
    unpack8(yv, y);
    load8f(gate, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = __builtin_fmaf(g[e], y[e], r[e]);
  }
}

// Persistent workgroups: the float32 vectors (gate; shift and 1 + scale) are staged in LDS once per
// workgroup, then each wave takes token rows in a grid-stride loop.  16 waves (4 per SIMD, 128
// registers each) hold up to 12 packed vectors of x and y per lane; wider rows with a residual
// branch use 8 waves and up to 256 registers.
template <int VPT, bool RESID>
constexpr int adaln_waves() { return RESID && VPT > 12 ? 8 : 16; }

template <int VPT, bool RESID, bool NORM>
__global__ void __launch_bounds__((64 * adaln_waves<VPT, RESID>())) adaln_kernel(BlockArgs a) {
  constexpr int kAdalnWaves = adaln_waves<VPT, RESID>();
  extern __shared__ __attribute__((aligned(16))) float vec[];   // [gate][shift][1 + scale], hidden each
  const int hidden = a.hidden;
  float* gate_s = vec;
  float* shift_s = vec + (RESID ? hidden : 0);
  float* opsc_s = shift_s + hidden;
  for (int c = threadIdx.x; c < hidden; c += 64 * kAdalnWaves) {
    if (RESID) gate_s[c] = a.gate[c];
    if (NORM) {
      shift_s[c] = a.shift[c];
      opsc_s[c] = 1.0f + a.scale[c];
    }
  }
  __syncthreads();
  const int nvec = hidden >> 3;
  const float n = (float)hidden;
  // the row index is wave-uniform: keep it (and the row base addresses) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  for (long long row = (long long)blockIdx.x * kAdalnWaves + wave; row < a.tokens;
       row += (long long)gridDim.x * kAdalnWaves) {
    const size_t base = (size_t)row * hidden;
    int lane = threadIdx.x & 63;
    __asm__ volatile("" : "+v"(lane));
    // VPT = ceil(nvec / 64): only the last vector of a lane can fall past the row.  Lanes past it
    // load and compute the row's last vector (in bounds) and neither store nor count it.
    bool tail_ok = lane + 64 * (VPT - 1) < nvec;
    int tail_v = tail_ok ? lane + 64 * (VPT - 1) : nvec - 1;
    // The row stays packed (bf16) in registers and float32 values are rebuilt in each pass, which
    // keeps enough waves resident to have every wave's whole row in flight.
    u32x4 xv[VPT], yv[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = i < VPT - 1 ? lane + 64 * i : tail_v;
      xv[i] = load_stream(a.x + base + 8 * v);
      if (RESID) yv[i] = load_stream(a.y + base + 8 * v);
    }
    lane = pass_fence<VPT, RESID>(xv, yv);
    tail_ok = lane + 64 * (VPT - 1) < nvec;
    tail_v = tail_ok ? lane + 64 * (VPT - 1) : nvec - 1;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = i < VPT - 1 ? lane + 64 * i : tail_v;
      const bool ok = i < VPT - 1 || tail_ok;
      __asm__ volatile("" ::: "memory");   // LDS reads one vector at a time
      float r[8];
      resid8<RESID>(xv[i], yv[i], gate_s + 8 * v, r);
      if (RESID && ok) store_stream(a.x_out + base + 8 * v, pack8(r));
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) t += r[e];
      s += ok ? t : 0.f;
      __asm__ volatile("" : "+v"(s));   // finish this vector's sum before the next vector's values exist
    }
    if (!NORM) continue;
    const float mean = wave_sum(s) / n;   // correctly rounded: a constant row has mean exactly
    lane = pass_fence<VPT, RESID>(xv, yv);
    tail_ok = lane + 64 * (VPT - 1) < nvec;
    tail_v = tail_ok ? lane + 64 * (VPT - 1) : nvec - 1;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = i < VPT - 1 ? lane + 64 * i : tail_v;
      const bool ok = i < VPT - 1 || tail_ok;
      __asm__ volatile("" ::: "memory");
      float r[8];
      resid8<RESID>(xv[i], yv[i], gate_s + 8 * v, r);
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = r[e] - mean;
        t = __builtin_fmaf(d, d, t);
      }
      q += ok ? t : 0.f;
      __asm__ volatile("" : "+v"(q));
    }
    const float rstd = 1.0f / __builtin_sqrtf(wave_sum(q) / n + a.eps);
    lane = pass_fence<VPT, RESID>(xv, yv);
    tail_ok = lane + 64 * (VPT - 1) < nvec;
    tail_v = tail_ok ? lane + 64 * (VPT - 1) : nvec - 1;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int v = i < VPT - 1 ? lane + 64 * i : tail_v;
      const bool ok = i < VPT - 1 || tail_ok;
      __asm__ volatile("" ::: "memory");
      float r[8], sh[8], sc[8], h[8];
      resid8<RESID>(xv[i], yv[i], gate_s + 8 * v, r);
      load8f(shift_s + 8 * v, sh);
      load8f(opsc_s + 8 * v, sc);
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = __builtin_fmaf((r[e] - mean) * rstd, sc[e], sh[e]);
      if (ok) store_stream(a.h + base + 8 * v, pack8(h));
    }
  }
}

template <int U>
__global__ void __launch_bounds__(256) swiglu_kernel(SwigluArgs a) {
  const int nvec = a.ffn >> 3;
  const long long total = a.tokens * a.chunks;
  for (long long w = blockIdx.x; w < total; w += gridDim.x) {
    const long long row = w / a.chunks;
    const int v0 = (int)(w - row * a.chunks) * (256 * U) + (int)threadIdx.x;
    const uint16_t* g = a.gu + (size_t)row * 2 * a.ffn;
    const uint16_t* u = g + a.ffn;
    uint16_t* o = a.out + (size_t)row * a.ffn;
    u32x4 gv[U], uv[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int v = v0 + 256 * i;
      if (v < nvec) {
        gv[i] = load_stream(g + 8 * v);
        uv[i] = load_stream(u + 8 * v);
      }
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int v = v0 + 256 * i;
      if (v < nvec) {
        float gf[8], uf[8], of[8];
        unpack8(gv[i], gf);
        unpack8(uv[i], uf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // silu(z) = z / (1 + e^-z); e^-z overflows to +inf for z < -88 and the quotient is -0
          const float den = 1.0f + __expf(-gf[e]);
          of[e] = __fdividef(gf[e], den) * uf[e];
        }
        store_stream(o + 8 * v, pack8(of));
      }
    }
  }
}

template <int VPT>
hipError_t launch_adaln_vpt(const BlockArgs& a, bool resid, bool norm, hipStream_t s) {
  const size_t lds = (size_t)((resid ? 1 : 0) + (norm ? 2 : 0)) * a.hidden * sizeof(float);
  const void* fn = resid && norm ? (const void*)adaln_kernel<VPT, true, true>
                   : resid      ? (const void*)adaln_kernel<VPT, true, false>
                                : (const void*)adaln_kernel<VPT, false, true>;
  const int waves = resid ? adaln_waves<VPT, true>() : adaln_waves<VPT, false>();
  const dim3 block(64 * waves);
  hipError_t e;
  if (lds > 64 * 1024) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  // as many persistent workgroups as are resident at once, at most one per 'waves' rows
  int per_cu = 1;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, (int)block.x, lds);
  if (e != hipSuccess) return e;
  int dev = 0, cus = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const long long resident = (long long)cus * (per_cu > 0 ? per_cu : 1);
  const long long need = (a.tokens + waves - 1) / waves;
  const dim3 grid((unsigned)(need < resident ? need : resident));
  if (resid && norm)
    hipLaunchKernelGGL((adaln_kernel<VPT, true, true>), grid, block, lds, s, a);
  else if (resid)
    hipLaunchKernelGGL((adaln_kernel<VPT, true, false>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((adaln_kernel<VPT, false, true>), grid, block, lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_adaln(const BlockArgs& a, bool resid, bool norm, hipStream_t s) {
  const int vpt = ((a.hidden >> 3) + 63) / 64;
  switch (vpt) {
    case 1: return launch_adaln_vpt<1>(a, resid, norm, s);
    case 2: return launch_adaln_vpt<2>(a, resid, norm, s);
    case 3: return launch_adaln_vpt<3>(a, resid, norm, s);
    case 4: return launch_adaln_vpt<4>(a, resid, norm, s);
    case 5: return launch_adaln_vpt<5>(a, resid, norm, s);
    case 6: return launch_adaln_vpt<6>(a, resid, norm, s);
    case 7: return launch_adaln_vpt<7>(a, resid, norm, s);
    case 8: return launch_adaln_vpt<8>(a, resid, norm, s);
    case 9: return launch_adaln_vpt<9>(a, resid, norm, s);
    case 10: return launch_adaln_vpt<10>(a, resid, norm, s);
    case 11: return launch_adaln_vpt<11>(a, resid, norm, s);
    case 12: return launch_adaln_vpt<12>(a, resid, norm, s);
    case 13: return launch_adaln_vpt<13>(a, resid, norm, s);
    case 14: return launch_adaln_vpt<14>(a, resid, norm, s);
    case 15: return launch_adaln_vpt<15>(a, resid, norm, s);
    case 16: return launch_adaln_vpt<16>(a, resid, norm, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_swiglu(SwigluArgs a, hipStream_t s) {
  const int nvec = a.ffn >> 3;
  const int u = (nvec + 255) / 256 < 8 ? (nvec + 255) / 256 : 8;
  a.chunks = (nvec + 256 * u - 1) / (256 * u);
  const long long wgs = a.tokens * a.chunks;
  const dim3 grid((unsigned)(wgs < (1 << 20) ? wgs : (1 << 20)));
  switch (u) {
    case 1: hipLaunchKernelGGL(swiglu_kernel<1>, grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(swiglu_kernel<2>, grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL(swiglu_kernel<3>, grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(swiglu_kernel<4>, grid, dim3(256), 0, s, a); break;
    case 5: hipLaunchKernelGGL(swiglu_kernel<5>, grid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL(swiglu_kernel<6>, grid, dim3(256), 0, s, a); break;
    case 7: hipLaunchKernelGGL(swiglu_kernel<7>, grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(swiglu_kernel<8>, grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace dit
