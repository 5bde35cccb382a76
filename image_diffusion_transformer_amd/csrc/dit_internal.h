// Internal interface between the host API (api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

constexpr int kHeadDim = 96;     // 5376 hidden / 56 heads; head dim 128 is the other instantiation
constexpr int kBlock = 128;      // router block and KV tile: 128 consecutive tokens

// RoPE channels of axis a (0 = t, 1 = h, 2 = w): three chunks of 32 at head dim 96; 44, 42, 42 at 128
// (the nearest-equal split into even widths).  Pair i of axis a rotates by pos * theta^(-2i/width).
constexpr int rope_width(int d, int axis) { return d == 96 ? 32 : (axis == 0 ? 44 : 42); }
// Floats per RoPE table row: cos of the axis's pairs, then (from half the row) their sin.
constexpr int rope_row_floats(int d) { return d == 96 ? 32 : 44; }
// Fragments of one (head, 128-key tile) image: 4 d/16 K^ plus 8 d/32 V^T fragments of 1 KB.
constexpr int tile_frags(int d) { return 4 * (d / 16) + 8 * (d / 32); }

// Exact unsigned division of n < 2^31 by a runtime divisor d >= 1:
// q = (n * m) >> s with s = 32 + ceil(log2 d), m = ceil(2^s / d) (fits in 33 bits).
struct FastDiv {
  uint64_t m;
  uint32_t s;
  uint32_t d;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  FastDiv f;
  f.s = 32 + l;
  f.m = (((unsigned __int128)1 << f.s) + d - 1) / d;
  f.d = d;
  return f;
}

struct GridDesc {
  int N, T, H, W, heads;
  FastDiv div_w, div_hw;
};

struct AttnArgs {
  const uint16_t* q;      // bf16 bits [N][heads][96]
  const uint16_t* k;
  const uint16_t* v;
  const float* wq;        // [96]
  const float* wk;
  const float* rope;      // [(T+H+W)][32]: row t, then T+h, then T+H+w; cos[16], sin[16]
  uint16_t* kvf;          // [heads][nb][48][512] bf16: K^ / V^T MFMA fragment image per 128-key tile
  uint16_t* o;
  GridDesc g;             // token grid (grid calls); heads is used by every call
  int nq, nk;             // query and key token counts (both N for grid calls)
  const int* q_pos;       // null for grid calls; else int32 [nq][3] (t, h, w) explicit positions
  const int* k_pos;       // null for grid calls; else int32 [nk][3]
  int max_pos;            // explicit positions: rows per axis section of the RoPE table (coordinates clamped)
  int rope_sec[3];        // explicit positions: first table row of each axis's section
  int head_dim;           // 96 or 128
  float qscale;           // log2(e) / sqrt(96): softmax runs in base 2
  float eps;
  int nqt;                // query tiles per head
  int total;              // heads * nqt
  int per_xcd;            // ceil(total / 8)
  int order;              // workgroup order: 0 = the tuned one, 1 = reversed (results must not change)
  // Dense tail split (see TailPlan): the attention kernel takes the first main_per_xcd query tiles of each
  // XCD's run; the last tail_rem of each run are split along the keys into tail_pieces pieces whose
  // unnormalised fp32 partials (`partial`) a merge kernel sums.  tail_pieces == 1: no split.
  int main_per_xcd;
  int tail_rem;
  int tail_pieces;
  float* partial;         // [8 * tail_rem * tail_pieces] x tail_partial_bytes(head_dim)
  // block-sparse iteration lists (null for dense)
  const int* list;        // [heads][nqt][nb]: visited KV tiles, ascending (plain tile indices < nb)
  const unsigned char* list_flags;  // [heads][nqt][nb]: bit s = slot s of the query tile keeps that KV tile
  const int* list_len;    // [heads][nqt]
  const int* perm;        // [heads][nqt][BQ/128]: router block in each slot of a query tile, -1 = none
  int nb;                 // 128-key tiles: ceil(nk / 128)
};

struct RouteArgs {
  const uint16_t* q;
  const uint16_t* k;
  const float* wq;
  const float* wk;
  const float* rope;
  GridDesc g;
  float eps;
  int nb;
  int keep;
  float* pooled;          // [2][heads][nb][d] block means of q (0) and k (1)
  uint32_t* scores;       // [heads][nb][nb] order keys of the block scores (nb <= route_topk_max_blocks())
  unsigned char* mask;    // [heads][nb][nb]
  int head_dim;           // 96 or 128
};

struct ScheduleArgs {
  const unsigned char* mask;   // [heads][nb][nb]
  unsigned long long* bits;    // [heads][nb][words] packed mask rows
  int* perm;                   // [heads][nqt][group] router block of each query-tile slot, -1 = none
  int* list;                   // [heads][nqt][nb] visited KV tiles
  unsigned char* list_flags;   // [heads][nqt][nb] slots of the query tile that keep each visited tile
  int* list_len;               // [heads][nqt]
  int heads, nb, nqt, group;   // group = router blocks per query tile (<= 8)
  int words;                   // schedule_words(nb)
};

// Operators around attention: AdaLN update and gated residual (one wave per token row).
struct BlockArgs {
  const uint16_t* x;      // bf16 [tokens][hidden]
  const uint16_t* y;      // bf16 [tokens][hidden] branch output (gated residual)
  const float* gate;      // [hidden]
  const float* shift;     // [hidden]
  const float* scale;     // [hidden]
  uint16_t* x_out;        // bf16 [tokens][hidden] residual sum (may equal x)
  uint16_t* h;            // bf16 [tokens][hidden] AdaLN update
  long long tokens;
  int hidden;             // multiple of 8, <= 8192
  float eps;
};

struct SwigluArgs {
  const uint16_t* gu;     // bf16 [tokens][2 ffn]: gate then up projection
  uint16_t* out;          // bf16 [tokens][ffn]
  long long tokens;
  int ffn;                // multiple of 8
  int chunks;             // workgroups per token row (set by launch_swiglu)
};

// Bytes of one (head, 128-key tile) fragment image: fragments of 64 lanes x 16 bytes.
constexpr size_t tile_image_bytes(int d) { return (size_t)tile_frags(d) * 1024; }

// Query tile of the attention kernel (tokens per workgroup) at head dim d -- a multiple of kBlock.
int attn_query_tile(int head_dim);

// Dense calls: how the query tiles of the last, partly filled round of workgroups are split.  The tiles run
// as 8 XCD runs of per_xcd (the launch index mod 8 picks the XCD); each XCD has 32 CUs and one workgroup
// fits a CU, so a run takes per_xcd / 32 rounds and a last round of rem tiles that leaves 32 - rem CUs idle.
// When that idle time is worth it, each of those rem tiles is split along the keys into `pieces` parts.
struct TailPlan {
  int per_xcd, main_per_xcd, rem, pieces;
};
TailPlan tail_plan(int total, int nk);
// Bytes of one piece's partial result at head dim d.
size_t tail_partial_bytes(int head_dim);
inline size_t tail_partial_area(const TailPlan& p, int head_dim) {
  return p.pieces > 1 ? (size_t)8 * p.rem * p.pieces * tail_partial_bytes(head_dim) : 0;
}

hipError_t launch_attn_dense(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_sparse(const AttnArgs& a, hipStream_t s);
// Packs the mask, groups router blocks into query tiles and writes the iteration lists (three kernels).
hipError_t launch_sparse_schedule(const ScheduleArgs& a, hipStream_t s);
// 64-bit words of a packed mask row.
int schedule_words(int nb);
hipError_t launch_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_adaln(const BlockArgs& a, bool resid, bool norm, hipStream_t s);
hipError_t launch_swiglu(SwigluArgs a, hipStream_t s);

// Largest block count whose score rows the top-k kernel holds in registers; above it the router
// scores and selects in one workgroup per row and needs no score matrix.
constexpr int route_topk_max_blocks() { return 4096; }

}  // namespace dit
