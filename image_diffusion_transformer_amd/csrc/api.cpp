// Host side of the C ABI declared in include/dit_attn.h and include/dit_block.h: argument
// validation, workspace layout, host RoPE tables and kernel launches.  Nothing here computes
// attention or the block operators; every arithmetic step runs in the gfx950 kernels.
#include "dit_attn.h"
#include "dit_block.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <new>
#include <tuple>
#include <vector>

#include "dit_internal.h"

namespace {

// Text of the calling thread's last error.  A fixed buffer: setting it allocates nothing and cannot throw.
thread_local char g_err[512];

dit_status fail(dit_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = '\0'; }

// Runs an entry point's body and turns any C++ exception (host allocation failure in the RoPE table cache
// being the only one the bodies can raise) into a status: nothing is thrown across the C ABI.
template <class F>
dit_status guarded(F&& body) noexcept {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return fail(DIT_ERR_HOST, "host memory exhausted");
  } catch (...) {
    return fail(DIT_ERR_HOST, "unexpected host-side exception");
  }
}

dit_status fail_hip(hipError_t e, const char* what) {
  return fail(DIT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Shape {
  int T, H, W, heads;
  int d;             // head dim: 96 or 128
  long long N;
  int nb;
  int nqt;
};

bool head_dim_ok(int d) { return d == 96 || d == 128; }

// Several kernels index heads with a launch grid dimension other than x, which holds at most 65535.
constexpr int kMaxHeads = 65535;

struct Layout {
  size_t tab;        // RoPE table [(T+H+W)][rope_row_floats(d)] f32
  size_t kvf;        // K^ / V^T fragment images [heads][nb] x tile_image_bytes(d) (dense and block-sparse)
  size_t route_pool; // [2][heads][nb][d] f32
  size_t route_score;// [heads][nb][nb] u32 order keys (nb <= dit::route_topk_max_blocks(), else unused)
  size_t list;       // [heads][nqt][nb] i32 visited KV tiles
  size_t list_flags; // [heads][nqt][nb] u8 slots that keep each visited tile
  size_t list_len;   // [heads][nqt] i32
  size_t perm;       // [heads][nqt][query tile / 128] i32 router block per query-tile slot
  size_t bits;       // [heads][nb][schedule_words(nb)] u64 packed mask rows
  size_t partial;    // dense tail pieces: fp32 partial results (dit::tail_partial_area)
  size_t total;
};

Layout make_layout(const Shape& s) {
  Layout L{};
  L.tab = 0;
  L.kvf = align256((size_t)(s.T + s.H + s.W) * dit::rope_row_floats(s.d) * sizeof(float));
  const size_t base = L.kvf + (size_t)s.heads * s.nb * dit::tile_image_bytes(s.d);
  const size_t pool_bytes = align256(2ull * s.heads * s.nb * s.d * sizeof(float));
  const size_t score_bytes =
      s.nb <= dit::route_topk_max_blocks() ? align256((size_t)s.heads * s.nb * s.nb * sizeof(uint32_t)) : 0;
  L.route_pool = base;
  L.route_score = base + pool_bytes;
  const size_t list_bytes = align256((size_t)s.heads * s.nqt * s.nb * sizeof(int));
  const size_t flag_bytes = align256((size_t)s.heads * s.nqt * s.nb);
  const size_t len_bytes = align256((size_t)s.heads * s.nqt * sizeof(int));
  const int group = dit::attn_query_tile(s.d) / dit::kBlock;
  const size_t perm_bytes = align256((size_t)s.heads * s.nqt * group * sizeof(int));
  const size_t bits_bytes = align256((size_t)s.heads * s.nb * dit::schedule_words(s.nb) * sizeof(uint64_t));
  L.list = base;
  L.list_flags = L.list + list_bytes;
  L.list_len = L.list_flags + flag_bytes;
  L.perm = L.list_len + len_bytes;
  L.bits = L.perm + perm_bytes;
  // Dense calls use neither the router's nor the block-sparse schedule's share: their tail partials
  // (if the call splits its last round) share that space.
  L.partial = base;
  const size_t partial_bytes = dit::tail_partial_area(dit::tail_plan(s.heads * s.nqt, (int)s.N), s.d);
  L.total = base + std::max({pool_bytes + score_bytes, list_bytes + flag_bytes + len_bytes + perm_bytes + bits_bytes,
                             partial_bytes});
  return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks shared by every entry point; fills `s`.
dit_status check_shape(int T, int H, int W, int heads, int head_dim, Shape& s) {
  if (T < 1 || H < 1 || W < 1 || heads < 1)
    return fail(DIT_ERR_INVALID_ARG, "grid and heads must be >= 1 (T=%d H=%d W=%d heads=%d)", T, H, W, heads);
  if (!head_dim_ok(head_dim))
    return fail(DIT_ERR_UNSUPPORTED, "head_dim %d is not supported (96 or 128)", head_dim);
  if (heads > kMaxHeads) return fail(DIT_ERR_UNSUPPORTED, "heads %d exceeds %d", heads, kMaxHeads);
  const long long N = (long long)T * H * W;
  if (N * heads * head_dim > 2147483647ll)
    return fail(DIT_ERR_UNSUPPORTED, "N*heads*head_dim = %lld exceeds 2^31-1 elements", N * heads * head_dim);
  const long long nb = (N + dit::kBlock - 1) / dit::kBlock;
  if (nb > 32768) return fail(DIT_ERR_UNSUPPORTED, "%lld blocks exceed the router limit of 32768", nb);
  if ((long long)T + H + W > (1 << 24)) return fail(DIT_ERR_UNSUPPORTED, "grid axes too long");
  s.T = T;
  s.H = H;
  s.W = W;
  s.heads = heads;
  s.d = head_dim;
  s.N = N;
  s.nb = (int)nb;
  const int bq = dit::attn_query_tile(head_dim);
  s.nqt = (int)((N + bq - 1) / bq);
  return DIT_OK;
}

dit_status check_common(const void* q, const void* k, const float* wq, const float* wk, float theta, float eps) {
  if (!q || !k || !wq || !wk) return fail(DIT_ERR_INVALID_ARG, "null q, k, wq or wk");
  if (!aligned16(q) || !aligned16(k) || !aligned16(wq) || !aligned16(wk))
    return fail(DIT_ERR_INVALID_ARG, "q, k, wq and wk must be 16-byte aligned");
  if (!std::isfinite(theta) || theta <= 0.f) return fail(DIT_ERR_INVALID_ARG, "rope_theta must be finite and > 0");
  if (!std::isfinite(eps) || eps < 0.f) return fail(DIT_ERR_INVALID_ARG, "eps must be finite and >= 0");
  return DIT_OK;
}

dit_status check_workspace(const Shape& s, void* ws, size_t ws_bytes, Layout& L) {
  L = make_layout(s);
  if (!ws) return fail(DIT_ERR_WORKSPACE, "workspace is null (need %zu bytes)", L.total);
  if (ws_bytes < L.total) return fail(DIT_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, L.total);
  if (((uintptr_t)ws & 255u) != 0) return fail(DIT_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return DIT_OK;
}

// cos / sin of pos * theta^(-2i/w_a) for the pairs i of axis a (w_a its channel width), angle in
// double, C library cos/sin, rounded once to float.  Rows: n0 rows of axis 0 (t), then n1 of axis 1 (h),
// then n2 of axis 2 (w); each row holds the axis's cos values from float 0 and its sin values from
// float rope_row_floats(d) / 2.
//
// Tables are cached per (rows, theta, head dim), at most kMaxTables of them; a new one evicts the least
// recently used.  Callers hold a shared reference, so an eviction by another thread never frees a table
// that is being uploaded.  Allocation failure throws std::bad_alloc, which the entry points' guard turns
// into DIT_ERR_HOST.
typedef std::tuple<int, int, int, uint32_t, int> TabKey;
struct TabEntry {
  std::shared_ptr<const std::vector<float>> tab;
  unsigned long long used;
};
constexpr size_t kMaxTables = 16;
std::mutex g_tab_mu;
std::map<TabKey, TabEntry> g_tabs;
unsigned long long g_tab_clock = 0;

std::shared_ptr<const std::vector<float>> rope_table(int n0, int n1, int n2, float theta, int d) {
  uint32_t tb;
  std::memcpy(&tb, &theta, 4);
  const TabKey key = std::make_tuple(n0, n1, n2, tb, d);
  {
    std::lock_guard<std::mutex> lk(g_tab_mu);
    auto it = g_tabs.find(key);
    if (it != g_tabs.end()) {
      it->second.used = ++g_tab_clock;
      return it->second.tab;
    }
  }
  const int rs = dit::rope_row_floats(d);
  auto tab = std::make_shared<std::vector<float>>((size_t)(n0 + n1 + n2) * rs, 0.0f);
  const int npos[3] = {n0, n1, n2};
  int row = 0;
  for (int a = 0; a < 3; ++a) {
    const int width = dit::rope_width(d, a);
    for (int p = 0; p < npos[a]; ++p, ++row) {
      for (int i = 0; i < width / 2; ++i) {
        const double inv = std::pow((double)theta, -2.0 * i / (double)width);
        const double ang = (double)p * inv;
        (*tab)[(size_t)row * rs + i] = (float)std::cos(ang);
        (*tab)[(size_t)row * rs + rs / 2 + i] = (float)std::sin(ang);
      }
    }
  }
  std::lock_guard<std::mutex> lk(g_tab_mu);
  while (g_tabs.size() >= kMaxTables) {
    auto lru = g_tabs.begin();
    for (auto it = g_tabs.begin(); it != g_tabs.end(); ++it)
      if (it->second.used < lru->second.used) lru = it;
    g_tabs.erase(lru);
  }
  TabEntry& e = g_tabs[key];   // another thread may have built the same table meanwhile: same contents
  e.tab = tab;
  e.used = ++g_tab_clock;
  return tab;
}

// Host -> device copy of a table.  The source is pageable host memory, which the runtime has finished
// reading when the call returns, so the table may be evicted from the cache right after.
dit_status upload(const std::vector<float>& tab, void* dst, hipStream_t st) {
  hipError_t e = hipMemcpyAsync(dst, tab.data(), tab.size() * sizeof(float), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(rope table)");
  return DIT_OK;
}

dit_status upload_table(const Shape& s, float theta, void* ws, const Layout& L, hipStream_t st) {
  const auto tab = rope_table(s.T, s.H, s.W, theta, s.d);
  return upload(*tab, (char*)ws + L.tab, st);
}

// [p, p + bytes) and [q, q + bytes2) share a byte.
bool overlaps(const void* p, size_t bytes, const void* q, size_t bytes2) {
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + bytes2 && b < a + bytes;
}

// A buffer of a call: where it starts, its size in bytes, its name, and whether the call writes it.
struct Buf {
  const void* p;
  size_t bytes;
  const char* name;
  bool written;
};

// Every buffer the call writes (outputs and workspace) must be disjoint from every other buffer of the
// call; read-only inputs may share memory with each other.
template <size_t K>
dit_status check_disjoint(const Buf (&b)[K]) {
  for (size_t i = 0; i < K; ++i)
    for (size_t j = i + 1; j < K; ++j)
      if ((b[i].written || b[j].written) && b[i].p && b[j].p && overlaps(b[i].p, b[i].bytes, b[j].p, b[j].bytes))
        return fail(DIT_ERR_INVALID_ARG, "%s overlaps %s", b[i].name, b[j].name);
  return DIT_OK;
}

// Workgroup order of the attention calls (diagnostic; see dit_attn_set_launch_order).
std::atomic<int> g_launch_order{0};

dit::GridDesc grid_desc(const Shape& s) {
  dit::GridDesc g;
  g.N = (int)s.N;
  g.T = s.T;
  g.H = s.H;
  g.W = s.W;
  g.heads = s.heads;
  g.div_w = dit::make_fastdiv((uint32_t)s.W);
  g.div_hw = dit::make_fastdiv((uint32_t)s.H * (uint32_t)s.W);
  return g;
}

dit::AttnArgs attn_args(const Shape& s, const void* q, const void* k, const void* v, const float* wq, const float* wk,
                        float eps, void* o, void* ws, const Layout& L) {
  dit::AttnArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.wq = wq;
  a.wk = wk;
  a.rope = (const float*)((const char*)ws + L.tab);
  a.kvf = (uint16_t*)((char*)ws + L.kvf);
  a.o = (uint16_t*)o;
  a.g = grid_desc(s);
  a.nq = (int)s.N;
  a.nk = (int)s.N;
  a.q_pos = nullptr;
  a.k_pos = nullptr;
  a.max_pos = 0;
  a.head_dim = s.d;
  a.qscale = (float)(1.4426950408889634 / std::sqrt((double)s.d));
  a.eps = eps;
  a.nqt = s.nqt;
  a.total = s.heads * s.nqt;
  const dit::TailPlan tp = dit::tail_plan(a.total, a.nk);
  a.per_xcd = tp.per_xcd;
  a.main_per_xcd = tp.main_per_xcd;
  a.tail_rem = tp.rem;
  a.tail_pieces = tp.pieces;
  a.partial = (float*)((char*)ws + L.partial);
  a.order = g_launch_order.load(std::memory_order_relaxed);
  a.nb = s.nb;
  return a;
}

int keep_count(int nb, float sparsity) {
  const double k = (double)nb - std::floor((double)sparsity * nb + 1e-9);
  return (int)std::max(1.0, std::min((double)nb, k));
}

// Joint attention: queries and keys are separate token sets with explicit positions.
constexpr int kMaxPos = 1 << 20;

struct JointShape {
  int nq, nk, heads, d, nb, nqt, max_pos;
  int sections;   // RoPE table sections of max_pos rows: 1 (the axes share one; d = 96) or 3 (d = 128)
};

struct JointLayout {
  size_t tab;       // RoPE table [sections * max_pos][rope_row_floats(d)] f32
  size_t kvf;       // K^ / V^T fragment images [heads][nb] x tile_image_bytes(d)
  size_t partial;   // tail partial results (dit::tail_partial_area)
  size_t total;
};

JointLayout make_joint_layout(const JointShape& j) {
  JointLayout L{};
  L.tab = 0;
  L.kvf = align256((size_t)j.sections * j.max_pos * dit::rope_row_floats(j.d) * sizeof(float));
  L.partial = align256(L.kvf + (size_t)j.heads * j.nb * dit::tile_image_bytes(j.d));
  L.total = L.partial + dit::tail_partial_area(dit::tail_plan(j.heads * j.nqt, j.nk), j.d);
  return L;
}

dit_status check_joint_shape(int nq, int nk, int heads, int head_dim, int max_pos, JointShape& j) {
  if (nq < 1 || nk < 1 || heads < 1)
    return fail(DIT_ERR_INVALID_ARG, "token counts and heads must be >= 1 (nq=%d nk=%d heads=%d)", nq, nk, heads);
  if (!head_dim_ok(head_dim))
    return fail(DIT_ERR_UNSUPPORTED, "head_dim %d is not supported (96 or 128)", head_dim);
  if (heads > kMaxHeads) return fail(DIT_ERR_UNSUPPORTED, "heads %d exceeds %d", heads, kMaxHeads);
  if (max_pos < 1) return fail(DIT_ERR_INVALID_ARG, "max_pos must be >= 1 (got %d)", max_pos);
  if (max_pos > kMaxPos) return fail(DIT_ERR_UNSUPPORTED, "max_pos %d exceeds %d", max_pos, kMaxPos);
  const long long big = std::max(nq, nk);
  if (big * heads * head_dim > 2147483647ll)
    return fail(DIT_ERR_UNSUPPORTED, "tokens*heads*head_dim = %lld exceeds 2^31-1 elements",
                big * heads * head_dim);
  j.nq = nq;
  j.nk = nk;
  j.heads = heads;
  j.d = head_dim;
  j.sections = head_dim == 96 ? 1 : 3;
  j.nb = (nk + dit::kBlock - 1) / dit::kBlock;
  const int bq = dit::attn_query_tile(head_dim);
  j.nqt = (nq + bq - 1) / bq;
  j.max_pos = max_pos;
  return DIT_OK;
}

}  // namespace

extern "C" {

size_t dit_attn_workspace_bytes(int T, int H, int W, int heads, int head_dim, int block, float sparsity) {
  // Computes a size only: the caller's last error is left as it was.
  char saved[sizeof(g_err)];
  std::memcpy(saved, g_err, sizeof(g_err));
  Shape s;
  const dit_status st = check_shape(T, H, W, heads, head_dim, s);
  std::memcpy(g_err, saved, sizeof(g_err));
  if (st != DIT_OK || block != dit::kBlock) return 0;
  if (!std::isfinite(sparsity) || sparsity < 0.f || sparsity >= 1.f) return 0;
  // The block-sparse lists are sized for any mask (block_sparse accepts masks from any source), so the
  // size does not depend on the sparsity.
  return make_layout(s).total;
}

dit_status dit_attn_set_launch_order(int order) {
  clear_error();
  if (order != 0 && order != 1) return fail(DIT_ERR_INVALID_ARG, "launch order must be 0 or 1 (got %d)", order);
  g_launch_order.store(order, std::memory_order_relaxed);
  return DIT_OK;
}

int dit_attn_keep_count(int nb, float sparsity) {
  if (nb < 1 || !std::isfinite(sparsity) || sparsity < 0.f || sparsity >= 1.f) return -1;
  return keep_count(nb, sparsity);
}

dit_status dit_attn_dense(const void* q, const void* k, const void* v, const float* wq, const float* wk, int T, int H,
                          int W, int heads, int head_dim, float rope_theta, float eps, void* o, void* workspace,
                          size_t workspace_bytes, void* hip_stream) {
  clear_error();
  return guarded([&]() -> dit_status {
    Shape s;
    dit_status st = check_shape(T, H, W, heads, head_dim, s);
    if (st != DIT_OK) return st;
    if ((st = check_common(q, k, wq, wk, rope_theta, eps)) != DIT_OK) return st;
    if (!v || !o) return fail(DIT_ERR_INVALID_ARG, "null v or o");
    if (!aligned16(v) || !aligned16(o)) return fail(DIT_ERR_INVALID_ARG, "v and o must be 16-byte aligned");
    Layout L;
    if ((st = check_workspace(s, workspace, workspace_bytes, L)) != DIT_OK) return st;
    const size_t tb = (size_t)s.N * s.heads * s.d * 2, wb = (size_t)s.d * 4;
    const Buf bufs[] = {{q, tb, "q", false},  {k, tb, "k", false},   {v, tb, "v", false},
                        {wq, wb, "wq", false}, {wk, wb, "wk", false}, {o, tb, "o", true},
                        {workspace, L.total, "workspace", true}};
    if ((st = check_disjoint(bufs)) != DIT_OK) return st;
    hipStream_t stream = (hipStream_t)hip_stream;
    if ((st = upload_table(s, rope_theta, workspace, L, stream)) != DIT_OK) return st;
    const dit::AttnArgs a = attn_args(s, q, k, v, wq, wk, eps, o, workspace, L);
    const hipError_t e = dit::launch_attn_dense(a, stream);
    if (e != hipSuccess) return fail_hip(e, "attention kernel launch");
    return DIT_OK;
  });
}

dit_status dit_attn_route(const void* q, const void* k, const float* wq, const float* wk, int T, int H, int W,
                          int heads, int head_dim, float rope_theta, float eps, float sparsity, int block,
                          unsigned char* mask, void* workspace, size_t workspace_bytes, void* hip_stream) {
  clear_error();
  return guarded([&]() -> dit_status {
    Shape s;
    dit_status st = check_shape(T, H, W, heads, head_dim, s);
    if (st != DIT_OK) return st;
    if (block != dit::kBlock) return fail(DIT_ERR_UNSUPPORTED, "block %d is not supported (only 128)", block);
    if ((st = check_common(q, k, wq, wk, rope_theta, eps)) != DIT_OK) return st;
    if (!std::isfinite(sparsity) || sparsity < 0.f || sparsity >= 1.f)
      return fail(DIT_ERR_INVALID_ARG, "sparsity must be in [0, 1)");
    if (!mask) return fail(DIT_ERR_INVALID_ARG, "null mask");
    Layout L;
    if ((st = check_workspace(s, workspace, workspace_bytes, L)) != DIT_OK) return st;
    const size_t tb = (size_t)s.N * s.heads * s.d * 2, wb = (size_t)s.d * 4;
    const Buf bufs[] = {{q, tb, "q", false},   {k, tb, "k", false},
                        {wq, wb, "wq", false},  {wk, wb, "wk", false},
                        {mask, (size_t)s.heads * s.nb * s.nb, "mask", true},
                        {workspace, L.total, "workspace", true}};
    if ((st = check_disjoint(bufs)) != DIT_OK) return st;
    hipStream_t stream = (hipStream_t)hip_stream;
    if ((st = upload_table(s, rope_theta, workspace, L, stream)) != DIT_OK) return st;
    dit::RouteArgs a{};
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.wq = wq;
    a.wk = wk;
    a.rope = (const float*)((const char*)workspace + L.tab);
    a.g = grid_desc(s);
    a.eps = eps;
    a.nb = s.nb;
    a.keep = keep_count(s.nb, sparsity);
    a.pooled = (float*)((char*)workspace + L.route_pool);
    a.scores = (uint32_t*)((char*)workspace + L.route_score);
    a.mask = mask;
    a.head_dim = s.d;
    const hipError_t e = dit::launch_route(a, stream);
    if (e != hipSuccess) return fail_hip(e, "router kernel launch");
    return DIT_OK;
  });
}

dit_status dit_attn_block_sparse(const void* q, const void* k, const void* v, const float* wq, const float* wk, int T,
                                 int H, int W, int heads, int head_dim, float rope_theta, float eps, int block,
                                 const unsigned char* mask, void* o, void* workspace, size_t workspace_bytes,
                                 void* hip_stream) {
  clear_error();
  return guarded([&]() -> dit_status {
    Shape s;
    dit_status st = check_shape(T, H, W, heads, head_dim, s);
    if (st != DIT_OK) return st;
    if (block != dit::kBlock) return fail(DIT_ERR_UNSUPPORTED, "block %d is not supported (only 128)", block);
    if ((st = check_common(q, k, wq, wk, rope_theta, eps)) != DIT_OK) return st;
    if (!v || !o || !mask) return fail(DIT_ERR_INVALID_ARG, "null v, o or mask");
    if (!aligned16(v) || !aligned16(o)) return fail(DIT_ERR_INVALID_ARG, "v and o must be 16-byte aligned");
    Layout L;
    if ((st = check_workspace(s, workspace, workspace_bytes, L)) != DIT_OK) return st;
    const size_t tb = (size_t)s.N * s.heads * s.d * 2, wb = (size_t)s.d * 4;
    const Buf bufs[] = {{q, tb, "q", false},   {k, tb, "k", false}, {v, tb, "v", false},
                        {wq, wb, "wq", false},  {wk, wb, "wk", false},
                        {mask, (size_t)s.heads * s.nb * s.nb, "mask", false},
                        {o, tb, "o", true},     {workspace, L.total, "workspace", true}};
    if ((st = check_disjoint(bufs)) != DIT_OK) return st;
    hipStream_t stream = (hipStream_t)hip_stream;
    if ((st = upload_table(s, rope_theta, workspace, L, stream)) != DIT_OK) return st;
    dit::ScheduleArgs c{};
    c.mask = mask;
    c.bits = (unsigned long long*)((char*)workspace + L.bits);
    c.perm = (int*)((char*)workspace + L.perm);
    c.list = (int*)((char*)workspace + L.list);
    c.list_flags = (unsigned char*)((char*)workspace + L.list_flags);
    c.list_len = (int*)((char*)workspace + L.list_len);
    c.heads = s.heads;
    c.nb = s.nb;
    c.nqt = s.nqt;
    c.group = dit::attn_query_tile(s.d) / dit::kBlock;
    c.words = dit::schedule_words(s.nb);
    hipError_t e = dit::launch_sparse_schedule(c, stream);
    if (e != hipSuccess) return fail_hip(e, "block-sparse schedule launch");
    dit::AttnArgs a = attn_args(s, q, k, v, wq, wk, eps, o, workspace, L);
    a.list = c.list;
    a.list_flags = c.list_flags;
    a.list_len = c.list_len;
    a.perm = c.perm;
    e = dit::launch_attn_sparse(a, stream);
    if (e != hipSuccess) return fail_hip(e, "sparse attention kernel launch");
    return DIT_OK;
  });
}

size_t dit_attn_joint_workspace_bytes(int nq, int nk, int heads, int head_dim, int max_pos) {
  char saved[sizeof(g_err)];
  std::memcpy(saved, g_err, sizeof(g_err));
  JointShape j;
  const dit_status st = check_joint_shape(nq, nk, heads, head_dim, max_pos, j);
  std::memcpy(g_err, saved, sizeof(g_err));
  if (st != DIT_OK) return 0;
  return make_joint_layout(j).total;
}

dit_status dit_attn_joint(const void* q, const void* k, const void* v, const float* wq, const float* wk,
                          const int* q_pos, const int* k_pos, int nq, int nk, int heads, int head_dim, int max_pos,
                          float rope_theta, float eps, void* o, void* workspace, size_t workspace_bytes,
                          void* hip_stream) {
  clear_error();
  return guarded([&]() -> dit_status {
    JointShape j;
    dit_status st = check_joint_shape(nq, nk, heads, head_dim, max_pos, j);
    if (st != DIT_OK) return st;
    if ((st = check_common(q, k, wq, wk, rope_theta, eps)) != DIT_OK) return st;
    if (!v || !o || !q_pos || !k_pos) return fail(DIT_ERR_INVALID_ARG, "null v, o, q_pos or k_pos");
    if (!aligned16(v) || !aligned16(o)) return fail(DIT_ERR_INVALID_ARG, "v and o must be 16-byte aligned");
    if (((uintptr_t)q_pos & 3u) || ((uintptr_t)k_pos & 3u))
      return fail(DIT_ERR_INVALID_ARG, "q_pos and k_pos must be 4-byte aligned");
    const JointLayout L = make_joint_layout(j);
    if (!workspace) return fail(DIT_ERR_WORKSPACE, "workspace is null (need %zu bytes)", L.total);
    if (workspace_bytes < L.total)
      return fail(DIT_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", workspace_bytes, L.total);
    if (((uintptr_t)workspace & 255u) != 0) return fail(DIT_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const size_t qb = (size_t)nq * heads * head_dim * 2, kb = (size_t)nk * heads * head_dim * 2;
    const size_t wb = (size_t)head_dim * 4;
    const Buf bufs[] = {{q, qb, "q", false},   {k, kb, "k", false},   {v, kb, "v", false},
                        {wq, wb, "wq", false},  {wk, wb, "wk", false},
                        {q_pos, (size_t)nq * 12, "q_pos", false},
                        {k_pos, (size_t)nk * 12, "k_pos", false},
                        {o, qb, "o", true},     {workspace, L.total, "workspace", true}};
    if ((st = check_disjoint(bufs)) != DIT_OK) return st;
    hipStream_t stream = (hipStream_t)hip_stream;
    // rows p = 0 .. max_pos-1 of each axis section; at head dim 96 the three axes have the same width and
    // share one section
    const auto tab = j.sections == 1 ? rope_table(max_pos, 0, 0, rope_theta, j.d)
                                     : rope_table(max_pos, max_pos, max_pos, rope_theta, j.d);
    if ((st = upload(*tab, (char*)workspace + L.tab, stream)) != DIT_OK) return st;
    dit::AttnArgs a{};
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.wq = wq;
    a.wk = wk;
    a.rope = (const float*)((const char*)workspace + L.tab);
    a.kvf = (uint16_t*)((char*)workspace + L.kvf);
    a.o = (uint16_t*)o;
    a.g = dit::GridDesc{};
    a.g.heads = heads;
    a.nq = nq;
    a.nk = nk;
    a.q_pos = q_pos;
    a.k_pos = k_pos;
    a.max_pos = max_pos;
    for (int i = 0; i < 3; ++i) a.rope_sec[i] = j.sections == 1 ? 0 : i * max_pos;
    a.head_dim = j.d;
    a.qscale = (float)(1.4426950408889634 / std::sqrt((double)j.d));
    a.eps = eps;
    a.nqt = j.nqt;
    a.total = heads * j.nqt;
    const dit::TailPlan tp = dit::tail_plan(a.total, nk);
    a.per_xcd = tp.per_xcd;
    a.main_per_xcd = tp.main_per_xcd;
    a.tail_rem = tp.rem;
    a.tail_pieces = tp.pieces;
    a.partial = (float*)((char*)workspace + L.partial);
    a.order = g_launch_order.load(std::memory_order_relaxed);
    a.nb = j.nb;
    const hipError_t e = dit::launch_attn_dense(a, stream);
    if (e != hipSuccess) return fail_hip(e, "joint attention kernel launch");
    return DIT_OK;
  });
}

}  // extern "C"

// ------------------------------------------------------------------------------------------------
// Allocation-free dense attention (dit_attn_dense_noalloc): the RoPE table and the K^/V fragment images
// live in `scratch`, a static device array of the library, instead of a caller's workspace.

namespace {

constexpr size_t kStaticScratchBytes = DIT_ATTN_NOALLOC_SCRATCH_BYTES;   // 64 MiB per GPU, held until exit
static_assert(kStaticScratchBytes == (64ull << 20), "static scratch size");

// The array's name is a host-side stand-in in host code: only the address hipGetSymbolAddress returns (per
// device) is handed to kernels or copies.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's `scratch`, looked up once per device with that device current.
dit_status static_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(DIT_ERR_UNSUPPORTED, "device %d is beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(DIT_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DIT_OK;
}

}  // namespace

extern "C" {

dit_status dit_attn_dense_noalloc(const void* q, const void* k, const void* v, const float* wq, const float* wk,
                                  int T, int H, int W, int heads, int head_dim, float rope_theta, float eps, void* o,
                                  void* hip_stream) {
  clear_error();
  return guarded([&]() -> dit_status {
    Shape s;
    dit_status st = check_shape(T, H, W, heads, head_dim, s);
    if (st != DIT_OK) return st;
    if ((st = check_common(q, k, wq, wk, rope_theta, eps)) != DIT_OK) return st;
    if (!v || !o) return fail(DIT_ERR_INVALID_ARG, "null v or o");
    if (!aligned16(v) || !aligned16(o)) return fail(DIT_ERR_INVALID_ARG, "v and o must be 16-byte aligned");
    // The dense part of the workspace layout: RoPE table, the fragment images, then the tail partials of a
    // call that splits its last round.
    const Layout L = make_layout(s);
    const size_t need = L.partial + dit::tail_partial_area(dit::tail_plan(s.heads * s.nqt, (int)s.N), s.d);
    if (need > kStaticScratchBytes)
      return fail(DIT_ERR_UNSUPPORTED,
                  "needs %zu bytes of scratch (heads x ceil(N/128) tiles of %zu bytes plus the RoPE table); the "
                  "static scratch holds %zu: use dit_attn_dense with a workspace",
                  need, dit::tile_image_bytes(s.d), kStaticScratchBytes);
    hipStream_t stream = (hipStream_t)hip_stream;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    if (stream != nullptr) {
      int sdev = -1;
      e = hipStreamGetDevice(stream, &sdev);
      if (e != hipSuccess) return fail_hip(e, "hipStreamGetDevice");
      if (sdev != dev)
        return fail(DIT_ERR_INVALID_ARG, "the stream belongs to device %d but device %d is current", sdev, dev);
    }
    void* ws = nullptr;
    if ((st = static_scratch(dev, &ws)) != DIT_OK) return st;
    const size_t tb = (size_t)s.N * s.heads * s.d * 2, wb = (size_t)s.d * 4;
    const Buf bufs[] = {{q, tb, "q", false},   {k, tb, "k", false},   {v, tb, "v", false},
                        {wq, wb, "wq", false},  {wk, wb, "wk", false}, {o, tb, "o", true},
                        {ws, need, "the static scratch", true}};
    if ((st = check_disjoint(bufs)) != DIT_OK) return st;
    // Nothing in the scratch needs to start at zero: the table is uploaded and every fragment-image byte
    // of the call's tiles is written by the prepass before the attention kernel reads it.
    if ((st = upload_table(s, rope_theta, ws, L, stream)) != DIT_OK) return st;
    const dit::AttnArgs a = attn_args(s, q, k, v, wq, wk, eps, o, ws, L);
    e = dit::launch_attn_dense(a, stream);
    if (e != hipSuccess) return fail_hip(e, "attention kernel launch");
    return DIT_OK;
  });
}

}  // extern "C"

// ------------------------------------------------------------------------------------------------
// Operators around attention (dit_block.h)

namespace {

constexpr int kMaxHidden = 8192;

dit_status check_rows(long long tokens, int width, const char* what) {
  if (tokens < 0) return fail(DIT_ERR_INVALID_ARG, "tokens must be >= 0 (got %lld)", tokens);
  if (width < 8 || width % 8 != 0) return fail(DIT_ERR_INVALID_ARG, "%s must be a positive multiple of 8 (got %d)", what, width);
  if (tokens > (1ll << 40) / width) return fail(DIT_ERR_UNSUPPORTED, "tokens * %s too large", what);
  return DIT_OK;
}

}  // namespace

// These calls allocate nothing on the host; no C++ exception can arise in them.
extern "C" {

dit_status dit_adaln_modulate(const void* x, const float* shift, const float* scale, long long tokens, int hidden,
                              float eps, void* h, void* hip_stream) {
  clear_error();
  dit_status st = check_rows(tokens, hidden, "hidden");
  if (st != DIT_OK) return st;
  if (hidden > kMaxHidden) return fail(DIT_ERR_UNSUPPORTED, "hidden %d exceeds %d", hidden, kMaxHidden);
  if (!x || !shift || !scale || !h) return fail(DIT_ERR_INVALID_ARG, "null x, shift, scale or h");
  if (!aligned16(x) || !aligned16(shift) || !aligned16(scale) || !aligned16(h))
    return fail(DIT_ERR_INVALID_ARG, "x, shift, scale and h must be 16-byte aligned");
  if (!std::isfinite(eps) || eps < 0.f) return fail(DIT_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const size_t bytes = (size_t)tokens * hidden * 2;
  if (overlaps(x, bytes, h, bytes)) return fail(DIT_ERR_INVALID_ARG, "h overlaps x");
  if (tokens == 0) return DIT_OK;
  dit::BlockArgs a{};
  a.x = (const uint16_t*)x;
  a.shift = shift;
  a.scale = scale;
  a.h = (uint16_t*)h;
  a.tokens = tokens;
  a.hidden = hidden;
  a.eps = eps;
  const hipError_t e = dit::launch_adaln(a, false, true, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail_hip(e, "AdaLN kernel launch");
  return DIT_OK;
}

dit_status dit_gated_residual(const void* x, const void* y, const float* gate, const float* shift, const float* scale,
                              long long tokens, int hidden, float eps, void* x_out, void* h, void* hip_stream) {
  clear_error();
  dit_status st = check_rows(tokens, hidden, "hidden");
  if (st != DIT_OK) return st;
  if (hidden > kMaxHidden) return fail(DIT_ERR_UNSUPPORTED, "hidden %d exceeds %d", hidden, kMaxHidden);
  if (!x || !y || !gate || !x_out) return fail(DIT_ERR_INVALID_ARG, "null x, y, gate or x_out");
  if (h && (!shift || !scale)) return fail(DIT_ERR_INVALID_ARG, "h needs shift and scale");
  if (!aligned16(x) || !aligned16(y) || !aligned16(gate) || !aligned16(x_out) || (h && !aligned16(h)) ||
      (h && (!aligned16(shift) || !aligned16(scale))))
    return fail(DIT_ERR_INVALID_ARG, "tensors and vectors must be 16-byte aligned");
  if (h && (!std::isfinite(eps) || eps < 0.f)) return fail(DIT_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const size_t bytes = (size_t)tokens * hidden * 2;
  if (x_out != x && overlaps(x_out, bytes, x, bytes))
    return fail(DIT_ERR_INVALID_ARG, "x_out must be x itself or not overlap it");
  if (overlaps(x_out, bytes, y, bytes)) return fail(DIT_ERR_INVALID_ARG, "x_out overlaps y");
  if (h && (overlaps(h, bytes, x, bytes) || overlaps(h, bytes, y, bytes) || overlaps(h, bytes, x_out, bytes)))
    return fail(DIT_ERR_INVALID_ARG, "h overlaps x, y or x_out");
  if (tokens == 0) return DIT_OK;
  dit::BlockArgs a{};
  a.x = (const uint16_t*)x;
  a.y = (const uint16_t*)y;
  a.gate = gate;
  a.shift = shift;
  a.scale = scale;
  a.x_out = (uint16_t*)x_out;
  a.h = (uint16_t*)h;
  a.tokens = tokens;
  a.hidden = hidden;
  a.eps = eps;
  const hipError_t e = dit::launch_adaln(a, true, h != nullptr, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail_hip(e, "gated residual kernel launch");
  return DIT_OK;
}

dit_status dit_swiglu(const void* gate_up, long long tokens, int ffn, void* out, void* hip_stream) {
  clear_error();
  dit_status st = check_rows(tokens, ffn, "ffn");
  if (st != DIT_OK) return st;
  if (ffn > (1 << 28)) return fail(DIT_ERR_UNSUPPORTED, "ffn %d too large", ffn);
  if (!gate_up || !out) return fail(DIT_ERR_INVALID_ARG, "null gate_up or out");
  if (!aligned16(gate_up) || !aligned16(out)) return fail(DIT_ERR_INVALID_ARG, "gate_up and out must be 16-byte aligned");
  if (overlaps(gate_up, (size_t)tokens * ffn * 4, out, (size_t)tokens * ffn * 2))
    return fail(DIT_ERR_INVALID_ARG, "out overlaps gate_up");
  if (tokens == 0) return DIT_OK;
  dit::SwigluArgs a{};
  a.gu = (const uint16_t*)gate_up;
  a.out = (uint16_t*)out;
  a.tokens = tokens;
  a.ffn = ffn;
  const hipError_t e = dit::launch_swiglu(a, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail_hip(e, "SwiGLU kernel launch");
  return DIT_OK;
}

const char* dit_attn_last_error(void) { return g_err; }

}  // extern "C"
