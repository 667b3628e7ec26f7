// C ABI of libnsa: host-side argument validation and kernel dispatch (see include/nsa.h).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/nsa.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

nsa_status fail(nsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

// A launch failure can be forced from the host (NSA_FORCE_HIP_ERROR=1) to test error handling
// without any device work.
bool forced_hip_error() {
  const char* e = getenv("NSA_FORCE_HIP_ERROR");
  return e != nullptr && e[0] == '1';
}

nsa_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(NSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return NSA_OK;
}

// Every tensor a kernel reads with 16-byte vector loads must start on a 16-byte boundary (NULL is
// accepted: unused pointers are checked elsewhere).
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Opt-in debug check of the device-side preconditions on blk_cnt (NSA_DEBUG_CHECKS=1): copies the
// counts to the host, which synchronises the device, and verifies 1 <= blk_cnt[b] <= blk_cap.  Off
// by default: the library otherwise never synchronises.
nsa_status debug_check_counts(const nsa_layout* L, const char* fn) {
  const char* e = getenv("NSA_DEBUG_CHECKS");
  if (e == nullptr || e[0] != '1') return NSA_OK;
  int32_t* h = static_cast<int32_t*>(malloc(sizeof(int32_t) * (size_t)L->n_blk));
  if (h == nullptr) return fail(NSA_ERR_INVALID, "%s: debug check: out of host memory", fn);
  const hipError_t err = hipMemcpy(h, L->blk_cnt, sizeof(int32_t) * (size_t)L->n_blk, hipMemcpyDeviceToHost);
  if (err != hipSuccess) {
    free(h);
    return fail(NSA_ERR_HIP, "%s: debug check: reading blk_cnt: %s", fn, hipGetErrorString(err));
  }
  nsa_status st = NSA_OK;
  for (int32_t b = 0; b < L->n_blk; ++b) {
    if (h[b] < 1 || h[b] > L->blk_cap) {
      st = fail(NSA_ERR_INVALID, "%s: debug check: blk_cnt[%d] = %d is outside 1..%d", fn, b, h[b], L->blk_cap);
      break;
    }
  }
  free(h);
  return st;
}

// Every entry point calls this after validation and before any HIP call.
#define NSA_FORCED_FAILURE(fn)                                                                 \
  do {                                                                                         \
    if (forced_hip_error()) return fail(NSA_ERR_HIP, "%s: launch failure forced by NSA_FORCE_HIP_ERROR", fn); \
  } while (0)

nsa_status check_layout(const nsa_layout* L, const char* fn) {
  if (L == nullptr) return fail(NSA_ERR_INVALID, "%s: layout is NULL", fn);
  if (L->n_blk < 1) return fail(NSA_ERR_INVALID, "%s: n_blk must be >= 1 (got %d)", fn, L->n_blk);
  if (L->blk_cap < 1 || L->blk_cap > 64)
    return fail(NSA_ERR_INVALID, "%s: blk_cap must be in 1..64 (got %d)", fn, L->blk_cap);
  if (L->n_qh < 1 || L->n_kvh < 1 || L->n_qh % L->n_kvh != 0)
    return fail(NSA_ERR_INVALID, "%s: n_qh (%d) must be a positive multiple of n_kvh (%d)", fn, L->n_qh, L->n_kvh);
  if (L->head_dim < 1) return fail(NSA_ERR_INVALID, "%s: head_dim must be >= 1", fn);
  if (!(L->scale > 0.f) || L->scale > 1e30f) return fail(NSA_ERR_INVALID, "%s: scale must be a positive finite value", fn);
  if (L->blk_cnt == nullptr) return fail(NSA_ERR_INVALID, "%s: blk_cnt is NULL", fn);
  if ((long long)L->n_blk * L->blk_cap > 0x7FFFFFFFLL) return fail(NSA_ERR_INVALID, "%s: too many slots", fn);
  return debug_check_counts(L, fn);
}

bool dtype_ok(nsa_dtype d) { return d == NSA_F32 || d == NSA_BF16; }


}  // namespace

extern "C" {

const char* nsa_last_error(void) { return g_err; }

nsa_status nsa_pool_blocks(const nsa_layout* L, nsa_dtype dtype, int32_t n_heads, const void* x,
                           void* x_cmp, hipStream_t stream) {
  nsa_status st = check_layout(L, "nsa_pool_blocks");
  if (st != NSA_OK) return st;
  if (!dtype_ok(dtype)) return fail(NSA_ERR_INVALID, "nsa_pool_blocks: unknown dtype %d", (int)dtype);
  if (x == nullptr || x_cmp == nullptr) return fail(NSA_ERR_INVALID, "nsa_pool_blocks: x or x_cmp is NULL");
  if (n_heads < 1) return fail(NSA_ERR_INVALID, "nsa_pool_blocks: n_heads must be >= 1");
  const int vec = dtype == NSA_BF16 ? 8 : 4;     // elements per 16-byte piece
  if (((long long)n_heads * L->head_dim) % vec != 0)
    return fail(NSA_ERR_UNSUPPORTED, "nsa_pool_blocks: n_heads * head_dim must be a multiple of %d for this dtype", vec);
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(x_cmp)) % 16 != 0)
    return fail(NSA_ERR_UNSUPPORTED, "nsa_pool_blocks: x and x_cmp must be 16-byte aligned");
  NSA_FORCED_FAILURE("nsa_pool_blocks");
  return hip_status(nsa::launch_pool(dtype == NSA_BF16, x, x_cmp, L->blk_cnt, L->n_blk, L->blk_cap, n_heads,
                                     L->head_dim, stream),
                    "nsa_pool_blocks");
}

nsa_status nsa_pool_blocks_resblock(const nsa_layout* L, nsa_dtype dtype, int32_t n_heads, const void* x,
                                    const float* w1, const float* b1, const float* w2, const float* b2,
                                    void* x_cmp, hipStream_t stream) {
  nsa_status st = check_layout(L, "nsa_pool_blocks_resblock");
  if (st != NSA_OK) return st;
  if (!dtype_ok(dtype)) return fail(NSA_ERR_INVALID, "nsa_pool_blocks_resblock: unknown dtype %d", (int)dtype);
  if (x == nullptr || x_cmp == nullptr || w1 == nullptr || b1 == nullptr || w2 == nullptr || b2 == nullptr)
    return fail(NSA_ERR_INVALID, "nsa_pool_blocks_resblock: NULL pointer");
  if (n_heads < 1) return fail(NSA_ERR_INVALID, "nsa_pool_blocks_resblock: n_heads must be >= 1");
  if (L->head_dim > 64) return fail(NSA_ERR_UNSUPPORTED, "nsa_pool_blocks_resblock: head_dim must be <= 64");
  if (nsa::pool_resblock_lds_bytes(L->blk_cap, L->head_dim) > 160 * 1024)
    return fail(NSA_ERR_UNSUPPORTED, "nsa_pool_blocks_resblock: LDS need exceeds 160 KiB");
  if ((long long)L->n_blk * n_heads > 0x7FFFFFFFLL)
    return fail(NSA_ERR_UNSUPPORTED, "nsa_pool_blocks_resblock: n_blk * n_heads too large");
  NSA_FORCED_FAILURE("nsa_pool_blocks_resblock");
  return hip_status(nsa::launch_pool_resblock(dtype == NSA_BF16, x, x_cmp, L->blk_cnt, w1, b1, w2, b2, L->n_blk,
                                              L->blk_cap, n_heads, L->head_dim, stream),
                    "nsa_pool_blocks_resblock");
}

nsa_status nsa_build_volume_blocks(const float* sdf, int32_t G, int32_t N, float tau, int32_t max_blk,
                                   uint64_t* cell_mask, int32_t* cell_block, int32_t* n_blk, int32_t* blk_cnt,
                                   uint32_t* blk_key, float* pts, hipStream_t stream) {
  if (sdf == nullptr || cell_mask == nullptr || cell_block == nullptr || n_blk == nullptr)
    return fail(NSA_ERR_INVALID, "nsa_build_volume_blocks: NULL pointer");
  if (max_blk > 0 && (blk_cnt == nullptr || blk_key == nullptr || pts == nullptr))
    return fail(NSA_ERR_INVALID, "nsa_build_volume_blocks: NULL output with max_blk > 0");
  if (G < 2) return fail(NSA_ERR_INVALID, "nsa_build_volume_blocks: G must be >= 2");
  if (N < 4 || N % 4 != 0) return fail(NSA_ERR_INVALID, "nsa_build_volume_blocks: N must be a positive multiple of 4");
  if (max_blk < 0) return fail(NSA_ERR_INVALID, "nsa_build_volume_blocks: max_blk must be >= 0");
  if (!(tau >= 0.f) || tau == INFINITY) return fail(NSA_ERR_INVALID, "nsa_build_volume_blocks: tau must be finite, >= 0");
  if (N > 512 || ((N / 4) & (N / 4 - 1)) != 0)
    return fail(NSA_ERR_UNSUPPORTED, "nsa_build_volume_blocks: N / 4 must be a power of two and N <= 512");
  if ((long long)8 * N * G >= (1LL << 24))
    return fail(NSA_ERR_UNSUPPORTED, "nsa_build_volume_blocks: 8 * N * G must stay below 2^24 (exact fp32 coordinates)");
  NSA_FORCED_FAILURE("nsa_build_volume_blocks");
  return hip_status(nsa::launch_build_volume_blocks(sdf, G, N, tau, max_blk,
                                                    reinterpret_cast<unsigned long long*>(cell_mask), cell_block,
                                                    n_blk, blk_cnt, blk_key, pts, stream),
                    "nsa_build_volume_blocks");
}

static bool range_ok(int32_t lo, int32_t hi, int32_t n) { return lo >= 0 && lo <= hi && hi <= n; }

static nsa_status route_geometric(const char* fn, const nsa_layout* L, const float* pts, int32_t top_k,
                                  int32_t q_lo, int32_t q_hi, int32_t kv_lo, int32_t kv_hi, int32_t* centroids,
                                  int32_t* sel, uint32_t* sel_d2, hipStream_t stream) {
  nsa_status st = check_layout(L, fn);
  if (st != NSA_OK) return st;
  if (pts == nullptr || centroids == nullptr || sel == nullptr || L->blk_key == nullptr)
    return fail(NSA_ERR_INVALID, "%s: pts, centroids, sel and blk_key must be non-NULL", fn);
  if (top_k < 1 || top_k > 64) return fail(NSA_ERR_INVALID, "%s: top_k must be in 1..64 (got %d)", fn, top_k);
  if (!range_ok(q_lo, q_hi, L->n_blk) || !range_ok(kv_lo, kv_hi, L->n_blk))
    return fail(NSA_ERR_INVALID, "%s: block ranges must satisfy 0 <= lo <= hi <= n_blk", fn);
  NSA_FORCED_FAILURE(fn);
  nsa::RouteArgs a{};
  a.q_blk0 = q_lo;
  a.n_qblk = q_hi - q_lo;
  a.kv_lo = kv_lo;
  a.kv_hi = kv_hi;
  a.pts = pts;
  a.blk_cnt = L->blk_cnt;
  a.blk_key = L->blk_key;
  a.cent = centroids;
  a.sel = sel;
  a.sel_d2 = sel_d2;
  a.n_blk = L->n_blk;
  a.cap = L->blk_cap;
  a.top_k = top_k;
  return hip_status(nsa::launch_route_geometric(a, stream), fn);
}

nsa_status nsa_route_geometric(const nsa_layout* L, const float* pts, int32_t top_k, int32_t* centroids,
                               int32_t* sel, uint32_t* sel_d2, hipStream_t stream) {
  const int32_t n = L != nullptr ? L->n_blk : 0;
  return route_geometric("nsa_route_geometric", L, pts, top_k, 0, n, 0, n, centroids, sel, sel_d2, stream);
}

nsa_status nsa_route_geometric_noalloc(const nsa_layout* L, const float* pts, int32_t top_k, int32_t* sel,
                                       uint32_t* sel_d2, hipStream_t stream) {
  const char* fn = "nsa_route_geometric_noalloc";
  nsa_status st = check_layout(L, fn);
  if (st != NSA_OK) return st;
  if (pts == nullptr || sel == nullptr || L->blk_key == nullptr)
    return fail(NSA_ERR_INVALID, "%s: pts, sel and blk_key must be non-NULL", fn);
  if (top_k < 1 || top_k > 64) return fail(NSA_ERR_INVALID, "%s: top_k must be in 1..64 (got %d)", fn, top_k);
  if (L->n_blk > nsa::kScratchMaxBlocks)
    return fail(NSA_ERR_UNSUPPORTED, "%s: n_blk %d exceeds the fixed centroid array (%d blocks)", fn, L->n_blk,
                nsa::kScratchMaxBlocks);
  NSA_FORCED_FAILURE(fn);
  int32_t* cent = nullptr;
  nsa_status hs = hip_status(nsa::route_scratch_centroids(&cent), fn);
  if (hs != NSA_OK) return hs;
  nsa::RouteArgs a{};
  a.q_blk0 = 0;
  a.n_qblk = L->n_blk;
  a.kv_lo = 0;
  a.kv_hi = L->n_blk;
  a.pts = pts;
  a.blk_cnt = L->blk_cnt;
  a.blk_key = L->blk_key;
  a.cent = cent;
  a.sel = sel;
  a.sel_d2 = sel_d2;
  a.n_blk = L->n_blk;
  a.cap = L->blk_cap;
  a.top_k = top_k;
  return hip_status(nsa::launch_route_geometric(a, stream), fn);
}

nsa_status nsa_route_geometric_views(const nsa_layout* L, const float* pts, int32_t top_k, int32_t n_vol_blk,
                                     int32_t n_views, const float* view_proj, const int32_t* cell_blk,
                                     int32_t n_cell, int32_t cell_size, int32_t radius, int32_t* centroids,
                                     int32_t* geom, int32_t* sel, uint32_t* sel_d2, hipStream_t stream) {
  const char* fn = "nsa_route_geometric_views";
  nsa_status st = check_layout(L, fn);
  if (st != NSA_OK) return st;
  if (pts == nullptr || centroids == nullptr || sel == nullptr || L->blk_key == nullptr)
    return fail(NSA_ERR_INVALID, "%s: pts, centroids, sel and blk_key must be non-NULL", fn);
  if (top_k < 1 || top_k > 64) return fail(NSA_ERR_INVALID, "%s: top_k must be in 1..64 (got %d)", fn, top_k);
  if (n_vol_blk < 0 || n_vol_blk > L->n_blk) return fail(NSA_ERR_INVALID, "%s: n_vol_blk must be in [0, n_blk]", fn);
  if (n_views < 0) return fail(NSA_ERR_INVALID, "%s: n_views must be >= 0", fn);
  if (n_views > 0) {
    if (view_proj == nullptr || cell_blk == nullptr || geom == nullptr)
      return fail(NSA_ERR_INVALID, "%s: view_proj, cell_blk and geom must be non-NULL with views", fn);
    if (n_cell < 1 || n_cell > 4096) return fail(NSA_ERR_INVALID, "%s: n_cell must be in 1..4096", fn);
    if (cell_size < 1 || cell_size > 1024 || (cell_size & (cell_size - 1)) != 0)
      return fail(NSA_ERR_INVALID, "%s: cell_size must be a power of two in 1..1024", fn);
    if (radius < 0 || radius > 16) return fail(NSA_ERR_INVALID, "%s: radius must be in 0..16", fn);
  }
  NSA_FORCED_FAILURE(fn);
  nsa::RouteArgs a{};
  a.q_blk0 = 0;
  a.n_qblk = L->n_blk;
  a.kv_lo = 0;
  a.kv_hi = n_vol_blk;
  a.pts = pts;
  a.blk_cnt = L->blk_cnt;
  a.blk_key = L->blk_key;
  a.cent = centroids;
  a.sel = sel;
  a.sel_d2 = sel_d2;
  a.n_blk = L->n_blk;
  a.cap = L->blk_cap;
  a.top_k = top_k;
  a.view_proj = view_proj;
  a.cell_blk = cell_blk;
  a.boxes = geom;
  a.lat = geom != nullptr ? geom + (size_t)8 * L->n_blk : nullptr;
  a.n_views = n_views;
  a.n_cell = n_cell;
  a.cell_shift = __builtin_ctz((unsigned)cell_size);
  a.radius = radius;
  return hip_status(nsa::launch_route_geometric(a, stream), fn);
}

nsa_status nsa_route_geometric_range(const nsa_layout* L, const float* pts, int32_t top_k, int32_t q_blk_lo,
                                     int32_t q_blk_hi, int32_t kv_blk_lo, int32_t kv_blk_hi, int32_t* centroids,
                                     int32_t* sel, uint32_t* sel_d2, hipStream_t stream) {
  return route_geometric("nsa_route_geometric_range", L, pts, top_k, q_blk_lo, q_blk_hi, kv_blk_lo, kv_blk_hi,
                         centroids, sel, sel_d2, stream);
}

nsa_status nsa_route_scores_topk(const nsa_layout* L, nsa_dtype dtype, nsa_qgran q_gran, const void* q,
                                 const void* k_cmp, const float* lse, int32_t top_k, int32_t* sel,
                                 hipStream_t stream) {
  nsa_status st = check_layout(L, "nsa_route_scores_topk");
  if (st != NSA_OK) return st;
  if (!dtype_ok(dtype)) return fail(NSA_ERR_INVALID, "nsa_route_scores_topk: unknown dtype");
  if (q_gran != NSA_Q_TOKEN && q_gran != NSA_Q_BLOCK) return fail(NSA_ERR_INVALID, "nsa_route_scores_topk: bad q_gran");
  if (q == nullptr || k_cmp == nullptr || sel == nullptr || L->blk_key == nullptr)
    return fail(NSA_ERR_INVALID, "nsa_route_scores_topk: q, k_cmp, sel and blk_key must be non-NULL");
  if (top_k < 1 || top_k > 64) return fail(NSA_ERR_INVALID, "nsa_route_scores_topk: top_k must be in 1..64");
  const int G = L->n_qh / L->n_kvh;
  if (G > 1 && lse == nullptr) return fail(NSA_ERR_INVALID, "nsa_route_scores_topk: lse is required when n_qh > n_kvh");
  if (!aligned16(q) || !aligned16(k_cmp) || !aligned16(lse))
    return fail(NSA_ERR_UNSUPPORTED, "nsa_route_scores_topk: q, k_cmp and lse must be 16-byte aligned");
  if (G == 1) {
    if (L->head_dim != 64 || q_gran != NSA_Q_BLOCK)
      return fail(NSA_ERR_UNSUPPORTED,
                  "nsa_route_scores_topk: with one query head per KV head the compiled kernel takes head_dim 64 "
                  "and NSA_Q_BLOCK rows");
    NSA_FORCED_FAILURE("nsa_route_scores_topk");
    nsa::G1Args g{};
    g.q_cmp = q;
    g.k_cmp = k_cmp;
    g.sel = sel;
    g.blk_cnt = L->blk_cnt;
    g.blk_key = L->blk_key;
    g.n_blk = L->n_blk;
    g.cap = L->blk_cap;
    g.n_qh = L->n_qh;
    g.n_kvh = L->n_kvh;
    g.top_k = top_k;
    g.scale = L->scale;
    return hip_status(nsa::launch_route_g1(dtype == NSA_BF16, g, stream), "nsa_route_scores_topk");
  }
  if (L->head_dim != 32 || G != 16)
    return fail(NSA_ERR_UNSUPPORTED, "nsa_route_scores_topk: compiled for head_dim 32 with 16 query heads per KV head");
  if (L->n_blk > 65536) return fail(NSA_ERR_UNSUPPORTED, "nsa_route_scores_topk: n_blk must be <= 65536");
  NSA_FORCED_FAILURE("nsa_route_scores_topk");
  nsa::ScoreRouteArgs a;
  a.q = q;
  a.k_cmp = k_cmp;
  a.lse = lse;
  a.blk_cnt = L->blk_cnt;
  a.blk_key = L->blk_key;
  a.sel = sel;
  // NSA_Q_BLOCK: the pooled rows, 64 per workgroup
  a.dense_rows = q_gran == NSA_Q_BLOCK ? 1 : 0;
  a.n_rows = a.dense_rows ? L->n_blk : L->n_blk * L->blk_cap;
  a.n_blk = L->n_blk;
  a.cap = a.dense_rows ? 64 : L->blk_cap;
  a.n_qh = L->n_qh;
  a.n_kvh = L->n_kvh;
  a.top_k = top_k;
  a.scale = L->scale;
  return hip_status(nsa::launch_route_scores(dtype == NSA_BF16, a, stream), "nsa_route_scores_topk");
}

static nsa_status attn_fwd(const char* fn, const nsa_layout* L, nsa_dtype dtype, uint32_t branches,
                           nsa_qgran q_gran, int32_t q_lo, int32_t q_hi, int32_t kv_lo, int32_t kv_hi,
                           const void* q, const void* k, const void* v, const void* q_cmp, const void* k_cmp,
                           const void* v_cmp, const int32_t* sel, int32_t top_k, int32_t sel_groups,
                           const void* gate_logits, int32_t gate_stride, void* o, float* lse, int32_t f_lo,
                           int32_t f_hi, hipStream_t stream) {
  nsa_status st = check_layout(L, fn);
  if (st != NSA_OK) return st;
  if (!range_ok(q_lo, q_hi, L->n_blk) || !range_ok(kv_lo, kv_hi, L->n_blk) || !range_ok(f_lo, f_hi, L->n_blk))
    return fail(NSA_ERR_INVALID, "%s: block ranges must satisfy 0 <= lo <= hi <= n_blk", fn);
  const bool forced = f_hi > f_lo;
  if (forced && !(branches & NSA_BR_SEL)) return fail(NSA_ERR_INVALID, "%s: a forced block range needs SEL", fn);
  const bool whole = q_lo == 0 && q_hi == L->n_blk && kv_lo == 0 && kv_hi == L->n_blk;
  if (!dtype_ok(dtype)) return fail(NSA_ERR_INVALID, "%s: unknown dtype", fn);
  if (branches == 0 || (branches & ~7u) != 0) return fail(NSA_ERR_INVALID, "%s: branches must be a non-empty OR of NSA_BR_* bits", fn);
  if (q_gran != NSA_Q_TOKEN && q_gran != NSA_Q_BLOCK) return fail(NSA_ERR_INVALID, "%s: bad q_gran", fn);
  const int n_named = __builtin_popcount(branches);
  if (gate_logits == nullptr && n_named != 1)
    return fail(NSA_ERR_INVALID, "%s: several branches need gate_logits to be combined", fn);
  if (gate_stride == 0) gate_stride = n_named;
  if (gate_stride < n_named || gate_stride > 64)
    return fail(NSA_ERR_INVALID, "%s: gate_stride must be in [number of branches, 64]", fn);
  if (gate_stride != n_named && L->n_qh == L->n_kvh)
    return fail(NSA_ERR_UNSUPPORTED, "%s: a gate stride needs the grouped-query kernel (head_dim 32)", fn);
  if (lse != nullptr && n_named != 1) return fail(NSA_ERR_INVALID, "%s: lse needs exactly one branch", fn);
  if (o == nullptr || q == nullptr) return fail(NSA_ERR_INVALID, "%s: q and o must be non-NULL", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_cmp) || !aligned16(k_cmp) ||
      !aligned16(v_cmp) || !aligned16(o))
    return fail(NSA_ERR_UNSUPPORTED, "%s: q, k, v, q_cmp, k_cmp, v_cmp and o must be 16-byte aligned", fn);
  if ((branches & (NSA_BR_SEL | NSA_BR_LOC)) && (k == nullptr || v == nullptr))
    return fail(NSA_ERR_INVALID, "%s: SEL and LOC need k and v", fn);
  if ((branches & NSA_BR_CMP) && (k_cmp == nullptr || v_cmp == nullptr))
    return fail(NSA_ERR_INVALID, "%s: CMP needs k_cmp and v_cmp", fn);
  if ((branches & NSA_BR_CMP) && q_gran == NSA_Q_BLOCK && q_cmp == nullptr)
    return fail(NSA_ERR_INVALID, "%s: CMP with NSA_Q_BLOCK needs q_cmp", fn);
  if (branches & NSA_BR_SEL) {
    if (sel == nullptr) return fail(NSA_ERR_INVALID, "%s: SEL needs sel", fn);
    if (top_k < 1 || top_k > 64) return fail(NSA_ERR_INVALID, "%s: top_k must be in 1..64 (got %d)", fn, top_k);
    if (sel_groups != 1 && sel_groups != L->n_kvh)
      return fail(NSA_ERR_INVALID, "%s: sel_groups must be 1 or n_kvh", fn);
    if (L->n_blk > 65536) return fail(NSA_ERR_UNSUPPORTED, "%s: SEL supports n_blk <= 65536", fn);
  }
  if (L->n_qh == L->n_kvh) {
    // one query head per KV head (score-routed, block-granular layout)
    if (L->head_dim != 64 || q_gran != NSA_Q_BLOCK || L->blk_cap > 16 || 64 % L->blk_cap != 0)
      return fail(NSA_ERR_UNSUPPORTED,
                  "%s: with one query head per KV head the compiled kernels take head_dim 64, NSA_Q_BLOCK "
                  "and blk_cap in {1, 2, 4, 8, 16}", fn);
    if (!whole) return fail(NSA_ERR_UNSUPPORTED, "%s: block ranges need the grouped-query kernel (head_dim 32)", fn);
    if (f_hi - f_lo > nsa::kMaxForcedBlocks)
      return fail(NSA_ERR_UNSUPPORTED, "%s: at most %d forced blocks", fn, nsa::kMaxForcedBlocks);
    NSA_FORCED_FAILURE(fn);
    nsa::G1Args g{};
    g.q = q;
    g.k = k;
    g.v = v;
    g.q_cmp = q_cmp;
    g.k_cmp = k_cmp;
    g.v_cmp = v_cmp;
    g.sel = sel;
    g.blk_cnt = L->blk_cnt;
    g.blk_key = L->blk_key;
    g.gates = gate_logits;
    g.o = o;
    g.lse = lse;
    g.n_blk = L->n_blk;
    g.cap = L->blk_cap;
    g.n_qh = L->n_qh;
    g.n_kvh = L->n_kvh;
    g.top_k = (branches & NSA_BR_SEL) ? top_k : 0;
    g.sel_groups = sel_groups < 1 ? 1 : sel_groups;
    g.n_gch = n_named;
    g.ch_cmp = 0;
    g.ch_sel = (branches & NSA_BR_CMP) ? 1 : 0;
    g.ch_loc = g.ch_sel + ((branches & NSA_BR_SEL) ? 1 : 0);
    g.scale = L->scale;
    g.branches = branches;
    g.f_lo = f_lo;
    g.f_hi = f_hi;
    return hip_status(nsa::launch_attn_g1(dtype == NSA_BF16, g, stream), fn);
  }
  if (forced)
    return fail(NSA_ERR_UNSUPPORTED, "%s: a forced block range needs the one-head-per-KV-head kernels (head_dim 64)", fn);
  if (L->head_dim != 32 || L->n_qh / L->n_kvh != 16)
    return fail(NSA_ERR_UNSUPPORTED, "%s: compiled for head_dim 32 with 16 query heads per KV head (or head_dim 64 "
                                     "with one query head per KV head and NSA_Q_BLOCK)", fn);
  if (q_gran == NSA_Q_BLOCK && !whole)
    return fail(NSA_ERR_UNSUPPORTED, "%s: block ranges take per-token query rows (NSA_Q_TOKEN)", fn);
  // the grouped-query kernels index rows of q, o, gate_logits, lse and sel in 32-bit arithmetic
  if ((long long)L->n_blk * L->blk_cap * L->n_qh * (gate_stride > 32 ? gate_stride : 32) > 0x7FFFFFFFLL)
    return fail(NSA_ERR_UNSUPPORTED, "%s: n_blk * blk_cap * n_qh * max(32, gate_stride) must be < 2^31", fn);
  nsa::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_cmp = k_cmp;
  a.v_cmp = v_cmp;
  a.sel = sel;
  a.blk_cnt = L->blk_cnt;
  a.gates = gate_logits;
  a.o = o;
  a.lse = lse;
  a.n_blk = L->n_blk;
  a.cap = L->blk_cap;
  a.n_qh = L->n_qh;
  a.n_kvh = L->n_kvh;
  a.top_k = (branches & NSA_BR_SEL) ? top_k : 0;
  a.sel_groups = sel_groups < 1 ? 1 : sel_groups;
  a.n_gch = gate_stride;
  a.scale = L->scale;
  a.branches = branches;
  a.n_words = (L->n_blk + 31) / 32;
  a.sel_per_block = q_gran == NSA_Q_BLOCK ? 1 : 0;
  // gate channels in the order CMP, SEL, LOC among the named branches (whatever each launch runs)
  a.ch_sel = (branches & NSA_BR_CMP) ? 1 : 0;
  a.ch_loc = n_named - 1;
  {
    // distinct selected blocks of one query block: one routing row per slot, or one per block
    long long u = (long long)(a.sel_per_block ? 1 : L->blk_cap) * (a.top_k > 0 ? a.top_k : 1);
    a.u_cap = (int)(u < L->n_blk ? u : L->n_blk);
  }
  // Test hook (NSA_TEST_RING_STALL=1): the selected branch's tile ring waits for one count more
  // than ever arrives, with a short bound, so the bounded-wait path runs (output NaN, no hang).
  // It and NSA_SEL_RING=1 keep the selected branch in the fused kernel's tile ring.
  bool sel_ring;
  {
    const char* e = getenv("NSA_TEST_RING_STALL");
    const bool stall = e != nullptr && e[0] == '1';
    a.ring_spins = stall ? 64 : (1 << 16);
    a.ring_stall = stall ? 1 : 0;
    const char* f = getenv("NSA_SEL_RING");
    sel_ring = stall || (f != nullptr && f[0] == '1');
  }
  a.q_blk0 = q_lo;
  a.n_qblk = q_hi - q_lo;
  a.kv_lo = kv_lo;
  a.kv_hi = kv_hi;
  const size_t lds = nsa::attn_lds_bytes(dtype == NSA_BF16, a);
  if (lds > 160 * 1024) return fail(NSA_ERR_UNSUPPORTED, "%s: LDS need %zu bytes exceeds 160 KiB", fn, lds);
  NSA_FORCED_FAILURE(fn);
  if (q_gran == NSA_Q_TOKEN) {
    // bf16: the local and selected branches run in kernels of wave-owned token clusters, each
    // adding its gated result to what the launches before it wrote (the compressed branch in the
    // fused kernel first)
    // (the wave kernels' block lists hold a block index in 16 bits: n_blk <= 65536, which the
    // selected branch requires anyway; a larger local-only call stays in the fused kernel)
    if (dtype != NSA_BF16 || !(branches & (NSA_BR_SEL | NSA_BR_LOC)) || sel_ring || L->n_blk > 65536)
      return hip_status(nsa::launch_attn(dtype == NSA_BF16, a, stream), fn);
    if (nsa::sel_wave_lds(a) > 160 * 1024)
      return fail(NSA_ERR_UNSUPPORTED, "%s: LDS need %zu bytes exceeds 160 KiB", fn, nsa::sel_wave_lds(a));
    // With the compressed branch named, the local branch stays in the fused kernel (its one tile
    // there costs less than a launch of its own that reads and writes o again); without it, it
    // runs in the wave kernel's local instantiation.
    int written = 0;
    if (branches & NSA_BR_CMP) {
      nsa::AttnArgs f = a;
      f.branches = branches & (NSA_BR_CMP | NSA_BR_LOC);
      f.top_k = 0;
      hipError_t e = nsa::launch_attn(1, f, stream);
      if (e != hipSuccess) return hip_status(e, fn);
      written = 1;
    } else if (branches & NSA_BR_LOC) {
      hipError_t e = nsa::launch_sel_wave(a, 1, written, stream);
      if (e != hipSuccess) return hip_status(e, fn);
      written = 1;
    }
    if (!(branches & NSA_BR_SEL)) return NSA_OK;
    return hip_status(nsa::launch_sel_wave(a, 0, written, stream), fn);
  }
  // block rows: the selected and local branches (token queries, the block's routing row) in the
  // fused kernel, reading the gate channels after the compressed one; then the compressed branch
  // of the pooled queries, adding each block's gated result to its tokens
  const uint32_t rest = branches & (NSA_BR_SEL | NSA_BR_LOC);
  const bool has_cmp = (branches & NSA_BR_CMP) != 0;
  if (rest) {
    nsa::AttnArgs f = a;
    f.branches = rest;   // gate channels stay those of the whole branch set (a.ch_sel, a.ch_loc)
    hipError_t e = nsa::launch_attn(dtype == NSA_BF16, f, stream);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  if (!has_cmp) return NSA_OK;
  nsa::AttnArgs c = a;
  c.q = q_cmp;
  return hip_status(nsa::launch_cmp_pooled(dtype == NSA_BF16, c, rest ? 1 : 0, 0, stream), fn);
}

nsa_status nsa_attn_fwd(const nsa_layout* L, nsa_dtype dtype, uint32_t branches, nsa_qgran q_gran,
                        const void* q, const void* k, const void* v, const void* q_cmp, const void* k_cmp,
                        const void* v_cmp, const int32_t* sel, int32_t top_k, int32_t sel_groups,
                        const void* gate_logits, void* o, float* lse, hipStream_t stream) {
  const int32_t n = L != nullptr ? L->n_blk : 0;
  return attn_fwd("nsa_attn_fwd", L, dtype, branches, q_gran, 0, n, 0, n, q, k, v, q_cmp, k_cmp, v_cmp, sel, top_k,
                  sel_groups, gate_logits, 0, o, lse, 0, 0, stream);
}

nsa_status nsa_attn_fwd_forced(const nsa_layout* L, nsa_dtype dtype, uint32_t branches, nsa_qgran q_gran,
                               const void* q, const void* k, const void* v, const void* q_cmp, const void* k_cmp,
                               const void* v_cmp, const int32_t* sel, int32_t top_k, int32_t sel_groups,
                               int32_t forced_lo, int32_t forced_hi, const void* gate_logits, void* o, float* lse,
                               hipStream_t stream) {
  const int32_t n = L != nullptr ? L->n_blk : 0;
  return attn_fwd("nsa_attn_fwd_forced", L, dtype, branches, q_gran, 0, n, 0, n, q, k, v, q_cmp, k_cmp, v_cmp, sel,
                  top_k, sel_groups, gate_logits, 0, o, lse, forced_lo, forced_hi, stream);
}

nsa_status nsa_attn_fwd_range(const nsa_layout* L, nsa_dtype dtype, uint32_t branches, int32_t q_blk_lo,
                              int32_t q_blk_hi, int32_t kv_blk_lo, int32_t kv_blk_hi, const void* q, const void* k,
                              const void* v, const void* k_cmp, const void* v_cmp, const int32_t* sel,
                              int32_t top_k, int32_t sel_groups, const void* gate_logits, int32_t gate_stride,
                              void* o, float* lse, hipStream_t stream) {
  return attn_fwd("nsa_attn_fwd_range", L, dtype, branches, NSA_Q_TOKEN, q_blk_lo, q_blk_hi, kv_blk_lo, kv_blk_hi,
                  q, k, v, nullptr, k_cmp, v_cmp, sel, top_k, sel_groups, gate_logits, gate_stride, o, lse, 0, 0,
                  stream);
}

nsa_status nsa_attn_fwd_scores_routed(const nsa_layout* L, nsa_dtype dtype, const void* q, const void* k,
                                      const void* v, const void* q_cmp, const void* k_cmp, const void* v_cmp,
                                      int32_t top_k, const void* gate_logits, void* o, int32_t* sel,
                                      hipStream_t stream) {
  const char* fn = "nsa_attn_fwd_scores_routed";
  nsa_status st = check_layout(L, fn);
  if (st != NSA_OK) return st;
  if (!dtype_ok(dtype)) return fail(NSA_ERR_INVALID, "%s: unknown dtype", fn);
  if (q == nullptr || k == nullptr || v == nullptr || q_cmp == nullptr || k_cmp == nullptr || v_cmp == nullptr ||
      gate_logits == nullptr || o == nullptr || sel == nullptr || L->blk_key == nullptr)
    return fail(NSA_ERR_INVALID, "%s: q, k, v, q_cmp, k_cmp, v_cmp, gate_logits, o, sel and blk_key must be non-NULL", fn);
  if (top_k < 1 || top_k > 64) return fail(NSA_ERR_INVALID, "%s: top_k must be in 1..64 (got %d)", fn, top_k);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_cmp) || !aligned16(k_cmp) || !aligned16(v_cmp) ||
      !aligned16(o))
    return fail(NSA_ERR_UNSUPPORTED, "%s: q, k, v, q_cmp, k_cmp, v_cmp and o must be 16-byte aligned", fn);
  if (L->n_qh != L->n_kvh || L->head_dim != 64 || L->blk_cap > 16 || 64 % L->blk_cap != 0 || top_k > 32)
    return fail(NSA_ERR_UNSUPPORTED, "%s: compiled for one query head per KV head, head_dim 64, blk_cap in "
                                     "{1, 2, 4, 8, 16} and top_k <= 32", fn);
  NSA_FORCED_FAILURE(fn);
  nsa::G1Args g{};
  g.q = q;
  g.k = k;
  g.v = v;
  g.q_cmp = q_cmp;
  g.k_cmp = k_cmp;
  g.v_cmp = v_cmp;
  g.sel = sel;
  g.blk_cnt = L->blk_cnt;
  g.blk_key = L->blk_key;
  g.gates = gate_logits;
  g.o = o;
  g.lse = nullptr;
  g.n_blk = L->n_blk;
  g.cap = L->blk_cap;
  g.n_qh = L->n_qh;
  g.n_kvh = L->n_kvh;
  g.top_k = top_k;
  g.sel_groups = L->n_kvh;
  g.n_gch = 2;
  g.ch_cmp = 0;
  g.ch_sel = 1;
  g.ch_loc = 2;
  g.scale = L->scale;
  g.branches = NSA_BR_CMP | NSA_BR_SEL;
  g.f_lo = 0;
  g.f_hi = 0;
  return hip_status(nsa::launch_attn_g1_routed(dtype == NSA_BF16, g, stream), fn);
}

nsa_status nsa_gate_combine(nsa_dtype dtype, int32_t n_rows, int32_t n_qh, int32_t head_dim, int32_t n_branch,
                            const void* const* o_branch, const void* gate_logits, void* o, hipStream_t stream) {
  if (!dtype_ok(dtype)) return fail(NSA_ERR_INVALID, "nsa_gate_combine: unknown dtype");
  if (n_rows < 1 || n_qh < 1 || head_dim < 1) return fail(NSA_ERR_INVALID, "nsa_gate_combine: sizes must be >= 1");
  if (n_branch < 1 || n_branch > 8) return fail(NSA_ERR_INVALID, "nsa_gate_combine: n_branch must be in 1..8");
  if (o_branch == nullptr || gate_logits == nullptr || o == nullptr)
    return fail(NSA_ERR_INVALID, "nsa_gate_combine: NULL pointer");
  for (int c = 0; c < n_branch; ++c)
    if (o_branch[c] == nullptr) return fail(NSA_ERR_INVALID, "nsa_gate_combine: o_branch[%d] is NULL", c);
  if (head_dim % 4 != 0) return fail(NSA_ERR_UNSUPPORTED, "nsa_gate_combine: head_dim must be a multiple of 4");
  {
    const uintptr_t align = dtype == NSA_BF16 ? 8 : 16;     // four elements per vector access
    uintptr_t bits = reinterpret_cast<uintptr_t>(o);
    for (int c = 0; c < n_branch; ++c) bits |= reinterpret_cast<uintptr_t>(o_branch[c]);
    if (bits % align != 0)
      return fail(NSA_ERR_UNSUPPORTED, "nsa_gate_combine: o and o_branch must be %d-byte aligned", (int)align);
  }
  NSA_FORCED_FAILURE("nsa_gate_combine");
  return hip_status(nsa::launch_gate(dtype == NSA_BF16, n_rows, n_qh, head_dim, n_branch, o_branch, gate_logits, o,
                                     stream),
                    "nsa_gate_combine");
}

nsa_status dense_gated_xattn_fwd(nsa_dtype dtype, int32_t n_tok, int32_t n_x, int32_t n_qh, int32_t n_kvh,
                                 int32_t head_dim, float scale, const void* q, const void* k, const void* v,
                                 const void* gate_logits, void* o, hipStream_t stream) {
  if (!dtype_ok(dtype)) return fail(NSA_ERR_INVALID, "dense_gated_xattn_fwd: unknown dtype");
  if (n_tok < 1 || n_x < 0 || n_x > n_tok) return fail(NSA_ERR_INVALID, "dense_gated_xattn_fwd: need n_tok >= 1 and 0 <= n_x <= n_tok");
  if (n_qh < 1 || n_kvh < 1 || n_qh % n_kvh != 0 || head_dim < 1)
    return fail(NSA_ERR_INVALID, "dense_gated_xattn_fwd: bad head counts");
  if (!(scale > 0.f) || scale > 1e30f) return fail(NSA_ERR_INVALID, "dense_gated_xattn_fwd: bad scale");
  if (q == nullptr || k == nullptr || v == nullptr || gate_logits == nullptr || o == nullptr)
    return fail(NSA_ERR_INVALID, "dense_gated_xattn_fwd: NULL pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(NSA_ERR_UNSUPPORTED, "dense_gated_xattn_fwd: q, k and v must be 16-byte aligned");
  if (head_dim != 32 || n_qh / n_kvh != 16)
    return fail(NSA_ERR_UNSUPPORTED, "dense_gated_xattn_fwd: compiled for head_dim 32, 16 query heads per KV head");
  if ((long long)n_tok * n_qh * 32 > 0x7FFFFFFFLL)   // rows of q, o and gate_logits are indexed in 32 bits
    return fail(NSA_ERR_UNSUPPORTED, "dense_gated_xattn_fwd: n_tok * n_qh * 32 must be < 2^31");
  NSA_FORCED_FAILURE("dense_gated_xattn_fwd");
  nsa::DenseArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.gates = gate_logits;
  a.o = o;
  a.n_tok = n_tok;
  a.n_x = n_x;
  a.n_qh = n_qh;
  a.n_kvh = n_kvh;
  a.scale = scale;
  return hip_status(nsa::launch_dense(dtype == NSA_BF16, a, stream), "dense_gated_xattn_fwd");
}

}  // extern "C"
