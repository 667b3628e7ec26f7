// Block routing for the selected branch, without materialising a score or distance matrix.
//
// Geometric routing (LSRM pages, hyper.ai summary of arXiv 2604.05182, section 方法, routing
// paragraph; Korean summary, section 2.2): a query keeps the blocks whose centres are nearest to its
// 3D point.  The metric is made exact and reproducible on an integer lattice: u = rint(4096 p) + 4096
// per axis, block centroid rounded half-up, squared distance < 2^28 in 32-bit integers; ranking is
// the total order (d2, blk_key).
//
// (Score routing in grouped-query form is in route_scores.hip.)
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace nsa {
namespace {

__device__ __forceinline__ int lattice(float p) { return (int)rintf(4096.0f * p) + 4096; }

// One wave per block: integer centroid of the block's valid points plus its key.
// With `boxes`, also the lattice bounding box of the block's points and (`lat`) each point's packed
// lattice coordinates.
__global__ __launch_bounds__(64) void centroid_kernel(const float* __restrict__ pts, const int32_t* __restrict__ blk_cnt,
                                                      const uint32_t* __restrict__ blk_key, int32_t* __restrict__ cent,
                                                      int32_t* __restrict__ boxes, int32_t* __restrict__ lat, int cap) {
  const int b = blockIdx.x, l = threadIdx.x;
  const int cnt = blk_cnt[b];
  int sx = 0, sy = 0, sz = 0;
  int lo[3] = {1 << 30, 1 << 30, 1 << 30}, hi[3] = {-(1 << 30), -(1 << 30), -(1 << 30)};
  for (int t = l; t < cnt; t += 64) {
    const float* p = pts + (size_t)(b * cap + t) * 3;
    const int x = lattice(p[0]), y = lattice(p[1]), z = lattice(p[2]);
    if (lat != nullptr) reinterpret_cast<int2*>(lat)[b * cap + t] = make_int2(x | (y << 16), z);
    sx += x;
    sy += y;
    sz += z;
    lo[0] = min(lo[0], x), lo[1] = min(lo[1], y), lo[2] = min(lo[2], z);
    hi[0] = max(hi[0], x), hi[1] = max(hi[1], y), hi[2] = max(hi[2], z);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sx += __shfl_xor(sx, o, 64);
    sy += __shfl_xor(sy, o, 64);
    sz += __shfl_xor(sz, o, 64);
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) {
      lo[ax] = min(lo[ax], __shfl_xor(lo[ax], o, 64));
      hi[ax] = max(hi[ax], __shfl_xor(hi[ax], o, 64));
    }
  }
  if (l == 0 && boxes != nullptr) {
    reinterpret_cast<int4*>(boxes)[2 * b] = make_int4(lo[0], lo[1], lo[2], 0);
    reinterpret_cast<int4*>(boxes)[2 * b + 1] = make_int4(hi[0], hi[1], hi[2], 0);
  }
  if (l == 0) {
    int4 c;
    c.x = (2 * sx + cnt) / (2 * cnt);
    c.y = (2 * sy + cnt) / (2 * cnt);
    c.z = (2 * sz + cnt) / (2 * cnt);
    c.w = (int)blk_key[b];
    reinterpret_cast<int4*>(cent)[b] = c;
  }
}

__device__ __forceinline__ bool before(uint32_t d, uint32_t k, uint32_t d2, uint32_t k2) {
  return d < d2 || (d == d2 && k < k2);
}

// Sorted insertion of (d, key, idx) into the lane's ascending top-K list, if it ranks within it.
template <int K>
__device__ __forceinline__ void topk_insert(uint32_t (&bd)[K], uint32_t (&bk)[K], int (&bi)[K], uint32_t d,
                                            uint32_t key, int idx) {
  if (!before(d, key, bd[K - 1], bk[K - 1])) return;
#pragma unroll
  for (int x = K - 1; x > 0; --x) {
    const bool bp = before(d, key, bd[x - 1], bk[x - 1]);
    const bool bc = before(d, key, bd[x], bk[x]);
    bd[x] = bp ? bd[x - 1] : (bc ? d : bd[x]);
    bk[x] = bp ? bk[x - 1] : (bc ? key : bk[x]);
    bi[x] = bp ? bi[x - 1] : (bc ? idx : bi[x]);
  }
  if (before(d, key, bd[0], bk[0])) {
    bd[0] = d;
    bk[0] = key;
    bi[0] = idx;
  }
}

typedef short short2v __attribute__((ext_vector_type(2)));

// Squared lattice distance: x and y as packed 16-bit differences through one dot2, z in 24 bits
// (|difference| <= 8192 per axis, so every product and the sum are exact).
__device__ __forceinline__ uint32_t dist2(uint32_t uxy, int uz, int2 c) {
  const short2v d = __builtin_bit_cast(short2v, uxy) - __builtin_bit_cast(short2v, c.x);
  const int dz = uz - c.y;
  return (uint32_t)__builtin_amdgcn_sdot2(d, d, __mul24(dz, dz), false);
}

// One wave per query block (blk_cap <= 64: lane t is the block's slot t).  Exact candidate pruning
// with the lattice bounding box [lo, hi] of the block's valid points:
//   for any point u of the box and centroid c,  dmin(box, c) <= d2(u, c) <= dmax(box, c);
//   T = the k-th smallest, over the 64 lanes, of each lane's minimum dmax over its share of the
//       candidates: k distinct centroids lie within T of every point of the box, so every token's
//       k-th best d2 is <= T;
//   a centroid with dmin > T is then farther than T from every token and cannot enter any token's
//       top k (one with d2 == T still can, on blk_key, and is kept).
// The surviving candidates are gathered in LDS a chunk at a time, sorted nearest box first, and each
// lane ranks them into its register top-K list in the total (d2, blk_key) order, so the result is
// that of the full scan; with the nearest candidates seen first, the list's threshold settles early
// and few later candidates still enter it.
constexpr int PCH = 512;    // candidates per LDS chunk

// Continuous patch coordinate of a point along one image axis: ((A0 x + A1 y) + A2 z) + A3, every
// operation rounded to float32 in this order (no fused multiply-add), so the cell decision is
// reproducible bit for bit.
__device__ __forceinline__ float project_axis(const float* A, float x, float y, float z) {
#pragma clang fp contract(off)
  return ((A[0] * x + A[1] * y) + A[2] * z) + A[3];
}

// floor(x / 2^shift) through an exact integer floor; far-off values are clamped to +-2^30, which
// leaves their window outside every cell grid.
__device__ __forceinline__ int cell_of(float x, int shift) {
  const float f = fminf(fmaxf(floorf(x), -1073741824.0f), 1073741824.0f);
  return (int)f >> shift;
}

__device__ __forceinline__ uint32_t box_dmax(int x, int y, int z, const int (&lo)[3], const int (&hi)[3]) {
  const int ax = max(x - lo[0], hi[0] - x), ay = max(y - lo[1], hi[1] - y), az = max(z - lo[2], hi[2] - z);
  return (uint32_t)(ax * ax + ay * ay + az * az);
}

__device__ __forceinline__ uint32_t box_dmin(int x, int y, int z, const int (&lo)[3], const int (&hi)[3]) {
  const int ax = max(lo[0] - x, 0) + max(x - hi[0], 0);
  const int ay = max(lo[1] - y, 0) + max(y - hi[1], 0);
  const int az = max(lo[2] - z, 0) + max(z - hi[2], 0);
  return (uint32_t)(ax * ax + ay * ay + az * az);
}

template <int K>
__global__ __launch_bounds__(64) void route_kernel(RouteArgs a) {
  __shared__ int2 cs[PCH];        // (x | y << 16, z) of the chunk's surviving centroids
  __shared__ uint32_t ck[PCH];    // their blk_key
  __shared__ int ci[PCH];         // their block index
  __shared__ unsigned long long so[PCH];   // (dmin << 32 | position), sorted
  const int b = a.q_blk0 + blockIdx.x;
  const int l = threadIdx.x;
  const int cnt = a.blk_cnt[b];
  const bool in_blk = l < a.cap;
  const bool valid = l < cnt;
  const int slot = b * a.cap + l;
  int ux = 0, uy = 0, uz = 0;
  if (valid) {
    const float* p = a.pts + (size_t)slot * 3;
    ux = lattice(p[0]);
    uy = lattice(p[1]);
    uz = lattice(p[2]);
  }
  // the block's bounding box (valid lanes only; lane 0 is always valid)
  int lo[3] = {valid ? ux : 1 << 30, valid ? uy : 1 << 30, valid ? uz : 1 << 30};
  int hi[3] = {valid ? ux : -(1 << 30), valid ? uy : -(1 << 30), valid ? uz : -(1 << 30)};
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
#pragma unroll
    for (int ax = 0; ax < 3; ++ax) {
      lo[ax] = min(lo[ax], __shfl_xor(lo[ax], o, 64));
      hi[ax] = max(hi[ax], __shfl_xor(hi[ax], o, 64));
    }
  const int4* cent = reinterpret_cast<const int4*>(a.cent);
  // pass 1: the bound T (eight centroid loads in flight per lane, not one round trip per step)
  uint32_t lmin = 0xFFFFFFFFu;
  {
    int c = a.kv_lo + l;
    for (; c + 7 * 64 < a.kv_hi; c += 8 * 64) {
      int4 e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = cent[c + 64 * j];
#pragma unroll
      for (int j = 0; j < 8; ++j) lmin = min(lmin, box_dmax(e[j].x, e[j].y, e[j].z, lo, hi));
    }
    for (; c < a.kv_hi; c += 64) {
      const int4 e = cent[c];
      lmin = min(lmin, box_dmax(e.x, e.y, e.z, lo, hi));
    }
  }
  int rank = 0;
  for (int i = 0; i < 64; ++i) {
    const uint32_t v = (uint32_t)__shfl((int)lmin, i, 64);
    rank += (v < lmin || (v == lmin && i < l)) ? 1 : 0;
  }
  const unsigned long long at_k = __builtin_amdgcn_ballot_w64(rank == a.top_k - 1);
  const uint32_t T = (uint32_t)__shfl((int)lmin, __builtin_ctzll(at_k), 64);   // ranks are a permutation
  // pass 2: gather the survivors chunk by chunk and rank them
  const uint32_t uxy = (uint32_t)ux | ((uint32_t)uy << 16);
  uint32_t bd[K], bk[K];
  int bi[K];
#pragma unroll
  for (int x = 0; x < K; ++x) {
    bd[x] = 0xFFFFFFFFu;
    bk[x] = 0xFFFFFFFFu;
    bi[x] = -1;
  }
  int c = a.kv_lo;
  // the next step's centroid is loaded one step ahead (lanes past the end load the last one)
  int4 e_nx = make_int4(0, 0, 0, 0);
  if (a.kv_hi > a.kv_lo) e_nx = cent[min(c + l, a.kv_hi - 1)];
  while (c < a.kv_hi) {
    int n = 0;
    // fill the chunk: up to PCH survivors (64 centroids per step; stop before a step could overflow)
    for (; c < a.kv_hi && n + 64 <= PCH; c += 64) {
      const int cc = c + l;
      const int4 e = e_nx;
      e_nx = cent[min(cc + 64, a.kv_hi - 1)];
      const uint32_t dm = box_dmin(e.x, e.y, e.z, lo, hi);
      const bool keep = cc < a.kv_hi && dm <= T;
      const unsigned long long m = __builtin_amdgcn_ballot_w64(keep);
      if (keep) {
        const int pos = n + __builtin_popcountll(m & ((1ull << l) - 1ull));
        cs[pos] = make_int2(e.x | (e.y << 16), e.z);
        ck[pos] = (uint32_t)e.w;
        ci[pos] = cc;
        so[pos] = ((unsigned long long)dm << 32) | (unsigned)pos;
      }
      n += __builtin_popcountll(m);
    }
    // sort the survivors nearest box first (bitonic, padded to a power of two)
    int N = 64;
    while (N < n) N <<= 1;
    for (int i = n + l; i < N; i += 64) so[i] = ~0ull;
    __syncthreads();
    for (int size = 2; size <= N; size <<= 1)
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = l; i < N; i += 64) {
          const int j = i ^ stride;
          if (j > i) {
            const unsigned long long x0 = so[i], x1 = so[j];
            if ((x0 > x1) == ((i & size) == 0)) {
              so[i] = x1;
              so[j] = x0;
            }
          }
        }
        __syncthreads();
      }
    if (valid) {
      int i = 0;
      // filter on d2 alone, eight at a time; each lane then walks only its own candidates
      constexpr int GR = 8;
      for (; i + GR <= n; i += GR) {
        uint32_t d[GR];
        int q[GR];
#pragma unroll
        for (int x = 0; x < GR; ++x) {
          q[x] = (int)(unsigned)so[i + x];
          d[x] = dist2(uxy, uz, cs[q[x]]);
        }
        const uint32_t thr = bd[K - 1];
        uint32_t m = 0u;
#pragma unroll
        for (int x = 0; x < GR; ++x) m |= (d[x] <= thr) ? (1u << x) : 0u;
        while (m != 0u) {
          const int x = __builtin_ctz(m);
          m &= m - 1u;
          uint32_t dd = d[0];
          int p = q[0];
#pragma unroll
          for (int y = 1; y < GR; ++y) {
            dd = x == y ? d[y] : dd;
            p = x == y ? q[y] : p;
          }
          topk_insert<K>(bd, bk, bi, dd, ck[p], ci[p]);
        }
      }
      for (; i < n; ++i) {
        const int p = (int)(unsigned)so[i];
        topk_insert<K>(bd, bk, bi, dist2(uxy, uz, cs[p]), ck[p], ci[p]);
      }
    }
    __syncthreads();
  }
  // image blocks through the views: every view's projection cell and its window; a candidate's
  // metric is its nearest member's d2, computed only when the block's box could still beat the
  // lane's current k-th (d2 == k-th may still win on blk_key)
  if (a.n_views > 0 && valid) {
    const float* pp = a.pts + (size_t)slot * 3;
    const float px = pp[0], py = pp[1], pz = pp[2];
    const int4* box = reinterpret_cast<const int4*>(a.boxes);
    for (int v = 0; v < a.n_views; ++v) {
      const float* A = a.view_proj + 8 * v;
      const int cx = cell_of(project_axis(A, px, py, pz), a.cell_shift);
      const int cy = cell_of(project_axis(A + 4, px, py, pz), a.cell_shift);
      const int y0 = max(cy - a.radius, 0), y1 = min(cy + a.radius, a.n_cell - 1);
      const int x0 = max(cx - a.radius, 0), x1 = min(cx + a.radius, a.n_cell - 1);
      for (int y = y0; y <= y1; ++y)
        for (int x = x0; x <= x1; ++x) {
          const int bb = a.cell_blk[((size_t)v * a.n_cell + y) * a.n_cell + x];
          if (bb < 0 || bb >= a.n_blk) continue;
          const int4 blo = box[2 * bb], bhi = box[2 * bb + 1];
          const int lo3[3] = {blo.x, blo.y, blo.z}, hi3[3] = {bhi.x, bhi.y, bhi.z};
          if (box_dmin(ux, uy, uz, lo3, hi3) > bd[K - 1]) continue;
          uint32_t best = 0xFFFFFFFFu;
          const int mc = a.blk_cnt[bb];
          const int2* mp = reinterpret_cast<const int2*>(a.lat) + (size_t)bb * a.cap;
          int t = 0;
          for (; t + 8 <= mc; t += 8) {        // eight member loads in flight, then their d2
            int2 m[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) m[j] = mp[t + j];
#pragma unroll
            for (int j = 0; j < 8; ++j) best = min(best, dist2(uxy, uz, m[j]));
          }
          for (; t < mc; ++t) best = min(best, dist2(uxy, uz, mp[t]));
          topk_insert<K>(bd, bk, bi, best, a.blk_key[bb], bb);
        }
    }
  }
  if (in_blk) {
    int32_t* so = a.sel + (size_t)slot * a.top_k;
    uint32_t* dout = a.sel_d2 ? a.sel_d2 + (size_t)slot * a.top_k : nullptr;
#pragma unroll
    for (int x = 0; x < K; ++x) {
      if (x < a.top_k) {
        so[x] = valid ? bi[x] : -1;
        if (dout) dout[x] = valid ? bd[x] : 0xFFFFFFFFu;
      }
    }
  }
}

template <int K>
hipError_t launch_route_k(const RouteArgs& a, hipStream_t s) {
  if (a.n_qblk == 0) return hipSuccess;
  hipLaunchKernelGGL(route_kernel<K>, dim3(a.n_qblk), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_geometric(const RouteArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(centroid_kernel, dim3(a.n_blk), dim3(64), 0, s, a.pts, a.blk_cnt, a.blk_key, a.cent,
                     a.n_views > 0 ? a.boxes : nullptr, a.n_views > 0 ? a.lat : nullptr, a.cap);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.top_k <= 4) return launch_route_k<4>(a, s);
  if (a.top_k <= 8) return launch_route_k<8>(a, s);
  if (a.top_k <= 16) return launch_route_k<16>(a, s);
  if (a.top_k <= 32) return launch_route_k<32>(a, s);
  return launch_route_k<64>(a, s);
}

// ---------------------------------------------------------------------------------------------
// the routing centroids in a fixed device array, for callers that cannot allocate
// ---------------------------------------------------------------------------------------------

namespace {
// [kScratchMaxBlocks][4] int32 centroids (1 MiB), one copy per device for the life of the process
static __device__ __align__(256) int32_t scratch[kScratchMaxBlocks * 4];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t route_scratch_centroids(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // the array's device address on the current device: the host-side name is not one
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}


}  // namespace nsa
