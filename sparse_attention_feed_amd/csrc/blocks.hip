// Volume token selection and the volume block table on the device (LSRM pages, hyper.ai summary of
// arXiv 2604.05182, section 方法: eq. M^vol selects the voxels near or crossed by the surface from
// the SDF at 4^3 sub-sample points; active tokens are grouped into spatial blocks).
//
// The SDF is given on a G^3 lattice over [-1, 1]^3 and read by trilinear interpolation.  Every
// operation of the activity decision is a single rounded fp32 operation in a fixed order (no
// contraction into fused multiply-adds), so the decision is reproducible bit for bit.
#include "common.h"
#include "kernels.h"

namespace nsa {
namespace {

// Compact every third bit of a Morton code (x: shift 0, y: shift 1, z: shift 2).
__device__ __forceinline__ int compact3(uint32_t m, int shift) {
  int v = 0;
#pragma unroll
  for (int b = 0; b < 10; ++b) v |= (int)((m >> (3 * b + shift)) & 1u) << b;
  return v;
}

// a + t (b - a) with every operation rounded (contraction into a fused multiply-add is disabled).
__device__ __forceinline__ float lerp_rn(float a, float b, float t) {
#pragma clang fp contract(off)
  return a + t * (b - a);
}

// Lattice cell and fraction of sub-sample m along one axis: u = (2m + 1)(G - 1) / (8N).
__device__ __forceinline__ void axis_coord(int m, int G, int N, int& g0, float& f) {
  const float u = (float)((2 * m + 1) * (G - 1)) / (float)(8 * N);    // correctly rounded division
  g0 = min((int)floorf(u), G - 2);
  f = u - (float)g0;                                                  // exact
}

// One wave per 4^3 cell (cells in Morton order); lane l is the voxel at local Morton position l.
__global__ __launch_bounds__(64) void activity_kernel(const float* __restrict__ sdf, int G, int N, float tau,
                                                      unsigned long long* __restrict__ cell_mask) {
  const uint32_t mc = blockIdx.x;
  const int l = threadIdx.x;
  const int i = 4 * compact3(mc, 0) + compact3((uint32_t)l, 0);
  const int j = 4 * compact3(mc, 1) + compact3((uint32_t)l, 1);
  const int k = 4 * compact3(mc, 2) + compact3((uint32_t)l, 2);
  int gx[4], gy[4], gz[4];
  float fx[4], fy[4], fz[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    axis_coord(4 * i + a, G, N, gx[a], fx[a]);
    axis_coord(4 * j + a, G, N, gy[a], fy[a]);
    axis_coord(4 * k + a, G, N, gz[a], fz[a]);
  }
  const size_t sy = (size_t)G, sz = (size_t)G * G;
  float mn = INFINITY, mx = -INFINITY, mabs = INFINITY;
  if (gx[0] == gx[3] && gy[0] == gy[3] && gz[0] == gz[3]) {
    // all 64 sub-samples in one lattice cell (the usual case when the lattice is no finer than the
    // voxels): its eight corners once, the same operations on the same values as below
    const float* p = sdf + gz[0] * sz + gy[0] * sy + gx[0];
    const float c000 = p[0], c001 = p[1], c010 = p[sy], c011 = p[sy + 1];
    const float c100 = p[sz], c101 = p[sz + 1], c110 = p[sz + sy], c111 = p[sz + sy + 1];
    for (int c = 0; c < 4; ++c)
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float s = lerp_rn(lerp_rn(lerp_rn(c000, c001, fx[a]), lerp_rn(c010, c011, fx[a]), fy[b]),
                                  lerp_rn(lerp_rn(c100, c101, fx[a]), lerp_rn(c110, c111, fx[a]), fy[b]), fz[c]);
          mn = fminf(mn, s);
          mx = fmaxf(mx, s);
          mabs = fminf(mabs, fabsf(s));
        }
  } else {
    for (int c = 0; c < 4; ++c)
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float* p = sdf + gz[c] * sz + gy[b] * sy + gx[a];
          const float s = lerp_rn(lerp_rn(lerp_rn(p[0], p[1], fx[a]), lerp_rn(p[sy], p[sy + 1], fx[a]), fy[b]),
                                  lerp_rn(lerp_rn(p[sz], p[sz + 1], fx[a]), lerp_rn(p[sz + sy], p[sz + sy + 1], fx[a]),
                                          fy[b]),
                                  fz[c]);
          mn = fminf(mn, s);
          mx = fmaxf(mx, s);
          mabs = fminf(mabs, fabsf(s));
        }
  }
  const bool active = mabs <= tau || mn * mx <= 0.f;
  const unsigned long long bits = __builtin_amdgcn_ballot_w64(active);
  if (l == 0) cell_mask[mc] = bits;
}

// Block index of every non-empty cell (exclusive prefix count in Morton order; -1 when empty) and
// the number of blocks.  One workgroup; thread t owns a contiguous range of cells.
constexpr int SCAN_T = 1024;

__global__ __launch_bounds__(SCAN_T) void block_scan_kernel(const unsigned long long* __restrict__ cell_mask,
                                                           int n_cells, int* __restrict__ cell_block,
                                                           int* __restrict__ n_blk) {
  __shared__ int part[SCAN_T / 64];
  const int t = threadIdx.x, l = lane_id(), w = t >> 6;
  const int per = (n_cells + SCAN_T - 1) / SCAN_T;
  const int lo = min(n_cells, t * per), hi = min(n_cells, lo + per);
  int mine = 0;
  for (int c = lo; c < hi; ++c) mine += cell_mask[c] != 0ull;
  int inc = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, 64);
    if (l >= o) inc += y;
  }
  if (l == 63) part[w] = inc;
  __syncthreads();
  int base = 0, total = 0;
  for (int x = 0; x < SCAN_T / 64; ++x) {
    if (x < w) base += part[x];
    total += part[x];
  }
  int next = base + inc - mine;
  for (int c = lo; c < hi; ++c) cell_block[c] = cell_mask[c] != 0ull ? next++ : -1;
  if (t == 0) *n_blk = total;
}

// Counts, keys and token points of the blocks (one wave per cell); blocks at or beyond max_blk are
// not written.
__global__ __launch_bounds__(64) void block_fill_kernel(const unsigned long long* __restrict__ cell_mask,
                                                       const int* __restrict__ cell_block, int N, int max_blk,
                                                       int32_t* __restrict__ blk_cnt, uint32_t* __restrict__ blk_key,
                                                       float* __restrict__ pts) {
  const uint32_t mc = blockIdx.x;
  const int b = cell_block[mc];
  if (b < 0 || b >= max_blk) return;
  const int l = threadIdx.x;
  const unsigned long long m = cell_mask[mc];
  const int cnt = __builtin_popcountll(m);
  float* out = pts + (size_t)b * 64 * 3;
  if ((m >> l) & 1ull) {
    const int r = __builtin_popcountll(m & ((1ull << l) - 1ull));
    const int i = 4 * compact3(mc, 0) + compact3((uint32_t)l, 0);
    const int j = 4 * compact3(mc, 1) + compact3((uint32_t)l, 1);
    const int k = 4 * compact3(mc, 2) + compact3((uint32_t)l, 2);
    out[r * 3 + 0] = (float)(2 * i + 1 - N) / (float)N;
    out[r * 3 + 1] = (float)(2 * j + 1 - N) / (float)N;
    out[r * 3 + 2] = (float)(2 * k + 1 - N) / (float)N;
  }
  if (l >= cnt) {
    out[l * 3 + 0] = 0.f;
    out[l * 3 + 1] = 0.f;
    out[l * 3 + 2] = 0.f;
  }
  if (l == 0) {
    blk_cnt[b] = cnt;
    blk_key[b] = mc;
  }
}

}  // namespace

hipError_t launch_build_volume_blocks(const float* sdf, int G, int N, float tau, int max_blk,
                                      unsigned long long* cell_mask, int* cell_block, int* n_blk, int32_t* blk_cnt,
                                      uint32_t* blk_key, float* pts, hipStream_t s) {
  const int n_cells = (N / 4) * (N / 4) * (N / 4);
  hipLaunchKernelGGL(activity_kernel, dim3(n_cells), dim3(64), 0, s, sdf, G, N, tau, cell_mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(block_scan_kernel, dim3(1), dim3(SCAN_T), 0, s, cell_mask, n_cells, cell_block, n_blk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(block_fill_kernel, dim3(n_cells), dim3(64), 0, s, cell_mask, cell_block, N, max_blk, blk_cnt,
                     blk_key, pts);
  return hipGetLastError();
}

}  // namespace nsa
