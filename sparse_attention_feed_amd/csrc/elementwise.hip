// HBM-bound passes: block mean pooling and the standalone sigmoid-gated combine.
#include "common.h"
#include "kernels.h"

namespace nsa {
namespace {

// Block compression (LSRM pages, section 方法, eq. k^cmp = AvgPool(ResBlock(k)), ResBlock = identity;
// Speed3R page, section 2.1, average pooling).  One thread per (block, 16-byte piece of the row):
// it reads that piece of each valid token (one coalesced 16-byte load per token, four in flight)
// and accumulates in fp32 in token order.
template <typename T>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ x, T* __restrict__ xc,
                                                   const int32_t* __restrict__ blk_cnt, int n_blk, int cap,
                                                   int row) {
  constexpr int VEC = 16 / sizeof(T);
  const int pieces = row / VEC;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)n_blk * pieces) return;
  const int b = (int)(i / pieces), pc = (int)(i % pieces);
  const int cnt = blk_cnt[b];
  const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)b * cap * row + pc * VEC);
  const size_t step = (size_t)row / VEC;      // uint4 per token row
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  int t = 0;
  for (; t + 4 <= cnt; t += 4) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = src[(size_t)(t + u) * step];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const T* e = reinterpret_cast<const T*>(&v[u]);
#pragma unroll
      for (int k = 0; k < VEC; ++k) acc[k] += to_f32(e[k]);
    }
  }
  for (; t < cnt; ++t) {
    const uint4 v = src[(size_t)t * step];
    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[k] += to_f32(e[k]);
  }
  uint4 out;
  T* oe = reinterpret_cast<T*>(&out);
#pragma unroll
  for (int k = 0; k < VEC; ++k) oe[k] = from_f32<T>(acc[k] / (float)cnt);
  *reinterpret_cast<uint4*>(xc + (size_t)b * row + pc * VEC) = out;
}

struct BranchPtrs {
  const void* p[8];
};

// o = sum_c sigmoid(g_c) o_c (LSRM pages, Sigmoid gates; Speed3R page, gated aggregation).
// One thread per (row, head, 4 consecutive dims): one vector load per branch, one vector store.
template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };

template <typename T>
__global__ void gate_kernel(BranchPtrs br, int n_branch, const T* __restrict__ gates, T* __restrict__ o,
                            long long n_vec, int n_qh, int head_dim) {
  typedef typename Vec4<T>::type V4;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_vec) return;
  const long long e0 = i * 4;
  const long long rh = e0 / head_dim;          // row * n_qh + head
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < n_branch; ++c) {
    const float wgt = sigmoidf_(to_f32(gates[rh * n_branch + c]));
    const V4 v = reinterpret_cast<const V4*>(br.p[c])[i];
#pragma unroll
    for (int x = 0; x < 4; ++x) acc[x] += wgt * to_f32(v[x]);
  }
  V4 out;
#pragma unroll
  for (int x = 0; x < 4; ++x) out[x] = from_f32<T>(acc[x]);
  reinterpret_cast<V4*>(o)[i] = out;
}

}  // namespace

hipError_t launch_pool(int is_bf16, const void* x, void* x_cmp, const int32_t* blk_cnt, int n_blk,
                       int cap, int n_heads, int head_dim, hipStream_t s) {
  const int row = n_heads * head_dim;
  const int vec = is_bf16 ? 8 : 4;
  if (row % vec != 0) return hipErrorInvalidValue;
  const long long n = (long long)n_blk * (row / vec);
  const unsigned nb = (unsigned)((n + 255) / 256);
  if (is_bf16)
    hipLaunchKernelGGL(pool_kernel<bf16>, dim3(nb), dim3(256), 0, s, (const bf16*)x, (bf16*)x_cmp,
                       blk_cnt, n_blk, cap, row);
  else
    hipLaunchKernelGGL(pool_kernel<float>, dim3(nb), dim3(256), 0, s, (const float*)x, (float*)x_cmp,
                       blk_cnt, n_blk, cap, row);
  return hipGetLastError();
}

hipError_t launch_gate(int is_bf16, int n_rows, int n_qh, int head_dim, int n_branch,
                       const void* const* o_branch, const void* gates, void* o, hipStream_t s) {
  BranchPtrs br;
  for (int c = 0; c < 8; ++c) br.p[c] = c < n_branch ? o_branch[c] : nullptr;
  const long long n_vec = (long long)n_rows * n_qh * head_dim / 4;
  const int nt = 256;
  const unsigned nb = (unsigned)((n_vec + nt - 1) / nt);
  if (is_bf16)
    hipLaunchKernelGGL(gate_kernel<bf16>, dim3(nb), dim3(nt), 0, s, br, n_branch, (const bf16*)gates,
                       (bf16*)o, n_vec, n_qh, head_dim);
  else
    hipLaunchKernelGGL(gate_kernel<float>, dim3(nb), dim3(nt), 0, s, br, n_branch, (const float*)gates,
                       (float*)o, n_vec, n_qh, head_dim);
  return hipGetLastError();
}

}  // namespace nsa
