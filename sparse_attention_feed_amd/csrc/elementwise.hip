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

// Block compression with the residual module (LSRM pages, section 方法, eq.
// k^cmp = AvgPool(ResBlock(k_t))): ResBlock(x) = x + W2 silu(W1 x + b1) + b2 per head, then the mean
// over the block's valid tokens.  One workgroup per (block, head): the head's weights and the
// block's rows are staged in LDS as fp32 (rows padded to D + 1 floats against bank conflicts);
// one thread per (token, unit) computes the hidden layer, then the output in place; the mean adds
// the tokens in order.
template <typename T>
__global__ __launch_bounds__(256) void pool_resblock_kernel(const T* __restrict__ x, T* __restrict__ xc,
                                                            const int32_t* __restrict__ blk_cnt,
                                                            const float* __restrict__ w1, const float* __restrict__ b1,
                                                            const float* __restrict__ w2, const float* __restrict__ b2,
                                                            int cap, int n_heads, int D) {
  extern __shared__ float sm[];
  const int Dp = D + 1;
  float* W1 = sm;                 // [D][Dp]
  float* W2 = W1 + D * Dp;        // [D][Dp]
  float* X = W2 + D * Dp;         // [cap][Dp]: token rows, then the module's outputs
  float* Hd = X + cap * Dp;       // [cap][Dp]: hidden layer
  const int b = blockIdx.x / n_heads, h = blockIdx.x % n_heads;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int cnt = blk_cnt[b];
  const float* w1h = w1 + (size_t)h * D * D;
  const float* w2h = w2 + (size_t)h * D * D;
  for (int i = tid; i < D * D; i += nt) {
    W1[(i / D) * Dp + i % D] = w1h[i];
    W2[(i / D) * Dp + i % D] = w2h[i];
  }
  for (int i = tid; i < cnt * D; i += nt) {
    const int t = i / D, d = i % D;
    X[t * Dp + d] = to_f32(x[((size_t)(b * cap + t) * n_heads + h) * D + d]);
  }
  __syncthreads();
  for (int i = tid; i < cnt * D; i += nt) {
    const int t = i / D, j = i % D;
    float a = b1[h * D + j];
    for (int k = 0; k < D; ++k) a += W1[j * Dp + k] * X[t * Dp + k];
    Hd[t * Dp + j] = a / (1.f + __builtin_amdgcn_exp2f(-a * kLog2e));     // silu(a)
  }
  __syncthreads();
  for (int i = tid; i < cnt * D; i += nt) {
    const int t = i / D, d = i % D;
    float y = X[t * Dp + d] + b2[h * D + d];
    for (int j = 0; j < D; ++j) y += W2[d * Dp + j] * Hd[t * Dp + j];
    X[t * Dp + d] = y;            // only this thread reads or writes element (t, d) in this pass
  }
  __syncthreads();
  for (int d = tid; d < D; d += nt) {
    float s = 0.f;
    for (int t = 0; t < cnt; ++t) s += X[t * Dp + d];
    xc[((size_t)b * n_heads + h) * D + d] = from_f32<T>(s / (float)cnt);
  }
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

size_t pool_resblock_lds_bytes(int cap, int head_dim) {
  return (size_t)(2 * head_dim + 2 * cap) * (head_dim + 1) * sizeof(float);
}

hipError_t launch_pool_resblock(int is_bf16, const void* x, void* x_cmp, const int32_t* blk_cnt, const float* w1,
                                const float* b1, const float* w2, const float* b2, int n_blk, int cap,
                                int n_heads, int head_dim, hipStream_t s) {
  const size_t lds = pool_resblock_lds_bytes(cap, head_dim);
  const dim3 grid((unsigned)n_blk * (unsigned)n_heads);
  if (is_bf16) {
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&pool_resblock_kernel<bf16>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(pool_resblock_kernel<bf16>, grid, dim3(256), lds, s, (const bf16*)x, (bf16*)x_cmp, blk_cnt,
                       w1, b1, w2, b2, cap, n_heads, head_dim);
  } else {
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&pool_resblock_kernel<float>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(pool_resblock_kernel<float>, grid, dim3(256), lds, s, (const float*)x, (float*)x_cmp,
                       blk_cnt, w1, b1, w2, b2, cap, n_heads, head_dim);
  }
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
