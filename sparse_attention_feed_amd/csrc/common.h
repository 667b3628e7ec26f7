// Shared device-side helpers for the libnsa kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// Eight consecutive elements a lane feeds to one 16x16 MFMA step: one 16x16x32 bf16 instruction
// (k = 8*(lane/16) + e), or eight 16x16x4 f32 instructions (instruction e uses element e).
template <typename T> struct Frag8;
template <> struct Frag8<bf16> { bf16x8 v; };
template <> struct Frag8<float> { f32x8 v; };

__device__ __forceinline__ f32x4 mma16(const Frag8<bf16>& a, const Frag8<bf16>& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const Frag8<float>& a, const Frag8<float>& b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
  return c;
}

// 16-byte and 32-byte vector loads of eight elements.
__device__ __forceinline__ Frag8<bf16> load_frag(const bf16* p) {
  Frag8<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag8<float> load_frag(const float* p) {
  Frag8<float> f;
  f.v = *reinterpret_cast<const f32x8*>(p);
  return f;
}

__device__ __forceinline__ float wave_max_across_rows(float x) {
  // lanes l, l^16, l^32, l^48 hold the same column; reduce across the four 16-lane rows
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}
__device__ __forceinline__ float wave_sum_across_rows(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Map a linear workgroup id so that consecutive logical tiles land on the same XCD (workgroups are
// dispatched round-robin over the 8 XCDs, each with its own L2).
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  const int nx = 8;
  int per = nwg / nx;
  int rem = nwg % nx;
  int x = bid % nx;
  int i = bid / nx;
  // XCD x owns logical ids [start(x), start(x) + per + (x < rem))
  int start = x * per + (x < rem ? x : rem);
  return start + i;
}

}  // namespace nsa
