// Microbenchmarks of the instruction rates that bound the grouped-query attention tile pass on
// gfx950 (measurement only; built into libnsa_probe.so, not part of libnsa).  Each kernel runs one
// workgroup per compute unit with 4 * k waves (k waves per SIMD; every workgroup reserves 96 KiB of
// LDS, so no compute unit hosts two); every wave times its own loop with the shader clock and
// writes the cycle count and a sink value (so nothing is optimised away).
//
//   0 exp     8 independent chains of v_exp_f32 per lane
//   1 mfma    4 independent accumulators of v_mfma_f32_16x16x32_bf16
//   2 mix     per iteration 8 MFMAs (as above) and 16 v_exp_f32 (as above), interleaved
//   3 fma     8 independent chains of v_fma_f32
//   4 mixfma  per iteration 8 MFMAs and 32 v_fma_f32
//   5 tile    the attention kernel's own token pass (attn_tile.h): 8 tokens against a 64-key tile
//             held in registers, one tile per iteration (8 x 131,072 FLOP per wave and iteration)
#include "attn_tile.h"
#include "common.h"

namespace nsa {
namespace {

// Makes the compiler forget a register's value (no instruction), so that loop-invariant work is
// not hoisted out of the timed loop.
template <typename V> __device__ __forceinline__ void launder(V& v) { asm volatile("" : "+v"(v)); }

template <int MAXT>
__global__ __launch_bounds__(MAXT) void probe_kernel(int which, int iters, float* sink, long long* cyc) {
  const int l = lane_id();
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  float acc_out = 0.f;
  long long t0 = 0, t1 = 0;
  if (which == 0 || which == 3) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 0.5f + 0.001f * (float)(l + i);
    t0 = clock64();
    if (which == 0) {
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);   // stays in (0.5, 0.71)
    } else {
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(x[i], 0.999f, 0.0005f);
    }
    t1 = clock64();
#pragma unroll
    for (int i = 0; i < 8; ++i) acc_out += x[i];
  } else if (which == 1 || which == 2 || which == 4) {
    Frag8<bf16> a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a.v[e] = (bf16)(0.01f * (float)((l + e) & 7));
      b.v[e] = (bf16)(0.02f * (float)((l * 3 + e) & 7));
    }
    f32x4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 0.5f + 0.001f * (float)(l + i);
    t0 = clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int rnd = 0; rnd < 2; ++rnd) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = mma16(a, b, acc[j]);
        if (which == 2) {
#pragma unroll
          for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
        } else if (which == 4) {
#pragma unroll
          for (int rep = 0; rep < 2; ++rep)
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(x[i], 0.999f, 0.0005f);
        }
      }
    }
    t1 = clock64();
#pragma unroll
    for (int j = 0; j < 4; ++j) acc_out += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc_out += x[i];
  } else if constexpr (MAXT <= 512) {
    constexpr int TPW = 8;
    TokState st[TPW];
    QF<bf16> qf[TPW];
    Frag8<bf16> kf[4], vf[2][2];
    f32x4 cm[4];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      tok_init(st[t]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[t].hi.v[e] = (bf16)(0.05f * (float)(((l + 5 * t + e) & 15) - 8));
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[kt].v[e] = (bf16)(0.05f * (float)(((l * 7 + kt + e) & 15) - 8));
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[dt][h].v[e] = (bf16)(0.1f * (float)(((l + dt * 3 + h + e) & 7) - 4));
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) cm[kt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    t0 = clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) launder(kf[kt].v);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int h = 0; h < 2; ++h) launder(vf[dt][h].v);
      tile_prefix<bf16, TPW>(st, qf, TPW, kf, vf, cm, true);
    }
    t1 = clock64();
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc_out += st[t].acc[0][0] + st[t].acc[1][0] + st[t].l;
  }
  extern __shared__ float reserve[];      // never touched: only keeps a second workgroup off the CU
  if (acc_out == 12345.f && iters < 0) reserve[threadIdx.x] = acc_out;
  sink[blockIdx.x * blockDim.x + threadIdx.x] = acc_out;
  if (l == 0) cyc[wave] = t1 - t0;
}

// Lane layout of gfx950's transposing LDS read (ds_read_b64_tr_b16), which the selected-branch
// kernels use for their V^T fragments: LDS holds lds[i] = i (4096 16-bit values); with pattern 0 lane
// l names elements 4l .. 4l+3, with pattern 1 elements 64 (l % 16) + 4 (l / 16) .. + 3 (every
// address inside the 8 KiB array); out[64 * 4 * pattern + 4 l + e] = element e of lane l's result.
__global__ __launch_bounds__(64) void lds_tr_layout_kernel(short* out) {
  __shared__ short lds[64 * 64];
  for (int i = threadIdx.x; i < 64 * 64; i += 64) lds[i] = (short)i;
  __syncthreads();
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const int l = threadIdx.x;
#pragma unroll
  for (int pattern = 0; pattern < 2; ++pattern) {
    const int elem = pattern == 0 ? 4 * l : 64 * (l % 16) + 4 * (l / 16);
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3)))*)(reinterpret_cast<s16x4*>(lds + elem)));
#pragma unroll
    for (int e = 0; e < 4; ++e) out[256 * pattern + 4 * l + e] = r[e];
  }
}

}  // namespace
}  // namespace nsa

// The transposing LDS read's lane layout (lds_tr_layout_kernel): out holds 512 int16.
extern "C" int nsa_probe_lds_tr_layout(short* out, hipStream_t stream) {
  if (out == nullptr) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(nsa::lds_tr_layout_kernel, dim3(1), dim3(64), 0, stream, out);
  return (int)hipGetLastError();
}

// Runs probe `which` with `waves_per_simd` waves on each SIMD of `n_cu` compute units, `iters`
// loop iterations.  sink: n_cu * 256 * waves_per_simd floats; cycles: n_cu * 4 * waves_per_simd
// int64 (per wave: shader-clock cycles of its timed loop).  Returns a hipError_t code.
extern "C" int nsa_probe_run(int which, int waves_per_simd, int n_cu, int iters, float* sink, long long* cycles,
                             hipStream_t stream) {
  if (which < 0 || which > 5 || waves_per_simd < 1 || waves_per_simd > 4 || n_cu < 1 || iters < 1)
    return (int)hipErrorInvalidValue;
  const size_t lds = 96 * 1024;          // one workgroup per compute unit
  if (which == 5) {   // the tile pass needs the register budget of two waves per SIMD
    if (waves_per_simd > 2) return (int)hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&nsa::probe_kernel<512>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(nsa::probe_kernel<512>, dim3(n_cu), dim3(256 * waves_per_simd), lds, stream, which, iters,
                       sink, cycles);
  } else {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&nsa::probe_kernel<1024>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(nsa::probe_kernel<1024>, dim3(n_cu), dim3(256 * waves_per_simd), lds, stream, which, iters,
                       sink, cycles);
  }
  return (int)hipGetLastError();
}
