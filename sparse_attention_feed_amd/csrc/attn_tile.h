// The per-token tile pass of the grouped-query attention kernels (one token's 16 query heads of a
// KV group against a 64-key tile held in registers): S^T = K Q^T on MFMA, the online softmax in
// base 2, and O^T += V^T P^T.  Shared by attn.hip and the microbenchmark in probe.hip.
#pragma once

#include "common.h"

namespace nsa {

// Online-softmax state of one token (16 heads of one KV group) held by one wave.
//
// Queries are pre-scaled by c2 = scale * log2(e) in fp32 and rounded once to the storage type, so
// S^T comes out in base-2 logit units (for bf16 this adds one rounding of relative size <= 2^-9
// per query element, the same order as the bf16 rounding of the probabilities).  The running
// maximum mc (base-2 units) starts at 0 and is allowed to go stale: it enters the QK^T product as
// the MFMA accumulator seed (-mc, together with -inf for padding keys), so exp2 reads the MFMA
// output directly.  The wave takes an exact path only when a lane's probability sum could exceed
// kStaleLimit (or is not finite), or when a head has no probability mass yet and the tile's sum is
// tiny; that path moves mc to the tile maximum and rescales.  Results equal the textbook online
// softmax up to rounding, every probability stays <= kStaleLimit, and no row underflows.
struct TokState {
  f32x4 acc[2];   // O^T: lane holds d = 16*dt + 4*(lane/16) + i for head lane%16
  float mc;       // running reference max (base-2 units) for head lane%16, same in all lane groups
  float l;        // this lane group's share of the running sum of probabilities
};

constexpr float kStaleLimit = 65536.0f;
constexpr float kTinyMass = 1.0e-30f;

__device__ __forceinline__ void tok_init(TokState& s) {
  s.acc[0] = (f32x4){0.f, 0.f, 0.f, 0.f};
  s.acc[1] = s.acc[0];
  s.mc = 0.f;
  s.l = 0.f;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Pre-scaled query fragment of one token: the MFMA B operand of S^T = K Q^T.
template <typename T> struct QF { Frag8<T> hi; };

// The lane's eight query elements as stored, and the fragment made from them (valid tokens) or
// zero: the loads of all of a wave's tokens are issued before any conversion, so they share one
// memory round trip.
__device__ __forceinline__ Frag8<bf16> load_q8(const bf16* p) {
  Frag8<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag8<float> load_q8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  Frag8<float> f;
  f.v = (f32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}
template <typename T> __device__ __forceinline__ QF<T> make_qf(const Frag8<T>& raw, float c2, bool valid) {
  QF<T> q;
#pragma unroll
  for (int e = 0; e < 8; ++e) q.hi.v[e] = valid ? (T)((float)raw.v[e] * c2) : (T)0.f;
  return q;
}

// p = exp2(x) for the lane's 16 base-2 logits, packed as the two B operands of the PV product;
// returns the lane's sum of the probabilities as rounded for that product.
template <typename T>
__device__ __forceinline__ float exp_pack(const f32x4 (&x)[4], Frag8<T> (&pf)[2]);

template <>
__device__ __forceinline__ float exp_pack<bf16>(const f32x4 (&x)[4], Frag8<bf16> (&pf)[2]) {
  float lt = 0.f;
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int kt = 2 * h + (e >> 2), i = e & 3;
      f32x2 p;
      p[0] = __builtin_amdgcn_exp2f(x[kt][i]);
      p[1] = __builtin_amdgcn_exp2f(x[kt][i + 1]);
      const bf16x2 pb = __builtin_convertvector(p, bf16x2);
      pf[h].v[e] = pb[0];
      pf[h].v[e + 1] = pb[1];
      lt = __builtin_amdgcn_fdot2_f32_bf16(pb, one, lt, false);
    }
  return lt;
}

template <>
__device__ __forceinline__ float exp_pack<float>(const f32x4 (&x)[4], Frag8<float> (&pf)[2]) {
  float lt = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kt = 2 * h + (e >> 2), i = e & 3;
      const float p = __builtin_amdgcn_exp2f(x[kt][i]);
      pf[h].v[e] = p;
      lt += p;
    }
  return lt;
}

__device__ __forceinline__ float lane_max16(const f32x4 (&s)[4]) {
  float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                   fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  return fmaxf(mx, fmaxf(fmaxf(fmaxf(s[2][0], s[2][1]), fmaxf(s[2][2], s[2][3])),
                         fmaxf(fmaxf(s[3][0], s[3][1]), fmaxf(s[3][2], s[3][3]))));
}

// Logits of one token against the tile, relative to its reference max: S^T = K Q^T + seed with
// seed = -mc on keys below nk and -inf on padding keys (cm holds 0 / -inf).
template <typename T>
__device__ __forceinline__ void tok_qk(const TokState& st, const QF<T>& qf, const Frag8<T> (&kf)[4],
                                       const f32x4 (&cm)[4], bool full, f32x4 (&x)[4]) {
  if (full) {
    const f32x4 seed = {-st.mc, -st.mc, -st.mc, -st.mc};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) x[kt] = mma16(kf[kt], qf.hi, seed);
  } else {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) x[kt] = mma16(kf[kt], qf.hi, cm[kt] - st.mc);
  }
}

template <typename T>
__device__ __forceinline__ void tok_softmax_pv(TokState& st, f32x4 (&x)[4], const Frag8<T> (&vf)[2][2]) {
  Frag8<T> pf[2];
  float lt = exp_pack<T>(x, pf);
  if (__builtin_amdgcn_ballot_w64(!(lt <= kStaleLimit) || !(st.l + lt >= kTinyMass)) != 0) {
    // exact path for every head of the token: move the reference max to the tile's maximum if it
    // is larger, or to it outright while the head has no mass yet; rescale and redo
    const float xm = wave_max_across_rows(lane_max16(x));
    const float lh = wave_sum_across_rows(st.l);
    float shift = lh > 0.f ? fmaxf(xm, 0.f) : xm;
    if (!(shift > -INFINITY)) shift = 0.f;         // no valid key for this lane's head
    if (lh > 0.f && shift > 0.f) {
      const float alpha = __builtin_amdgcn_exp2f(-shift);
      st.l *= alpha;
      st.acc[0] *= alpha;
      st.acc[1] *= alpha;
    }
    st.mc += shift;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) x[kt] -= shift;
    lt = exp_pack<T>(x, pf);
  }
  st.l += lt;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int h = 0; h < 2; ++h) st.acc[dt] = mma16(vf[dt][h], pf[h], st.acc[dt]);
}

// Tokens t < n (a prefix of the wave's tokens) against one tile, one token at a time (the other
// wave on the SIMD covers the wait for each token's QK^T results; a software pipeline across
// tokens costs more in register copies than it saves at this register budget).
template <typename T, int TPW>
__device__ __forceinline__ void tile_prefix(TokState (&st)[TPW], const QF<T> (&qf)[TPW], int n, const Frag8<T> (&kf)[4],
                                            const Frag8<T> (&vf)[2][2], const f32x4 (&cm)[4], bool full) {
  n = __builtin_amdgcn_readfirstlane(n);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    if (t < n) {
      f32x4 x[4];
      tok_qk<T>(st[t], qf[t], kf, cm, full, x);
      tok_softmax_pv<T>(st[t], x, vf);
    }
  }
}

// Tokens named by a mask (selected branch).
template <typename T, int TPW>
__device__ __forceinline__ void tile_masked(TokState (&st)[TPW], const QF<T> (&qf)[TPW], uint32_t pm,
                                            const Frag8<T> (&kf)[4], const Frag8<T> (&vf)[2][2],
                                            const f32x4 (&cm)[4], bool full) {
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    if (pm & (1u << t)) {
      f32x4 x[4];
      tok_qk<T>(st[t], qf[t], kf, cm, full, x);
      tok_softmax_pv<T>(st[t], x, vf);
    }
  }
}


}  // namespace nsa
