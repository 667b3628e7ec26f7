// Score routing in grouped-query form ("standard NSA" selection that the LSRM pages compare with:
// hyper.ai summary of arXiv 2604.05182, section 方法, routing paragraph; Speed3R page, section 2.1,
// top-k from the compressed scores without storing them).  For a query token and KV group j the
// importance of pooled block b is the group's summed softmax probability
//     imp(b) = sum over the 16 heads h of group j of exp(scale <q_h, k_cmp[b][j]> - lse_h),
// with lse the compressed branch's log-partition function; each token keeps the top_k blocks by
// (importance descending, blk_key ascending).
//
// Work decomposition: one workgroup per (query block, KV group), 8 waves x 8 tokens, as the fused
// attention kernel.  With pooled query rows (one per block) the rows are taken 64 at a time in
// storage order instead.  Tiles of 64 pooled keys are staged once in LDS and serve all 64 tokens.
// Per (token, tile), with S = Q K^T on v_mfma_f32_16x16x32 (A = the token's 16 pre-scaled query
// rows, B = 16 keys): lane (r, g) gets heads 4g..4g+3 of key 16 kt + r, and the accumulator seed
// -lse_h log2(e) makes the MFMA output the exponent itself.  The head sum is three adds in the lane
// and a two-step reduce-scatter across the four lane groups, after which lane (r, g) holds the
// importance of key 16 g + r of the tile.
//
// Top-k without a score matrix: every token has a candidate buffer in LDS.  A key enters it when its
// importance reaches the token's threshold (the k-th best importance among the kept candidates, 0
// at first); when the buffer could overflow on the next tile, it is compacted to exactly the top_k
// candidates under the (importance, blk_key) order, found by a bisection on the importance bits
// (and on the keys among exact ties), and the threshold moves up.  At the end the kept candidates
// are ranked by the same order.  The result is the exact top_k of all blocks for the importances as
// computed.
#include "common.h"
#include "kernels.h"

namespace nsa {
namespace {

constexpr int RT = 64;                       // pooled keys per tile
constexpr int RHD = 32;                      // head dim
constexpr int RGRP = 16;                     // query heads per KV head
constexpr int RWAVES = 8, RTPW = 8;          // 64 token slots per workgroup
// candidate slots per token: 128, or 256 when top_k > 32 (fewer compactions of the longer lists)
__host__ __device__ constexpr int rcap_for(int top_k) { return top_k <= 32 ? 128 : 256; }
// The pre-scaled query q * scale * log2(e) as a sum of two bf16 parts (hi + lo, two MFMAs per key
// step): the rounding of one part alone would move every logit by up to 2^-9 of its size.
constexpr bool kSplitQuery = true;

template <typename T> struct RPad;           // LDS row stride of a key tile (elements)
template <> struct RPad<bf16> { static constexpr int K = 40; };
template <> struct RPad<float> { static constexpr int K = 36; };

template <typename T> struct RTile { T k[RT][RPad<T>::K]; };

struct Cand {
  float v;      // importance (>= 0)
  int idx;      // storage block index
};

// Staging of one key tile: chunk c = tid of the tile's 16-byte pieces (rows past n_blk repeat the
// last block; those keys never become candidates).
template <typename T> struct RStager {
  static constexpr int E = 16 / sizeof(T), CPR = RHD / E, CH = RT * CPR;
  uint4 r;
  __device__ __forceinline__ void load(const T* base, int stride, int k0, int n_blk) {
    const int c = threadIdx.x;
    if (c < CH) {
      const int key = min(k0 + c / CPR, n_blk - 1), part = c % CPR;
      r = *reinterpret_cast<const uint4*>(base + (size_t)key * stride + part * E);
    }
  }
  __device__ __forceinline__ void store(RTile<T>& t) const {
    const int c = threadIdx.x;
    if (c < CH) *reinterpret_cast<uint4*>(&t.k[c / CPR][(c % CPR) * E]) = r;
  }
};

__device__ __forceinline__ int wave_count(bool p) { return __builtin_popcountll(__builtin_amdgcn_ballot_w64(p)); }

// Candidate buffer of one token, compacted by the whole wave to the best `keep` entries under the
// (importance descending, blk_key ascending) order; returns the importance of the worst kept entry
// (the new threshold).  keep < n <= 64 * NE on entry; lane l holds entries l + 64 e.
template <int NE>
__device__ __forceinline__ float compact(Cand* c, int& n, int keep, const uint32_t* __restrict__ blk_key) {
  const int l = lane_id();
  Cand e[NE];
  uint32_t bb[NE];
  bool h[NE];
#pragma unroll
  for (int x = 0; x < NE; ++x) {
    e[x] = l + 64 * x < n ? c[l + 64 * x] : Cand{-1.f, -1};
    h[x] = e[x].v >= 0.f;
    bb[x] = h[x] ? __float_as_uint(e[x].v) : 0u;
  }
  auto count = [&](auto pred) {
    int s = 0;
#pragma unroll
    for (int x = 0; x < NE; ++x) s += wave_count(pred(x));
    return s;
  };
  // the keep-th largest importance: the largest bit pattern T with at least `keep` entries >= T
  // (non-negative floats order as their bits; empty entries are -1)
  uint32_t lo = 0u, hi = 0x7F800000u;
  while (lo < hi) {
    const uint32_t mid = lo + (hi - lo + 1u) / 2u;
    if (count([&](int x) { return h[x] && bb[x] >= mid; }) >= keep) lo = mid;
    else hi = mid - 1u;
  }
  const float th = __uint_as_float(lo);
  const int n_gt = count([&](int x) { return h[x] && e[x].v > th; });
  const int need = keep - n_gt;                 // >= 1 ties at th to keep, by smallest blk_key
  const int n_eq = count([&](int x) { return h[x] && e[x].v == th; });
  bool kp[NE];
#pragma unroll
  for (int x = 0; x < NE; ++x) kp[x] = h[x] && e[x].v > th;
  if (n_eq <= need) {
#pragma unroll
    for (int x = 0; x < NE; ++x) kp[x] = kp[x] || (h[x] && e[x].v == th);
  } else {
    // the need-th smallest key among the ties: the smallest X with at least `need` tie keys <= X
    uint32_t key[NE];
#pragma unroll
    for (int x = 0; x < NE; ++x) key[x] = (h[x] && e[x].v == th) ? blk_key[e[x].idx] : 0xFFFFFFFFu;
    uint32_t klo = 0u, khi = 0xFFFFFFFFu;
    while (klo < khi) {
      const uint32_t mid = klo + (khi - klo) / 2u;
      if (count([&](int x) { return h[x] && e[x].v == th && key[x] <= mid; }) >= need) khi = mid;
      else klo = mid + 1u;
    }
#pragma unroll
    for (int x = 0; x < NE; ++x) kp[x] = kp[x] || (h[x] && e[x].v == th && key[x] <= klo);
  }
  // write the kept entries to the front (all reads above are done: the values are in registers)
  __builtin_amdgcn_s_waitcnt(0);
  int base = 0;
#pragma unroll
  for (int x = 0; x < NE; ++x) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(kp[x]);
    const int p = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
    if (kp[x]) c[p] = e[x];
    base += __builtin_popcountll(m);
  }
  n = keep;
  return th;
}

template <typename T, int RCAP>
__global__ __launch_bounds__(RWAVES * 64) void score_route_gqa_kernel(ScoreRouteArgs a) {
  constexpr int NE = RCAP / 64;                 // candidate entries per lane in a compaction
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  RTile<T>* tiles = reinterpret_cast<RTile<T>*>(smem);
  Cand* cand = reinterpret_cast<Cand*>(smem + 2 * sizeof(RTile<T>));
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int cap = a.cap;
  const int j = wg % a.n_kvh, b = wg / a.n_kvh;
  // rows [b * cap, b * cap + cnt): a storage block's valid slots, or (dense rows, cap = 64) the
  // next 64 pooled rows
  const int cnt = a.dense_rows ? min(cap, a.n_rows - b * cap) : a.blk_cnt[b];
  const int w = threadIdx.x >> 6, l = lane_id(), r = l & 15, g = l >> 4;
  const int n_valid = cnt > w ? min(RTPW, (cnt - w + RWAVES - 1) / RWAVES) : 0;   // tokens t < n_valid
  const int kk = min(a.top_k, a.n_blk);
  const float c2 = a.scale * kLog2e;
  const T* q = reinterpret_cast<const T*>(a.q);

  // padding slots of the block: rows of -1 (dense rows have none)
  for (int t = 0; t < RTPW; ++t) {
    const int slot = t * RWAVES + w;
    if (slot < cap && slot >= cnt && !a.dense_rows) {
      int32_t* so = a.sel + ((size_t)(b * cap + slot) * a.n_kvh + j) * a.top_k;
      for (int x = l; x < a.top_k; x += 64) so[x] = -1;
    }
  }

  // pre-scaled query rows (A operand: head r, elements 8g..8g+7) and the seeds -lse_h log2(e) of
  // heads 4g..4g+3 (rows of the S tile this lane holds)
  Frag8<T> qf[RTPW], ql[RTPW];
  f32x4 sd[RTPW];
  {
    Frag8<T> raw[RTPW];
    f32x4 ls[RTPW];
#pragma unroll
    for (int t = 0; t < RTPW; ++t) {
      const size_t row = (size_t)b * cap + min(t * RWAVES + w, cnt - 1);
      if constexpr (sizeof(T) == 2) {
        raw[t].v = *reinterpret_cast<const bf16x8*>(q + (row * a.n_qh + j * RGRP + r) * RHD + 8 * g);
      } else {
        const float* p = reinterpret_cast<const float*>(q) + (row * a.n_qh + j * RGRP + r) * RHD + 8 * g;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(p), x1 = *reinterpret_cast<const f32x4*>(p + 4);
        raw[t].v = (f32x8){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      }
      ls[t] = *reinterpret_cast<const f32x4*>(a.lse + row * a.n_qh + j * RGRP + 4 * g);
    }
#pragma unroll
    for (int t = 0; t < RTPW; ++t) {
      const bool ok = t < n_valid;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = ok ? to_f32(raw[t].v[e]) * c2 : 0.f;
        qf[t].v[e] = (T)x;
        ql[t].v[e] = (T)(x - to_f32(qf[t].v[e]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sd[t][i] = ok ? -ls[t][i] * kLog2e : 0.f;
    }
  }
  float th[RTPW];     // per token: candidates need importance >= th (uniform over the wave)
  int nc[RTPW];       // per token: kept candidates
#pragma unroll
  for (int t = 0; t < RTPW; ++t) {
    th[t] = 0.f;
    nc[t] = 0;
  }
  Cand* cw = cand + (size_t)w * RTPW * RCAP;    // this wave's buffers: token t at cw + t * RCAP

  const int kstride = a.n_kvh * RHD;
  const T* kbase = reinterpret_cast<const T*>(a.k_cmp) + j * RHD;
  const int ntiles = (a.n_blk + RT - 1) / RT;
  RStager<T> sa, sb;
  sa.load(kbase, kstride, 0, a.n_blk);
  sa.store(tiles[0]);
  sa.load(kbase, kstride, min(1, ntiles - 1) * RT, a.n_blk);
  __syncthreads();
  auto step = [&](int u, RStager<T>& cur, RStager<T>& nxt) {
    nxt.load(kbase, kstride, min(u + 2, ntiles - 1) * RT, a.n_blk);   // past the end: a harmless reload
    const RTile<T>& tb = tiles[u & 1];
    if (n_valid > 0) {
      Frag8<T> kf[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        if constexpr (sizeof(T) == 2) {
          kf[kt].v = *reinterpret_cast<const bf16x8*>(&tb.k[16 * kt + r][8 * g]);
        } else {
          const float* p = reinterpret_cast<const float*>(&tb.k[16 * kt + r][8 * g]);
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(p), x1 = *reinterpret_cast<const f32x4*>(p + 4);
          kf[kt].v = (f32x8){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        }
      }
      const int idx = u * RT + 16 * g + r;      // the key this lane ranks after the reduce-scatter
      const bool in_range = idx < a.n_blk;
      const bool gb0 = (g & 1) != 0, gb1 = (g & 2) != 0;
#pragma unroll
      for (int t = 0; t < RTPW; ++t) {
        if (t < n_valid) {
          float s[4];
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            // heads 4g + i of key 16 kt + r in base-2 units, minus lse
            const f32x4 x = (kSplitQuery && sizeof(T) == 2) ? mma16(qf[t], kf[kt], mma16(ql[t], kf[kt], sd[t]))
                                                            : mma16(qf[t], kf[kt], sd[t]);
            s[kt] = (__builtin_amdgcn_exp2f(x[0]) + __builtin_amdgcn_exp2f(x[1])) +
                    (__builtin_amdgcn_exp2f(x[2]) + __builtin_amdgcn_exp2f(x[3]));
          }
          // reduce-scatter over the lane groups: keep key tiles kt with bit 0 = g's bit 0, then bit 1
          float a0 = gb0 ? s[1] : s[0], a1 = gb0 ? s[3] : s[2];
          const float o0 = gb0 ? s[0] : s[1], o1 = gb0 ? s[2] : s[3];
          a0 += __shfl_xor(o0, 16, 64);
          a1 += __shfl_xor(o1, 16, 64);
          const float keep = gb1 ? a1 : a0, send = gb1 ? a0 : a1;
          const float imp = keep + __shfl_xor(send, 32, 64);
          const bool pass = in_range && imp >= th[t];
          const uint64_t bal = __builtin_amdgcn_ballot_w64(pass);
          if (bal != 0ull) {
            const int pos = nc[t] + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
            if (pass) cw[t * RCAP + pos] = Cand{imp, idx};
            nc[t] += __builtin_popcountll(bal);
            if (nc[t] > RCAP - RT) th[t] = compact<NE>(cw + t * RCAP, nc[t], kk, a.blk_key);
          }
        }
      }
    }
    if (u + 1 < ntiles) cur.store(tiles[(u + 1) & 1]);
    __syncthreads();
  };
  for (int u = 0; u < ntiles; u += 2) {
    step(u, sa, sb);
    if (u + 1 < ntiles) step(u + 1, sb, sa);
  }

  // the kept candidates of each token: the best kk, ranked best first
#pragma unroll
  for (int t = 0; t < RTPW; ++t) {
    if (t < n_valid) {
      Cand* ct = cw + t * RCAP;
      if (nc[t] > kk) th[t] = compact<NE>(ct, nc[t], kk, a.blk_key);
      const int n = nc[t];
      __builtin_amdgcn_s_waitcnt(0);
      const Cand e = l < n ? ct[l] : Cand{-1.f, -1};
      const uint32_t key = l < n ? a.blk_key[e.idx] : 0xFFFFFFFFu;
      int rank = 0;
      for (int x = 0; x < n; ++x) {
        const float vx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e.v), x));
        const uint32_t kx = (uint32_t)__builtin_amdgcn_readlane((int)key, x);
        rank += (vx > e.v || (vx == e.v && kx < key)) ? 1 : 0;
      }
      int32_t* so = a.sel + ((size_t)(b * cap + t * RWAVES + w) * a.n_kvh + j) * a.top_k;
      if (l < n) so[rank] = e.idx;
      for (int x = n + l; x < a.top_k; x += 64) so[x] = -1;
    }
  }
}

template <typename T, int RCAP>
hipError_t launch_cap(const ScoreRouteArgs& a, hipStream_t s) {
  const size_t lds = 2 * sizeof(RTile<T>) + (size_t)RWAVES * RTPW * RCAP * sizeof(Cand);
  const int nwg = (a.dense_rows ? (a.n_rows + RT - 1) / RT : a.n_blk) * a.n_kvh;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&score_route_gqa_kernel<T, RCAP>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((score_route_gqa_kernel<T, RCAP>), dim3(nwg), dim3(RWAVES * 64), lds, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const ScoreRouteArgs& a, hipStream_t s) {
  return rcap_for(a.top_k) == 128 ? launch_cap<T, 128>(a, s) : launch_cap<T, 256>(a, s);
}

}  // namespace

hipError_t launch_route_scores(int is_bf16, const ScoreRouteArgs& a, hipStream_t s) {
  return is_bf16 ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}

}  // namespace nsa
