// Score-routed NSA with one query head per KV head and head dim 64 (the Speed3R layout: Speed3R page,
// gist.science summary of arXiv 2603.08055, section 2.1).  Queries of the compressed branch and the
// routing rows are per block: pooled Q attends pooled K/V, top-k blocks per (query block, head) come
// from the same compressed scores, and every token of a query block attends its block's selected
// blocks for each head.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16): the N = 16 columns of S^T = K Q^T are 16 query rows of
// one head (16 pooled blocks in the compressed branch and routing, the up to 16 tokens of one block
// in the selected branch).  With D = 64 a 16-key step takes two MFMAs (d halves) and the value
// product four 16-row d tiles.  Lane l then holds query row l%16 and keys 16*kt + 4*(l/16) + i.
#include "common.h"
#include "kernels.h"

namespace nsa {
namespace {

constexpr int KT = 64;      // keys per tile
constexpr int DG = 64;      // head dim of these kernels
constexpr int KP = 72;      // LDS row stride (elements) of K and V^T tiles

struct TileG1 {
  bf16 k[KT][KP];           // K rows
  bf16 vt[DG][KP];          // V^T with the key order permuted as in vt_pos_g1
};

// Column of V^T holding key `key`: lane group g of a 32-key product step reads keys
// {32c+4g+i, 32c+16+4g+i}, i<4, as its eight k-slots.
__device__ __forceinline__ int vt_pos_g1(int key) {
  const int c = key >> 5, r = key & 31;
  const int hi = r >> 4, rr = r & 15;
  return 32 * c + 8 * (rr >> 2) + 4 * hi + (rr & 3);
}

__device__ __forceinline__ Frag8<bf16> ld8(const bf16* p) {
  Frag8<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Query fragments (two d halves) of one row: B operand of S^T.  With c2 != 1 every element is
// multiplied by c2 = scale * log2(e) in fp32 and rounded once to bf16, so S^T comes out in base-2
// logit units (the routing kernel keeps the raw query: c2 = 1).
struct QG1 { Frag8<bf16> h[2]; };

__device__ __forceinline__ QG1 load_q_row(const bf16* row, bool valid, float c2 = 1.f) {
  QG1 q;
  const int g = lane_id() >> 4;
  if (valid) {
    q.h[0] = ld8(row + 8 * g);
    q.h[1] = ld8(row + 32 + 8 * g);
    if (c2 != 1.f) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) q.h[hh].v[e] = (bf16)((float)q.h[hh].v[e] * c2);
    }
  } else {
    q.h[0].v = bf16x8{};
    q.h[1].v = bf16x8{};
  }
  return q;
}

// K and V^T fragments of a staged tile.
struct TileFragsG1 {
  Frag8<bf16> k[4][2];      // [key tile][d half]
  Frag8<bf16> v[4][2];      // [d tile][key chunk]
};

__device__ __forceinline__ void load_frags_g1(const TileG1& t, TileFragsG1& f) {
  const int l = lane_id(), r = l & 15, g = l >> 4;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int h = 0; h < 2; ++h) f.k[kt][h] = ld8(&t.k[16 * kt + r][32 * h + 8 * g]);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c) f.v[dt][c] = ld8(&t.vt[16 * dt + r][32 * c + 8 * g]);
}

// Raw scores S^T = K Q^T (+ seed) for one column group.
__device__ __forceinline__ void scores_g1(const TileFragsG1& f, const QG1& q, const f32x4 (&seed)[4], f32x4 (&s)[4]) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) s[kt] = mma16(f.k[kt][1], q.h[1], mma16(f.k[kt][0], q.h[0], seed[kt]));
}

// One wave's share of a gathered 64-key tile: chunk tid + 64 i (i < 8) of the 512 16-byte chunks
// of K and the same chunk of V.  All sixteen loads are issued before any is used, so a tile costs one
// memory round trip, and the next tile's gather runs during the current tile's compute.  Padding
// keys (row -1) read row 0: their scores are masked to -inf, so they weigh nothing.
// (vector types, not arrays: an array carried across the tile loop was placed in scratch memory)
typedef uint32_t u32x32 __attribute__((ext_vector_type(32)));
struct RowsG1 { u32x32 k, v; };

__device__ __forceinline__ void put4(u32x32& d, int i, uint4 x) {
  d[4 * i] = x.x;
  d[4 * i + 1] = x.y;
  d[4 * i + 2] = x.z;
  d[4 * i + 3] = x.w;
}

__device__ __forceinline__ void gather_rows_g1(RowsG1& g, const bf16* kb, const bf16* vb, int stride,
                                               const int* rows /* LDS [64] */, int tid) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int cc = tid + i * 64;
    const int key = cc >> 3, part = cc & 7;
    const size_t off = (size_t)max(rows[key], 0) * stride + part * 8;
    put4(g.k, i, *reinterpret_cast<const uint4*>(kb + off));
    put4(g.v, i, *reinterpret_cast<const uint4*>(vb + off));
  }
}

__device__ __forceinline__ void store_rows_g1(TileG1& t, const RowsG1& g, int tid) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int cc = tid + i * 64;
    const int key = cc >> 3, part = cc & 7;
    *reinterpret_cast<uint4*>(&t.k[key][part * 8]) = make_uint4(g.k[4 * i], g.k[4 * i + 1], g.k[4 * i + 2], g.k[4 * i + 3]);
    // the eight bf16 values by shifts
    const uint32_t wd[4] = {g.v[4 * i], g.v[4 * i + 1], g.v[4 * i + 2], g.v[4 * i + 3]};
    const int pos = vt_pos_g1(key);
#pragma unroll
    for (int x = 0; x < 8; ++x)
      t.vt[part * 8 + x][pos] = __builtin_bit_cast(bf16, (uint16_t)(wd[x >> 1] >> (16 * (x & 1))));
  }
}

// Online softmax state of one column group (16 rows of one head), base-2 units.  The reference
// maximum mc starts at 0 and may go stale: it enters S^T as the MFMA accumulator seed (-mc), and
// it moves (with a rescale) only when a lane's probability sum could exceed kStaleLimitG1 or is
// not finite, or when a row has no mass yet and the tile's mass is tiny.  The result equals the
// textbook online softmax up to rounding.
struct StateG1 {
  f32x4 acc[4];             // O^T[d = 16*dt + 4*(lane/16) + i][row lane%16]
  float mc;                 // reference max of row lane%16 (identical across lane groups)
  float l;                  // this lane group's share of the sum
};

constexpr float kStaleLimitG1 = 65536.0f;
constexpr float kTinyMassG1 = 1.0e-30f;

__device__ __forceinline__ void state_init(StateG1& s) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) s.acc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  s.mc = 0.f;
  s.l = 0.f;
}

__device__ __forceinline__ float rows_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float rows_sum(float x) {
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
}

// p = exp2(x) for the lane's 16 logits, packed as the two B operands of the value product;
// returns the lane's sum of the probabilities as rounded for that product.
__device__ __forceinline__ float exp_pack_g1(const f32x4 (&x)[4], Frag8<bf16> (&pf)[2]) {
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

// One tile: x = S^T - mc (padding keys -inf) from scores_g1; probabilities rounded to bf16 for the
// value product.
__device__ __forceinline__ void softmax_pv_g1(StateG1& st, f32x4 (&x)[4], const TileFragsG1& f) {
  Frag8<bf16> pf[2];
  float lt = exp_pack_g1(x, pf);
  if (__builtin_amdgcn_ballot_w64(!(lt <= kStaleLimitG1) || !(st.l + lt >= kTinyMassG1)) != 0) {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[kt][i]);
    const float xm = rows_max(mx);
    const float lh = rows_sum(st.l);
    float shift = lh > 0.f ? fmaxf(xm, 0.f) : xm;
    if (!(shift > -INFINITY)) shift = 0.f;          // no valid key in this row
    if (lh > 0.f && shift > 0.f) {
      const float alpha = __builtin_amdgcn_exp2f(-shift);
      st.l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) st.acc[dt] *= alpha;
    }
    st.mc += shift;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) x[kt] -= shift;
    lt = exp_pack_g1(x, pf);
  }
  st.l += lt;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c) st.acc[dt] = mma16(f.v[dt][c], pf[c], st.acc[dt]);
}

// Seeds of S^T for a column group: -mc on valid keys, -inf on the keys of a partial tile.
__device__ __forceinline__ void row_seed(const StateG1& st, bool full, const f32x4 (&cm)[4], f32x4 (&seed)[4]) {
  if (full) {
    const f32x4 m = {-st.mc, -st.mc, -st.mc, -st.mc};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) seed[kt] = m;
  } else {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) seed[kt] = cm[kt] - st.mc;
  }
}

// 0 on the keys of a tile below nk, -inf beyond (the lane's keys are 16*kt + 4*(lane/16) + i).
__device__ __forceinline__ void mask_seed(int nk, f32x4 (&cm)[4]) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) cm[kt][i] = (16 * kt + 4 * g + i < nk) ? 0.f : -INFINITY;
}

// ---------------------------------------------------------------------------------------------
// compressed branch with block queries
// ---------------------------------------------------------------------------------------------

constexpr int CW = 8;       // waves per workgroup
constexpr int CG = 2;       // column groups (16 rows each) per wave

__global__ __launch_bounds__(CW * 64) void cmp_g1_kernel(G1Args a) {
  static_assert(CW * 64 == KT * 8, "one 16-byte piece of K and of V per thread");
  __shared__ TileG1 tb[2];
  const int n_rowgrp = (a.n_blk + CW * CG * 16 - 1) / (CW * CG * 16);
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wg / n_rowgrp, rg = wg % n_rowgrp;
  const int w = threadIdx.x >> 6, l = lane_id(), r = l & 15, g = l >> 4;
  const int stride = a.n_kvh * DG;
  const bf16* qc = reinterpret_cast<const bf16*>(a.q_cmp);
  const bf16* kb = reinterpret_cast<const bf16*>(a.k_cmp) + h * DG;
  const bf16* vb = reinterpret_cast<const bf16*>(a.v_cmp) + h * DG;
  const float c2 = a.scale * kLog2e;

  QG1 q[CG];
  StateG1 st[CG];
  int row_of[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    row_of[c] = (rg * CW * CG + w * CG + c) * 16 + r;
    const bool ok = row_of[c] < a.n_blk;
    q[c] = load_q_row(qc + ((size_t)row_of[c] * a.n_qh + h) * DG, ok, c2);
    state_init(st[c]);
  }
  const int ntiles = (a.n_blk + KT - 1) / KT;
  // staging: thread t copies the 16-byte piece (key t / 8, part t % 8) of both K and V; the next
  // tile's loads are issued before the current tile's compute
  const int s_key = threadIdx.x >> 3, s_part = threadIdx.x & 7;
  // (no branch around the loads and no unpacking before the store: either would make the next
  // tile's load wait at once; keys past the end repeat the last row, masked out of the scores)
  auto fetch = [&](int u, uint4& kv, uint4& vv) {
    const size_t off = (size_t)min(u * KT + s_key, a.n_blk - 1) * stride + s_part * 8;
    kv = *reinterpret_cast<const uint4*>(kb + off);
    vv = *reinterpret_cast<const uint4*>(vb + off);
  };
  auto store = [&](TileG1& t, const uint4& kv, const uint4& vv) {
    *reinterpret_cast<uint4*>(&t.k[s_key][s_part * 8]) = kv;
    const uint32_t wd[4] = {vv.x, vv.y, vv.z, vv.w};
    const int pos = vt_pos_g1(s_key);
#pragma unroll
    for (int x = 0; x < 8; ++x)
      t.vt[s_part * 8 + x][pos] = __builtin_bit_cast(bf16, (uint16_t)(wd[x >> 1] >> (16 * (x & 1))));
  };
  uint4 kv, vv;
  fetch(0, kv, vv);
  store(tb[0], kv, vv);
  __syncthreads();
  for (int u = 0; u < ntiles; ++u) {
    const int cur = u & 1;
    if (u + 1 < ntiles) fetch(u + 1, kv, vv);
    TileFragsG1 f;
    load_frags_g1(tb[cur], f);
    const int nk = min(KT, a.n_blk - u * KT);
    const bool full = nk == KT;
    f32x4 cm[4];
    if (!full) mask_seed(nk, cm);
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      f32x4 seed[4], x[4];
      row_seed(st[c], full, cm, seed);
      scores_g1(f, q[c], seed, x);
      softmax_pv_g1(st[c], x, f);
    }
    // every wave finished tile u - 1 (the previous barrier), so buffer cur ^ 1 is free
    if (u + 1 < ntiles) store(tb[cur ^ 1], kv, vv);
    __syncthreads();
  }
  // finish: normalise, gate per token, give the block's pooled result to each of its tokens
  bf16* o = reinterpret_cast<bf16*>(a.o);
  const bf16* gp = reinterpret_cast<const bf16*>(a.gates);
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const int b = row_of[c];
    const float lsum = rows_sum(st[c].l);
    if (b >= a.n_blk) continue;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    if (a.lse && g == 0) a.lse[(size_t)b * a.n_qh + h] = lsum > 0.f ? (st[c].mc + __log2f(lsum)) * kLn2 : -INFINITY;
    const int cnt = a.blk_cnt[b];
    for (int t = 0; t < a.cap; ++t) {
      const size_t row = (size_t)b * a.cap + t;
      float wgt = 0.f;
      if (t < cnt) wgt = gp ? sigmoidf_((float)gp[(row * a.n_qh + h) * a.n_gch + a.ch_cmp]) * inv : inv;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        bf16x4* dst = reinterpret_cast<bf16x4*>(o + (row * a.n_qh + h) * DG + 16 * dt + 4 * g);
        *dst = __builtin_convertvector(st[c].acc[dt] * wgt, bf16x4);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// routing: top-k blocks per (query block, head) by compressed score, no score matrix stored
// ---------------------------------------------------------------------------------------------
//
// Each wave scores CG column groups (16 query rows each) against a staged 64-key tile with MFMA.
// Lane (r, g) sees a quarter of every row's keys and keeps a sorted list of its best K.  Candidates
// are filtered first against a row-level bound of the row's current k-th best (the lists of the
// four lanes of a row give one): after the first tiles few scores pass.  The tile's scores go to
// wave-private LDS so that each lane can walk only its own candidates into a short queue; the
// sorted insertions run for the whole wave at once whenever some lane's queue is full (a pass in
// one lane alone would otherwise cost the wave a whole insertion), and the row bound is refreshed
// after each such step.  Ranking key: (score, then smaller blk_key) packed
// into 64 bits so that one unsigned compare orders both.

constexpr int RW = 8;       // waves per workgroup

__device__ __forceinline__ uint32_t ord_f32(float v) {
  uint32_t u = __float_as_uint(v == 0.f ? 0.f : v);      // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t o) {
  if (o == 0u) return -INFINITY;                         // empty list slot: everything passes
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ uint64_t rank_key(float v, uint32_t blk_key) {
  return ((uint64_t)ord_f32(v) << 32) | (uint64_t)(~blk_key);
}

template <int K>
struct TopList {
  uint64_t key[K];          // descending; 0 = empty
  int idx[K];
};

template <int K>
__device__ __forceinline__ void toplist_init(TopList<K>& t) {
#pragma unroll
  for (int x = 0; x < K; ++x) {
    t.key[x] = 0ull;
    t.idx[x] = -1;
  }
}

template <int K>
__device__ __forceinline__ void toplist_insert(TopList<K>& t, uint64_t ck, int ci) {
  if (ck <= t.key[K - 1]) return;
#pragma unroll
  for (int x = K - 1; x > 0; --x) {
    const bool gp = ck > t.key[x - 1];
    const bool gc = ck > t.key[x];
    t.key[x] = gp ? t.key[x - 1] : (gc ? ck : t.key[x]);
    t.idx[x] = gp ? t.idx[x - 1] : (gc ? ci : t.idx[x]);
  }
  if (ck > t.key[0]) {
    t.key[0] = ck;
    t.idx[0] = ci;
  }
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64), hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Lower bound on the row's K-th best key: each lane list holds K distinct keys >= its last entry,
// and the four lists together hold K distinct keys >= the smallest of their (K/4)-th entries.
template <int K>
__device__ __forceinline__ float row_threshold(const TopList<K>& t) {
  uint64_t hi = t.key[K - 1], lo = t.key[K / 4 - 1];
#pragma unroll
  for (int m = 16; m <= 32; m <<= 1) {
    const uint64_t h2 = shfl_xor_u64(hi, m), l2 = shfl_xor_u64(lo, m);
    hi = h2 > hi ? h2 : hi;
    lo = l2 < lo ? l2 : lo;
  }
  const uint64_t b = hi > lo ? hi : lo;
  return unord_f32((uint32_t)(b >> 32));
}

template <int K, int CG>
__global__ __launch_bounds__(RW * 64) void route_g1_kernel(G1Args a) {
  __shared__ bf16 kt_lds[2][KT][KP];
  __shared__ uint32_t keys_lds[2][KT];
  __shared__ f32x4 sc_lds[RW][4][64];      // one column group's tile scores per wave, slot-major
  const int rows_per_wg = RW * CG * 16;
  const int n_rowgrp = (a.n_blk + rows_per_wg - 1) / rows_per_wg;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wg / n_rowgrp, rg = wg % n_rowgrp;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), r = l & 15, g = l >> 4;
  const int stride = a.n_kvh * DG;
  const bf16* qc = reinterpret_cast<const bf16*>(a.q_cmp);
  const bf16* kb = reinterpret_cast<const bf16*>(a.k_cmp) + h * DG;

  QG1 q[CG];
  TopList<K> lst[CG];
  float thr[CG];
  int row_of[CG];
  // candidates that passed the row bound but are not yet ranked: QN per lane and column group
  // (one for the 64-long lists, whose registers leave no room for a queue)
  constexpr int QN = K <= 32 ? 4 : 1;
  uint64_t qk[CG][QN];
  int qi[CG][QN];
  int qn[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    row_of[c] = rg * rows_per_wg + (w * CG + c) * 16 + r;
    q[c] = load_q_row(qc + ((size_t)row_of[c] * a.n_qh + h) * DG, row_of[c] < a.n_blk);
    toplist_init(lst[c]);
    thr[c] = -INFINITY;
    qn[c] = 0;
#pragma unroll
    for (int x = 0; x < QN; ++x) {
      qk[c][x] = 0ull;
      qi[c][x] = -1;
    }
  }
  // rank the queued candidates of column group c (every lane, so the row bound can be shared)
  auto flush = [&](int c) {
#pragma unroll
    for (int x = 0; x < QN; ++x)
      if (x < qn[c]) toplist_insert(lst[c], qk[c][x], qi[c][x]);
    qn[c] = 0;
    thr[c] = row_threshold(lst[c]);
  };
  const int ntiles = (a.n_blk + KT - 1) / KT;
  // staging: thread t copies 16 bytes (key t / 8, piece t % 8) of the K tile; threads < 64 the keys
  const int s_key = tid >> 3, s_part = tid & 7;
  auto fetch = [&](int u, uint4& kv, uint32_t& bkey) {
    const int key = u * KT + s_key;
    kv = make_uint4(0u, 0u, 0u, 0u);
    if (key < a.n_blk) kv = *reinterpret_cast<const uint4*>(kb + (size_t)key * stride + s_part * 8);
    const int kk = u * KT + tid;
    bkey = (tid < KT && kk < a.n_blk) ? a.blk_key[kk] : 0u;
  };
  auto store = [&](int buf, const uint4& kv, uint32_t bkey) {
    *reinterpret_cast<uint4*>(&kt_lds[buf][s_key][s_part * 8]) = kv;
    if (tid < KT) keys_lds[buf][tid] = bkey;
  };
  uint4 kv;
  uint32_t bkey;
  fetch(0, kv, bkey);
  store(0, kv, bkey);
  __syncthreads();
  for (int u = 0; u < ntiles; ++u) {
    const int cur = u & 1;
    if (u + 1 < ntiles) fetch(u + 1, kv, bkey);
    Frag8<bf16> kf[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) kf[kt][hh] = ld8(&kt_lds[cur][16 * kt + r][32 * hh + 8 * g]);
    const int nk = min(KT, a.n_blk - u * KT);
    uint32_t vmask = 0xFFFFu;                 // slot j = 4*kt + i holds key 16*kt + 4*g + i
    if (nk < KT) {
      vmask = 0u;
#pragma unroll
      for (int j = 0; j < 16; ++j) vmask |= (16 * (j >> 2) + 4 * g + (j & 3) < nk) ? (1u << j) : 0u;
    }
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      f32x4 s[4];
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[kt] = mma16(kf[kt][1], q[c].h[1], mma16(kf[kt][0], q[c].h[0], z));
      uint32_t m = 0u;
#pragma unroll
      for (int j = 0; j < 16; ++j) m |= (s[j >> 2][j & 3] >= thr[c]) ? (1u << j) : 0u;
      m &= vmask;
      if (__builtin_amdgcn_ballot_w64(m != 0u) == 0ull) continue;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) sc_lds[w][kt][l] = s[kt];
      // one candidate per lane per round into its queue; whenever some lane's queue is full, the
      // whole wave ranks its queues (so the sorted insertions run in few, shared steps)
      while (__builtin_amdgcn_ballot_w64(m != 0u) != 0ull) {
        if (m != 0u) {
          const int j = __builtin_ctz(m);
          m &= m - 1u;
          const float v = reinterpret_cast<const float*>(&sc_lds[w][j >> 2][l])[j & 3];
          const int key = 16 * (j >> 2) + 4 * g + (j & 3);
          const uint64_t ck = rank_key(v, keys_lds[cur][key]);
          const int ci = u * KT + key;
#pragma unroll
          for (int x = 0; x < QN; ++x) {
            qk[c][x] = qn[c] == x ? ck : qk[c][x];
            qi[c][x] = qn[c] == x ? ci : qi[c][x];
          }
          ++qn[c];
        }
        if (__builtin_amdgcn_ballot_w64(qn[c] == QN) != 0ull) flush(c);
      }
    }
    // every wave finished tile u - 1 (the previous barrier), so buffer cur ^ 1 is free
    if (u + 1 < ntiles) store(cur ^ 1, kv, bkey);
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < CG; ++c) flush(c);
  // merge the four lane lists of each row: top_k rounds of arg-best over the list heads
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const int row = row_of[c];
    int32_t* so = const_cast<int32_t*>(a.sel) + ((size_t)row * a.n_kvh + h) * a.top_k;
    for (int x = 0; x < a.top_k; ++x) {
      uint64_t best = lst[c].key[0];
      int src = g;
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const uint64_t b2 = shfl_xor_u64(best, o);
        const int s2 = __shfl_xor(src, o, 64);
        if (b2 > best) {
          best = b2;
          src = s2;
        }
      }
      const int win = __shfl(lst[c].idx[0], r + 16 * src, 64);
      if (g == 0 && row < a.n_blk) so[x] = best == 0ull ? -1 : win;
      if (g == src) {
#pragma unroll
        for (int y = 0; y < K - 1; ++y) {
          lst[c].key[y] = lst[c].key[y + 1];
          lst[c].idx[y] = lst[c].idx[y + 1];
        }
        lst[c].key[K - 1] = 0ull;
        lst[c].idx[K - 1] = -1;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// selected branch with block routing rows: one wave per (query block, head)
// ---------------------------------------------------------------------------------------------

// NF: capacity for forced blocks (0: the forced range is ignored, and the key list stays small)
// Two waves per SIMD (at most 256 registers each) where LDS allows eight workgroups per CU; the
// forced variant's key list allows four.
template <int NF>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NF > 0 ? 1 : 2))) void sel_g1_kernel(G1Args a) {
  __shared__ TileG1 tb;
  __shared__ int keys_lds[(64 + NF) * 16 + KT];   // source rows of the selected valid tokens, packed
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int b = wg / a.n_kvh, h = wg % a.n_kvh;
  const int l = lane_id(), r = l & 15, g = l >> 4;
  const int cap = a.cap, cnt = a.blk_cnt[b];
  const int stride = a.n_kvh * DG;
  const bf16* q = reinterpret_cast<const bf16*>(a.q);
  const bf16* kb = reinterpret_cast<const bf16*>(a.k) + h * DG;
  const bf16* vb = reinterpret_cast<const bf16*>(a.v) + h * DG;
  const float c2 = a.scale * kLog2e;
  // lane x < top_k holds entry x of this block's routing row for head h; -1, out-of-range and
  // repeated entries count no keys; the valid tokens of the rest are packed one after another
  const int grp = a.sel_groups == 1 ? 0 : h;
  const int32_t* srow = a.sel + ((size_t)b * a.sel_groups + grp) * a.top_k;
  const int sb = l < a.top_k ? srow[l] : -1;
  const int nf = NF > 0 ? a.f_hi - a.f_lo : 0;
  bool keep = sb >= 0 && sb < a.n_blk && !(sb >= a.f_lo && sb - a.f_lo < nf);   // forced blocks come below
  for (int y = 0; y < a.top_k; ++y) {
    const int sy = __builtin_amdgcn_readlane(sb, y);
    keep = keep && !(y < l && sy == sb);
  }
  int total = 0;
  // the routed blocks, then the forced range 64 blocks at a time, packed one after another
  for (int f0 = -64; f0 < nf; f0 += 64) {
    const int fb = a.f_lo + f0 + l;                          // forced block of this lane (f0 >= 0)
    const int blk = f0 < 0 ? sb : fb;
    const bool on = f0 < 0 ? keep : (f0 + l < nf);
    const int c = on ? a.blk_cnt[blk] : 0;
    int inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o, 64);
      if (l >= o) inc += y;
    }
    for (int t = 0; t < c; ++t) keys_lds[total + inc - c + t] = blk * cap + t;
    total += __builtin_amdgcn_readlane(inc, 63);
  }
  const int ntiles = (total + KT - 1) / KT;
  for (int i = total + l; i < ntiles * KT; i += 64) keys_lds[i] = -1;
  __syncthreads();
  StateG1 st;
  state_init(st);
  const QG1 qq = load_q_row(q + ((size_t)(b * cap + r) * a.n_qh + h) * DG, r < cnt, c2);
  RowsG1 pre;
  if (ntiles > 0) gather_rows_g1(pre, kb, vb, stride, keys_lds, l);
  for (int u = 0; u < ntiles; ++u) {
    store_rows_g1(tb, pre, l);
    __syncthreads();
    if (u + 1 < ntiles) gather_rows_g1(pre, kb, vb, stride, keys_lds + (u + 1) * KT, l);
    TileFragsG1 f;
    load_frags_g1(tb, f);
    const int nk = min(KT, total - u * KT);
    f32x4 cm[4], seed[4], x[4];
    if (nk < KT) mask_seed(nk, cm);
    row_seed(st, nk == KT, cm, seed);
    scores_g1(f, qq, seed, x);
    softmax_pv_g1(st, x, f);
    __syncthreads();
  }
  const float lsum = rows_sum(st.l);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  bf16* o = reinterpret_cast<bf16*>(a.o);
  const bf16* gp = reinterpret_cast<const bf16*>(a.gates);
  if (r < cap) {
    const size_t row = (size_t)b * cap + r;
    if (a.lse && g == 0) a.lse[row * a.n_qh + h] = (r < cnt && lsum > 0.f) ? (st.mc + __log2f(lsum)) * kLn2 : -INFINITY;
    const bool valid = r < cnt;
    const float wgt = valid ? (gp ? sigmoidf_((float)gp[(row * a.n_qh + h) * a.n_gch + a.ch_sel]) * inv : inv) : 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      bf16x4* dst = reinterpret_cast<bf16x4*>(o + (row * a.n_qh + h) * DG + 16 * dt + 4 * g);
      f32x4 v = st.acc[dt] * wgt;
      if (a.accumulate && valid) {
        const bf16x4 prev = *dst;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += (float)prev[i];
      }
      *dst = __builtin_convertvector(v, bf16x4);
    }
  }
}

template <int K, int CG>
hipError_t launch_route_g1_k(const G1Args& a, hipStream_t s) {
  const int n_rowgrp = (a.n_blk + RW * CG * 16 - 1) / (RW * CG * 16);
  hipLaunchKernelGGL((route_g1_kernel<K, CG>), dim3(n_rowgrp * a.n_kvh), dim3(RW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_g1(const G1Args& a, hipStream_t s) {
  if (a.top_k <= 8) return launch_route_g1_k<8, 2>(a, s);
  if (a.top_k <= 16) return launch_route_g1_k<16, 2>(a, s);
  if (a.top_k <= 32) return launch_route_g1_k<32, 1>(a, s);
  return launch_route_g1_k<64, 1>(a, s);
}

hipError_t launch_attn_g1(const G1Args& a0, hipStream_t s) {
  G1Args a = a0;
  if (a.branches & 1) {
    const int n_rowgrp = (a.n_blk + CW * CG * 16 - 1) / (CW * CG * 16);
    hipLaunchKernelGGL(cmp_g1_kernel, dim3(n_rowgrp * a.n_kvh), dim3(CW * 64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.branches & 2) {
    a.accumulate = (a.branches & 1) ? 1 : 0;
    if (a.f_hi > a.f_lo)
      hipLaunchKernelGGL(sel_g1_kernel<kMaxForcedBlocks>, dim3(a.n_blk * a.n_kvh), dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL(sel_g1_kernel<0>, dim3(a.n_blk * a.n_kvh), dim3(64), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace nsa
