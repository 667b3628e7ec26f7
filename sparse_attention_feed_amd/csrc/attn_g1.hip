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
//
// The kernels are templated on the element type of q, k, v and o.  fp32 inputs take eight
// v_mfma_f32_16x16x4f32 per bf16 instruction on the same lane data, keep the probabilities in fp32
// for the value product, and move each row piece of eight elements as 32 bytes instead of 16.
#include "common.h"
#include "kernels.h"

namespace nsa {
namespace {

constexpr int KT = 64;      // keys per tile
constexpr int DG = 64;      // head dim of these kernels
constexpr int KP = 72;      // LDS row stride (elements) of K and V^T tiles

template <typename T>
struct TileG1 {
  T k[KT][KP];              // K rows
  T vt[DG][KP];             // V^T with the key order permuted as in vt_pos_g1
};

// Column of V^T holding key `key`: lane group g of a 32-key product step reads keys
// {32c+4g+i, 32c+16+4g+i}, i<4, as its eight k-slots.
__device__ __forceinline__ int vt_pos_g1(int key) {
  const int c = key >> 5, r = key & 31;
  const int hi = r >> 4, rr = r & 15;
  return 32 * c + 8 * (rr >> 2) + 4 * hi + (rr & 3);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Eight consecutive elements of a row as one thread moves them: one 16-byte word of bf16, two of
// fp32 (kept as raw words, so no unpacking stands between a load and its use).
template <typename T> struct Oct;
template <> struct Oct<bf16> { uint4 a; };
template <> struct Oct<float> { uint4 a, b; };

__device__ __forceinline__ Oct<bf16> load_oct(const bf16* p) { return {*reinterpret_cast<const uint4*>(p)}; }
__device__ __forceinline__ Oct<float> load_oct(const float* p) {
  const uint4* s = reinterpret_cast<const uint4*>(p);
  return {s[0], s[1]};
}
__device__ __forceinline__ void store_oct(bf16* p, const Oct<bf16>& o) { *reinterpret_cast<uint4*>(p) = o.a; }
__device__ __forceinline__ void store_oct(float* p, const Oct<float>& o) {
  uint4* d = reinterpret_cast<uint4*>(p);
  d[0] = o.a;
  d[1] = o.b;
}
__device__ __forceinline__ uint32_t word(const uint4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }
// element x (< 8) of an eight-element piece
__device__ __forceinline__ bf16 oct_elem(const Oct<bf16>& o, int x) {
  return __builtin_bit_cast(bf16, (uint16_t)(word(o.a, x >> 1) >> (16 * (x & 1))));
}
__device__ __forceinline__ float oct_elem(const Oct<float>& o, int x) { return __uint_as_float(word(x < 4 ? o.a : o.b, x & 3)); }

// Four consecutive output elements
template <typename T> struct V4;
template <> struct V4<bf16> { typedef bf16x4 t; };
template <> struct V4<float> { typedef f32x4 t; };

// Query fragments (two d halves) of one row: B operand of S^T.  With c2 != 1 every element is
// multiplied by c2 = scale * log2(e) in fp32 and rounded once to bf16, so S^T comes out in base-2
// logit units (the routing kernel keeps the raw query: c2 = 1).
// (with fp32 inputs the product is formed in fp32, no rounding beyond it)
template <typename T>
struct QG1 { Frag8<T> h[2]; };

template <typename T>
__device__ __forceinline__ QG1<T> load_q_row(const T* row, bool valid, float c2 = 1.f) {
  QG1<T> q;
  const int g = lane_id() >> 4;
  if (valid) {
    q.h[0] = load_frag(row + 8 * g);
    q.h[1] = load_frag(row + 32 + 8 * g);
    if (c2 != 1.f) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) q.h[hh].v[e] = (T)((float)q.h[hh].v[e] * c2);
    }
  } else {
    q.h[0].v = decltype(q.h[0].v){};
    q.h[1].v = decltype(q.h[1].v){};
  }
  return q;
}

// K and V^T fragments of a staged tile.
template <typename T>
struct TileFragsG1 {
  Frag8<T> k[4][2];         // [key tile][d half]
  Frag8<T> v[4][2];         // [d tile][key chunk]
};

template <typename T>
__device__ __forceinline__ void load_frags_g1(const TileG1<T>& t, TileFragsG1<T>& f) {
  const int l = lane_id(), r = l & 15, g = l >> 4;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int h = 0; h < 2; ++h) f.k[kt][h] = load_frag(&t.k[16 * kt + r][32 * h + 8 * g]);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c) f.v[dt][c] = load_frag(&t.vt[16 * dt + r][32 * c + 8 * g]);
}

// Raw scores S^T = K Q^T (+ seed) for one column group.
template <typename T>
__device__ __forceinline__ void scores_g1(const TileFragsG1<T>& f, const QG1<T>& q, const f32x4 (&seed)[4],
                                          f32x4 (&s)[4]) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) s[kt] = mma16(f.k[kt][1], q.h[1], mma16(f.k[kt][0], q.h[0], seed[kt]));
}

// One wave's share of a gathered 64-key tile: chunk tid + 64 i (i < NCH) of the 16-byte chunks of
// K and the same chunk of V (512 each in bf16, 1024 in fp32).  All loads are issued before any is
// used, so a tile costs one memory round trip, and the next tile's gather runs during the current
// tile's compute.  Padding keys (row -1) read row 0: their scores are masked to -inf, so they weigh
// nothing.
// (vector types, not arrays: an array carried across the tile loop was placed in scratch memory)
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x32 __attribute__((ext_vector_type(32)));
typedef uint32_t u32x64 __attribute__((ext_vector_type(64)));
// a thread's share of a tile gathered by NTH threads
template <typename T, int NTH> struct RowsG1;
template <> struct RowsG1<bf16, 64> { u32x32 k, v; };
template <> struct RowsG1<float, 64> { u32x64 k, v; };
template <> struct RowsG1<bf16, 128> { u32x16 k, v; };
template <> struct RowsG1<float, 128> { u32x32 k, v; };

template <typename T, int NTH = 64> struct ChunkG1 {
  static constexpr int EPC = 16 / sizeof(T);     // elements per 16-byte chunk
  static constexpr int CPK = DG / EPC;           // chunks per key row
  static constexpr int NCH = KT * CPK / NTH;     // chunks per thread
};

template <typename V>
__device__ __forceinline__ void put4(V& d, int i, uint4 x) {
  d[4 * i] = x.x;
  d[4 * i + 1] = x.y;
  d[4 * i + 2] = x.z;
  d[4 * i + 3] = x.w;
}

// element x of chunk i of a gathered row piece
template <typename V>
__device__ __forceinline__ bf16 chunk_elem(const V& d, int i, int x, bf16) {
  return __builtin_bit_cast(bf16, (uint16_t)(d[4 * i + (x >> 1)] >> (16 * (x & 1))));
}
template <typename V>
__device__ __forceinline__ float chunk_elem(const V& d, int i, int x, float) { return __uint_as_float(d[4 * i + x]); }

template <int NTH, typename T>
__device__ __forceinline__ void gather_rows_g1(RowsG1<T, NTH>& g, const T* kb, const T* vb, int stride,
                                               const int* rows /* LDS [64] */, int tid) {
  typedef ChunkG1<T, NTH> C;
#pragma unroll
  for (int i = 0; i < C::NCH; ++i) {
    const int cc = tid + i * NTH;
    const int key = cc / C::CPK, part = cc % C::CPK;
    const size_t off = (size_t)max(rows[key], 0) * stride + part * C::EPC;
    put4(g.k, i, *reinterpret_cast<const uint4*>(kb + off));
    put4(g.v, i, *reinterpret_cast<const uint4*>(vb + off));
  }
}

template <int NTH, typename T>
__device__ __forceinline__ void store_rows_g1(TileG1<T>& t, const RowsG1<T, NTH>& g, int tid) {
  typedef ChunkG1<T, NTH> C;
#pragma unroll
  for (int i = 0; i < C::NCH; ++i) {
    const int cc = tid + i * NTH;
    const int key = cc / C::CPK, part = cc % C::CPK;
    *reinterpret_cast<uint4*>(&t.k[key][part * C::EPC]) =
        make_uint4(g.k[4 * i], g.k[4 * i + 1], g.k[4 * i + 2], g.k[4 * i + 3]);
    const int pos = vt_pos_g1(key);
#pragma unroll
    for (int x = 0; x < C::EPC; ++x) t.vt[part * C::EPC + x][pos] = chunk_elem(g.v, i, x, T());
  }
}

// bf16 tiles of the selected branch: V kept as rows (as gathered) and read back transposed.
struct TileG1R {
  bf16 k[KT][KP];           // K rows
  bf16 v[KT][KP];           // V rows
};
template <typename T> struct SelTile { typedef TileG1<T> type; };
template <> struct SelTile<bf16> { typedef TileG1R type; };

template <int NTH>
__device__ __forceinline__ void store_rows_g1(TileG1R& t, const RowsG1<bf16, NTH>& g, int tid) {
  typedef ChunkG1<bf16, NTH> C;
#pragma unroll
  for (int i = 0; i < C::NCH; ++i) {
    const int cc = tid + i * NTH;
    const int key = cc / C::CPK, part = cc % C::CPK;
    *reinterpret_cast<uint4*>(&t.k[key][part * C::EPC]) =
        make_uint4(g.k[4 * i], g.k[4 * i + 1], g.k[4 * i + 2], g.k[4 * i + 3]);
    *reinterpret_cast<uint4*>(&t.v[key][part * C::EPC]) =
        make_uint4(g.v[4 * i], g.v[4 * i + 1], g.v[4 * i + 2], g.v[4 * i + 3]);
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
// gfx950's transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, source lane s names
// 4 consecutive 16-bit elements; result lane i receives, as its element e, element i % 4 of source
// lane 4e + i / 4.
__device__ __forceinline__ bf16x4 lds_read_tr4_g1(const bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4 __attribute__((address_space(3)))*)(reinterpret_cast<const s16x4*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// K fragments as load_frags_g1; V^T fragment [dt][c] (keys 32c + 4g + i and 32c + 16 + 4g + i of
// column 16 dt + r): lane (r, g) names key 32c + 4g + r / 4 (and + 16), columns 16 dt + 4 (r % 4)
// .. + 3 of the V rows, and the transposing read returns those four keys of column 16 dt + r.
__device__ __forceinline__ void load_frags_g1(const TileG1R& t, TileFragsG1<bf16>& f) {
  const int l = lane_id(), r = l & 15, g = l >> 4;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int h = 0; h < 2; ++h) f.k[kt][h] = load_frag(&t.k[16 * kt + r][32 * h + 8 * g]);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16* base = &t.v[32 * c + 4 * g + (r >> 2)][16 * dt + 4 * (r & 3)];
      const bf16x4 lo = lds_read_tr4_g1(base);
      const bf16x4 hi = lds_read_tr4_g1(base + 16 * KP);
      f.v[dt][c].v = (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
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

// fp32: the probabilities enter the value product unrounded
__device__ __forceinline__ float exp_pack_g1(const f32x4 (&x)[4], Frag8<float> (&pf)[2]) {
  float lt = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(x[2 * h + (e >> 2)][e & 3]);
      pf[h].v[e] = p;
      lt += p;
    }
  return lt;
}

// One tile: x = S^T - mc (padding keys -inf) from scores_g1; probabilities rounded to bf16 for the
// value product (bf16 inputs).
template <typename T>
__device__ __forceinline__ void softmax_pv_g1(StateG1& st, f32x4 (&x)[4], const TileFragsG1<T>& f) {
  Frag8<T> pf[2];
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
// column groups (16 rows each) per wave: two in bf16; one in fp32, whose fragments take twice the
// registers
template <typename T> struct CmpGroups { static constexpr int value = sizeof(T) == 2 ? 2 : 1; };

template <typename T>
__global__ __launch_bounds__(CW * 64) void cmp_g1_kernel(G1Args a) {
  static_assert(CW * 64 == KT * 8, "one eight-element piece of K and of V per thread");
  constexpr int CG = CmpGroups<T>::value;
  __shared__ TileG1<T> tb[2];
  const int n_rowgrp = (a.n_blk + CW * CG * 16 - 1) / (CW * CG * 16);
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wg / n_rowgrp, rg = wg % n_rowgrp;
  const int w = threadIdx.x >> 6, l = lane_id(), r = l & 15, g = l >> 4;
  const int stride = a.n_kvh * DG;
  const T* qc = reinterpret_cast<const T*>(a.q_cmp);
  const T* kb = reinterpret_cast<const T*>(a.k_cmp) + h * DG;
  const T* vb = reinterpret_cast<const T*>(a.v_cmp) + h * DG;
  const float c2 = a.scale * kLog2e;

  QG1<T> q[CG];
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
  // staging: thread t copies the eight-element piece (key t / 8, part t % 8) of both K and V; the
  // next tile's loads are issued before the current tile's compute
  const int s_key = threadIdx.x >> 3, s_part = threadIdx.x & 7;
  // (no branch around the loads and no unpacking before the store: either would make the next
  // tile's load wait at once; keys past the end repeat the last row, masked out of the scores)
  auto fetch = [&](int u, Oct<T>& kv, Oct<T>& vv) {
    const size_t off = (size_t)min(u * KT + s_key, a.n_blk - 1) * stride + s_part * 8;
    kv = load_oct(kb + off);
    vv = load_oct(vb + off);
  };
  auto store = [&](TileG1<T>& t, const Oct<T>& kv, const Oct<T>& vv) {
    store_oct(&t.k[s_key][s_part * 8], kv);
    const int pos = vt_pos_g1(s_key);
#pragma unroll
    for (int x = 0; x < 8; ++x) t.vt[s_part * 8 + x][pos] = oct_elem(vv, x);
  };
  Oct<T> kv, vv;
  fetch(0, kv, vv);
  store(tb[0], kv, vv);
  __syncthreads();
  for (int u = 0; u < ntiles; ++u) {
    const int cur = u & 1;
    if (u + 1 < ntiles) fetch(u + 1, kv, vv);
    TileFragsG1<T> f;
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
  T* o = reinterpret_cast<T*>(a.o);
  const T* gp = reinterpret_cast<const T*>(a.gates);
  typedef typename V4<T>::t v4;
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
        v4* dst = reinterpret_cast<v4*>(o + (row * a.n_qh + h) * DG + 16 * dt + 4 * g);
        *dst = __builtin_convertvector(st[c].acc[dt] * wgt, v4);
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

template <typename T, int K, int CG>
__global__ __launch_bounds__(RW * 64) void route_g1_kernel(G1Args a) {
  __shared__ T kt_lds[2][KT][KP];
  __shared__ uint32_t keys_lds[2][KT];
  __shared__ f32x4 sc_lds[RW][4][64];      // one column group's tile scores per wave, slot-major
  const int rows_per_wg = RW * CG * 16;
  const int n_rowgrp = (a.n_blk + rows_per_wg - 1) / rows_per_wg;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wg / n_rowgrp, rg = wg % n_rowgrp;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), r = l & 15, g = l >> 4;
  const int stride = a.n_kvh * DG;
  const T* qc = reinterpret_cast<const T*>(a.q_cmp);
  const T* kb = reinterpret_cast<const T*>(a.k_cmp) + h * DG;

  QG1<T> q[CG];
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
  // staging: thread t copies eight elements (key t / 8, piece t % 8) of the K tile; threads < 64
  // the keys
  const int s_key = tid >> 3, s_part = tid & 7;
  auto fetch = [&](int u, Oct<T>& kv, uint32_t& bkey) {
    const int key = u * KT + s_key;
    kv = Oct<T>{};
    if (key < a.n_blk) kv = load_oct(kb + (size_t)key * stride + s_part * 8);
    const int kk = u * KT + tid;
    bkey = (tid < KT && kk < a.n_blk) ? a.blk_key[kk] : 0u;
  };
  auto store = [&](int buf, const Oct<T>& kv, uint32_t bkey) {
    store_oct(&kt_lds[buf][s_key][s_part * 8], kv);
    if (tid < KT) keys_lds[buf][tid] = bkey;
  };
  Oct<T> kv;
  uint32_t bkey;
  fetch(0, kv, bkey);
  store(0, kv, bkey);
  __syncthreads();
  for (int u = 0; u < ntiles; ++u) {
    const int cur = u & 1;
    if (u + 1 < ntiles) fetch(u + 1, kv, bkey);
    Frag8<T> kf[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) kf[kt][hh] = load_frag(&kt_lds[cur][16 * kt + r][32 * hh + 8 * g]);
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
// compressed branch and routing in one pass (block queries)
// ---------------------------------------------------------------------------------------------
//
// The compressed branch and the routing of the selected branch read the same scores, pooled Q
// against pooled K (Speed3R page, section 2.1: the blocks are picked from the compressed
// attention's scores; with one query head per KV head the probability order is the score order).
// This kernel forms S^T = K Q^T once per tile from the raw pooled queries, ranks it for the
// routing with the products and ranking key of route_g1_kernel (so the routing rows are the same),
// and feeds scale * log2(e) * S to the compressed branch's online softmax.
//
// A row's running top-K list is spread over its four lanes: lane group g holds ranks
// [gE, gE + E) in descending order (K = 4E), so the row's K-th best key, the bound a score must
// reach to be a candidate, is lane group 3's last entry.  A candidate enters in one step of all
// four lane groups: a group whose last entry the candidate beats takes the candidate, or, when the
// candidate also beats the previous group's last entry, that entry (which the previous group
// pushes out); a bounded sorted insert of that value keeps every group sorted and the list exact.
// Each round inserts one pending candidate per row, from the row's lowest lane group that has one.
//
// The first tiles would make nearly every key a candidate.  A short first sweep over the first
// eighth of the key tiles (scores only) gives each row a lower bound T0 on its k-th best score:
// lane (r, g) keeps the 2E largest of its per-tile maxima there, each the best of 16 keys no other
// lane or tile sees, so the k-th largest of the row's 2k kept values is at most the row's k-th best
// score; the running bound starts at T0.

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = __shfl((uint32_t)v, src, 64), hi = __shfl((uint32_t)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

template <typename T, int E, int CGF>
__global__ __launch_bounds__(CW * 64) void cmp_route_g1_kernel(G1Args a) {
  static_assert(CW * 64 == KT * 8, "one eight-element piece of K and of V per thread");
  __shared__ TileG1<T> tb[2];
  __shared__ uint32_t keys_lds[2][KT];
  __shared__ f32x4 sc_lds[CW][4][64];        // one column group's tile scores per wave, slot-major
  constexpr int ROWS = CW * CGF * 16;
  const int n_rowgrp = (a.n_blk + ROWS - 1) / ROWS;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wg / n_rowgrp, rg = wg % n_rowgrp;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), r = l & 15, g = l >> 4;
  const int stride = a.n_kvh * DG;
  const T* qc = reinterpret_cast<const T*>(a.q_cmp);
  const T* kb = reinterpret_cast<const T*>(a.k_cmp) + h * DG;
  const T* vb = reinterpret_cast<const T*>(a.v_cmp) + h * DG;
  const float c2 = a.scale * kLog2e;

  QG1<T> q[CGF];
  StateG1 st[CGF];
  TopList<E> lst[CGF];
  float thr[CGF], t0[CGF];
  int row_of[CGF];
#pragma unroll
  for (int c = 0; c < CGF; ++c) {
    row_of[c] = (rg * CW * CGF + w * CGF + c) * 16 + r;
    q[c] = load_q_row(qc + ((size_t)row_of[c] * a.n_qh + h) * DG, row_of[c] < a.n_blk);   // raw
    state_init(st[c]);
    toplist_init(lst[c]);
  }
  const int ntiles = (a.n_blk + KT - 1) / KT;
  // ---- first sweep: the bound T0 from the first eighth of the key tiles (K only) ----
  {
    constexpr int E2 = 2 * E;
    const int n1 = max(1, ntiles / 8);
    const int k_key = tid >> 3, k_part = tid & 7;
    auto fetch_k = [&](int u) { return load_oct(kb + (size_t)min(u * KT + k_key, a.n_blk - 1) * stride + k_part * 8); };
    float top[CGF][E2];
#pragma unroll
    for (int c = 0; c < CGF; ++c)
#pragma unroll
      for (int e = 0; e < E2; ++e) top[c][e] = -INFINITY;
    Oct<T> kn = fetch_k(0);
    store_oct(&tb[0].k[k_key][k_part * 8], kn);
    __syncthreads();
    for (int u = 0; u < n1; ++u) {
      const int cur = u & 1;
      if (u + 1 < n1) kn = fetch_k(u + 1);
      Frag8<T> kf[4][2];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) kf[kt][hh] = load_frag(&tb[cur].k[16 * kt + r][32 * hh + 8 * g]);
      const int nk = min(KT, a.n_blk - u * KT);
#pragma unroll
      for (int c = 0; c < CGF; ++c) {
        f32x4 sc[4];
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) sc[kt] = mma16(kf[kt][1], q[c].h[1], mma16(kf[kt][0], q[c].h[0], z));
        if (nk < KT) {
#pragma unroll
          for (int j = 0; j < 16; ++j)
            sc[j >> 2][j & 3] = (16 * (j >> 2) + 4 * g + (j & 3) < nk) ? sc[j >> 2][j & 3] : -INFINITY;
        }
        const float lm = fmaxf(fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3]))),
                               fmaxf(fmaxf(fmaxf(sc[2][0], sc[2][1]), fmaxf(sc[2][2], sc[2][3])),
                                     fmaxf(fmaxf(sc[3][0], sc[3][1]), fmaxf(sc[3][2], sc[3][3]))));
        // bounded insert into the descending list: entry e becomes the median of its old value,
        // its predecessor's and lm
#pragma unroll
        for (int e = E2 - 1; e > 0; --e) top[c][e] = __builtin_amdgcn_fmed3f(top[c][e - 1], top[c][e], lm);
        top[c][0] = fmaxf(top[c][0], lm);
      }
      if (u + 1 < n1) store_oct(&tb[cur ^ 1].k[k_key][k_part * 8], kn);
      __syncthreads();
    }
    // T0 = the k-th largest of the row's 4 * E2 kept maxima: k rounds, each popping the largest
    // head among the row's four lanes (the lowest lane group on equal heads)
#pragma unroll
    for (int c = 0; c < CGF; ++c) {
      float kth = -INFINITY;
      for (int i = 0; i < 4 * E; ++i) {
        const float hd = top[c][0];
        float m = fmaxf(hd, __shfl_xor(hd, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        const uint64_t bal = __builtin_amdgcn_ballot_w64(hd == m);
        const uint32_t rowbits = (uint32_t)((bal >> r) & 1ull) | (uint32_t)((bal >> (r + 15)) & 2ull) |
                                 (uint32_t)((bal >> (r + 30)) & 4ull) | (uint32_t)((bal >> (r + 45)) & 8ull);
        if (g == __builtin_ctz(rowbits | 16u)) {
#pragma unroll
          for (int e = 0; e < E2 - 1; ++e) top[c][e] = top[c][e + 1];
          top[c][E2 - 1] = -INFINITY;
        }
        kth = m;
      }
      t0[c] = kth;
      thr[c] = kth;
    }
  }
  // staging as in cmp_g1_kernel, plus the tile's 64 ranking keys (threads < 64)
  const int s_key = tid >> 3, s_part = tid & 7;
  auto fetch = [&](int u, Oct<T>& kv, Oct<T>& vv, uint32_t& bkey) {
    const size_t off = (size_t)min(u * KT + s_key, a.n_blk - 1) * stride + s_part * 8;
    kv = load_oct(kb + off);
    vv = load_oct(vb + off);
    bkey = a.blk_key[min(u * KT + (tid & (KT - 1)), a.n_blk - 1)];
  };
  auto store = [&](int buf, const Oct<T>& kv, const Oct<T>& vv, uint32_t bkey) {
    TileG1<T>& t = tb[buf];
    store_oct(&t.k[s_key][s_part * 8], kv);
    const int pos = vt_pos_g1(s_key);
#pragma unroll
    for (int x = 0; x < 8; ++x) t.vt[s_part * 8 + x][pos] = oct_elem(vv, x);
    if (tid < KT) keys_lds[buf][tid] = bkey;
  };
  Oct<T> kv, vv;
  uint32_t bkey;
  fetch(0, kv, vv, bkey);
  store(0, kv, vv, bkey);
  __syncthreads();
  for (int u = 0; u < ntiles; ++u) {
    const int cur = u & 1;
    if (u + 1 < ntiles) fetch(u + 1, kv, vv, bkey);
    TileFragsG1<T> f;
    load_frags_g1(tb[cur], f);
    const int nk = min(KT, a.n_blk - u * KT);
    uint32_t vmask = 0xFFFFu;                 // slot j = 4*kt + i holds key 16*kt + 4*g + i
    if (nk < KT) {
      vmask = 0u;
#pragma unroll
      for (int j = 0; j < 16; ++j) vmask |= (16 * (j >> 2) + 4 * g + (j & 3) < nk) ? (1u << j) : 0u;
    }
#pragma unroll
    for (int c = 0; c < CGF; ++c) {
      f32x4 s[4];
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[kt] = mma16(f.k[kt][1], q[c].h[1], mma16(f.k[kt][0], q[c].h[0], z));
      // ---- routing: candidates reach the row's K-th best score ----
      uint32_t m = 0u;
#pragma unroll
      for (int j = 0; j < 16; ++j) m |= (s[j >> 2][j & 3] >= thr[c]) ? (1u << j) : 0u;
      m &= vmask;
      if (row_of[c] >= a.n_blk) m = 0u;       // rows past the end rank nothing
      if (__builtin_amdgcn_ballot_w64(m != 0u) != 0ull) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) sc_lds[w][kt][l] = s[kt];
        for (;;) {
          const uint64_t bal = __builtin_amdgcn_ballot_w64(m != 0u);
          if (bal == 0ull) break;
          // the previous group's last entry does not depend on this round's candidate: its
          // cross-lane reads go out first, together with the candidate's score and key reads
          const uint64_t pk = shfl_u64(lst[c].key[E - 1], (l + 48) & 63);
          const int pi = __shfl(lst[c].idx[E - 1], (l + 48) & 63, 64);
          const uint32_t rowbits = (uint32_t)((bal >> r) & 1ull) | (uint32_t)((bal >> (r + 15)) & 2ull) |
                                   (uint32_t)((bal >> (r + 30)) & 4ull) | (uint32_t)((bal >> (r + 45)) & 8ull);
          const int gs = rowbits != 0u ? __builtin_ctz(rowbits) : g;
          uint64_t ck = 0ull;
          int ci = -1;
          if (rowbits != 0u && g == gs) {
            const int j = __builtin_ctz(m);
            m &= m - 1u;
            const int key = 16 * (j >> 2) + 4 * g + (j & 3);
            const float v = reinterpret_cast<const float*>(&sc_lds[w][j >> 2][l])[j & 3];
            const uint32_t bk = keys_lds[cur][key];            // read with the score, used if it passes
            const uint64_t rk = rank_key(v, bk);
            const bool pass = v >= thr[c];
            ck = pass ? rk : 0ull;
            ci = pass ? u * KT + key : -1;
          }
          const int src = r + 16 * gs;
          ck = shfl_u64(ck, src);
          ci = __shfl(ci, src, 64);
          const bool push = g > 0 && ck > pk;
          toplist_insert(lst[c], push ? pk : ck, push ? pi : ci);
        }
        // the bound moves once per tile: a candidate that no longer beats the k-th best is only
        // dropped by the insert, so a stale bound inside the rounds changes no result
        thr[c] = fmaxf(t0[c], unord_f32((uint32_t)(shfl_u64(lst[c].key[E - 1], r + 48) >> 32)));
      }
      // ---- compressed branch: base-2 logits relative to the running reference max ----
      f32x4 x[4];
      if (nk == KT) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[kt][i] = __builtin_fmaf(s[kt][i], c2, -st[c].mc);
      } else {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            x[kt][i] = ((vmask >> (4 * kt + i)) & 1u) ? __builtin_fmaf(s[kt][i], c2, -st[c].mc) : -INFINITY;
      }
      softmax_pv_g1(st[c], x, f);
    }
    // every wave finished tile u - 1 (the previous barrier), so buffer cur ^ 1 is free
    if (u + 1 < ntiles) store(cur ^ 1, kv, vv, bkey);
    __syncthreads();
  }
  // finish: normalise, gate per token, give the block's pooled result to each of its tokens; the
  // routing row is the list itself (lane group g holds ranks gE .. gE + E - 1)
  T* o = reinterpret_cast<T*>(a.o);
  const T* gp = reinterpret_cast<const T*>(a.gates);
  typedef typename V4<T>::t v4;
  int32_t* sel = const_cast<int32_t*>(a.sel);
#pragma unroll
  for (int c = 0; c < CGF; ++c) {
    const int b = row_of[c];
    const float lsum = rows_sum(st[c].l);
    if (b >= a.n_blk) continue;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int rank = g * E + e;
      if (rank < a.top_k) sel[((size_t)b * a.n_kvh + h) * a.top_k + rank] = lst[c].key[e] == 0ull ? -1 : lst[c].idx[e];
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const int cnt = a.blk_cnt[b];
    for (int t = 0; t < a.cap; ++t) {
      const size_t row = (size_t)b * a.cap + t;
      float wgt = 0.f;
      if (t < cnt) wgt = gp ? sigmoidf_((float)gp[(row * a.n_qh + h) * a.n_gch + a.ch_cmp]) * inv : inv;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        v4* dst = reinterpret_cast<v4*>(o + (row * a.n_qh + h) * DG + 16 * dt + 4 * g);
        *dst = __builtin_convertvector(st[c].acc[dt] * wgt, v4);
      }
    }
  }
}

template <typename T, int E, int CGF>
hipError_t launch_cmp_route_g1_k(const G1Args& a, hipStream_t s) {
  const int n_rowgrp = (a.n_blk + CW * CGF * 16 - 1) / (CW * CGF * 16);
  hipLaunchKernelGGL((cmp_route_g1_kernel<T, E, CGF>), dim3(n_rowgrp * a.n_kvh), dim3(CW * 64), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// selected branch with block routing rows: one wave per (query block, head)
// ---------------------------------------------------------------------------------------------

// Append the valid token slots of lane l's block `blk` (when `on`) to a packed key list after its
// first `total` entries, in lane order; returns the new length.
__device__ __forceinline__ int pack_block_tokens(int* keys, int total, int blk, bool on, const int32_t* blk_cnt,
                                                 int cap) {
  const int l = lane_id();
  const int c = on ? blk_cnt[blk] : 0;
  int inc = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, 64);
    if (l >= o) inc += y;
  }
  for (int t = 0; t < c; ++t) keys[total + inc - c + t] = blk * cap + t;
  return total + __builtin_amdgcn_readlane(inc, 63);
}

// Two waves per SIMD (at most 256 registers each) where LDS allows eight workgroups per CU; the
// fp32 tile (twice the LDS and registers) allows fewer.
template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 4 ? 1 : 2)))
void sel_g1_kernel(G1Args a) {
  __shared__ typename SelTile<T>::type tb;
  // source rows of the selected valid tokens, packed: (entries x blk_cap + KT) ints, sized at launch
  // so that eight bf16 workgroups fit a compute unit's LDS at top_k 16 and blk_cap 16
  extern __shared__ int keys_lds[];
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int b = wg / a.n_kvh, h = wg % a.n_kvh;
  const int l = lane_id(), r = l & 15, g = l >> 4;
  const int cap = a.cap, cnt = a.blk_cnt[b];
  const int stride = a.n_kvh * DG;
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* kb = reinterpret_cast<const T*>(a.k) + h * DG;
  const T* vb = reinterpret_cast<const T*>(a.v) + h * DG;
  const float c2 = a.scale * kLog2e;
  // loads that do not depend on the routing row are issued first, so their round trips overlap
  // the row's: the token's query, its gate logit and (accumulating) the output written before
  const bool valid = r < cnt;
  const size_t row = (size_t)b * cap + min(r, cap - 1);
  const QG1<T> qq = load_q_row(q + (row * a.n_qh + h) * DG, valid, c2);
  T* o = reinterpret_cast<T*>(a.o);
  const T* gp = reinterpret_cast<const T*>(a.gates);
  const float glog = (gp && valid) ? (float)gp[(row * a.n_qh + h) * a.n_gch + a.ch_sel] : 0.f;
  typedef typename V4<T>::t v4;
  v4 prev[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    prev[dt] = v4{};
    if (a.accumulate && valid) prev[dt] = *reinterpret_cast<const v4*>(o + (row * a.n_qh + h) * DG + 16 * dt + 4 * g);
  }
  // lane x < top_k holds entry x of this block's routing row for head h; -1, out-of-range and
  // repeated entries count no keys; the valid tokens of the rest are packed one after another
  // (local branch: the one entry is the block itself)
  const int grp = a.sel_groups == 1 ? 0 : h;
  const int n_ent = a.local ? 1 : a.top_k;
  const int sb = a.local ? (l == 0 ? b : -1) : (l < a.top_k ? a.sel[((size_t)b * a.sel_groups + grp) * a.top_k + l] : -1);
  bool keep = sb >= 0 && sb < a.n_blk;
  for (int y = 0; y < n_ent; ++y) {
    const int sy = __builtin_amdgcn_readlane(sb, y);
    keep = keep && !(y < l && sy == sb);
  }
  const int total = pack_block_tokens(keys_lds, 0, sb, keep, a.blk_cnt, cap);
  const int ntiles = (total + KT - 1) / KT;
  for (int i = total + l; i < ntiles * KT; i += 64) keys_lds[i] = -1;
  __syncthreads();
  StateG1 st;
  state_init(st);
  RowsG1<T, 64> pre;
  if (ntiles > 0) gather_rows_g1<64>(pre, kb, vb, stride, keys_lds, l);
  for (int u = 0; u < ntiles; ++u) {
    store_rows_g1<64>(tb, pre, l);
    __syncthreads();
    if (u + 1 < ntiles) gather_rows_g1<64>(pre, kb, vb, stride, keys_lds + (u + 1) * KT, l);
    TileFragsG1<T> f;
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
  if (r < cap) {
    if (a.lse && g == 0) a.lse[row * a.n_qh + h] = (valid && lsum > 0.f) ? (st.mc + __log2f(lsum)) * kLn2 : -INFINITY;
    const float wgt = valid ? (gp ? sigmoidf_(glog) * inv : inv) : 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      v4* dst = reinterpret_cast<v4*>(o + (row * a.n_qh + h) * DG + 16 * dt + 4 * g);
      f32x4 v = st.acc[dt] * wgt;
      if (a.accumulate && valid) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += (float)prev[dt][i];
      }
      *dst = __builtin_convertvector(v, v4);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// selected branch with a forced block range: NQ query blocks of one head per wave
// ---------------------------------------------------------------------------------------------
//
// The forced range (Speed3R page, section 2.2: the reference frame's tokens, attended by every
// query) is the same key set for every query block, and fetching it is most of the branch's cost
// when each (block, head) wave gathers it alone.  A wave here serves NQ consecutive query blocks
// of one head: it runs each block over the block's routed blocks outside the range, one block
// after the other (as sel_g1_kernel does); then the FW waves of the workgroup gather the range's
// valid tokens together, once per tile for all their FW * NQ blocks, each tile continuing every
// block's online softmax.  Each block's key set is the union of its routed blocks and the range,
// every block once; only the order in which its keys are visited differs from one packed list.

// query blocks per wave: the most that keep the kernel free of scratch at one wave per SIMD (bf16:
// 8.3, 7.5 and 7.1 ms for 4, 5 and 6 blocks, one wave per workgroup, at the speed3r shape with the
// reference frame forced, where one block per wave took 20.5 ms)
template <typename T> struct ForcedGroup { static constexpr int value = sizeof(T) == 2 ? 6 : 2; };
// waves per workgroup: FW * NQ query blocks share each gathered range tile (7.12 -> 6.80 ms for
// FW = 1 -> 2 at the same shape; the range's gather is then no longer what bounds the kernel)
constexpr int FW = 2;

// Wave-local ordering of LDS accesses (a wave's own LDS operations complete in issue order).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T, int NQ>
__global__ __launch_bounds__(FW * 64) __attribute__((amdgpu_waves_per_eu(1))) void sel_forced_g1_kernel(G1Args a) {
  // wave w's tile and key list for its blocks' routed parts; the FW tiles then double-buffer the
  // shared range
  __shared__ typename SelTile<T>::type tb[FW];
  __shared__ int keys_w[FW][64 * 16 + KT];
  __shared__ int keys_f[kMaxForcedBlocks * 16 + KT];
  __shared__ int f_total;
  static_assert(FW == 2, "the range's tiles are double-buffered in the FW wave tiles");
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bg = wg / a.n_kvh, h = wg % a.n_kvh;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id(), r = l & 15, g = l >> 4;
  const int b0 = (bg * FW + w) * NQ;               // this wave's first query block
  const int cap = a.cap;
  const int stride = a.n_kvh * DG;
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* kb = reinterpret_cast<const T*>(a.k) + h * DG;
  const T* vb = reinterpret_cast<const T*>(a.v) + h * DG;
  const float c2 = a.scale * kLog2e;
  T* o = reinterpret_cast<T*>(a.o);
  const T* gp = reinterpret_cast<const T*>(a.gates);
  typedef typename V4<T>::t v4;
  const int grp = a.sel_groups == 1 ? 0 : h;
  const int nf = a.f_hi - a.f_lo;
  // every block's query (blocks past the end: none valid)
  QG1<T> qq[NQ];
  StateG1 st[NQ];
  int cnt[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int b = b0 + j;
    cnt[j] = b < a.n_blk ? a.blk_cnt[b] : 0;
    const size_t row = (size_t)min(b, a.n_blk - 1) * cap + min(r, cap - 1);
    qq[j] = load_q_row(q + (row * a.n_qh + h) * DG, r < cnt[j], c2);
    state_init(st[j]);
  }
  // each block's routed blocks outside the range (lane x < top_k: entry x; -1, out-of-range and
  // repeated entries count no keys), in the wave's own tile: no workgroup barrier, since the
  // waves' tile counts differ
  typename SelTile<T>::type& tw = tb[w];
  int* kw = keys_w[w];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int b = b0 + j;
    if (b >= a.n_blk) break;
    const int sb = l < a.top_k ? a.sel[((size_t)b * a.sel_groups + grp) * a.top_k + l] : -1;
    bool keep = sb >= 0 && sb < a.n_blk && !(sb >= a.f_lo && sb - a.f_lo < nf);
    for (int y = 0; y < a.top_k; ++y) {
      const int sy = __builtin_amdgcn_readlane(sb, y);
      keep = keep && !(y < l && sy == sb);
    }
    const int total = pack_block_tokens(kw, 0, sb, keep, a.blk_cnt, cap);
    const int ntiles = (total + KT - 1) / KT;
    for (int i = total + l; i < ntiles * KT; i += 64) kw[i] = -1;
    wave_sync();
    RowsG1<T, 64> pre;
    if (ntiles > 0) gather_rows_g1<64>(pre, kb, vb, stride, kw, l);
    for (int u = 0; u < ntiles; ++u) {
      store_rows_g1<64>(tw, pre, l);
      wave_sync();
      if (u + 1 < ntiles) gather_rows_g1<64>(pre, kb, vb, stride, kw + (u + 1) * KT, l);
      TileFragsG1<T> f;
      load_frags_g1(tw, f);
      const int nk = min(KT, total - u * KT);
      f32x4 cm[4], seed[4], x[4];
      if (nk < KT) mask_seed(nk, cm);
      row_seed(st[j], nk == KT, cm, seed);
      scores_g1(f, qq[j], seed, x);
      softmax_pv_g1(st[j], x, f);
      wave_sync();
    }
  }
  // the range's valid tokens (64 blocks per packing step), each tile gathered once by the whole
  // workgroup for its FW * NQ blocks
  __syncthreads();
  if (w == 0) {
    int total = 0;
    for (int f0 = 0; f0 < nf; f0 += 64)
      total = pack_block_tokens(keys_f, total, a.f_lo + f0 + l, f0 + l < nf, a.blk_cnt, cap);
    const int nt = (total + KT - 1) / KT;
    for (int i = total + l; i < nt * KT; i += 64) keys_f[i] = -1;
    if (l == 0) f_total = total;
  }
  __syncthreads();
  const int total_f = f_total;
  const int nft = (total_f + KT - 1) / KT;
  RowsG1<T, FW * 64> pf;
  if (nft > 0) gather_rows_g1<FW * 64>(pf, kb, vb, stride, keys_f, tid);
  for (int u = 0; u < nft; ++u) {
    // buffer u & 1 was last read in tile u - 2, before every wave passed the previous barrier
    store_rows_g1<FW * 64>(tb[u & 1], pf, tid);
    __syncthreads();
    if (u + 1 < nft) gather_rows_g1<FW * 64>(pf, kb, vb, stride, keys_f + (u + 1) * KT, tid);
    TileFragsG1<T> f;
    load_frags_g1(tb[u & 1], f);
    const int nk = min(KT, total_f - u * KT);
    f32x4 cm[4];
    if (nk < KT) mask_seed(nk, cm);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      if (cnt[j] == 0) continue;
      f32x4 seed[4], x[4];
      row_seed(st[j], nk == KT, cm, seed);
      scores_g1(f, qq[j], seed, x);
      softmax_pv_g1(st[j], x, f);
    }
  }
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int b = b0 + j;
    if (b >= a.n_blk) break;
    const float lsum = rows_sum(st[j].l);
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const bool valid = r < cnt[j];
    const size_t row = (size_t)b * cap + min(r, cap - 1);
    if (r < cap) {
      if (a.lse && g == 0) a.lse[row * a.n_qh + h] = (valid && lsum > 0.f) ? (st[j].mc + __log2f(lsum)) * kLn2 : -INFINITY;
      const float glog = (gp && valid) ? (float)gp[(row * a.n_qh + h) * a.n_gch + a.ch_sel] : 0.f;
      const float wgt = valid ? (gp ? sigmoidf_(glog) * inv : inv) : 0.f;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        v4* dst = reinterpret_cast<v4*>(o + (row * a.n_qh + h) * DG + 16 * dt + 4 * g);
        f32x4 v = st[j].acc[dt] * wgt;
        if (a.accumulate && valid) v += __builtin_convertvector(*dst, f32x4);
        *dst = __builtin_convertvector(v, v4);
      }
    }
  }
}

template <typename T, int K, int CG>
hipError_t launch_route_g1_k(const G1Args& a, hipStream_t s) {
  const int n_rowgrp = (a.n_blk + RW * CG * 16 - 1) / (RW * CG * 16);
  hipLaunchKernelGGL((route_g1_kernel<T, K, CG>), dim3(n_rowgrp * a.n_kvh), dim3(RW * 64), 0, s, a);
  return hipGetLastError();
}

// fp32 takes one column group per wave throughout: its query fragments and key tile take twice the
// registers of bf16 ones
template <typename T>
hipError_t launch_route_g1_t(const G1Args& a, hipStream_t s) {
  constexpr int C2 = sizeof(T) == 2 ? 2 : 1;
  if (a.top_k <= 8) return launch_route_g1_k<T, 8, C2>(a, s);
  if (a.top_k <= 16) return launch_route_g1_k<T, 16, C2>(a, s);
  if (a.top_k <= 32) return launch_route_g1_k<T, 32, 1>(a, s);
  return launch_route_g1_k<T, 64, 1>(a, s);
}

// dynamic LDS of sel_g1_kernel: the packed key list of one query block's selection
size_t sel_g1_keys_lds(const G1Args& a) {
  return (size_t)((a.local ? 1 : a.top_k) * a.cap + KT) * sizeof(int);
}

hipError_t launch_attn_g1_routed_bf16(const G1Args& a0, hipStream_t s) {
  G1Args a = a0;
  hipError_t e;
  if (a.top_k <= 8) e = launch_cmp_route_g1_k<bf16, 2, 2>(a, s);
  else if (a.top_k <= 16) e = launch_cmp_route_g1_k<bf16, 4, 2>(a, s);
  else e = launch_cmp_route_g1_k<bf16, 8, 1>(a, s);
  if (e != hipSuccess) return e;
  a.accumulate = 1;
  hipLaunchKernelGGL(sel_g1_kernel<bf16>, dim3(a.n_blk * a.n_kvh), dim3(64), sel_g1_keys_lds(a), s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attn_g1_t(const G1Args& a0, hipStream_t s) {
  G1Args a = a0;
  if (a.branches & 1) {
    constexpr int CG = CmpGroups<T>::value;
    const int n_rowgrp = (a.n_blk + CW * CG * 16 - 1) / (CW * CG * 16);
    hipLaunchKernelGGL(cmp_g1_kernel<T>, dim3(n_rowgrp * a.n_kvh), dim3(CW * 64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.branches & 2) {
    a.accumulate = (a.branches & 1) ? 1 : 0;
    a.local = 0;
    if (a.f_hi > a.f_lo) {
      constexpr int NB = ForcedGroup<T>::value * FW;   // query blocks per workgroup
      hipLaunchKernelGGL((sel_forced_g1_kernel<T, ForcedGroup<T>::value>), dim3((a.n_blk + NB - 1) / NB * a.n_kvh),
                         dim3(FW * 64), 0, s, a);
    } else {
      hipLaunchKernelGGL(sel_g1_kernel<T>, dim3(a.n_blk * a.n_kvh), dim3(64), sel_g1_keys_lds(a), s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.branches & 4) {
    // local branch: the selected branch's kernel with the block's own block as its one entry
    a.accumulate = (a.branches & 3) ? 1 : 0;
    a.local = 1;
    a.ch_sel = a.ch_loc;
    a.f_lo = a.f_hi = 0;
    hipLaunchKernelGGL(sel_g1_kernel<T>, dim3(a.n_blk * a.n_kvh), dim3(64), sel_g1_keys_lds(a), s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_route_g1(int is_bf16, const G1Args& a, hipStream_t s) {
  return is_bf16 ? launch_route_g1_t<bf16>(a, s) : launch_route_g1_t<float>(a, s);
}

hipError_t launch_attn_g1_routed(int is_bf16, const G1Args& a, hipStream_t s) {
  if (is_bf16) return launch_attn_g1_routed_bf16(a, s);
  // fp32: the routing pass, then the compressed and selected branches (the fused pass's ranked lists
  // next to fp32 tiles exceed the registers of two waves per SIMD); the same rows and outputs
  hipError_t e = launch_route_g1_t<float>(a, s);
  if (e != hipSuccess) return e;
  return launch_attn_g1_t<float>(a, s);
}

hipError_t launch_attn_g1(int is_bf16, const G1Args& a, hipStream_t s) {
  return is_bf16 ? launch_attn_g1_t<bf16>(a, s) : launch_attn_g1_t<float>(a, s);
}

}  // namespace nsa
