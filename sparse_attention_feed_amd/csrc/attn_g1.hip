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

// Query fragments (two d halves) of one row: B operand of S^T.
struct QG1 { Frag8<bf16> h[2]; };

__device__ __forceinline__ QG1 load_q_row(const bf16* row, bool valid) {
  QG1 q;
  const int g = lane_id() >> 4;
  if (valid) {
    q.h[0] = ld8(row + 8 * g);
    q.h[1] = ld8(row + 32 + 8 * g);
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

// Stage 64 keys into LDS: rows given by a per-key source row (or -1 for padding: zero).  Every thread
// of the group (nt threads) copies 16-byte pieces; V goes to the permuted transposed layout.
__device__ __forceinline__ void stage_rows_g1(TileG1& t, const bf16* kb, const bf16* vb, int stride,
                                              const int* rows /* LDS [64] */, int tid, int nt) {
  for (int c = tid; c < 2 * KT * 8; c += nt) {       // 8 pieces of 8 elements per 64-element row
    const bool isv = c >= KT * 8;
    const int cc = isv ? c - KT * 8 : c;
    const int key = cc >> 3, part = cc & 7;
    const int src = rows[key];
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (src >= 0) val = *reinterpret_cast<const uint4*>((isv ? vb : kb) + (size_t)src * stride + part * 8);
    if (!isv) {
      *reinterpret_cast<uint4*>(&t.k[key][part * 8]) = val;
    } else {
      const bf16* e = reinterpret_cast<const bf16*>(&val);
      const int pos = vt_pos_g1(key);
#pragma unroll
      for (int x = 0; x < 8; ++x) t.vt[part * 8 + x][pos] = e[x];
    }
  }
}

// Online softmax state of one column group (16 rows of one head).
struct StateG1 {
  f32x4 acc[4];             // O^T[d = 16*dt + 4*(lane/16) + i][row lane%16]
  float m;                  // running max of raw scores for row lane%16 (identical across lane groups)
  float l;                  // this lane group's share of the sum
};

__device__ __forceinline__ void state_init(StateG1& s) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) s.acc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  s.m = -INFINITY;
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

// One tile: scores s (raw, padding keys already -inf), exact running max (the max costs little next
// to the 16 MFMAs per tile at head dim 64), probabilities rounded to bf16 for the value product.
__device__ __forceinline__ void softmax_pv_g1(StateG1& st, const f32x4 (&s)[4], const TileFragsG1& f, float c2) {
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kt][i]);
  mx = rows_max(mx);
  const float mn = fmaxf(st.m, mx);
  // (mn stays -inf only if no key has been valid yet; every probability is then exactly 0)
  const float alpha = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((st.m - mn) * c2);
  const float mcn = mn == -INFINITY ? 0.f : mn * c2;
  Frag8<bf16> pf[2];
  float lt = 0.f;
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int kt = 2 * h + (e >> 2), i = e & 3;
      f32x2 p;
      p[0] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i], c2, -mcn));
      p[1] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i + 1], c2, -mcn));
      const bf16x2 pb = __builtin_convertvector(p, bf16x2);
      pf[h].v[e] = pb[0];
      pf[h].v[e + 1] = pb[1];
      lt = __builtin_amdgcn_fdot2_f32_bf16(pb, one, lt, false);
    }
  st.l = st.l * alpha + lt;
  st.m = mn;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    st.acc[dt] *= alpha;
#pragma unroll
    for (int c = 0; c < 2; ++c) st.acc[dt] = mma16(f.v[dt][c], pf[c], st.acc[dt]);
  }
}

__device__ __forceinline__ void mask_seed(int nk, const bool* kvalid /* LDS or null */, f32x4 (&seed)[4]) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 16 * kt + 4 * g + i;
      const bool ok = key < nk && (kvalid == nullptr || kvalid[key]);
      seed[kt][i] = ok ? 0.f : -INFINITY;
    }
}

// ---------------------------------------------------------------------------------------------
// compressed branch with block queries
// ---------------------------------------------------------------------------------------------

constexpr int CW = 8;       // waves per workgroup
constexpr int CG = 2;       // column groups (16 rows each) per wave

__global__ __launch_bounds__(CW * 64) void cmp_g1_kernel(G1Args a) {
  __shared__ TileG1 tb[2];
  __shared__ int rows_lds[2][KT];
  const int nt = CW * 64;
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
    q[c] = load_q_row(qc + ((size_t)row_of[c] * a.n_qh + h) * DG, ok);
    state_init(st[c]);
  }
  const int ntiles = (a.n_blk + KT - 1) / KT;
  for (int i = threadIdx.x; i < KT; i += nt) rows_lds[0][i] = i < a.n_blk ? i : -1;
  __syncthreads();
  stage_rows_g1(tb[0], kb, vb, stride, rows_lds[0], threadIdx.x, nt);
  __syncthreads();
  for (int u = 0; u < ntiles; ++u) {
    const int cur = u & 1;
    if (u + 1 < ntiles) {
      for (int i = threadIdx.x; i < KT; i += nt) {
        const int key = (u + 1) * KT + i;
        rows_lds[cur ^ 1][i] = key < a.n_blk ? key : -1;
      }
    }
    TileFragsG1 f;
    load_frags_g1(tb[cur], f);
    const int nk = min(KT, a.n_blk - u * KT);
    f32x4 seed[4];
    mask_seed(nk, nullptr, seed);
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      f32x4 s[4];
      scores_g1(f, q[c], seed, s);
      softmax_pv_g1(st[c], s, f, c2);
    }
    __syncthreads();
    if (u + 1 < ntiles) stage_rows_g1(tb[cur ^ 1], kb, vb, stride, rows_lds[cur ^ 1], threadIdx.x, nt);
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
    if (a.lse && g == 0) a.lse[(size_t)b * a.n_qh + h] = lsum > 0.f ? st[c].m * a.scale + __logf(lsum) : -INFINITY;
    const int cnt = a.blk_cnt[b];
    for (int t = 0; t < a.cap; ++t) {
      const size_t row = (size_t)b * a.cap + t;
      float wgt = 0.f;
      if (t < cnt) wgt = gp ? sigmoidf_((float)gp[(row * a.n_qh + h) * a.n_gch + a.ch_cmp]) * inv : inv;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        bf16* dst = o + (row * a.n_qh + h) * DG + 16 * dt + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = (bf16)(st[c].acc[dt][i] * wgt);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// routing: top-k blocks per (query block, head) by compressed score, no score matrix stored
// ---------------------------------------------------------------------------------------------

constexpr int RW = 8;       // waves per workgroup; one column group (16 query rows) per wave

__device__ __forceinline__ bool rbetter(float v, uint32_t k, float v2, uint32_t k2) {
  return v > v2 || (v == v2 && k < k2);
}

template <int K>
__global__ __launch_bounds__(RW * 64) void route_g1_kernel(G1Args a) {
  __shared__ TileG1 tb[2];
  __shared__ int rows_lds[2][KT];
  __shared__ uint32_t keys_lds[2][KT];
  const int nt = RW * 64;
  const int n_rowgrp = (a.n_blk + RW * 16 - 1) / (RW * 16);
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wg / n_rowgrp, rg = wg % n_rowgrp;
  const int w = threadIdx.x >> 6, l = lane_id(), r = l & 15, g = l >> 4;
  const int stride = a.n_kvh * DG;
  const bf16* qc = reinterpret_cast<const bf16*>(a.q_cmp);
  const bf16* kb = reinterpret_cast<const bf16*>(a.k_cmp) + h * DG;
  const int row = (rg * RW + w) * 16 + r;
  const QG1 q = load_q_row(qc + ((size_t)row * a.n_qh + h) * DG, row < a.n_blk);

  float bv[K];
  uint32_t bk[K];
  int bi[K];
#pragma unroll
  for (int x = 0; x < K; ++x) {
    bv[x] = -INFINITY;
    bk[x] = 0xFFFFFFFFu;
    bi[x] = -1;
  }
  const int ntiles = (a.n_blk + KT - 1) / KT;
  for (int i = threadIdx.x; i < KT; i += nt) {
    rows_lds[0][i] = i < a.n_blk ? i : -1;
    keys_lds[0][i] = i < a.n_blk ? a.blk_key[i] : 0u;
  }
  __syncthreads();
  stage_rows_g1(tb[0], kb, kb, stride, rows_lds[0], threadIdx.x, nt);   // V part unused
  __syncthreads();
  for (int u = 0; u < ntiles; ++u) {
    const int cur = u & 1;
    if (u + 1 < ntiles) {
      for (int i = threadIdx.x; i < KT; i += nt) {
        const int key = (u + 1) * KT + i;
        rows_lds[cur ^ 1][i] = key < a.n_blk ? key : -1;
        keys_lds[cur ^ 1][i] = key < a.n_blk ? a.blk_key[key] : 0u;
      }
    }
    TileFragsG1 f;
    load_frags_g1(tb[cur], f);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const f32x4 zs[4] = {z, z, z, z};
    f32x4 s[4];
    scores_g1(f, q, zs, s);
    const int nk = min(KT, a.n_blk - u * KT);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * kt + 4 * g + i;
        if (key >= nk) continue;
        const float v = s[kt][i];
        const uint32_t kk = keys_lds[cur][key];
        if (rbetter(v, kk, bv[K - 1], bk[K - 1])) {
          const int idx = u * KT + key;
#pragma unroll
          for (int x = K - 1; x > 0; --x) {
            const bool bp = rbetter(v, kk, bv[x - 1], bk[x - 1]);
            const bool bc = rbetter(v, kk, bv[x], bk[x]);
            if (bp) {
              bv[x] = bv[x - 1];
              bk[x] = bk[x - 1];
              bi[x] = bi[x - 1];
            } else if (bc) {
              bv[x] = v;
              bk[x] = kk;
              bi[x] = idx;
            }
          }
          if (rbetter(v, kk, bv[0], bk[0])) {
            bv[0] = v;
            bk[0] = kk;
            bi[0] = idx;
          }
        }
      }
    __syncthreads();
    if (u + 1 < ntiles) stage_rows_g1(tb[cur ^ 1], kb, kb, stride, rows_lds[cur ^ 1], threadIdx.x, nt);
    __syncthreads();
  }
  // merge the four lane groups' lists of each row (lanes r, r+16, r+32, r+48): top_k rounds of an
  // arg-best over the four list heads
  if (row < a.n_blk) {
    int32_t* so = const_cast<int32_t*>(a.sel) + ((size_t)row * a.n_kvh + h) * a.top_k;
    for (int x = 0; x < a.top_k; ++x) {
      float v = bv[0];
      uint32_t kk = bk[0];
      int src = g;
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        const float v2 = __shfl_xor(v, o, 64);
        const uint32_t k2 = __shfl_xor(kk, o, 64);
        const int s2 = __shfl_xor(src, o, 64);
        if (rbetter(v2, k2, v, kk)) {
          v = v2;
          kk = k2;
          src = s2;
        }
      }
      const int win = __shfl(bi[0], r + 16 * src, 64);
      if (g == 0) so[x] = (v == -INFINITY) ? -1 : win;
      if (g == src) {
#pragma unroll
        for (int y = 0; y < K - 1; ++y) {
          bv[y] = bv[y + 1];
          bk[y] = bk[y + 1];
          bi[y] = bi[y + 1];
        }
        bv[K - 1] = -INFINITY;
        bk[K - 1] = 0xFFFFFFFFu;
        bi[K - 1] = -1;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// selected branch with block routing rows: one wave per (query block, head)
// ---------------------------------------------------------------------------------------------

__global__ __launch_bounds__(64) void sel_g1_kernel(G1Args a) {
  __shared__ TileG1 tb;
  __shared__ int rows_lds[KT];
  __shared__ bool kvalid[KT];
  __shared__ int blist[64];
  __shared__ int nlist;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int b = wg / a.n_kvh, h = wg % a.n_kvh;
  const int l = lane_id(), r = l & 15, g = l >> 4;
  const int cap = a.cap, cnt = a.blk_cnt[b];
  const int stride = a.n_kvh * DG;
  const bf16* q = reinterpret_cast<const bf16*>(a.q);
  const bf16* kb = reinterpret_cast<const bf16*>(a.k) + h * DG;
  const bf16* vb = reinterpret_cast<const bf16*>(a.v) + h * DG;
  const float c2 = a.scale * kLog2e;
  // this block's selected blocks for head h, duplicates and -1 removed (order kept)
  const int grp = a.sel_groups == 1 ? 0 : h;
  const int32_t* srow = a.sel + ((size_t)b * a.sel_groups + grp) * a.top_k;
  if (l == 0) {
    int n = 0;
    for (int x = 0; x < a.top_k; ++x) {
      const int s = srow[x];
      if (s < 0 || s >= a.n_blk) continue;
      bool dup = false;
      for (int y = 0; y < n; ++y) dup |= blist[y] == s;
      if (!dup) blist[n++] = s;
    }
    nlist = n;
  }
  __syncthreads();
  const int nb = nlist;
  const int per = KT / cap;                       // blocks per 64-key tile
  const int ntiles = (nb + per - 1) / per;
  StateG1 st;
  state_init(st);
  const QG1 qq = load_q_row(q + ((size_t)(b * cap + r) * a.n_qh + h) * DG, r < cnt);
  for (int u = 0; u < ntiles; ++u) {
    // key slot i of the tile: block blist[u*per + i/cap], token i%cap
    {
      const int i = l;
      const int bi = u * per + i / cap, tk = i % cap;
      int src = -1;
      if (i < per * cap && bi < nb) {
        const int blk = blist[bi];
        if (tk < a.blk_cnt[blk]) src = blk * cap + tk;
      }
      rows_lds[i] = src;
      kvalid[i] = src >= 0;
    }
    __syncthreads();
    stage_rows_g1(tb, kb, vb, stride, rows_lds, l, 64);
    __syncthreads();
    TileFragsG1 f;
    load_frags_g1(tb, f);
    f32x4 seed[4];
    mask_seed(KT, kvalid, seed);
    f32x4 s[4];
    scores_g1(f, qq, seed, s);
    softmax_pv_g1(st, s, f, c2);
    __syncthreads();
  }
  const float lsum = rows_sum(st.l);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  bf16* o = reinterpret_cast<bf16*>(a.o);
  const bf16* gp = reinterpret_cast<const bf16*>(a.gates);
  if (r < cap) {
    const size_t row = (size_t)b * cap + r;
    if (a.lse && g == 0) a.lse[row * a.n_qh + h] = (r < cnt && lsum > 0.f) ? st.m * a.scale + __logf(lsum) : -INFINITY;
    const bool valid = r < cnt;
    const float wgt = valid ? (gp ? sigmoidf_((float)gp[(row * a.n_qh + h) * a.n_gch + a.ch_sel]) * inv : inv) : 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      bf16* dst = o + (row * a.n_qh + h) * DG + 16 * dt + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = st.acc[dt][i] * wgt;
        if (a.accumulate && valid) v += (float)dst[i];
        dst[i] = (bf16)v;
      }
    }
  }
}

template <int K>
hipError_t launch_route_g1_k(const G1Args& a, hipStream_t s) {
  const int n_rowgrp = (a.n_blk + RW * 16 - 1) / (RW * 16);
  hipLaunchKernelGGL(route_g1_kernel<K>, dim3(n_rowgrp * a.n_kvh), dim3(RW * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_g1(const G1Args& a, hipStream_t s) {
  if (a.top_k <= 8) return launch_route_g1_k<8>(a, s);
  if (a.top_k <= 16) return launch_route_g1_k<16>(a, s);
  if (a.top_k <= 32) return launch_route_g1_k<32>(a, s);
  return launch_route_g1_k<64>(a, s);
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
    hipLaunchKernelGGL(sel_g1_kernel, dim3(a.n_blk * a.n_kvh), dim3(64), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace nsa
