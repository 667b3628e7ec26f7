// NSA attention branches (compressed / selected / local) with a fused sigmoid-gate epilogue, and the
// stage-1 dense gated self/cross attention, for gfx950.
//
// Math (LSRM pages, hyper.ai summary of arXiv 2604.05182, section 方法; Speed3R page, section 2.1):
// per query row and head, o = softmax(scale * q K^T) V over a branch's key set, then
// o = sum_c sigmoid(g_c) o_c over the branches.
//
// Work decomposition.  One workgroup owns one storage block (up to 64 query slots) and one KV
// head j.  The 16 query heads of group j that share KV head j form the N = 16 columns of every MFMA,
// so a K/V tile staged once in LDS serves all 16 heads of every token of the block.
//
// Per 64-key tile and token (all in registers, transposed so no cross-lane moves are needed):
//   S^T[key][head] = K Q^T     4 x v_mfma_f32_16x16x32_bf16 (A = K rows from LDS, B = the token's q)
//   lane (l) then holds head l%16 and keys 16*kt + 4*(l/16) + i, i.e. one head per lane;
//   online softmax in base 2 (running max, rescale factor, row sum) per lane;
//   O^T[d][head] += V^T P^T    4 MFMAs, B = P straight from the S^T registers (bf16), A = V^T from
//   LDS, where V is stored transposed with the key order permuted so that each lane's eight
//   probabilities line up with eight contiguous V^T elements.
// The f32 variant issues eight v_mfma_f32_16x16x4f32 per step on the same lane data.
#include "attn_tile.h"
#include "common.h"
#include "kernels.h"

namespace nsa {
namespace {

constexpr int TILE = 64;     // keys per LDS tile
constexpr int HD = 32;       // head dim of the compiled kernels
constexpr int GRP = 16;      // query heads per KV head of the compiled kernels

template <typename T> struct Pad;
template <> struct Pad<bf16> { static constexpr int K = 40, V = 72; };   // LDS row strides (elements)
template <> struct Pad<float> { static constexpr int K = 36, V = 68; };

template <typename T> struct TileBuf {
  T k[TILE][Pad<T>::K];
  T vt[HD][Pad<T>::V];
};

// Column of V^T (LDS) holding key `key` of the tile: lane group g of an MFMA step over keys
// [32c, 32c+32) reads probabilities of keys {32c+4g+i, 32c+16+4g+i}, i<4, as k-slots 8g..8g+7.
__device__ __forceinline__ int vt_pos(int key) {
  int c = key >> 5, r = key & 31;
  int hi = r >> 4, rr = r & 15;
  return 32 * c + 8 * (rr >> 2) + 4 * hi + (rr & 3);
}

template <typename T, int NT> struct Stager {
  static constexpr int E = 16 / sizeof(T);        // elements per 16-byte chunk
  static constexpr int CPR = HD / E;               // chunks per key row
  static constexpr int CH = TILE * CPR;            // chunks per tensor per tile
  static constexpr int PER = (2 * CH + NT - 1) / NT;
  uint4 r[PER];

  __device__ __forceinline__ void load(const T* kb, const T* vb, int stride, int nk) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int c = threadIdx.x + i * NT;
      if (c < 2 * CH) {
        bool isv = c >= CH;
        int cc = isv ? c - CH : c;
        int key = cc / CPR, part = cc % CPR;
        if (key < nk)   // 32-bit offset within the tile: key < TILE, so key * stride fits
          r[i] = *reinterpret_cast<const uint4*>((isv ? vb : kb) + (key * stride + part * E));
        else
          r[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  // Every lane loads: rows at or beyond nk repeat row nk - 1 (row 0 if nk < 1), which the -inf
  // seed of the padding keys masks out of every result.  With no branch around the load, the
  // wait before the store of this set need not cover a load issued later into another set.
  __device__ __forceinline__ void load_all(const T* kb, const T* vb, int stride, int nk) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int c = threadIdx.x + i * NT;
      if (PER * NT == 2 * CH || c < 2 * CH) {     // no branch when the threads cover the tile exactly
        bool isv = c >= CH;
        int cc = isv ? c - CH : c;
        int key = min(cc / CPR, max(nk - 1, 0)), part = cc % CPR;
        r[i] = *reinterpret_cast<const uint4*>((isv ? vb : kb) + (key * stride + part * E));
      }
    }
  }
  __device__ __forceinline__ void store(TileBuf<T>& b) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int c = threadIdx.x + i * NT;
      if (c < 2 * CH) {
        bool isv = c >= CH;
        int cc = isv ? c - CH : c;
        int key = cc / CPR, part = cc % CPR;
        if (!isv) {
          *reinterpret_cast<uint4*>(&b.k[key][part * E]) = r[i];
        } else {
          const T* e = reinterpret_cast<const T*>(&r[i]);
          int pos = vt_pos(key);
#pragma unroll
          for (int x = 0; x < E; ++x) b.vt[part * E + x][pos] = e[x];
        }
      }
    }
  }
};

__device__ __forceinline__ Frag8<bf16> lds_frag(const bf16* p) {
  Frag8<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag8<float> lds_frag(const float* p) {
  Frag8<float> f;
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f.v = (f32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return f;
}


template <typename T>
__device__ __forceinline__ void load_tile_frags(const TileBuf<T>& b, Frag8<T> (&kf)[4], Frag8<T> (&vf)[2][2]) {
  const int l = lane_id();
  const int r = l & 15, g = l >> 4;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) kf[kt] = lds_frag(&b.k[16 * kt + r][8 * g]);
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int h = 0; h < 2; ++h) vf[dt][h] = lds_frag(&b.vt[16 * dt + r][32 * h + 8 * g]);
}

// MFMA accumulator seed that masks the keys of a tile at or beyond nk (-inf) and leaves the rest.
__device__ __forceinline__ void tile_mask(int nk, f32x4 (&cm)[4]) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) cm[kt][i] = (16 * kt + 4 * g + i < nk) ? 0.f : -INFINITY;
}

// Finish one branch for one token: normalise and gate; optionally write lse (natural log).
__device__ __forceinline__ void tok_finish(const TokState& st, f32x4 (&res)[2], float wgt, float* lse_out) {
  const float l = wave_sum_across_rows(st.l);
  const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) res[dt] = st.acc[dt] * (inv * wgt);
  if (lse_out != nullptr && (lane_id() >> 4) == 0)
    *lse_out = l > 0.f ? (st.mc + __log2f(l)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------------------------
// generic tile loop: double-buffered LDS staging shared by the workgroup
// ---------------------------------------------------------------------------------------------

// Part::kAll: every wave's participating tokens are the prefix t < n_valid (compressed, local and
// dense phases); otherwise a per-tile mask (selected phase).
template <typename T, int NT, int TPW, class Src, class Part>
__device__ __forceinline__ void run_tiles(TileBuf<T>* buf, const Src& src, int ntiles, const Part& part,
                                          TokState (&st)[TPW], const QF<T> (&qf)[TPW]) {
  // Global loads run two tiles ahead of the compute (two register sets), LDS holds two tiles.  The
  // loop is unrolled by two so the register sets swap roles without a copy.
  Stager<T, NT> sa, sb;
  if (ntiles <= 0) return;
  // Settle every outstanding load of earlier phases here: the compiler's wait insertion would
  // otherwise merge them with the prefetch in flight and wait for that prefetch inside the loop.
  __builtin_amdgcn_s_waitcnt(0);
  sa.load_all(src.kptr(0), src.vptr(0), src.stride, src.nk(0));
  sa.store(buf[0]);
  sa.load_all(src.kptr(min(1, ntiles - 1)), src.vptr(min(1, ntiles - 1)), src.stride, src.nk(min(1, ntiles - 1)));
  __syncthreads();
  // one step: tile u+1's rows are in cur, start tile u+2's load into nxt, compute tile u, store cur
  auto step = [&](int u, Stager<T, NT>& cur, Stager<T, NT>& nxt) {
    const int xl = min(u + 2, ntiles - 1);       // past the end: a harmless load of the last tile
    nxt.load_all(src.kptr(xl), src.vptr(xl), src.stride, src.nk(xl));
    const TileBuf<T>& b = buf[u & 1];
    const int nk = src.nk(u);
    const uint32_t pm = Part::kAll ? 0u : part.wave_mask(u);
    if (Part::kAll ? part.n > 0 : pm != 0u) {
      Frag8<T> kf[4], vf[2][2];
      f32x4 cm[4];
      load_tile_frags(b, kf, vf);
      if (nk < TILE) tile_mask(nk, cm);
      if constexpr (Part::kAll) tile_prefix<T, TPW>(st, qf, part.n, kf, vf, cm, nk == TILE);
      else tile_masked<T, TPW>(st, qf, pm, kf, vf, cm, nk == TILE);
    }
    if (u + 1 < ntiles) cur.store(buf[(u + 1) & 1]);
    __syncthreads();
  };
  for (int u = 0; u < ntiles; u += 2) {
    step(u, sa, sb);
    if (u + 1 < ntiles) step(u + 1, sb, sa);
  }
}

// Barrier-free tile ring for the selected branch.  R LDS buffers; tile t lives in buffer t % R.
// Every wave stages its own share of each tile (the chunks its threads own) and then adds 1 to
// ready[t % R]; it computes tile t once ready shows all WAVES shares of that use of the buffer, and
// adds 1 to done[t % R] after its last read.  A wave stages tile t + R - L into the buffer of tile
// t - L only after done shows that every wave has finished tile t - L (the lag L is 3 with 8
// buffers, 2 with fewer).  Both counts are read early (the next tile's ready count and tile t - L's
// done count before tile t's compute), so a wait that
// is already satisfied costs no LDS round trip of its own; only a short count is read again.  Each
// wait names a strictly earlier event of other waves, so the ring cannot deadlock; it lets a wave
// run ahead of the slowest instead of meeting at a barrier after every tile (the work per wave and
// tile varies with how many of its tokens selected the tile's block).  Waits are bounded: if a
// count ever failed to arrive, the wave marks the workgroup broken and stops waiting; the kernel
// still ends and the branch's output is NaN.
__device__ __forceinline__ void ring_wait(const int* ctr, int target, int* broken, int spin_limit) {
  int spins = 0;
  while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) <
         target) {
    if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(broken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)))
      break;
    if (++spins > spin_limit) {
      __hip_atomic_store(broken, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ void ring_signal(int* ctr) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (lane_id() == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Buffers 0 and 1 of the ring are the workgroup's two staging tiles at the start of LDS; buffers 2
// and up sit one after another from byte offset hi_off.  The address is formed from the LDS base by integer offsets so
// that every access stays an LDS (ds_*) access.
template <typename T> struct RingBufs {
  unsigned char* lds;
  int hi_off;
  __device__ __forceinline__ TileBuf<T>& operator[](int i) const {
    const int off = i < 2 ? i * (int)sizeof(TileBuf<T>) : hi_off + (i - 2) * (int)sizeof(TileBuf<T>);
    return *reinterpret_cast<TileBuf<T>*>(lds + off);
  }
};

template <typename T, int NT, int TPW, int R, class Src, class Part>
__device__ __forceinline__ void run_tiles_ring(const RingBufs<T>& rb, int* ready, int* done, int* broken,
                                               int spin_limit, int stall, const Src& src, int ntiles,
                                               const Part& part, TokState (&st)[TPW], const QF<T> (&qf)[TPW]) {
  static_assert(R >= 4, "the ring needs four buffers or more");
  constexpr int WAVES = NT / 64;
  constexpr int L = R >= 8 ? 3 : 2;                // lag between a tile's compute and its buffer's reuse
  // global loads run one step ahead of the store that needs them (two register sets)
  Stager<T, NT> sg, nx;
  __builtin_amdgcn_s_waitcnt(0);   // as in run_tiles: no earlier load stays in flight into the loop
  for (int t = 0; t < R - L && t < ntiles; ++t) {
    sg.load(src.kptr(t), src.vptr(t), src.stride, src.nk(t));
    sg.store(rb[t]);
    ring_signal(&ready[t]);
  }
  if (R - L < ntiles) sg.load_all(src.kptr(R - L), src.vptr(R - L), src.stride, src.nk(R - L));
  int rdy = -1;                                   // ready count of tile u's buffer read early
  // one step: compute tile u, stage tile u + R - L from cur (loaded one step earlier), and start
  // the load of the tile after it into nxt; the loop is unrolled by two so the sets swap roles
  // without a register copy (a copy would wait for the load it is meant to leave in flight)
  auto step = [&](int u, Stager<T, NT>& cur, Stager<T, NT>& nxt) {
    const int x = u + R - L;
    const int xl = min(x + 1, ntiles - 1);        // past the end: a harmless load of the last tile
    nxt.load_all(src.kptr(xl), src.vptr(xl), src.stride, src.nk(xl));
    const int bu = u % R;
    const int need = WAVES * (u / R + 1) + stall;
    if (rdy < need) ring_wait(&ready[bu], need, broken, spin_limit);
    else __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const int rdy_next =
        u + 1 < ntiles ? __hip_atomic_load(&ready[(u + 1) % R], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : 0;
    const int dn = (x < ntiles && u >= L)
                       ? __hip_atomic_load(&done[(u - L) % R], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
                       : 0;
    const TileBuf<T>& b = rb[bu];
    const int nk = src.nk(u);
    const uint32_t pm = part.wave_mask(u);
    if (pm != 0u) {
      Frag8<T> kf[4], vf[2][2];
      f32x4 cm[4];
      load_tile_frags(b, kf, vf);
      if (nk < TILE) tile_mask(nk, cm);
      tile_masked<T, TPW>(st, qf, pm, kf, vf, cm, nk == TILE);
    }
    ring_signal(&done[bu]);
    if (x < ntiles) {
      const int bp = x % R;                        // == (u - L) % R, the buffer of tile u - L
      if (u >= L) {
        const int fin = WAVES * ((u - L) / R + 1);
        if (__builtin_amdgcn_readfirstlane(dn) < fin) ring_wait(&done[bp], fin, broken, spin_limit);
        else __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      }
      cur.store(rb[bp]);
      ring_signal(&ready[bp]);
    }
    rdy = __builtin_amdgcn_readfirstlane(rdy_next);
  };
  for (int u = 0; u < ntiles; u += 2) {
    step(u, sg, nx);
    if (u + 1 < ntiles) step(u + 1, nx, sg);
  }
  __syncthreads();
  if (*broken) {
    // a wait gave up: make the branch's output NaN rather than silently wrong
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      st[t].acc[0] = (f32x4){NAN, NAN, NAN, NAN};
      st[t].acc[1] = st[t].acc[0];
    }
  }
}

// Key tile sources ------------------------------------------------------------------------------

template <typename T> struct RangeSrc {     // tiles of 64 consecutive rows [lo, hi) of [rows][n_kvh][D]
  const T* base;   // &x[0][j][0]
  int stride, lo, hi;
  __device__ const T* kptr(int u) const { return base + (size_t)(lo + TILE * u) * stride; }
  __device__ const T* vptr(int u) const { return vbase + (size_t)(lo + TILE * u) * stride; }
  __device__ int nk(int u) const { int r = hi - lo - TILE * u; return r < TILE ? r : TILE; }
  const T* vbase;
};

template <typename T> struct UnionSrc {     // one tile per block in the selection union
  const T* kb;     // &k[0][j][0]
  const T* vb;
  int stride;      // n_kvh * D
  int cap;
  const int* ulist;        // LDS: block index | valid-token count << 16
  __device__ const T* kptr(int u) const { return kb + (size_t)(ulist[u] & 0xFFFF) * cap * stride; }
  __device__ const T* vptr(int u) const { return vb + (size_t)(ulist[u] & 0xFFFF) * cap * stride; }
  __device__ int nk(int u) const { return ulist[u] >> 16; }
};

struct AllPart {                 // the wave's valid tokens (a prefix) take part in every tile
  static constexpr bool kAll = true;
  int n;
  __device__ uint32_t wave_mask(int) const { return (1u << n) - 1u; }
};
template <int WAVES, int TPW>
struct UnionPart {               // tokens whose routing row holds the tile's block
  static constexpr bool kAll = false;
  const unsigned long long* umask;  // LDS: bits [TPW w, TPW w + TPW) of umask[u] = wave w's tokens that selected union block u
  int w;                            // wave index; its token t is slot t * WAVES + w
  int n = 0;                        // unused
  __device__ uint32_t wave_mask(int u) const {
    return __builtin_amdgcn_readfirstlane((uint32_t)(umask[u] >> (TPW * w)) & ((1u << TPW) - 1u));
  }
};

// ---------------------------------------------------------------------------------------------
// block-wide helpers for the selection union
// ---------------------------------------------------------------------------------------------

template <int NT>
__device__ int block_exclusive_scan(int x, int* scratch /* NT/64 + 1 ints */) {
  const int l = lane_id(), w = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(inc, o, 64);
    if (l >= o) inc += y;
  }
  if (l == 63) scratch[w] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int i = 0; i < NT / 64; ++i) { int t = scratch[i]; scratch[i] = s; s += t; }
    scratch[NT / 64] = s;
  }
  __syncthreads();
  return scratch[w] + inc - x;
}

// ---------------------------------------------------------------------------------------------
// the NSA kernel
// ---------------------------------------------------------------------------------------------

// Where the gated sum of finished branches lives between branch phases: registers for f32 (the
// small fp32 path), LDS (fp32, 64 slots x 16 heads x 32 dims = 128 KiB) for bf16, which keeps the
// bf16 kernel within 256 VGPRs per lane.
template <typename T> struct OutInLds { static constexpr bool value = sizeof(T) == 2; };

// Tile buffers of the selected branch's ring.  The bf16 ring's extra buffers fit beside the union
// tables inside the region the running gated sum takes later, so they cost no LDS.
template <typename T> struct RingSize { static constexpr int value = sizeof(T) == 2 ? 8 : 4; };

// kSel: the selected branch's phase is compiled in (launches whose branches include it); without
// it the compressed and local phases get the registers to themselves.
template <typename T, int WAVES, int TPW, bool kSel>
__global__ __launch_bounds__(WAVES * 64) void nsa_attn_kernel(AttnArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr bool kOutLds = OutInLds<T>::value;
  constexpr int SLOTS = WAVES * TPW;             // query slots of one workgroup: a block or half a block
  static_assert(SLOTS == 64 || SLOTS == 32, "a workgroup covers 64 or 32 query slots");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  TileBuf<T>* buf = reinterpret_cast<TileBuf<T>*>(smem);
  // region after the tiles: the selection-union tables during the SEL phase, then (bf16, several
  // gated branches) the fp32 running gated sum; SEL runs first so the two never overlap in time
  unsigned char* extra = smem + 2 * sizeof(TileBuf<T>);
  float* out_lds = reinterpret_cast<float*>(extra);

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int cap = a.cap, n_part = (cap + SLOTS - 1) / SLOTS;
  const int j = wg % a.n_kvh, bp = wg / a.n_kvh;
  const int b = a.q_blk0 + bp / n_part;
  const int s0 = (bp % n_part) * SLOTS;          // first block slot of this workgroup
  const int cnt = a.blk_cnt[b];
  const int cnt_p = min(max(cnt - s0, 0), SLOTS);  // valid slots of this workgroup: [s0, s0 + cnt_p)
  const int w = threadIdx.x >> 6, l = lane_id();
  const int r = l & 15, g = l >> 4;
  const int hh = j * GRP + r;                  // query head of this lane
  const int kvs = a.n_kvh * HD;                // key row stride (elements)
  const float c2 = a.scale * kLog2e;
  const T* q = reinterpret_cast<const T*>(a.q);
  const int n_named = __builtin_popcount(a.branches);

  // queries of this wave's tokens: token t of wave w is block slot s0 + t * WAVES + w, so the
  // valid slots spread evenly over the waves and each wave's valid tokens are a prefix
  QF<T> qf[TPW];
  const int n_valid = cnt_p > w ? min(TPW, (cnt_p - w + WAVES - 1) / WAVES) : 0;
  const uint32_t valid = (1u << n_valid) - 1u;
  {
    Frag8<T> raw[TPW];   // every slot of the block has a query row (padding rows are never used)
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      raw[t] = load_q8(q + ((b * cap + min(s0 + t * WAVES + w, cap - 1)) * a.n_qh + hh) * HD + 8 * g);
#pragma unroll
    for (int t = 0; t < TPW; ++t) qf[t] = make_qf<T>(raw[t], c2, t < n_valid);
  }

  f32x4 out_reg[kOutLds ? 1 : TPW][2];
  TokState st[TPW];
  T* o = reinterpret_cast<T*>(a.o);
  int done = 0;   // branches finished so far

  // Close a branch: normalise, gate, and either store (last branch) or fold into the running sum.
  auto finish_all = [&](int ch) {
    const bool first = done == 0, last = done == n_named - 1;
    // gate logits of the wave's tokens, loaded together: loaded inside the token loop, each would
    // wait a memory round trip behind the previous token's output stores
    // (every slot of the block has a gate row, so the loads need no per-token branch)
    T gl[TPW];
    if (a.gates) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int row = b * cap + min(s0 + t * WAVES + w, cap - 1);
        gl[t] = reinterpret_cast<const T*>(a.gates)[(row * a.n_qh + hh) * a.n_gch + ch];
      }
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int slot = s0 + t * WAVES + w;
      if (!(valid & (1u << t))) continue;
      const int row = b * cap + slot;
      const float wgt = a.gates ? sigmoidf_(to_f32(gl[t])) : 1.f;
      float* lp = a.lse ? a.lse + row * a.n_qh + hh : nullptr;
      f32x4 res[2];
      tok_finish(st[t], res, wgt, lp);
      float* ol = out_lds + ((slot - s0) * GRP + r) * HD + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        f32x4 acc = res[dt];
        if (!first) {
          if constexpr (kOutLds) acc += *reinterpret_cast<const f32x4*>(ol + 16 * dt);
          else acc += out_reg[kOutLds ? 0 : t][dt];
        }
        if (last) {
          T* dst = o + (row * a.n_qh + hh) * HD + 16 * dt + 4 * g;
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[i] = from_f32<T>(acc[i]);
        } else if constexpr (kOutLds) {
          *reinterpret_cast<f32x4*>(ol + 16 * dt) = acc;
        } else {
          out_reg[kOutLds ? 0 : t][dt] = acc;
        }
      }
    }
    ++done;
  };

  // ---- selected branch: union of the block's routing rows, streamed once ----
  if (kSel && (a.branches & 2)) {
    // byte offsets from `extra` (kept as offsets so the pointers stay LDS pointers): bitmap,
    // per-word prefix, union list, scan scratch, per-wave token masks, ring buffers 2 .. R-1, and
    // the ring counters ready[R], done[R], broken
    constexpr int R = RingSize<T>::value;
    const int off_wpre = a.n_words * 4;
    const int off_ulist = off_wpre + a.n_words * 4;
    const int off_scratch = off_ulist + a.u_cap * 4;
    const int off_umask = (off_scratch + (NT / 64 + 1) * 4 + 7) & ~7;
    const int off_ring = (off_umask + a.u_cap * 8 + 15) & ~15;
    const int off_ctr = off_ring + (R - 2) * (int)sizeof(TileBuf<T>);
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(extra);
    int* wpre = reinterpret_cast<int*>(extra + off_wpre);
    int* ulist = reinterpret_cast<int*>(extra + off_ulist);
    int* scratch = reinterpret_cast<int*>(extra + off_scratch);
    unsigned long long* umask = reinterpret_cast<unsigned long long*>(extra + off_umask);
    int* ring_ctr = reinterpret_cast<int*>(extra + off_ctr);
    const int grp = a.sel_groups == 1 ? 0 : j;
    const int kk = a.top_k;
    for (int i = threadIdx.x; i < a.n_words; i += NT) bitmap[i] = 0u;
    if (threadIdx.x < 2 * R + 1) ring_ctr[threadIdx.x] = 0;
    // this thread's routing entries e = tid + i NT (row e / kk, entry e % kk of the workgroup's
    // rows) and their blocks' token counts, all loads issued at once: a loop of dependent loads
    // would pay one memory round trip per entry, exposed with one workgroup per CU
    constexpr int MAXE = (64 * 64 + NT - 1) / NT;   // rows <= 64, entries per row <= 64
    // routing row of slot s0 + t: sel_wg + t * sel_tstride (block rows: every slot reads row b)
    const int sel_tstride = a.sel_per_block ? 0 : a.sel_groups * kk;
    const int32_t* sel_wg = a.sel + ((size_t)(a.sel_per_block ? b : b * cap + s0) * a.sel_groups + grp) * kk;
    int eblk[MAXE], ecnt[MAXE];
#pragma unroll
    for (int i = 0; i < MAXE; ++i) {
      const int e = threadIdx.x + i * NT;
      eblk[i] = e < cnt_p * kk ? sel_wg[(e / kk) * sel_tstride + e % kk] : -1;
    }
#pragma unroll
    for (int i = 0; i < MAXE; ++i) ecnt[i] = (eblk[i] >= 0 && eblk[i] < a.n_blk) ? a.blk_cnt[eblk[i]] : 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MAXE; ++i)
      if (eblk[i] >= 0 && eblk[i] < a.n_blk) atomicOr(&bitmap[eblk[i] >> 5], 1u << (eblk[i] & 31));
    __syncthreads();
    // union position of a block = exclusive prefix of popcounts over the bitmap words (contiguous
    // word ranges per thread) plus its rank inside its word
    const int per = (a.n_words + NT - 1) / NT;
    const int w0 = threadIdx.x * per;
    int mine = 0;
    for (int i = 0; i < per; ++i)
      if (w0 + i < a.n_words) mine += __builtin_popcount(bitmap[w0 + i]);
    int base = block_exclusive_scan<NT>(mine, scratch);
    const int n_union = scratch[NT / 64];
    for (int i = 0; i < per; ++i) {
      const int wi = w0 + i;
      if (wi < a.n_words) {
        wpre[wi] = base;
        base += __builtin_popcount(bitmap[wi]);
      }
    }
    for (int i = threadIdx.x; i < n_union; i += NT) umask[i] = 0ull;
    __syncthreads();
    // every union block is named by some entry: each entry writes its block's list word (the
    // same value from every entry of that block) and its token's bit of the block's mask
#pragma unroll
    for (int i = 0; i < MAXE; ++i) {
      const int blk = eblk[i];
      if (blk >= 0 && blk < a.n_blk) {
        const int t = (threadIdx.x + i * NT) / kk;   // row: slot s0 + t
        const int wi = blk >> 5;
        const int u = wpre[wi] + __builtin_popcount(bitmap[wi] & ((1u << (blk & 31)) - 1u));
        ulist[u] = blk | (ecnt[i] << 16);
        atomicOr(&umask[u], 1ull << (TPW * (t % WAVES) + t / WAVES));   // wave t % WAVES, its token t / WAVES
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TPW; ++t) tok_init(st[t]);
    UnionSrc<T> src;
    src.kb = reinterpret_cast<const T*>(a.k) + j * HD;
    src.vb = reinterpret_cast<const T*>(a.v) + j * HD;
    src.stride = kvs;
    src.cap = cap;
    src.ulist = ulist;
    UnionPart<WAVES, TPW> part{umask, w};
    const RingBufs<T> rb{smem, 2 * (int)sizeof(TileBuf<T>) + off_ring};
    run_tiles_ring<T, NT, TPW, R>(rb, ring_ctr, ring_ctr + R, ring_ctr + 2 * R, a.ring_spins, a.ring_stall, src, n_union,
                                  part, st, qf);   // ends with a barrier
    finish_all(a.ch_sel);
  }

  // ---- local branch: the query's own block ----
  if (a.branches & 4) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) tok_init(st[t]);
    RangeSrc<T> src;
    src.base = reinterpret_cast<const T*>(a.k) + j * HD;
    src.vbase = reinterpret_cast<const T*>(a.v) + j * HD;
    src.stride = kvs;
    src.lo = b * cap;
    src.hi = b * cap + cnt;
    AllPart part{n_valid};
    // the own block is a key block only when it lies in the key range (an empty key set adds 0)
    run_tiles<T, NT, TPW>(buf, src, (b >= a.kv_lo && b < a.kv_hi) ? 1 : 0, part, st, qf);
    finish_all(a.ch_loc);
  }

  // ---- compressed branch: every pooled block ----
  if (a.branches & 1) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) tok_init(st[t]);
    RangeSrc<T> src;
    src.base = reinterpret_cast<const T*>(a.k_cmp) + j * HD;
    src.vbase = reinterpret_cast<const T*>(a.v_cmp) + j * HD;
    src.stride = kvs;
    src.lo = a.kv_lo;
    src.hi = a.kv_hi;
    AllPart part{n_valid};
    run_tiles<T, NT, TPW>(buf, src, (a.kv_hi - a.kv_lo + TILE - 1) / TILE, part, st, qf);
    finish_all(0);
  }

  // ---- padding slots of the block: zero output (and -inf lse) ----
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int slot = s0 + t * WAVES + w;
    if (slot >= cap || slot < cnt) continue;
    const int row = b * cap + slot;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      T* dst = o + (row * a.n_qh + hh) * HD + 16 * dt + 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = from_f32<T>(0.f);
    }
    if (a.lse && g == 0) a.lse[row * a.n_qh + hh] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------------
// selected branch with wave-owned token clusters (bf16, per-token routing rows)
// ---------------------------------------------------------------------------------------------
//
// One wave per (8 consecutive slots of a block, KV head), no workgroup barrier and no shared
// staging.  Slots are stored in Morton order, so 8 consecutive slots are spatial neighbours whose
// routing rows largely agree: the wave walks the union of its 8 rows once, in ascending block
// order, and each block's tile serves the tokens that selected it (LSRM pages, section 方法: the
// selected active blocks give each query its fine detail).  A tile's K rows are loaded from
// global memory straight into the MFMA A-operand layout (one 16-byte load per lane and 16-key
// step).  The V rows, loaded the same way, go to a tile in the wave's own LDS as they are and come
// back as V^T fragments through gfx950's transposing LDS read, in the permuted key order in which
// the softmax hands over its probabilities.  The result is gated and written to o, or added to
// what o holds (accumulate).

constexpr int SEL_TPW = 8;   // tokens (consecutive slots) per wave
constexpr int SEL_WPG = 4;   // waves per workgroup (independent)
constexpr int SEL_MAXE = SEL_TPW;   // routing entries per lane: 8 rows x top_k <= 64 entries / 64 lanes

// LDS bytes of one wave's tables: bitmap and per-word prefix (n_words each), union list and
// per-block token masks (ucap each).
constexpr int SEL_VPAD = 40;                          // LDS row stride (elements) of the staged V rows
constexpr int SEL_VT_BYTES = TILE * SEL_VPAD * 2;      // one wave's staged V tile (bf16)
__host__ __device__ inline int sel_wave_lds_bytes(int n_words, int ucap) {
  return SEL_VT_BYTES + (((2 * n_words + 2 * ucap) * 4 + 15) & ~15);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each 16-lane group, source lane s names
// 4 consecutive 16-bit elements; result lane i receives, as its element e, element i % 4 of source
// lane 4e + i / 4.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4 __attribute__((address_space(3)))*)(reinterpret_cast<const s16x4*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// Orders this wave's LDS accesses (all lanes) before the next ones.  A wave's LDS instructions
// execute in order, so only compiler reordering has to be stopped.
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int wave_exclusive_scan(int x, int& total) {
  const int l = lane_id();
  int inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, 64);
    if (l >= o) inc += y;
  }
  total = __shfl(inc, 63, 64);
  return inc - x;
}

struct SelRaw {                 // one tile's K and V rows as loaded: 16 keys per step
  Frag8<bf16> k[4], v[4];
};

// kLoc: the local branch instead (the query block's own block is the one tile, every valid token
// takes part; no routing rows are read).
template <bool kLoc>
__global__ __launch_bounds__(SEL_WPG * 64, 2) void sel_wave_kernel(AttnArgs a, int accumulate, int ucap) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int l = lane_id(), r = l & 15, g = l >> 4;
  const int cap = a.cap;
  const int nclu = (cap + SEL_TPW - 1) / SEL_TPW;
  const int n_waves = a.n_qblk * nclu * a.n_kvh;
  const int wv = xcd_remap(blockIdx.x, gridDim.x) * SEL_WPG + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wv >= n_waves) return;                     // waves never wait for each other
  const int c = wv % nclu, j = (wv / nclu) % a.n_kvh;
  const int b = a.q_blk0 + wv / (nclu * a.n_kvh);
  const int s0 = c * SEL_TPW;
  const int cnt = a.blk_cnt[b];
  const int n_valid = min(max(cnt - s0, 0), SEL_TPW);
  const int hh = j * GRP + r;
  const int kvs = a.n_kvh * HD;
  bf16* o = reinterpret_cast<bf16*>(a.o);

  TokState st[SEL_TPW];
#pragma unroll
  for (int t = 0; t < SEL_TPW; ++t) tok_init(st[t]);

  if (n_valid > 0) {
    // queries of the wave's tokens (padding slots read a valid row of the block; never used)
    QF<bf16> qf[SEL_TPW];
    {
      const bf16* q = reinterpret_cast<const bf16*>(a.q);
      const float c2 = a.scale * kLog2e;
      Frag8<bf16> raw[SEL_TPW];
#pragma unroll
      for (int t = 0; t < SEL_TPW; ++t)
        raw[t] = load_q8(q + ((b * cap + s0 + min(t, n_valid - 1)) * a.n_qh + hh) * HD + 8 * g);
#pragma unroll
      for (int t = 0; t < SEL_TPW; ++t) qf[t] = make_qf<bf16>(raw[t], c2, t < n_valid);
    }

    const int nw = kLoc ? 0 : a.n_words;
    unsigned char* vtile = smem + (threadIdx.x >> 6) * sel_wave_lds_bytes(nw, ucap);
    bf16* vrows = reinterpret_cast<bf16*>(vtile);               // the tile's V rows, row-major
    unsigned char* tab = vtile + SEL_VT_BYTES;
    int* ulist = reinterpret_cast<int*>(tab + nw * 8);
    uint32_t* umask = reinterpret_cast<uint32_t*>(tab + nw * 8 + ucap * 4);
    int n_union;
    if constexpr (kLoc) {
      // the own block, when it lies in the key range (an empty key set adds 0)
      if (l == 0) {
        ulist[0] = b | (cnt << 16);
        umask[0] = (1u << n_valid) - 1u;
      }
      n_union = (b >= a.kv_lo && b < a.kv_hi) ? 1 : 0;
      wave_lds_order();
    } else {
    // routing entries of the wave's rows (entry e: row e / top_k, position e % top_k) and their
    // blocks' token counts, all loads issued at once
    const int kk = a.top_k;
    const int grp = a.sel_groups == 1 ? 0 : j;
    const int ne = n_valid * kk;
    int eblk[SEL_MAXE], ecnt[SEL_MAXE];
#pragma unroll
    for (int i = 0; i < SEL_MAXE; ++i) {
      const int e = l + 64 * i;
      const int t = e / kk;
      eblk[i] = e < ne ? a.sel[((b * cap + s0 + t) * a.sel_groups + grp) * kk + (e - t * kk)] : -1;
    }
#pragma unroll
    for (int i = 0; i < SEL_MAXE; ++i) ecnt[i] = (eblk[i] >= 0 && eblk[i] < a.n_blk) ? a.blk_cnt[eblk[i]] : 0;

    // union of the rows in this wave's LDS tables: bitmap, per-word prefix, list, token masks
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(tab);
    int* wpre = reinterpret_cast<int*>(tab + nw * 4);
    for (int i = l; i < nw; i += 64) bitmap[i] = 0u;
    wave_lds_order();
#pragma unroll
    for (int i = 0; i < SEL_MAXE; ++i)
      if (eblk[i] >= 0 && eblk[i] < a.n_blk) atomicOr(&bitmap[eblk[i] >> 5], 1u << (eblk[i] & 31));
    wave_lds_order();
    const int per = (nw + 63) / 64, w0 = l * per;
    int mine = 0;
    for (int i = 0; i < per; ++i)
      if (w0 + i < nw) mine += __builtin_popcount(bitmap[w0 + i]);
    int base = wave_exclusive_scan(mine, n_union);
    for (int i = 0; i < per; ++i) {
      const int wi = w0 + i;
      if (wi < nw) {
        wpre[wi] = base;
        base += __builtin_popcount(bitmap[wi]);
      }
    }
    for (int i = l; i < n_union; i += 64) umask[i] = 0u;
    wave_lds_order();
#pragma unroll
    for (int i = 0; i < SEL_MAXE; ++i) {
      const int blk = eblk[i];
      if (blk >= 0 && blk < a.n_blk) {
        const int wi = blk >> 5;
        const int u = wpre[wi] + __builtin_popcount(bitmap[wi] & ((1u << (blk & 31)) - 1u));
        ulist[u] = blk | (ecnt[i] << 16);
        atomicOr(&umask[u], 1u << ((l + 64 * i) / kk));
      }
    }
    wave_lds_order();
    }

    const bf16* kb = reinterpret_cast<const bf16*>(a.k) + j * HD;
    const bf16* vb = reinterpret_cast<const bf16*>(a.v) + j * HD;
    // rows past the block's count repeat its last valid row (masked by the -inf seed); the
    // block's base is wave-uniform and the lane's part a 32-bit offset
    const unsigned kvs2 = 2u * kvs, goff = 16u * g;   // row stride and the lane's part, in bytes
    auto load_tile = [&](int u, SelRaw& x) {
      const int ent = __builtin_amdgcn_readfirstlane(ulist[u]);
      const int blk = ent & 0xFFFF, last = max((ent >> 16) - 1, 0);
      const size_t base = (size_t)(blk * cap) * kvs2;
      const char* kt = reinterpret_cast<const char*>(kb) + base;
      const char* vt = reinterpret_cast<const char*>(vb) + base;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const unsigned off = __umul24((unsigned)min(16 * q4 + r, last), kvs2) + goff;
        x.k[q4].v = *reinterpret_cast<const bf16x8*>(kt + off);
        x.v[q4].v = *reinterpret_cast<const bf16x8*>(vt + off);
      }
    };
    auto step = [&](int u, SelRaw& cur, SelRaw& nxt) {
      // V^T fragments of tile u: vf[dt][h] takes keys 32h + 4g + i and 32h + 16 + 4g + i (i < 4) of
      // head-dim column 16 dt + r.  The rows go to the wave's LDS tile as loaded (lane (r, g): key
      // 16 q4 + r, dims 8g..8g+7); a transposing read in which lane (r, g) names key
      // 32h + 4g + r / 4 (+ 16), dims 16 dt + 4 (r % 4) .. + 3 returns exactly those four keys of
      // column 16 dt + r to lane (r, g).
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<bf16x8*>(vrows + (16 * q4 + r) * SEL_VPAD + 8 * g) = cur.v[q4].v;
      Frag8<bf16> vf[2][2];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16* base = vrows + (32 * h + 4 * g + (r >> 2)) * SEL_VPAD + 16 * dt + 4 * (r & 3);
          const bf16x4 lo = lds_read_tr4(base);
          const bf16x4 hi = lds_read_tr4(base + 16 * SEL_VPAD);
          vf[dt][h].v = (bf16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      const int nk = ulist[u] >> 16;
      const uint32_t pm = __builtin_amdgcn_readfirstlane(umask[u]);
      if (u + 1 < n_union) load_tile(u + 1, nxt);
      f32x4 cm[4];
      if (nk < TILE) tile_mask(nk, cm);
      tile_masked<bf16, SEL_TPW>(st, qf, pm, cur.k, vf, cm, nk == TILE);
    };
    SelRaw ra, rb;
    if (n_union > 0) load_tile(0, ra);
    for (int u = 0; u < n_union; u += 2) {
      step(u, ra, rb);
      if (u + 1 < n_union) step(u + 1, rb, ra);
    }
  }

  // gate, then write or add; padding slots get 0 (write) or are left alone (add)
  bf16 gl[SEL_TPW];
  if (a.gates) {
#pragma unroll
    for (int t = 0; t < SEL_TPW; ++t) {
      const int row = b * cap + min(s0 + t, cap - 1);
      gl[t] = reinterpret_cast<const bf16*>(a.gates)[(row * a.n_qh + hh) * a.n_gch + (kLoc ? a.ch_loc : a.ch_sel)];
    }
  }
#pragma unroll
  for (int t = 0; t < SEL_TPW; ++t) {
    const int slot = s0 + t;
    if (slot >= cap) continue;
    const int row = b * cap + slot;
    bf16x4* dst = reinterpret_cast<bf16x4*>(o + (row * a.n_qh + hh) * HD + 4 * g);
    if (t >= n_valid) {
      if (!accumulate) {
        const bf16x4 z = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
        dst[0] = z;
        dst[4] = z;
      }
      if (a.lse && g == 0) a.lse[row * a.n_qh + hh] = -INFINITY;
      continue;
    }
    const float wgt = a.gates ? sigmoidf_(to_f32(gl[t])) : 1.f;
    f32x4 res[2];
    tok_finish(st[t], res, wgt, a.lse ? a.lse + row * a.n_qh + hh : nullptr);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      f32x4 acc = res[dt];
      if (accumulate) {
        const bf16x4 prev = dst[4 * dt];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += (float)prev[i];
      }
      dst[4 * dt] = (bf16x4){(bf16)acc[0], (bf16)acc[1], (bf16)acc[2], (bf16)acc[3]};
    }
  }
}

// ---------------------------------------------------------------------------------------------
// compressed branch of pooled queries (block-granular query rows)
// ---------------------------------------------------------------------------------------------
//
// The rows are the pooled queries [n_blk][n_qh][D], SLOTS of them per workgroup in storage order,
// each with its KV group's 16 heads; the tile loop over every pooled key block is the fused
// kernel's compressed phase.  Each block's result is then given to every valid token of the block,
// with that token's gate, added to what o holds (accumulate) or written with zeros on padding
// slots.  Speed3R page, section 2.1: the compression branch attends with block-pooled queries.

template <typename T, int WAVES, int TPW>
__global__ __launch_bounds__(WAVES * 64) void cmp_pooled_kernel(AttnArgs a, int accumulate, int gate_ch) {
  constexpr int NT = WAVES * 64;
  constexpr int SLOTS = WAVES * TPW;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  TileBuf<T>* buf = reinterpret_cast<TileBuf<T>*>(smem);
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int rg = wg / a.n_kvh, j = wg % a.n_kvh;
  const int w = threadIdx.x >> 6, l = lane_id();
  const int r = l & 15, g = l >> 4;
  const int hh = j * GRP + r;
  const int kvs = a.n_kvh * HD;
  const float c2 = a.scale * kLog2e;
  const T* q = reinterpret_cast<const T*>(a.q);
  // pooled row t of wave w: rg * SLOTS + t * WAVES + w; this workgroup's rows are [0, rem)
  const int rem = a.n_blk - rg * SLOTS;
  const int n_valid = rem > w ? min(TPW, (rem - w + WAVES - 1) / WAVES) : 0;
  QF<T> qf[TPW];
  {
    Frag8<T> raw[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      raw[t] = load_q8(q + ((size_t)(rg * SLOTS + min(t * WAVES + w, rem - 1)) * a.n_qh + hh) * HD + 8 * g);
#pragma unroll
    for (int t = 0; t < TPW; ++t) qf[t] = make_qf<T>(raw[t], c2, t < n_valid);
  }
  TokState st[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) tok_init(st[t]);
  RangeSrc<T> src;
  src.base = reinterpret_cast<const T*>(a.k_cmp) + j * HD;
  src.vbase = reinterpret_cast<const T*>(a.v_cmp) + j * HD;
  src.stride = kvs;
  src.lo = 0;
  src.hi = a.n_blk;
  AllPart part{n_valid};
  run_tiles<T, NT, TPW>(buf, src, (a.n_blk + TILE - 1) / TILE, part, st, qf);
  T* o = reinterpret_cast<T*>(a.o);
  const T* gp = reinterpret_cast<const T*>(a.gates);
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    if (t >= n_valid) continue;
    const int b = rg * SLOTS + t * WAVES + w;
    f32x4 res[2];
    tok_finish(st[t], res, 1.f, a.lse ? a.lse + (size_t)b * a.n_qh + hh : nullptr);
    const int cnt = a.blk_cnt[b];
    for (int sl = 0; sl < a.cap; ++sl) {
      const size_t row = (size_t)b * a.cap + sl;
      T* dst = o + (row * a.n_qh + hh) * HD + 4 * g;
      if (sl >= cnt && accumulate) continue;
      const float wgt = sl >= cnt ? 0.f : (gp ? sigmoidf_(to_f32(gp[(row * a.n_qh + hh) * a.n_gch + gate_ch])) : 1.f);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float prev = accumulate ? to_f32(dst[16 * dt + i]) : 0.f;
          dst[16 * dt + i] = from_f32<T>(prev + wgt * res[dt][i]);
        }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// stage-1 dense gated self/cross attention
// ---------------------------------------------------------------------------------------------

template <typename T, int WAVES, int TPW>
__global__ __launch_bounds__(WAVES * 64) void dense_xattn_kernel(DenseArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr bool kOutLds = OutInLds<T>::value;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  TileBuf<T>* buf = reinterpret_cast<TileBuf<T>*>(smem);
  float* out_lds = reinterpret_cast<float*>(smem + 2 * sizeof(TileBuf<T>));
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int qb = wg / a.n_kvh, j = wg % a.n_kvh;
  const int w = threadIdx.x >> 6, l = lane_id();
  const int r = l & 15, g = l >> 4;
  const int hh = j * GRP + r;
  const int kvs = a.n_kvh * HD;
  const float c2 = a.scale * kLog2e;
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* gp = reinterpret_cast<const T*>(a.gates);

  constexpr int SLOTS = WAVES * TPW;             // tokens of one workgroup
  QF<T> qf[TPW];
  const int rem = a.n_tok - qb * SLOTS;         // tokens of this workgroup: slots [0, rem)
  const int n_valid = rem > w ? min(TPW, (rem - w + WAVES - 1) / WAVES) : 0;
  const uint32_t valid = (1u << n_valid) - 1u;
  {
    Frag8<T> raw[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      raw[t] = load_q8(q + (min(qb * SLOTS + t * WAVES + w, a.n_tok - 1) * a.n_qh + hh) * HD + 8 * g);
#pragma unroll
    for (int t = 0; t < TPW; ++t) qf[t] = make_qf<T>(raw[t], c2, t < n_valid);
  }
  f32x4 out_reg[kOutLds ? 1 : TPW][2];
  TokState st[TPW];
  T* o = reinterpret_cast<T*>(a.o);
  for (int ph = 0; ph < 2; ++ph) {
    const int lo = ph == 0 ? 0 : a.n_x, hi = ph == 0 ? a.n_x : a.n_tok;
#pragma unroll
    for (int t = 0; t < TPW; ++t) tok_init(st[t]);
    RangeSrc<T> src;
    src.base = reinterpret_cast<const T*>(a.k) + j * HD;
    src.vbase = reinterpret_cast<const T*>(a.v) + j * HD;
    src.stride = kvs;
    src.lo = lo;
    src.hi = hi;
    AllPart part{n_valid};
    run_tiles<T, NT, TPW>(buf, src, (hi - lo + TILE - 1) / TILE, part, st, qf);
    // gate logits of the wave's tokens, loaded together (phase 0 holds x keys: self for x tokens,
    // cross for y tokens)
    T gl[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int tok = min(qb * SLOTS + t * WAVES + w, a.n_tok - 1);
      const int ch = ((tok < a.n_x) == (ph == 0)) ? 0 : 1;
      gl[t] = gp[(tok * a.n_qh + hh) * 2 + ch];
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int slot = t * WAVES + w;
      const int tok = qb * SLOTS + slot;
      if (!(valid & (1u << t))) continue;
      const float wgt = sigmoidf_(to_f32(gl[t]));
      f32x4 res[2];
      tok_finish(st[t], res, wgt, nullptr);
      float* ol = out_lds + (slot * GRP + r) * HD + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        if (ph == 0) {
          if constexpr (kOutLds) *reinterpret_cast<f32x4*>(ol + 16 * dt) = res[dt];
          else out_reg[kOutLds ? 0 : t][dt] = res[dt];
        } else {
          f32x4 acc = res[dt];
          if constexpr (kOutLds) acc += *reinterpret_cast<const f32x4*>(ol + 16 * dt);
          else acc += out_reg[kOutLds ? 0 : t][dt];
          T* dst = o + (tok * a.n_qh + hh) * HD + 16 * dt + 4 * g;
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[i] = from_f32<T>(acc[i]);
        }
      }
    }
  }
}

template <typename T> struct Shape;
template <> struct Shape<bf16> { static constexpr int WAVES = 8, TPW = 8; };
template <> struct Shape<float> { static constexpr int WAVES = 8, TPW = 4; };   // half a block per workgroup

template <typename T>
size_t attn_lds_t(const AttnArgs& a) {
  constexpr int NT = Shape<T>::WAVES * 64;
  size_t extra = 0;
  constexpr int R = RingSize<T>::value;
  if (a.branches & 2)   // union tables, R - 2 more ring buffers, ring counters (with alignment slack)
    extra = (size_t)a.n_words * 8 + (size_t)a.u_cap * 4 + (NT / 64 + 1) * 4 + 8 + (size_t)a.u_cap * 8 + 16 +
            (R - 2) * sizeof(TileBuf<T>) + (2 * R + 1) * sizeof(int);
  if (OutInLds<T>::value && __builtin_popcount(a.branches) > 1) {
    const size_t out_bytes = (size_t)Shape<T>::WAVES * Shape<T>::TPW * GRP * HD * sizeof(float);
    if (out_bytes > extra) extra = out_bytes;
  }
  return 2 * sizeof(TileBuf<T>) + extra;
}

template <typename T>
hipError_t launch_attn_t(const AttnArgs& a, hipStream_t s) {
  constexpr int WAVES = Shape<T>::WAVES, TPW = Shape<T>::TPW, NT = WAVES * 64;
  const size_t lds = attn_lds_t<T>(a);
  const int n_part = (a.cap + WAVES * TPW - 1) / (WAVES * TPW);   // workgroups per block and KV head
  const int nwg = a.n_qblk * n_part * a.n_kvh;
  if (nwg == 0) return hipSuccess;
  auto go = [&](auto kernel) -> hipError_t {
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kernel, dim3(nwg), dim3(NT), lds, s, a);
    return hipGetLastError();
  };
  return (a.branches & 2) ? go(&nsa_attn_kernel<T, WAVES, TPW, true>) : go(&nsa_attn_kernel<T, WAVES, TPW, false>);
}

int sel_wave_ucap(const AttnArgs& a) {
  const long long u = (long long)SEL_TPW * (a.top_k > 0 ? a.top_k : 1);
  return (int)(u < a.n_blk ? u : a.n_blk);
}

template <typename T>
hipError_t launch_cmp_pooled_t(const AttnArgs& a, int accumulate, int gate_ch, hipStream_t s) {
  constexpr int WAVES = Shape<T>::WAVES, TPW = Shape<T>::TPW, NT = WAVES * 64;
  const size_t lds = 2 * sizeof(TileBuf<T>);
  const int nwg = ((a.n_blk + WAVES * TPW - 1) / (WAVES * TPW)) * a.n_kvh;
  hipLaunchKernelGGL((cmp_pooled_kernel<T, WAVES, TPW>), dim3(nwg), dim3(NT), lds, s, a, accumulate, gate_ch);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dense_t(const DenseArgs& a, hipStream_t s) {
  constexpr int WAVES = Shape<T>::WAVES, TPW = Shape<T>::TPW, NT = WAVES * 64;
  constexpr int SLOTS = WAVES * TPW;
  const size_t lds = 2 * sizeof(TileBuf<T>) + (OutInLds<T>::value ? (size_t)SLOTS * GRP * HD * sizeof(float) : 0);
  const int nwg = ((a.n_tok + SLOTS - 1) / SLOTS) * a.n_kvh;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dense_xattn_kernel<T, WAVES, TPW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((dense_xattn_kernel<T, WAVES, TPW>), dim3(nwg), dim3(NT), lds, s, a);
  return hipGetLastError();
}

}  // namespace

size_t attn_lds_bytes(int is_bf16, const AttnArgs& a) {
  return is_bf16 ? attn_lds_t<bf16>(a) : attn_lds_t<float>(a);
}

hipError_t launch_attn(int is_bf16, const AttnArgs& a, hipStream_t s) {
  return is_bf16 ? launch_attn_t<bf16>(a, s) : launch_attn_t<float>(a, s);
}

size_t sel_wave_lds(const AttnArgs& a) {
  return (size_t)SEL_WPG * sel_wave_lds_bytes(a.n_words, sel_wave_ucap(a));
}

hipError_t launch_sel_wave(const AttnArgs& a, int local, int accumulate, hipStream_t s) {
  const int nclu = (a.cap + SEL_TPW - 1) / SEL_TPW;
  const long long waves = (long long)a.n_qblk * nclu * a.n_kvh;
  if (waves == 0) return hipSuccess;
  const int nwg = (int)((waves + SEL_WPG - 1) / SEL_WPG);
  if (local) {
    hipLaunchKernelGGL(sel_wave_kernel<true>, dim3(nwg), dim3(SEL_WPG * 64), (size_t)SEL_WPG * sel_wave_lds_bytes(0, 1),
                       s, a, accumulate, 1);
    return hipGetLastError();
  }
  const size_t lds = sel_wave_lds(a);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&sel_wave_kernel<false>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(sel_wave_kernel<false>, dim3(nwg), dim3(SEL_WPG * 64), lds, s, a, accumulate, sel_wave_ucap(a));
  return hipGetLastError();
}

hipError_t launch_cmp_pooled(int is_bf16, const AttnArgs& a, int accumulate, int gate_ch, hipStream_t s) {
  return is_bf16 ? launch_cmp_pooled_t<bf16>(a, accumulate, gate_ch, s) : launch_cmp_pooled_t<float>(a, accumulate, gate_ch, s);
}

hipError_t launch_dense(int is_bf16, const DenseArgs& a, hipStream_t s) {
  return is_bf16 ? launch_dense_t<bf16>(a, s) : launch_dense_t<float>(a, s);
}

}  // namespace nsa
