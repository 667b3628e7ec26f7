// Internal interface between the C ABI (api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nsa {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* k_cmp;
  const void* v_cmp;
  const int32_t* sel;
  const int32_t* blk_cnt;
  const void* gates;   // nullable
  void* o;
  float* lse;          // nullable
  int n_blk, cap, n_qh, n_kvh, top_k, sel_groups, n_gch;
  float scale;
  uint32_t branches;
  int n_words;         // ceil(n_blk / 32): selection bitmap words
  int u_cap;           // bound on the number of distinct selected blocks of one query block
  int ring_spins;      // bound on each wait of the selected branch's tile ring
  int ring_stall;      // test hook: extra count the ring waits for (0 in normal use)
  int q_blk0, n_qblk;  // query blocks [q_blk0, q_blk0 + n_qblk)
  int kv_lo, kv_hi;    // key blocks of the compressed and local branches: [kv_lo, kv_hi)
  int sel_per_block;   // routing rows are per query block ([n_blk][sel_groups][top_k]), not per slot
  int ch_sel, ch_loc;  // gate channels of the selected and local branches (the compressed one is 0)
};

struct DenseArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* gates;
  void* o;
  int n_tok, n_x, n_qh, n_kvh;
  float scale;
};

struct RouteArgs {
  const float* pts;
  const int32_t* blk_cnt;
  const uint32_t* blk_key;
  int32_t* cent;        // [n_blk][4]
  int32_t* sel;
  uint32_t* sel_d2;     // nullable
  int n_blk, cap, top_k;
  int q_blk0, n_qblk;   // routed query slots: those of blocks [q_blk0, q_blk0 + n_qblk)
  int kv_lo, kv_hi;     // candidate blocks [kv_lo, kv_hi) (with views: the volume blocks)
  // image blocks found through the views (n_views == 0: none)
  const float* view_proj;   // [n_views][2][4]
  const int32_t* cell_blk;  // [n_views][n_cell][n_cell]
  int32_t* boxes;           // [n_blk][8] workspace: lattice box (lo xyz, -, hi xyz, -) of each block
  int32_t* lat;             // [S][2] workspace: lattice point (x | y << 16, z) of every valid slot
  int n_views, n_cell, cell_shift, radius;
};

struct ScoreRouteArgs {
  const void* q;
  const void* k_cmp;
  const float* lse;
  const int32_t* blk_cnt;
  const uint32_t* blk_key;
  int32_t* sel;
  int n_rows, n_blk, cap, n_qh, n_kvh, top_k;
  float scale;
  int dense_rows;       // rows are n_rows pooled rows, 64 per workgroup (cap = 64), not token slots
};

// One query head per KV head, head dim 64, block-granular queries and routing rows (bf16 or fp32).
struct G1Args {
  const void* q;        // [S][n_qh][64] token queries (selected branch)
  const void* k;        // [S][n_kvh][64]
  const void* v;
  const void* q_cmp;    // [n_blk][n_qh][64] pooled queries
  const void* k_cmp;    // [n_blk][n_kvh][64]
  const void* v_cmp;
  const int32_t* sel;   // routing rows [n_blk][sel_groups][top_k] (attention input, routing output)
  const int32_t* blk_cnt;
  const uint32_t* blk_key;
  const void* gates;    // nullable
  void* o;
  float* lse;           // nullable
  int n_blk, cap, n_qh, n_kvh, top_k, sel_groups, n_gch, ch_cmp, ch_sel, ch_loc;
  float scale;
  uint32_t branches;
  int accumulate;       // selected/local branch adds to o (an earlier branch wrote it first)
  int local;            // sel_g1_kernel: the key set is the query block's own block (local branch)
  int f_lo, f_hi;       // blocks [f_lo, f_hi) are always in the selected branch's key set
};

constexpr int kMaxForcedBlocks = 192;   // longest forced range of the selected branch (blk_cap <= 16)
hipError_t launch_route_g1(int is_bf16, const G1Args& a, hipStream_t s);
hipError_t launch_attn_g1(int is_bf16, const G1Args& a, hipStream_t s);
// compressed branch with the routing of its scores (sel is written), then the selected branch
hipError_t launch_attn_g1_routed(int is_bf16, const G1Args& a, hipStream_t s);

size_t attn_lds_bytes(int is_bf16, const AttnArgs& a);
hipError_t launch_attn(int is_bf16, const AttnArgs& a, hipStream_t s);
// selected branch (bf16, per-token routing rows), or with `local` the local branch, by wave-owned
// clusters of 8 consecutive slots: o = (accumulate ? o : 0) + sigmoid(gates[.., a.ch_sel or
// a.ch_loc]) * result (no gate when a.gates is NULL); padding slots 0 when not accumulating; lse
// when a.lse is set.  Query blocks [q_blk0, +n_qblk); the local branch attends the own block only
// inside [kv_lo, kv_hi).  sel_wave_lds: the selected branch's LDS per workgroup.
size_t sel_wave_lds(const AttnArgs& a);
hipError_t launch_sel_wave(const AttnArgs& a, int local, int accumulate, hipStream_t s);
// compressed branch of pooled queries (a.q = [n_blk][n_qh][D]), each block's result given to its
// valid tokens: o = (accumulate ? o : 0) + sigmoid(gates[.., gate_ch]) * result (no gate when
// a.gates is NULL), padding slots 0 when not accumulating; lse [n_blk][n_qh] when a.lse is set
hipError_t launch_cmp_pooled(int is_bf16, const AttnArgs& a, int accumulate, int gate_ch, hipStream_t s);
hipError_t launch_dense(int is_bf16, const DenseArgs& a, hipStream_t s);
hipError_t launch_pool(int is_bf16, const void* x, void* x_cmp, const int32_t* blk_cnt, int n_blk,
                       int cap, int n_heads, int head_dim, hipStream_t s);
size_t pool_resblock_lds_bytes(int cap, int head_dim);
hipError_t launch_pool_resblock(int is_bf16, const void* x, void* x_cmp, const int32_t* blk_cnt, const float* w1,
                                const float* b1, const float* w2, const float* b2, int n_blk, int cap,
                                int n_heads, int head_dim, hipStream_t s);
hipError_t launch_build_volume_blocks(const float* sdf, int G, int N, float tau, int max_blk,
                                      unsigned long long* cell_mask, int* cell_block, int* n_blk, int32_t* blk_cnt,
                                      uint32_t* blk_key, float* pts, hipStream_t s);
hipError_t launch_route_geometric(const RouteArgs& a, hipStream_t s);
constexpr int kScratchMaxBlocks = 65536;   // blocks of the allocation-free routing entry point
// Device address of the library's fixed centroid array on the current device (looked up once per
// device, then cached); kScratchMaxBlocks x 4 int32.
hipError_t route_scratch_centroids(int32_t** out);
hipError_t launch_route_scores(int is_bf16, const ScoreRouteArgs& a, hipStream_t s);
hipError_t launch_gate(int is_bf16, int n_rows, int n_qh, int head_dim, int n_branch,
                       const void* const* o_branch, const void* gates, void* o, hipStream_t s);

}  // namespace nsa
