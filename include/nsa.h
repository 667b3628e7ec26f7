/*
 * libnsa — Native Sparse Attention forward pass for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is a DEVICE pointer unless it is marked "host".  Every call only
 * validates its arguments on the host and enqueues kernels on the caller's stream: NSA_OK means
 * "enqueued", not "finished".  The library never allocates, frees or synchronises (apart from the
 * opt-in debug check below), keeps no per-call state, and is safe to call from several host
 * threads.  The caller owns every buffer.
 *
 * Status convention for every call:
 *   NSA_ERR_INVALID      a null pointer, a non-positive size, inconsistent sizes (e.g. n_qh not a
 *                        multiple of n_kvh) or a value outside the documented range; nothing is
 *                        launched and no output is touched;
 *   NSA_ERR_UNSUPPORTED  a valid request outside the compiled kernel set (see each call);
 *                        nothing is launched;
 *   NSA_ERR_HIP          a HIP launch error; outputs are unspecified.
 * nsa_last_error() returns a thread-local, human-readable reason for the last non-OK status.
 *
 * Token storage is BLOCK-MAJOR (the spatial block partition of the LSRM pages: hyper.ai summary
 * of arXiv 2604.05182, section 方法, block paragraph): block b owns the slots
 * [b*blk_cap, b*blk_cap + blk_cnt[b]); the other slots of the block are padding.  S = n_blk*blk_cap.
 * Tensors are row-major and contiguous:  q [S][n_qh][D],  k, v [S][n_kvh][D],
 * pooled x_cmp [n_blk][H][D],  gate logits [rows][n_qh][channels],  points [S][3].
 * Query head h reads KV head h / (n_qh / n_kvh) (grouped-query attention of the LSRM pages,
 * dense-transformer paragraph: 32 query heads share 2 KV heads).
 * Padding slots are never read as keys or queries; every output row of a padding slot is written
 * as 0 (attention, gate), -1 (routing indices) or -inf (lse).
 * Device-side preconditions (not checked on the host): 1 <= blk_cnt[b] <= blk_cap; blk_key values
 * are unique; points lie in [-1, 1]; routing indices are -1 or in [0, n_blk).  With the environment
 * variable NSA_DEBUG_CHECKS=1, every call that takes a layout first copies blk_cnt to the host
 * (synchronising the device) and returns NSA_ERR_INVALID if a count lies outside 1..blk_cap.
 * Alignment: every q, k, v, q_cmp, k_cmp, v_cmp, o and lse pointer must be 16-byte aligned
 * (NSA_ERR_UNSUPPORTED otherwise): the kernels read them with 16-byte vector loads.
 */
#ifndef NSA_H
#define NSA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NSA_OK = 0,
  NSA_ERR_INVALID = -1,
  NSA_ERR_UNSUPPORTED = -2,
  NSA_ERR_HIP = -3
} nsa_status;

typedef enum { NSA_F32 = 0, NSA_BF16 = 1 } nsa_dtype;   /* element type of q, k, v, o, gates */

/* Branch bits for nsa_attn_fwd. */
enum {
  NSA_BR_CMP = 1,   /* compressed branch: all pooled blocks                              */
  NSA_BR_SEL = 2,   /* selected branch: the blocks of the routing table                  */
  NSA_BR_LOC = 4    /* local (window) branch: the query's own block                      */
};

typedef enum {
  NSA_Q_TOKEN = 0,  /* routing rows and compressed-branch queries are per token           */
  NSA_Q_BLOCK = 1   /* per block: pooled queries for the compressed branch (output given  */
                    /* to every valid token of the block), one routing row per block      */
} nsa_qgran;

/* Host struct describing the block-major layout.  blk_cnt and blk_key are DEVICE arrays. */
typedef struct {
  int32_t n_blk;            /* >= 1                                                          */
  int32_t blk_cap;          /* 1..64                                                         */
  int32_t n_qh, n_kvh;      /* n_qh % n_kvh == 0                                             */
  int32_t head_dim;         /* D                                                             */
  float scale;              /* softmax scale, callers pass 1/sqrt(D); > 0                    */
  const int32_t* blk_cnt;   /* [n_blk] valid tokens per block, 1..blk_cap                    */
  const uint32_t* blk_key;  /* [n_blk] unique logical block ids; the routing tie-break order */
} nsa_layout;

/*
 * Volume token selection and the volume block table.  LSRM pages, section 方法: eq. M^vol marks a
 * voxel active iff, over its 4^3 sub-sample points p_t, min |s_t| <= tau or
 * (min s_t)(max s_t) <= 0; active tokens are grouped into spatial blocks.
 *   sdf  [G][G][G] float32 (z, y, x): SDF values at the lattice points -1 + 2g/(G-1) of [-1, 1]^3;
 *        s_t is its trilinear interpolation (the dense stage's SDF decoder taken as the identity).
 *   Voxels: N^3 over [-1, 1]^3; sub-sample m = 4i + a of an axis lies at lattice coordinate
 *   u = (2m + 1)(G - 1)/(8N).  The decision is taken in fp32 with every operation rounded in a
 *   fixed order: u by one division; g0 = min(floor(u), G - 2), f = u - g0; lerp(a, b, f) =
 *   a + f (b - a) along x, then y, then z (no fused multiply-adds).
 *   Blocks: the 4^3-voxel cells with at least one active voxel, in ascending Morton order of the
 *   cell (bits interleaved x, y, z from the least significant); inside a block the active voxels in
 *   ascending Morton order of their position in the cell; capacity 64.
 * Outputs: n_blk (device int32) = the number of blocks; for b < min(n_blk, max_blk):
 *   blk_cnt[b] (1..64), blk_key[b] = the cell's Morton code, pts[b*64 + r][3] = the r-th token's
 *   voxel centre ((2i + 1) - N)/N per axis (one rounded division), 0 on padding slots.  Blocks at
 *   or beyond max_blk are not written (compare n_blk with max_blk after the call).
 * Workspace: cell_mask [(N/4)^3] uint64 (active voxels of each cell) and cell_block [(N/4)^3]
 * int32 (block index of each cell, -1 if empty), both indexed by the cell's Morton code and
 * written.  N a positive multiple of 4 (else NSA_ERR_INVALID); N / 4 a power of two, N <= 512 and
 * 8*N*G < 2^24 (else NSA_ERR_UNSUPPORTED); G >= 2 and tau finite and >= 0 (else NSA_ERR_INVALID).
 * The device buffers are caller-owned; the call is asynchronous on `stream`.
 */
nsa_status nsa_build_volume_blocks(const float* sdf, int32_t G, int32_t N, float tau, int32_t max_blk,
                                   uint64_t* cell_mask, int32_t* cell_block, int32_t* n_blk,
                                   int32_t* blk_cnt, uint32_t* blk_key, float* pts,
                                   hipStream_t stream);

/*
 * Block compression.  LSRM pages, section 方法, eq. k^cmp = AvgPool(ResBlock(k_t)) (ResBlock taken
 * as the identity); Speed3R page (arXiv 2603.08055 summary), section 2.1, 4x4 average pooling of
 * Q/K/V.  x_cmp[b][h][:] = mean of x[s][h][:] over the valid slots s of block b, accumulated in
 * fp32 and rounded to `dtype`.
 *   x      [S][n_heads][head_dim]      x_cmp  [n_blk][n_heads][head_dim]
 * n_heads * head_dim must be a multiple of 8 (bf16) or 4 (f32) and x, x_cmp 16-byte aligned
 * (NSA_ERR_UNSUPPORTED otherwise): each row is read in 16-byte pieces.
 */
nsa_status nsa_pool_blocks(const nsa_layout* layout, nsa_dtype dtype, int32_t n_heads,
                           const void* x, void* x_cmp, hipStream_t stream);

/*
 * Block compression with the residual module: LSRM pages, section 方法, eq.
 * k^cmp = AvgPool(ResBlock(k_t)), v^cmp = AvgPool(ResBlock(v_t)).  The pages do not define the
 * module; this call takes one residual MLP per head,
 *     ResBlock(x) = x + W2 silu(W1 x + b1) + b2,  silu(a) = a / (1 + e^-a),
 * applied to each valid token's head vector, then the mean over the block's valid tokens,
 * accumulated in fp32 and rounded to `dtype`.
 *   x [S][n_heads][head_dim] (dtype);  x_cmp [n_blk][n_heads][head_dim] (dtype)
 *   w1, w2 [n_heads][head_dim][head_dim] float32 (row j of w1[h] feeds hidden unit j, row d of
 *   w2[h] feeds output d);  b1, b2 [n_heads][head_dim] float32.
 * head_dim <= 64 (NSA_ERR_UNSUPPORTED otherwise).  Zero weights give nsa_pool_blocks.
 */
nsa_status nsa_pool_blocks_resblock(const nsa_layout* layout, nsa_dtype dtype, int32_t n_heads,
                                    const void* x, const float* w1, const float* b1,
                                    const float* w2, const float* b2, void* x_cmp,
                                    hipStream_t stream);

/*
 * 3D-aware geometric routing.  LSRM pages, section 方法, routing paragraph (and the Korean summary,
 * section 2.2): each query token keeps the blocks whose centres lie nearest to its 3D point.
 * Exact integer form: u = rint(4096*p) + 4096 per axis; block centroid
 * c_b = floor((2*sum u + cnt_b) / (2*cnt_b)); d2 = |u_t - c_b|^2 (< 2^28).  Each valid token gets
 * the top_k blocks in ascending (d2, blk_key) order, best first.  One list per token, shared by all
 * heads.
 *   pts        [S][3] float32 in [-1, 1]
 *   centroids  [n_blk][4] int32 workspace and output: (cx, cy, cz, blk_key bits)
 *   sel        [S][top_k] int32 storage block indices; -1 on padding rows and beyond n_blk
 *   sel_d2     [S][top_k] uint32 or NULL; 0xFFFFFFFF where sel is -1
 * 1 <= top_k <= 64.
 */
nsa_status nsa_route_geometric(const nsa_layout* layout, const float* pts, int32_t top_k,
                               int32_t* centroids, int32_t* sel, uint32_t* sel_d2,
                               hipStream_t stream);

/*
 * nsa_route_geometric for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same routing, with the
 * centroid workspace taken from a fixed array inside the library (65,536 blocks x 4 int32 = 1 MiB
 * per device, held until the process ends) instead of a caller buffer.  The call allocates
 * nothing.  Every call on one device shares that device's array and rewrites the centroids of
 * blocks [0, n_blk) before reading them, so nothing carries over from an earlier call; calls that
 * overlap in time on one device (two streams, two host threads) race on the array and must not be
 * issued.  n_blk > 65536 returns NSA_ERR_UNSUPPORTED; other arguments and results are those of
 * nsa_route_geometric.
 */
nsa_status nsa_route_geometric_noalloc(const nsa_layout* layout, const float* pts, int32_t top_k,
                                       int32_t* sel, uint32_t* sel_d2, hipStream_t stream);

/*
 * Geometric routing with the image blocks found through the views (LSRM pages, section 方法,
 * routing paragraph: for image blocks the query point is projected into every input view, nearby
 * image blocks are gathered per view and ranked by their smallest 3D distance to the query; volume
 * blocks are ranked by the distance to their centres).  On the lattice of nsa_route_geometric:
 *   volume candidates: blocks [0, n_vol_blk), metric d2(u_t, c_b) to the block centroid;
 *   image candidates: for each view v, the cell (cx, cy) = floor(proj_v(p_t) / cell_size) with
 *     proj_v(p) = ((A0 p.x + A1 p.y) + A2 p.z) + A3 per image axis (A = view_proj[v][axis][0..3],
 *     every operation rounded to float32 in that order), then the blocks cell_blk[v][y][x] >= 0 of
 *     the cells |x - cx| <= radius, |y - cy| <= radius inside the n_cell x n_cell grid; metric =
 *     min over the block's valid tokens s of d2(u_t, u_s).
 * One ranking of all candidates by ascending (d2, blk_key), top_k best first, as in
 * nsa_route_geometric; every valid slot's row is written (-1 / 0xFFFFFFFF past the candidates).
 *   view_proj [n_views][2][4] float32, cell_blk [n_views][n_cell][n_cell] int32 (device); every
 *   entry >= 0 names a block outside [0, n_vol_blk), and a block appears at most once;
 *   centroids [n_blk][4] and geom [n_blk * 8 + S * 2] int32 are workspaces (geom: each block's
 *   lattice bounding box, used to skip candidates that cannot reach a token's current top k, then
 *   every slot's lattice point).
 * 0 <= n_vol_blk <= n_blk, n_views >= 0 (0: volume blocks only), 1 <= n_cell <= 4096, cell_size
 * a power of two <= 1024, 0 <= radius <= 16, 1 <= top_k <= 64 (NSA_ERR_INVALID otherwise).
 */
nsa_status nsa_route_geometric_views(const nsa_layout* layout, const float* pts, int32_t top_k,
                                     int32_t n_vol_blk, int32_t n_views, const float* view_proj,
                                     const int32_t* cell_blk, int32_t n_cell, int32_t cell_size,
                                     int32_t radius, int32_t* centroids, int32_t* geom,
                                     int32_t* sel, uint32_t* sel_d2, hipStream_t stream);

/*
 * Geometric routing over a block range, for the split self/cross form of stage 2 (LSRM pages,
 * section 方法: stage 2 keeps stage 1's decoupled self and cross attention, eq. o^x, o^y, with
 * sparse attention in place of dense; volume and image blocks are routed separately).  The metric
 * and order are those of nsa_route_geometric; only the blocks [kv_blk_lo, kv_blk_hi) are
 * candidates, and only the rows of the slots of blocks [q_blk_lo, q_blk_hi) are written (other
 * rows of sel / sel_d2 are left untouched).  Positions beyond the candidate count hold -1.
 * centroids is rewritten for every block.  0 <= lo <= hi <= n_blk for both ranges
 * (NSA_ERR_INVALID otherwise); an empty query range launches nothing.
 */
nsa_status nsa_route_geometric_range(const nsa_layout* layout, const float* pts, int32_t top_k,
                                     int32_t q_blk_lo, int32_t q_blk_hi, int32_t kv_blk_lo,
                                     int32_t kv_blk_hi, int32_t* centroids, int32_t* sel,
                                     uint32_t* sel_d2, hipStream_t stream);

/*
 * Score routing against the compressed keys ("standard NSA" selection the LSRM pages compare
 * with; Speed3R page, section 2.1, top-K from the compressed score matrix), without storing the
 * score matrix.
 *   G = n_qh/n_kvh > 1: importance of block b for (row r, group j) is
 *       sum over the group's heads h of exp(scale*<q[r][h], k_cmp[b][j]> - lse[r][h]);
 *   G == 1: importance of block b for (row r, head h) is <q[r][h], k_cmp[b][h]>.
 * Blocks are ranked by descending importance, ties by ascending blk_key.
 *   q_gran NSA_Q_TOKEN: rows = S, q [S][n_qh][D] (padding rows get -1)
 *   q_gran NSA_Q_BLOCK: rows = n_blk, q is the pooled query [n_blk][n_qh][D] (with G > 1, lse is
 *   then the pooled rows' compressed-branch lse, as nsa_attn_fwd returns it for CMP with
 *   NSA_Q_BLOCK)
 *   k_cmp [n_blk][n_kvh][D];  lse [rows][n_qh] float32 natural-log partition function of the
 *   compressed branch (required iff G > 1);  sel [rows][n_kvh][top_k] int32.
 * Supported: (D, G) = (32, 16) with either q_gran (bf16 or f32, n_blk <= 65536), and (64, 1) with
 * q_gran BLOCK (bf16 or f32; scores are fp32 products of the stored rows); 1 <= top_k <= 64.
 */
nsa_status nsa_route_scores_topk(const nsa_layout* layout, nsa_dtype dtype, nsa_qgran q_gran,
                                 const void* q, const void* k_cmp, const float* lse,
                                 int32_t top_k, int32_t* sel, hipStream_t stream);

/*
 * NSA attention branches, optionally gated and fused.  LSRM pages, section 方法: compressed block
 * features give global coarse context, selected blocks give fine detail, window attention runs
 * inside a block; Speed3R page, section 2.1: a learned gate combines the branches.
 * For query row r, head h and the key set K of a branch:
 *     o_h = sum_{i in K} softmax_i(scale * <q_h, k_i>) v_i        (empty K gives o_h = 0)
 *   CMP: K = every pooled block (k_cmp, v_cmp); queries are q (NSA_Q_TOKEN) or the block's pooled
 *        query q_cmp (NSA_Q_BLOCK, result given to each valid token of the block);
 *   SEL: K = valid tokens of the blocks in the routing row (duplicates count once, -1 skipped);
 *        rows are per token (NSA_Q_TOKEN) or per block (NSA_Q_BLOCK);
 *        sel_groups == 1: sel [rows][top_k] shared by all heads;
 *        sel_groups == n_kvh: sel [rows][n_kvh][top_k], head h uses group h / (n_qh/n_kvh);
 *   LOC: K = valid tokens of the query's own block.
 * `branches` is a non-empty OR of NSA_BR_* bits.  If gate_logits is NULL, exactly one branch must
 * be named and o receives it.  Otherwise o = sum over the named branches c of
 * sigmoid(gate_logits[s][h][ch(c)]) * o_c, where ch(c) is c's rank among the named branches in the
 * order CMP, SEL, LOC and gate_logits is [S][n_qh][popcount(branches)] in `dtype`.
 *   q [S][n_qh][D]; k, v [S][n_kvh][D] (SEL, LOC); q_cmp [n_blk][n_qh][D] (CMP with NSA_Q_BLOCK);
 *   k_cmp, v_cmp [n_blk][n_kvh][D] (CMP); unused pointers may be NULL.  o [S][n_qh][D].
 *   lse: NULL, or (single branch only) float32 [rows][n_qh] natural-log partition function,
 *        rows = n_blk for CMP with NSA_Q_BLOCK, else S; -inf on padding rows and empty key sets.
 * Supported: (D, G) = (32, 16) for NSA_F32 and NSA_BF16 (n_blk <= 65536 when SEL is named;
 * n_blk * blk_cap * n_qh * max(32, gate_stride) < 2^31, row offsets being 32-bit).  With NSA_Q_TOKEN
 * and NSA_BF16 the selected branch runs in a second kernel after the fused kernel's other branches
 * and adds its gated result to o (o is rounded to bf16 in between); without the compressed branch
 * the local branch runs in that kernel family too, first (the environment variable NSA_SEL_RING=1
 * keeps every branch in the fused kernel instead).  With NSA_Q_BLOCK
 * the selected and local branches run first in the fused kernel (token queries, the block's
 * routing row for every token) and the compressed branch of the pooled queries then adds each
 * block's gated result to its tokens (o is rounded to `dtype` in between).  And
 * (D, G) = (64, 1) for NSA_F32 and NSA_BF16 with NSA_Q_BLOCK (pooled queries in the compressed
 * branch, token queries in the selected and local ones), blk_cap in {1, 2, 4, 8, 16}: each named
 * branch runs in its own launch, the first writing its gated result to o in `dtype` and the later
 * ones adding to it.  top_k <= 64.  Accumulation is fp32; with bf16 inputs bf16 probabilities feed
 * the value product, with fp32 inputs fp32 ones.
 */
nsa_status nsa_attn_fwd(const nsa_layout* layout, nsa_dtype dtype, uint32_t branches,
                        nsa_qgran q_gran, const void* q, const void* k, const void* v,
                        const void* q_cmp, const void* k_cmp, const void* v_cmp,
                        const int32_t* sel, int32_t top_k, int32_t sel_groups,
                        const void* gate_logits, void* o, float* lse, hipStream_t stream);

/*
 * The compressed and selected branches with block queries, routed by the compressed branch's own
 * scores in the same pass (Speed3R page, section 2.1: every query block picks, per head, the
 * top-k key blocks by its pooled scores, and its tokens attend those blocks).  Equals
 * nsa_route_scores_topk(layout, dtype, NSA_Q_BLOCK, q_cmp, k_cmp, NULL, top_k, sel) followed by
 * nsa_attn_fwd(layout, dtype, NSA_BR_CMP | NSA_BR_SEL, NSA_Q_BLOCK, q, k, v, q_cmp, k_cmp, v_cmp,
 * sel, top_k, n_kvh, gate_logits, o, NULL): sel receives the same routing rows
 * [n_blk][n_kvh][top_k] (descending by score, ties to the smaller blk_key, -1 past the last
 * block), while the compressed branch's logits are formed in fp32 from the raw pooled queries
 * (rather than from bf16 queries pre-scaled by scale * log2(e)), so o agrees with the two-call
 * sequence to rounding.  gate_logits [S][n_qh][2] (channel 0 compressed, 1 selected), in `dtype`.
 * With NSA_F32 the routing runs as its own pass before the two branches (exactly the two-call
 * sequence); with NSA_BF16 it shares the compressed branch's pass.
 * Supported (NSA_ERR_UNSUPPORTED otherwise): n_qh == n_kvh, head_dim 64, blk_cap in
 * {1, 2, 4, 8, 16}, top_k <= 32.  sel and o must not overlap any input.
 */
nsa_status nsa_attn_fwd_scores_routed(const nsa_layout* layout, nsa_dtype dtype, const void* q,
                                      const void* k, const void* v, const void* q_cmp,
                                      const void* k_cmp, const void* v_cmp, int32_t top_k,
                                      const void* gate_logits, void* o, int32_t* sel,
                                      hipStream_t stream);

/*
 * nsa_attn_fwd with a forced block range in the selected branch (Speed3R page, section 2.2: in the
 * variant for a model with a reference frame, that frame's tokens are always attended, whatever the
 * routing picks).  SEL's key set for every row becomes the valid tokens of the union of the routed
 * blocks and the blocks [forced_lo, forced_hi); a block both routed and forced counts once.  All
 * other arguments, branches and gates are those of nsa_attn_fwd.  forced_lo == forced_hi is
 * nsa_attn_fwd itself.  Supported for (D, G) = (64, 1) with NSA_Q_BLOCK (the score-routed path)
 * and at most 192 forced blocks (NSA_ERR_UNSUPPORTED otherwise); 0 <= forced_lo <= forced_hi <=
 * n_blk, and SEL among the branches when the range is non-empty (NSA_ERR_INVALID).
 */
nsa_status nsa_attn_fwd_forced(const nsa_layout* layout, nsa_dtype dtype, uint32_t branches,
                               nsa_qgran q_gran, const void* q, const void* k, const void* v,
                               const void* q_cmp, const void* k_cmp, const void* v_cmp,
                               const int32_t* sel, int32_t top_k, int32_t sel_groups,
                               int32_t forced_lo, int32_t forced_hi, const void* gate_logits,
                               void* o, float* lse, hipStream_t stream);

/*
 * nsa_attn_fwd over a block range, for the split self/cross form of stage 2 (LSRM pages, section
 * 方法: eq. o^x, o^y with each attention over one token type's blocks): only the query blocks
 * [q_blk_lo, q_blk_hi) are computed (their rows of o and lse are written, the others are left
 * untouched); CMP attends the pooled blocks [kv_blk_lo, kv_blk_hi) only; LOC attends the own block
 * only when it lies in that range (else it adds 0); SEL attends the routing rows as given (route
 * them with nsa_route_geometric_range).  Gate channels: the named branches read channels 0, 1, ...
 * of gate_logits[s][h][*], whose row length is gate_stride (0 means the number of named branches),
 * so a caller can point gate_logits into a wider gate tensor.  Other arguments and rules are those
 * of nsa_attn_fwd with NSA_Q_TOKEN; supported for (D, G) = (32, 16) only (NSA_ERR_UNSUPPORTED
 * otherwise); 0 <= lo <= hi <= n_blk for both ranges and gate_stride <= 64 (NSA_ERR_INVALID).
 */
nsa_status nsa_attn_fwd_range(const nsa_layout* layout, nsa_dtype dtype, uint32_t branches,
                              int32_t q_blk_lo, int32_t q_blk_hi, int32_t kv_blk_lo,
                              int32_t kv_blk_hi, const void* q, const void* k, const void* v,
                              const void* k_cmp, const void* v_cmp, const int32_t* sel,
                              int32_t top_k, int32_t sel_groups, const void* gate_logits,
                              int32_t gate_stride, void* o, float* lse, hipStream_t stream);

/*
 * Sigmoid-gated sum of branch outputs (LSRM pages, section 方法, Sigmoid gates; Speed3R page,
 * section 2.1, gated aggregation), as a standalone pass:
 *     o[r][h][:] = sum_c sigmoid(gate_logits[r][h][c]) * o_branch[c][r][h][:]
 *   o_branch   host array of n_branch device pointers, each [n_rows][n_qh][head_dim]
 *   gate_logits [n_rows][n_qh][n_branch];  o [n_rows][n_qh][head_dim];  1 <= n_branch <= 8.
 * head_dim must be a multiple of 4 and o, o_branch[c] aligned to 4 elements (NSA_ERR_UNSUPPORTED
 * otherwise): each thread moves four consecutive elements.
 */
nsa_status nsa_gate_combine(nsa_dtype dtype, int32_t n_rows, int32_t n_qh, int32_t head_dim,
                            int32_t n_branch, const void* const* o_branch,
                            const void* gate_logits, void* o, hipStream_t stream);

/*
 * Stage-1 dense gated self/cross attention (LSRM pages, section 方法, eq. o^x and o^y):
 * tokens [0, n_x) are volume tokens x, [n_x, n_tok) image tokens y, and
 *     o_t = sigmoid(g[t][h][0]) * Attn(q_t; keys of t's own type)
 *         + sigmoid(g[t][h][1]) * Attn(q_t; keys of the other type),
 * an empty key set contributing 0.  q [n_tok][n_qh][D]; k, v [n_tok][n_kvh][D];
 * gate_logits [n_tok][n_qh][2]; o [n_tok][n_qh][D].  0 <= n_x <= n_tok.
 * Supported: (D, G) = (32, 16) for NSA_F32 and NSA_BF16, n_tok * n_qh * 32 < 2^31
 * (NSA_ERR_UNSUPPORTED otherwise: row offsets are 32-bit).
 */
nsa_status dense_gated_xattn_fwd(nsa_dtype dtype, int32_t n_tok, int32_t n_x, int32_t n_qh,
                                 int32_t n_kvh, int32_t head_dim, float scale, const void* q,
                                 const void* k, const void* v, const void* gate_logits, void* o,
                                 hipStream_t stream);

/* Thread-local description of the last non-OK status returned on this thread (host string). */
const char* nsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NSA_H */
