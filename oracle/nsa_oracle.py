"""Plain fp64 CPU oracle for the NSA forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the benchmark's CPU-baseline leg
may import this module.  It shares no code with the HIP library and does not import it; the only
module both sides use is the seeded input generator (`workloads`), which holds none of the
method's arithmetic.

Every function is written from the pages' statement of the method, in the plainest form: explicit
loops over query rows and blocks, numpy for the small per-row vector products, float64 throughout
(inputs are first widened exactly from their float32 / bfloat16 values).  The active-voxel rule and
the view projection are float64 too: a device that decides them in float32 can differ only where
the float64 value lies within its rounding error of a threshold or a cell edge, and the tests
count and leave out exactly those cases.  check_route_geometric is a vectorised whole-table check
of a routing result against route_geometric's definition (test infrastructure for full-size
tables); every function here is pinned by tests/test_oracle*.py.

Sources (cited by page title and section; no page prints code or worked numbers):
  [LSRM-cn]  hyper.ai summary of "LSRM" (arXiv 2604.05182), section 方法 (Method):
             gated self/cross attention (eq. o^x, o^y and the Sigmoid gates), block partition,
             compression eq. k^cmp / v^cmp = AvgPool(ResBlock(.)), compressed + selected branches,
             3D-aware block routing (voxel centre / surface point, distance to block centres),
             window (local) attention inside a block.
  [LSRM-ko]  gist.science Korean technical summary of LSRM, section 2.2: geometric routing and
             block-aware locality.
  [Speed3R]  gist.science summary of "Speed3R" (arXiv 2603.08055), section 2.1 Global Sparse
             Attention: pooled Q/K/V compression branch, top-K selection from the compressed score
             matrix, learned gate combining the branches.

Readings where the pages are silent:
  * softmax scale is a parameter (callers pass 1/sqrt(D)); attention is non-causal;
  * ResBlock before AvgPool is the identity for the layer's compression (the mean over a block's
    valid tokens); with seeded weights it is one residual MLP per head, x + W2 silu(W1 x + b1) + b2;
  * padded slots are neither keys nor queries; padded outputs are 0, padded routing rows are -1;
  * geometric routing ranks blocks by the exact integer squared distance between the query point
    and the block centroid on a 2^-12 lattice (u = rint(4096 p) + 4096), ties by ascending blk_key;
  * GQA score routing sums the group's softmax probabilities against the compressed keys;
  * each gate channel is an independent sigmoid; an empty key set contributes 0;
  * the split self/cross form of stage 2 keeps stage 1's two sigmoid gates over an NSA per token
    type, each NSA with its own branch gates (cross: compressed + selected, no local window).
"""
from __future__ import annotations

import math

import numpy as np

CMP, SEL, LOC = 0, 1, 2
BRANCH_NAMES = {"cmp": CMP, "sel": SEL, "loc": LOC}


# ----------------------------------------------------------------------------------------------
# basic pieces
# ----------------------------------------------------------------------------------------------

def sigmoid(x):
    """Logistic gate of [LSRM-cn] eq. w = Sigmoid(Linear_gate(.)); exact 0 and 1 at -inf / +inf."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def valid_mask(blk_cnt, cap):
    """Slot s (in block s // cap) holds a token iff s % cap < cnt[s // cap]."""
    blk_cnt = np.asarray(blk_cnt)
    slot = np.arange(blk_cnt.shape[0] * cap)
    return (slot % cap) < blk_cnt[slot // cap]


def block_slots(blk_cnt, cap, b):
    """The storage slots of block b's valid tokens."""
    return np.arange(b * cap, b * cap + int(blk_cnt[b]))


def attend(qrow, keys, vals, scale, return_weights=False):
    """Softmax attention of one query row against an explicit key set.

    qrow [Hq, D]; keys, vals [n, Hkv, D]; query head h reads KV head h // (Hq // Hkv) (grouped-query
    attention, [LSRM-cn] dense transformer paragraph).  For each head:
        s_i = scale * <q_h, k_i>,  a_i = exp(s_i - max s) / sum_j exp(s_j - max s),  o_h = sum_i a_i v_i
    Returns (o [Hq, D], lse [Hq]) with lse = max s + log(sum exp(s - max s)); an empty key set gives
    o = 0 and lse = -inf.
    """
    qrow = np.asarray(qrow, dtype=np.float64)
    Hq, D = qrow.shape
    n = keys.shape[0]
    if n == 0:
        o = np.zeros((Hq, D))
        lse = np.full(Hq, -np.inf)
        return (o, lse, np.zeros((Hq, 0))) if return_weights else (o, lse)
    Hkv = keys.shape[1]
    G = Hq // Hkv
    o = np.zeros((Hq, D))
    lse = np.zeros(Hq)
    weights = np.zeros((Hq, n))
    for h in range(Hq):
        j = h // G
        s = scale * (keys[:, j, :].astype(np.float64) @ qrow[h])
        m = s.max()
        e = np.exp(s - m)
        z = e.sum()
        a = e / z
        o[h] = a @ vals[:, j, :].astype(np.float64)
        lse[h] = m + math.log(z)
        weights[h] = a
    return (o, lse, weights) if return_weights else (o, lse)


# ----------------------------------------------------------------------------------------------
# A1: block compression
# ----------------------------------------------------------------------------------------------

def pool_blocks(x, blk_cnt, cap):
    """Compressed block features, [LSRM-cn] eq. k^cmp = AvgPool(ResBlock(k_t)) with the ResBlock
    taken as the identity, and the 4x4 average pooling of Q/K/V in [Speed3R] 2.1: the mean of the
    block's valid tokens.  x [S, H, D] -> [n_blk, H, D] (float64)."""
    blk_cnt = np.asarray(blk_cnt)
    n_blk = blk_cnt.shape[0]
    out = np.zeros((n_blk,) + x.shape[1:])
    for b in range(n_blk):
        rows = x[block_slots(blk_cnt, cap, b)].astype(np.float64)
        out[b] = rows.sum(axis=0) / rows.shape[0]
    return out


def silu(x):
    """x * sigmoid(x), the residual module's activation (a reading: the pages name no activation)."""
    return np.asarray(x, dtype=np.float64) * sigmoid(x)


def resblock(x, w1, b1, w2, b2):
    """The residual module applied to token keys / values before pooling, [LSRM-cn] eq.
    k^cmp = AvgPool(ResBlock(k_t)).  The pages do not define the module; the reading here is one
    residual MLP per head with its own weights, hidden width D:
        ResBlock(x) = x + W2 silu(W1 x + b1) + b2          (x a token's D-vector of head h)
    x [..., H, D]; w1, w2 [H, D, D] (row j of w1[h] feeds hidden unit j; row d of w2[h] feeds
    output d); b1, b2 [H, D]."""
    x = np.asarray(x, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    b1 = np.asarray(b1, dtype=np.float64)
    b2 = np.asarray(b2, dtype=np.float64)
    out = np.empty_like(x)
    for h in range(x.shape[-2]):
        hidden = silu(x[..., h, :] @ w1[h].T + b1[h])
        out[..., h, :] = x[..., h, :] + hidden @ w2[h].T + b2[h]
    return out


def pool_blocks_resblock(x, blk_cnt, cap, w1, b1, w2, b2):
    """[LSRM-cn] eq. k^cmp = AvgPool(ResBlock(k_t)): the residual module on every valid token, then
    the mean over the block's valid tokens.  x [S, H, D] -> [n_blk, H, D] (float64)."""
    blk_cnt = np.asarray(blk_cnt)
    out = np.zeros((blk_cnt.shape[0],) + x.shape[1:])
    for b in range(blk_cnt.shape[0]):
        rows = resblock(x[block_slots(blk_cnt, cap, b)], w1, b1, w2, b2)
        out[b] = rows.sum(axis=0) / rows.shape[0]
    return out


# ----------------------------------------------------------------------------------------------
# A0 on the device: active-voxel selection and the volume block table
# ----------------------------------------------------------------------------------------------

def _morton3_u(x, y, z):
    """Morton code with bits interleaved x (least significant), y, z, for coordinates < 2^10."""
    code = np.zeros(np.broadcast(x, y, z).shape, dtype=np.int64)
    for bit in range(10):
        code |= ((np.asarray(x) >> bit) & 1) << (3 * bit)
        code |= ((np.asarray(y) >> bit) & 1) << (3 * bit + 1)
        code |= ((np.asarray(z) >> bit) & 1) << (3 * bit + 2)
    return code


def voxel_activity(sdf, N, tau, return_values=False):
    """Active voxels of an N^3 grid over [-1, 1]^3, [LSRM-cn] eq. M^vol: voxel (i, j, k) is active iff
    over its 4^3 sub-sample points min |s_t| <= tau or (min s_t) (max s_t) <= 0, with
    s_t = Trilinear(sdf; p_t) (the dense stage's decoder taken as the identity on an SDF volume).

    sdf [G][G][G] (z, y, x) holds values at the lattice points -1 + 2 g / (G - 1).  Sub-sample m of an
    axis (m = 4 i + a, a < 4) sits at the centre of its quarter of the voxel, -1 + (2m + 1) / (4N),
    i.e. at lattice coordinate u = (2m + 1)(G - 1) / (8N).  Trilinear interpolation in the lattice
    cell holding u: linear interpolation a + f (b - a) along x, then y, then z (exact on a constant
    field and at the lattice points); everything in float64, and tau is taken as given.
    Returns bool [N][N][N] (z, y, x); with return_values also the float64 per-voxel min |s|, min s
    and max s over the sub-samples (for callers that bound another precision's decision)."""
    sdf = np.asarray(sdf, dtype=np.float64)
    G = sdf.shape[0]
    m = np.arange(4 * N, dtype=np.int64)
    u = (2 * m + 1) * (G - 1) / (8.0 * N)                # exact rational, one float64 rounding
    g0 = np.minimum(np.floor(u).astype(np.int64), G - 2)
    fr = u - g0

    def lerp(a, b, t):
        return a + t * (b - a)

    # the interpolation is separable: along x for every lattice row, then y, then z
    ax = lerp(sdf[:, :, g0], sdf[:, :, g0 + 1], fr[None, None, :])             # [G][G][4N]
    ay = lerp(ax[:, g0, :], ax[:, g0 + 1, :], fr[None, :, None])               # [G][4N][4N]
    act = np.zeros((N, N, N), dtype=bool)
    mabs = np.zeros((N, N, N))
    mins = np.zeros((N, N, N))
    maxs = np.zeros((N, N, N))
    for k in range(N):                                 # one z-slab of voxels (4 sub-sample planes)
        mz = np.arange(4 * k, 4 * k + 4)
        s = lerp(ay[g0[mz]], ay[g0[mz] + 1], fr[mz][:, None, None])              # [4][4N][4N]
        s = s.reshape(4, N, 4, N, 4).transpose(1, 3, 0, 2, 4).reshape(N, N, 64)   # [j][i][64 samples]
        mn, mx, ma = s.min(axis=2), s.max(axis=2), np.abs(s).min(axis=2)
        act[k] = (ma <= tau) | ((mn <= 0) & (mx >= 0))     # (min s)(max s) <= 0, as a sign test
        mabs[k], mins[k], maxs[k] = ma, mn, mx
    if return_values:
        return act, mabs, mins, maxs
    return act


def volume_block_table(sdf, N, tau):
    """The volume block table built from the active voxels ([LSRM-cn] block paragraph: active tokens
    grouped into spatial blocks that keep 3D locality): blocks are the 4^3-voxel cells holding at
    least one active voxel, in ascending Morton order of the cell; inside a block the active voxels
    follow ascending Morton order of their position in the cell; capacity 64.
    Returns blk_cnt int32 [n_blk], blk_key uint32 [n_blk] (the cell's Morton code) and pts float32
    [n_blk * 64, 3] (voxel centres ((2i + 1) - N) / N per axis, one rounded division; padding 0)."""
    act = voxel_activity(sdf, N, tau)
    kz, jy, ix = np.nonzero(act)
    cell = _morton3_u(ix >> 2, jy >> 2, kz >> 2)
    local = _morton3_u(ix & 3, jy & 3, kz & 3)
    order = np.lexsort((local, cell))
    kz, jy, ix, cell = kz[order], jy[order], ix[order], cell[order]
    keys, start, cnt = np.unique(cell, return_index=True, return_counts=True)
    n_blk = keys.shape[0]
    pts = np.zeros((n_blk * 64, 3), dtype=np.float32)
    f32 = np.float32
    for b in range(n_blk):
        sl = slice(start[b], start[b] + cnt[b])
        for ax, c in enumerate((ix[sl], jy[sl], kz[sl])):
            pts[b * 64: b * 64 + cnt[b], ax] = ((2 * c + 1).astype(f32) - f32(N)) / f32(N)
    return cnt.astype(np.int32), keys.astype(np.uint32), pts


# ----------------------------------------------------------------------------------------------
# A2: 3D-aware geometric routing
# ----------------------------------------------------------------------------------------------

def lattice_coords(pts):
    """Query points on the 2^-12 lattice: u = rint(4096 p) + 4096 per axis, p in [-1, 1] -> [0, 8192]."""
    return (np.rint(4096.0 * np.asarray(pts, dtype=np.float64)) + 4096.0).astype(np.int64)


def block_centroids(pts, blk_cnt, cap):
    """Centroid of each block's member points on the lattice, rounded half-up:
    c_b = floor((2 * sum_t u_t + cnt_b) / (2 * cnt_b)) per axis (all quantities non-negative)."""
    u = lattice_coords(pts)
    blk_cnt = np.asarray(blk_cnt)
    c = np.zeros((blk_cnt.shape[0], 3), dtype=np.int64)
    for b in range(blk_cnt.shape[0]):
        tot = u[block_slots(blk_cnt, cap, b)].sum(axis=0)
        n = int(blk_cnt[b])
        c[b] = (2 * tot + n) // (2 * n)
    return c


def route_geometric(pts, blk_cnt, blk_key, cap, top_k, rows=None):
    """3D-aware block routing ([LSRM-cn] routing paragraph; [LSRM-ko] 2.2): each query token keeps
    the blocks whose centres are nearest to its 3D point.  The metric is the exact squared distance
    d2(t, b) = |u_t - c_b|^2 (an integer < 2^28); blocks are taken in ascending (d2, blk_key) order.

    Returns sel int32 [len(rows), top_k] (storage block indices, best first) and d2 uint32 of the
    same shape.  Padding rows and positions beyond n_blk hold -1 / 0xFFFFFFFF.
    rows defaults to every slot.
    """
    blk_cnt = np.asarray(blk_cnt)
    blk_key = np.asarray(blk_key, dtype=np.int64)
    S = blk_cnt.shape[0] * cap
    rows = np.arange(S) if rows is None else np.asarray(rows)
    valid = valid_mask(blk_cnt, cap)
    cen = block_centroids(pts, blk_cnt, cap)
    u = lattice_coords(pts)
    sel = np.full((rows.shape[0], top_k), -1, dtype=np.int32)
    dd = np.full((rows.shape[0], top_k), 0xFFFFFFFF, dtype=np.uint32)
    kk = min(top_k, blk_cnt.shape[0])
    for i, r in enumerate(rows):
        if not valid[r]:
            continue
        d2 = ((u[r][None, :] - cen) ** 2).sum(axis=1)
        order = np.lexsort((blk_key, d2))[:kk]
        sel[i, :kk] = order
        dd[i, :kk] = d2[order]
    return sel, dd


def check_route_scores(q_rows, k_cmp, blk_key, sel, eps_rel, chunk=1024, scale=None, row_valid=None):
    """Whole-table check of score-routing rows against the definition of route_scores, vectorised so
    that it covers every row of a full-size table.
      * one query head per KV head ([Speed3R] 2.1): the importance of block b for (row r, head h) is
        the compressed score <q_rh, k_bh>;
      * several query heads per KV head ([LSRM-cn] "standard NSA" selection): the importance for
        (row r, KV group j) is the group's summed softmax probability,
        sum over its heads h of exp(scale <q_rh, k_bj> - lse_rh), where lse_rh is the compressed
        branch's log-partition function over all blocks (computed here from the same products).
    Importances are float64 functions of the given rows; a device that ranks float32 values of the
    same stored inputs may order blocks whose importances lie within eps = eps_rel * |k-th best|
    either way.  A row (r, j) passes when:
      * rows with row_valid False hold -1 throughout;
      * it lists kk = min(top_k, n_blk) distinct blocks in [0, n_blk), then -1;
      * every listed block's importance is at least the k-th best minus eps;
      * no unlisted block's importance exceeds the lowest listed one plus eps;
      * consecutive listed importances never rise by more than eps (descending order up to eps).
    Returns (valid rows failing, valid rows equal to the exact ranking by (importance descending,
    blk_key ascending), the first failing (row, group) pairs)."""
    import torch
    q = torch.from_numpy(np.asarray(q_rows, dtype=np.float64))          # [R, Hq, D]
    k = torch.from_numpy(np.asarray(k_cmp, dtype=np.float64))           # [n_blk, Hkv, D]
    key = torch.from_numpy(np.asarray(blk_key, dtype=np.int64))
    sel_t = torch.from_numpy(np.asarray(sel).astype(np.int64))          # [R, Hkv, top_k]
    R, Hq, _ = q.shape
    n_blk, Hkv, _ = k.shape
    G = Hq // Hkv
    if G > 1 and scale is None:
        raise ValueError("grouped score routing needs the softmax scale")
    rv = torch.ones(R, dtype=torch.bool) if row_valid is None else torch.from_numpy(np.asarray(row_valid, bool))
    top_k = sel_t.shape[2]
    kk = min(top_k, n_blk)
    n_bad, n_exact, first = 0, 0, []
    for j in range(Hkv):
        kj = k[:, j, :].T.contiguous()                                  # [D, n_blk]
        for lo in range(0, R, chunk):
            hi = min(lo + chunk, R)
            if G == 1:
                s = q[lo:hi, j, :] @ kj                                 # [c, n_blk] scores
            else:
                s = torch.zeros((hi - lo, n_blk), dtype=torch.float64)
                for h in range(j * G, (j + 1) * G):
                    z = scale * (q[lo:hi, h, :] @ kj)
                    s += torch.exp(z - torch.logsumexp(z, dim=1, keepdim=True))
            row = sel_t[lo:hi, j, :]
            v = rv[lo:hi]
            pad_ok = (row == -1).all(1)
            head = row[:, :kk]
            ok = (row[:, kk:] == -1).all(1) & ((head >= 0) & (head < n_blk)).all(1)
            hc = head.clamp(0, n_blk - 1)
            if kk > 1:
                srt = torch.sort(hc, dim=1).values
                ok &= (srt[:, 1:] != srt[:, :-1]).all(1)
            # the exact ranking: the best kk + 8 by importance, equal values ordered by blk_key
            m = min(kk + 8, n_blk)
            vals, idx = torch.topk(s, m, dim=1)
            o1 = torch.argsort(key[idx], dim=1, stable=True)
            idx1, v1 = torch.gather(idx, 1, o1), torch.gather(vals, 1, o1)
            ref = torch.gather(idx1, 1, torch.argsort(-v1, dim=1, stable=True))[:, :kk]
            kth = vals[:, kk - 1]
            # rows whose k-th value is tied beyond those m: rank the whole row
            for i in torch.nonzero((vals[:, m - 1] == kth) & (m < n_blk) & v).flatten().tolist():
                ref[i] = torch.from_numpy(np.lexsort((key.numpy(), -s[i].numpy()))[:kk])
            eps = eps_rel * kth.abs()
            ls = torch.gather(s, 1, hc)                                  # the listed blocks' values
            ok &= (ls >= (kth - eps)[:, None]).all(1)
            unl = s.scatter(1, hc, float("-inf")).max(1).values if kk < n_blk else torch.full_like(kth, -np.inf)
            ok &= unl <= ls.min(1).values + eps
            if kk > 1:
                ok &= (ls[:, 1:] <= ls[:, :-1] + eps[:, None]).all(1)
            ok = torch.where(v, ok, pad_ok)
            n_exact += int(((ref == head).all(1) & ok & v).sum())
            bad = torch.nonzero(~ok).flatten()
            n_bad += int(bad.numel())
            first += [(lo + int(i), j) for i in bad[:max(0, 8 - len(first))]]
    return n_bad, n_exact, first


def check_route_geometric(pts, blk_cnt, blk_key, cap, sel, d2, rows=None, chunk=2048):
    """Whole-table check of a geometric routing result (rows of sel / d2 for the slots `rows`,
    default every slot) against the definition of route_geometric, vectorised so that it covers
    every row of a full-size table:
      * padding rows hold -1 / 0xFFFFFFFF throughout;
      * a valid row lists kk = min(top_k, n_blk) block indices in [0, n_blk), then -1 / 0xFFFFFFFF;
      * each listed d2 is the exact integer squared distance from the token's lattice point to the
        block centroid;
      * the listed (d2, blk_key) pairs strictly ascend (so they are distinct);
      * exactly kk - 1 blocks of all n_blk have a (d2, blk_key) pair smaller than the last listed
        one, so the listed blocks are the kk smallest: the unique top-k of the total order.
    Returns the number of rows that fail (0 for a correct table) and the first failing slots."""
    import torch
    blk_cnt = np.asarray(blk_cnt)
    n_blk = blk_cnt.shape[0]
    S = n_blk * cap
    rows = np.arange(S) if rows is None else np.asarray(rows)
    sel = np.asarray(sel).astype(np.int64)
    d2 = np.asarray(d2).astype(np.int64)
    top_k = sel.shape[1]
    kk = min(top_k, n_blk)
    valid = valid_mask(blk_cnt, cap)[rows]
    cen = torch.from_numpy(block_centroids(pts, blk_cnt, cap).astype(np.int32))      # [n_blk, 3]
    u = torch.from_numpy(lattice_coords(np.asarray(pts)[rows]).astype(np.int32))      # [R, 3]
    key = torch.from_numpy(np.asarray(blk_key, dtype=np.int64))
    tsel = torch.from_numpy(sel)
    td2 = torch.from_numpy(d2)
    bad = torch.zeros(rows.shape[0], dtype=torch.bool)
    # padding rows and the tails of valid rows
    tail_ok = (tsel[:, kk:] == -1).all(1) & (td2[:, kk:] == 0xFFFFFFFF).all(1)
    pad_ok = (tsel == -1).all(1) & (td2 == 0xFFFFFFFF).all(1)
    tv = torch.from_numpy(valid)
    bad |= ~tv & ~pad_ok
    bad |= tv & ~tail_ok
    head = tsel[:, :kk]
    in_range = ((head >= 0) & (head < n_blk)).all(1)
    bad |= tv & ~in_range
    key32 = (key - (1 << 31)).to(torch.int32)          # order-preserving shift of the uint32 keys
    for lo in range(0, rows.shape[0], chunk):
        hi = min(lo + chunk, rows.shape[0])
        v = tv[lo:hi] & in_range[lo:hi]
        if not bool(v.any()):
            continue
        h = head[lo:hi].clamp(0, n_blk - 1)
        # exact squared distances to every centroid, int32 (each < 2^28)
        dall = u[lo:hi, 0:1] - cen[None, :, 0]
        dall.mul_(dall)
        for ax in (1, 2):
            t = u[lo:hi, ax:ax + 1] - cen[None, :, ax]
            dall.add_(t.mul_(t))
        listed = torch.gather(dall, 1, h).to(torch.int64)                               # exact d2 of the list
        lkey = key[h]
        ok = (listed == td2[lo:hi, :kk]).all(1)
        if kk > 1:
            ok &= ((listed[:, 1:] > listed[:, :-1]) |
                   ((listed[:, 1:] == listed[:, :-1]) & (lkey[:, 1:] > lkey[:, :-1]))).all(1)
        dk = listed[:, -1:].to(torch.int32)
        kk32 = key32[h[:, -1:]]
        better = (dall < dk) | ((dall == dk) & (key32[None, :] < kk32))
        ok &= better.sum(1) == kk - 1
        bad[lo:hi] |= v & ~ok
    nbad = int(bad.sum())
    return nbad, rows[bad.numpy()][:10]


# ----------------------------------------------------------------------------------------------
# A3: score routing against the compressed keys
# ----------------------------------------------------------------------------------------------

def route_scores(q_rows, k_cmp, blk_key, scale, top_k, lse=None, row_valid=None):
    """Top-k block selection from compressed attention scores.

    [Speed3R] 2.1 selection branch / [LSRM-cn] ("standard NSA selects KV blocks by attention score
    against the compressed keys").  q_rows [R, Hq, D], k_cmp [n_blk, Hkv, D].
      * Hq == Hkv (one query head per KV head): block b's importance for (row r, head h) is the
        compressed score <q_rh, k_cmp[b, h]> (same order as its softmax probability);
      * Hq > Hkv: importance for (row r, KV group j) is sum over the group's heads h of
        exp(scale * <q_rh, k_cmp[b, j]> - lse[r, h]), i.e. the group's summed softmax probability.
    Blocks are ranked by descending importance, ties by ascending blk_key.
    Returns sel int32 [R, Hkv, top_k] (rows where row_valid is False hold -1) and the importance of
    every block, float64 [R, Hkv, n_blk].
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k_cmp = np.asarray(k_cmp, dtype=np.float64)
    blk_key = np.asarray(blk_key, dtype=np.int64)
    R, Hq, D = q_rows.shape
    n_blk, Hkv, _ = k_cmp.shape
    G = Hq // Hkv
    if G > 1 and lse is None:
        raise ValueError("grouped score routing needs the compressed branch's lse")
    kk = min(top_k, n_blk)
    sel = np.full((R, Hkv, top_k), -1, dtype=np.int32)
    imp_all = np.zeros((R, Hkv, n_blk))
    for r in range(R):
        if row_valid is not None and not row_valid[r]:
            continue
        for j in range(Hkv):
            if G == 1:
                imp = k_cmp[:, j, :] @ q_rows[r, j]
            else:
                imp = np.zeros(n_blk)
                for h in range(j * G, (j + 1) * G):
                    imp += np.exp(scale * (k_cmp[:, j, :] @ q_rows[r, h]) - lse[r, h])
            imp_all[r, j] = imp
            order = np.lexsort((blk_key, -imp))[:kk]
            sel[r, j, :kk] = order
    return sel, imp_all


# ----------------------------------------------------------------------------------------------
# A4-A6: the three attention branches
# ----------------------------------------------------------------------------------------------

def attn_branch(branch, q, k, v, blk_cnt, cap, scale, sel=None, q_gran="token", rows=None, forced=None):
    """One NSA branch for the query rows `rows` (storage slots; default all).

    branch CMP ([LSRM-cn] compressed branch; [Speed3R] compression branch): keys/values are the
      pooled arrays k, v [n_blk, Hkv, D].  q_gran 'token': every valid token's own query attends all
      blocks.  q_gran 'block': q is pooled [n_blk, Hq, D]; block b's pooled query attends all blocks
      and its output is given to each valid token of block b.
    branch LOC ([LSRM-cn] window attention): the valid tokens of the query's own block.
    branch SEL ([LSRM-cn] selected blocks; [Speed3R] selection branch): the valid tokens of the
      blocks listed in sel (a set; -1 entries skipped), together with the blocks of the range
      forced = (lo, hi) when given ([Speed3R] 2.2, VGGT variant: the reference frame is always
      attended).  sel is [S, top_k] (one list per token,
      shared by all heads), [S, Hkv, top_k] (one list per token and KV group), or with q_gran
      'block' [n_blk, top_k] / [n_blk, Hkv, top_k] (one list per query block).
    Returns o [len(rows), Hq, D] and lse [len(rows), Hq] (padding rows: 0 and -inf).
    """
    blk_cnt = np.asarray(blk_cnt)
    n_blk = blk_cnt.shape[0]
    S = n_blk * cap
    rows = np.arange(S) if rows is None else np.asarray(rows)
    valid = valid_mask(blk_cnt, cap)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = np.zeros((rows.shape[0], Hq, D))
    lse = np.full((rows.shape[0], Hq), -np.inf)
    cache = {}
    for i, r in enumerate(rows):
        if not valid[r]:
            continue
        b = r // cap
        if branch == CMP:
            if q_gran == "block":
                if b not in cache:
                    cache[b] = attend(q[b], k, v, scale)
                o[i], lse[i] = cache[b]
            else:
                o[i], lse[i] = attend(q[r], k, v, scale)
        elif branch == LOC:
            ks = block_slots(blk_cnt, cap, b)
            o[i], lse[i] = attend(q[r], k[ks], v[ks], scale)
        elif branch == SEL:
            lst = sel[b] if q_gran == "block" else sel[r]
            lst = np.asarray(lst)
            always = set(range(forced[0], forced[1])) if forced is not None else set()
            if lst.ndim == 1:
                blocks = sorted(set(int(x) for x in lst if x >= 0) | always)
                ks = np.concatenate([block_slots(blk_cnt, cap, x) for x in blocks]) if blocks else np.zeros(0, int)
                o[i], lse[i] = attend(q[r], k[ks], v[ks], scale)
            else:
                for j in range(Hkv):
                    blocks = sorted(set(int(x) for x in lst[j] if x >= 0) | always)
                    ks = np.concatenate([block_slots(blk_cnt, cap, x) for x in blocks]) if blocks else np.zeros(0, int)
                    hs = slice(j * G, (j + 1) * G)
                    oj, lj = attend(q[r, hs], k[ks][:, j:j + 1], v[ks][:, j:j + 1], scale)
                    o[i, hs], lse[i, hs] = oj, lj
        else:
            raise ValueError(branch)
    return o, lse


# ----------------------------------------------------------------------------------------------
# A7: gate
# ----------------------------------------------------------------------------------------------

def gate_combine(outs, gate_logits):
    """o = sum_c sigmoid(g_c) * o_c per (row, query head): [LSRM-cn] Sigmoid gates; [Speed3R] 2.1
    gated aggregation of the branch outputs.  outs: list of [R, Hq, D]; gate_logits [R, Hq, n]."""
    g = sigmoid(np.asarray(gate_logits, dtype=np.float64))
    o = np.zeros(np.asarray(outs[0]).shape)
    for c, oc in enumerate(outs):
        o += g[:, :, c:c + 1] * np.asarray(oc, dtype=np.float64)
    return o


# ----------------------------------------------------------------------------------------------
# A8: stage-1 dense gated self/cross attention
# ----------------------------------------------------------------------------------------------

def dense_gated_xattn(q, k, v, n_x, gate_logits, scale, rows=None):
    """[LSRM-cn] eq. o^x = w^{x-self} CrossAttn(x, x) + w^{x-cross} CrossAttn(x, y) and the same for
    y: tokens [0, n_x) are volume tokens x, the rest image tokens y.  One q, k, v per token serves
    both terms; gate channel 0 is the self gate, channel 1 the cross gate.  An empty key set adds 0."""
    N = q.shape[0]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    g = sigmoid(np.asarray(gate_logits, dtype=np.float64))
    xs = np.arange(0, n_x)
    ys = np.arange(n_x, N)
    o = np.zeros((rows.shape[0], q.shape[1], q.shape[2]))
    for i, t in enumerate(rows):
        own, other = (xs, ys) if t < n_x else (ys, xs)
        o_self, _ = attend(q[t], k[own], v[own], scale)
        o_cross, _ = attend(q[t], k[other], v[other], scale)
        o[i] = g[t, :, 0:1] * o_self + g[t, :, 1:2] * o_cross
    return o


# ----------------------------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------------------------

def nsa_forward(w, rows=None, return_parts=False, forced=None):
    """One NSA layer on a block-major workload `w` (see workloads.Workload):
    compress K and V (and Q for block-granular queries), route, run the branches listed in
    w.branches and combine them with the sigmoid gates (channel c = c-th listed branch).
    Geometric routing ([LSRM-cn]) is per token and shared by all heads; score routing ([Speed3R])
    with one query head per KV head is per (query block, head) from the pooled queries; score
    routing with several query heads per KV head is per (token, KV group) from the summed group
    probabilities, with the compressed branch's lse, or per (query block, KV group) from the pooled
    queries when w.q_gran is 'block'."""
    cap = w.blk_cap
    S = w.n_slots
    rows = np.arange(S) if rows is None else np.asarray(rows)
    k_cmp = pool_blocks(w.k, w.blk_cnt, cap)
    v_cmp = pool_blocks(w.v, w.blk_cnt, cap)
    parts = {"k_cmp": k_cmp, "v_cmp": v_cmp}
    if w.q_gran == "block":
        q_cmp = pool_blocks(w.q, w.blk_cnt, cap)
        parts["q_cmp"] = q_cmp
    if w.routing == "geometric":
        sel_rows, _ = route_geometric(w.pts, w.blk_cnt, w.blk_key, cap, w.top_k, rows=rows)
        sel = np.full((S, w.top_k), -1, dtype=np.int32)
        sel[rows] = sel_rows
        q_gran_sel = "token"
    elif w.n_qh == w.n_kvh:
        # [Speed3R] 2.1: routing rows are per query block, from the pooled queries; only the blocks
        # holding the requested rows are needed
        need = np.unique(rows // cap)
        sel = np.full((w.n_blk, w.n_kvh, w.top_k), -1, dtype=np.int32)
        sel[need], _ = route_scores(parts["q_cmp"][need], k_cmp, w.blk_key, w.scale, w.top_k)
        q_gran_sel = "block"
    elif w.q_gran == "block":
        # grouped-query score routing with pooled query rows: per (query block, KV group), the blocks
        # with the largest summed softmax probability of the group's heads for the block's pooled
        # query, normalised by that pooled row's compressed-branch lse
        need = np.unique(rows // cap)
        lse_b = np.stack([attend(parts["q_cmp"][b], k_cmp, v_cmp, w.scale)[1] for b in need])
        sel = np.full((w.n_blk, w.n_kvh, w.top_k), -1, dtype=np.int32)
        sel[need], _ = route_scores(parts["q_cmp"][need], k_cmp, w.blk_key, w.scale, w.top_k, lse=lse_b)
        q_gran_sel = "block"
    else:
        # [LSRM-cn] "standard NSA" selection under grouped-query attention: per token and KV group,
        # the blocks with the largest summed softmax probability of the group's heads against the
        # compressed keys; the normalisers are the compressed branch's lse for the same rows
        _, lse_rows = attn_branch(CMP, w.q, k_cmp, v_cmp, w.blk_cnt, cap, w.scale, rows=rows)
        ok = valid_mask(w.blk_cnt, cap)[rows]
        sel = np.full((S, w.n_kvh, w.top_k), -1, dtype=np.int32)
        sel[rows], _ = route_scores(w.q[rows], k_cmp, w.blk_key, w.scale, w.top_k, lse=lse_rows, row_valid=ok)
        q_gran_sel = "token"
    parts["sel"] = sel
    outs = []
    for name in w.branches:
        br = BRANCH_NAMES[name]
        if br == CMP:
            if w.q_gran == "block":
                oc, lc = attn_branch(CMP, parts["q_cmp"], k_cmp, v_cmp, w.blk_cnt, cap, w.scale,
                                     q_gran="block", rows=rows)
            else:
                oc, lc = attn_branch(CMP, w.q, k_cmp, v_cmp, w.blk_cnt, cap, w.scale, rows=rows)
        elif br == SEL:
            oc, lc = attn_branch(SEL, w.q, w.k, w.v, w.blk_cnt, cap, w.scale, sel=sel,
                                 q_gran=q_gran_sel, rows=rows, forced=forced)
        else:
            oc, lc = attn_branch(LOC, w.q, w.k, w.v, w.blk_cnt, cap, w.scale, rows=rows)
        parts["o_" + name] = oc
        parts["lse_" + name] = lc
        outs.append(oc)
    o = gate_combine(outs, w.gates[rows])
    o[~valid_mask(w.blk_cnt, cap)[rows]] = 0.0
    return (o, parts) if return_parts else o


# ----------------------------------------------------------------------------------------------
# routing with image blocks found through the views
# ----------------------------------------------------------------------------------------------

def project_coord(p, proj_row):
    """Continuous patch coordinate of point p along one image axis of a view: the affine map
    A0 p0 + A1 p1 + A2 p2 + A3 (an orthographic camera), in float64 on the given float32 values."""
    a = np.asarray(proj_row, dtype=np.float64)
    x = np.asarray(p, dtype=np.float64)
    return float(a[0] * x[0] + a[1] * x[1] + a[2] * x[2] + a[3])


def project_cell(p, proj_row, cell):
    """Cell coordinate of point p along one image axis: floor(patch coordinate / cell size)."""
    return int(math.floor(project_coord(p, proj_row) / cell))  # cells far outside the grid give empty windows


def route_geometric_views(pts, blk_cnt, blk_key, cap, top_k, n_vol_blk, view_proj, cell_blk, cell, radius,
                          rows=None):
    """3D-aware routing with the image-block rule of [LSRM-cn] (routing paragraph): the query point is
    projected into every view, the image blocks of the cells within `radius` cells of the projection
    are that view's candidates, and an image candidate's metric is the smallest squared distance
    between the query and any of its tokens' points.  Volume blocks [0, n_vol_blk) keep the
    block-centre metric (d2 to the centroid).  Both on the 2^-12 lattice, exact integers; one
    ranking over all candidates in ascending (d2, blk_key) order, top_k, best first.
    view_proj [V, 2, 4] float32 maps a point to continuous patch coordinates (project_cell);
    cell_blk [V, n_cell, n_cell] int32 is the block of each (view, cell row, cell column) or -1.
    Returns sel int32 [len(rows), top_k] and d2 uint32 (padding rows and missing ranks: -1 /
    0xFFFFFFFF)."""
    blk_cnt = np.asarray(blk_cnt)
    blk_key = np.asarray(blk_key, dtype=np.int64)
    S = blk_cnt.shape[0] * cap
    rows = np.arange(S) if rows is None else np.asarray(rows)
    valid = valid_mask(blk_cnt, cap)
    cen = block_centroids(pts, blk_cnt, cap)
    u = lattice_coords(pts)
    V, nc = cell_blk.shape[0], cell_blk.shape[1]
    sel = np.full((rows.shape[0], top_k), -1, dtype=np.int32)
    dd = np.full((rows.shape[0], top_k), 0xFFFFFFFF, dtype=np.uint32)
    vol = np.arange(n_vol_blk)
    for i, r in enumerate(rows):
        if not valid[r]:
            continue
        cand = list(vol)
        metric = list(((u[r][None, :] - cen[vol]) ** 2).sum(axis=1)) if n_vol_blk else []
        for v in range(V):
            cx = project_cell(pts[r], view_proj[v, 0], cell)
            cy = project_cell(pts[r], view_proj[v, 1], cell)
            for y in range(max(cy - radius, 0), min(cy + radius, nc - 1) + 1):
                for x in range(max(cx - radius, 0), min(cx + radius, nc - 1) + 1):
                    b = int(cell_blk[v, y, x])
                    if b < 0:
                        continue
                    members = u[block_slots(blk_cnt, cap, b)]
                    cand.append(b)
                    metric.append(int(((members - u[r][None, :]) ** 2).sum(axis=1).min()))
        cand = np.asarray(cand, dtype=np.int64)
        metric = np.asarray(metric, dtype=np.int64)
        kk = min(top_k, cand.shape[0])
        order = np.lexsort((blk_key[cand], metric))[:kk]
        sel[i, :kk] = cand[order]
        dd[i, :kk] = metric[order]
    return sel, dd


# ----------------------------------------------------------------------------------------------
# split self/cross NSA: stage 2 keeping stage 1's decoupled branches
# ----------------------------------------------------------------------------------------------

def route_geometric_range(pts, blk_cnt, blk_key, cap, top_k, q_blocks, kv_blocks):
    """Geometric routing (the metric and order of route_geometric) for the query slots of the
    blocks [q_lo, q_hi) with the candidates restricted to the blocks [kv_lo, kv_hi).
    Returns sel int32 and d2 uint32 [(q_hi - q_lo) * cap, top_k] (storage block indices, best
    first); padding rows and positions beyond the candidate count hold -1 / 0xFFFFFFFF."""
    blk_cnt = np.asarray(blk_cnt)
    blk_key = np.asarray(blk_key, dtype=np.int64)
    q_lo, q_hi = q_blocks
    kv_lo, kv_hi = kv_blocks
    valid = valid_mask(blk_cnt, cap)
    cen = block_centroids(pts, blk_cnt, cap)
    u = lattice_coords(pts)
    cand = np.arange(kv_lo, kv_hi)
    rows = np.arange(q_lo * cap, q_hi * cap)
    sel = np.full((rows.shape[0], top_k), -1, dtype=np.int32)
    dd = np.full((rows.shape[0], top_k), 0xFFFFFFFF, dtype=np.uint32)
    kk = min(top_k, cand.shape[0])
    for i, r in enumerate(rows):
        if not valid[r] or kk == 0:
            continue
        d2 = ((u[r][None, :] - cen[cand]) ** 2).sum(axis=1)
        order = np.lexsort((blk_key[cand], d2))[:kk]
        sel[i, :kk] = cand[order]
        dd[i, :kk] = d2[order]
    return sel, dd


def _keys_of_blocks(blk_cnt, cap, blocks):
    blocks = sorted(set(int(x) for x in blocks if x >= 0))
    if not blocks:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([block_slots(blk_cnt, cap, x) for x in blocks])


def nsa_split_forward(w, n_x_blk, gates, rows=None, return_parts=False):
    """Stage-2 NSA that keeps stage 1's decoupled self and cross branches ([LSRM-cn] eq. o^x, o^y
    with Sigmoid gates, each dense attention replaced by NSA over the blocks of one token type).
    Blocks [0, n_x_blk) hold volume tokens x, blocks [n_x_blk, n_blk) image tokens y.  For a token
    whose own block lies in subset A (its type) with B the other subset:
        o = s(g0) NSA_A + s(g1) NSA_B,   s = sigmoid,
        NSA_A = s(g2) CMP_A + s(g3) SEL_A + s(g4) LOC,
        NSA_B = s(g5) CMP_B + s(g6) SEL_B,
    CMP_X attends the pooled blocks of X, SEL_X the valid tokens of the top-k blocks of X by
    geometric routing (route_geometric_range), LOC the valid tokens of the own block.  gates is
    [S, Hq, 7] in that channel order.  An empty subset contributes 0.  Returns o [len(rows), Hq, D]."""
    cap = w.blk_cap
    S = w.n_slots
    n_blk = w.n_blk
    rows = np.arange(S) if rows is None else np.asarray(rows)
    valid = valid_mask(w.blk_cnt, cap)
    k_cmp = pool_blocks(w.k, w.blk_cnt, cap)
    v_cmp = pool_blocks(w.v, w.blk_cnt, cap)
    g = sigmoid(np.asarray(gates, dtype=np.float64))
    ranges = ((0, n_x_blk), (n_x_blk, n_blk))
    sel_self = np.full((S, w.top_k), -1, dtype=np.int32)
    sel_cross = np.full((S, w.top_k), -1, dtype=np.int32)
    need = np.unique(rows // cap)
    for qi, qr in enumerate(ranges):
        blocks_here = need[(need >= qr[0]) & (need < qr[1])]
        for b in blocks_here:
            sl = slice(b * cap, (b + 1) * cap)
            sel_self[sl], _ = route_geometric_range(w.pts, w.blk_cnt, w.blk_key, cap, w.top_k, (b, b + 1), qr)
            sel_cross[sl], _ = route_geometric_range(w.pts, w.blk_cnt, w.blk_key, cap, w.top_k, (b, b + 1),
                                                     ranges[1 - qi])
    Hq, D = w.q.shape[1], w.q.shape[2]
    o = np.zeros((rows.shape[0], Hq, D))
    for i, r in enumerate(rows):
        if not valid[r]:
            continue
        b = r // cap
        own, other = (ranges[0], ranges[1]) if b < n_x_blk else (ranges[1], ranges[0])
        cmp_a, _ = attend(w.q[r], k_cmp[own[0]:own[1]], v_cmp[own[0]:own[1]], w.scale)
        cmp_b, _ = attend(w.q[r], k_cmp[other[0]:other[1]], v_cmp[other[0]:other[1]], w.scale)
        ks = _keys_of_blocks(w.blk_cnt, cap, sel_self[r])
        sel_a, _ = attend(w.q[r], w.k[ks], w.v[ks], w.scale)
        ks = _keys_of_blocks(w.blk_cnt, cap, sel_cross[r])
        sel_b, _ = attend(w.q[r], w.k[ks], w.v[ks], w.scale)
        ks = block_slots(w.blk_cnt, cap, b)
        loc, _ = attend(w.q[r], w.k[ks], w.v[ks], w.scale)
        gr = g[r][:, :, None]
        nsa_a = gr[:, 2] * cmp_a + gr[:, 3] * sel_a + gr[:, 4] * loc
        nsa_b = gr[:, 5] * cmp_b + gr[:, 6] * sel_b
        o[i] = gr[:, 0] * nsa_a + gr[:, 1] * nsa_b
    if return_parts:
        return o, {"k_cmp": k_cmp, "v_cmp": v_cmp, "sel_self": sel_self, "sel_cross": sel_cross}
    return o
