"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each test checks the oracle against something independent: a hand-worked fixture, a closed form,
a textbook library routine (torch's scaled-dot-product attention in float64 on the CPU), brute
force on tiny inputs, or an invariant of the definition (row sums, storage-order invariance).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa(q, k, v, scale):
    """Library attention: q [n, Hq, D], k/v [m, Hkv, D] -> [n, Hq, D] (torch, float64, CPU)."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    tq = torch.from_numpy(np.asarray(q, dtype=np.float64)).permute(1, 0, 2)
    tk = torch.from_numpy(np.asarray(k, dtype=np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)
    tv = torch.from_numpy(np.asarray(v, dtype=np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    return o.permute(1, 0, 2).numpy()


def small(seed=1, cnt=(5, 8, 1, 3, 8, 6), cap=8, Hq=4, Hkv=2, D=8, top_k=3, dtype="f32"):
    return W.custom_block_workload(seed, list(cnt), cap, Hq, Hkv, D, dtype, top_k)


# ---------------------------------------------------------------------------------------------
# hand-worked fixtures
# ---------------------------------------------------------------------------------------------

def test_attend_hand_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "attend_hand.json")))
    o, lse, wts = O.attend(np.array(fx["q"]), np.array(fx["k"]), np.array(fx["v"]), fx["scale"],
                           return_weights=True)
    np.testing.assert_allclose(o, fx["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, fx["lse"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(wts, fx["weights"], rtol=0, atol=1e-15)


def test_route_hand_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "route_hand.json")))
    for case in fx["cases"]:
        sel, d2 = O.route_geometric(np.array(case["pts"], dtype=np.float32), np.array(case["blk_cnt"]),
                                    np.array(case["blk_key"], dtype=np.uint32), case["cap"], case["top_k"])
        assert sel.tolist() == case["sel"], case["name"]
        assert d2.tolist() == case["d2"], case["name"]


def test_sigmoid_closed_forms():
    g = O.sigmoid(np.array([0.0, math.log(3.0), -math.log(3.0), np.inf, -np.inf, 800.0, -800.0]))
    np.testing.assert_allclose(g, [0.5, 0.75, 0.25, 1.0, 0.0, 1.0, 0.0], rtol=0, atol=1e-15)
    assert g[3] == 1.0 and g[4] == 0.0


# ---------------------------------------------------------------------------------------------
# attention branches against library attention
# ---------------------------------------------------------------------------------------------

def test_attend_matches_library_and_rows_sum_to_one():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((6, 8))
    k = rng.standard_normal((11, 2, 8))
    v = rng.standard_normal((11, 2, 8))
    o, lse, wts = O.attend(q, k, v, 0.3, return_weights=True)
    ref = sdpa(q[None], k, v, 0.3)[0]
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(wts.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    assert (wts >= 0).all()
    # lse is the log of the partition function
    G = 3
    for h in range(6):
        s = 0.3 * k[:, h // G, :] @ q[h]
        assert abs(lse[h] - math.log(np.exp(s).sum())) < 1e-12


@pytest.mark.parametrize("name", ["tiny", "custom"])
def test_dense_equivalence(name):
    """top_k = n_blk with only the selected branch gated on reproduces dense attention."""
    w = W.make("tiny") if name == "tiny" else small()
    w.top_k = w.n_blk
    w.gates = np.zeros_like(w.gates)
    w.gates[..., 0] = -np.inf
    w.gates[..., 1] = np.inf
    w.gates[..., 2] = -np.inf
    o = O.nsa_forward(w)
    vs = w.valid_slots()
    ref = sdpa(w.q[vs], w.k[vs], w.v[vs], w.scale)
    np.testing.assert_allclose(o[vs], ref, rtol=0, atol=1e-12)
    assert np.all(o[~w.valid_mask()] == 0)


def test_local_branch_is_blockwise_attention():
    w = small(seed=3)
    o, lse = O.attn_branch(O.LOC, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale)
    for b in range(w.n_blk):
        s = O.block_slots(w.blk_cnt, w.blk_cap, b)
        np.testing.assert_allclose(o[s], sdpa(w.q[s], w.k[s], w.v[s], w.scale), rtol=0, atol=1e-13)


def test_compressed_branch_against_library_pooling():
    w = small(seed=4)
    kc = O.pool_blocks(w.k, w.blk_cnt, w.blk_cap)
    vc = O.pool_blocks(w.v, w.blk_cnt, w.blk_cap)
    # pooling against a scatter-mean from torch
    vs = w.valid_slots()
    seg = torch.from_numpy(vs // w.blk_cap)
    for x, xc in ((w.k, kc), (w.v, vc)):
        acc = torch.zeros((w.n_blk,) + x.shape[1:], dtype=torch.float64)
        acc.index_add_(0, seg, torch.from_numpy(x[vs].astype(np.float64)))
        cnt = torch.bincount(seg, minlength=w.n_blk).to(torch.float64)
        np.testing.assert_allclose(xc, (acc / cnt[:, None, None]).numpy(), rtol=0, atol=1e-14)
    o, _ = O.attn_branch(O.CMP, w.q, kc, vc, w.blk_cnt, w.blk_cap, w.scale)
    np.testing.assert_allclose(o[vs], sdpa(w.q[vs], kc, vc, w.scale), rtol=0, atol=1e-13)


def test_selected_branch_per_group_lists():
    """Per-KV-group selection lists: each group attends exactly its own blocks."""
    w = small(seed=5)
    rng = np.random.default_rng(9)
    S = w.n_slots
    sel = np.full((S, 2, 3), -1, dtype=np.int32)
    for r in range(S):
        for j in range(2):
            sel[r, j, :2] = rng.choice(w.n_blk, 2, replace=False)
    o, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel)
    for r in w.valid_slots()[:10]:
        for j in range(2):
            ks = np.concatenate([O.block_slots(w.blk_cnt, w.blk_cap, b) for b in sorted(sel[r, j, :2])])
            ref = sdpa(w.q[r:r + 1, 2 * j:2 * j + 2], w.k[ks][:, j:j + 1], w.v[ks][:, j:j + 1], w.scale)
            np.testing.assert_allclose(o[r, 2 * j:2 * j + 2], ref[0], rtol=0, atol=1e-13)


def test_single_block_closed_forms():
    w = small(seed=6, cnt=(7,), top_k=1)
    vs = w.valid_slots()
    kc = O.pool_blocks(w.k, w.blk_cnt, w.blk_cap)
    vc = O.pool_blocks(w.v, w.blk_cnt, w.blk_cap)
    o_cmp, _ = O.attn_branch(O.CMP, w.q, kc, vc, w.blk_cnt, w.blk_cap, w.scale)
    # a one-key softmax has weight 1: the compressed branch returns the block mean of v
    for r in vs:
        np.testing.assert_allclose(o_cmp[r], np.repeat(w.v[vs].astype(np.float64).mean(0), 2, axis=0),
                                   rtol=0, atol=1e-14)
    sel = np.zeros((w.n_slots, 1), dtype=np.int32)
    o_sel, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel)
    o_loc, _ = O.attn_branch(O.LOC, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale)
    ref = sdpa(w.q[vs], w.k[vs], w.v[vs], w.scale)
    np.testing.assert_allclose(o_sel[vs], ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(o_loc[vs], ref, rtol=0, atol=1e-13)


def test_constant_values_closed_form():
    w = small(seed=7)
    w.v[:] = 0.0
    vs = w.valid_slots()
    w.v[vs] = np.array([0.5, -1.25, 2.0, 0.0, 3.5, -0.75, 1.0, 4.0], dtype=np.float32)
    o = O.nsa_forward(w)
    gsum = O.sigmoid(w.gates[vs]).sum(axis=2)          # [n, Hq]
    ref = gsum[:, :, None] * w.v[vs][:, :1, :].astype(np.float64)
    np.testing.assert_allclose(o[vs], ref, rtol=0, atol=1e-13)


def test_gate_combine_selects_single_branch():
    rng = np.random.default_rng(1)
    outs = [rng.standard_normal((5, 4, 3)) for _ in range(3)]
    for c in range(3):
        g = np.full((5, 4, 3), -np.inf)
        g[..., c] = np.inf
        np.testing.assert_array_equal(O.gate_combine(outs, g), outs[c])
    g = np.zeros((5, 4, 3))
    np.testing.assert_allclose(O.gate_combine(outs, g), 0.5 * (outs[0] + outs[1] + outs[2]), atol=1e-15)


# ---------------------------------------------------------------------------------------------
# storage-order invariance of the whole layer
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1])
def test_storage_permutation_invariance(seed):
    w = W.make("tiny") if seed == 0 else small(seed=11)
    o1, p1 = O.nsa_forward(w, return_parts=True)
    w2, smap = W.permute_storage(w, seed=100 + seed)
    o2, p2 = O.nsa_forward(w2, return_parts=True)
    new = np.nonzero(smap >= 0)[0]
    np.testing.assert_allclose(o2[new], o1[smap[new]], rtol=0, atol=1e-12)
    # routed blocks, named by blk_key, are identical
    keys1 = np.where(p1["sel"] >= 0, w.blk_key[p1["sel"]], 0)
    keys2 = np.where(p2["sel"] >= 0, w2.blk_key[p2["sel"]], 0)
    np.testing.assert_array_equal(keys2[new], keys1[smap[new]])


# ---------------------------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------------------------

def brute_route(pts, blk_cnt, blk_key, cap, k):
    """Pure-Python brute force over real-valued points: quantise, average, sort tuples."""
    n_blk = len(blk_cnt)
    members = [[b * cap + i for i in range(blk_cnt[b])] for b in range(n_blk)]
    lat = lambda x: int(round(4096 * float(x))) + 4096  # noqa: E731  (exact: 4096*x is a float64)
    cents = []
    for b in range(n_blk):
        c = []
        for ax in range(3):
            tot = sum(lat(pts[s][ax]) for s in members[b])
            n = blk_cnt[b]
            c.append((2 * tot + n) // (2 * n))
        cents.append(c)
    out = {}
    for b in range(n_blk):
        for s in members[b]:
            u = [lat(pts[s][ax]) for ax in range(3)]
            cand = sorted((sum((u[a] - cents[c][a]) ** 2 for a in range(3)), int(blk_key[c]), c)
                          for c in range(n_blk))
            out[s] = [c for _, _, c in cand[:k]]
    return out


@pytest.mark.parametrize("mode", ["random", "lattice"])
def test_geometric_routing_brute_force(mode):
    if mode == "random":
        w = W.custom_block_workload(21, [5, 8, 1, 3, 8, 6, 2, 7, 8], 8, 4, 2, 8, "f32", 4, pts_mode=mode)
    else:
        # one token per block on a coarse lattice: centroids coincide with lattice points
        w = W.custom_block_workload(21, [1] * 40, 1, 4, 2, 8, "f32", 6, pts_mode=mode)
    sel, d2 = O.route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k)
    ref = brute_route(w.pts.tolist(), w.blk_cnt.tolist(), w.blk_key, w.blk_cap, w.top_k)
    for s in range(w.n_slots):
        if s in ref:
            assert sel[s].tolist() == ref[s]
        else:
            assert (sel[s] == -1).all()
    if mode == "lattice":
        # the lattice inputs do create exact distance ties among the top candidates
        assert any(len(set(row[:4].tolist())) < 4 for row in d2[w.valid_mask()])


def test_geometric_routing_own_block_first_in_full_grid():
    """In a full voxel grid partitioned into 4^3 cells the centroids form a cubic lattice, so every
    voxel's nearest centroid is its own cell's (Voronoi cell of a cubic lattice)."""
    side = 16
    g = np.arange(side)
    zz, yy, xx = np.meshgrid(g, g, g, indexing="ij")
    vox = np.stack([xx.ravel(), yy.ravel(), zz.ravel()], axis=1)
    cell = W.morton3(vox[:, 0] // 4, vox[:, 1] // 4, vox[:, 2] // 4)
    order = np.lexsort((W.morton3(vox[:, 0], vox[:, 1], vox[:, 2]), cell))
    pts = (-1.0 + (2.0 * vox[order] + 1.0) / side).astype(np.float32)
    n_blk = (side // 4) ** 3
    blk_cnt = np.full(n_blk, 64, dtype=np.int32)
    blk_key = np.arange(n_blk, dtype=np.uint32)
    sel, d2 = O.route_geometric(pts, blk_cnt, blk_key, 64, 1)
    np.testing.assert_array_equal(sel[:, 0], np.arange(n_blk * 64) // 64)


def test_geometric_routing_k_beyond_blocks():
    w = small(seed=8)
    sel, d2 = O.route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.n_blk + 3)
    vm = w.valid_mask()
    assert (sel[vm][:, w.n_blk:] == -1).all()
    assert (d2[vm][:, w.n_blk:] == 0xFFFFFFFF).all()
    for row in sel[vm]:
        assert sorted(row[:w.n_blk].tolist()) == list(range(w.n_blk))


def test_score_routing_exact_on_integer_inputs():
    """One query head per KV head: integer-valued inputs make every score exact; compare with a
    pure-Python sort of (-score, key)."""
    rng = np.random.default_rng(3)
    R, H, D, n_blk, k = 7, 3, 4, 12, 5
    q = rng.integers(-3, 4, size=(R, H, D)).astype(np.float64)
    kc = rng.integers(-3, 4, size=(n_blk, H, D)).astype(np.float64)
    key = rng.permutation(n_blk).astype(np.uint32) + 100
    sel, imp = O.route_scores(q, kc, key, 0.5, k)
    for r in range(R):
        for h in range(H):
            sc = [(-int(sum(q[r, h, d] * kc[b, h, d] for d in range(D))), int(key[b]), b) for b in range(n_blk)]
            assert sel[r, h].tolist() == [b for _, _, b in sorted(sc)[:k]]


def test_grouped_score_routing_importance_sums_to_group_size():
    """With lse from the compressed branch, each head's probabilities over all blocks sum to one, so a
    group's summed importance over all blocks equals the group size."""
    w = small(seed=12)
    kc = O.pool_blocks(w.k, w.blk_cnt, w.blk_cap)
    vc = O.pool_blocks(w.v, w.blk_cnt, w.blk_cap)
    vs = w.valid_slots()
    _, lse = O.attn_branch(O.CMP, w.q, kc, vc, w.blk_cnt, w.blk_cap, w.scale, rows=vs)
    sel, imp = O.route_scores(w.q[vs], kc, w.blk_key, w.scale, 3, lse=lse)
    np.testing.assert_allclose(imp.sum(axis=2), 2.0, rtol=0, atol=1e-12)
    # the selection holds the largest importances
    for r in range(len(vs)):
        for j in range(2):
            kth = np.sort(imp[r, j])[::-1][2]
            assert (imp[r, j, sel[r, j]] >= kth).all()


# ---------------------------------------------------------------------------------------------
# stage-1 dense gated self/cross attention
# ---------------------------------------------------------------------------------------------

def test_dense_gated_reduces_to_library_attention():
    w = W.make("dense_small", dtype="f32")
    N, nx = w.n_tok, w.n_x
    rows = np.array([0, 1, nx - 1, nx, nx + 5, N - 1])
    g = np.zeros_like(w.gates)
    g[..., 0], g[..., 1] = np.inf, -np.inf
    o = O.dense_gated_xattn(w.q, w.k, w.v, nx, g, w.scale, rows=rows)
    for i, t in enumerate(rows):
        own = slice(0, nx) if t < nx else slice(nx, N)
        np.testing.assert_allclose(o[i], sdpa(w.q[t:t + 1], w.k[own], w.v[own], w.scale)[0], atol=1e-13)
    g[..., 0], g[..., 1] = -np.inf, np.inf
    o = O.dense_gated_xattn(w.q, w.k, w.v, nx, g, w.scale, rows=rows)
    for i, t in enumerate(rows):
        oth = slice(nx, N) if t < nx else slice(0, nx)
        np.testing.assert_allclose(o[i], sdpa(w.q[t:t + 1], w.k[oth], w.v[oth], w.scale)[0], atol=1e-13)
    # all tokens of one type: the cross term is empty and contributes nothing
    g = w.gates.copy()
    o = O.dense_gated_xattn(w.q, w.k, w.v, N, g, w.scale, rows=rows)
    ref = O.sigmoid(g[rows][..., 0:1]) * sdpa(w.q[rows], w.k, w.v, w.scale)
    np.testing.assert_allclose(o, ref, atol=1e-13)


def test_dense_gated_swap_symmetry():
    w = W.make("dense_small", dtype="f32")
    N, nx = w.n_tok, w.n_x
    perm = np.concatenate([np.arange(nx, N), np.arange(0, nx)])     # image tokens first
    rows = np.array([0, 7, nx, N - 1])
    o1 = O.dense_gated_xattn(w.q, w.k, w.v, nx, w.gates, w.scale, rows=rows)
    inv = np.argsort(perm)
    o2 = O.dense_gated_xattn(w.q[perm], w.k[perm], w.v[perm], N - nx, w.gates[perm], w.scale,
                             rows=inv[rows])
    np.testing.assert_allclose(o2, o1, atol=1e-13)


# ---------------------------------------------------------------------------------------------
# pooling
# ---------------------------------------------------------------------------------------------

def test_pool_identity_linearity_constant():
    rng = np.random.default_rng(2)
    cnt = np.array([1, 4, 2, 1])
    x = rng.standard_normal((16, 3, 5))
    y = rng.standard_normal((16, 3, 5))
    p = O.pool_blocks(x, cnt, 4)
    np.testing.assert_array_equal(p[0], x[0])
    np.testing.assert_array_equal(p[3], x[12])
    np.testing.assert_allclose(O.pool_blocks(2 * x - 3 * y, cnt, 4), 2 * p - 3 * O.pool_blocks(y, cnt, 4),
                               atol=1e-14)
    c = np.full((16, 3, 5), 1.75)
    np.testing.assert_array_equal(O.pool_blocks(c, cnt, 4), np.full((4, 3, 5), 1.75))


def test_resblock_pool_reduces_and_closed_forms():
    """Pins of the residual module before pooling: zero weights give the plain block mean; a bias
    b2 alone shifts every pooled row by b2; with W1 = W2 = I and zero biases a single-token block
    gives x + silu(x) elementwise, silu written out as x / (1 + e^-x) (checked at a few points
    against its closed values silu(0) = 0 and silu(ln 3) = 0.75 ln 3)."""
    rng = np.random.default_rng(21)
    cnt = np.array([1, 3, 4, 2])
    H, D = 2, 3
    x = rng.standard_normal((16, H, D))
    z = np.zeros((H, D, D))
    zb = np.zeros((H, D))
    np.testing.assert_allclose(O.pool_blocks_resblock(x, cnt, 4, z, zb, z, zb), O.pool_blocks(x, cnt, 4),
                               atol=1e-15)
    b2 = rng.standard_normal((H, D))
    np.testing.assert_allclose(O.pool_blocks_resblock(x, cnt, 4, z, zb, z, b2), O.pool_blocks(x, cnt, 4) + b2,
                               atol=1e-14)
    eye = np.broadcast_to(np.eye(D), (H, D, D))
    got = O.pool_blocks_resblock(x, cnt, 4, eye, zb, eye, zb)[0]
    np.testing.assert_allclose(got, x[0] + x[0] / (1.0 + np.exp(-x[0])), atol=1e-14)
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15


def test_resblock_matches_a_dense_restatement():
    """The per-head residual MLP equals a block-diagonal dense MLP over the whole token row."""
    rng = np.random.default_rng(22)
    H, D = 3, 4
    x = rng.standard_normal((5, H, D))
    w1 = rng.standard_normal((H, D, D)); w2 = rng.standard_normal((H, D, D))
    b1 = rng.standard_normal((H, D)); b2 = rng.standard_normal((H, D))
    W1 = np.zeros((H * D, H * D)); W2 = np.zeros((H * D, H * D))
    for h in range(H):
        W1[h * D:(h + 1) * D, h * D:(h + 1) * D] = w1[h]
        W2[h * D:(h + 1) * D, h * D:(h + 1) * D] = w2[h]
    flat = x.reshape(5, H * D)
    pre = flat @ W1.T + b1.reshape(-1)
    dense = flat + (pre * (0.5 + 0.5 * np.tanh(pre / 2))) @ W2.T + b2.reshape(-1)
    np.testing.assert_allclose(O.resblock(x, w1, b1, w2, b2).reshape(5, H * D), dense, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# active-voxel selection and the volume block table
# ---------------------------------------------------------------------------------------------

def test_volume_ramp_hand_fixture():
    fx = json.load(open(os.path.join(GOLDEN, "volume_ramp.json"), encoding="utf-8"))
    cnt, key, pts = O.volume_block_table(np.array(fx["sdf"], dtype=np.float32), fx["N"], fx["tau"])
    assert cnt.tolist() == fx["blk_cnt"] and key.tolist() == fx["blk_key"]
    np.testing.assert_array_equal(pts[:3], np.array(fx["first_points"], dtype=np.float32))
    assert np.all(pts[32:] == 0)


def test_volume_constant_sdf():
    g = np.full((3, 3, 3), 0.3, dtype=np.float32)
    assert not O.voxel_activity(g, 8, 0.2).any()
    assert O.voxel_activity(g, 8, float(np.float32(0.3))).all()       # tau equal to the stored value
    assert O.voxel_activity(np.zeros((3, 3, 3), np.float32), 8, 0.0).all()       # s = 0: min * max <= 0


def _subsample_coords(N):
    """Sub-sample positions of one axis in [-1, 1] (float64)."""
    return -1.0 + (np.arange(4 * N) + 0.5) / (2.0 * N)


def test_volume_linear_sdf_matches_closed_form():
    """Trilinear interpolation reproduces a linear SDF, so activity follows from the analytic values
    at the sub-samples.  The oracle computes in float64 on the float32 lattice, whose values carry
    the float32 rounding of the linear function (below 1e-7 here), so only voxels within 1e-6 of
    the threshold or of zero are left out; their count is reported and must be tiny."""
    G, N, tau = 5, 8, 0.07
    a = np.array([0.6, -0.3, 0.2])
    c0 = 0.013
    g = np.linspace(-1.0, 1.0, G)
    zz, yy, xx = np.meshgrid(g, g, g, indexing="ij")
    sdf = (a[0] * xx + a[1] * yy + a[2] * zz + c0).astype(np.float32)
    act = O.voxel_activity(sdf, N, tau)
    x = _subsample_coords(N)
    Z, Y, X = np.meshgrid(x, x, x, indexing="ij")
    s = a[0] * X + a[1] * Y + a[2] * Z + c0
    s = s.reshape(N, 4, N, 4, N, 4).transpose(0, 2, 4, 1, 3, 5).reshape(N, N, N, 64)
    want = (np.abs(s).min(axis=3) <= tau) | (s.min(axis=3) * s.max(axis=3) <= 0)
    margin = np.minimum(np.abs(np.abs(s).min(axis=3) - tau), np.abs(s).min(axis=3))
    ok = margin > 1e-6
    print("linear SDF: %d of %d voxels within 1e-6 of a threshold" % ((~ok).sum(), ok.size))
    assert ok.mean() > 0.999
    np.testing.assert_array_equal(act[ok], want[ok])


def test_volume_sphere_sdf_bounds():
    """A sphere SDF sampled on the lattice: voxels whose analytic sub-sample values all keep
    |s| > tau + 0.02 (above the interpolation error) are inactive; voxels with a sub-sample within
    tau - 0.02 of the surface, or cut by it with that margin, are active."""
    G, N, r, tau = 33, 32, 0.55, 0.03
    g = np.linspace(-1.0, 1.0, G)
    zz, yy, xx = np.meshgrid(g, g, g, indexing="ij")
    sdf = (np.sqrt(xx ** 2 + yy ** 2 + zz ** 2) - r).astype(np.float32)
    act = O.voxel_activity(sdf, N, tau)
    x = _subsample_coords(N)
    Z, Y, X = np.meshgrid(x, x, x, indexing="ij")
    s = (np.sqrt(X ** 2 + Y ** 2 + Z ** 2) - r).reshape(N, 4, N, 4, N, 4).transpose(0, 2, 4, 1, 3, 5)
    s = s.reshape(N, N, N, 64)
    mn, mx, mabs = s.min(axis=3), s.max(axis=3), np.abs(s).min(axis=3)
    surely_off = (mabs > tau + 0.02) & ((mn > 0.02) | (mx < -0.02))
    surely_on = (mabs < tau - 0.02) | ((mn < -0.02) & (mx > 0.02))
    assert surely_on.sum() > 500 and surely_off.sum() > 20000
    assert not act[surely_off].any()
    assert act[surely_on].all()


def test_volume_block_grouping_rules():
    """Block table of a random SDF lattice: every block's points lie in one 4^3 cell whose Morton
    code is its key, keys ascend, points inside a block ascend in local Morton order, counts add
    up to the active voxels, padding points are zero."""
    rng = np.random.default_rng(31)
    N = 16
    sdf = rng.standard_normal((7, 7, 7)).astype(np.float32)
    act = O.voxel_activity(sdf, N, 0.05)
    cnt, key, pts = O.volume_block_table(sdf, N, 0.05)
    assert cnt.sum() == act.sum() and np.all(np.diff(key.astype(np.int64)) > 0)
    for b in range(cnt.shape[0]):
        p = pts[b * 64: b * 64 + cnt[b]].astype(np.float64)
        idx = np.rint((p * N + N - 1) / 2).astype(np.int64)            # voxel indices back from centres
        cx, cy, cz = idx[:, 0] >> 2, idx[:, 1] >> 2, idx[:, 2] >> 2
        assert len(set(zip(cx, cy, cz))) == 1
        code = 0
        for bit in range(3):
            code |= ((int(cx[0]) >> bit) & 1) << (3 * bit) | ((int(cy[0]) >> bit) & 1) << (3 * bit + 1) | \
                    ((int(cz[0]) >> bit) & 1) << (3 * bit + 2)
        assert code == key[b]
        loc = [int(((x & 1) | ((y & 1) << 1) | ((z & 1) << 2) | ((x & 2) << 2) | ((y & 2) << 3) | ((z & 2) << 4)))
               for x, y, z in zip(idx[:, 0] & 3, idx[:, 1] & 3, idx[:, 2] & 3)]
        assert loc == sorted(loc) and len(set(loc)) == len(loc)
        assert all(act[z, y, x] for x, y, z in idx)
        assert np.all(pts[b * 64 + cnt[b]: (b + 1) * 64] == 0)


# ---------------------------------------------------------------------------------------------
# split self/cross NSA
# ---------------------------------------------------------------------------------------------

def brute_route_range(pts, blk_cnt, blk_key, cap, k, q_blocks, kv_blocks):
    """brute_route with the candidates restricted to the blocks kv_blocks, for the slots of q_blocks."""
    full = {}
    lat = lambda x: int(round(4096 * float(x))) + 4096  # noqa: E731
    cents = {}
    for b in range(len(blk_cnt)):
        members = [b * cap + i for i in range(blk_cnt[b])]
        n = blk_cnt[b]
        cents[b] = [(2 * sum(lat(pts[s][ax]) for s in members) + n) // (2 * n) for ax in range(3)]
    for b in range(*q_blocks):
        for i in range(blk_cnt[b]):
            s = b * cap + i
            u = [lat(pts[s][ax]) for ax in range(3)]
            cand = sorted((sum((u[a] - cents[c][a]) ** 2 for a in range(3)), int(blk_key[c]), c)
                          for c in range(*kv_blocks))
            full[s] = [c for _, _, c in cand[:k]]
    return full


@pytest.mark.parametrize("q_blocks,kv_blocks", [((0, 4), (0, 4)), ((0, 4), (4, 9)), ((4, 9), (0, 4)),
                                                ((2, 7), (5, 6)), ((0, 9), (3, 3))])
def test_route_range_brute_force(q_blocks, kv_blocks):
    w = W.custom_block_workload(22, [5, 8, 1, 3, 8, 6, 2, 7, 8], 8, 4, 2, 8, "f32", 4)
    sel, d2 = O.route_geometric_range(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k, q_blocks, kv_blocks)
    ref = brute_route_range(w.pts.tolist(), w.blk_cnt.tolist(), w.blk_key, w.blk_cap, w.top_k, q_blocks, kv_blocks)
    for i, s in enumerate(range(q_blocks[0] * w.blk_cap, q_blocks[1] * w.blk_cap)):
        want = ref.get(s, [])
        assert sel[i, :len(want)].tolist() == want
        assert (sel[i, len(want):] == -1).all()
    # with every block a candidate the range form is the plain routing
    full, _ = O.route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k)
    rng_all, _ = O.route_geometric_range(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k, (0, 9), (0, 9))
    np.testing.assert_array_equal(full, rng_all)


def _split_case(seed=23, n_x_blk=4, dtype="f32"):
    w = W.custom_block_workload(seed, [5, 8, 1, 3, 8, 6, 2, 7, 8], 8, 4, 2, 8, dtype, 3, n_gate=7)
    return w, n_x_blk


def test_split_reduces_to_dense_gated_self_cross():
    """All blocks of a type routed and only the selected branches gated on: every token gets
    s(g0) Attn(own-type tokens) + s(g1) Attn(other-type tokens), checked with library attention."""
    w, nx = _split_case()
    w.top_k = 5                               # at least the block count of either type
    g = w.gates.copy()
    g[..., 2] = g[..., 4] = g[..., 5] = -np.inf
    g[..., 3] = g[..., 6] = np.inf
    o = O.nsa_split_forward(w, nx, g)
    vs = w.valid_slots()
    xs = vs[vs // w.blk_cap < nx]
    ys = vs[vs // w.blk_cap >= nx]
    sg = 1.0 / (1.0 + np.exp(-g.astype(np.float64)))
    for own, oth in ((xs, ys), (ys, xs)):
        a = sdpa(w.q[own], w.k[own], w.v[own], w.scale)
        c = sdpa(w.q[own], w.k[oth], w.v[oth], w.scale)
        ref = sg[own][:, :, 0:1] * a + sg[own][:, :, 1:2] * c
        np.testing.assert_allclose(o[own], ref, rtol=0, atol=1e-12)
    assert np.all(o[~w.valid_mask()] == 0)


@pytest.mark.parametrize("nx", [0, 9])
def test_split_single_type_is_gated_nsa(nx):
    """With one token type the cross term is empty and the layer is s(g0) times the three-branch
    NSA layer whose gates are channels 2..4."""
    w, _ = _split_case(seed=24)
    o = O.nsa_split_forward(w, nx, w.gates)
    w3 = W.custom_block_workload(24, [5, 8, 1, 3, 8, 6, 2, 7, 8], 8, 4, 2, 8, "f32", 3, n_gate=7)
    w3.gates = w.gates[..., 2:5].copy()
    ref = O.nsa_forward(w3)
    sg0 = 1.0 / (1.0 + np.exp(-w.gates[..., 0:1].astype(np.float64)))
    np.testing.assert_allclose(o, sg0 * ref, rtol=0, atol=1e-12)


def test_split_cross_compressed_orientation():
    """Only the other-type compressed branch on: a volume token attends the pooled image blocks and
    an image token the pooled volume blocks (plain means, library attention)."""
    w, nx = _split_case(seed=25)
    g = np.full_like(w.gates, -np.inf)
    g[..., 1] = np.inf
    g[..., 5] = np.inf
    o = O.nsa_split_forward(w, nx, g)
    pooled_k = np.stack([w.k[O.block_slots(w.blk_cnt, w.blk_cap, b)].astype(np.float64).mean(0) for b in range(w.n_blk)])
    pooled_v = np.stack([w.v[O.block_slots(w.blk_cnt, w.blk_cap, b)].astype(np.float64).mean(0) for b in range(w.n_blk)])
    for s in w.valid_slots():
        other = slice(nx, w.n_blk) if s // w.blk_cap < nx else slice(0, nx)
        ref = sdpa(w.q[s:s + 1], pooled_k[other], pooled_v[other], w.scale)[0]
        np.testing.assert_allclose(o[s], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# routing with image blocks found through the views
# ---------------------------------------------------------------------------------------------

def test_views_projection_recovers_own_cell():
    w = W.make("stage2_small")
    proj, cell_blk = W.view_cameras(w)
    for b in np.nonzero(w.blk_type == 1)[0]:
        v = int((int(w.blk_key[b]) >> 20) & 0x7FF)
        cy, cx = [int(x[0]) for x in np.nonzero(cell_blk[v] == b)]
        for s in O.block_slots(w.blk_cnt, w.blk_cap, b):
            assert O.project_cell(w.pts[s], proj[v, 0], 8) == cx
            assert O.project_cell(w.pts[s], proj[v, 1], 8) == cy


def test_views_whole_grid_window_is_all_blocks():
    """A window covering every cell makes every image block a candidate: the ranking is then the
    plain one over all blocks with each image block's nearest-member metric (vectorised here)."""
    w = W.make("stage2_small")
    proj, cell_blk = W.view_cameras(w)
    nv = int((w.blk_type == 0).sum())
    rows = np.array([0, 5, 63, nv * 64 + 3, nv * 64 + 200, (w.n_blk - 1) * 64])
    rows = rows[w.valid_mask()[rows]]
    sel, d2 = O.route_geometric_views(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k, nv, proj, cell_blk, 8,
                                      cell_blk.shape[1], rows=rows)
    u = O.lattice_coords(w.pts).astype(np.int64)
    cen = O.block_centroids(w.pts, w.blk_cnt, w.blk_cap).astype(np.int64)
    for i, r in enumerate(rows):
        m = ((cen - u[r]) ** 2).sum(axis=1)
        for b in range(nv, w.n_blk):
            m[b] = ((u[O.block_slots(w.blk_cnt, w.blk_cap, b)] - u[r]) ** 2).sum(axis=1).min()
        order = np.lexsort((w.blk_key.astype(np.int64), m))[:w.top_k]
        assert sel[i].tolist() == order.tolist()
        assert d2[i].astype(np.int64).tolist() == m[order].tolist()


def test_views_brute_force_python():
    """Two axis-aligned views on a 2x2 cell grid, hand-made: pure-Python candidate windows and
    nearest-member metrics, sorted as tuples."""
    w = W.custom_block_workload(41, [3, 5, 2, 4, 6, 1, 3, 2], 8, 4, 2, 8, "f32", 4)
    nv = 3                                                   # blocks 0..2 volume, 3..7 image
    # view 0 sees (x, y), view 1 sees (y, z): patch coordinate 8 (c + 1) on a 16-patch side
    proj = np.zeros((2, 2, 4), dtype=np.float32)
    proj[0, 0, 0] = proj[0, 1, 1] = proj[1, 0, 1] = proj[1, 1, 2] = 8.0
    proj[:, :, 3] = 8.0
    cell_blk = np.full((2, 2, 2), -1, dtype=np.int32)
    cell_blk[0, 0, 0], cell_blk[0, 1, 1], cell_blk[1, 0, 1], cell_blk[1, 1, 0], cell_blk[1, 1, 1] = 3, 4, 5, 6, 7
    for radius in (0, 1):
        sel, d2 = O.route_geometric_views(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k, nv, proj, cell_blk, 8, radius)
        lat = lambda x: int(round(4096 * float(x))) + 4096  # noqa: E731
        P = w.pts.tolist()
        U = [[lat(c) for c in p] for p in P]
        members = {b: [b * 8 + i for i in range(int(w.blk_cnt[b]))] for b in range(8)}
        cents = {b: [(2 * sum(U[t][a] for t in members[b]) + len(members[b])) // (2 * len(members[b]))
                     for a in range(3)] for b in range(8)}
        where = {int(cell_blk[v, y, x]): (v, y, x) for v in range(2) for y in range(2) for x in range(2)
                 if cell_blk[v, y, x] >= 0}
        for s in range(w.n_slots):
            if s % 8 >= w.blk_cnt[s // 8]:
                assert (sel[s] == -1).all()
                continue
            d = lambda a, b: sum((a[i] - b[i]) ** 2 for i in range(3))  # noqa: E731
            cand = [(d(U[s], cents[b]), int(w.blk_key[b]), b) for b in range(nv)]
            for b, (v, y, x) in where.items():
                cx = O.project_cell(P[s], proj[v, 0], 8)
                cy = O.project_cell(P[s], proj[v, 1], 8)
                if abs(x - cx) <= radius and abs(y - cy) <= radius:
                    cand.append((min(d(U[s], U[t]) for t in members[b]), int(w.blk_key[b]), b))
            cand.sort()
            want = [b for _, _, b in cand[:w.top_k]]
            assert sel[s, :len(want)].tolist() == want
            assert (sel[s, len(want):] == -1).all()


def test_views_image_query_finds_its_own_block():
    """An image token lies in its own view's projection cell and is its own block's member at
    distance 0, so with any window its own block ranks first (or ties at d2 = 0)."""
    w = W.make("stage2_small")
    proj, cell_blk = W.view_cameras(w)
    nv = int((w.blk_type == 0).sum())
    rows = np.arange(nv * 64, w.n_slots, 37)
    rows = rows[w.valid_mask()[rows]]
    sel, d2 = O.route_geometric_views(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k, nv, proj, cell_blk, 8, 0,
                                      rows=rows)
    assert np.all(d2[:, 0] == 0)
    assert np.mean(sel[:, 0] == rows // 64) > 0.9


# ---------------------------------------------------------------------------------------------
# forced-include blocks in the selected branch (Speed3R, VGGT variant)
# ---------------------------------------------------------------------------------------------

def _s3_case():
    w = W.custom_block_workload(61, [16, 4, 16, 1, 16, 4, 9, 16], 16, 4, 4, 8, "f32", 2, routing="scores",
                                q_gran="block", branches=("cmp", "sel"))
    rng = np.random.default_rng(62)
    sel = rng.integers(-1, w.n_blk, size=(w.n_blk, w.n_kvh, w.top_k)).astype(np.int32)
    return w, sel


def test_forced_all_blocks_is_dense_attention():
    """Forcing every block makes each query attend every valid token, whatever its routing row."""
    w, sel = _s3_case()
    o, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel, q_gran="block",
                         forced=(0, w.n_blk))
    vs = w.valid_slots()
    np.testing.assert_allclose(o[vs], sdpa(w.q[vs], w.k[vs], w.v[vs], w.scale), rtol=0, atol=1e-12)


def test_forced_range_adds_its_blocks_once():
    """An empty forced range changes nothing; forcing blocks every routing row already lists changes
    nothing either (a block counts once); forcing other blocks equals listing them explicitly."""
    w, sel = _s3_case()
    base, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel, q_gran="block")
    empty, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel, q_gran="block",
                             forced=(3, 3))
    np.testing.assert_array_equal(empty, base)
    sel2 = sel.copy()
    sel2[:, :, 0] = 5
    a, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel2, q_gran="block")
    b, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel2, q_gran="block",
                         forced=(5, 6))
    np.testing.assert_array_equal(a, b)
    wide = np.concatenate([sel, np.broadcast_to(np.array([1, 2], np.int32), sel.shape[:2] + (2,))], axis=2)
    c, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=wide, q_gran="block")
    f, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel, q_gran="block",
                         forced=(1, 3))
    np.testing.assert_allclose(f, c, rtol=0, atol=1e-13)
