"""GPU parity: every libnsa call against the fp64 oracle on the same seeded inputs.

Bars: routed block indices bit-exact; outputs within max-abs 2e-2 (bf16 inputs) or 1e-4 (fp32).
Oracle-side inputs never come from the GPU: where a call consumes an upstream result (pooled K/V,
routing rows, lse), the test feeds the oracle's value, rounded to the storage dtype, to both sides.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import host, max_err, rounded, say, tdt, to_dev, tol

pytestmark = pytest.mark.gpu

SMALL = ["tiny", "stage2_small", "large_small"]
_cache = {}


def wl(name):
    if name not in _cache:
        _cache[name] = W.make(name)
    return _cache[name]


def edge(kind):
    if kind == "ragged_cap16":
        return W.custom_block_workload(5, [16, 1, 7, 16, 3, 9, 12, 2] * 9, 16, 32, 2, 32, "bf16", 8)
    if kind == "single_block":
        return W.custom_block_workload(6, [37], 64, 32, 2, 32, "bf16", 1)
    if kind == "k_beyond_blocks":
        return W.custom_block_workload(7, [64, 5, 33], 64, 32, 2, 32, "bf16", 6)
    if kind == "lattice_ties":
        return W.custom_block_workload(8, [1] * 150, 1, 32, 2, 32, "f32", 12, pts_mode="lattice")
    if kind == "cnt_one_blocks":
        return W.custom_block_workload(9, [1, 64, 1, 1, 64, 2] * 20, 64, 32, 2, 32, "f32", 5)
    if kind == "k48_cap16":       # the 64-entry routing list and selections of up to 48 blocks
        cnt = np.random.default_rng(10).integers(1, 17, size=100).tolist()
        return W.custom_block_workload(10, cnt, 16, 32, 2, 32, "bf16", 48)
    if kind == "k64_cap8":
        cnt = np.random.default_rng(11).integers(1, 9, size=90).tolist()
        return W.custom_block_workload(11, cnt, 8, 32, 2, 32, "f32", 64)
    if kind == "k64_cap8_bf16":   # every lane of the selected-branch wave holds eight routing entries
        cnt = np.random.default_rng(12).integers(1, 9, size=90).tolist()
        return W.custom_block_workload(12, cnt, 8, 32, 2, 32, "bf16", 64)
    if kind == "cap1_bf16":       # one slot per block: one-token clusters, one-key tiles
        return W.custom_block_workload(13, [1] * 150, 1, 32, 2, 32, "bf16", 12)
    if kind == "ragged_cap64_bf16":   # partial 8-slot clusters at every block end
        cnt = np.random.default_rng(14).integers(1, 65, size=40).tolist()
        return W.custom_block_workload(14, cnt, 64, 32, 2, 32, "bf16", 24)
    raise KeyError(kind)


EDGES = ["ragged_cap16", "single_block", "k_beyond_blocks", "lattice_ties", "cnt_one_blocks", "k48_cap16", "k64_cap8",
         "k64_cap8_bf16", "cap1_bf16", "ragged_cap64_bf16"]


def get(name):
    return edge(name) if name in EDGES else wl(name)


# ---------------------------------------------------------------------------------------------
# pooling
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "stage2_small", "ragged_cap16"])
def test_pool_blocks(name):
    import sparse_attention_feed_amd as S
    w = get(name)
    d = to_dev(w)
    say("pool", name)
    for key in ("k", "v", "q"):
        got = host(S.pool_blocks(d["layout"], d[key]))
        torch.cuda.synchronize()
        ref = O.pool_blocks(getattr(w, key), w.blk_cnt, w.blk_cap)
        err = max_err(got, ref)
        assert err <= (1e-5 if w.dtype == "f32" else 8e-3), (key, err)


@pytest.mark.parametrize("name", ["tiny", "stage2_small", "ragged_cap16", "cnt_one_blocks", "speed3r_small"])
def test_pool_blocks_resblock(name):
    """AvgPool(ResBlock(x)) with seeded weights against the oracle, and with zero weights exactly the
    plain block mean of nsa_pool_blocks."""
    import sparse_attention_feed_amd as S
    w = get(name)
    d = to_dev(w)
    for key in ("k", "v"):
        H = d[key].shape[1]
        wts = W.resblock_weights(31 if key == "k" else 32, H, w.head_dim)
        w1, b1, w2, b2 = (torch.from_numpy(a).cuda() for a in wts)
        say("pool resblock", name, key)
        got = host(S.pool_blocks_resblock(d["layout"], d[key], w1, b1, w2, b2))
        torch.cuda.synchronize()
        ref = O.pool_blocks_resblock(getattr(w, key), w.blk_cnt, w.blk_cap, *wts)
        err = max_err(got, ref)
        assert err <= (1e-4 if w.dtype == "f32" else 2e-2), (key, err)
        z3 = torch.zeros_like(w1)
        z2 = torch.zeros_like(b1)
        plain = S.pool_blocks(d["layout"], d[key])
        zero = S.pool_blocks_resblock(d["layout"], d[key], z3, z2, z3, z2)
        torch.cuda.synchronize()
        assert torch.equal(plain, zero)


# ---------------------------------------------------------------------------------------------
# geometric routing: bit-exact
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", SMALL + ["ragged_cap16", "single_block", "k_beyond_blocks", "lattice_ties",
                                          "cnt_one_blocks", "k48_cap16", "k64_cap8"])
def test_route_geometric_bit_exact(name):
    import sparse_attention_feed_amd as S
    w = get(name)
    d = to_dev(w)
    say("route_geometric", name, "n_blk", w.n_blk, "k", w.top_k)
    sel, d2, cent = S.route_geometric(d["layout"], d["pts"], w.top_k)
    torch.cuda.synchronize()
    ref_sel, ref_d2 = O.route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k)
    np.testing.assert_array_equal(host(sel), ref_sel)
    np.testing.assert_array_equal(host(d2).view(np.uint32), ref_d2)
    ref_c = O.block_centroids(w.pts, w.blk_cnt, w.blk_cap)
    np.testing.assert_array_equal(host(cent)[:, :3], ref_c)


# ---------------------------------------------------------------------------------------------
# single branches (with lse)
# ---------------------------------------------------------------------------------------------

def _branch_inputs(w, d):
    kc = rounded(O.pool_blocks(w.k, w.blk_cnt, w.blk_cap), w.dtype)
    vc = rounded(O.pool_blocks(w.v, w.blk_cnt, w.blk_cap), w.dtype)
    sel, _ = O.route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k)
    dt = tdt(w)
    return (kc, vc, sel, torch.from_numpy(kc).cuda().to(dt), torch.from_numpy(vc).cuda().to(dt),
            torch.from_numpy(sel).cuda())


@pytest.mark.parametrize("name", SMALL + ["ragged_cap16", "single_block", "k_beyond_blocks", "cnt_one_blocks"])
@pytest.mark.parametrize("branch", ["cmp", "sel", "loc"])
def test_single_branch(name, branch):
    import sparse_attention_feed_amd as S
    w = get(name)
    d = to_dev(w)
    kc, vc, sel, kc_d, vc_d, sel_d = _branch_inputs(w, d)
    bit = {"cmp": S.BR_CMP, "sel": S.BR_SEL, "loc": S.BR_LOC}[branch]
    lse = torch.empty((w.n_slots, w.n_qh), dtype=torch.float32, device="cuda")
    say("attn", name, branch)
    o = S.attn_fwd(d["layout"], bit, d["q"], d["k"], d["v"], k_cmp=kc_d, v_cmp=vc_d, sel=sel_d,
                   top_k=w.top_k, sel_groups=1, lse=lse)
    torch.cuda.synchronize()
    br = O.BRANCH_NAMES[branch]
    if br == O.CMP:
        ref, ref_lse = O.attn_branch(O.CMP, w.q, kc.astype(np.float64), vc.astype(np.float64), w.blk_cnt,
                                     w.blk_cap, w.scale)
    else:
        ref, ref_lse = O.attn_branch(br, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel)
    vm = w.valid_mask()
    err = max_err(host(o), ref)
    assert err <= tol(w), err
    assert np.all(host(o)[~vm] == 0)
    gl = host(lse)
    assert np.all(np.isneginf(gl[~vm]))
    # bf16 bound, from the arithmetic: probabilities are rounded to bf16 (relative error <= 2^-9)
    # before they are summed, so |d ln l| <= -ln(1 - 2^-9) ~= 1.96e-3; the query is scaled by
    # scale*log2(e) and rounded once to bf16, which moves every logit by at most
    # 2^-9 * scale * |q_h| * |k| (Cauchy-Schwarz); plus fp32 rounding
    if w.dtype == "f32":
        bound = 1e-4
    else:
        keys = kc if br == O.CMP else w.k
        qn = np.linalg.norm(w.q.astype(np.float64), axis=2).max()
        kn = np.linalg.norm(keys.astype(np.float64), axis=2).max()
        bound = 1.96e-3 + 2.0 ** -9 * w.scale * qn * kn + 1e-4
    assert max_err(gl[vm], ref_lse[vm]) <= bound


# ---------------------------------------------------------------------------------------------
# fused gated layer (pool + route + three branches + gate) against the whole oracle layer
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", SMALL + ["ragged_cap16", "k_beyond_blocks", "cnt_one_blocks", "k48_cap16",
                                          "k64_cap8", "k64_cap8_bf16", "cap1_bf16", "ragged_cap64_bf16"])
def test_fused_layer(name):
    import sparse_attention_feed_amd as S
    w = get(name)
    d = to_dev(w)
    say("layer", name)
    o = S.nsa_layer(d["layout"], d["q"], d["k"], d["v"], d["pts"], d["gates"], w.top_k)
    torch.cuda.synchronize()
    ref = O.nsa_forward(w)
    err = max_err(host(o), ref)
    assert err <= tol(w), err
    assert np.all(host(o)[~w.valid_mask()] == 0)


def test_fused_equals_unfused_combine():
    """Fused three-branch output equals the standalone gate over the three single-branch outputs."""
    import sparse_attention_feed_amd as S
    w = wl("stage2_small")
    d = to_dev(w)
    kc, vc, sel, kc_d, vc_d, sel_d = _branch_inputs(w, d)
    say("fused-vs-unfused stage2_small")
    outs = [S.attn_fwd(d["layout"], bit, d["q"], d["k"], d["v"], k_cmp=kc_d, v_cmp=vc_d, sel=sel_d,
                       top_k=w.top_k) for bit in (S.BR_CMP, S.BR_SEL, S.BR_LOC)]
    comb = S.gate_combine(outs, d["gates"])
    fused = S.attn_fwd(d["layout"], 7, d["q"], d["k"], d["v"], k_cmp=kc_d, v_cmp=vc_d, sel=sel_d,
                       top_k=w.top_k, gates=d["gates"])
    torch.cuda.synchronize()
    ref_outs = [O.attn_branch(O.CMP, w.q, kc.astype(np.float64), vc.astype(np.float64), w.blk_cnt, w.blk_cap,
                              w.scale)[0],
                O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel)[0],
                O.attn_branch(O.LOC, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale)[0]]
    ref = O.gate_combine(ref_outs, w.gates)
    assert max_err(host(comb), ref) <= tol(w)
    assert max_err(host(fused), ref) <= tol(w)
    # two-branch fused call: channel c is the c-th named branch
    g2 = d["gates"][:, :, 1:3].contiguous()
    two = S.attn_fwd(d["layout"], S.BR_SEL | S.BR_LOC, d["q"], d["k"], d["v"], sel=sel_d, top_k=w.top_k, gates=g2)
    torch.cuda.synchronize()
    ref2 = O.gate_combine(ref_outs[1:], w.gates[:, :, 1:3])
    assert max_err(host(two), ref2) <= tol(w)


@pytest.mark.parametrize("kind", ["peaked", "flat", "far_below", "far_above"])
def test_logit_range_extremes(kind):
    """Logits far from the running reference max's start at 0 exercise the online softmax's exact
    path: peaked (q x 64: the max moves up often), flat (q / 64), every logit about -230 or +230
    (base 2; the first tile has no representable mass, or overflows, until the max moves).  The
    fused layer against the whole oracle layer on fp32 inputs."""
    import copy
    import sparse_attention_feed_amd as S
    w = copy.copy(wl("tiny"))
    rng = np.random.default_rng(12)
    if kind in ("peaked", "flat"):
        w.q = (w.q * (64.0 if kind == "peaked" else 1.0 / 64)).astype(np.float32)
    else:
        u = rng.standard_normal((1, w.n_kvh, w.head_dim))
        u /= np.linalg.norm(u, axis=2, keepdims=True)
        sign = -1.0 if kind == "far_below" else 1.0
        w.k = (3.0 * u + 0.05 * rng.standard_normal(w.k.shape)).astype(np.float32)
        qu = np.repeat(u, w.n_qh // w.n_kvh, axis=1)
        w.q = (sign * 300.0 * qu + 0.5 * rng.standard_normal(w.q.shape)).astype(np.float32)
        w.q[~w.valid_mask()] = 0
        w.k[~w.valid_mask()] = 0
    d = to_dev(w)
    say("layer logit range", kind)
    o = S.nsa_layer(d["layout"], d["q"], d["k"], d["v"], d["pts"], d["gates"], w.top_k)
    torch.cuda.synchronize()
    ref = O.nsa_forward(w)
    got = host(o)
    assert np.all(np.isfinite(got))
    assert max_err(got, ref) <= tol(w)


def test_per_group_selection_lists():
    import sparse_attention_feed_amd as S
    w = wl("stage2_small")
    d = to_dev(w)
    rng = np.random.default_rng(4)
    sel = np.full((w.n_slots, 2, w.top_k), -1, dtype=np.int32)
    vm = w.valid_mask()
    for s in np.nonzero(vm)[0]:
        for j in range(2):
            n = rng.integers(1, w.top_k + 1)
            sel[s, j, :n] = rng.choice(w.n_blk, n, replace=False)
    sel[5, 0, :] = -1   # one empty list: that group's output is 0
    say("attn per-group sel stage2_small")
    o = S.attn_fwd(d["layout"], S.BR_SEL, d["q"], d["k"], d["v"], sel=torch.from_numpy(sel).cuda(),
                   top_k=w.top_k, sel_groups=2)
    torch.cuda.synchronize()
    ref, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel)
    assert max_err(host(o), ref) <= tol(w)


def test_gate_combine_standalone():
    import sparse_attention_feed_amd as S
    rng = np.random.default_rng(0)
    outs = [rounded(rng.standard_normal((300, 32, 32)), "bf16") for _ in range(3)]
    g = rounded(rng.standard_normal((300, 32, 3)), "bf16")
    g[0, 0, :] = [np.inf, -np.inf, 0.0]
    say("gate_combine")
    got = S.gate_combine([torch.from_numpy(x).cuda().to(torch.bfloat16) for x in outs],
                         torch.from_numpy(g).cuda().to(torch.bfloat16))
    torch.cuda.synchronize()
    assert max_err(host(got), O.gate_combine(outs, g)) <= 2e-2


# ---------------------------------------------------------------------------------------------
# stage-1 dense gated self/cross attention
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_x", ["default", 500, 0, "all"])
def test_dense_gated(dtype, n_x):
    import sparse_attention_feed_amd as S
    w = W.make("dense_small", dtype=dtype)
    nx = {"default": w.n_x, "all": w.n_tok}.get(n_x, n_x)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = {k: torch.from_numpy(getattr(w, k)).cuda().to(dt) for k in ("q", "k", "v", "gates")}
    say("dense", dtype, nx)
    o = S.dense_gated_xattn(t["q"], t["k"], t["v"], nx, t["gates"])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, w.n_tok, 7), [0, max(nx - 1, 0), min(nx, w.n_tok - 1),
                                                                 w.n_tok - 1]]))
    ref = O.dense_gated_xattn(w.q, w.k, w.v, nx, w.gates, w.scale, rows=rows)
    assert max_err(host(o)[rows], ref) <= (2e-2 if dtype == "bf16" else 1e-4)


# ---------------------------------------------------------------------------------------------
# score routing (grouped-query form) — epsilon-tie agreement
# ---------------------------------------------------------------------------------------------

def _gqa_k64_ragged():
    """150 blocks (two full 64-block steps and a ragged third) with ragged counts, top_k 64."""
    cnt = np.random.default_rng(21).integers(1, 65, size=150).tolist()
    return W.custom_block_workload(21, cnt, 64, 32, 2, 32, "bf16", 64)


def _score_route_case(name, top_k, n_rows=None, seed=0):
    """Grouped-query score routing against the oracle on the oracle's own pooled keys (rounded to
    bf16) and lse: epsilon-tie agreement on every checked row (a block listed by only one side
    must have an oracle importance within eps of the oracle's k-th), and the fraction of rows that
    agree exactly reported.  Returns that fraction."""
    import sparse_attention_feed_amd as S
    w = _gqa_k64_ragged() if name == "k64_ragged" else get(name)
    d = to_dev(w)
    kc = rounded(O.pool_blocks(w.k, w.blk_cnt, w.blk_cap), w.dtype)
    vc = rounded(O.pool_blocks(w.v, w.blk_cnt, w.blk_cap), w.dtype)
    vs = w.valid_slots()
    rows = vs if n_rows is None else np.sort(np.random.default_rng(seed).choice(vs, n_rows, replace=False))
    _, lse_rows = O.attn_branch(O.CMP, w.q, kc.astype(np.float64), vc.astype(np.float64), w.blk_cnt,
                                w.blk_cap, w.scale, rows=rows)
    lse = np.full((w.n_slots, w.n_qh), -np.inf, dtype=np.float32)
    lse[rows] = lse_rows
    # rows the oracle did not compute get a finite lse (their routing is not compared)
    rest = np.setdiff1d(vs, rows)
    lse[rest] = 0.0
    k = min(top_k, w.n_blk)
    say("score_route", name, "n_blk", w.n_blk, "k", k, "rows", len(rows))
    sel = S.route_scores_topk(d["layout"], d["q"], torch.from_numpy(kc).cuda().to(tdt(w)),
                              torch.from_numpy(lse).cuda(), k)
    torch.cuda.synchronize()
    got = host(sel)
    ref_sel, imp = O.route_scores(w.q[rows], kc, w.blk_key, w.scale, k, lse=lse.astype(np.float64)[rows])
    assert np.all(got[~w.valid_mask()] == -1)
    eps_rel = 1e-2 if w.dtype == "bf16" else 1e-5
    exact = 0
    for i, s_ in enumerate(rows):
        for j in range(w.n_kvh):
            g_row, r_row = got[s_, j], ref_sel[i, j]
            assert len(set(g_row.tolist())) == k and g_row.min() >= 0 and g_row.max() < w.n_blk
            if np.array_equal(g_row, r_row):
                exact += 1
                continue
            kth = np.sort(imp[i, j])[::-1][k - 1]
            for b in set(g_row.tolist()) ^ set(r_row.tolist()):
                assert abs(imp[i, j, b] - kth) <= eps_rel * abs(kth), (s_, j, b)
    frac = exact / (len(rows) * w.n_kvh)
    print("score routing %s k=%d: %.3f of rows exact" % (name, k, frac), flush=True)
    return frac


@pytest.mark.parametrize("name,top_k", [("tiny", 4), ("stage2_small", 16), ("stage2_small", 8),
                                        ("large_small", 32), ("k64_ragged", 64), ("k64_ragged", 5)])
def test_score_routing(name, top_k):
    """Every valid row; the list sizes 8, 16, 32 and 64 (one compiled instance each), more than two
    64-block steps with a ragged last step (k64_ragged: 150 blocks)."""
    assert _score_route_case(name, top_k) >= 0.9


@pytest.mark.parametrize("name,top_k", [("stage2", 16), ("large", 32), ("large", 64)])
def test_score_routing_full_size_sampled(name, top_k):
    """The full-size workloads (2.6k and 8.7k pooled blocks) on sampled rows."""
    assert _score_route_case(name, top_k, n_rows=192, seed=5) >= 0.6


@pytest.mark.parametrize("name,n_rows", [("stage2", None), ("large", 32768)])
def test_score_routing_whole_table(name, n_rows):
    """Grouped-query score routing through the device's own pipeline (pooling, the compressed
    branch's lse, routing) against the definition on the oracle's pooled keys (rounded to bf16), by
    a vectorised whole-table check: every row of stage2 (112,768 valid tokens, top-16 of 2,615
    pooled blocks, 2 KV groups), and 32,768 seeded random rows of large (top-32 of 8,715 blocks;
    its every row would take the fp64 check about ten minutes).  The device's lse comes from queries
    pre-scaled and rounded to bf16 (reading R18), which moves each head's probabilities by a factor
    of at most exp(2^-9 * scale * |q| * |k|); importances that close to the k-th may order either
    way."""
    import sparse_attention_feed_amd as S
    w = wl(name)
    d = to_dev(w)
    L = d["layout"]
    say("score routing whole table", w.name, w.n_blk)
    kc = S.pool_blocks(L, d["k"])
    vc = S.pool_blocks(L, d["v"])
    lse = torch.empty((w.n_slots, w.n_qh), dtype=torch.float32, device="cuda")
    S.attn_fwd(L, S.BR_CMP, d["q"], k_cmp=kc, v_cmp=vc, lse=lse)
    sel = S.route_scores_topk(L, d["q"], kc, lse, w.top_k)
    torch.cuda.synchronize()
    selh = host(sel)
    vm = w.valid_mask()
    assert np.all(selh[~vm] == -1)
    kr = rounded(O.pool_blocks(w.k, w.blk_cnt, w.blk_cap), w.dtype)
    vs = w.valid_slots()
    if n_rows is not None:
        vs = np.sort(np.random.default_rng(17).choice(vs, n_rows, replace=False))
    qn = np.linalg.norm(w.q.astype(np.float64), axis=2).max()
    kn = np.linalg.norm(kr.astype(np.float64), axis=2).max()
    eps = 2.0 * np.expm1(2.0 ** -9 * w.scale * qn * kn) + 2e-3
    n_bad, n_exact, first = 0, 0, []
    step = 16384
    for lo in range(0, len(vs), step):
        rows = vs[lo:lo + step]
        b, e, f = O.check_route_scores(w.q[rows], kr, w.blk_key, selh[rows], eps, chunk=512, scale=w.scale)
        n_bad, n_exact, first = n_bad + b, n_exact + e, first + [(int(rows[r]), j) for r, j in f]
        say("checked rows", lo + len(rows), "of", len(vs), "failing", n_bad)
    print("%s score routing, %d rows: %d failing, %.4f exact (eps %.3g)"
          % (name, len(vs), n_bad, n_exact / (len(vs) * w.n_kvh), eps), flush=True)
    assert n_bad == 0, first[:8]
    assert n_exact / (len(vs) * w.n_kvh) >= 0.6


def test_gqa_score_routed_layer():
    """The grouped-query score-routed layer end to end on the GPU (pooled K/V, the compressed
    branch's lse, score routing per (token, KV group), the gated compressed + selected + local
    branches with per-group routing rows) against the oracle's steps of nsa_forward's score-routed
    layer, with the pooled values rounded to bf16 where the GPU layer stores them.  Routing: every
    row agrees with the oracle's up to epsilon ties (against the oracle's own lse, while the GPU
    routes with its own); outputs are compared on the (token, group) pairs whose rows agree."""
    import sparse_attention_feed_amd as S
    w = wl("stage2_small")
    d = to_dev(w)
    L = d["layout"]
    say("gqa score-routed layer", w.name)
    kc = S.pool_blocks(L, d["k"])
    vc = S.pool_blocks(L, d["v"])
    lse = torch.empty((w.n_slots, w.n_qh), dtype=torch.float32, device="cuda")
    S.attn_fwd(L, S.BR_CMP, d["q"], k_cmp=kc, v_cmp=vc, lse=lse)
    sel = S.route_scores_topk(L, d["q"], kc, lse, w.top_k)
    o = S.attn_fwd(L, S.BR_CMP | S.BR_SEL | S.BR_LOC, d["q"], d["k"], d["v"], k_cmp=kc, v_cmp=vc, sel=sel,
                   top_k=w.top_k, sel_groups=w.n_kvh, gates=d["gates"])
    torch.cuda.synchronize()
    kr = rounded(O.pool_blocks(w.k, w.blk_cnt, w.blk_cap), w.dtype).astype(np.float64)
    vr = rounded(O.pool_blocks(w.v, w.blk_cnt, w.blk_cap), w.dtype).astype(np.float64)
    vs = w.valid_slots()
    o_cmp, lse_o = O.attn_branch(O.CMP, w.q, kr, vr, w.blk_cnt, w.blk_cap, w.scale)
    ref_sel = np.full((w.n_slots, w.n_kvh, w.top_k), -1, dtype=np.int32)
    ref_sel[vs], imp = O.route_scores(w.q[vs], kr, w.blk_key, w.scale, w.top_k, lse=lse_o[vs])
    o_sel, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=ref_sel)
    o_loc, _ = O.attn_branch(O.LOC, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale)
    ref = O.gate_combine([o_cmp, o_sel, o_loc], w.gates)
    got_sel = host(sel)
    vm = w.valid_mask()
    for i, s_ in enumerate(vs):
        for j in range(w.n_kvh):
            if np.array_equal(got_sel[s_, j], ref_sel[s_, j]):
                continue
            kth = np.sort(imp[i, j])[::-1][w.top_k - 1]
            for b in set(got_sel[s_, j].tolist()) ^ set(ref_sel[s_, j].tolist()):
                assert abs(imp[i, j, b] - kth) <= 1e-2 * kth, (s_, j, b)
    same = np.all(got_sel == ref_sel, axis=2) & vm[:, None]                # [S, Hkv]
    print("gqa score-routed layer: %.3f of (token, group) rows exact" % same[vm].mean(), flush=True)
    assert same[vm].mean() > 0.85, same[vm].mean()
    G = w.n_qh // w.n_kvh
    diff = np.abs(host(o) - ref).max(axis=2).reshape(w.n_slots, w.n_kvh, G).max(axis=2)
    assert diff[same].max() <= tol(w), diff[same].max()
    assert np.all(host(o)[~vm] == 0)


# ---------------------------------------------------------------------------------------------
# full-size configurations on sampled rows
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["stage2", "large"])
def test_full_size_layer_sampled(name):
    import sparse_attention_feed_amd as S
    say("generate", name)
    w = wl(name)
    d = to_dev(w)
    ws = {}
    say("layer full size", name, "n_valid", w.n_valid, "n_blk", w.n_blk)
    o = S.nsa_layer(d["layout"], d["q"], d["k"], d["v"], d["pts"], d["gates"], w.top_k, ws=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    vs = w.valid_slots()
    rows = np.sort(rng.choice(vs, 384, replace=False))
    ref = O.nsa_forward(w, rows=rows)
    assert max_err(host(o)[rows], ref) <= tol(w)
    # routing bit-exact on a larger sample of tokens, and structurally valid everywhere
    rows_r = np.sort(rng.choice(vs, 4096, replace=False))
    ref_sel, _ = O.route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k, rows=rows_r)
    got = host(ws["sel"])
    np.testing.assert_array_equal(got[rows_r], ref_sel)
    vm = w.valid_mask()
    assert np.all(got[~vm] == -1)
    assert got[vm].min() >= 0 and got[vm].max() < w.n_blk
    assert np.all(host(o)[~vm] == 0)


@pytest.mark.parametrize("name", ["stage2", "large"])
def test_full_size_route_every_token(name):
    """Geometric routing of every token of the full-size workloads: the oracle's whole-table checker
    (exact d2 to the oracle's centroids, (d2, blk_key) order, and no unlisted block better than the
    k-th) passes on every row, and the centroids equal the oracle's."""
    import sparse_attention_feed_amd as S
    say("generate", name)
    w = wl(name)
    d = to_dev(w)
    say("route every token", name, "n_valid", w.n_valid, "n_blk", w.n_blk, "k", w.top_k)
    sel, d2, cent = S.route_geometric(d["layout"], d["pts"], w.top_k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(cent)[:, :3], O.block_centroids(w.pts, w.blk_cnt, w.blk_cap))
    nbad, first = O.check_route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, host(sel),
                                          host(d2).view(np.uint32))
    assert nbad == 0, (nbad, first)


def test_layer_at_the_block_limit_sampled():
    """The largest layout the selected branch takes: 65536 blocks (2048 bitmap words in the union
    tables), ragged counts of 1 or 2 tokens, top_k = 64 (the longest routing row): the fused layer
    on sampled tokens and routing bit-exact on a larger sample."""
    import sparse_attention_feed_amd as S
    cnt = np.random.default_rng(14).integers(1, 3, size=65536).tolist()
    w = W.custom_block_workload(14, cnt, 2, 32, 2, 32, "bf16", 64)
    d = to_dev(w)
    ws = {}
    say("layer at the block limit", w.n_blk, "blocks,", w.n_valid, "tokens, k", w.top_k)
    o = S.nsa_layer(d["layout"], d["q"], d["k"], d["v"], d["pts"], d["gates"], w.top_k, ws=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(15)
    vs = w.valid_slots()
    rows = np.sort(rng.choice(vs, 32, replace=False))
    ref = O.nsa_forward(w, rows=rows)
    assert max_err(host(o)[rows], ref) <= tol(w)
    rows_r = np.sort(rng.choice(vs, 256, replace=False))
    ref_sel, _ = O.route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k, rows=rows_r)
    np.testing.assert_array_equal(host(ws["sel"])[rows_r], ref_sel)
    assert np.all(host(o)[~w.valid_mask()] == 0)


@pytest.mark.parametrize("n_blk", [65536, 65537])
def test_local_branch_one_token_blocks(n_blk):
    """Local branch alone over one-token blocks: each token attends only itself, so o equals its
    own v row for every head of the group, exactly (one key: probability 1), and lse equals
    scale * <q, k>.  65,536 blocks take the wave-cluster kernel, 65,537 the fused kernel."""
    import sparse_attention_feed_amd as S
    w = W.custom_block_workload(16, [1] * n_blk, 1, 32, 2, 32, "bf16", 1)
    d = to_dev(w)
    lse = torch.empty((w.n_slots, w.n_qh), dtype=torch.float32, device="cuda")
    say("local branch, one-token blocks", n_blk)
    o = S.attn_fwd(d["layout"], S.BR_LOC, d["q"], d["k"], d["v"], lse=lse)
    torch.cuda.synchronize()
    grp = w.n_qh // w.n_kvh
    want = np.repeat(w.v, grp, axis=1)                     # head h reads KV head h // grp
    np.testing.assert_array_equal(host(o), want)
    ref_lse = w.scale * np.einsum("shd,shd->sh", w.q.astype(np.float64), np.repeat(w.k, grp, axis=1).astype(np.float64))
    qn = np.linalg.norm(w.q.astype(np.float64), axis=2).max()
    kn = np.linalg.norm(w.k.astype(np.float64), axis=2).max()
    # the probability is rounded to bf16 (|d ln l| <= 1.96e-3) and the pre-scaled query once to bf16
    assert max_err(host(lse), ref_lse) <= 1.96e-3 + 2.0 ** -9 * w.scale * qn * kn + 1e-4


def test_full_size_dense_sampled():
    import sparse_attention_feed_amd as S
    w = W.make("dense")
    t = {k: torch.from_numpy(getattr(w, k)).cuda().to(torch.bfloat16) for k in ("q", "k", "v", "gates")}
    say("dense full size", w.n_tok)
    o = S.dense_gated_xattn(t["q"], t["k"], t["v"], w.n_x, t["gates"])
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(3).choice(w.n_tok, 96, replace=False))
    ref = O.dense_gated_xattn(w.q, w.k, w.v, w.n_x, w.gates, w.scale, rows=rows)
    assert max_err(host(o)[rows], ref) <= 2e-2


# ---------------------------------------------------------------------------------------------
# reproducibility and storage-order invariance
# ---------------------------------------------------------------------------------------------

def test_ring_wait_bound_ends_with_nan(monkeypatch):
    """The selected branch's tile ring waits only a bounded time.  A test hook makes it wait for a
    count that never arrives: the kernel still completes and the branch output is NaN (no hang);
    without the hook the same call matches the oracle."""
    import sparse_attention_feed_amd as S
    w = wl("stage2_small")
    d = to_dev(w)
    sel_ref, _ = O.route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k)
    sel = torch.from_numpy(sel_ref).cuda()
    vm = w.valid_mask()
    monkeypatch.setenv("NSA_TEST_RING_STALL", "1")
    say("ring stall hook")
    o = S.attn_fwd(d["layout"], S.BR_SEL, d["q"], d["k"], d["v"], sel=sel, top_k=w.top_k)
    torch.cuda.synchronize()
    assert np.all(np.isnan(host(o)[vm]))
    monkeypatch.delenv("NSA_TEST_RING_STALL")
    say("ring normal")
    o = S.attn_fwd(d["layout"], S.BR_SEL, d["q"], d["k"], d["v"], sel=sel, top_k=w.top_k)
    torch.cuda.synchronize()
    ref, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel_ref)
    assert max_err(host(o), ref) <= tol(w)


@pytest.mark.parametrize("name", ["stage2_small", "k48_cap16", "ragged_cap16", "k64_cap8_bf16", "cap1_bf16",
                                  "ragged_cap64_bf16", "k_beyond_blocks", "single_block"])
def test_selected_branch_paths_agree(name, monkeypatch):
    """bf16 token queries take the selected branch to its own kernel (wave-owned token clusters)
    after the fused kernel's other branches; NSA_SEL_RING=1 keeps it in the fused kernel's tile
    ring.  Both orders of the same sums meet the oracle, alone and in the gated three-branch layer,
    and agree with each other to bf16 rounding of the output."""
    import sparse_attention_feed_amd as S
    w = get(name)
    d = to_dev(w)
    kc, vc, sel, kc_d, vc_d, sel_d = _branch_inputs(w, d)
    ref_sel = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel)[0]
    ref_outs = [O.attn_branch(O.CMP, w.q, kc.astype(np.float64), vc.astype(np.float64), w.blk_cnt, w.blk_cap,
                              w.scale)[0], ref_sel,
                O.attn_branch(O.LOC, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale)[0]]
    ref = O.gate_combine(ref_outs, w.gates)
    res = {}
    for ring in ("0", "1"):
        monkeypatch.setenv("NSA_SEL_RING", ring)
        say("selected branch path", name, "ring", ring)
        o1 = S.attn_fwd(d["layout"], S.BR_SEL, d["q"], d["k"], d["v"], sel=sel_d, top_k=w.top_k)
        o3 = S.attn_fwd(d["layout"], 7, d["q"], d["k"], d["v"], k_cmp=kc_d, v_cmp=vc_d, sel=sel_d,
                        top_k=w.top_k, gates=d["gates"])
        torch.cuda.synchronize()
        res[ring] = (host(o1), host(o3))
        assert max_err(res[ring][0], ref_sel) <= tol(w)
        assert max_err(res[ring][1], ref) <= tol(w)
        vm = w.valid_mask()
        assert np.all(res[ring][0][~vm] == 0) and np.all(res[ring][1][~vm] == 0)
    monkeypatch.delenv("NSA_SEL_RING")
    assert max_err(res["0"][0], res["1"][0]) <= 2.0 ** -7
    assert max_err(res["0"][1], res["1"][1]) <= 2.0 ** -6


def test_repeat_runs_bit_identical():
    import sparse_attention_feed_amd as S
    w = wl("large_small")
    d = to_dev(w)
    say("determinism large_small")
    o1 = S.nsa_layer(d["layout"], d["q"], d["k"], d["v"], d["pts"], d["gates"], w.top_k).clone()
    o2 = S.nsa_layer(d["layout"], d["q"], d["k"], d["v"], d["pts"], d["gates"], w.top_k)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_storage_permutation_invariance_gpu():
    import sparse_attention_feed_amd as S
    w = wl("stage2_small")
    w2, smap = W.permute_storage(w, seed=5)
    outs = []
    for ww in (w, w2):
        d = to_dev(ww)
        say("permutation", ww.n_blk)
        ws = {}
        o = S.nsa_layer(d["layout"], d["q"], d["k"], d["v"], d["pts"], d["gates"], ww.top_k, ws=ws)
        torch.cuda.synchronize()
        outs.append((host(o), host(ws["sel"])))
    new = np.nonzero(smap >= 0)[0]
    assert max_err(outs[1][0][new], outs[0][0][smap[new]]) <= 2e-2
    k1 = w.blk_key[outs[0][1][smap[new]]]
    k2 = w2.blk_key[outs[1][1][new]]
    np.testing.assert_array_equal(k1, k2)
