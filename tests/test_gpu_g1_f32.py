"""GPU parity of the score-routed, block-granular path in fp32 (one query head per KV head, head
dim 64): score routing, the three branches, the forced range, the fused entry point and the whole
layer, against the fp64 oracle.  Bars: routing rows bit-exact on integer inputs and epsilon ties
(relative 1e-4, fp32 scores) on random ones; outputs max-abs 1e-4; lse 1e-4."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import host, max_err, say, to_dev
from test_gpu_speed3r import check_eps_ties

pytestmark = pytest.mark.gpu
TOL = 1e-4
H = 4                       # query heads = KV heads


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def case(seed, n_blk, k, branches=("cmp", "sel"), n_gate=2):
    """Ragged block counts (1..16 of 16 slots), n_blk spanning several 64-key tiles."""
    rng = np.random.default_rng(seed)
    cnt = rng.integers(1, 17, size=n_blk)
    return W.custom_block_workload(300 + seed, cnt, 16, H, H, 64, "f32", k, routing="scores", q_gran="block",
                                   branches=branches, n_gate=n_gate)


def pooled(w):
    """The oracle's block means, stored in fp32 as the device stores its own."""
    return [O.pool_blocks(x, w.blk_cnt, w.blk_cap).astype(np.float32) for x in (w.q, w.k, w.v)]


def test_f32_pooling_block_queries():
    import sparse_attention_feed_amd as S
    w = case(1, 150, 16)
    d = to_dev(w)
    say("pool f32 g1")
    for x, ref in zip((d["q"], d["k"], d["v"]), pooled(w)):
        got = host(S.pool_blocks(d["layout"], x))
        # fp32 accumulation of at most 16 values against the fp64 mean
        assert np.all(np.abs(got - ref) <= 1e-6 * np.maximum(1.0, np.abs(ref))), max_err(got, ref)


@pytest.mark.parametrize("n_blk,k", [(150, 16), (150, 5), (150, 32), (150, 40), (10, 16), (1, 8), (77, 64)])
def test_f32_routing_exact_on_integer_inputs(n_blk, k):
    """Small-integer pooled queries and keys: every fp32 score is exact, so the ranking is bit-exact,
    ties (resolved by blk_key) included; every list size (k <= 8, 16, 32, 64), fewer blocks than k."""
    import sparse_attention_feed_amd as S
    w = case(2 + n_blk, n_blk, k)
    d = to_dev(w)
    rng = np.random.default_rng(n_blk + k)
    qc = rng.integers(-2, 3, size=(n_blk, H, 64)).astype(np.float32)
    kc = rng.integers(-2, 3, size=(n_blk, H, 64)).astype(np.float32)
    say("route_g1 f32 exact", n_blk, k)
    sel = S.route_scores_topk(d["layout"], dev(qc), dev(kc), None, k, q_gran=S.Q_BLOCK)
    torch.cuda.synchronize()
    ref_sel, _ = O.route_scores(qc, kc, w.blk_key, w.scale, k)
    np.testing.assert_array_equal(host(sel), ref_sel)


def test_f32_routing_eps_ties():
    import sparse_attention_feed_amd as S
    w = case(3, 200, 16)
    d = to_dev(w)
    qc, kc, _ = pooled(w)
    say("route_g1 f32 random")
    sel = S.route_scores_topk(d["layout"], dev(qc), dev(kc), None, w.top_k, q_gran=S.Q_BLOCK)
    torch.cuda.synchronize()
    ref_sel, imp = O.route_scores(qc, kc, w.blk_key, w.scale, w.top_k)
    frac = check_eps_ties(host(sel), ref_sel, imp, w.top_k, 1e-4)
    assert frac >= 0.99, frac


@pytest.mark.parametrize("branch", ["cmp", "sel", "loc"])
def test_f32_single_branch(branch):
    import sparse_attention_feed_amd as S
    w = case(4, 150, 16)
    d = to_dev(w)
    qc, kc, vc = pooled(w)
    sel, _ = O.route_scores(qc, kc, w.blk_key, w.scale, w.top_k)
    rows = w.n_blk if branch == "cmp" else w.n_slots
    lse = torch.empty((rows, H), dtype=torch.float32, device="cuda")
    bit = {"cmp": S.BR_CMP, "sel": S.BR_SEL, "loc": S.BR_LOC}[branch]
    say("attn_g1 f32", branch)
    o = S.attn_fwd(d["layout"], bit, d["q"], d["k"], d["v"], q_cmp=dev(qc), k_cmp=dev(kc), v_cmp=dev(vc),
                   sel=torch.from_numpy(sel).cuda(), top_k=w.top_k, sel_groups=H, lse=lse, q_gran=S.Q_BLOCK)
    torch.cuda.synchronize()
    vm = w.valid_mask()
    gl = host(lse)
    if branch == "cmp":
        ref, _ = O.attn_branch(O.CMP, qc, kc, vc, w.blk_cnt, w.blk_cap, w.scale, q_gran="block")
        ref_lse = np.stack([O.attend(qc[b], kc, vc, w.scale)[1] for b in range(w.n_blk)])
        assert max_err(gl, ref_lse) <= TOL
    else:
        if branch == "sel":
            ref, ref_lse = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel,
                                         q_gran="block")
        else:
            ref, ref_lse = O.attn_branch(O.LOC, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale)
        assert np.all(np.isneginf(gl[~vm]))
        assert max_err(gl[vm], ref_lse[vm]) <= TOL
    got = host(o)
    assert max_err(got, ref) <= TOL
    assert np.all(got[~vm] == 0)


@pytest.mark.parametrize("lo,hi,k,n_blk", [(0, 0, 40, 150), (13, 147, 16, 151), (60, 61, 8, 149)])
def test_f32_selected_rows_repeats_gaps_forced(lo, hi, k, n_blk):
    """Routing rows with repeated entries, -1 and whole empty rows; k = 40 packs several 64-key tiles;
    forced ranges that span the sequence or hold one block; block counts that leave the last wave of
    the forced kernel (two query blocks per wave in fp32) with one block."""
    import sparse_attention_feed_amd as S
    w = case(5 + k, n_blk, k)
    d = to_dev(w)
    rng = np.random.default_rng(lo + hi + k)
    sel = rng.integers(-1, w.n_blk, size=(w.n_blk, H, k)).astype(np.int32)
    sel[:, :, 1] = sel[:, :, 0]
    sel[::5, :, 2] = lo
    sel[::7, :, :] = -1
    say("sel_g1 f32", lo, hi, k)
    o = S.attn_fwd(d["layout"], S.BR_SEL, d["q"], d["k"], d["v"], sel=torch.from_numpy(sel).cuda(), top_k=k,
                   sel_groups=H, q_gran=S.Q_BLOCK, forced=(lo, hi) if hi > lo else None)
    torch.cuda.synchronize()
    ref, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel, q_gran="block",
                           forced=(lo, hi) if hi > lo else None)
    assert max_err(host(o), ref) <= TOL


def test_f32_three_branch_layer():
    """The whole layer on the device (pooling, score routing, three gated branches) against the
    oracle's layer from the same inputs (its own pooling and routing), on every valid token of the
    (block, head) pairs whose routing rows agree; the rows must agree on nearly all pairs."""
    import sparse_attention_feed_amd as S
    w = case(6, 150, 16, branches=("cmp", "sel", "loc"), n_gate=3)
    d = to_dev(w)
    L = d["layout"]
    say("layer g1 f32")
    qd, kd, vd = S.pool_blocks(L, d["q"]), S.pool_blocks(L, d["k"]), S.pool_blocks(L, d["v"])
    sel = S.route_scores_topk(L, qd, kd, None, w.top_k, q_gran=S.Q_BLOCK)
    o = S.attn_fwd(L, S.BR_CMP | S.BR_SEL | S.BR_LOC, d["q"], d["k"], d["v"], q_cmp=qd, k_cmp=kd, v_cmp=vd,
                   sel=sel, top_k=w.top_k, sel_groups=H, gates=d["gates"], q_gran=S.Q_BLOCK)
    torch.cuda.synchronize()
    ref, parts = O.nsa_forward(w, return_parts=True)
    ref_sel = parts["sel"]
    same = np.all(host(sel) == ref_sel, axis=2)                     # [n_blk, H]
    assert same.mean() >= 0.99, same.mean()
    vm = w.valid_mask()
    blk = np.arange(w.n_slots) // w.blk_cap
    agree = same[blk] & vm[:, None]
    got = host(o)
    assert np.abs(got - ref).max(axis=2)[agree].max() <= TOL
    assert np.all(got[~vm] == 0)


@pytest.mark.parametrize("n_blk,k", [(150, 16), (77, 32), (10, 16), (130, 5)])
def test_f32_scores_routed_entry_point(n_blk, k):
    """nsa_attn_fwd_scores_routed in fp32 is the routing pass followed by the two branches: the same
    routing rows and the same output bits as the two calls, and the oracle's steps on the device's
    pooled values agree to the fp32 bar."""
    import sparse_attention_feed_amd as S
    w = case(7 + n_blk, n_blk, k)
    d = to_dev(w)
    L = d["layout"]
    qd, kd, vd = S.pool_blocks(L, d["q"]), S.pool_blocks(L, d["k"]), S.pool_blocks(L, d["v"])
    say("scores_routed f32", n_blk, k)
    o_f, sel_f = S.attn_fwd_scores_routed(L, d["q"], d["k"], d["v"], qd, kd, vd, k, d["gates"])
    sel_2 = S.route_scores_topk(L, qd, kd, None, k, q_gran=S.Q_BLOCK)
    o_2 = S.attn_fwd(L, S.BR_CMP | S.BR_SEL, d["q"], d["k"], d["v"], q_cmp=qd, k_cmp=kd, v_cmp=vd, sel=sel_2,
                     top_k=k, sel_groups=H, gates=d["gates"], q_gran=S.Q_BLOCK)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(sel_f), host(sel_2))
    np.testing.assert_array_equal(host(o_f), host(o_2))
    qc, kc, vc = host(qd), host(kd), host(vd)
    o_cmp, _ = O.attn_branch(O.CMP, qc, kc, vc, w.blk_cnt, w.blk_cap, w.scale, q_gran="block")
    o_sel, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=host(sel_f), q_gran="block")
    ref = O.gate_combine([o_cmp, o_sel], w.gates)
    assert max_err(host(o_f), ref) <= TOL
