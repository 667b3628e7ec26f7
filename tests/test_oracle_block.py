"""Pins of the oracle's block-granular paths, its score routing and its whole-table routing checker.

Block-granular queries (the Speed3R form: pooled queries for the compressed branch, one routing row
per query block, token queries for the selected branch) are checked against a hand-worked fixture
and against torch's attention on torch-pooled tensors.  Grouped-query score routing is checked
against torch's softmax probabilities (no lse involved).  The geometric-routing checker is checked
on correct tables and on tables with planted mistakes.  The fp64 volume selection is checked
against scipy's trilinear interpolation.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa(q, k, v, scale):
    """torch attention, float64 on the CPU: q [n, Hq, D], k/v [m, Hkv, D] -> [n, Hq, D]."""
    G = q.shape[1] // k.shape[1]
    tq = torch.from_numpy(np.asarray(q, dtype=np.float64)).permute(1, 0, 2)
    tk = torch.from_numpy(np.asarray(k, dtype=np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)
    tv = torch.from_numpy(np.asarray(v, dtype=np.float64)).permute(1, 0, 2).repeat_interleave(G, dim=0)
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale).permute(1, 0, 2).numpy()


def torch_pool(x, blk_cnt, cap):
    """Block means by a torch scatter-add over the valid slots."""
    blk_cnt = np.asarray(blk_cnt)
    S = blk_cnt.shape[0] * cap
    slot = np.arange(S)
    vs = slot[(slot % cap) < blk_cnt[slot // cap]]
    seg = torch.from_numpy(vs // cap)
    acc = torch.zeros((blk_cnt.shape[0],) + x.shape[1:], dtype=torch.float64)
    acc.index_add_(0, seg, torch.from_numpy(np.asarray(x, dtype=np.float64)[vs]))
    return (acc / torch.from_numpy(blk_cnt.astype(np.float64))[:, None, None]).numpy()


def _val(x):
    if isinstance(x, str):
        if x in ("inf", "-inf"):
            return float(x)
        if x.startswith("ln"):
            return math.log(float(x[2:]))
        return float(Fraction(x))
    return float(x)


def _arr(a):
    return np.vectorize(_val, otypes=[np.float64])(np.array(a, dtype=object))


# ---------------------------------------------------------------------------------------------
# hand-worked fixture: two blocks, two heads, block-granular queries, score routing
# ---------------------------------------------------------------------------------------------

def _hand_workload():
    fx = json.load(open(os.path.join(GOLDEN, "nsa_block_queries_hand.json"), encoding="utf-8"))
    L = fx["layout"]
    f32 = lambda a: _arr(a).astype(np.float32)      # noqa: E731  (every input value is exact in fp32)
    cnt = np.array(L["blk_cnt"], dtype=np.int32)
    w = W.Workload(name="hand", dtype="f32", n_qh=L["n_qh"], n_kvh=L["n_kvh"], head_dim=L["head_dim"],
                   blk_cap=L["cap"], blk_cnt=cnt, blk_key=np.array(L["blk_key"], dtype=np.uint32),
                   blk_type=np.ones(cnt.shape[0], dtype=np.int8), pts=np.zeros((4, 3), np.float32),
                   q=f32(fx["q"]), k=f32(fx["k"]), v=f32(fx["v"]), gates=f32(fx["gates"]), top_k=L["top_k"],
                   routing="scores", q_gran="block", branches=("cmp", "sel"), meta={"scale": math.log(3.0)})
    return w, fx


def test_block_queries_hand_fixture():
    w, fx = _hand_workload()
    o, parts = O.nsa_forward(w, return_parts=True)
    np.testing.assert_allclose(parts["q_cmp"], _arr(fx["q_cmp"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(parts["k_cmp"], _arr(fx["k_cmp"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(parts["v_cmp"], _arr(fx["v_cmp"]), rtol=0, atol=1e-15)
    assert parts["sel"].tolist() == fx["sel"]
    np.testing.assert_allclose(parts["o_cmp"], _arr(fx["o_cmp"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(parts["o_sel"], _arr(fx["o_sel_fractions"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(parts["lse_cmp"], _arr(fx["lse_cmp_ln"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(parts["lse_sel"], _arr(fx["lse_sel_ln"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o, _arr(fx["o_fractions"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o, np.array(fx["o"]), rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------------------------
# block-granular branches against torch
# ---------------------------------------------------------------------------------------------

def _block_case(seed=31, H=3, D=8, cap=4, top_k=3):
    cnt = [4, 1, 3, 4, 2, 4, 1, 3, 4, 2]
    return W.custom_block_workload(seed, cnt, cap, H, H, D, "f32", top_k, routing="scores", q_gran="block",
                                   branches=("cmp", "sel"))


def test_cmp_block_queries_against_torch():
    """Compressed branch with pooled queries: torch attention of the torch-pooled query of each block
    over the torch-pooled keys and values, given to every valid token of that block."""
    w = _block_case()
    qc = torch_pool(w.q, w.blk_cnt, w.blk_cap)
    kc = torch_pool(w.k, w.blk_cnt, w.blk_cap)
    vc = torch_pool(w.v, w.blk_cnt, w.blk_cap)
    ref_blk = sdpa(qc, kc, vc, w.scale)                                  # [n_blk, H, D]
    # the pooled queries differ from block to block, so a wrong-block broadcast cannot pass
    assert np.abs(ref_blk[1:] - ref_blk[:-1]).max(axis=(1, 2)).min() > 1e-3
    o, lse = O.attn_branch(O.CMP, O.pool_blocks(w.q, w.blk_cnt, w.blk_cap), O.pool_blocks(w.k, w.blk_cnt, w.blk_cap),
                           O.pool_blocks(w.v, w.blk_cnt, w.blk_cap), w.blk_cnt, w.blk_cap, w.scale, q_gran="block")
    vm = w.valid_mask()
    for s in range(w.n_slots):
        if vm[s]:
            np.testing.assert_allclose(o[s], ref_blk[s // w.blk_cap], rtol=0, atol=1e-13)
        else:
            assert np.all(o[s] == 0) and np.all(lse[s] == -np.inf)


def test_sel_block_rows_against_torch():
    """Selected branch with one routing row per (query block, KV head): every valid token of block b
    attends, for head h, the valid tokens of the distinct blocks of row [b, h]; torch attention over
    the concatenated key sets.  Rows differ per block, and the slot count exceeds the block count,
    so reading the row of the slot index instead of its block fails."""
    w = _block_case(seed=32)
    rng = np.random.default_rng(33)
    sel = np.full((w.n_blk, w.n_kvh, w.top_k), -1, dtype=np.int32)
    for b in range(w.n_blk):
        for h in range(w.n_kvh):
            n = 1 + (b + h) % w.top_k
            sel[b, h, :n] = rng.choice(w.n_blk, n, replace=False)
    sel[3, 1, 0] = sel[3, 1, 1] = 6                                      # a duplicate counts once
    sel[3, 1, 2] = -1
    assert w.n_slots > w.n_blk
    o, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel, q_gran="block")
    n_checked = 0
    for s in w.valid_slots():
        b = s // w.blk_cap
        for h in range(w.n_kvh):
            blocks = sorted(set(int(x) for x in sel[b, h] if x >= 0))
            ks = np.concatenate([np.arange(x * w.blk_cap, x * w.blk_cap + w.blk_cnt[x]) for x in blocks])
            ref = sdpa(w.q[s:s + 1, h:h + 1], w.k[ks][:, h:h + 1], w.v[ks][:, h:h + 1], w.scale)
            np.testing.assert_allclose(o[s, h], ref[0, 0], rtol=0, atol=1e-13)
            n_checked += 1
    assert n_checked == w.n_valid * w.n_kvh
    # slot s < n_blk of another block is among the checked rows with a different row of its own
    assert any(s // w.blk_cap != s and not np.array_equal(sel[s], sel[s // w.blk_cap]) for s in w.valid_slots()
               if s < w.n_blk)


def test_score_routed_layer_block_queries_against_torch():
    """The whole Speed3R-form layer: torch-pooled q, k, v; routing by a plain sort of the pooled dot
    products (ties by key); torch attention for both branches; sigmoid gates."""
    w = _block_case(seed=34, top_k=2)
    o, parts = O.nsa_forward(w, return_parts=True)
    qc, kc, vc = (torch_pool(x, w.blk_cnt, w.blk_cap) for x in (w.q, w.k, w.v))
    g = 1.0 / (1.0 + np.exp(-w.gates.astype(np.float64)))
    ocmp = sdpa(qc, kc, vc, w.scale)
    for s in w.valid_slots():
        b = s // w.blk_cap
        for h in range(w.n_kvh):
            sc = [(-(qc[b, h] @ kc[x, h]), int(w.blk_key[x]), x) for x in range(w.n_blk)]
            blocks = sorted(x for _, _, x in sorted(sc)[:w.top_k])
            assert sorted(parts["sel"][b, h].tolist()) == blocks
            ks = np.concatenate([np.arange(x * w.blk_cap, x * w.blk_cap + w.blk_cnt[x]) for x in blocks])
            osel = sdpa(w.q[s:s + 1, h:h + 1], w.k[ks][:, h:h + 1], w.v[ks][:, h:h + 1], w.scale)[0, 0]
            ref = g[s, h, 0] * ocmp[b, h] + g[s, h, 1] * osel
            np.testing.assert_allclose(o[s, h], ref, rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------------------------
# grouped-query score routing against torch softmax probabilities
# ---------------------------------------------------------------------------------------------

def _gqa_case(seed=41, top_k=3):
    return W.custom_block_workload(seed, [5, 8, 1, 3, 8, 6, 2, 7], 8, 4, 2, 8, "f32", top_k, routing="scores",
                                   q_gran="token", branches=("cmp", "sel", "loc"))


def _torch_group_importance(w, rows, kc):
    """Summed softmax probability of each KV group's heads over all pooled blocks (torch softmax,
    no lse): [R, Hkv, n_blk]."""
    G = w.n_qh // w.n_kvh
    q = torch.from_numpy(w.q[rows].astype(np.float64))                        # [R, Hq, D]
    k = torch.from_numpy(kc).repeat_interleave(G, dim=1)                      # [n_blk, Hq, D]
    p = torch.softmax(w.scale * torch.einsum("rhd,bhd->rhb", q, k), dim=2)     # [R, Hq, n_blk]
    return p.reshape(len(rows), w.n_kvh, G, -1).sum(2).numpy()


def test_gqa_score_routing_equals_torch_softmax_ranking():
    w = _gqa_case()
    vs = w.valid_slots()
    kc = torch_pool(w.k, w.blk_cnt, w.blk_cap)
    vc = torch_pool(w.v, w.blk_cnt, w.blk_cap)
    _, lse = O.attn_branch(O.CMP, w.q, kc, vc, w.blk_cnt, w.blk_cap, w.scale, rows=vs)
    sel, imp = O.route_scores(w.q[vs], kc, w.blk_key, w.scale, w.top_k, lse=lse)
    ref = _torch_group_importance(w, vs, kc)
    np.testing.assert_allclose(imp, ref, rtol=0, atol=1e-13)
    for i in range(len(vs)):
        for j in range(w.n_kvh):
            order = sorted(range(w.n_blk), key=lambda b: (-ref[i, j, b], int(w.blk_key[b])))
            assert sel[i, j].tolist() == order[:w.top_k]


def test_nsa_forward_gqa_score_routing_against_torch():
    """nsa_forward with score routing under grouped-query attention: per (token, group) selection by
    the torch softmax ranking, and each branch by torch attention."""
    w = _gqa_case(seed=42)
    o, parts = O.nsa_forward(w, return_parts=True)
    vs = w.valid_slots()
    kc = torch_pool(w.k, w.blk_cnt, w.blk_cap)
    vc = torch_pool(w.v, w.blk_cnt, w.blk_cap)
    imp = _torch_group_importance(w, vs, kc)
    g = 1.0 / (1.0 + np.exp(-w.gates.astype(np.float64)))
    G = w.n_qh // w.n_kvh
    ocmp = sdpa(w.q[vs], kc, vc, w.scale)
    for i, s in enumerate(vs):
        b = s // w.blk_cap
        own = np.arange(b * w.blk_cap, b * w.blk_cap + w.blk_cnt[b])
        oloc = sdpa(w.q[s:s + 1], w.k[own], w.v[own], w.scale)[0]
        for j in range(w.n_kvh):
            order = sorted(range(w.n_blk), key=lambda x: (-imp[i, j, x], int(w.blk_key[x])))[:w.top_k]
            assert parts["sel"][s, j].tolist() == order
            ks = np.concatenate([np.arange(x * w.blk_cap, x * w.blk_cap + w.blk_cnt[x]) for x in sorted(order)])
            hs = slice(j * G, (j + 1) * G)
            osel = sdpa(w.q[s:s + 1, hs], w.k[ks][:, j:j + 1], w.v[ks][:, j:j + 1], w.scale)[0]
            ref = g[s, hs, 0:1] * ocmp[i, hs] + g[s, hs, 1:2] * osel + g[s, hs, 2:3] * oloc[hs]
            np.testing.assert_allclose(o[s, hs], ref, rtol=0, atol=1e-13)
    assert np.all(parts["sel"][~w.valid_mask()] == -1)
    assert np.all(o[~w.valid_mask()] == 0)


def test_nsa_forward_gqa_scores_all_blocks_is_dense():
    w = _gqa_case(seed=43, top_k=8)
    w.gates = np.zeros_like(w.gates)
    w.gates[..., 0] = -np.inf
    w.gates[..., 1] = np.inf
    w.gates[..., 2] = -np.inf
    o = O.nsa_forward(w)
    vs = w.valid_slots()
    np.testing.assert_allclose(o[vs], sdpa(w.q[vs], w.k[vs], w.v[vs], w.scale), rtol=0, atol=1e-12)


def _gqa_block_case(seed=44, top_k=3):
    return W.custom_block_workload(seed, [5, 8, 1, 3, 8, 6, 2, 7], 8, 4, 2, 8, "f32", top_k, routing="scores",
                                   q_gran="block", branches=("cmp", "sel", "loc"))


def test_nsa_forward_gqa_block_queries_against_torch():
    """Grouped-query attention with pooled query rows: routing per (query block, KV group) by the
    torch softmax ranking of the torch-pooled query, the compressed branch as torch attention of
    that pooled query given to each valid token, the selected branch per token over its block's
    row, the local branch per token."""
    w = _gqa_block_case()
    o, parts = O.nsa_forward(w, return_parts=True)
    qc = torch_pool(w.q, w.blk_cnt, w.blk_cap)
    kc = torch_pool(w.k, w.blk_cnt, w.blk_cap)
    vc = torch_pool(w.v, w.blk_cnt, w.blk_cap)
    G = w.n_qh // w.n_kvh
    k = torch.from_numpy(kc).repeat_interleave(G, dim=1)
    p = torch.softmax(w.scale * torch.einsum("rhd,bhd->rhb", torch.from_numpy(qc), k), dim=2)
    imp = p.reshape(w.n_blk, w.n_kvh, G, -1).sum(2).numpy()            # [n_blk, Hkv, n_blk]
    ocmp = sdpa(qc, kc, vc, w.scale)                                    # [n_blk, Hq, D]
    g = 1.0 / (1.0 + np.exp(-w.gates.astype(np.float64)))
    assert parts["sel"].shape == (w.n_blk, w.n_kvh, w.top_k)
    for b in range(w.n_blk):
        for j in range(w.n_kvh):
            order = sorted(range(w.n_blk), key=lambda x: (-imp[b, j, x], int(w.blk_key[x])))[:w.top_k]
            assert parts["sel"][b, j].tolist() == order
    for s in w.valid_slots():
        b = s // w.blk_cap
        own = np.arange(b * w.blk_cap, b * w.blk_cap + w.blk_cnt[b])
        oloc = sdpa(w.q[s:s + 1], w.k[own], w.v[own], w.scale)[0]
        for j in range(w.n_kvh):
            blocks = sorted(parts["sel"][b, j].tolist())
            ks = np.concatenate([np.arange(x * w.blk_cap, x * w.blk_cap + w.blk_cnt[x]) for x in blocks])
            hs = slice(j * G, (j + 1) * G)
            osel = sdpa(w.q[s:s + 1, hs], w.k[ks][:, j:j + 1], w.v[ks][:, j:j + 1], w.scale)[0]
            ref = g[s, hs, 0:1] * ocmp[b, hs] + g[s, hs, 1:2] * osel + g[s, hs, 2:3] * oloc[hs]
            np.testing.assert_allclose(o[s, hs], ref, rtol=0, atol=1e-13)
    assert np.all(o[~w.valid_mask()] == 0)


def test_nsa_forward_gqa_block_equals_token_rows_when_queries_repeat():
    """When every token of a block carries the same query, the pooled query is that query, so
    block-granular rows give exactly the per-token layer (routing rows repeated per token)."""
    w = _gqa_block_case(seed=45)
    for b in range(w.n_blk):
        w.q[b * w.blk_cap:(b + 1) * w.blk_cap] = w.q[b * w.blk_cap]
    ob, pb = O.nsa_forward(w, return_parts=True)
    w.q_gran = "token"
    ot, pt = O.nsa_forward(w, return_parts=True)
    np.testing.assert_allclose(ob, ot, rtol=0, atol=1e-14)
    vs = w.valid_slots()
    np.testing.assert_array_equal(pt["sel"][vs], pb["sel"][vs // w.blk_cap])


# ---------------------------------------------------------------------------------------------
# the whole-table score routing checker (one query head per KV head)
# ---------------------------------------------------------------------------------------------

def _score_case(seed, n_blk=300, rows=48, heads=3, d=16, integer=False):
    rng = np.random.default_rng(seed)
    if integer:
        q = rng.integers(-1, 2, size=(rows, heads, d)).astype(np.float64)
        k = rng.integers(-1, 2, size=(n_blk, heads, d)).astype(np.float64)
    else:
        q = rng.standard_normal((rows, heads, d))
        k = rng.standard_normal((n_blk, heads, d))
    key = rng.permutation(np.arange(n_blk, dtype=np.uint32) * 5 + 1)
    return q, k, key


@pytest.mark.parametrize("case", ["random", "integer_ties", "k_beyond"])
def test_score_checker_accepts_the_definition(case):
    q, k, key = _score_case(61, integer=case == "integer_ties", n_blk=5 if case == "k_beyond" else 300)
    top_k = 8
    sel, _ = O.route_scores(q, k, key, 1.0, top_k)
    n_bad, n_exact, _ = O.check_route_scores(q, k, key, sel, 1e-6, chunk=7)
    assert n_bad == 0 and n_exact == q.shape[0] * q.shape[1]


def test_score_checker_tolerates_only_near_ties():
    """Two adjacent entries swapped pass (not as exact) when their scores lie within eps of each
    other, and fail when they do not."""
    q, k, key = _score_case(62)
    sel, imp = O.route_scores(q, k, key, 1.0, 8)
    r, h = 5, 1
    s = imp[r, h]
    a, b = sel[r, h, 3], sel[r, h, 4]
    gap = (s[a] - s[b]) / abs(s[sel[r, h, 7]])
    sel[r, h, [3, 4]] = sel[r, h, [4, 3]]
    n_bad, n_exact, _ = O.check_route_scores(q, k, key, sel, 2 * gap)
    assert n_bad == 0 and n_exact == q.shape[0] * q.shape[1] - 1
    n_bad, _, first = O.check_route_scores(q, k, key, sel, gap / 2)
    assert n_bad == 1 and first == [(r, h)]


@pytest.mark.parametrize("mistake", ["swap_ends", "worse_block", "duplicate", "out_of_range", "tail", "skip_best"])
def test_score_checker_rejects_planted_mistakes(mistake):
    q, k, key = _score_case(63, n_blk=6 if mistake == "tail" else 300)
    top_k = 8
    sel, imp = O.route_scores(q, k, key, 1.0, top_k)
    r, h = 7, 2
    s = imp[r, h]
    if mistake == "swap_ends":
        sel[r, h, [0, 5]] = sel[r, h, [5, 0]]
    elif mistake == "worse_block":
        sel[r, h, -1] = int(np.argmin(s))
    elif mistake == "duplicate":
        sel[r, h, 4] = sel[r, h, 3]
    elif mistake == "out_of_range":
        sel[r, h, 2] = k.shape[0]
    elif mistake == "tail":                    # k beyond the block count: the tail stays -1
        assert top_k > k.shape[0]
        sel[r, h, -1] = int(sel[r, h, 0])
    elif mistake == "skip_best":               # the best block left out, the rest moved up
        sel[r, h, :-1] = sel[r, h, 1:].copy()
        sel[r, h, -1] = int(np.argsort(-s, kind="stable")[top_k])
    n_bad, _, first = O.check_route_scores(q, k, key, sel, 1e-6, chunk=5)
    assert n_bad == 1 and first == [(r, h)]


def _grouped_score_case(seed, n_blk=120, rows=40, hkv=2, g=4, d=8, top_k=6):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((rows, hkv * g, d))
    k = rng.standard_normal((n_blk, hkv, d))
    key = rng.permutation(np.arange(n_blk, dtype=np.uint32) * 3 + 2)
    scale = 0.35
    valid = np.ones(rows, dtype=bool)
    valid[::7] = False
    # the compressed branch's lse of each row (attention over every pooled block)
    lse = np.stack([O.attend(q[r], k, k, scale)[1] for r in range(rows)])
    sel, imp = O.route_scores(q, k, key, scale, top_k, lse=lse, row_valid=valid)
    return q, k, key, scale, valid, sel, imp


@pytest.mark.parametrize("n_blk", [120, 5])
def test_grouped_score_checker_accepts_the_definition(n_blk):
    """Several query heads per KV head: the checker's own importances (softmax over all blocks,
    summed over the group) agree with route_scores fed the compressed branch's lse; padding rows
    hold -1; k beyond the block count leaves a -1 tail."""
    q, k, key, scale, valid, sel, _ = _grouped_score_case(64, n_blk=n_blk)
    n_bad, n_exact, _ = O.check_route_scores(q, k, key, sel, 1e-9, chunk=9, scale=scale, row_valid=valid)
    assert n_bad == 0 and n_exact == int(valid.sum()) * k.shape[1]


@pytest.mark.parametrize("mistake", ["swap_ends", "worse_block", "duplicate", "padding_filled"])
def test_grouped_score_checker_rejects_planted_mistakes(mistake):
    q, k, key, scale, valid, sel, imp = _grouped_score_case(65)
    r, j = 3, 1
    if mistake == "swap_ends":
        sel[r, j, [0, 5]] = sel[r, j, [5, 0]]
    elif mistake == "worse_block":
        sel[r, j, -1] = int(np.argmin(imp[r, j]))
    elif mistake == "duplicate":
        sel[r, j, 2] = sel[r, j, 1]
    else:
        r = int(np.nonzero(~valid)[0][1])
        sel[r, j, 0] = 0
    n_bad, _, first = O.check_route_scores(q, k, key, sel, 1e-9, chunk=9, scale=scale, row_valid=valid)
    assert n_bad == 1 and first == [(r, j)]


# ---------------------------------------------------------------------------------------------
# the whole-table geometric routing checker
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("case", ["random", "lattice", "k_beyond"])
def test_route_checker_accepts_the_definition(case):
    if case == "random":
        w = W.custom_block_workload(51, np.random.default_rng(1).integers(1, 17, 40).tolist(), 16, 4, 2, 8, "f32", 6)
    elif case == "lattice":
        w = W.custom_block_workload(52, [1] * 60, 1, 4, 2, 8, "f32", 9, pts_mode="lattice")
    else:
        w = W.custom_block_workload(53, [3, 7, 1], 8, 4, 2, 8, "f32", 5)
    sel, d2 = O.route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k)
    nbad, _ = O.check_route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, sel, d2, chunk=7)
    assert nbad == 0


@pytest.mark.parametrize("mistake", ["swap", "worse_block", "d2", "pad_row", "duplicate", "tail", "skip_best",
                                     "tie_order"])
def test_route_checker_rejects_planted_mistakes(mistake):
    w = W.custom_block_workload(54, [1] * 50, 1, 4, 2, 8, "f32", 6, pts_mode="lattice")
    w2 = W.custom_block_workload(55, [4, 2, 6, 1, 8, 3, 5, 7], 8, 4, 2, 8, "f32", 10)
    if mistake in ("pad_row", "tail"):
        w = w2
    sel, d2 = O.route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k)
    vs = w.valid_slots()
    r = vs[len(vs) // 2]
    cen = O.block_centroids(w.pts, w.blk_cnt, w.blk_cap)
    u = O.lattice_coords(w.pts)
    dist = lambda rr, b: int(((u[rr] - cen[b]) ** 2).sum())      # noqa: E731
    if mistake == "swap":
        sel[r, [0, 1]] = sel[r, [1, 0]]
        d2[r, [0, 1]] = d2[r, [1, 0]]
    elif mistake == "worse_block":
        others = [b for b in range(w.n_blk) if b not in sel[r]]
        far = max(others, key=lambda b: dist(r, b))
        sel[r, -1], d2[r, -1] = far, dist(r, far)
    elif mistake == "d2":
        d2[r, 2] += 1
    elif mistake == "pad_row":
        pad = np.nonzero(~w.valid_mask())[0][0]
        sel[pad, 0] = 0
    elif mistake == "duplicate":
        sel[r, 3], d2[r, 3] = sel[r, 2], d2[r, 2]
    elif mistake == "tail":                     # k beyond the block count: the tail must stay -1
        assert w.top_k > w.n_blk
        sel[r, w.n_blk] = 0
    elif mistake == "skip_best":                # drop the best, shift, append the next one
        nxt = sorted(range(w.n_blk), key=lambda b: (dist(r, b), int(w.blk_key[b])))[w.top_k]
        sel[r] = np.concatenate([sel[r, 1:], [nxt]])
        d2[r] = np.concatenate([d2[r, 1:], [dist(r, nxt)]])
    else:                                       # equal distances listed in descending key order
        rows = [rr for rr in vs if any(d2[rr, i] == d2[rr, i + 1] for i in range(w.top_k - 1))]
        assert rows, "the lattice case has exact distance ties"
        r = rows[0]
        i = next(i for i in range(w.top_k - 1) if d2[r, i] == d2[r, i + 1])
        sel[r, [i, i + 1]] = sel[r, [i + 1, i]]
    nbad, first = O.check_route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, sel, d2)
    assert nbad == 1, (mistake, nbad, first)


# ---------------------------------------------------------------------------------------------
# eq. M^vol in fp64 against a library trilinear interpolation
# ---------------------------------------------------------------------------------------------

def test_voxel_activity_against_scipy_trilinear():
    from scipy.interpolate import RegularGridInterpolator
    rng = np.random.default_rng(61)
    G, N, tau = 6, 8, 0.2
    sdf = rng.standard_normal((G, G, G)).astype(np.float32)
    act, mabs, mn, mx = O.voxel_activity(sdf, N, tau, return_values=True)
    g = np.linspace(-1.0, 1.0, G)
    f = RegularGridInterpolator((g, g, g), sdf.astype(np.float64), method="linear")
    x = -1.0 + (2.0 * np.arange(4 * N) + 1.0) / (4.0 * N)           # sub-sample centres
    zz, yy, xx = np.meshgrid(x, x, x, indexing="ij")
    s = f(np.stack([zz.ravel(), yy.ravel(), xx.ravel()], axis=1)).reshape(4 * N, 4 * N, 4 * N)
    s = s.reshape(N, 4, N, 4, N, 4).transpose(0, 2, 4, 1, 3, 5).reshape(N, N, N, 64)
    np.testing.assert_allclose(mabs, np.abs(s).min(axis=3), rtol=0, atol=1e-12)
    np.testing.assert_allclose(mn, s.min(axis=3), rtol=0, atol=1e-12)
    np.testing.assert_allclose(mx, s.max(axis=3), rtol=0, atol=1e-12)
    want = (np.abs(s).min(axis=3) <= tau) | ((s.min(axis=3) <= 0) & (s.max(axis=3) >= 0))
    band = np.abs(np.abs(s).min(axis=3) - tau) < 1e-9
    assert band.sum() == 0
    np.testing.assert_array_equal(act, want)
    assert 0 < act.sum() < act.size
