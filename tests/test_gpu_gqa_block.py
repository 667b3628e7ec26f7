"""GPU parity of block-granular query rows in the grouped-query layout (32 query heads over 2 KV
heads, head dim 32): pooled queries in the compressed branch and the score routing (one row per
query block and KV group), token queries over the block's routing row in the selected branch,
against the fp64 oracle.  Bars as in the per-token tests: routing rows up to epsilon ties of the
oracle's importance, outputs max-abs 2e-2 (bf16) or 1e-4 (fp32)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import host, max_err, rounded, say, tdt, to_dev, tol

pytestmark = pytest.mark.gpu
_cache = {}


def case(name):
    """Named workloads with block-granular query rows; 'ragged150' has 150 blocks of up to 64 valid
    tokens (two full 64-row groups of pooled rows and a ragged third) and top_k 64."""
    if name not in _cache:
        if name == "ragged150":
            cnt = np.random.default_rng(31).integers(1, 65, size=150).tolist()
            w = W.custom_block_workload(31, cnt, 64, 32, 2, 32, "bf16", 64, routing="scores", q_gran="block")
        else:
            w = dataclasses.replace(W.make(name), routing="scores", q_gran="block")
        _cache[name] = w
    return _cache[name]


def pooled(w):
    return [rounded(O.pool_blocks(x, w.blk_cnt, w.blk_cap), w.dtype) for x in (w.q, w.k, w.v)]


def dev(w, x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(tdt(w))


def block_lse(w, qc, kc, vc, blocks=None):
    blocks = range(w.n_blk) if blocks is None else blocks
    return np.stack([O.attend(qc[b].astype(np.float64), kc.astype(np.float64), vc.astype(np.float64),
                              w.scale)[1] for b in blocks])


def check_rows(got, ref_sel, imp, k, eps_rel):
    """Every row: k distinct blocks, and any block listed by one side only lies within eps of the
    oracle's k-th importance.  Returns the fraction of rows equal to the oracle's."""
    exact = 0
    R, H = ref_sel.shape[:2]
    for r in range(R):
        for j in range(H):
            g_row, r_row = got[r, j], ref_sel[r, j]
            assert len(set(g_row.tolist())) == k and g_row.min() >= 0
            if np.array_equal(g_row, r_row):
                exact += 1
                continue
            kth = np.sort(imp[r, j])[::-1][k - 1]
            for b in set(g_row.tolist()) ^ set(r_row.tolist()):
                assert abs(imp[r, j, b] - kth) <= eps_rel * abs(kth), (r, j, b)
    return exact / (R * H)


@pytest.mark.parametrize("name,top_k", [("tiny", 4), ("stage2_small", 16), ("ragged150", 64), ("ragged150", 5)])
def test_block_rows_score_routing(name, top_k):
    """Pooled query rows, 64 per workgroup (a ragged last group at 150 blocks); the oracle's pooled
    values (rounded to the storage type) and lse feed both sides."""
    import sparse_attention_feed_amd as S
    w = case(name)
    d = to_dev(w)
    qc, kc, vc = pooled(w)
    lse = block_lse(w, qc, kc, vc).astype(np.float32)
    k = min(top_k, w.n_blk)
    say("route block rows", name, w.n_blk, k)
    sel = S.route_scores_topk(d["layout"], dev(w, qc), dev(w, kc), torch.from_numpy(lse).cuda(), k,
                              q_gran=S.Q_BLOCK)
    torch.cuda.synchronize()
    assert tuple(sel.shape) == (w.n_blk, w.n_kvh, k)
    ref_sel, imp = O.route_scores(qc, kc, w.blk_key, w.scale, k, lse=lse.astype(np.float64))
    frac = check_rows(host(sel), ref_sel, imp, k, 1e-2 if w.dtype == "bf16" else 1e-5)
    print("block-row routing %s k=%d: %.3f of rows exact" % (name, k, frac), flush=True)
    assert frac >= 0.9, frac


@pytest.mark.parametrize("name", ["tiny", "stage2_small", "ragged150"])
def test_block_rows_compressed_branch(name):
    """The pooled queries' compressed branch, given to every valid token of each block, with its
    per-block lse."""
    import sparse_attention_feed_amd as S
    w = case(name)
    d = to_dev(w)
    qc, kc, vc = pooled(w)
    lse = torch.empty((w.n_blk, w.n_qh), dtype=torch.float32, device="cuda")
    say("cmp block rows", name)
    o = S.attn_fwd(d["layout"], S.BR_CMP, d["q"], q_cmp=dev(w, qc), k_cmp=dev(w, kc), v_cmp=dev(w, vc), lse=lse,
                   q_gran=S.Q_BLOCK)
    torch.cuda.synchronize()
    ref, _ = O.attn_branch(O.CMP, qc.astype(np.float64), kc.astype(np.float64), vc.astype(np.float64), w.blk_cnt,
                           w.blk_cap, w.scale, q_gran="block")
    vm = w.valid_mask()
    got = host(o)
    assert max_err(got, ref) <= tol(w)
    assert np.all(got[~vm] == 0)
    bound = 1e-4 if w.dtype == "f32" else (
        1.96e-3 + 2.0 ** -9 * w.scale * np.linalg.norm(qc.astype(np.float64), axis=2).max()
        * np.linalg.norm(kc.astype(np.float64), axis=2).max() + 1e-4)
    assert max_err(host(lse), block_lse(w, qc, kc, vc)) <= bound


@pytest.mark.parametrize("name,groups", [("tiny", 2), ("stage2_small", 2), ("stage2_small", 1), ("ragged150", 2)])
def test_block_rows_selected_branch(name, groups):
    """Token queries over the union of their block's routing row (per KV group, or one row shared by
    both groups), with repeated and -1 entries in the rows."""
    import sparse_attention_feed_amd as S
    w = case(name)
    d = to_dev(w)
    k = min(w.top_k, w.n_blk)
    rng = np.random.default_rng(7)
    shape = (w.n_blk, w.n_kvh, k) if groups == 2 else (w.n_blk, k)
    sel = rng.integers(-1, w.n_blk, size=shape).astype(np.int32)
    if k > 1:
        sel[..., 1] = sel[..., 0]
    sel[::5] = -1
    say("sel block rows", name, groups)
    o = S.attn_fwd(d["layout"], S.BR_SEL, d["q"], d["k"], d["v"], sel=torch.from_numpy(sel).cuda(), top_k=k,
                   sel_groups=groups, q_gran=S.Q_BLOCK)
    torch.cuda.synchronize()
    ref, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel, q_gran="block")
    assert max_err(host(o), ref) <= tol(w)


@pytest.mark.parametrize("name", ["tiny", "stage2_small"])
def test_block_rows_layer(name):
    """The whole layer on the GPU (pooling, the pooled queries' compressed branch for lse, routing per
    (query block, KV group), the three gated branches) against the oracle's layer from the same
    inputs (its own pooling, lse and routing); outputs compared on the tokens whose block's rows
    agree with the oracle's (others are checked for epsilon ties).  A pooled query averages up to
    64 token queries, so its logits are small and a group's block importances nearly flat: the
    bf16 rounding of the device's own pooled rows reorders blocks near the k-th value more often
    than with token rows, hence the lower exact fraction asked for (0.80 measured at stage2_small)."""
    import sparse_attention_feed_amd as S
    w = case(name)
    d = to_dev(w)
    L = d["layout"]
    say("layer block rows", name)
    qd, kd, vd = S.pool_blocks(L, d["q"]), S.pool_blocks(L, d["k"]), S.pool_blocks(L, d["v"])
    lse = torch.empty((w.n_blk, w.n_qh), dtype=torch.float32, device="cuda")
    S.attn_fwd(L, S.BR_CMP, d["q"], q_cmp=qd, k_cmp=kd, v_cmp=vd, lse=lse, q_gran=S.Q_BLOCK)
    sel = S.route_scores_topk(L, qd, kd, lse, w.top_k, q_gran=S.Q_BLOCK)
    o = S.attn_fwd(L, S.BR_CMP | S.BR_SEL | S.BR_LOC, d["q"], d["k"], d["v"], q_cmp=qd, k_cmp=kd, v_cmp=vd,
                   sel=sel, top_k=w.top_k, sel_groups=w.n_kvh, gates=d["gates"], q_gran=S.Q_BLOCK)
    torch.cuda.synchronize()
    ref, parts = O.nsa_forward(w, return_parts=True)
    qr, kr, _ = (O.pool_blocks(x, w.blk_cnt, w.blk_cap) for x in (w.q, w.k, w.v))
    _, imp = O.route_scores(qr, kr, w.blk_key, w.scale, w.top_k, lse=block_lse(w, qr, kr, parts["v_cmp"]))
    frac = check_rows(host(sel), parts["sel"], imp, w.top_k, 1e-2 if w.dtype == "bf16" else 1e-5)
    print("block-row layer %s: %.3f of rows exact" % (name, frac), flush=True)
    assert frac >= 0.75, frac
    same = np.all(host(sel) == parts["sel"], axis=2)                   # [n_blk, Hkv]
    vm = w.valid_mask()
    blk = np.arange(w.n_slots) // w.blk_cap
    G = w.n_qh // w.n_kvh
    got = host(o)
    diff = np.abs(got - ref).max(axis=2).reshape(w.n_slots, w.n_kvh, G).max(axis=2)
    agree = same[blk] & vm[:, None]
    assert diff[agree].max() <= tol(w), diff[agree].max()
    assert np.all(got[~vm] == 0)
