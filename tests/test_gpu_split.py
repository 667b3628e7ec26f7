"""GPU parity of the split self/cross form of stage 2 (LSRM pages, section 方法, eq. o^x, o^y with
sparse attention over each token type's blocks): ranged geometric routing bit-exact, ranged
attention and the composed layer against the fp64 oracle (max-abs 2e-2 for bf16, 1e-4 for fp32)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import host, max_err, say, tdt, to_dev, tol

pytestmark = pytest.mark.gpu

_cache = {}


def wl(name):
    if name not in _cache:
        _cache[name] = W.make(name)
    return _cache[name]


def n_x_blocks(w):
    t = w.blk_type.astype(np.int64)
    assert np.all(np.diff(t) >= 0), "volume blocks come first"
    return int((t == 0).sum())


def ranges(w):
    nx = n_x_blocks(w)
    x, y = (0, nx), (nx, w.n_blk)
    return nx, [(x, x), (x, y), (y, y), (y, x)]


@pytest.mark.parametrize("name", ["tiny", "stage2_small", "large_small"])
def test_route_range_bit_exact(name):
    import sparse_attention_feed_amd as S
    w = wl(name)
    d = to_dev(w)
    pts = torch.from_numpy(w.pts).cuda()
    nx, prs = ranges(w)
    for qr, kr in prs:
        say("route range", name, qr, kr)
        sel = torch.full((w.n_slots, w.top_k), -7, dtype=torch.int32, device="cuda")
        d2 = torch.full((w.n_slots, w.top_k), -7, dtype=torch.int32, device="cuda")
        S.route_geometric(d["layout"], pts, w.top_k, sel=sel, sel_d2=d2, q_blocks=qr, kv_blocks=kr)
        torch.cuda.synchronize()
        ref, ref_d2 = O.route_geometric_range(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k, qr, kr)
        s0, s1 = qr[0] * w.blk_cap, qr[1] * w.blk_cap
        g = sel.cpu().numpy()
        np.testing.assert_array_equal(g[s0:s1], ref)
        np.testing.assert_array_equal(d2.cpu().numpy()[s0:s1].view(np.uint32), ref_d2)
        assert np.all(g[:s0] == -7) and np.all(g[s1:] == -7)      # rows outside the range untouched


def test_route_range_fewer_candidates_than_k():
    import sparse_attention_feed_amd as S
    w = W.custom_block_workload(31, [5, 8, 1, 3, 8, 6, 2, 7, 8], 8, 32, 2, 32, "f32", 6)
    d = to_dev(w)
    pts = torch.from_numpy(w.pts).cuda()
    for qr, kr in (((0, 9), (2, 5)), ((3, 7), (8, 9)), ((0, 9), (4, 4))):
        say("route range k beyond candidates", qr, kr)
        sel = torch.full((w.n_slots, w.top_k), -7, dtype=torch.int32, device="cuda")
        S.route_geometric(d["layout"], pts, w.top_k, sel=sel, want_d2=False, q_blocks=qr, kv_blocks=kr)
        torch.cuda.synchronize()
        ref, _ = O.route_geometric_range(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k, qr, kr)
        np.testing.assert_array_equal(sel.cpu().numpy()[qr[0] * 8:qr[1] * 8], ref)


@pytest.mark.parametrize("name", ["tiny", "large_small"])
def test_attn_range_rows_and_gate_channels(name):
    """One ranged call: only the query blocks of the range are written; CMP sees the key range only;
    the gate channels start at gate_channel of a wider gate tensor."""
    import sparse_attention_feed_amd as S
    w = wl(name)
    d = to_dev(w)
    nx, _ = ranges(w)
    g7 = W.split_gates(w, 71)
    gd = torch.from_numpy(g7).cuda().to(tdt(w)).contiguous()
    k_cmp = S.pool_blocks(d["layout"], d["k"])
    v_cmp = S.pool_blocks(d["layout"], d["v"])
    qr, kr = (nx, w.n_blk), (0, nx)                 # image queries against the volume blocks
    say("attn range", name, qr, kr)
    out = torch.full_like(d["q"], 7.0)
    S.attn_fwd(d["layout"], S.BR_CMP, d["q"], k_cmp=k_cmp, v_cmp=v_cmp, gates=gd, gate_channel=5, out=out,
               q_blocks=qr, kv_blocks=kr)
    torch.cuda.synchronize()
    o = host(out)
    s0, s1 = qr[0] * w.blk_cap, qr[1] * w.blk_cap
    assert np.all(o[:s0] == 7.0) and np.all(o[s1:] == 7.0)
    rng = np.random.default_rng(5)
    vs = w.valid_slots()
    rows = vs[(vs >= s0) & (vs < s1)]
    rows = rows if rows.shape[0] <= 200 else rng.choice(rows, 200, replace=False)
    kc = O.pool_blocks(w.k, w.blk_cnt, w.blk_cap)
    vc = O.pool_blocks(w.v, w.blk_cnt, w.blk_cap)
    sg = O.sigmoid(g7[..., 5].astype(np.float64))
    for r in rows:
        ref, _ = O.attend(w.q[r], kc[kr[0]:kr[1]], vc[kr[0]:kr[1]], w.scale)
        assert max_err(o[r], sg[r][:, None] * ref) <= tol(w), r


@pytest.mark.parametrize("name", ["tiny", "stage2_small", "large_small"])
def test_split_layer(name):
    import sparse_attention_feed_amd as S
    w = wl(name)
    d = to_dev(w)
    nx, _ = ranges(w)
    g7 = W.split_gates(w, 72)
    gd = torch.from_numpy(g7).cuda().to(tdt(w)).contiguous()
    pts = torch.from_numpy(w.pts).cuda()
    say("split layer", name, "n_x_blk", nx, "of", w.n_blk)
    out = S.nsa_split_layer(d["layout"], d["q"], d["k"], d["v"], pts, nx, gd, w.top_k)
    torch.cuda.synchronize()
    o = host(out)
    vs = w.valid_slots()
    rng = np.random.default_rng(6)
    rows = vs if vs.shape[0] <= 160 else np.sort(rng.choice(vs, 160, replace=False))
    ref = O.nsa_split_forward(w, nx, g7, rows=rows)
    err = max_err(o[rows], ref)
    say("split layer", name, "max err", err)
    assert err <= tol(w)
    assert np.all(o[~w.valid_mask()] == 0)


@pytest.mark.parametrize("nx", ["none", "all"])
def test_split_layer_single_type(nx):
    """One token type only: the cross term has no keys and adds nothing."""
    import sparse_attention_feed_amd as S
    w = wl("tiny")
    n = 0 if nx == "none" else w.n_blk
    d = to_dev(w)
    g7 = W.split_gates(w, 73)
    gd = torch.from_numpy(g7).cuda().contiguous()
    pts = torch.from_numpy(w.pts).cuda()
    say("split layer single type", nx)
    out = S.nsa_split_layer(d["layout"], d["q"], d["k"], d["v"], pts, n, gd, w.top_k)
    torch.cuda.synchronize()
    ref = O.nsa_split_forward(w, n, g7)
    assert max_err(host(out), ref) <= tol(w)


def test_attn_range_local_outside_key_range_is_zero():
    """The local branch over a key range that excludes the query's own block has no keys: 0."""
    import sparse_attention_feed_amd as S
    w = wl("large_small")
    d = to_dev(w)
    nx, _ = ranges(w)
    say("attn range, local branch outside the key range")
    out = torch.full_like(d["q"], 7.0)
    S.attn_fwd(d["layout"], S.BR_LOC, d["q"], d["k"], d["v"], out=out, q_blocks=(0, nx), kv_blocks=(nx, w.n_blk))
    torch.cuda.synchronize()
    o = host(out)
    assert np.all(o[:nx * w.blk_cap] == 0.0)
    assert np.all(o[nx * w.blk_cap:] == 7.0)
