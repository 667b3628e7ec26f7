"""GPU parity of geometric routing with the image blocks found through the views (LSRM pages,
section 方法, routing paragraph): selected blocks and their distances bit-exact against the oracle
on the same fp32 points and cameras, except for rows whose projection lies within the float32
evaluation error of a cell edge (the oracle projects in float64), which are counted and left out."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu

_cache = {}


def wl(name):
    if name not in _cache:
        _cache[name] = W.make(name)
    return _cache[name]


def _gpu_views(w, n_vol, proj, cell_blk, cell, radius):
    import sparse_attention_feed_amd as S
    d = to_dev(w)
    pts = torch.from_numpy(w.pts).cuda()
    sel, d2, _ = S.route_geometric_views(d["layout"], pts, w.top_k, n_vol, torch.from_numpy(proj).cuda(),
                                         torch.from_numpy(cell_blk).cuda(), cell_size=cell, radius=radius)
    torch.cuda.synchronize()
    return sel.cpu().numpy(), d2.cpu().numpy().view(np.uint32)


def near_cell_edge(pts, proj, cell):
    """Rows whose projection into some view lies within the float32 evaluation error of a cell
    edge: the device evaluates the affine map ((A0 p0 + A1 p1) + A2 p2) + A3 with every operation
    rounded to float32 (at most six roundings, each <= 2^-24 of a partial sum bounded by
    sum |A_i p_i| + |A3|), the oracle in float64; only there may the two pick different cells."""
    p = np.asarray(pts, dtype=np.float64)
    A = np.asarray(proj, dtype=np.float64)                              # [V, 2, 4]
    x = np.einsum("rc,vac->rva", p, A[:, :, :3]) + A[None, :, :, 3]      # [R, V, 2]
    mag = np.einsum("rc,vac->rva", np.abs(p), np.abs(A[:, :, :3])) + np.abs(A[None, :, :, 3])
    E = 2.0 * 6.0 * mag * 2.0 ** -24
    d = np.abs(x - cell * np.round(x / cell))
    return np.any(d <= E, axis=(1, 2))


def _check(w, n_vol, proj, cell_blk, cell, radius, rows=None):
    say("route views", w.name, "n_vol", n_vol, "views", proj.shape[0], "radius", radius)
    sel, d2 = _gpu_views(w, n_vol, proj, cell_blk, cell, radius)
    rows = np.arange(w.n_slots) if rows is None else rows
    edge = near_cell_edge(w.pts[rows], proj, cell) & w.valid_mask()[rows]
    print("route views %s: %d of %d rows project within the fp32 error of a cell edge (not compared)"
          % (w.name, edge.sum(), len(rows)), flush=True)
    assert edge.mean() < 0.01
    rows = rows[~edge]
    ref, ref_d2 = O.route_geometric_views(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k, n_vol, proj, cell_blk,
                                          cell, radius, rows=rows)
    np.testing.assert_array_equal(sel[rows], ref)
    np.testing.assert_array_equal(d2[rows], ref_d2)


@pytest.mark.parametrize("name", ["stage2_small", "large_small"])
@pytest.mark.parametrize("radius", [0, 1, 2])
def test_route_views_bit_exact(name, radius):
    w = wl(name)
    proj, cell_blk = W.view_cameras(w)
    n_vol = int((w.blk_type == 0).sum())
    vs = w.valid_slots()
    rows = np.sort(np.random.default_rng(radius).choice(vs, min(400, vs.shape[0]), replace=False))
    pad = np.nonzero(~w.valid_mask())[0][:20]
    _check(w, n_vol, proj, cell_blk, 8, radius, rows=np.concatenate([rows, pad]))


def test_route_views_full_size_sampled():
    w = wl("large")
    proj, cell_blk = W.view_cameras(w)
    n_vol = int((w.blk_type == 0).sum())
    rows = np.sort(np.random.default_rng(9).choice(w.valid_slots(), 2000, replace=False))
    _check(w, n_vol, proj, cell_blk, 8, 1, rows=rows)


def test_route_views_hand_cameras_all_rows():
    w = W.custom_block_workload(41, [3, 5, 2, 4, 6, 1, 3, 2], 8, 32, 2, 32, "f32", 4)
    proj = np.zeros((2, 2, 4), dtype=np.float32)
    proj[0, 0, 0] = proj[0, 1, 1] = proj[1, 0, 1] = proj[1, 1, 2] = 8.0
    proj[:, :, 3] = 8.0
    cell_blk = np.full((2, 2, 2), -1, dtype=np.int32)
    cell_blk[0, 0, 0], cell_blk[0, 1, 1], cell_blk[1, 0, 1], cell_blk[1, 1, 0], cell_blk[1, 1, 1] = 3, 4, 5, 6, 7
    for radius in (0, 1):
        _check(w, 3, proj, cell_blk, 8, radius)


def test_route_views_without_views_is_volume_routing():
    w = wl("stage2_small")
    n_vol = int((w.blk_type == 0).sum())
    say("route views, no views")
    sel, d2 = _gpu_views(w, n_vol, np.zeros((0, 2, 4), np.float32), np.zeros((0, 1, 1), np.int32), 8, 1)
    ref, ref_d2 = O.route_geometric_range(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k, (0, w.n_blk), (0, n_vol))
    np.testing.assert_array_equal(sel, ref)
    np.testing.assert_array_equal(d2, ref_d2)
