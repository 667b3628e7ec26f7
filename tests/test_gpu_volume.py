"""GPU parity of the active-voxel selection and the volume block table (LSRM pages, section 方法,
eq. M^vol and the block paragraph).

The oracle takes the decision in float64; the device in float32 with a fixed operation order.  A
voxel whose float64 sub-sample values lie within the float32 evaluation's error bound of the
threshold tau (or of zero, for the sign test) may legitimately decide differently: such voxels are
counted and reported, every other voxel must agree exactly.  When no voxel differs, the whole block
table (counts, keys, token points, block count) must equal the oracle's bit for bit; the GPU table
must in any case satisfy the grouping rules (one 4^3 cell per block named by its Morton key, keys
ascending, tokens in local Morton order, float32 voxel centres, zero padding)."""
import ctypes
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _gpu(sdf, N, tau, max_blk=None):
    import sparse_attention_feed_amd as S
    t = torch.from_numpy(np.ascontiguousarray(sdf, dtype=np.float32)).to("cuda:0")
    nb, cnt, key, pts = S.build_volume_blocks(t, N, tau, max_blk)
    torch.cuda.synchronize()
    return nb, cnt.cpu().numpy(), key.cpu().numpy().view(np.uint32), pts.cpu().numpy()


def fp32_error_bound(sdf):
    """Bound on |s_fp32 - s| for the device's trilinear sample (three nested lerps a + f (b - a),
    each operation rounded to float32, the fraction f carrying the rounding of one division of
    size <= G): per lerp at most (2G + 5) M 2^-24 with M = max |sdf|; three levels, doubled."""
    G = sdf.shape[0]
    M = float(np.abs(sdf.astype(np.float64)).max())
    return 6.0 * (2 * G + 5) * max(M, 1e-30) * 2.0 ** -24


def certain_voxels(mabs, mn, mx, tau, E):
    """Voxels whose decision cannot change under an evaluation error below E."""
    tau_true = mabs < tau - E
    tau_false = mabs > tau + E
    signs_sure = mabs > E
    sign_true = signs_sure & (mn <= 0) & (mx >= 0)
    return tau_true | sign_true | (tau_false & signs_sure)


def _morton3_decode(code):
    x = y = z = 0
    for b in range(10):
        x |= ((code >> (3 * b)) & 1) << b
        y |= ((code >> (3 * b + 1)) & 1) << b
        z |= ((code >> (3 * b + 2)) & 1) << b
    return x, y, z


def gpu_table_active(N, nb, cnt, key, pts):
    """Check the grouping rules of a device block table; return its active voxels [z][y][x]."""
    act = np.zeros((N, N, N), dtype=bool)
    assert np.all((cnt >= 1) & (cnt <= 64))
    assert np.all(np.diff(key.astype(np.int64)) > 0)
    f32 = np.float32
    for b in range(nb):
        p = pts[b * 64: b * 64 + cnt[b]].astype(np.float64)
        idx = np.rint((p * N + (N - 1)) / 2.0).astype(np.int64)
        assert np.all((idx >= 0) & (idx < N))
        cen = ((2 * idx + 1).astype(f32) - f32(N)) / f32(N)
        np.testing.assert_array_equal(cen.astype(f32).view(np.uint32), pts[b * 64: b * 64 + cnt[b]].view(np.uint32))
        cx, cy, cz = _morton3_decode(int(key[b]))
        assert np.all(idx[:, 0] >> 2 == cx) and np.all(idx[:, 1] >> 2 == cy) and np.all(idx[:, 2] >> 2 == cz)
        local = W.morton3(idx[:, 0] & 3, idx[:, 1] & 3, idx[:, 2] & 3).astype(np.int64)
        assert np.all(np.diff(local) > 0)
        act[idx[:, 2], idx[:, 1], idx[:, 0]] = True
        assert np.all(pts[b * 64 + cnt[b]: (b + 1) * 64] == 0)
    return act


def _check(sdf, N, tau, require_exact=False):
    tau = float(np.float32(tau))          # the device takes tau in float32; the oracle the same number
    say("volume blocks", "G=%d" % sdf.shape[0], "N=%d" % N, "tau=%r" % tau)
    act, mabs, mn, mx = O.voxel_activity(sdf, N, tau, return_values=True)
    E = fp32_error_bound(sdf)
    sure = certain_voxels(mabs, mn, mx, tau, E)
    nb, gc, gk, gp = _gpu(sdf, N, tau)
    gact = gpu_table_active(N, nb, gc, gk, gp)
    n_unsure = int((~sure).sum())
    n_diff = int((gact != act).sum())
    print("volume G=%d N=%d: %d voxels within the fp32 bound %.3g of a threshold, %d decided differently"
          % (sdf.shape[0], N, n_unsure, E, n_diff), flush=True)
    np.testing.assert_array_equal(gact[sure], act[sure])
    if require_exact:
        assert n_diff == 0
    if n_diff == 0:
        cnt, key, pts = O.volume_block_table(sdf, N, tau)
        assert nb == cnt.shape[0]
        np.testing.assert_array_equal(gc, cnt)
        np.testing.assert_array_equal(gk, key)
        np.testing.assert_array_equal(gp.view(np.uint32), pts.view(np.uint32))     # bit-exact, padding 0
    return nb


def _linear(G, a, c0):
    g = np.linspace(-1.0, 1.0, G)
    zz, yy, xx = np.meshgrid(g, g, g, indexing="ij")
    return (a[0] * xx + a[1] * yy + a[2] * zz + c0).astype(np.float32)


def _sphere(G, r, c=(0.0, 0.0, 0.0)):
    g = np.linspace(-1.0, 1.0, G)
    zz, yy, xx = np.meshgrid(g, g, g, indexing="ij")
    return (np.sqrt((xx - c[0]) ** 2 + (yy - c[1]) ** 2 + (zz - c[2]) ** 2) - r).astype(np.float32)


def test_volume_ramp_hand_fixture_gpu():
    fx = json.load(open(os.path.join(GOLDEN, "volume_ramp.json"), encoding="utf-8"))
    sdf = np.array(fx["sdf"], dtype=np.float32)
    nb, gc, gk, gp = _gpu(sdf, fx["N"], fx["tau"])
    assert nb == 1 and gc.tolist() == fx["blk_cnt"] and gk.tolist() == fx["blk_key"]
    np.testing.assert_array_equal(gp[:3], np.array(fx["first_points"], dtype=np.float32))
    assert np.all(gp[fx["blk_cnt"][0]:] == 0)
    _check(sdf, fx["N"], fx["tau"], require_exact=True)


def test_volume_empty_and_full():
    g = np.full((3, 3, 3), 0.3, dtype=np.float32)
    assert _check(g, 8, 0.2, require_exact=True) == 0     # no active voxel: zero blocks
    assert _check(g, 8, 0.3, require_exact=True) == 8     # every voxel active: 8 full blocks
    assert _check(np.zeros((2, 2, 2), np.float32), 4, 0.0, require_exact=True) == 1


@pytest.mark.parametrize("case", ["linear", "random9", "random3_coarse", "sphere33", "sphere_offcentre",
                                  "ties_at_tau"])
def test_volume_blocks_bit_exact(case):
    rng = np.random.default_rng(np.random.PCG64(77))
    if case == "linear":
        _check(_linear(5, (0.6, -0.3, 0.2), 0.013), 8, 0.07)
    elif case == "random9":
        _check(rng.standard_normal((9, 9, 9)).astype(np.float32), 16, 0.05)
    elif case == "random3_coarse":                     # one lattice cell spans 16 voxels per axis
        _check(rng.standard_normal((3, 3, 3)).astype(np.float32), 32, 0.02)
    elif case == "sphere33":
        _check(_sphere(33, 0.55), 32, 0.03)
    elif case == "sphere_offcentre":
        _check(_sphere(17, 0.4, (0.21, -0.13, 0.3)), 64, 0.011)
    else:                                              # lattice values equal to tau and to -tau
        sdf = np.round(rng.uniform(-4, 4, size=(5, 5, 5))).astype(np.float32) * np.float32(0.25)
        _check(sdf, 16, 0.25)


def test_volume_large_small_workload_lattice():
    w = W.make("large_small")
    lat, tau = W.sdf_lattice(w, 33)
    nb = _check(lat, 32, tau)
    assert nb > 50


def test_volume_full_size_large_lattice():
    """The 128^3 volume of the large sparse stage (SDF lattice 129^3): every voxel outside the fp32
    band decided as the oracle decides, and the table bit-exact when no voxel differs."""
    w = W.make("large")
    lat, tau = W.sdf_lattice(w, 129)
    nb = _check(lat, 128, tau)
    assert nb > 5000


def test_volume_max_blk_truncates_and_reports():
    import sparse_attention_feed_amd as S
    rng = np.random.default_rng(np.random.PCG64(78))
    sdf = rng.standard_normal((9, 9, 9)).astype(np.float32)
    N, tau = 16, float(np.float32(0.05))
    _, mabs, mn, mx = O.voxel_activity(sdf, N, tau, return_values=True)
    assert certain_voxels(mabs, mn, mx, tau, fp32_error_bound(sdf)).all()    # no voxel near a threshold
    cnt, key, pts = O.volume_block_table(sdf, N, tau)
    nb_all = cnt.shape[0]
    cap = nb_all // 2
    say("volume blocks max_blk", cap, "of", nb_all)
    dev = "cuda:0"
    t = torch.from_numpy(sdf).to(dev)
    n_cells = (N // 4) ** 3
    cell_mask = torch.empty(n_cells, dtype=torch.int64, device=dev)
    cell_block = torch.empty(n_cells, dtype=torch.int32, device=dev)
    n_blk = torch.zeros(1, dtype=torch.int32, device=dev)
    sentinel = -7
    blk_cnt = torch.full((cap + 1,), sentinel, dtype=torch.int32, device=dev)
    blk_key = torch.full((cap + 1,), sentinel, dtype=torch.int32, device=dev)
    out_pts = torch.full(((cap + 1) * 64, 3), -7.0, dtype=torch.float32, device=dev)
    p = lambda x: ctypes.c_void_p(x.data_ptr())      # noqa: E731
    rc = S.lib.nsa_build_volume_blocks(p(t), 9, N, tau, cap, p(cell_mask), p(cell_block), p(n_blk), p(blk_cnt),
                                       p(blk_key), p(out_pts), None)
    torch.cuda.synchronize()
    assert rc == 0
    assert int(n_blk.item()) == nb_all
    np.testing.assert_array_equal(blk_cnt.cpu().numpy()[:cap], cnt[:cap])
    np.testing.assert_array_equal(blk_key.cpu().numpy()[:cap].view(np.uint32), key[:cap])
    np.testing.assert_array_equal(out_pts.cpu().numpy()[:cap * 64], pts[:cap * 64])
    assert blk_cnt[cap].item() == sentinel and blk_key[cap].item() == sentinel    # nothing past max_blk
    assert torch.all(out_pts[cap * 64:] == -7.0).item()
    cb = cell_block.cpu().numpy()
    assert sorted(cb[cb >= 0].tolist()) == list(range(nb_all))
    with pytest.raises(ValueError):
        S.build_volume_blocks(t, N, tau, cap)


def test_volume_workspace_reuse():
    """Two tables in a row through one workspace: the second call leaves nothing of the first."""
    import sparse_attention_feed_amd as S
    rng = np.random.default_rng(np.random.PCG64(79))
    N = 16
    ws = S.volume_workspace(N)
    for G, tau in ((9, 0.3), (5, 0.01)):
        sdf = rng.standard_normal((G, G, G)).astype(np.float32)
        tau = float(np.float32(tau))
        say("volume workspace reuse", G, tau)
        _, mabs, mn, mx = O.voxel_activity(sdf, N, tau, return_values=True)
        assert certain_voxels(mabs, mn, mx, tau, fp32_error_bound(sdf)).all()
        cnt, key, pts = O.volume_block_table(sdf, N, tau)
        nb, gc, gk, gp = S.build_volume_blocks(torch.from_numpy(sdf).to("cuda:0"), N, tau, workspace=ws)
        assert nb == cnt.shape[0]
        np.testing.assert_array_equal(gc.cpu().numpy(), cnt)
        np.testing.assert_array_equal(gk.cpu().numpy().view(np.uint32), key)
        np.testing.assert_array_equal(gp.cpu().numpy(), pts)
