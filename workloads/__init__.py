"""Seeded synthetic inputs for the NSA forward pass (shared by the oracle and the HIP path).

This module builds *inputs only*: token geometry, the block-major storage layout, and the
random q/k/v/gate tensors.  It holds none of the method's arithmetic (no pooling, routing,
attention or gating) so that the CPU oracle and the GPU path stay independent of each other.

Workload shapes follow the LSRM pages (hyper.ai summary of arXiv 2604.05182, section "方法"):
volume tokens on a voxel grid near the object surface (here a plain band around the surface of an
analytic SDF, sized to the target count), image tokens from
foreground patches of several views, grouped-query attention with 32 query heads over 2 KV heads
of dimension 32, and spatial blocks of 64 tokens.  The score-routed long-sequence shape follows the
Speed3R page (gist.science summary of arXiv 2603.08055, section 2.1): 4x4-pooled multi-view grids.

Storage convention (block-major): block b owns slots [b*cap, b*cap + cnt[b]); remaining slots of
the block are padding.  Volume blocks come first (Morton order of 4^3 voxel cells), then image
blocks in (view, Morton order of the patch cell).  blk_key = type<<31 | view<<20 | cell Morton code
is a unique logical id used for deterministic tie-breaks.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "DenseWorkload", "make", "CONFIGS", "bf16_round", "morton2", "morton3",
    "permute_storage", "custom_block_workload", "resblock_weights", "sdf_lattice", "split_gates",
    "view_cameras", "reference_view_blocks",
]


# ----------------------------------------------------------------------------------------------
# small helpers (input preparation only)
# ----------------------------------------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bfloat16 (ties to even); float32 storage."""
    a = np.array(x, dtype=np.float32, copy=True, order="C")
    u = a.view(np.uint32)
    lsb = u >> 16
    lsb &= 1
    lsb += 0x7FFF
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return a


def _spread3(v: np.ndarray) -> np.ndarray:
    v = v.astype(np.uint64) & 0x1FFFFF
    v = (v | (v << 32)) & 0x1F00000000FFFF
    v = (v | (v << 16)) & 0x1F0000FF0000FF
    v = (v | (v << 8)) & 0x100F00F00F00F00F
    v = (v | (v << 4)) & 0x10C30C30C30C30C3
    v = (v | (v << 2)) & 0x1249249249249249
    return v


def _spread2(v: np.ndarray) -> np.ndarray:
    v = v.astype(np.uint64) & 0xFFFFFFFF
    v = (v | (v << 16)) & 0x0000FFFF0000FFFF
    v = (v | (v << 8)) & 0x00FF00FF00FF00FF
    v = (v | (v << 4)) & 0x0F0F0F0F0F0F0F0F
    v = (v | (v << 2)) & 0x3333333333333333
    v = (v | (v << 1)) & 0x5555555555555555
    return v


def morton3(x, y, z) -> np.ndarray:
    """3D Morton code, bits interleaved x (least significant), y, z."""
    return _spread3(np.asarray(x)) | (_spread3(np.asarray(y)) << 1) | (_spread3(np.asarray(z)) << 2)


def morton2(x, y) -> np.ndarray:
    """2D Morton code, bits interleaved x (least significant), y."""
    return _spread2(np.asarray(x)) | (_spread2(np.asarray(y)) << 1)


# ----------------------------------------------------------------------------------------------
# workload containers
# ----------------------------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    """A block-major NSA input.  Arrays are numpy; float data is float32 (bf16-representable
    when dtype == 'bf16').  Padding slots hold zeros."""
    name: str
    dtype: str                    # 'f32' or 'bf16'
    n_qh: int
    n_kvh: int
    head_dim: int
    blk_cap: int
    blk_cnt: np.ndarray           # int32 [n_blk], 1..cap
    blk_key: np.ndarray           # uint32 [n_blk], unique
    blk_type: np.ndarray          # int8 [n_blk]: 0 volume, 1 image
    pts: np.ndarray               # float32 [S, 3] in [-1, 1]; zeros on padding
    q: np.ndarray                 # float32 [S, n_qh, D]
    k: np.ndarray                 # float32 [S, n_kvh, D]
    v: np.ndarray                 # float32 [S, n_kvh, D]
    gates: np.ndarray             # float32 [S, n_qh, n_branch]
    top_k: int
    routing: str                  # 'geometric' or 'scores'
    q_gran: str                   # 'token' or 'block' (pooled queries for the compressed branch)
    branches: tuple               # subset of ('cmp', 'sel', 'loc'), in gate-channel order
    n_vol_tokens: int = 0
    n_img_tokens: int = 0
    meta: dict = dataclasses.field(default_factory=dict)

    @property
    def n_blk(self) -> int:
        return int(self.blk_cnt.shape[0])

    @property
    def n_slots(self) -> int:
        return self.n_blk * self.blk_cap

    @property
    def n_valid(self) -> int:
        return int(self.blk_cnt.sum())

    @property
    def scale(self) -> float:
        """Softmax scale: 1/sqrt(D), unless the input names another in meta['scale']."""
        return float(self.meta.get("scale", 1.0 / math.sqrt(self.head_dim)))

    def valid_mask(self) -> np.ndarray:
        slot = np.arange(self.n_slots)
        return (slot % self.blk_cap) < self.blk_cnt[slot // self.blk_cap]

    def valid_slots(self) -> np.ndarray:
        return np.nonzero(self.valid_mask())[0]


@dataclasses.dataclass
class DenseWorkload:
    """Stage-1 dense gated self/cross input: tokens [0, n_x) are volume (x), the rest image (y)."""
    name: str
    dtype: str
    n_qh: int
    n_kvh: int
    head_dim: int
    n_x: int
    q: np.ndarray                 # [N, n_qh, D]
    k: np.ndarray                 # [N, n_kvh, D]
    v: np.ndarray
    gates: np.ndarray             # [N, n_qh, 2] = (self, cross) logits
    meta: dict = dataclasses.field(default_factory=dict)

    @property
    def n_tok(self) -> int:
        return int(self.q.shape[0])

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# ----------------------------------------------------------------------------------------------
# geometry
# ----------------------------------------------------------------------------------------------

def _voxel_centres(idx: np.ndarray, side: int) -> np.ndarray:
    """Voxel integer coords [n,3] -> centres in [-1, 1]^3 (exact in float32 for side | 4096)."""
    return (-1.0 + (2.0 * idx.astype(np.float64) + 1.0) / side).astype(np.float32)


def _active_voxels(side: int, sdf, target: int) -> tuple:
    """The `target` voxels whose centres lie nearest the surface: a band |sdf(centre)| <= tau, with
    tau the target-th smallest |sdf| over the voxel centres (ties by voxel index), so the count is
    exact.  A plain surface band for shaping the input geometry; the method's own activation rule
    is not applied here.  sdf takes voxel-unit coordinates [n,3] and returns [n]."""
    g = np.arange(side, dtype=np.float64) + 0.5
    zz, yy, xx = np.meshgrid(g, g, g, indexing="ij")
    centres = np.stack([xx.ravel(), yy.ravel(), zz.ravel()], axis=1)
    a = np.abs(sdf(centres))
    order = np.argsort(a, kind="stable")
    active = np.sort(order[:target])
    tau = float(a[order[target - 1]])
    ix = active % side
    iy = (active // side) % side
    iz = active // (side * side)
    return np.stack([ix, iy, iz], axis=1).astype(np.int64), tau


def _fibonacci_dirs(n: int) -> np.ndarray:
    i = np.arange(n, dtype=np.float64) + 0.5
    phi = np.arccos(1.0 - 2.0 * i / n)
    theta = math.pi * (1.0 + 5.0 ** 0.5) * i
    return np.stack([np.cos(theta) * np.sin(phi), np.sin(theta) * np.sin(phi), np.cos(phi)], axis=1)


def _view_basis(d: np.ndarray):
    up = np.array([0.0, 0.0, 1.0]) if abs(d[2]) < 0.9 else np.array([1.0, 0.0, 0.0])
    r = np.cross(up, d)
    r /= np.linalg.norm(r)
    u = np.cross(d, r)
    return r, u


def _foreground_patches(side: int, frac: float) -> np.ndarray:
    """Patch (a, b) indices of the `frac` fraction nearest the view centre, ties by row-major index."""
    g = np.arange(side)
    b, a = np.meshgrid(g, g, indexing="ij")
    a = a.ravel()
    b = b.ravel()
    c = (side - 1) / 2.0
    d2 = (a - c) ** 2 + (b - c) ** 2
    order = np.lexsort((np.arange(side * side), d2))
    keep = np.sort(order[: int(round(frac * side * side))])
    return np.stack([a[keep], b[keep]], axis=1)


def _image_points(views: np.ndarray, patches: np.ndarray, side: int, centre: np.ndarray,
                  rho: float) -> np.ndarray:
    """Front-surface point of a sphere (centre, radius rho; normalised units) seen by an orthographic
    camera looking along -view.  The image plane half-extent is rho*sqrt(pi/2) so the silhouette
    covers half of the image.  Patches outside the silhouette use the nearest rim point."""
    half = rho * math.sqrt(math.pi / 2.0)
    out = []
    for d in views:
        r, u = _view_basis(d)
        x = (-1.0 + (2.0 * patches[:, 0] + 1.0) / side) * half
        y = (-1.0 + (2.0 * patches[:, 1] + 1.0) / side) * half
        rr = np.sqrt(x * x + y * y)
        s = np.where(rr > rho, rho / np.maximum(rr, 1e-30), 1.0)
        x, y = x * s, y * s
        depth = np.sqrt(np.maximum(rho * rho - x * x - y * y, 0.0))
        p = centre[None, :] + x[:, None] * r[None, :] + y[:, None] * u[None, :] + depth[:, None] * d[None, :]
        out.append(p)
    return np.clip(np.concatenate(out, axis=0), -1.0, 1.0).astype(np.float32)


# ----------------------------------------------------------------------------------------------
# block-major layout
# ----------------------------------------------------------------------------------------------

def _build_layout(groups, cap: int):
    """groups: list of (type, view, cell_codes[n], token_order_codes[n], pts[n,3]).  Tokens are
    grouped by (type, view, cell); blocks are emitted in list order then by cell code; inside a block
    tokens follow token_order_codes."""
    cnts, keys, types, pts_rows, slot_of = [], [], [], [], []
    n_blk = 0
    for typ, view, cell, tok, pts in groups:
        order = np.lexsort((tok, cell))
        cell_s = cell[order]
        uniq, start, count = np.unique(cell_s, return_index=True, return_counts=True)
        if count.max() > cap:
            raise ValueError("a cell holds more tokens than the block capacity")
        blk_of_tok = np.repeat(np.arange(uniq.shape[0]), count)
        rank = np.arange(cell_s.shape[0]) - np.repeat(start, count)
        cnts.append(count.astype(np.int32))
        keys.append(((np.uint64(typ) << np.uint64(31)) | (np.uint64(view) << np.uint64(20))
                     | uniq.astype(np.uint64)).astype(np.uint32))
        types.append(np.full(uniq.shape[0], typ, dtype=np.int8))
        slot_of.append(((blk_of_tok + n_blk) * cap + rank).astype(np.int64))
        pts_rows.append(pts[order])
        n_blk += uniq.shape[0]
    blk_cnt = np.concatenate(cnts)
    blk_key = np.concatenate(keys)
    blk_type = np.concatenate(types)
    slots = np.concatenate(slot_of)
    S = n_blk * cap
    pts = np.zeros((S, 3), dtype=np.float32)
    pts[slots] = np.concatenate(pts_rows)
    return blk_cnt, blk_key, blk_type, pts, slots


def _draw_tensors(rng, S, slots, n_qh, n_kvh, D, n_gate, dtype):
    nv = slots.shape[0]
    order = np.sort(slots)

    def draw(h):
        a = np.zeros((S, h, D), dtype=np.float32)
        x = rng.standard_normal((nv, h, D), dtype=np.float32)
        a[order] = bf16_round(x) if dtype == "bf16" else x
        return a

    q = draw(n_qh)
    k = draw(n_kvh)
    v = draw(n_kvh)
    g = np.zeros((S, n_qh, n_gate), dtype=np.float32)
    x = rng.standard_normal((nv, n_qh, n_gate), dtype=np.float32)
    g[order] = bf16_round(x) if dtype == "bf16" else x
    return q, k, v, g


# ----------------------------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------------------------

def _sphere_sdf(c, r):
    return lambda p: np.linalg.norm(p - c[None, :], axis=1) - r


def _sphere_torus_sdf(side, ph):
    """Noisy union of a sphere and a torus centred in a side^3 voxel grid; voxel-unit coordinates."""
    half = side / 2.0
    cen = np.full(3, half)
    r_s, R_t, r_t = 0.62 * half, 0.55 * half, 0.18 * half
    f = 2.0 * math.pi / (side / 4.0)

    def sdf(p):
        d = p - cen[None, :]
        s1 = np.linalg.norm(d, axis=1) - r_s
        q = np.sqrt(d[:, 0] ** 2 + d[:, 1] ** 2) - R_t
        s2 = np.sqrt(q * q + d[:, 2] ** 2) - r_t
        n = 1.5 * np.sin(f * p[:, 0] + ph[0]) * np.sin(f * p[:, 1] + ph[1]) * np.sin(f * p[:, 2] + ph[2])
        return np.minimum(s1, s2) + n

    return sdf


def sdf_lattice(w, G):
    """The SDF behind a geometric workload's volume, sampled at the (G)^3 lattice points
    -1 + 2 g / (G - 1) of [-1, 1]^3 in normalised units (float32 [G][G][G], z, y, x), with its
    activation threshold tau in the same units.  Returns (lattice, tau)."""
    m = w.meta
    side = int(m["vol_side"])
    half = side / 2.0
    if "sdf_phases" in m:
        sdf = _sphere_torus_sdf(side, np.array(m["sdf_phases"]))
    elif "sphere_centre" in m:
        sdf = _sphere_sdf(np.array(m["sphere_centre"]), float(m["sphere_radius"]))
    else:
        raise ValueError("workload %s carries no volume SDF" % w.name)
    g = np.linspace(-1.0, 1.0, G)
    zz, yy, xx = np.meshgrid(g, g, g, indexing="ij")
    p = (np.stack([xx.ravel(), yy.ravel(), zz.ravel()], axis=1) + 1.0) * half
    lat = (sdf(p) / half).reshape(G, G, G).astype(np.float32)
    return lat, float(m["tau"]) / half


def _lsrm_geometric(name, seed, dtype, vol_side, vol_shape, vol_target, n_views, img_side, fg,
                    top_k, n_qh=32, n_kvh=2, D=32, cap=64, vol_all=False, img_all_sphere=False):
    rng = np.random.default_rng(np.random.PCG64(seed))
    half = vol_side / 2.0
    meta = {"vol_side": vol_side}
    # --- geometry: volume ---
    if vol_all:
        g = np.arange(vol_side)
        zz, yy, xx = np.meshgrid(g, g, g, indexing="ij")
        vox = np.stack([xx.ravel(), yy.ravel(), zz.ravel()], axis=1).astype(np.int64)
        sph_c = np.zeros(3)
        sph_r = 1.0
    elif vol_shape == "sphere":
        cen = np.full(3, half) + rng.uniform(-2.0, 2.0, size=3)
        rad = rng.uniform(0.80, 0.90) * half
        vox, tau = _active_voxels(vol_side, _sphere_sdf(cen, rad), vol_target)
        sph_c = -1.0 + 2.0 * cen / vol_side
        sph_r = rad / half
        meta.update(tau=tau, sphere_centre=cen.tolist(), sphere_radius=rad)
    elif vol_shape == "sphere_torus":
        ph = rng.uniform(0.0, 2.0 * math.pi, size=3)
        vox, tau = _active_voxels(vol_side, _sphere_torus_sdf(vol_side, ph), vol_target)
        sph_c = np.zeros(3)
        sph_r = 0.62
        meta.update(tau=tau, sdf_phases=ph.tolist())
    else:
        raise ValueError(vol_shape)
    vol_pts = _voxel_centres(vox, vol_side)
    vol_cell = morton3(vox[:, 0] // 4, vox[:, 1] // 4, vox[:, 2] // 4)
    vol_tok = morton3(vox[:, 0], vox[:, 1], vox[:, 2])
    groups = [(0, 0, vol_cell, vol_tok, vol_pts)]
    # --- geometry: image ---
    if img_all_sphere:
        patches = _foreground_patches(img_side, 1.0)
        for vi in range(n_views):
            g3 = rng.standard_normal((patches.shape[0], 3))
            p = (g3 / np.linalg.norm(g3, axis=1, keepdims=True)).astype(np.float32)
            cell = morton2(patches[:, 0] // 8, patches[:, 1] // 8)
            tok = morton2(patches[:, 0], patches[:, 1])
            groups.append((1, vi, cell, tok, p))
    else:
        patches = _foreground_patches(img_side, fg)
        dirs = _fibonacci_dirs(n_views)
        meta.update(cam_dirs=dirs.tolist(), cam_centre=np.asarray(sph_c, dtype=np.float64).tolist(),
                    cam_half=float(sph_r * math.sqrt(math.pi / 2.0)), img_side=img_side, n_views=n_views)
        for vi in range(n_views):
            p = _image_points(dirs[vi:vi + 1], patches, img_side, sph_c, sph_r)
            cell = morton2(patches[:, 0] // 8, patches[:, 1] // 8)
            tok = morton2(patches[:, 0], patches[:, 1])
            groups.append((1, vi, cell, tok, p))
    blk_cnt, blk_key, blk_type, pts, slots = _build_layout(groups, cap)
    q, k, v, gates = _draw_tensors(rng, blk_cnt.shape[0] * cap, slots, n_qh, n_kvh, D, 3, dtype)
    n_img = sum(gr[2].shape[0] for gr in groups[1:])
    return Workload(name=name, dtype=dtype, n_qh=n_qh, n_kvh=n_kvh, head_dim=D, blk_cap=cap,
                    blk_cnt=blk_cnt, blk_key=blk_key, blk_type=blk_type, pts=pts, q=q, k=k, v=v,
                    gates=gates, top_k=top_k, routing="geometric", q_gran="token",
                    branches=("cmp", "sel", "loc"), n_vol_tokens=int(vox.shape[0]),
                    n_img_tokens=int(n_img), meta=meta)


def _speed3r(name, seed, dtype, n_views, side, cell=4, n_heads=16, D=64, top_k=16):
    """Speed3R-style multi-view grid: side x side patch tokens per view, padded up to a multiple of
    the 4x4 pooling cell; blocks are the non-empty cells (edge cells hold fewer tokens)."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    g = np.arange(side)
    b, a = np.meshgrid(g, g, indexing="ij")
    a = a.ravel()
    b = b.ravel()
    groups = []
    for vi in range(n_views):
        p = np.zeros((a.shape[0], 3), dtype=np.float32)
        p[:, 0] = -1.0 + (2.0 * a + 1.0) / side
        p[:, 1] = -1.0 + (2.0 * b + 1.0) / side
        groups.append((1, vi, morton2(a // cell, b // cell), morton2(a, b), p))
    blk_cnt, blk_key, blk_type, pts, slots = _build_layout(groups, cell * cell)
    q, k, v, gates = _draw_tensors(rng, blk_cnt.shape[0] * cell * cell, slots, n_heads, n_heads, D, 2, dtype)
    return Workload(name=name, dtype=dtype, n_qh=n_heads, n_kvh=n_heads, head_dim=D,
                    blk_cap=cell * cell, blk_cnt=blk_cnt, blk_key=blk_key, blk_type=blk_type, pts=pts,
                    q=q, k=k, v=v, gates=gates, top_k=top_k, routing="scores", q_gran="block",
                    branches=("cmp", "sel"), n_vol_tokens=0, n_img_tokens=int(slots.shape[0]))


def _dense(name, seed, dtype, vol_side, n_views, img_side, n_qh=32, n_kvh=2, D=32):
    rng = np.random.default_rng(np.random.PCG64(seed))
    n_x = vol_side ** 3
    n = n_x + n_views * img_side * img_side

    def draw(h):
        a = rng.standard_normal((n, h, D), dtype=np.float32)
        return bf16_round(a) if dtype == "bf16" else a

    q = draw(n_qh)
    k = draw(n_kvh)
    v = draw(n_kvh)
    g = rng.standard_normal((n, n_qh, 2), dtype=np.float32)
    if dtype == "bf16":
        g = bf16_round(g)
    return DenseWorkload(name=name, dtype=dtype, n_qh=n_qh, n_kvh=n_kvh, head_dim=D, n_x=n_x,
                         q=q, k=k, v=v, gates=g)


# name -> (builder, kwargs).  The five headline shapes and reduced variants of the same structure.
CONFIGS = {
    # tiny fp32 case: 8^3 voxel grid + 2 views x 16^2 patches with points on the unit sphere
    "tiny": (_lsrm_geometric, dict(seed=1000, dtype="f32", vol_side=8, vol_shape=None, vol_target=0,
                                   n_views=2, img_side=16, fg=1.0, top_k=4, vol_all=True,
                                   img_all_sphere=True)),
    # stage-1 dense gated self/cross attention: 16^3 volume + 12 views x 32^2
    "dense": (_dense, dict(seed=1001, dtype="bf16", vol_side=16, n_views=12, img_side=32)),
    "dense_small": (_dense, dict(seed=1101, dtype="bf16", vol_side=8, n_views=12, img_side=8)),
    # stage-2 sparse NSA, sphere shell in a 64^3 grid (~80k) + 16 views x 64^2 at 50% foreground
    "stage2": (_lsrm_geometric, dict(seed=1002, dtype="bf16", vol_side=64, vol_shape="sphere",
                                     vol_target=80000, n_views=16, img_side=64, fg=0.5, top_k=16)),
    "stage2_small": (_lsrm_geometric, dict(seed=1102, dtype="bf16", vol_side=16, vol_shape="sphere",
                                           vol_target=1250, n_views=16, img_side=16, fg=0.5, top_k=16)),
    # Speed3R-style score routing: 256 views x 37^2, 4x4 pooling cells, 16 heads of dim 64
    "speed3r": (_speed3r, dict(seed=1003, dtype="bf16", n_views=256, side=37)),
    "speed3r_small": (_speed3r, dict(seed=1103, dtype="bf16", n_views=4, side=37)),
    # large LSRM sparse stage: noisy sphere+torus in a 128^3 grid (~300k) + 16 views x 128^2 at 50%
    "large": (_lsrm_geometric, dict(seed=1004, dtype="bf16", vol_side=128, vol_shape="sphere_torus",
                                    vol_target=300000, n_views=16, img_side=128, fg=0.5, top_k=32)),
    "large_small": (_lsrm_geometric, dict(seed=1104, dtype="bf16", vol_side=32, vol_shape="sphere_torus",
                                          vol_target=4700, n_views=16, img_side=16, fg=0.5, top_k=32)),
}


def make(name: str, **overrides):
    """Build the named workload.  Keyword overrides replace builder arguments (e.g. dtype)."""
    fn, kw = CONFIGS[name]
    kw = dict(kw)
    kw.update(overrides)
    return fn(name=name, **kw)


def custom_block_workload(seed: int, blk_cnt, cap: int, n_qh: int, n_kvh: int, D: int, dtype: str,
                          top_k: int, pts_mode: str = "random", n_gate: int = 3, routing="geometric",
                          q_gran="token", branches=("cmp", "sel", "loc")) -> Workload:
    """Free-form block-major input (for edge cases): explicit per-block counts, random points in
    [-1,1]^3 (or 'lattice': a few coarse coordinates to create exact distance ties)."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    blk_cnt = np.asarray(blk_cnt, dtype=np.int32)
    n_blk = blk_cnt.shape[0]
    S = n_blk * cap
    slot = np.arange(S)
    valid = (slot % cap) < blk_cnt[slot // cap]
    slots = np.nonzero(valid)[0]
    pts = np.zeros((S, 3), dtype=np.float32)
    if pts_mode == "random":
        pts[slots] = rng.uniform(-1.0, 1.0, size=(slots.shape[0], 3)).astype(np.float32)
    elif pts_mode == "lattice":
        pts[slots] = (rng.integers(-2, 3, size=(slots.shape[0], 3)) * 0.25).astype(np.float32)
    else:
        raise ValueError(pts_mode)
    blk_key = rng.permutation(np.arange(n_blk, dtype=np.uint32) * 7 + 3).astype(np.uint32)
    q, k, v, gates = _draw_tensors(rng, S, slots, n_qh, n_kvh, D, n_gate, dtype)
    return Workload(name="custom", dtype=dtype, n_qh=n_qh, n_kvh=n_kvh, head_dim=D, blk_cap=cap,
                    blk_cnt=blk_cnt, blk_key=blk_key, blk_type=np.zeros(n_blk, dtype=np.int8),
                    pts=pts, q=q, k=k, v=v, gates=gates, top_k=top_k, routing=routing,
                    q_gran=q_gran, branches=tuple(branches))


def permute_storage(w: Workload, seed: int) -> tuple:
    """Return (w2, slot_map) where w2 stores the same logical tokens with the block storage order and
    the token order inside every block randomly permuted; slot_map[new_slot] = old_slot (-1 on
    padding).  blk_key travels with its block."""
    rng = np.random.default_rng(seed)
    cap = w.blk_cap
    perm_blk = rng.permutation(w.n_blk)
    slot_map = np.full(w.n_slots, -1, dtype=np.int64)
    for nb, ob in enumerate(perm_blk):
        c = int(w.blk_cnt[ob])
        inner = rng.permutation(c)
        slot_map[nb * cap: nb * cap + c] = ob * cap + inner
    src = np.where(slot_map >= 0, slot_map, 0)
    pad = slot_map < 0

    def move(a):
        b = a[src].copy()
        b[pad] = 0
        return b

    w2 = dataclasses.replace(w, blk_cnt=w.blk_cnt[perm_blk].copy(), blk_key=w.blk_key[perm_blk].copy(),
                             blk_type=w.blk_type[perm_blk].copy(), pts=move(w.pts), q=move(w.q),
                             k=move(w.k), v=move(w.v), gates=move(w.gates))
    return w2, slot_map


def resblock_weights(seed: int, n_heads: int, D: int):
    """Seeded weights of the residual module applied before block pooling (one per head):
    w1, w2 [H, D, D] ~ N(0, 1/D) and b1, b2 [H, D] ~ N(0, 0.1^2), float32."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    w1 = (rng.standard_normal((n_heads, D, D)) / np.sqrt(D)).astype(np.float32)
    b1 = (0.1 * rng.standard_normal((n_heads, D))).astype(np.float32)
    w2 = (rng.standard_normal((n_heads, D, D)) / np.sqrt(D)).astype(np.float32)
    b2 = (0.1 * rng.standard_normal((n_heads, D))).astype(np.float32)
    return w1, b1, w2, b2


def split_gates(w, seed: int) -> np.ndarray:
    """Gate logits for the split self/cross layer: [S, Hq, 7] iid N(0, 1) on valid slots (0 on
    padding), rounded to the workload's dtype; channel order (self, cross, own-cmp, own-sel,
    own-loc, other-cmp, other-sel)."""
    rng = np.random.default_rng(np.random.PCG64(seed))
    S = w.n_slots
    g = np.zeros((S, w.n_qh, 7), dtype=np.float32)
    vs = w.valid_slots()
    x = rng.standard_normal((vs.shape[0], w.n_qh, 7), dtype=np.float32)
    g[vs] = bf16_round(x) if w.dtype == "bf16" else x
    return g


def view_cameras(w, cell: int = 8):
    """The orthographic cameras of a geometric workload's image views, as the routing takes them:
    view_proj float32 [V, 2, 4], an affine map from a 3D point to continuous patch coordinates
    (a, b) of the view (patch (a, b) covers [a, a + 1) x [b, b + 1)), and cell_blk int32
    [V, side / cell, side / cell], the storage block of each (view, cell) or -1.  Returns
    (view_proj, cell_blk)."""
    m = w.meta
    side = int(m["img_side"])
    half = float(m["cam_half"])
    c = np.asarray(m["cam_centre"], dtype=np.float64)
    dirs = np.asarray(m["cam_dirs"], dtype=np.float64)
    k = side / (2.0 * half)
    proj = np.zeros((dirs.shape[0], 2, 4))
    for v, d in enumerate(dirs):
        r, u = _view_basis(d)
        for row, e in enumerate((r, u)):
            proj[v, row, :3] = e * k
            proj[v, row, 3] = side / 2.0 - float(c @ e) * k
    nc = side // cell
    cell_blk = np.full((dirs.shape[0], nc, nc), -1, dtype=np.int32)
    keys = w.blk_key.astype(np.int64)
    for b in np.nonzero(w.blk_type == 1)[0]:
        view = int((keys[b] >> 20) & 0x7FF)
        code = int(keys[b] & 0xFFFFF)
        cx = cy = 0
        for bit in range(10):
            cx |= ((code >> (2 * bit)) & 1) << bit
            cy |= ((code >> (2 * bit + 1)) & 1) << bit
        cell_blk[view, cy, cx] = b
    return proj.astype(np.float32), cell_blk


def reference_view_blocks(w, view: int = 0):
    """The storage block range (lo, hi) of one image view (by default the first, the reference
    frame of a multi-view sequence); its blocks are contiguous in storage."""
    keys = w.blk_key.astype(np.int64)
    b = np.nonzero((w.blk_type == 1) & (((keys >> 20) & 0x7FF) == view))[0]
    if b.shape[0] == 0:
        return (0, 0)
    assert np.all(np.diff(b) == 1), "a view's blocks are contiguous"
    return (int(b[0]), int(b[-1]) + 1)
