"""Python binding of libnsa (NSA forward pass for MI355X).

Argument marshalling only: every step runs in the HIP kernels of libnsa.so.  Tensors are torch
tensors on the GPU (PyTorch provides device memory and the current stream); each function checks
shapes, dtypes and contiguity, then calls the C ABI declared in include/nsa.h with raw pointers.
There is no CPU fallback: importing this package fails if the library has not been built, and any
call with tensors that are not on a GPU raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnsa.so")

NSA_OK, NSA_ERR_INVALID, NSA_ERR_UNSUPPORTED, NSA_ERR_HIP = 0, -1, -2, -3
NSA_F32, NSA_BF16 = 0, 1
BR_CMP, BR_SEL, BR_LOC = 1, 2, 4
Q_TOKEN, Q_BLOCK = 0, 1
EXPORTS = ("nsa_build_volume_blocks", "nsa_pool_blocks", "nsa_pool_blocks_resblock", "nsa_route_geometric",
           "nsa_route_geometric_range", "nsa_route_geometric_views", "nsa_attn_fwd_range", "nsa_route_scores_topk", "nsa_attn_fwd",
           "nsa_attn_fwd_forced", "nsa_attn_fwd_scores_routed",
           "nsa_gate_combine", "dense_gated_xattn_fwd", "nsa_route_geometric_noalloc", "nsa_last_error")


class NsaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("libnsa status %d: %s" % (status, msg))
        self.status = status


class Layout(ctypes.Structure):
    _fields_ = [("n_blk", ctypes.c_int32), ("blk_cap", ctypes.c_int32), ("n_qh", ctypes.c_int32),
                ("n_kvh", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("scale", ctypes.c_float),
                ("blk_cnt", ctypes.c_void_p), ("blk_key", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libnsa.so is not built; run `python sparse_attention_feed_amd/build.py` first (%s)"
                          % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I, U, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float
    LP = ctypes.POINTER(Layout)
    sig = {
        "nsa_build_volume_blocks": [P, I, I, F, I, P, P, P, P, P, P, P],
        "nsa_pool_blocks": [LP, I, I, P, P, P],
        "nsa_pool_blocks_resblock": [LP, I, I, P, P, P, P, P, P, P],
        "nsa_route_geometric": [LP, P, I, P, P, P, P],
        "nsa_route_geometric_noalloc": [LP, P, I, P, P, P],
        "nsa_route_geometric_range": [LP, P, I, I, I, I, I, P, P, P, P],
        "nsa_route_geometric_views": [LP, P, I, I, I, P, P, I, I, I, P, P, P, P, P],
        "nsa_attn_fwd_range": [LP, I, U, I, I, I, I, P, P, P, P, P, P, I, I, P, I, P, P, P],
        "nsa_route_scores_topk": [LP, I, I, P, P, P, I, P, P],
        "nsa_attn_fwd": [LP, I, U, I, P, P, P, P, P, P, P, I, I, P, P, P, P],
        "nsa_attn_fwd_forced": [LP, I, U, I, P, P, P, P, P, P, P, I, I, I, I, P, P, P, P],
        "nsa_attn_fwd_scores_routed": [LP, I, P, P, P, P, P, P, I, P, P, P, P],
        "nsa_gate_combine": [I, I, I, I, I, ctypes.POINTER(ctypes.c_void_p), P, P, P],
        "dense_gated_xattn_fwd": [I, I, I, I, I, I, F, P, P, P, P, P, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.nsa_last_error.argtypes = []
    lib.nsa_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def _check(status):
    if status != NSA_OK:
        raise NsaError(status, lib.nsa_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libnsa needs GPU tensors")
    if not t.is_contiguous():
        raise ValueError("libnsa needs contiguous tensors")
    return t.data_ptr()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return NSA_BF16
    if t.dtype == torch.float32:
        return NSA_F32
    raise ValueError("unsupported dtype %s" % t.dtype)


def validate_layout(blk_cnt, blk_key, blk_cap):
    """Host-side check of the layout preconditions the kernels assume without checking:
    1 <= blk_cnt[b] <= blk_cap and unique blk_key values.  Copies the tensors to the host (which
    synchronises a device); raises ValueError naming the first violation."""
    cnt = blk_cnt.detach().cpu().to(torch.int64)
    bad = torch.nonzero((cnt < 1) | (cnt > int(blk_cap))).flatten()
    if bad.numel():
        b = int(bad[0])
        raise ValueError("blk_cnt[%d] = %d is outside 1..%d" % (b, int(cnt[b]), int(blk_cap)))
    if blk_key is not None:
        key = blk_key.detach().cpu().to(torch.int64) & 0xFFFFFFFF
        if torch.unique(key).numel() != key.numel():
            raise ValueError("blk_key values are not unique")


class BlockLayout:
    """Block-major token layout: blk_cnt / blk_key device tensors plus the head shape.  With
    validate=True the preconditions are checked on the host first (validate_layout)."""

    def __init__(self, blk_cnt, blk_key, blk_cap, n_qh, n_kvh, head_dim, scale=None, validate=False):
        if validate:
            validate_layout(blk_cnt, blk_key, blk_cap)
        self.blk_cnt = blk_cnt
        self.blk_key = blk_key
        self.blk_cap = int(blk_cap)
        self.n_blk = int(blk_cnt.shape[0])
        self.n_qh, self.n_kvh, self.head_dim = int(n_qh), int(n_kvh), int(head_dim)
        self.scale = float(scale) if scale is not None else 1.0 / math.sqrt(head_dim)
        if blk_cnt.dtype != torch.int32:
            raise ValueError("blk_cnt must be int32")
        if blk_key is not None and blk_key.dtype not in (torch.int32, torch.uint32):
            raise ValueError("blk_key must be 32-bit")
        self._c = Layout(self.n_blk, self.blk_cap, self.n_qh, self.n_kvh, self.head_dim, self.scale,
                         _ptr(blk_cnt), _ptr(blk_key) if blk_key is not None else None)

    @property
    def n_slots(self):
        return self.n_blk * self.blk_cap

    @property
    def c(self):
        return ctypes.byref(self._c)


def volume_workspace(N, max_blk=None, device="cuda:0"):
    """Device buffers for build_volume_blocks: cell_mask, cell_block, n_blk, blk_cnt, blk_key, pts."""
    n_cells = (N // 4) ** 3
    max_blk = n_cells if max_blk is None else int(max_blk)
    m = max(max_blk, 1)
    return {
        "max_blk": max_blk,
        "cell_mask": torch.empty(n_cells, dtype=torch.int64, device=device),
        "cell_block": torch.empty(n_cells, dtype=torch.int32, device=device),
        "n_blk": torch.zeros(1, dtype=torch.int32, device=device),
        "blk_cnt": torch.empty(m, dtype=torch.int32, device=device),
        "blk_key": torch.empty(m, dtype=torch.int32, device=device),
        "pts": torch.empty((m * 64, 3), dtype=torch.float32, device=device),
    }


def build_volume_blocks(sdf, N, tau, max_blk=None, workspace=None, sync=True):
    """Active voxels of an N^3 grid (eq. M^vol on the trilinear SDF lattice `sdf` [G, G, G]) grouped
    into Morton-ordered 4^3-voxel blocks.  With sync (default) returns (n_blk, blk_cnt, blk_key, pts)
    cut to n_blk and raises if n_blk exceeds max_blk (default: every cell); without, launches
    asynchronously and returns the workspace (n_blk stays on the device)."""
    G = int(sdf.shape[0])
    if sdf.dtype != torch.float32 or tuple(sdf.shape) != (G, G, G):
        raise ValueError("sdf must be a float32 [G, G, G] lattice")
    ws = volume_workspace(N, max_blk, sdf.device) if workspace is None else workspace
    if ws["cell_mask"].shape[0] != (N // 4) ** 3:
        raise ValueError("workspace was made for another grid size")
    mb = ws["max_blk"]
    _check(lib.nsa_build_volume_blocks(_ptr(sdf), G, int(N), float(tau), mb, _ptr(ws["cell_mask"]),
                                       _ptr(ws["cell_block"]), _ptr(ws["n_blk"]), _ptr(ws["blk_cnt"]),
                                       _ptr(ws["blk_key"]), _ptr(ws["pts"]), _stream()))
    if not sync:
        return ws
    nb = int(ws["n_blk"].item())
    if nb > mb:
        raise ValueError("%d blocks exceed max_blk = %d" % (nb, mb))
    return nb, ws["blk_cnt"][:nb], ws["blk_key"][:nb], ws["pts"][:nb * 64]


def pool_blocks(layout: BlockLayout, x, out=None):
    """Mean of each block's valid token rows: x [S, H, D] -> [n_blk, H, D]."""
    S, H, D = x.shape
    assert S == layout.n_slots and D == layout.head_dim
    if out is None:
        out = torch.empty((layout.n_blk, H, D), dtype=x.dtype, device=x.device)
    _check(lib.nsa_pool_blocks(layout.c, _dtype(x), H, _ptr(x), _ptr(out), _stream()))
    return out


def pool_blocks_resblock(layout: BlockLayout, x, w1, b1, w2, b2, out=None):
    """Mean over each block's valid tokens of x + W2 silu(W1 x + b1) + b2 (one residual MLP per
    head; weights float32 [H, D, D], biases [H, D]): x [S, H, D] -> [n_blk, H, D]."""
    S, H, D = x.shape
    assert S == layout.n_slots and D == layout.head_dim
    for t, shape in ((w1, (H, D, D)), (w2, (H, D, D)), (b1, (H, D)), (b2, (H, D))):
        if t.dtype != torch.float32 or tuple(t.shape) != shape:
            raise ValueError("resblock weights must be float32 of shapes [H, D, D] / [H, D]")
    if out is None:
        out = torch.empty((layout.n_blk, H, D), dtype=x.dtype, device=x.device)
    _check(lib.nsa_pool_blocks_resblock(layout.c, _dtype(x), H, _ptr(x), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2),
                                        _ptr(out), _stream()))
    return out


def route_geometric(layout: BlockLayout, pts, top_k, sel=None, sel_d2=None, centroids=None, want_d2=True,
                    q_blocks=None, kv_blocks=None):
    """Top-k nearest blocks per token on the integer lattice; returns (sel, sel_d2, centroids).
    With q_blocks / kv_blocks = (lo, hi): only the slots of those query blocks are routed, among
    the candidate blocks kv_blocks (nsa_route_geometric_range)."""
    S = layout.n_slots
    assert pts.shape == (S, 3) and pts.dtype == torch.float32
    dev = pts.device
    if sel is None:
        sel = torch.empty((S, top_k), dtype=torch.int32, device=dev)
    if want_d2 and sel_d2 is None:
        sel_d2 = torch.empty((S, top_k), dtype=torch.int32, device=dev)
    if centroids is None:
        centroids = torch.empty((layout.n_blk, 4), dtype=torch.int32, device=dev)
    if q_blocks is None and kv_blocks is None:
        _check(lib.nsa_route_geometric(layout.c, _ptr(pts), int(top_k), _ptr(centroids), _ptr(sel),
                                       _ptr(sel_d2) if want_d2 else None, _stream()))
    else:
        ql, qh = (0, layout.n_blk) if q_blocks is None else q_blocks
        kl, kh = (0, layout.n_blk) if kv_blocks is None else kv_blocks
        _check(lib.nsa_route_geometric_range(layout.c, _ptr(pts), int(top_k), int(ql), int(qh), int(kl), int(kh),
                                             _ptr(centroids), _ptr(sel), _ptr(sel_d2) if want_d2 else None,
                                             _stream()))
    return sel, sel_d2, centroids


def route_geometric_views(layout: BlockLayout, pts, top_k, n_vol_blk, view_proj, cell_blk, cell_size=8,
                          radius=1, sel=None, sel_d2=None, centroids=None, geom=None, want_d2=True):
    """Top-k blocks per token: volume blocks [0, n_vol_blk) by centroid distance, image blocks found
    by projecting the token into every view (view_proj [V, 2, 4], cell_blk [V, n_cell, n_cell]) and
    ranked by their nearest member; returns (sel, sel_d2, centroids)."""
    S = layout.n_slots
    dev = pts.device
    if sel is None:
        sel = torch.empty((S, top_k), dtype=torch.int32, device=dev)
    if want_d2 and sel_d2 is None:
        sel_d2 = torch.empty((S, top_k), dtype=torch.int32, device=dev)
    if centroids is None:
        centroids = torch.empty((layout.n_blk, 4), dtype=torch.int32, device=dev)
    if geom is None:
        geom = torch.empty(layout.n_blk * 8 + S * 2, dtype=torch.int32, device=dev)
    n_views = int(view_proj.shape[0])
    n_cell = int(cell_blk.shape[1])
    if n_views and (tuple(view_proj.shape) != (n_views, 2, 4) or tuple(cell_blk.shape) != (n_views, n_cell, n_cell)):
        raise ValueError("view_proj must be [V, 2, 4] and cell_blk [V, n_cell, n_cell]")
    _check(lib.nsa_route_geometric_views(layout.c, _ptr(pts), int(top_k), int(n_vol_blk), n_views,
                                         _ptr(view_proj), _ptr(cell_blk), n_cell, int(cell_size), int(radius),
                                         _ptr(centroids), _ptr(geom), _ptr(sel),
                                         _ptr(sel_d2) if want_d2 else None, _stream()))
    return sel, sel_d2, centroids


def route_scores_topk(layout: BlockLayout, q, k_cmp, lse, top_k, q_gran=Q_TOKEN, sel=None):
    """Top-k blocks by compressed score (GQA: summed group probability, needs lse; one query head
    per KV head: raw score).  Returns sel [rows, n_kvh, top_k]."""
    rows = layout.n_slots if q_gran == Q_TOKEN else layout.n_blk
    if sel is None:
        sel = torch.empty((rows, layout.n_kvh, top_k), dtype=torch.int32, device=q.device)
    _check(lib.nsa_route_scores_topk(layout.c, _dtype(q), int(q_gran), _ptr(q), _ptr(k_cmp),
                                     _ptr(lse), int(top_k), _ptr(sel), _stream()))
    return sel


def attn_fwd(layout: BlockLayout, branches, q, k=None, v=None, q_cmp=None, k_cmp=None, v_cmp=None,
             sel=None, top_k=0, sel_groups=1, gates=None, out=None, lse=None, q_gran=Q_TOKEN,
             q_blocks=None, kv_blocks=None, gate_channel=0, forced=None):
    """NSA branches (bitmask of BR_CMP | BR_SEL | BR_LOC), gated and fused when gates is given.
    With q_blocks / kv_blocks = (lo, hi) (nsa_attn_fwd_range): only those query blocks are
    computed, against the key blocks kv_blocks; the named branches then read the gate channels
    gate_channel, gate_channel + 1, ... of gates [S, Hq, C].  With forced = (lo, hi)
    (nsa_attn_fwd_forced) the selected branch also attends every block of [lo, hi)."""
    if out is None:
        out = torch.empty_like(q)
    if forced is not None:
        if q_blocks is not None or kv_blocks is not None or gate_channel != 0:
            raise ValueError("a forced block range does not combine with block ranges")
        _check(lib.nsa_attn_fwd_forced(layout.c, _dtype(q), int(branches), int(q_gran), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(q_cmp), _ptr(k_cmp), _ptr(v_cmp), _ptr(sel), int(top_k),
                                       int(sel_groups), int(forced[0]), int(forced[1]), _ptr(gates), _ptr(out),
                                       _ptr(lse), _stream()))
        return out
    if q_blocks is None and kv_blocks is None and gate_channel == 0:
        _check(lib.nsa_attn_fwd(layout.c, _dtype(q), int(branches), int(q_gran), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(q_cmp), _ptr(k_cmp), _ptr(v_cmp), _ptr(sel), int(top_k), int(sel_groups),
                                _ptr(gates), _ptr(out), _ptr(lse), _stream()))
        return out
    if q_gran != Q_TOKEN:
        raise ValueError("block ranges take per-token queries")
    ql, qh = (0, layout.n_blk) if q_blocks is None else q_blocks
    kl, kh = (0, layout.n_blk) if kv_blocks is None else kv_blocks
    gp, gs = None, 0
    if gates is not None:
        if not gates.is_contiguous() or gates.dim() != 3:
            raise ValueError("gates must be a contiguous [S, Hq, C] tensor")
        gs = int(gates.shape[2])
        if not 0 <= gate_channel < gs:
            raise ValueError("gate_channel out of range")
        gp = ctypes.c_void_p(_ptr(gates) + int(gate_channel) * gates.element_size())
    _check(lib.nsa_attn_fwd_range(layout.c, _dtype(q), int(branches), int(ql), int(qh), int(kl), int(kh), _ptr(q),
                                  _ptr(k), _ptr(v), _ptr(k_cmp), _ptr(v_cmp), _ptr(sel), int(top_k), int(sel_groups),
                                  gp, gs, _ptr(out), _ptr(lse), _stream()))
    return out


def attn_fwd_scores_routed(layout: BlockLayout, q, k, v, q_cmp, k_cmp, v_cmp, top_k, gates, out=None, sel=None):
    """Compressed + selected branches with block queries, the routing taken from the compressed
    pass's own scores (nsa_attn_fwd_scores_routed).  Returns (out, sel [n_blk, n_kvh, top_k])."""
    if out is None:
        out = torch.empty_like(q)
    if sel is None:
        sel = torch.empty((layout.n_blk, layout.n_kvh, top_k), dtype=torch.int32, device=q.device)
    _check(lib.nsa_attn_fwd_scores_routed(layout.c, _dtype(q), _ptr(q), _ptr(k), _ptr(v), _ptr(q_cmp), _ptr(k_cmp),
                                          _ptr(v_cmp), int(top_k), _ptr(gates), _ptr(out), _ptr(sel), _stream()))
    return out, sel


def gate_combine(outs, gates, out=None):
    n_rows, n_qh, D = outs[0].shape
    if out is None:
        out = torch.empty_like(outs[0])
    arr = (ctypes.c_void_p * len(outs))(*[_ptr(o) for o in outs])
    _check(lib.nsa_gate_combine(_dtype(outs[0]), n_rows, n_qh, D, len(outs), arr, _ptr(gates), _ptr(out),
                                _stream()))
    return out


def dense_gated_xattn(q, k, v, n_x, gates, scale=None, out=None):
    n_tok, n_qh, D = q.shape
    n_kvh = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check(lib.dense_gated_xattn_fwd(_dtype(q), n_tok, int(n_x), n_qh, n_kvh, D, float(scale), _ptr(q),
                                     _ptr(k), _ptr(v), _ptr(gates), _ptr(out), _stream()))
    return out


def nsa_split_layer(layout: BlockLayout, q, k, v, pts, n_x_blk, gates, top_k, ws=None):
    """Stage-2 layer with decoupled self and cross NSA: blocks [0, n_x_blk) hold volume tokens, the
    rest image tokens; each token gets sigmoid(g0) NSA(own type) + sigmoid(g1) NSA(other type),
    NSA(own) = CMP + SEL + LOC and NSA(other) = CMP + SEL over that type's blocks, each branch with
    its own sigmoid gate.  gates [S, Hq, 7] = (self, cross, own-cmp, own-sel, own-loc, other-cmp,
    other-sel).  A composition of library calls; `ws` may hold preallocated buffers."""
    ws = {} if ws is None else ws
    n = layout.n_blk
    S = layout.n_slots
    dev = q.device
    k_cmp = pool_blocks(layout, k, ws.get("k_cmp"))
    v_cmp = pool_blocks(layout, v, ws.get("v_cmp"))
    for name in ("sel_self", "sel_cross"):
        if ws.get(name) is None:
            ws[name] = torch.empty((S, top_k), dtype=torch.int32, device=dev)
    if ws.get("centroids") is None:
        ws["centroids"] = torch.empty((n, 4), dtype=torch.int32, device=dev)
    for name in ("o_self", "o_cross", "out"):
        if ws.get(name) is None:
            ws[name] = torch.empty_like(q)
    if ws.get("g_outer") is None:
        ws["g_outer"] = torch.empty((S, q.shape[1], 2), dtype=gates.dtype, device=dev)
    ws["g_outer"].copy_(gates[:, :, 0:2])
    x, y = (0, n_x_blk), (n_x_blk, n)
    for own, other in ((x, y), (y, x)):
        if own[0] == own[1]:
            continue
        route_geometric(layout, pts, top_k, sel=ws["sel_self"], centroids=ws["centroids"], want_d2=False,
                        q_blocks=own, kv_blocks=own)
        route_geometric(layout, pts, top_k, sel=ws["sel_cross"], centroids=ws["centroids"], want_d2=False,
                        q_blocks=own, kv_blocks=other)
        attn_fwd(layout, BR_CMP | BR_SEL | BR_LOC, q, k, v, k_cmp=k_cmp, v_cmp=v_cmp, sel=ws["sel_self"],
                 top_k=top_k, gates=gates, gate_channel=2, out=ws["o_self"], q_blocks=own, kv_blocks=own)
        attn_fwd(layout, BR_CMP | BR_SEL, q, k, v, k_cmp=k_cmp, v_cmp=v_cmp, sel=ws["sel_cross"], top_k=top_k,
                 gates=gates, gate_channel=5, out=ws["o_cross"], q_blocks=own, kv_blocks=other)
    gate_combine([ws["o_self"], ws["o_cross"]], ws["g_outer"], out=ws["out"])
    ws.update(k_cmp=k_cmp, v_cmp=v_cmp)
    return ws["out"]


def nsa_layer(layout: BlockLayout, q, k, v, pts, gates, top_k, ws=None):
    """One geometric-routed NSA layer: pool K and V, route, then the fused three-branch attention
    with the sigmoid gate.  `ws` may hold preallocated k_cmp, v_cmp, sel, centroids and out."""
    ws = {} if ws is None else ws
    k_cmp = pool_blocks(layout, k, ws.get("k_cmp"))
    v_cmp = pool_blocks(layout, v, ws.get("v_cmp"))
    sel, _, cent = route_geometric(layout, pts, top_k, sel=ws.get("sel"), centroids=ws.get("centroids"),
                                   want_d2=False)
    o = attn_fwd(layout, BR_CMP | BR_SEL | BR_LOC, q, k, v, k_cmp=k_cmp, v_cmp=v_cmp, sel=sel, top_k=top_k,
                 sel_groups=1, gates=gates, out=ws.get("out"))
    ws.update(k_cmp=k_cmp, v_cmp=v_cmp, sel=sel, centroids=cent, out=o)
    return o
