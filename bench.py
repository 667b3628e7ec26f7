"""Benchmark of one NSA layer forward (the LSRM sparse stage) on one MI355X.

A step is one pass of the whole hot path over the resident synthetic batch: block-mean pooling of
K and V, exact geometric routing (top-32 blocks per token), and the fused compressed + selected +
local attention with the three-way sigmoid gate.  Inputs are generated on the host (seeded) and
copied to HBM before timing.

Prints ONE JSON line.  Besides the throughput it reports, for the dominant stage (the attention
call: with bf16 inputs the fused compressed + local kernel, then the selected-branch kernel that
adds its gated result; `roofline.launches` names them), achieved algorithmic TFLOP/s against the
bf16 MFMA peak, the per-stage times measured with HIP events on the launch stream, per-branch
throughput, the fp64 CPU oracle timed on the host's cores on a bounded sample of the same workload,
and the same step measurements for the other four workloads (stage2, speed3r, dense, tiny) with
fewer steps.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn fwd tokens/sec + % bf16 MFMA peak, 1 MI355X, ~430k-token config"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (no sparsity)
PEAK_F32_TFLOPS = 157.3        # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_flops(w, sel):
    """4*D*Hq per attended (query, key) pair; only valid pairs count (no padding, no duplicates)."""
    cnt = w.blk_cnt.astype(np.int64)
    nv = int(cnt.sum())
    per = 4 * w.head_dim * w.n_qh
    cmp_pairs = nv * w.n_blk
    loc_pairs = int((cnt * cnt).sum())
    vm = w.valid_mask()
    s = sel[vm]
    s_cnt = np.where(s >= 0, cnt[np.clip(s, 0, None)], 0)
    sel_pairs = int(s_cnt.sum())
    return {"cmp": per * cmp_pairs, "sel": per * sel_pairs, "loc": per * loc_pairs}


def _source_digest():
    """Digest of the sources the fused attention kernel and its launch are built from."""
    import hashlib
    h = hashlib.sha256()
    for f in ("attn.hip", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "sparse_attention_feed_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


# the kernels one call of each timed attention stage launches, in order
LAUNCHES = {
    "attn_fused": {"bf16": ["nsa_attn_kernel (compressed + local branches, writes o)",
                            "sel_wave_kernel (selected branch, adds its gated result to o)"],
                   "f32": ["nsa_attn_kernel (all three branches)"]},
    "attn_routed": {"bf16": ["cmp_route_g1_kernel (compressed branch + score routing)",
                             "sel_g1_kernel (selected branch, adds to o)"]},
    "dense_gated_xattn": {"bf16": ["dense_xattn_kernel"]},
}


def measured_traffic(kernel, config):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter summary, if
    that summary was taken on the current kernel sources (same digest); otherwise None."""
    path = os.path.join(ROOT, "profiles", "%s_%s_hbm_traffic.md" % (kernel, config))
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                kk, vv = line[2:].split(": ", 1)
                vals[kk.strip()] = vv.strip().strip("`")
    if vals.get("source digest") != _source_digest():
        return None
    try:
        return float(vals["HBM bytes per launch"])
    except (KeyError, ValueError):
        return None


_CPU_W = None     # the workload the CPU-baseline workers read (inherited at fork)
_CPU_POOLED = None


def _oracle_rows(rows):
    """The oracle's layer on a chunk of query rows with the pooled K/V computed once beforehand:
    the same oracle functions that nsa_forward composes (routing, the branches, the gate)."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    w = _CPU_W
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        if hasattr(w, "n_x"):
            O.dense_gated_xattn(w.q, w.k, w.v, w.n_x, w.gates, w.scale, rows=rows)
        elif w.routing == "scores":
            O.nsa_forward(w, rows=rows)
        else:
            k_cmp, v_cmp = _CPU_POOLED
            sel_rows, _ = O.route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k, rows=rows)
            sel = np.full((w.n_slots, w.top_k), -1, dtype=np.int32)
            sel[rows] = sel_rows
            outs = []
            for name in w.branches:
                br = O.BRANCH_NAMES[name]
                if br == O.CMP:
                    oc, _ = O.attn_branch(O.CMP, w.q, k_cmp, v_cmp, w.blk_cnt, w.blk_cap, w.scale, rows=rows)
                elif br == O.SEL:
                    oc, _ = O.attn_branch(O.SEL, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, sel=sel, rows=rows)
                else:
                    oc, _ = O.attn_branch(O.LOC, w.q, w.k, w.v, w.blk_cnt, w.blk_cap, w.scale, rows=rows)
                outs.append(oc)
            O.gate_combine(outs, w.gates[rows])
    return len(rows), time.perf_counter() - t0


def cpu_baseline(w, budget_s):
    """The fp64 oracle on the host's cores: worker processes (one per core of this process's
    affinity, at most 16, each single-threaded) run chunks of randomly sampled query rows of the
    same workload until the time budget is spent.  Geometric workloads pool K and V once first
    (timed, and included in the extrapolated whole-layer rate).  Runs before any GPU work."""
    import concurrent.futures
    import multiprocessing
    global _CPU_W, _CPU_POOLED
    import oracle as O
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    rng = np.random.default_rng(123)
    vs = np.arange(w.n_tok) if hasattr(w, "n_x") else w.valid_slots()
    n_all = len(vs)
    _CPU_W = w
    t_setup = 0.0
    if not hasattr(w, "n_x") and w.routing != "scores":
        t0 = time.perf_counter()
        _CPU_POOLED = (O.pool_blocks(w.k, w.blk_cnt, w.blk_cap), O.pool_blocks(w.v, w.blk_cnt, w.blk_cap))
        t_setup = time.perf_counter() - t0
    # a probe chunk in this process sizes the chunks for the budget
    probe = np.sort(rng.choice(vs, min(8, n_all), replace=False))
    n_p, t_p = _oracle_rows(probe)
    per_row = t_p / n_p
    chunk = int(max(4, min(2048, 0.1 * budget_s / per_row)))
    n_chunks = max(cores, int(budget_s * cores / (per_row * chunk)))
    ctx = multiprocessing.get_context("fork")
    t0 = time.perf_counter()
    done_rows = 0
    with concurrent.futures.ProcessPoolExecutor(max_workers=cores, mp_context=ctx) as ex:
        futs = [ex.submit(_oracle_rows, np.sort(rng.choice(vs, min(chunk, n_all), replace=False)))
                for _ in range(n_chunks)]
        for f in concurrent.futures.as_completed(futs):
            done_rows += f.result()[0]
    wall = time.perf_counter() - t0
    rate = done_rows / wall
    whole = n_all / (t_setup + n_all / rate)
    desc = ("%d random query tokens of the same workload in %d chunks on %d worker processes, %.1f s wall"
            % (done_rows, n_chunks, cores, wall))
    if t_setup:
        desc += ("; K/V pooling once %.1f s, included in value (whole-layer rate %.1f tokens/s = %d tokens / "
                 "(pooling + tokens / %.1f tokens/s))" % (t_setup, whole, n_all, rate))
    return {"value": round(whole, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "rows_per_s": round(rate, 2), "sample": desc}


def setup_geometric(w, S, torch, dev):
    import workloads as W
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v, g = (torch.from_numpy(getattr(w, n)).to(dev).to(dt).contiguous() for n in ("q", "k", "v", "gates"))
    pts = torch.from_numpy(w.pts).to(dev)
    L = S.BlockLayout(torch.from_numpy(w.blk_cnt).to(dev), torch.from_numpy(w.blk_key.view(np.int32)).to(dev),
                      w.blk_cap, w.n_qh, w.n_kvh, w.head_dim)
    ws = {
        "k_cmp": torch.empty((w.n_blk, w.n_kvh, w.head_dim), dtype=dt, device=dev),
        "v_cmp": torch.empty((w.n_blk, w.n_kvh, w.head_dim), dtype=dt, device=dev),
        "sel": torch.empty((w.n_slots, w.top_k), dtype=torch.int32, device=dev),
        "centroids": torch.empty((w.n_blk, 4), dtype=torch.int32, device=dev),
        "out": torch.empty_like(q),
    }

    def stages():
        return [
            ("pool_kv", lambda: (S.pool_blocks(L, k, ws["k_cmp"]), S.pool_blocks(L, v, ws["v_cmp"]))),
            ("route_geometric", lambda: S.route_geometric(L, pts, w.top_k, sel=ws["sel"],
                                                         centroids=ws["centroids"], want_d2=False)),
            ("attn_fused", lambda: S.attn_fwd(L, S.BR_CMP | S.BR_SEL | S.BR_LOC, q, k, v, k_cmp=ws["k_cmp"],
                                              v_cmp=ws["v_cmp"], sel=ws["sel"], top_k=w.top_k, gates=g,
                                              out=ws["out"])),
        ]

    def flops():
        out = algorithmic_flops(w, ws["sel"].cpu().numpy())
        # grouped-query score routing: the compressed pass (for the lse) and the group scores
        out["route_scores_gqa"] = out["cmp"] + 2 * w.head_dim * w.n_qh * int(w.blk_cnt.sum()) * w.n_blk
        return out

    def branch(bits):
        nb = bin(bits).count("1")
        gg = g[:, :, :nb].contiguous() if nb > 1 else None
        return lambda: S.attn_fwd(L, bits, q, k, v, k_cmp=ws["k_cmp"], v_cmp=ws["v_cmp"], sel=ws["sel"],
                                  top_k=w.top_k, gates=gg, out=ws["out"])

    combos = {"cmp": S.BR_CMP, "sel": S.BR_SEL, "loc": S.BR_LOC, "sel+loc": S.BR_SEL | S.BR_LOC}
    fns = {n: branch(b) for n, b in combos.items()}
    # the unfused alternative of the gate: a standalone combine of three branch outputs (HBM-bound);
    # its inputs are any three [S, Hq, D] tensors of the right shape
    extra = [q, torch.empty_like(q).copy_(q), torch.empty_like(q).copy_(q)]
    gout = torch.empty_like(q)
    fns["gate_combine_unfused"] = lambda: S.gate_combine(extra, g, out=gout)
    # compression through the residual module (seeded weights) in place of the plain block mean
    rb = [tuple(torch.from_numpy(a).to(dev) for a in W.resblock_weights(s, w.n_kvh, w.head_dim)) for s in (31, 32)]
    fns["pool_kv_resblock"] = lambda: (S.pool_blocks_resblock(L, k, *rb[0], out=ws["k_cmp"]),
                                       S.pool_blocks_resblock(L, v, *rb[1], out=ws["v_cmp"]))
    # the split self/cross form of the layer (volume blocks first, then image blocks)
    t = w.blk_type.astype(np.int64)
    if np.all(np.diff(t) >= 0):
        n_x_blk = int((t == 0).sum())
        g7 = torch.from_numpy(W.split_gates(w, 72)).to(dev).to(dt).contiguous()
        sws = {}
        fns["split_layer"] = lambda: S.nsa_split_layer(L, q, k, v, pts, n_x_blk, g7, w.top_k, ws=sws)
    # routing with the image blocks found through the views (radius 1: the 3 x 3 cells around the
    # projection in every view)
    if "cam_dirs" in w.meta:
        vp, cb = W.view_cameras(w)
        vp_d, cb_d = torch.from_numpy(vp).to(dev), torch.from_numpy(cb).to(dev)
        n_vol = int((w.blk_type == 0).sum())
        vsel = torch.empty((w.n_slots, w.top_k), dtype=torch.int32, device=dev)
        vcent = torch.empty((w.n_blk, 4), dtype=torch.int32, device=dev)
        vgeom = torch.empty(w.n_blk * 8 + w.n_slots * 2, dtype=torch.int32, device=dev)
        fns["route_views"] = lambda: S.route_geometric_views(L, pts, w.top_k, n_vol, vp_d, cb_d, cell_size=8, radius=1,
                                                             sel=vsel, centroids=vcent, geom=vgeom, want_d2=False)
    # score routing in grouped-query form, the alternative to geometric routing: the compressed
    # pass that gives every (token, head) its lse, then the top-k blocks by summed group probability
    if w.dtype == "bf16" and w.top_k <= 64:
        lse = torch.empty((w.n_slots, w.n_qh), dtype=torch.float32, device=dev)
        ssel = torch.empty((w.n_slots, w.n_kvh, w.top_k), dtype=torch.int32, device=dev)
        fns["route_scores_gqa"] = lambda: (
            S.attn_fwd(L, S.BR_CMP, q, k_cmp=ws["k_cmp"], v_cmp=ws["v_cmp"], lse=lse, out=ws["out"]),
            S.route_scores_topk(L, q, ws["k_cmp"], lse, w.top_k, sel=ssel))
    # the volume block table from the workload's SDF sampled on a (side + 1)^3 lattice
    if "tau" in w.meta:
        side = int(w.meta["vol_side"])
        lat, tau = W.sdf_lattice(w, side + 1)
        lat_d = torch.from_numpy(lat).to(dev)
        vws = S.volume_workspace(side, device=dev)
        fns["volume_blocks"] = lambda: S.build_volume_blocks(lat_d, side, tau, workspace=vws, sync=False)
    return stages, flops, fns, "attn_fused"


def setup_speed3r(w, S, torch, dev):
    import workloads as W
    dt = torch.bfloat16
    q, k, v, g = (torch.from_numpy(getattr(w, n)).to(dev).to(dt).contiguous() for n in ("q", "k", "v", "gates"))
    L = S.BlockLayout(torch.from_numpy(w.blk_cnt).to(dev), torch.from_numpy(w.blk_key.view(np.int32)).to(dev),
                      w.blk_cap, w.n_qh, w.n_kvh, w.head_dim)
    shp = (w.n_blk, w.n_kvh, w.head_dim)
    fr = W.reference_view_blocks(w)
    ws = {n: torch.empty(shp, dtype=dt, device=dev) for n in ("q_cmp", "k_cmp", "v_cmp")}
    ws["sel"] = torch.empty((w.n_blk, w.n_kvh, w.top_k), dtype=torch.int32, device=dev)
    ws["out"] = torch.empty_like(q)

    def stages():
        return [
            ("pool_qkv", lambda: (S.pool_blocks(L, q, ws["q_cmp"]), S.pool_blocks(L, k, ws["k_cmp"]),
                                  S.pool_blocks(L, v, ws["v_cmp"]))),
            # the routing comes out of the compressed branch's own pass (nsa_attn_fwd_scores_routed)
            ("attn_routed", lambda: S.attn_fwd_scores_routed(L, q, k, v, ws["q_cmp"], ws["k_cmp"], ws["v_cmp"],
                                                             w.top_k, g, out=ws["out"], sel=ws["sel"])),
        ]

    def flops():
        cnt = w.blk_cnt.astype(np.int64)
        per = 4 * w.head_dim
        sel = ws["sel"].cpu().numpy()                       # [n_blk, H, k]
        sel_cnt = np.where(sel >= 0, cnt[np.clip(sel, 0, None)], 0).sum(axis=2)   # [n_blk, H]
        out = {"cmp": per * w.n_blk * w.n_blk * w.n_qh,
               "sel": per * int((sel_cnt * cnt[:, None]).sum()),
               "route": per // 2 * w.n_blk * w.n_blk * w.n_qh}
        if fr[1] > fr[0]:
            # routed blocks outside the forced range (a routing row lists distinct blocks), plus the range
            inside = (sel >= fr[0]) & (sel < fr[1])
            keys = np.where((sel >= 0) & ~inside, cnt[np.clip(sel, 0, None)], 0).sum(axis=2) + cnt[fr[0]:fr[1]].sum()
            out["sel_forced_ref_frame"] = per * int((keys * cnt[:, None]).sum())
        return out

    def branch(bits):
        nb = bin(bits).count("1")
        gg = g[:, :, :nb].contiguous() if nb > 1 else None
        return lambda: S.attn_fwd(L, bits, q, k, v, q_cmp=ws["q_cmp"], k_cmp=ws["k_cmp"], v_cmp=ws["v_cmp"],
                                  sel=ws["sel"], top_k=w.top_k, sel_groups=w.n_kvh, gates=gg, out=ws["out"],
                                  q_gran=S.Q_BLOCK)

    fns = {"cmp": branch(S.BR_CMP), "sel": branch(S.BR_SEL),
           # the two-call sequence the fused pass replaces: stand-alone routing, then both branches
           "route": lambda: S.route_scores_topk(L, ws["q_cmp"], ws["k_cmp"], None, w.top_k, q_gran=S.Q_BLOCK,
                                                sel=ws["sel"]),
           "cmp+sel": branch(S.BR_CMP | S.BR_SEL)}
    if fr[1] > fr[0]:
        # the variant with a reference frame: its blocks are attended by every query
        fns["sel_forced_ref_frame"] = lambda: S.attn_fwd(
            L, S.BR_SEL, q, k, v, sel=ws["sel"], top_k=w.top_k, sel_groups=w.n_kvh, out=ws["out"],
            q_gran=S.Q_BLOCK, forced=fr)
    return stages, flops, fns, "attn_routed"


def setup_dense(w, S, torch, dev):
    dt = torch.bfloat16
    t = {n: torch.from_numpy(getattr(w, n)).to(dev).to(dt).contiguous() for n in ("q", "k", "v", "gates")}
    out = torch.empty_like(t["q"])

    def stages():
        return [("dense_gated_xattn", lambda: S.dense_gated_xattn(t["q"], t["k"], t["v"], w.n_x, t["gates"],
                                                                  out=out))]

    def flops():
        return {"dense": 4 * w.head_dim * w.n_qh * w.n_tok * w.n_tok}

    return stages, flops, {}, "dense_gated_xattn"


def describe(name, w, dense):
    if name == "large":
        return ("large: 128^3 volume (%d active surface voxels) + 16 views x 128^2 at 50%% foreground (%d), "
                "32q/2kv heads, D=32, 64-token blocks, top-%d geometric routing + local + compressed, "
                "3-way sigmoid gate" % (w.n_vol_tokens, w.n_img_tokens, w.top_k))
    if dense:
        return "%s: stage-1 dense gated self/cross attention, %d tokens (%d volume), 32q/2kv, D=32" % (
            name, w.n_tok, w.n_x)
    return "%s: %d tokens, %d blocks of %d, %dq/%dkv heads, D=%d, top-%d %s routing" % (
        name, w.n_valid, w.n_blk, w.blk_cap, w.n_qh, w.n_kvh, w.head_dim, w.top_k, w.routing)


def run_config(name, w, steps, warmup, breakdown_on, torch, S, dev):
    """Time `steps` layer steps of workload w (after `warmup` untimed ones) with HIP events on the
    launch stream; optionally time the per-branch and next-row items.  Returns a result dict."""
    import workloads as W
    dense = isinstance(w, W.DenseWorkload)
    n_tok = w.n_tok if dense else w.n_valid
    if dense:
        stages_fn, flops_fn, branches, dominant = setup_dense(w, S, torch, dev)
    elif w.routing == "scores":
        stages_fn, flops_fn, branches, dominant = setup_speed3r(w, S, torch, dev)
    else:
        stages_fn, flops_fn, branches, dominant = setup_geometric(w, S, torch, dev)
    stages = stages_fn()
    stream = torch.cuda.current_stream()

    def step(ev=None):
        for i, (_, fn) in enumerate(stages):
            if ev is not None:
                ev[i].record(stream)
            fn()
        if ev is not None:
            ev[len(stages)].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / steps
    kern_ms = {nm: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, (nm, _) in enumerate(stages)}
    value = n_tok / (ms_step * 1e-3)

    fl = flops_fn()
    # the dominant kernel's branches: routing runs in its own kernel, and the forced-range variant
    # and the score routing are separate breakdown items, not part of the timed step
    dom_flops = sum(v for kk, v in fl.items() if kk not in ("route", "sel_forced_ref_frame", "route_scores_gqa"))
    achieved = dom_flops / (kern_ms[dominant] * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    log("%s: step %.3f ms; %s; %s %.1f TFLOP/s" % (name, ms_step, ", ".join("%s %.3f" % kv for kv in kern_ms.items()),
                                                  dominant, achieved))

    breakdown = None
    if branches and breakdown_on:
        breakdown = {}
        for bname, fn in branches.items():
            for _ in range(2):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 5
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            if bname == "pool_kv_resblock":
                # K and V: 4*D^2 FLOP per valid token and KV head (two D x D products)
                f = 2 * 4 * w.head_dim * w.head_dim * w.n_kvh * int(w.blk_cnt.sum())
                breakdown[bname] = {"ms": round(ms, 4), "tflops": round(f / (ms * 1e-3) / 1e12, 2)}
                continue
            if bname == "route_views":
                breakdown[bname] = {"ms": round(ms, 4)}
                continue
            if bname == "split_layer":
                nt = int(w.blk_cnt.sum())
                breakdown[bname] = {"ms": round(ms, 4), "tokens_per_s": round(nt / (ms * 1e-3), 1)}
                continue
            if bname == "volume_blocks":
                # 64 trilinear SDF samples per voxel of the side^3 grid
                side = int(w.meta["vol_side"])
                nb = int(fn()["n_blk"].item())
                breakdown[bname] = {"ms": round(ms, 4), "n_blk": nb,
                                    "gvoxel_per_s": round(side ** 3 / (ms * 1e-3) / 1e9, 3)}
                continue
            if bname == "gate_combine_unfused":
                # bytes: three branch outputs and the gate logits read, the output written
                esz = 2 if w.dtype == "bf16" else 4
                nbytes = (4 * w.n_slots * w.n_qh * w.head_dim + w.n_slots * w.n_qh * 3) * esz
                breakdown[bname] = {"ms": round(ms, 4), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                    "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
                continue
            f = sum(fl[p] for p in bname.split("+"))
            breakdown[bname] = {"ms": round(ms, 4), "tflops": round(f / (ms * 1e-3) / 1e12, 1),
                                "mfma_frac": round(f / (ms * 1e-3) / 1e12 / peak, 4)}
        step()
        torch.cuda.synchronize()

    cfg = {"workload": describe(name, w, dense), "n_tokens": n_tok, "n_qh": w.n_qh, "n_kvh": w.n_kvh,
           "head_dim": w.head_dim}
    if not dense:
        cfg.update(n_blk=w.n_blk, blk_cap=w.blk_cap, top_k=w.top_k)
    return {
        "value": round(value, 1),
        "ms_per_step": round(ms_step, 4),
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "config": cfg,
        "roofline": {
            "kernel": dominant,
            "launches": LAUNCHES.get(dominant, {}).get("bf16" if w.dtype == "bf16" else "f32"),
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(dominant, name),
        },
        "kernels_ms": {kk: round(vv, 4) for kk, vv in kern_ms.items()},
        # geometric routing depends only on the token points, so a 24-layer model routes once per
        # instance: the step with its routing time spread over 24 layers (context, not `value`)
        "routing_amortised_24_layers": (
            {"ms_per_step": round(ms_step - kern_ms["route_geometric"] * 23 / 24, 4),
             "tokens_per_s": round(n_tok / ((ms_step - kern_ms["route_geometric"] * 23 / 24) * 1e-3), 1)}
            if "route_geometric" in kern_ms else None),
        "algorithmic_gflop": {kk: round(vv / 1e9, 2) for kk, vv in fl.items()},
        "branch_breakdown": breakdown,
    }


PROBES = {0: ("exp", 8, 0), 1: ("mfma", 0, 8), 2: ("mfma+exp", 16, 8), 3: ("fma", 8, 0), 4: ("mfma+fma", 32, 8),
          5: ("tile_pass", 0, 0)}


def run_probes():
    """Instruction-rate microbenchmarks (libnsa_probe.so): SIMD cycles per instruction (or per loop
    iteration for the mixes) from the shader clock, at 1, 2 and 4 waves per SIMD, and the attention
    kernel's own token pass on register-resident tiles (its compute ceiling)."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_feed_amd", "libnsa_probe.so"))
    lib.nsa_probe_run.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3
    lib.nsa_probe_run.restype = ctypes.c_int
    props = torch.cuda.get_device_properties(0)
    n_cu = props.multi_processor_count
    stream = torch.cuda.current_stream()
    out = {"n_cu": n_cu, "device": props.name, "probes": []}
    for which, (name, n_valu, n_mfma) in PROBES.items():
        for k in ((1, 2) if which == 5 else (1, 2, 4)):
            iters = 2000 if which == 5 else 20000
            sink = torch.empty(n_cu * 256 * k, dtype=torch.float32, device="cuda")
            cyc = torch.empty(n_cu * 4 * k, dtype=torch.int64, device="cuda")
            run = lambda: lib.nsa_probe_run(which, k, n_cu, iters, sink.data_ptr(), cyc.data_ptr(),  # noqa: E731
                                            ctypes.c_void_p(stream.cuda_stream))
            assert run() == 0
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            assert run() == 0
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            c = float(cyc.float().median().item())
            rec = {"probe": name, "waves_per_simd": k, "iters": iters, "ms": round(ms, 4),
                   "cycles_per_wave": c, "clock_ghz": round(c / (ms * 1e6), 3)}
            per_iter = c / (iters * k)                     # SIMD cycles per loop iteration
            if which == 5:
                passes = 8
                rec["simd_cycles_per_token_pass"] = round(per_iter / passes, 1)
                flop = n_cu * 4 * k * iters * passes * 131072
                rec["tflops"] = round(flop / (ms * 1e-3) / 1e12, 1)
                rec["frac_of_bf16_peak"] = round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
            elif n_mfma and n_valu:
                rec["simd_cycles_per_iteration"] = round(per_iter, 1)
                rec["instructions_per_iteration"] = {"mfma": n_mfma, "valu": n_valu}
            else:
                rec["simd_cycles_per_instruction"] = round(per_iter / (n_valu or n_mfma), 2)
            log(json.dumps(rec))
            out["probes"].append(rec)
    # HBM: a 4 GiB device-to-device copy (torch's copy kernel), read + write bytes over event time
    n = 1 << 30
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    rec = {"probe": "hbm_copy", "bytes_moved": 2 * 4 * n, "ms": round(ms, 4),
           "gbs": round(2 * 4 * n / (ms * 1e-3) / 1e9, 1)}
    log(json.dumps(rec))
    out["probes"].append(rec)
    return out


# the other workloads, timed after the headline one with fewer steps
OTHER_CONFIGS = ("stage2", "speed3r", "dense", "tiny")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="large")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="time the headline workload only")
    ap.add_argument("--config-steps", type=int, default=5, help="timed steps of each other workload")
    ap.add_argument("--probes", action="store_true",
                    help="run the instruction-rate microbenchmarks instead of the layer benchmark")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the timed region, copy 1 GiB device to device twice: the reference kernel "
                         "that scales rocprofv3's FETCH_SIZE / WRITE_SIZE readings to bytes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: libnsa has no multi-GPU path (the NSA layer would shard "
              "whole blocks across GPUs and all-gather the pooled K/V).", file=sys.stderr)
        sys.exit(2)

    if args.probes:
        print(json.dumps(run_probes()), flush=True)
        return

    import workloads as W

    t0 = time.time()
    w = W.make(args.config)
    log("workload %s (%.1fs)" % (args.config, time.time() - t0))
    # the CPU oracle first, in forked worker processes, before anything touches the GPU
    cpu = None
    if not args.no_cpu:
        log("timing the fp64 oracle on a bounded sample (~%.0f s)" % args.cpu_seconds)
        cpu = cpu_baseline(w, args.cpu_seconds)
        log("oracle: %.1f tokens/s on %d cores" % (cpu["value"], cpu["cores"]))

    import torch
    import sparse_attention_feed_amd as S
    dev = "cuda:0"
    head = run_config(args.config, w, args.steps, args.warmup, not args.no_breakdown, torch, S, dev)

    if args.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    others = None
    if not args.no_configs:
        others = {}
        del w
        torch.cuda.empty_cache()
        for name in OTHER_CONFIGS:
            if name == args.config:
                continue
            t0 = time.time()
            wo = W.make(name)
            log("workload %s (%.1fs)" % (name, time.time() - t0))
            r = run_config(name, wo, args.config_steps, 2, False, torch, S, dev)
            others[name] = {"ms_per_step": r["ms_per_step"], "tokens_per_s": r["value"], "dtype": r["dtype"],
                            "workload": r["config"]["workload"], "kernels_ms": r["kernels_ms"],
                            "dominant": {kk: r["roofline"][kk] for kk in ("kernel", "achieved", "peak", "unit",
                                                                          "frac")}}
            del wo
            torch.cuda.empty_cache()

    rec = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded; token geometry and head shapes of the pages' workloads)",
        "config": head["config"],
        "roofline": head["roofline"],
        "kernels_ms": head["kernels_ms"],
        "routing_amortised_24_layers": head["routing_amortised_24_layers"],
        "algorithmic_gflop": head["algorithmic_gflop"],
        "branch_breakdown": head["branch_breakdown"],
        "cpu_baseline": cpu,
        "gpu_over_oracle": round(head["value"] / cpu["value"], 1) if cpu else None,
        "other_configs": others,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
