"""Benchmark of one NSA layer forward (the LSRM sparse stage) on one MI355X.

A step is one pass of the whole hot path over the resident synthetic batch: block-mean pooling of
K and V, exact geometric routing (top-32 blocks per token), and the fused compressed + selected +
local attention with the three-way sigmoid gate.  Inputs are generated on the host (seeded) and
copied to HBM before timing.

Prints ONE JSON line.  Besides the throughput it reports, for the dominant kernel (the fused
attention), achieved algorithmic TFLOP/s against the bf16 MFMA peak, the per-kernel times measured
with HIP events on the launch stream, per-branch throughput, and the fp64 CPU oracle timed on a
bounded sample of the same workload.
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


def cpu_baseline(w, budget_s):
    """fp64 oracle on a bounded sample of query rows of the same workload, one thread: a probe call
    of 16 rows sizes a second call that fills the time budget."""
    from threadpoolctl import threadpool_limits
    import oracle as O
    rng = np.random.default_rng(123)
    vs = w.valid_slots()
    with threadpool_limits(limits=1):
        rows = np.sort(rng.choice(vs, 16, replace=False))
        t0 = time.perf_counter()
        O.nsa_forward(w, rows=rows)
        t1 = time.perf_counter() - t0
        n2 = int(min(4096, max(16, (budget_s - t1) / (t1 / 16))))
        rows = np.sort(rng.choice(vs, n2, replace=False))
        t0 = time.perf_counter()
        O.nsa_forward(w, rows=rows)
        t2 = time.perf_counter() - t0
    n = 16 + n2
    return {"value": round(n / (t1 + t2), 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%d random query tokens of the same workload in two calls, %.1f s; every call also "
                      "pools all blocks and computes all block centroids" % (n, t1 + t2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="large")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the NSA layer would "
              "shard by whole blocks with an all-gather of pooled K/V; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_feed_amd as S
    import workloads as W

    t0 = time.time()
    w = W.make(args.config)
    log("workload %s: %d valid tokens, %d blocks, cap %d, top_k %d (%.1fs)" %
        (args.config, w.n_valid, w.n_blk, w.blk_cap, w.top_k, time.time() - t0))
    dev = "cuda:0"
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
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        S.pool_blocks(L, k, ws["k_cmp"])
        S.pool_blocks(L, v, ws["v_cmp"])
        if ev is not None:
            ev[1].record(stream)
        S.route_geometric(L, pts, w.top_k, sel=ws["sel"], centroids=ws["centroids"], want_d2=False)
        if ev is not None:
            ev[2].record(stream)
        S.attn_fwd(L, S.BR_CMP | S.BR_SEL | S.BR_LOC, q, k, v, k_cmp=ws["k_cmp"], v_cmp=ws["v_cmp"],
                   sel=ws["sel"], top_k=w.top_k, gates=g, out=ws["out"])
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    pool_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    route_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    attn_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    value = w.n_valid / (ms_step * 1e-3)

    sel = ws["sel"].cpu().numpy()
    fl = algorithmic_flops(w, sel)
    attn_flops = fl["cmp"] + fl["sel"] + fl["loc"]
    achieved = attn_flops / (attn_ms * 1e-3) / 1e12
    log("step %.3f ms: pool %.3f, route %.3f, attn %.3f ms; attention %.1f TFLOP/s" %
        (ms_step, pool_ms, route_ms, attn_ms, achieved))

    breakdown = None
    if not args.no_breakdown:
        breakdown = {}
        combos = {"cmp": S.BR_CMP, "sel": S.BR_SEL, "loc": S.BR_LOC, "sel+loc": S.BR_SEL | S.BR_LOC}
        for name, bits in combos.items():
            nb = bin(bits).count("1")
            gg = g[:, :, :nb].contiguous() if nb > 1 else None
            for _ in range(2):
                S.attn_fwd(L, bits, q, k, v, k_cmp=ws["k_cmp"], v_cmp=ws["v_cmp"], sel=ws["sel"], top_k=w.top_k,
                           gates=gg, out=ws["out"])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 5
            e0.record(stream)
            for _ in range(reps):
                S.attn_fwd(L, bits, q, k, v, k_cmp=ws["k_cmp"], v_cmp=ws["v_cmp"], sel=ws["sel"], top_k=w.top_k,
                           gates=gg, out=ws["out"])
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            f = sum(fl[p] for p in name.split("+"))
            breakdown[name] = {"ms": round(ms, 4), "tflops": round(f / (ms * 1e-3) / 1e12, 1),
                               "mfma_frac": round(f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        # restore the step's output
        step()
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu:
        log("timing the fp64 oracle on a bounded sample (~%.0f s)" % args.cpu_seconds)
        cpu = cpu_baseline(w, args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; shapes of the LSRM sparse stage)",
        "config": {
            "workload": "%s: 128^3 volume (%d active surface voxels) + 16 views x 128^2 at 50%% fg (%d), "
                        "32q/2kv heads, D=32, 64-token blocks, top-%d geometric routing + local + "
                        "compressed, 3-way sigmoid gate" % (args.config, w.n_vol_tokens, w.n_img_tokens, w.top_k)
            if args.config == "large" else args.config,
            "n_valid_tokens": w.n_valid, "n_blk": w.n_blk, "blk_cap": w.blk_cap, "top_k": w.top_k,
            "n_qh": w.n_qh, "n_kvh": w.n_kvh, "head_dim": w.head_dim,
        },
        "roofline": {
            "kernel": "nsa_attn_kernel (fused CMP+SEL+LOC+gate)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
        },
        "kernels_ms": {"pool_kv": round(pool_ms, 4), "route_geometric": round(route_ms, 4),
                       "attn_fused": round(attn_ms, 4)},
        "algorithmic_gflop": {kk: round(vv / 1e9, 2) for kk, vv in fl.items()},
        "branch_breakdown": breakdown,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
