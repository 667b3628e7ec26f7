"""Helpers shared by the GPU parity tests: move a seeded workload to the device and compare."""
import sys

import numpy as np
import torch


def say(*a):
    """Name the case before each GPU step, flushed, so a failing run identifies it."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def tdt(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def to_dev(w, dev="cuda:0"):
    """Device tensors of a block-major workload (values already representable in its dtype)."""
    import sparse_attention_feed_amd as S
    dt = tdt(w)
    d = {
        "q": torch.from_numpy(w.q).to(dev).to(dt).contiguous(),
        "k": torch.from_numpy(w.k).to(dev).to(dt).contiguous(),
        "v": torch.from_numpy(w.v).to(dev).to(dt).contiguous(),
        "gates": torch.from_numpy(w.gates).to(dev).to(dt).contiguous(),
        "pts": torch.from_numpy(w.pts).to(dev).contiguous(),
        "blk_cnt": torch.from_numpy(w.blk_cnt.astype(np.int32)).to(dev),
        "blk_key": torch.from_numpy(w.blk_key.view(np.int32)).to(dev),
    }
    d["layout"] = S.BlockLayout(d["blk_cnt"], d["blk_key"], w.blk_cap, w.n_qh, w.n_kvh, w.head_dim, w.scale)
    return d


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def tol(w):
    """Output tolerance: max-abs 2e-2 for bf16 inputs, 1e-4 for fp32 inputs."""
    return 2e-2 if w.dtype == "bf16" else 1e-4


def rounded(x, dtype):
    """Round an oracle value to the storage dtype (for feeding oracle results back as inputs)."""
    import workloads as W
    x = np.asarray(x, dtype=np.float32)
    return W.bf16_round(x) if dtype == "bf16" else x


def max_err(a, b, mask=None):
    d = np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))
    if mask is not None:
        d = d[mask]
    return float(d.max()) if d.size else 0.0
