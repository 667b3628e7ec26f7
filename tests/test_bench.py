"""Host-side checks of the benchmark script: the one-GPU contract, the algorithmic FLOP count
against a direct count of attended (query, key) pairs, and the traffic summary's source check."""
import os
import shutil
import subprocess
import sys

import numpy as np

import oracle as O
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert out.returncode != 0
    assert "one GPU" in out.stderr


def test_algorithmic_flops_count_valid_pairs():
    """FLOP = 4 D Hq per attended (query, key) pair: every valid query against every pooled block
    (compressed), the valid tokens of its own block (local) and of its routed blocks (selected)."""
    w = W.custom_block_workload(51, [5, 8, 1, 3, 8, 6, 2], 8, 4, 2, 8, "f32", 3)
    sel, _ = O.route_geometric(w.pts, w.blk_cnt, w.blk_key, w.blk_cap, w.top_k)
    fl = bench.algorithmic_flops(w, sel)
    per = 4 * w.head_dim * w.n_qh
    cmp_pairs = sel_pairs = loc_pairs = 0
    for s in w.valid_slots():
        b = s // w.blk_cap
        cmp_pairs += w.n_blk
        loc_pairs += int(w.blk_cnt[b])
        sel_pairs += sum(int(w.blk_cnt[x]) for x in set(sel[s].tolist()) if x >= 0)
    assert fl == {"cmp": per * cmp_pairs, "sel": per * sel_pairs, "loc": per * loc_pairs}


def test_measured_traffic_needs_matching_sources(tmp_path, monkeypatch):
    prof = os.path.join(ROOT, "profiles")
    fake = tmp_path / "profiles"
    shutil.copytree(prof, fake)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # the kernel sources of this tree are absent under tmp_path: copy them, then alter one byte
    csrc = tmp_path / "sparse_attention_feed_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "sparse_attention_feed_amd", "csrc"), csrc)
    path = fake / "attn_fused_large_hbm_traffic.md"
    text = path.read_text()
    digest = bench._source_digest()
    text = "\n".join(("- source digest: `%s`" % digest) if l.startswith("- source digest:") else l
                     for l in text.split("\n"))
    path.write_text(text)
    v = bench.measured_traffic("attn_fused", "large")
    assert v is not None and v > 1e9
    with open(csrc / "attn.hip", "a") as fh:
        fh.write("\n")
    assert bench.measured_traffic("attn_fused", "large") is None
    assert bench.measured_traffic("attn_fused", "no_such_config") is None
    assert np.isfinite(v)
