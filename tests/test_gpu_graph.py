"""The layer under HIP graph capture.  The library allocates, synchronises and clears nothing on its
own (every buffer is the caller's, every kernel is enqueued on the caller's stream), so a whole
layer can be captured once and replayed, as a serving loop would.  Every replay, with eager work
and synchronisations between the replays, must equal the eager result bit for bit: the kernels
are deterministic."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def _replays_equal_eager(step, outs_eager, reps=4):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        outs = step()
    for rep in range(reps):
        for o in outs:
            o.fill_(-7.0) if o.is_floating_point() else o.fill_(-7)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, outs_eager):
            assert torch.equal(o, e), ("replay", rep)


def test_geometric_layer_graph_replays():
    """Pooling, geometric routing and the fused three-branch gated attention (stage2_small)."""
    import sparse_attention_feed_amd as S
    w = W.make("stage2_small")
    d = to_dev(w)
    L = d["layout"]
    say("graph geometric layer", w.n_blk)
    ws = {}
    eager = S.nsa_layer(L, d["q"], d["k"], d["v"], d["pts"], d["gates"], w.top_k, ws=ws).clone()
    sel_eager = ws["sel"].clone()
    torch.cuda.synchronize()

    def step():
        o = S.nsa_layer(L, d["q"], d["k"], d["v"], d["pts"], d["gates"], w.top_k, ws=ws)
        return [o, ws["sel"]]
    _replays_equal_eager(step, [eager, sel_eager])


def test_score_routed_layer_graph_replays():
    """Pooling of Q, K and V and the fused compressed pass with its routing, then the selected
    branch (speed3r_small, the score-routed layout)."""
    import sparse_attention_feed_amd as S
    w = W.make("speed3r_small")
    d = to_dev(w)
    L = d["layout"]
    say("graph score-routed layer", w.n_blk)
    qc, kc, vc = (torch.empty((w.n_blk, w.n_qh, w.head_dim), dtype=d["q"].dtype, device="cuda") for _ in range(3))
    out = torch.empty_like(d["q"])
    sel = torch.empty((w.n_blk, w.n_kvh, w.top_k), dtype=torch.int32, device="cuda")

    def step():
        S.pool_blocks(L, d["q"], qc)
        S.pool_blocks(L, d["k"], kc)
        S.pool_blocks(L, d["v"], vc)
        S.attn_fwd_scores_routed(L, d["q"], d["k"], d["v"], qc, kc, vc, w.top_k, d["gates"], out=out, sel=sel)
        return [out, sel]
    step()
    torch.cuda.synchronize()
    eager = [out.clone(), sel.clone()]
    _replays_equal_eager(step, eager)
    assert np.all(sel.cpu().numpy() >= 0)
