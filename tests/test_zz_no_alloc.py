"""The allocation-free geometric routing entry point (centroids in the library's fixed device array)
against nsa_route_geometric with a caller workspace: identical routing rows and distances, bit for
bit, on two calls in a row, the second on a smaller layout (so that nothing of the first call's
centroids may leak into it)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _route_both(w):
    import sparse_attention_feed_amd as S
    d = to_dev(w)
    L = d["layout"]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    shape = (w.n_slots, w.top_k)
    sel_ref = torch.full(shape, -7, dtype=torch.int32, device="cuda")
    d2_ref = torch.full(shape, -7, dtype=torch.int32, device="cuda")
    cent = torch.empty((w.n_blk, 4), dtype=torch.int32, device="cuda")
    rc = S.lib.nsa_route_geometric(L.c, _p(d["pts"]), w.top_k, _p(cent), _p(sel_ref), _p(d2_ref), stream)
    assert rc == 0, S.lib.nsa_last_error()
    sel = torch.full(shape, -9, dtype=torch.int32, device="cuda")
    d2 = torch.full(shape, -9, dtype=torch.int32, device="cuda")
    rc = S.lib.nsa_route_geometric_noalloc(L.c, _p(d["pts"]), w.top_k, _p(sel), _p(d2), stream)
    assert rc == 0, S.lib.nsa_last_error()
    torch.cuda.synchronize()
    return sel.cpu().numpy(), d2.cpu().numpy(), sel_ref.cpu().numpy(), d2_ref.cpu().numpy()


def test_noalloc_routing_equals_workspace_routing_twice():
    big = W.make("large_small")
    small = W.custom_block_workload(91, [3, 64, 17, 1, 40, 8, 22], 64, 32, 2, 32, "bf16", 5)
    assert small.n_blk < big.n_blk
    for w in (big, small):
        say("route noalloc", w.name, "n_blk", w.n_blk, "k", w.top_k)
        sel, d2, sel_ref, d2_ref = _route_both(w)
        np.testing.assert_array_equal(sel, sel_ref)
        np.testing.assert_array_equal(d2, d2_ref)
        assert sel[w.valid_mask()].min() >= 0
