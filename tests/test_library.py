"""Host-side tests of libnsa that need no GPU: the library loads, exports every symbol declared in
include/nsa.h, and rejects invalid arguments (or reports a forced launch failure) before any HIP
call is made."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nsa.h")
LIB = os.path.join(ROOT, "sparse_attention_feed_amd", "libnsa.so")



def test_library_is_built():
    """The boundary tests below need the library; a missing build is a failure, not a skip."""
    assert os.path.exists(LIB), "libnsa.so is not built: run __graft_entry__.build()"


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:nsa_status|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert "nsa_attn_fwd" in names and "dense_gated_xattn_fwd" in names and len(names) == 15
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(names) <= exported


def test_binding_names_match_header():
    import sparse_attention_feed_amd as S
    assert sorted(S.EXPORTS) == declared_functions()


@pytest.fixture()
def S():
    import sparse_attention_feed_amd as mod
    return mod


def layout(S, **kw):
    d = dict(n_blk=4, blk_cap=64, n_qh=32, n_kvh=2, head_dim=32, scale=0.17677669, blk_cnt=0x1000, blk_key=0x2000)
    d.update(kw)
    return S.Layout(d["n_blk"], d["blk_cap"], d["n_qh"], d["n_kvh"], d["head_dim"], d["scale"], d["blk_cnt"],
                    d["blk_key"])


FAKE = 0x10000   # never dereferenced: validation returns before any device work


def attn(S, L, **kw):
    a = dict(dtype=1, branches=7, q_gran=0, q=FAKE, k=FAKE, v=FAKE, q_cmp=None, k_cmp=FAKE, v_cmp=FAKE,
             sel=FAKE, top_k=4, sel_groups=1, gates=FAKE, o=FAKE, lse=None)
    a.update(kw)
    return S.lib.nsa_attn_fwd(ctypes.byref(L), a["dtype"], a["branches"], a["q_gran"], a["q"], a["k"], a["v"],
                              a["q_cmp"], a["k_cmp"], a["v_cmp"], a["sel"], a["top_k"], a["sel_groups"],
                              a["gates"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_blk=0), -1), (dict(blk_cap=65), -1), (dict(blk_cap=0), -1), (dict(n_qh=31), -1),
    (dict(scale=0.0), -1), (dict(scale=float("nan")), -1), (dict(blk_cnt=None), -1),
    (dict(head_dim=64), -2), (dict(n_qh=16, n_kvh=16), -2),
])
def test_attn_layout_validation(S, kw, status):
    assert attn(S, layout(S, **kw)) == status
    assert S.lib.nsa_last_error().decode().startswith("nsa_attn_fwd")


@pytest.mark.parametrize("kw", [
    dict(branches=0), dict(branches=8), dict(gates=None), dict(lse=FAKE), dict(q=None), dict(o=None),
    dict(k=None), dict(v_cmp=None), dict(sel=None), dict(top_k=0), dict(top_k=65), dict(sel_groups=3),
    dict(dtype=7), dict(q_gran=5), dict(branches=1, q_gran=1, q_cmp=None),
])
def test_attn_argument_validation(S, kw):
    assert attn(S, layout(S), **kw) == -1


def attn_range(S, L, **kw):
    a = dict(dtype=1, branches=7, q_lo=0, q_hi=4, kv_lo=0, kv_hi=4, q=FAKE, k=FAKE, v=FAKE, k_cmp=FAKE, v_cmp=FAKE,
             sel=FAKE, top_k=4, sel_groups=1, gates=FAKE, gate_stride=0, o=FAKE, lse=None)
    a.update(kw)
    return S.lib.nsa_attn_fwd_range(ctypes.byref(L), a["dtype"], a["branches"], a["q_lo"], a["q_hi"], a["kv_lo"],
                                    a["kv_hi"], a["q"], a["k"], a["v"], a["k_cmp"], a["v_cmp"], a["sel"], a["top_k"],
                                    a["sel_groups"], a["gates"], a["gate_stride"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw", [
    dict(q_lo=-1), dict(q_lo=3, q_hi=2), dict(q_hi=5), dict(kv_lo=-1), dict(kv_lo=4, kv_hi=3), dict(kv_hi=5),
    dict(gate_stride=2), dict(gate_stride=65), dict(gate_stride=-1), dict(branches=0), dict(o=None),
])
def test_attn_range_argument_validation(S, kw):
    assert attn_range(S, layout(S), **kw) == -1
    assert S.lib.nsa_last_error().decode().startswith("nsa_attn_fwd_range")


def test_attn_range_unsupported_and_forced(S, monkeypatch):
    g1 = layout(S, n_qh=16, n_kvh=16, head_dim=64, blk_cap=16)
    assert attn_range(S, g1, branches=3) == -2                      # the D = 64 kernels take no ranges
    monkeypatch.setenv("NSA_FORCE_HIP_ERROR", "1")
    assert attn_range(S, layout(S), q_lo=1, q_hi=3, kv_lo=2, kv_hi=4, gate_stride=7) == -3
    assert attn_range(S, layout(S), q_lo=2, q_hi=2, kv_lo=0, kv_hi=0) == -3   # empty ranges are valid


def attn_forced(S, L, lo, hi, **kw):
    a = dict(dtype=1, branches=3, q_gran=1, q=FAKE, k=FAKE, v=FAKE, q_cmp=FAKE, k_cmp=FAKE, v_cmp=FAKE,
             sel=FAKE, top_k=4, sel_groups=1, gates=FAKE, o=FAKE, lse=None)
    a.update(kw)
    return S.lib.nsa_attn_fwd_forced(ctypes.byref(L), a["dtype"], a["branches"], a["q_gran"], a["q"], a["k"],
                                     a["v"], a["q_cmp"], a["k_cmp"], a["v_cmp"], a["sel"], a["top_k"],
                                     a["sel_groups"], lo, hi, a["gates"], a["o"], a["lse"], None)


def test_attn_forced_validation(S, monkeypatch):
    g1 = layout(S, n_blk=400, n_qh=16, n_kvh=16, head_dim=64, blk_cap=16)
    for lo, hi in ((-1, 2), (3, 2), (0, 401)):
        assert attn_forced(S, g1, lo, hi) == -1, (lo, hi)
    assert attn_forced(S, g1, 0, 4, branches=1, sel=None) == -1            # forcing needs SEL
    assert S.lib.nsa_last_error().decode().startswith("nsa_attn_fwd_forced")
    assert attn_forced(S, g1, 0, 193) == -2                                 # more than 192 forced blocks
    assert attn_forced(S, layout(S), 0, 2, branches=7, q_gran=0) == -2     # grouped-query kernels: no forcing
    monkeypatch.setenv("NSA_FORCE_HIP_ERROR", "1")
    assert attn_forced(S, g1, 0, 192) == -3
    assert attn_forced(S, g1, 5, 5, branches=1, sel=None) == -3             # empty range: plain nsa_attn_fwd
    assert attn_forced(S, layout(S), 1, 1, branches=7, q_gran=0) == -3


def test_route_range_validation(S, monkeypatch):
    L = layout(S)
    r = S.lib.nsa_route_geometric_range
    assert r(ctypes.byref(L), FAKE, 4, 0, 5, 0, 4, FAKE, FAKE, None, None) == -1
    assert r(ctypes.byref(L), FAKE, 4, 0, 4, 3, 2, FAKE, FAKE, None, None) == -1
    assert r(ctypes.byref(L), FAKE, 0, 0, 4, 0, 4, FAKE, FAKE, None, None) == -1
    assert r(ctypes.byref(L), None, 4, 0, 4, 0, 4, FAKE, FAKE, None, None) == -1
    assert S.lib.nsa_last_error().decode().startswith("nsa_route_geometric_range")
    monkeypatch.setenv("NSA_FORCE_HIP_ERROR", "1")
    assert r(ctypes.byref(L), FAKE, 4, 1, 3, 0, 0, FAKE, FAKE, None, None) == -3


def test_route_views_validation(S, monkeypatch):
    L = layout(S)
    r = S.lib.nsa_route_geometric_views
    ok = dict(pts=FAKE, k=4, nv=2, views=3, proj=FAKE, cells=FAKE, n_cell=4, cell=8, radius=1, cent=FAKE, geom=FAKE,
              sel=FAKE)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return r(ctypes.byref(L), a["pts"], a["k"], a["nv"], a["views"], a["proj"], a["cells"], a["n_cell"], a["cell"],
                 a["radius"], a["cent"], a["geom"], a["sel"], None, None)
    for kw in (dict(nv=5), dict(nv=-1), dict(views=-1), dict(proj=None), dict(cells=None), dict(geom=None),
               dict(n_cell=0), dict(cell=6), dict(cell=2048), dict(radius=17), dict(k=0), dict(sel=None)):
        assert call(**kw) == -1, kw
    assert S.lib.nsa_last_error().decode().startswith("nsa_route_geometric_views")
    monkeypatch.setenv("NSA_FORCE_HIP_ERROR", "1")
    assert call() == -3
    assert call(views=0, proj=None, cells=None, geom=None) == -3       # no views: volume blocks only


def test_attn_single_branch_needs_no_gate(S, monkeypatch):
    # a single branch without gates is valid: with a forced launch failure it reaches the launch
    monkeypatch.setenv("NSA_FORCE_HIP_ERROR", "1")
    assert attn(S, layout(S), branches=4, gates=None, sel=None) == -3
    assert "forced" in S.lib.nsa_last_error().decode()


def test_other_calls_validate(S, monkeypatch):
    L = layout(S)
    lib = S.lib
    assert lib.nsa_pool_blocks(ctypes.byref(L), 1, 2, None, FAKE, None) == -1
    w = FAKE
    assert lib.nsa_pool_blocks_resblock(ctypes.byref(L), 1, 2, FAKE, w, w, None, w, FAKE, None) == -1
    assert lib.nsa_pool_blocks_resblock(ctypes.byref(L), 1, 0, FAKE, w, w, w, w, FAKE, None) == -1
    assert lib.nsa_pool_blocks_resblock(ctypes.byref(layout(S, head_dim=128)), 1, 1, FAKE, w, w, w, w, FAKE,
                                        None) == -2
    L3 = layout(S, head_dim=3)
    assert lib.nsa_pool_blocks(ctypes.byref(L3), 1, 2, FAKE, FAKE, None) == -2      # row of 6 bf16
    assert lib.nsa_pool_blocks(ctypes.byref(L3), 0, 1, FAKE, FAKE, None) == -2      # row of 3 f32
    assert lib.nsa_pool_blocks(ctypes.byref(L), 1, 2, FAKE + 8, FAKE, None) == -2    # misaligned
    assert lib.nsa_route_geometric(ctypes.byref(L), FAKE, 0, FAKE, FAKE, None, None) == -1
    assert lib.nsa_route_geometric(ctypes.byref(L), FAKE, 65, FAKE, FAKE, None, None) == -1
    assert lib.nsa_route_geometric(ctypes.byref(L), None, 4, FAKE, FAKE, None, None) == -1
    assert lib.nsa_route_geometric(ctypes.byref(layout(S, blk_key=None)), FAKE, 4, FAKE, FAKE, None, None) == -1
    assert lib.nsa_route_scores_topk(ctypes.byref(L), 1, 0, FAKE, FAKE, None, 4, FAKE, None) == -1  # lse needed
    assert lib.nsa_route_scores_topk(ctypes.byref(L), 1, 2, FAKE, FAKE, FAKE, 4, FAKE, None) == -1  # bad q_gran
    # 16-byte alignment of the vector-loaded operands
    assert lib.nsa_route_scores_topk(ctypes.byref(L), 1, 0, FAKE, FAKE, FAKE + 4, 4, FAKE, None) == -2
    assert lib.nsa_route_scores_topk(ctypes.byref(L), 1, 0, FAKE + 8, FAKE, FAKE, 4, FAKE, None) == -2
    assert lib.nsa_route_scores_topk(ctypes.byref(L), 1, 0, FAKE, FAKE + 2, FAKE, 4, FAKE, None) == -2
    assert lib.dense_gated_xattn_fwd(1, 100, 50, 32, 2, 32, 0.17, FAKE + 8, FAKE, FAKE, FAKE, FAKE, None) == -2
    arr = (ctypes.c_void_p * 2)(FAKE, None)
    assert lib.nsa_gate_combine(1, 10, 32, 32, 2, arr, FAKE, FAKE, None) == -1
    assert lib.nsa_gate_combine(1, 10, 32, 32, 9, arr, FAKE, FAKE, None) == -1
    assert lib.dense_gated_xattn_fwd(1, 100, 101, 32, 2, 32, 0.17, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert lib.dense_gated_xattn_fwd(1, 100, -1, 32, 2, 32, 0.17, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert lib.dense_gated_xattn_fwd(1, 100, 50, 32, 2, 64, 0.125, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -2
    vb = lib.nsa_build_volume_blocks
    assert vb(None, 9, 16, 0.1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1           # no lattice
    assert vb(FAKE, 9, 16, 0.1, 8, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == -1           # no counts
    assert vb(FAKE, 1, 16, 0.1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1           # G < 2
    assert vb(FAKE, 9, 14, 0.1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1           # N % 4
    assert vb(FAKE, 9, 0, 0.1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert vb(FAKE, 9, 16, -0.1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1          # tau < 0
    assert vb(FAKE, 9, 16, float("nan"), 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert vb(FAKE, 9, 16, float("inf"), 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert vb(FAKE, 9, 16, 0.1, -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert vb(FAKE, 9, 24, 0.1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -2           # N/4 = 6
    assert vb(FAKE, 9, 1024, 0.1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert vb(FAKE, 8193, 256, 0.1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -2       # 8NG >= 2^24
    mis = (ctypes.c_void_p * 2)(FAKE, FAKE + 2)
    assert lib.nsa_gate_combine(1, 10, 32, 32, 2, mis, FAKE, FAKE, None) == -2         # misaligned branch
    monkeypatch.setenv("NSA_FORCE_HIP_ERROR", "1")
    assert lib.nsa_pool_blocks(ctypes.byref(L), 1, 2, FAKE, FAKE, None) == -3
    assert lib.nsa_pool_blocks_resblock(ctypes.byref(L), 1, 2, FAKE, w, w, w, w, FAKE, None) == -3
    assert lib.nsa_route_geometric(ctypes.byref(L), FAKE, 4, FAKE, FAKE, None, None) == -3
    assert lib.nsa_route_scores_topk(ctypes.byref(L), 1, 0, FAKE, FAKE, FAKE, 4, FAKE, None) == -3
    assert lib.nsa_route_scores_topk(ctypes.byref(L), 1, 1, FAKE, FAKE, FAKE, 4, FAKE, None) == -3  # pooled rows
    assert lib.nsa_route_scores_topk(ctypes.byref(L), 1, 1, FAKE, FAKE, None, 4, FAKE, None) == -1  # lse needed
    g1 = layout(S, n_blk=64, n_qh=16, n_kvh=16, head_dim=64, blk_cap=16)
    for dt in (0, 1):                                            # block rows, f32 and bf16
        assert lib.nsa_route_scores_topk(ctypes.byref(g1), dt, 1, FAKE, FAKE, None, 16, FAKE, None) == -3
    assert lib.nsa_route_scores_topk(ctypes.byref(g1), 0, 0, FAKE, FAKE, None, 16, FAKE, None) == -2
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE)
    assert lib.nsa_gate_combine(1, 10, 32, 32, 2, arr, FAKE, FAKE, None) == -3
    assert lib.dense_gated_xattn_fwd(1, 100, 50, 32, 2, 32, 0.17, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -3
    assert lib.nsa_build_volume_blocks(FAKE, 9, 16, 0.1, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -3
    assert lib.nsa_build_volume_blocks(FAKE, 9, 16, 0.1, 0, FAKE, FAKE, FAKE, None, None, None, None) == -3
    assert attn(S, L) == -3


def test_error_message_is_thread_local(S):
    import threading
    assert attn(S, layout(S, n_blk=0)) == -1
    msgs = []

    def other():
        msgs.append(S.lib.nsa_last_error().decode())

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert msgs == [""]
    assert "n_blk" in S.lib.nsa_last_error().decode()


def test_binding_refuses_cpu_tensors(S):
    import torch
    with pytest.raises(ValueError):
        S._ptr(torch.zeros(3))


def test_build_is_hip_only():
    """The package has no CPU fallback: it exposes only the library wrappers."""
    src = open(os.path.join(ROOT, "sparse_attention_feed_amd", "__init__.py")).read()
    assert "import oracle" not in src and "from oracle" not in src


@pytest.mark.parametrize("field", ["q", "k", "v", "k_cmp", "v_cmp", "o"])
def test_attn_alignment(S, field):
    assert attn(S, layout(S), **{field: FAKE + 8}) == -2
    assert "16-byte aligned" in S.lib.nsa_last_error().decode()


def test_host_layout_validation():
    """The binding's host-side check of the preconditions the kernels take on trust."""
    import torch
    import sparse_attention_feed_amd as S
    S.validate_layout(torch.tensor([1, 64, 7], dtype=torch.int32), torch.tensor([3, 9, 1], dtype=torch.int32), 64)
    with pytest.raises(ValueError, match="blk_cnt\\[1\\] = 65"):
        S.validate_layout(torch.tensor([1, 65], dtype=torch.int32), None, 64)
    with pytest.raises(ValueError, match="blk_cnt\\[0\\] = 0"):
        S.validate_layout(torch.tensor([0, 5], dtype=torch.int32), None, 64)
    with pytest.raises(ValueError, match="not unique"):
        S.validate_layout(torch.tensor([1, 2], dtype=torch.int32), torch.tensor([4, 4], dtype=torch.int32), 8)


def test_noalloc_routing_validation(S, monkeypatch):
    """The allocation-free routing call validates like nsa_route_geometric and refuses layouts
    beyond its fixed centroid array before any device work."""
    r = S.lib.nsa_route_geometric_noalloc
    assert r(ctypes.byref(layout(S, n_blk=65537, blk_cap=1)), FAKE, 4, FAKE, None, None) == -2
    assert "65536" in S.lib.nsa_last_error().decode()
    assert r(ctypes.byref(layout(S)), FAKE, 0, FAKE, None, None) == -1
    assert r(ctypes.byref(layout(S)), None, 4, FAKE, None, None) == -1
    assert r(ctypes.byref(layout(S)), FAKE, 4, None, None, None) == -1
    assert r(ctypes.byref(layout(S, blk_key=None)), FAKE, 4, FAKE, None, None) == -1
    monkeypatch.setenv("NSA_FORCE_HIP_ERROR", "1")
    assert r(ctypes.byref(layout(S, n_blk=65536, blk_cap=1)), FAKE, 4, FAKE, None, None) == -3


def test_scores_routed_validation(S, monkeypatch):
    """nsa_attn_fwd_scores_routed: argument checks and the supported set, before any device work."""
    f = S.lib.nsa_attn_fwd_scores_routed
    g1 = dict(n_blk=64, blk_cap=16, n_qh=16, n_kvh=16, head_dim=64, scale=0.125)

    def call(L, top_k=16, dtype=1, gates=FAKE, sel=FAKE, q_cmp=FAKE):
        return f(ctypes.byref(L), dtype, FAKE, FAKE, FAKE, q_cmp, FAKE, FAKE, top_k, gates, FAKE, sel, None)

    monkeypatch.setenv("NSA_FORCE_HIP_ERROR", "1")
    assert call(layout(S, **g1)) == -3                           # valid: reaches the launch
    assert call(layout(S, **g1), top_k=32) == -3
    assert call(layout(S, **g1), top_k=0) == -1
    assert call(layout(S, **g1), top_k=33) == -2                 # compiled lists hold at most 32
    assert "top_k <= 32" in S.lib.nsa_last_error().decode()
    assert call(layout(S, **g1), gates=None) == -1
    assert call(layout(S, **g1), sel=None) == -1
    assert call(layout(S, **g1), q_cmp=None) == -1
    assert call(layout(S, **dict(g1, blk_key=None))) == -1
    assert call(layout(S, **g1), dtype=0) == -3                  # f32: routing pass, then the branches
    assert call(layout(S, **g1), dtype=2) == -1                  # unknown dtype
    assert call(layout(S, **dict(g1, blk_cap=32))) == -2
    assert call(layout(S, **dict(g1, blk_cap=12))) == -2
    assert call(layout(S)) == -2                                 # grouped-query layout
    assert f(ctypes.byref(layout(S, **g1)), 1, FAKE + 8, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, FAKE, FAKE,
             None) == -2                                         # misaligned q


def test_score_routed_layout_takes_the_local_branch(S, monkeypatch):
    """One query head per KV head: the local branch is accepted alone (no routing rows needed) and
    with the other two, in bf16 and in f32."""
    g1 = layout(S, n_blk=64, n_qh=16, n_kvh=16, head_dim=64, blk_cap=16)
    monkeypatch.setenv("NSA_FORCE_HIP_ERROR", "1")
    assert attn(S, g1, branches=4, q_gran=1, sel=None, gates=None, q_cmp=FAKE) == -3
    assert attn(S, g1, branches=7, q_gran=1, q_cmp=FAKE) == -3
    assert attn(S, g1, branches=5, q_gran=1, q_cmp=FAKE, sel=None) == -3
    assert attn(S, g1, branches=4, q_gran=1, dtype=0, sel=None, gates=None) == -3
    assert attn(S, g1, branches=7, q_gran=1, dtype=0, q_cmp=FAKE) == -3
    assert attn(S, g1, branches=4, q_gran=0, dtype=0, sel=None, gates=None) == -2      # token rows


def test_row_offsets_fit_32_bits(S, monkeypatch):
    """The grouped-query and dense kernels index rows in 32 bits: sizes past 2^31 elements are
    refused before any launch, sizes just inside reach it."""
    monkeypatch.setenv("NSA_FORCE_HIP_ERROR", "1")
    big = layout(S, n_blk=32768, blk_cap=64)          # 32768 * 64 * 32 * 32 = 2^31
    assert attn(S, big, branches=1, sel=None, gates=None) == -2
    assert "2^31" in S.lib.nsa_last_error().decode()
    ok = layout(S, n_blk=32767, blk_cap=64)
    assert attn(S, ok, branches=1, sel=None, gates=None) == -3
    lib = S.lib
    assert lib.dense_gated_xattn_fwd(1, 1 << 21, 0, 32, 2, 32, 0.17, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert lib.dense_gated_xattn_fwd(1, (1 << 21) - 1, 0, 32, 2, 32, 0.17, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -3


def test_grouped_query_block_rows(S, monkeypatch):
    """Grouped-query layout with pooled query rows (NSA_Q_BLOCK): every branch combination reaches
    the launch; the compressed branch needs q_cmp; block ranges keep per-token rows."""
    monkeypatch.setenv("NSA_FORCE_HIP_ERROR", "1")
    L = layout(S)
    for br in (1, 2, 4, 3, 5, 6, 7):
        kw = dict(branches=br, q_gran=1, q_cmp=FAKE)
        if br in (1, 2, 4):
            kw["gates"] = None
        assert attn(S, L, **kw) == -3, br
    assert attn(S, L, branches=1, q_gran=1, q_cmp=None, gates=None) == -1
    lse = FAKE
    assert attn(S, L, branches=1, q_gran=1, q_cmp=FAKE, gates=None, lse=lse) == -3
