"""Host-only checks of the C ABI: the library loads, exports every function
include/ice.h declares, and rejects bad arguments before any HIP call (the
fake pointers below are never dereferenced because each call fails its
checks first)."""
import ctypes
import os
import re

import pytest

from sparse_attention_dci_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x100000)   # aligned, never dereferenced
ODD = ctypes.c_void_p(0x100001)    # misaligned


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from sparse_attention_dci_amd import build_lib
        build_lib.build()
    return B.lib()


def good(**kw):
    base = dict(d=128, page_size=16, budget_k=256, m=8, L=4, gqa_group=4)
    base.update(kw)
    return B.make_params(**base)


def test_exports_every_declared_symbol(L):
    header = open(os.path.join(ROOT, "include", "ice.h")).read()
    names = set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(ice_\w+)\s*\(", header, re.M))
    assert {"ice_workspace_bytes", "ice_build_scratch_bytes", "ice_build_index", "ice_insert",
            "ice_query_pages", "ice_sparse_attn", "ice_decode_step", "ice_destroy_index",
            "ice_status_string", "ice_index_layout"} <= names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert L.ice_status_string(s)
    assert L.ice_status_string(-99) == b"unknown status"


def test_workspace_size_rules(L):
    p = good()
    a = L.ice_workspace_bytes(ctypes.byref(p), 8, 36864, 36864)
    b = L.ice_workspace_bytes(ctypes.byref(p), 8, 36864, 36864 + 128)
    assert 0 < a < b
    assert L.ice_build_scratch_bytes(ctypes.byref(p), 8, 36864) >= 8 * 32 * 36864 * 12
    assert L.ice_workspace_bytes(ctypes.byref(p), 8, 0, 16) > 0


@pytest.mark.parametrize("bad", [
    dict(d=96), dict(page_size=12), dict(page_size=128), dict(budget_k=250), dict(budget_k=0),
    dict(m=0), dict(L=0), dict(m=16, L=9), dict(gqa_group=0), dict(gqa_group=17),
    dict(tree_depth=14), dict(tree_depth=-1), dict(m=2, L=2, tree_depth=5), dict(c=-1.0),
    dict(c=float("inf")), dict(c=float("nan")), dict(k0=-1), dict(k1=-5),
])
def test_bad_params_rejected(L, bad):
    p = good(**bad)
    assert L.ice_workspace_bytes(ctypes.byref(p), 8, 1000, 1000) == 0
    h = ctypes.c_void_p()
    st = L.ice_build_index(ctypes.byref(p), 8, 1000, 1000, FAKE, FAKE, FAKE, FAKE, 1 << 40, FAKE,
                           1 << 40, None, ctypes.byref(h))
    assert st == B.ICE_ERR_INVALID_ARG and not h.value


def test_bad_dtype_rejected(L):
    p = good()
    p.dtype = 7
    assert L.ice_workspace_bytes(ctypes.byref(p), 8, 1000, 1000) == 0


@pytest.mark.parametrize("S,n,cap", [(0, 10, 10), (1, 20, 10), (1, -1, 10), (1, 0, 0),
                                     (1, 10, 1 << 31)])
def test_bad_sizes_rejected(L, S, n, cap):
    p = good()
    assert L.ice_workspace_bytes(ctypes.byref(p), S, n, cap) == 0


def test_unsupported_settings(L):
    h = ctypes.c_void_p()
    for p in (good(budget_k=4096, page_size=32, m=8, L=4),
              good(budget_k=65536 + 16, k0=64)):
        assert L.ice_workspace_bytes(ctypes.byref(p), 1, 1000, 1000) == 0
        st = L.ice_build_index(ctypes.byref(p), 1, 1000, 1000, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                               FAKE, 1 << 40, None, ctypes.byref(h))
        assert st == B.ICE_ERR_UNSUPPORTED


def test_visit_budget_accepted(L):
    """Bounded walks are accepted; the page-capacity limit keeps m * capacity
    (the list entries a composite's selection counts) below 2^29."""
    p = good(k1=1000)
    assert L.ice_workspace_bytes(ctypes.byref(p), 1, 1000, 1000) > 0
    wide = good(k1=1 << 40, m=128, L=1, page_size=64, tree_depth=8)
    cap = (65536 - 256) * 64
    assert L.ice_workspace_bytes(ctypes.byref(wide), 1, 1000, cap) > 0
    assert 128 * cap < 1 << 29
    assert L.ice_workspace_bytes(ctypes.byref(wide), 1, 1000, cap + 64) == 0


def test_build_size_limit(L):
    """Builds of more than 2^24 tokens per stream are refused before any launch."""
    p = good()
    big = (1 << 24) + 1
    assert L.ice_workspace_bytes(ctypes.byref(p), 1, big, big) == 0
    assert L.ice_build_scratch_bytes(ctypes.byref(p), 1, big) == 0
    p64 = good(page_size=64, budget_k=256)
    assert L.ice_workspace_bytes(ctypes.byref(p64), 1, 1 << 20, 1 << 20) > 0


def test_build_argument_checks(L):
    p = good()
    ws = L.ice_workspace_bytes(ctypes.byref(p), 2, 1000, 1000)
    sb = L.ice_build_scratch_bytes(ctypes.byref(p), 2, 1000)
    h = ctypes.c_void_p()
    call = lambda **a: L.ice_build_index(
        ctypes.byref(p), 2, 1000, 1000, a.get("K", FAKE), a.get("V", FAKE), a.get("U", FAKE),
        a.get("ws", FAKE), a.get("wsb", ws), a.get("sc", FAKE), a.get("scb", sb), None,
        a.get("out", ctypes.byref(h)))
    assert call(out=None) == B.ICE_ERR_INVALID_ARG
    assert call(U=None) == B.ICE_ERR_INVALID_ARG
    assert call(K=None) == B.ICE_ERR_INVALID_ARG
    assert call(K=ODD) == B.ICE_ERR_INVALID_ARG
    assert call(ws=None) == B.ICE_ERR_WORKSPACE
    assert call(ws=ODD) == B.ICE_ERR_WORKSPACE
    assert call(wsb=ws - 1) == B.ICE_ERR_WORKSPACE
    assert call(sc=None) == B.ICE_ERR_WORKSPACE
    assert call(scb=sb - 1) == B.ICE_ERR_WORKSPACE
    assert not h.value


def test_null_handles(L):
    assert L.ice_insert(None, FAKE, FAKE, None) == B.ICE_ERR_INVALID_ARG
    assert L.ice_query_pages(None, FAKE, FAKE, FAKE, None, None, None) == B.ICE_ERR_INVALID_ARG
    assert L.ice_sparse_attn(None, FAKE, FAKE, FAKE, FAKE, None) == B.ICE_ERR_INVALID_ARG
    assert L.ice_decode_step(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                             None) == B.ICE_ERR_INVALID_ARG
    assert L.ice_decode_step_reuse(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None) == B.ICE_ERR_INVALID_ARG
    y = B.IceLayout()
    assert L.ice_index_layout(None, ctypes.byref(y)) == B.ICE_ERR_INVALID_ARG
    L.ice_destroy_index(None)


def test_stats_record_layout():
    """ice_query_stats: 32 int64 visit counts, then four int32 (272 bytes), as
    the binding reads it."""
    import torch
    assert B.STATS_WORDS * 8 == 32 * 8 + 4 * 4
    t = torch.zeros(2, B.STATS_WORDS, dtype=torch.int64)
    t[1, :3] = torch.tensor([5, 6, 7])
    t[1, 32:].view(torch.int32)[:3] = torch.tensor([11, 12, 13], dtype=torch.int32)
    r = B.parse_stats(t, 3)
    assert r[1] == {"visits": [5, 6, 7], "n_cand": 11, "n_pages": 12, "n_tokens": 13}


def test_tree_depth_matches_oracle_reading(L, ora):
    """The derived depth is visible through the workspace size: the cell tables
    grow with 2^D.  Compare the sizes with D given explicitly."""
    for n, pg, m, Lc in [(4096, 16, 4, 2), (36864, 16, 8, 4), (131072, 16, 10, 4), (3000, 8, 4, 2),
                         (100, 16, 2, 2), (0, 16, 4, 2)]:
        D = ora.tree_depth(n, pg, m * Lc)
        auto = good(page_size=pg, budget_k=4 * pg, m=m, L=Lc)
        fixed = good(page_size=pg, budget_k=4 * pg, m=m, L=Lc, tree_depth=D)
        cap = max(n, 1)
        assert (L.ice_workspace_bytes(ctypes.byref(auto), 1, n, cap)
                == L.ice_workspace_bytes(ctypes.byref(fixed), 1, n, cap)), (n, pg, D)
        if D < min(m * Lc, 13):
            other = good(page_size=pg, budget_k=4 * pg, m=m, L=Lc, tree_depth=D + 1)
            assert (L.ice_workspace_bytes(ctypes.byref(auto), 1, n, cap)
                    != L.ice_workspace_bytes(ctypes.byref(other), 1, n, cap))


def test_noalloc_build_limits(L):
    """The no-allocation build refuses, before any HIP call, a build whose
    scratch exceeds its fixed array, and bad arguments as the plain build does."""
    p = good()
    h = ctypes.c_void_p()
    # 8 heads x 40,000 tokens x 32 directions needs more than 128 MiB of scratch
    assert L.ice_build_scratch_bytes(ctypes.byref(p), 8, 40000) > B.NOALLOC_SCRATCH_BYTES
    st = L.ice_build_index_noalloc(ctypes.byref(p), 8, 40000, 40000, FAKE, FAKE, FAKE, FAKE,
                                  1 << 40, None, ctypes.byref(h))
    assert st == B.ICE_ERR_SCRATCH_LIMIT and not h.value
    # the 36,864-token Llama-3.1-8B layer fits
    assert L.ice_build_scratch_bytes(ctypes.byref(p), 8, 36864) <= B.NOALLOC_SCRATCH_BYTES
    bad = good(page_size=12)
    st = L.ice_build_index_noalloc(ctypes.byref(bad), 8, 1000, 1000, FAKE, FAKE, FAKE, FAKE,
                                  1 << 40, None, ctypes.byref(h))
    assert st == B.ICE_ERR_INVALID_ARG and not h.value
    st = L.ice_build_index_noalloc(ctypes.byref(p), 8, 1000, 1000, FAKE, FAKE, FAKE, FAKE,
                                  1 << 40, None, None)
    assert st == B.ICE_ERR_INVALID_ARG


def test_gqa_mode_rules(L):
    """GQA max mode: an unknown mode is refused; g * L walks above 32, or
    g * L * k0 above 4,096 pooled candidates, are UNSUPPORTED (ice_workspace_bytes
    reports 0 and the build refuses before any HIP call)."""
    h = ctypes.c_void_p()
    bad = good()
    bad.gqa_mode = 2
    assert L.ice_workspace_bytes(ctypes.byref(bad), 8, 1000, 1000) == 0
    ok = good(gqa_mode="max")  # g 4 x L 4 = 16 walks x k0 256 = 4,096
    assert L.ice_workspace_bytes(ctypes.byref(ok), 8, 36864, 36864) > \
        L.ice_workspace_bytes(ctypes.byref(good()), 8, 36864, 36864)
    for kw in (dict(gqa_group=8, L=5, m=2), dict(budget_k=512)):
        p = good(gqa_mode="max", **kw)
        st = L.ice_build_index(ctypes.byref(p), 8, 1000, 1000, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                               FAKE, 1 << 40, None, ctypes.byref(h))
        assert st == B.ICE_ERR_UNSUPPORTED and not h.value, kw


def test_offload_entry_rules(L):
    """The offloaded pool: ice_build_index refuses offload = 1 and 2 and the
    offload entry refuses offload = 0; a missing or short host pool is a
    workspace error, all before any HIP call; the workspace then holds no pool
    (offload 1) or the key pages alone (offload 2, half the host pool)."""
    h = ctypes.c_void_p()
    off = good(offload=True)
    res = good()
    assert L.ice_host_pool_bytes(ctypes.byref(res), 8, 36864, 36864) == 0
    hp = L.ice_host_pool_bytes(ctypes.byref(off), 8, 36864, 36864)
    assert hp >= 2 * 8 * (36864 // 16) * 16 * 128 * 2
    assert (L.ice_workspace_bytes(ctypes.byref(res), 8, 36864, 36864)
            - L.ice_workspace_bytes(ctypes.byref(off), 8, 36864, 36864)) > hp // 2
    st = L.ice_build_index(ctypes.byref(off), 8, 1000, 1000, FAKE, FAKE, FAKE, FAKE, 1 << 40, FAKE,
                           1 << 40, None, ctypes.byref(h))
    assert st == B.ICE_ERR_INVALID_ARG and not h.value
    st = L.ice_build_index_offload(ctypes.byref(res), 8, 1000, 1000, FAKE, FAKE, FAKE, FAKE,
                                   1 << 40, FAKE, 1 << 40, FAKE, 1 << 40, None, ctypes.byref(h))
    assert st == B.ICE_ERR_INVALID_ARG and not h.value
    for pool, nbytes in ((None, 1 << 40), (FAKE, 16)):
        st = L.ice_build_index_offload(ctypes.byref(off), 8, 1000, 1000, FAKE, FAKE, FAKE, FAKE,
                                       1 << 40, FAKE, 1 << 40, pool, nbytes, None, ctypes.byref(h))
        assert st == B.ICE_ERR_WORKSPACE and not h.value
    # offload 2: the values alone in host memory (half the host pool), the keys
    # in the workspace; ice_build_index refuses it too
    vo = good(offload="values")
    assert vo.offload == 2
    hv = L.ice_host_pool_bytes(ctypes.byref(vo), 8, 36864, 36864)
    assert hv * 2 >= hp - 512 and hv * 2 <= hp + 512
    assert (L.ice_workspace_bytes(ctypes.byref(vo), 8, 36864, 36864)
            - L.ice_workspace_bytes(ctypes.byref(off), 8, 36864, 36864)) >= hv - 256
    st = L.ice_build_index(ctypes.byref(vo), 8, 1000, 1000, FAKE, FAKE, FAKE, FAKE, 1 << 40, FAKE,
                           1 << 40, None, ctypes.byref(h))
    assert st == B.ICE_ERR_INVALID_ARG and not h.value
    bad = good(offload=True)
    bad.offload = 3
    assert L.ice_workspace_bytes(ctypes.byref(bad), 8, 1000, 1000) == 0
