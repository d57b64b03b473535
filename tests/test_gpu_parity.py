"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle
on the same seeded inputs.

Integer and index results (projection codes, sorted lists, cells, page
tables, pool contents, query codes, candidate sets, top-k, selected pages)
must be bit-identical; attention outputs must be within 2e-3 max-abs of the
oracle's fp64 result.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_dci_amd import workloads as W

pytestmark = pytest.mark.gpu

ATTN_TOL = 2e-3


@pytest.fixture(scope="module")
def B():
    from sparse_attention_dci_amd import binding
    binding.lib()
    return binding


def _inputs(S, n, d, g, clusters, seed, dtype, needle=0, device="cpu"):
    Ks, Vs, qs, p0 = [], [], [], []
    for s in range(S):
        K, V, q, p = W.stream(n, d, clusters, g, seed * 100 + s, dtype, needle=needle,
                              device=device)
        Ks.append(K)
        Vs.append(V)
        qs.append(q)
        p0.append(p)
    return torch.stack(Ks), torch.stack(Vs), torch.cat(qs), p0


def _np(t):
    return t.float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float32) else t.cpu().numpy()


def _stored_lists(idx, s):
    """The per-direction lists of stream s as stored: [mL][n] codes and ids."""
    n = idx.layout()["n_tokens"]
    lc = idx.view("list_code")[s, :, :n].cpu().numpy()
    li = idx.view("list_id")[s, :, :n].cpu().numpy()
    return lc, li


def _check_list_storage(idx, s, codes):
    """The stored lists keep the documented order: entries [0, n_build) sorted
    by (code, token), then the inserted tokens n_build .. n-1 in insertion
    order with their codes.  `codes` is the expected [n][mL] code table."""
    lay = idx.layout()
    nb, n = lay["n_build"], lay["n_tokens"]
    lc, li = _stored_lists(idx, s)
    for t in range(lc.shape[0]):
        c, i = lc[t, :nb].astype(np.int64), li[t, :nb].astype(np.int64)
        assert np.all((c[1:] > c[:-1]) | ((c[1:] == c[:-1]) & (i[1:] > i[:-1]))), t
    np.testing.assert_array_equal(li[:, nb:], np.broadcast_to(np.arange(nb, n), (lc.shape[0], n - nb)))
    np.testing.assert_array_equal(lc[:, nb:], codes[nb:n].T)


def _logical_lists(idx, s):
    """Per-direction lists in logical order: the sorted build prefix merged
    with the inserted entries (checked to be stored in the documented order
    before they are merged)."""
    lc, li = _stored_lists(idx, s)
    out_c, out_i = [], []
    for t in range(lc.shape[0]):
        o = np.lexsort((li[t], lc[t]))
        out_c.append(lc[t][o])
        out_i.append(li[t][o])
    return np.stack(out_c), np.stack(out_i)


def _check_index(idx, st, s, n):
    """Every index array of stream s against the oracle stream."""
    lay = idx.layout()
    assert lay["tree_depth"] == st.D
    assert idx.view("norm_c")[s].item() == np.float32(st.c)
    np.testing.assert_array_equal(idx.view("codes")[s, :n].cpu().numpy(), st.codes[:n])
    # the build prefix as stored (no re-sort) equals the oracle's build-time
    # lists; the inserted tail is in insertion order; then the merge
    nb = lay["n_build"]
    assert nb == st.n_build
    lc, li = _stored_lists(idx, s)
    np.testing.assert_array_equal(lc[:, :nb], st.lcode_build)
    np.testing.assert_array_equal(li[:, :nb], st.lid_build)
    _check_list_storage(idx, s, st.codes)
    lc, li = _logical_lists(idx, s)
    np.testing.assert_array_equal(lc, st.lcode[:, :n])
    np.testing.assert_array_equal(li, st.lid[:, :n])
    npg = int(idx.view("npages")[s].item())
    assert npg == st.npages
    loc = idx.view("loc")[s, :n].cpu().numpy()
    p = st.prm.p
    np.testing.assert_array_equal(loc // p, st.page_of[:n])
    np.testing.assert_array_equal(loc % p, st.slot_of[:n])
    np.testing.assert_array_equal(idx.view("page_tokens")[s, :npg].cpu().numpy(),
                                  st.page_tokens[:npg])
    np.testing.assert_array_equal(idx.view("page_len")[s, :npg].cpu().numpy(), st.page_len[:npg])
    np.testing.assert_array_equal(idx.view("page_cell")[s, :npg].cpu().numpy(),
                                  st.page_cell[:npg])
    pk, pv = st.pool()
    tok = st.page_tokens[:npg]
    ok = tok >= 0
    gk = idx.view("pool_k")[s, :npg].float().cpu().numpy()
    gv = idx.view("pool_v")[s, :npg].float().cpu().numpy()
    np.testing.assert_array_equal(gk[ok], pk[:npg][ok])
    np.testing.assert_array_equal(gv[ok], pv[:npg][ok])


def _check_query(idx, st, s, r, page_ids, n_pages, topk, out, q_s):
    np.testing.assert_array_equal(idx.view("qcode")[s].cpu().numpy(), r["qcode"])
    cand = idx.view("cand")[s].cpu().numpy()
    cc = idx.view("cand_count")[s].cpu().numpy()
    for l in range(len(r["S"])):  # every walk: L, or g * L in the GQA max mode
        np.testing.assert_array_equal(np.sort(cand[l, :cc[l]]), np.sort(r["S"][l]),
                                      err_msg=f"candidates of composite {l}")
    nsel = int(n_pages[s].item())
    np.testing.assert_array_equal(page_ids[s, :nsel].cpu().numpy(), r["page_ids"])
    assert np.all(page_ids[s, nsel:].cpu().numpy() == -1)
    if topk is not None:
        kk = len(r["topk"])
        np.testing.assert_array_equal(topk[s, :kk].cpu().numpy(), r["topk"])
        assert np.all(topk[s, kk:].cpu().numpy() == -1)
    ref = st.attend(q_s, r["page_ids"])
    err = float(np.max(np.abs(out.cpu().numpy() - ref))) if ref.size else 0.0
    assert err <= ATTN_TOL, err


def run_case(B, *, S, n, d=128, g=1, p=16, k=256, m=4, L=2, dtype="bf16", clusters=32,
             seed=1, inserts=0, k0=0, k1=0, check=None, keys=None, literal=True, gqa="mean"):
    dev = torch.device("cuda")
    cap = n + inserts
    if keys is None:
        K, V, q, _ = _inputs(S, cap, d, g, clusters, seed, dtype)
    else:
        K, V, q = keys
    U = W.directions(m * L, d, seed, dtype)
    print(f"[case] S={S} n={n} inserts={inserts} d={d} g={g} p={p} k={k} m={m} L={L} {dtype} "
          f"k0={k0} k1={k1}", flush=True)
    idx = B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U.to(dev),
                  page_size=p, budget_k=k, m=m, L=L, gqa_group=g, k0=k0, k1=k1,
                  capacity=max(cap, 1), gqa_mode=gqa)
    for t in range(inserts):
        idx.insert(K[:, n + t].contiguous().to(dev), V[:, n + t].contiguous().to(dev))
    qd = q.to(dev)
    page_ids, n_pages, topk = idx.query_pages(qd, with_topk=True)
    out = idx.sparse_attn(qd, page_ids, n_pages)
    torch.cuda.synchronize()
    prm = oracle.Params(d=d, p=p, k=k, m=m, L=L, g=g, k0=k0, k1=k1, gqa_max=gqa == "max")
    Un = _np(U)
    for s in (check if check is not None else range(S)):
        st = oracle.OracleStream(prm, _np(K[s, :n]), _np(V[s, :n]), Un, n_cap=max(cap, 1))
        for t in range(inserts):
            st.insert(_np(K[s, n + t]), _np(V[s, n + t]))
        _check_index(idx, st, s, cap)
        q_s = _np(q[s * g:(s + 1) * g])
        r = st.query(q_s, literal=literal)
        _check_query(idx, st, s, r, page_ids, n_pages, topk, out[s * g:(s + 1) * g], q_s)
    return idx


def test_golden_tiny_worked_example(B):
    """The HIP path on tests/golden/tiny_worked_example.json, a three-token
    stream worked through the decode path by hand: the key-norm bound, codes,
    query codes, candidates, top-k and pages equal the hand-worked values
    exactly; the attention is within the attention tolerance of them."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_worked_example.json")) as f:
        gd = json.load(f)
    prm, e = gd["params"], gd["expected"]
    d, n = prm["d"], 3
    K = torch.zeros(1, n, d)
    V = torch.zeros(1, n, d)
    U = torch.zeros(1, d + 1)
    q = torch.zeros(1, d)
    for t, key in ((K[0], "keys_nonzero"), (V[0], "values_nonzero"), (U, "direction_nonzero"),
                   (q, "query_nonzero")):
        for r, c, v in gd["inputs"][key]:
            t[r, c] = v
    dev = torch.device("cuda")
    idx = B.Index(K.to(dev), V.to(dev), U.to(dev), page_size=prm["p"], budget_k=prm["k"],
                  m=prm["m"], L=prm["L"], gqa_group=prm["g"], k0=prm["k0"], capacity=n)
    qd = q.to(dev)
    pg, npg, tk = idx.query_pages(qd, with_topk=True)
    out = idx.sparse_attn(qd, pg, npg)
    torch.cuda.synchronize()
    assert float(idx.view("norm_c")[0]) == e["norm_bound"]
    assert idx.view("codes")[0, :n, 0].tolist() == e["codes"]
    assert idx.view("qcode")[0].tolist() == e["qcode"]
    cc = int(idx.view("cand_count")[0, 0])
    assert sorted(idx.view("cand")[0, 0, :cc].tolist()) == e["candidates"]
    assert tk[0].tolist() == e["topk"]
    assert int(npg[0]) == e["n_pages"] and pg[0, :e["n_pages"]].tolist() == e["page_ids"]
    o = out[0].cpu().numpy()
    assert np.max(np.abs(o[:2] - np.array(e["attention_first_two"]))) <= ATTN_TOL
    assert np.max(np.abs(o[2:])) <= ATTN_TOL


@pytest.mark.parametrize("case", ["unbounded", "bounded"])
def test_golden_tiny_pdci_two_lists(B, case):
    """The HIP path on tests/golden/tiny_pdci_two_lists.json (two lists per
    composite, a score tie, a visit budget of 4 in the bounded case), worked
    by hand: codes, query codes, candidates, visits (query statistics), top-k
    and pages exactly; the attention within the attention tolerance."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_pdci_two_lists.json")) as f:
        gd = json.load(f)
    prm, e = gd["params"], gd["expected"]
    c = e[case]
    d, n, mL = prm["d"], 4, prm["m"] * prm["L"]
    K = torch.zeros(1, n, d)
    V = torch.zeros(1, n, d)
    U = torch.zeros(mL, d + 1)
    q = torch.zeros(1, d)
    for t, key in ((K[0], "keys_nonzero"), (V[0], "values_nonzero"), (U, "directions_nonzero"),
                   (q, "query_nonzero")):
        for r, col, v in gd["inputs"][key]:
            t[r, col] = v
    dev = torch.device("cuda")
    idx = B.Index(K.to(dev), V.to(dev), U.to(dev), page_size=prm["p"], budget_k=prm["k"],
                  m=prm["m"], L=prm["L"], gqa_group=prm["g"], k0=prm["k0"], k1=c["k1"],
                  capacity=n)
    qd = q.to(dev)
    stats = B.stats_tensor(1, dev)
    pg, npg, tk = idx.query_pages(qd, with_topk=True, stats=stats)
    out = idx.sparse_attn(qd, pg, npg)
    torch.cuda.synchronize()
    assert float(idx.view("norm_c")[0]) == e["norm_bound"]
    assert idx.view("codes")[0, :n].tolist() == e["codes"]
    assert idx.view("qcode")[0].tolist() == e["qcode"]
    cc = int(idx.view("cand_count")[0, 0])
    assert sorted(idx.view("cand")[0, 0, :cc].tolist()) == sorted(c["candidates_in_order"])
    assert B.parse_stats(stats, prm["L"])[0]["visits"] == c["visits"]
    assert tk[0].tolist() == c["topk"]
    assert int(npg[0]) == len(c["page_ids"]) and pg[0, :int(npg[0])].tolist() == c["page_ids"]
    o = out[0].cpu().numpy()
    assert np.max(np.abs(o[:4] - np.array(e["attention_first_four"]))) <= ATTN_TOL
    assert np.max(np.abs(o[4:])) <= ATTN_TOL


def test_single_stream_fp32_ragged(B):
    run_case(B, S=1, n=3037, g=1, p=16, k=256, m=4, L=2, dtype="f32", seed=2)


def test_gqa_bf16_ragged(B):
    run_case(B, S=3, n=5003, g=4, p=16, k=128, m=8, L=4, seed=3)


def test_page8_d64_odd_directions(B):
    run_case(B, S=2, n=2501, d=64, g=2, p=8, k=64, m=3, L=3, seed=4)


def test_page64(B):
    run_case(B, S=2, n=4000, g=2, p=64, k=256, m=6, L=2, seed=5)


def test_page32_k0(B):
    run_case(B, S=2, n=6000, g=4, p=32, k=256, m=5, L=3, k0=300, seed=6)


def test_inserts_match_oracle(B):
    run_case(B, S=2, n=2000, inserts=77, g=4, p=16, k=128, m=4, L=3, seed=7)


def test_empty_build_then_inserts(B):
    run_case(B, S=2, n=0, inserts=40, g=2, p=16, k=32, m=2, L=2, seed=8)


def test_fewer_tokens_than_budget(B):
    run_case(B, S=2, n=100, g=1, p=16, k=256, m=4, L=2, seed=9)


def test_identical_keys(B):
    """Every key equal: all distances tie and candidates go by token index."""
    S, n, d, g = 2, 700, 128, 2
    K = torch.full((S, n, d), 0.5, dtype=torch.bfloat16)
    V = torch.randn(S, n, d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    q = torch.randn(S * g, d, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    run_case(B, S=S, n=n, d=d, g=g, p=16, k=64, m=4, L=2, keys=(K, V, q), seed=10)


def test_query_along_a_direction(B):
    """The query is the first direction itself: every key's distance on that
    composite is near the top of the code range, so its threshold bin lies
    far above the usual low bins (the collect reads its whole histogram); the
    other composites stay in the low bins."""
    S, n, d, g, m, L, seed = 2, 3000, 128, 2, 4, 3, 21
    K, V, _, _ = _inputs(S, n, d, g, 16, seed, "bf16")
    U = W.directions(m * L, d, seed, "bf16")
    q = U[0, :d].float().repeat(S * g, 1).to(torch.bfloat16)
    run_case(B, S=S, n=n, d=d, g=g, p=16, k=128, m=m, L=L, keys=(K, V, q), seed=seed)


def test_many_equal_top_scores(B):
    """128 copies of one key of four times the usual norm, and the query is
    that key: the copies lead the ranking with equal scores (token order)
    across about 5 pages.  Pages and top-k against the oracle; the page walk
    with and without the top-k asked gives the same pages."""
    S, n, d, g = 2, 3000, 128, 1
    K, V, _, _ = _inputs(S, n, d, g, 16, 23, "bf16")
    K[:, 1000:1128] = (K[:, 1000:1001].float() * 4).to(torch.bfloat16)
    q = K[:, 1000].clone()
    for with_topk in (True, False):
        idx = run_case(B, S=S, n=n, d=d, g=g, p=16, k=256, m=4, L=2, keys=(K, V, q), seed=23)
        if not with_topk:  # the page walk alone (no top-k asked): same pages
            qd = q.to(torch.device("cuda"))
            pg, npg, _ = idx.query_pages(qd, with_topk=True)
            pg2, npg2, _ = idx.query_pages(qd)
            torch.cuda.synchronize()
            assert torch.equal(pg, pg2) and torch.equal(npg, npg2)


def test_single_head_4k_workload(B):
    w = W.WORKLOADS["single_head_4k_f32"]
    K, V, q, U, _ = W.layer_inputs(w)
    run_case(B, S=w.streams, n=w.n, d=w.d, g=w.g, p=w.p, k=w.k, m=w.m, L=w.L, dtype=w.dtype,
             keys=(K, V, q), seed=w.seed)


def test_llama8b_layer_36k_workload(B):
    """All 8 KV heads of the 36,864-token Llama-3.1-8B layer, every stage."""
    w = W.WORKLOADS["llama8b_layer_36k"]
    K, V, q, U, _ = W.layer_inputs(w)
    dev = torch.device("cuda")
    print("[case] llama8b_layer_36k", flush=True)
    idx = B.Index(K.to(dev), V.to(dev), U.to(dev), page_size=w.p, budget_k=w.k, m=w.m, L=w.L,
                  gqa_group=w.g, capacity=w.n + 64)
    qd = q.to(dev)
    page_ids, n_pages, topk = idx.query_pages(qd, with_topk=True)
    out = idx.sparse_attn(qd, page_ids, n_pages)
    torch.cuda.synchronize()
    prm = oracle.Params(d=w.d, p=w.p, k=w.k, m=w.m, L=w.L, g=w.g)
    for s in range(w.streams):
        st = oracle.OracleStream(prm, _np(K[s]), _np(V[s]), _np(U), n_cap=w.n + 64)
        _check_index(idx, st, s, w.n)
        q_s = _np(q[s * w.g:(s + 1) * w.g])
        r = st.query(q_s)
        _check_query(idx, st, s, r, page_ids, n_pages, topk, out[s * w.g:(s + 1) * w.g], q_s)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_projection_wide_exponents(B, dtype):
    """Key elements spread over 2^-30 .. 2^10: every fp64 partial sum of the
    projection rounds differently under any reordering, so the codes (and
    everything after them) match the oracle's sequential chain only if the
    matrix-core projection accumulates in ascending element order."""
    S, n, d, g = 2, 2100, 128, 2
    gen = torch.Generator().manual_seed(71)
    K = torch.randn(S, n, d, generator=gen) * torch.exp2(
        torch.randint(-30, 11, (S, n, d), generator=gen).float())
    V = torch.randn(S, n, d, generator=gen)
    q = torch.randn(S * g, d, generator=gen) * 4.0
    td = W.torch_dtype(dtype)
    run_case(B, S=S, n=n, d=d, g=g, p=16, k=128, m=4, L=3, dtype=dtype, seed=71,
             keys=(K.to(td), V.to(td), q.to(td)))


def test_small_union_hash_membership(B):
    """More tokens than the finaliser's membership bitmap covers (262,144):
    the small-union finaliser (L*k0 = 512) tracks the union in its LDS hash
    instead; every stage against the oracle."""
    run_case(B, S=1, n=263144, g=2, p=16, k=256, m=4, L=2, dtype="bf16", clusters=64, seed=81)


def test_insert_equals_rebuild_on_gpu(B):
    """ice_insert x t, then query == rebuild over n+t tokens with the stored c
    and D, then the same query (every array and every output)."""
    S, n, t, d, g = 3, 3000, 90, 128, 4
    p, k, m, L = 16, 128, 6, 3
    dev = torch.device("cuda")
    K, V, q, _ = _inputs(S, n + t, d, g, 24, 11, "bf16")
    U = W.directions(m * L, d, 11, "bf16").to(dev)
    Kd, Vd, qd = K.to(dev), V.to(dev), q.to(dev)
    a = B.Index(Kd[:, :n].contiguous(), Vd[:, :n].contiguous(), U, page_size=p, budget_k=k, m=m,
                L=L, gqa_group=g, capacity=n + t)
    for i in range(n, n + t):
        a.insert(Kd[:, i].contiguous(), Vd[:, i].contiguous())
    torch.cuda.synchronize()
    c = a.view("norm_c").cpu()
    D = a.layout()["tree_depth"]
    for s in range(S):
        b = B.Index(Kd[s:s + 1].contiguous(), Vd[s:s + 1].contiguous(), U, page_size=p,
                    budget_k=k, m=m, L=L, gqa_group=g, capacity=n + t, c=float(c[s]),
                    tree_depth=D)
        pa, na, ta = a.query_pages(qd, with_topk=True)
        pb, nb, tb = b.query_pages(qd[s * g:(s + 1) * g].contiguous(), with_topk=True)
        oa = a.sparse_attn(qd, pa, na)
        ob = b.sparse_attn(qd[s * g:(s + 1) * g].contiguous(), pb, nb)
        torch.cuda.synchronize()
        assert torch.equal(a.view("codes")[s, :n + t], b.view("codes")[0, :n + t])
        _check_list_storage(a, s, a.view("codes")[s].cpu().numpy())
        _check_list_storage(b, 0, b.view("codes")[0].cpu().numpy())
        la = _logical_lists(a, s)
        lb = _logical_lists(b, 0)
        assert np.array_equal(la[0], lb[0]) and np.array_equal(la[1], lb[1])
        for f in ("loc",):
            assert torch.equal(a.view(f)[s, :n + t], b.view(f)[0, :n + t])
        npg = int(a.view("npages")[s])
        assert npg == int(b.view("npages")[0])
        for f in ("page_tokens", "page_len", "page_cell"):
            assert torch.equal(a.view(f)[s, :npg], b.view(f)[0, :npg]), f
        filled = a.view("page_tokens")[s, :npg] >= 0  # empty slots hold no token
        for f in ("pool_k", "pool_v"):
            assert torch.equal(a.view(f)[s, :npg][filled], b.view(f)[0, :npg][filled]), f
        assert torch.equal(pa[s], pb[0]) and torch.equal(na[s], nb[0]) and torch.equal(ta[s], tb[0])
        assert torch.equal(oa[s * g:(s + 1) * g], ob)


def test_repeated_queries_are_deterministic(B):
    S, n, d, g = 4, 4096, 128, 4
    dev = torch.device("cuda")
    K, V, q, _ = _inputs(S, n, d, g, 16, 12, "bf16")
    U = W.directions(32, d, 12, "bf16").to(dev)
    idx = B.Index(K.to(dev), V.to(dev), U, page_size=16, budget_k=256, m=8, L=4, gqa_group=g)
    qd = q.to(dev)
    first = None
    for rep in range(5):
        pg, npg, tk = idx.query_pages(qd, with_topk=True)
        out = idx.sparse_attn(qd, pg, npg)
        torch.cuda.synchronize()
        cur = (pg.clone(), npg.clone(), tk.clone(), out.clone())
        if first is None:
            first = cur
        else:
            for a_, b_ in zip(first, cur):
                assert torch.equal(a_, b_)


@pytest.mark.parametrize("dtype,S,g,d,p,m,L,k,n", [
    ("bf16", 8, 4, 128, 16, 8, 4, 128, 3000),
    ("f32", 2, 2, 64, 8, 3, 3, 128, 3000),
    ("bf16", 2, 2, 128, 16, 4, 6, 1024, 3000),
    # the 131k batch-4 workload's index shape (m 10, L 4: 40 directions, three
    # 16-code rounds in the scan; L*k0 = 4,096, the largest union the fused
    # finaliser holds, 64 pages)
    ("bf16", 2, 4, 128, 16, 10, 4, 1024, 14000),
    # the 262k workload's index shape (m 12, L 6: 72 directions, five rounds;
    # L*k0 = 12,288: the large-union finaliser, then the attention in eight
    # 256-token splits and their merge)
    ("bf16", 2, 4, 128, 32, 12, 6, 2048, 17000),
])
def test_decode_step_equals_separate_calls(B, dtype, S, g, d, p, m, L, k, n):
    """ice_decode_step gives bit-identical pages, top-k and attention to
    ice_insert + ice_query_pages + ice_sparse_attn, step after step, and its
    last step matches the oracle (every index array, candidates, pages,
    top-k, attention)."""
    steps = 6
    dev = torch.device("cuda")
    K, V, q0, _ = _inputs(S, n + steps, d, g, 24, 31, dtype)
    U = W.directions(m * L, d, 31, dtype).to(dev)
    print(f"[case] decode_step {dtype} S={S} g={g} d={d} p={p} m={m} L={L} k={k} n={n}",
          flush=True)
    mk = lambda: B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U,
                         page_size=p, budget_k=k, m=m, L=L, gqa_group=g, capacity=n + steps)
    a, b = mk(), mk()
    gen = torch.Generator().manual_seed(5)
    for t in range(steps):
        qt = torch.randn(S * g, d, generator=gen).to(q0.dtype).to(dev)
        kn, vn = K[:, n + t].contiguous().to(dev), V[:, n + t].contiguous().to(dev)
        pa, na, oa, ta = a.decode_step(kn, vn, qt, with_topk=True)
        b.insert(kn, vn)
        pb, nb, tb = b.query_pages(qt, with_topk=True)
        ob = b.sparse_attn(qt, pb, nb)
        torch.cuda.synchronize()
        assert torch.equal(pa, pb) and torch.equal(na, nb) and torch.equal(ta, tb)
        assert torch.equal(oa, ob)
    prm = oracle.Params(d=d, p=p, k=k, m=m, L=L, g=g)
    st = oracle.OracleStream(prm, _np(K[0, :n]), _np(V[0, :n]), _np(U), n_cap=n + steps)
    for t in range(steps):
        st.insert(_np(K[0, n + t]), _np(V[0, n + t]))
    q_s = _np(qt[:g])
    r = st.query(q_s, literal=False)
    _check_index(a, st, 0, n + steps)
    _check_query(a, st, 0, r, pa, na, ta, oa[:g], q_s)
    with pytest.raises(B.IceError) as e:
        a.decode_step(kn, vn, qt)
    assert e.value.status == B.ICE_ERR_CAPACITY


@pytest.mark.parametrize("dtype,g,d,p,k,k0,gqa", [
    ("bf16", 4, 128, 16, 256, 0, "mean"),   # the 36k layer's shape: 16 pages
    ("f32", 2, 64, 8, 128, 0, "mean"),      # 16 pages of 8
    ("bf16", 2, 128, 8, 256, 0, "mean"),    # 32 pages of 8: the largest selection waves walk alone
    ("bf16", 2, 128, 32, 256, 0, "mean"),   # 8 pages of 32
    ("bf16", 1, 128, 16, 256, 6, "mean"),   # a union of at most 24 tokens: fewer pages than 16
    ("bf16", 4, 128, 16, 256, 0, "max"),    # the GQA max mode (pooled walks of 4 heads)
])
def test_decode_step_without_topk_equals_with(B, dtype, g, d, p, k, k0, gqa):
    """ice_decode_step without a top-k output (the fused attention's waves
    then walk the first 64 ranks for themselves when those hold the whole
    selection) gives the pages and the attention of the same step with the
    top-k asked (one wave walks, the others wait), bit for bit, step after
    step on twin indices; the last step also against the oracle."""
    S, n, m, L, steps = 3, 4000, 4, 4, 5
    dev = torch.device("cuda")
    K, V, _, _ = _inputs(S, n + steps, d, g, 24, 47, dtype)
    U = W.directions(m * L, d, 47, dtype).to(dev)
    print(f"[case] decode without top-k {dtype} g={g} d={d} p={p} k={k} k0={k0} {gqa}", flush=True)
    mk = lambda: B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U,
                         page_size=p, budget_k=k, m=m, L=L, gqa_group=g, k0=k0,
                         capacity=n + steps, gqa_mode=gqa)
    a, b = mk(), mk()
    gen = torch.Generator().manual_seed(9)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for t in range(steps):
        qt = torch.randn(S * g, d, generator=gen).to(tdt).to(dev)
        kn, vn = K[:, n + t].contiguous().to(dev), V[:, n + t].contiguous().to(dev)
        pa, na, oa, _ = a.decode_step(kn, vn, qt)
        pb, nb, ob, tb = b.decode_step(kn, vn, qt, with_topk=True)
        torch.cuda.synchronize()
        assert torch.equal(na, nb)
        for s in range(S):
            assert torch.equal(pa[s, :int(na[s])], pb[s, :int(nb[s])])
        assert torch.equal(oa, ob)
    prm = oracle.Params(d=d, p=p, k=k, m=m, L=L, g=g, k0=k0, gqa_max=gqa == "max")
    st = oracle.OracleStream(prm, _np(K[1, :n]), _np(V[1, :n]), _np(U), n_cap=n + steps)
    for t in range(steps):
        st.insert(_np(K[1, n + t]), _np(V[1, n + t]))
    q_s = _np(qt[g:2 * g])
    r = st.query(q_s, literal=False)
    _check_query(a, st, 1, r, pb, nb, tb, oa[g:2 * g], q_s)


def test_decode_step_many_streams(B):
    """64 streams of 20,011 tokens (1,280 scan blocks, more than the device
    holds at once; the new token in the last, ragged range of every stream):
    decode steps match separate calls bit for bit and the oracle on two
    streams."""
    S, n, g, d, p, m, L, k, steps = 64, 20011, 1, 128, 16, 4, 2, 128, 3
    dev = torch.device("cuda")
    K, V, q0, _ = _inputs(S, n + steps, d, g, 16, 33, "bf16")
    U = W.directions(m * L, d, 33, "bf16").to(dev)
    print("[case] decode_step S=64 n=20011", flush=True)
    mk = lambda: B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U,
                         page_size=p, budget_k=k, m=m, L=L, gqa_group=g, capacity=n + steps)
    a, b = mk(), mk()
    gen = torch.Generator().manual_seed(9)
    for t in range(steps):
        qt = torch.randn(S * g, d, generator=gen).to(torch.bfloat16).to(dev)
        kn, vn = K[:, n + t].contiguous().to(dev), V[:, n + t].contiguous().to(dev)
        pa, na, oa, ta = a.decode_step(kn, vn, qt, with_topk=True)
        b.insert(kn, vn)
        pb, nb, tb = b.query_pages(qt, with_topk=True)
        ob = b.sparse_attn(qt, pb, nb)
        torch.cuda.synchronize()
        assert torch.equal(pa, pb) and torch.equal(na, nb) and torch.equal(ta, tb)
        assert torch.equal(oa, ob)
    prm = oracle.Params(d=d, p=p, k=k, m=m, L=L, g=g)
    for s_ in (0, 37):
        st = oracle.OracleStream(prm, _np(K[s_, :n]), _np(V[s_, :n]), _np(U), n_cap=n + steps)
        for t in range(steps):
            st.insert(_np(K[s_, n + t]), _np(V[s_, n + t]))
        q_s = _np(qt[s_ * g:(s_ + 1) * g])
        r = st.query(q_s, literal=False)
        _check_index(a, st, s_, n + steps)
        _check_query(a, st, s_, r, pa, na, ta, oa[s_ * g:(s_ + 1) * g], q_s)


def test_llama8b_decode_loop_36k_128_steps(B):
    """The 32-layer decode loop's per-layer work at full size: one
    36,864-token layer of 8 KV heads (32 query heads), 128 consecutive
    ice_decode_step calls, each appending one fresh (k, v) per head and
    querying with a fresh query cluster.  Two heads are followed by the oracle
    (insert, literal P-DCI walk, rerank, page walk, fp64 attention) and must
    match at every step; all 8 heads' index arrays are checked after the last
    step for those two heads."""
    w = W.WORKLOADS["llama8b_decode_36k"]
    layer, steps, follow = 31, 128, (0, 5)
    K, V, q0, U, _ = W.layer_inputs(w, layer=layer)
    dev = torch.device("cuda")
    print(f"[case] llama8b_decode_36k layer={layer} steps={steps}", flush=True)
    idx = B.Index(K.to(dev), V.to(dev), U.to(dev), page_size=w.p, budget_k=w.k, m=w.m, L=w.L,
                  gqa_group=w.g, capacity=w.n + steps)
    res = []
    ins = []
    for t in range(steps):
        kn, vn, qt = W.step_inputs(w, layer, t)
        pg, npg, out, tk = idx.decode_step(kn.to(dev), vn.to(dev), qt.to(dev), with_topk=True)
        res.append((pg.cpu(), npg.cpu(), out.cpu(), tk.cpu()))
        ins.append((kn, vn, qt))
    torch.cuda.synchronize()
    prm = oracle.Params(d=w.d, p=w.p, k=w.k, m=w.m, L=w.L, g=w.g)
    g = w.g
    for s in follow:
        st = oracle.OracleStream(prm, _np(K[s]), _np(V[s]), _np(U), n_cap=w.n + steps)
        for t in range(steps):
            kn, vn, qt = ins[t]
            st.insert(_np(kn[s]), _np(vn[s]))
            q_s = _np(qt[s * g:(s + 1) * g])
            r = st.query(q_s)
            pg, npg, out, tk = res[t]
            nsel = int(npg[s])
            np.testing.assert_array_equal(pg[s, :nsel].numpy(), r["page_ids"],
                                          err_msg=f"pages, head {s} step {t}")
            kk = len(r["topk"])
            np.testing.assert_array_equal(tk[s, :kk].numpy(), r["topk"],
                                          err_msg=f"top-k, head {s} step {t}")
            ref = st.attend(q_s, r["page_ids"])
            err = float(np.max(np.abs(out[s * g:(s + 1) * g].numpy() - ref)))
            assert err <= ATTN_TOL, (s, t, err)
        _check_index(idx, st, s, w.n + steps)


def test_long_generation_equals_rebuild(B):
    """A long generation on the full 36,864-token layer: 2,048 consecutive
    ice_decode_step calls (one generated token per head per step), then a
    rebuild over all 38,912 tokens with the stored c and tree depth.  Every
    index array and the next query's pages, top-k and attention are identical
    (inserts never drift from a rebuild); one head also against the oracle."""
    w = W.WORKLOADS["llama8b_decode_36k"]
    layer, steps = 7, 2048
    K, V, q0, U, _ = W.layer_inputs(w, layer=layer)
    dev = torch.device("cuda")
    print(f"[case] long generation layer={layer} steps={steps}", flush=True)
    cap = w.n + steps
    a = B.Index(K.to(dev), V.to(dev), U.to(dev), page_size=w.p, budget_k=w.k, m=w.m, L=w.L,
                gqa_group=w.g, capacity=cap)
    ks, vs = [], []
    for t in range(steps):
        kn, vn, qt = W.step_inputs(w, layer, t, device=dev)
        a.decode_step(kn, vn, qt)
        ks.append(kn)
        vs.append(vn)
    torch.cuda.synchronize()
    Kall = torch.cat([K.to(dev), torch.stack(ks, 1)], 1).contiguous()
    Vall = torch.cat([V.to(dev), torch.stack(vs, 1)], 1).contiguous()
    c = a.view("norm_c").cpu()
    D = a.layout()["tree_depth"]
    _, _, qn = W.step_inputs(w, layer, steps, device=dev)
    pa, na, ta = a.query_pages(qn, with_topk=True)
    oa = a.sparse_attn(qn, pa, na)
    n = w.n + steps
    for s in range(w.streams):
        b = B.Index(Kall[s:s + 1], Vall[s:s + 1], U.to(dev), page_size=w.p, budget_k=w.k, m=w.m,
                    L=w.L, gqa_group=w.g, capacity=cap, c=float(c[s]), tree_depth=D)
        qs = qn[s * w.g:(s + 1) * w.g].contiguous()
        pb, nb, tb = b.query_pages(qs, with_topk=True)
        ob = b.sparse_attn(qs, pb, nb)
        torch.cuda.synchronize()
        assert torch.equal(a.view("codes")[s, :n], b.view("codes")[0, :n])
        _check_list_storage(a, s, a.view("codes")[s].cpu().numpy())
        _check_list_storage(b, 0, b.view("codes")[0].cpu().numpy())
        la, lb = _logical_lists(a, s), _logical_lists(b, 0)
        assert np.array_equal(la[0], lb[0]) and np.array_equal(la[1], lb[1])
        if s == 0:  # the delta-merge turns the stored lists into the rebuild's, as stored
            a.merge_lists()
            assert a.layout()["n_build"] == n
        if s >= 0 and a.layout()["n_build"] == n:
            sa, sb = _stored_lists(a, s), _stored_lists(b, 0)
            assert np.array_equal(sa[0], sb[0]) and np.array_equal(sa[1], sb[1])
        assert torch.equal(a.view("loc")[s, :n], b.view("loc")[0, :n])
        npg = int(a.view("npages")[s])
        assert npg == int(b.view("npages")[0])
        for f in ("page_tokens", "page_len", "page_cell"):
            assert torch.equal(a.view(f)[s, :npg], b.view(f)[0, :npg]), f
        assert torch.equal(pa[s], pb[0]) and torch.equal(na[s], nb[0]) and torch.equal(ta[s], tb[0])
        assert torch.equal(oa[s * w.g:(s + 1) * w.g], ob)
        del b
    prm = oracle.Params(d=w.d, p=w.p, k=w.k, m=w.m, L=w.L, g=w.g)
    s = 3
    st = oracle.OracleStream(prm, _np(Kall[s, :w.n]), _np(Vall[s, :w.n]), _np(U), n_cap=cap)
    for t in range(steps):
        st.insert(_np(Kall[s, w.n + t]), _np(Vall[s, w.n + t]))
    q_s = _np(qn[s * w.g:(s + 1) * w.g])
    r = st.query(q_s)
    _check_query(a, st, s, r, pa, na, ta, oa[s * w.g:(s + 1) * w.g], q_s)


@pytest.mark.parametrize("n", [45000, 60000])
def test_scan_block_shapes(B, n):
    """8 streams of 45,000 and 60,000 tokens: scan and collect blocks of 768 and
    1,024 threads (the smallest shape that gives every block its own CU), with
    a decode step; two streams against the oracle."""
    S, g, d, p, m, L, k = 8, 4, 128, 16, 8, 4, 256
    dev = torch.device("cuda")
    K, V, q, _ = _inputs(S, n + 1, d, g, 64, 91, "bf16")
    U = W.directions(m * L, d, 91, "bf16").to(dev)
    print(f"[case] block shapes n={n}", flush=True)
    idx = B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U, page_size=p,
                  budget_k=k, m=m, L=L, gqa_group=g, capacity=n + 1)
    qd = q.to(dev)
    pg, npg, out, tk = idx.decode_step(K[:, n].contiguous().to(dev), V[:, n].contiguous().to(dev),
                                        qd, with_topk=True)
    torch.cuda.synchronize()
    prm = oracle.Params(d=d, p=p, k=k, m=m, L=L, g=g)
    for s in (0, 5):
        st = oracle.OracleStream(prm, _np(K[s, :n]), _np(V[s, :n]), _np(U), n_cap=n + 1)
        st.insert(_np(K[s, n]), _np(V[s, n]))
        q_s = _np(q[s * g:(s + 1) * g])
        r = st.query(q_s)
        _check_index(idx, st, s, n + 1)
        _check_query(idx, st, s, r, pg, npg, tk, out[s * g:(s + 1) * g], q_s)


@pytest.mark.parametrize("n", [50500, 50000])
def test_more_scan_blocks_than_the_device_holds(B, n):
    """16 streams of about 50,000 tokens: 512-thread scan and collect blocks,
    800 or 784 of them, more than the device holds at once (three per CU), so
    the blocks run in two waves.  n = 50,500 puts the decode step's new token
    in an even range, n = 50,000 in an odd one of a ragged last block.  Two
    decode steps, each against the oracle on the first and the last stream
    (every index array, candidates, pages, top-k, attention)."""
    S, g, d, p, m, L, k, steps = 16, 2, 128, 16, 8, 4, 256, 2
    dev = torch.device("cuda")
    K, V, q0, _ = _inputs(S, n + steps, d, g, 64, 93, "bf16")
    U = W.directions(m * L, d, 93, "bf16").to(dev)
    print(f"[case] more scan blocks than the device holds n={n}", flush=True)
    idx = B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U, page_size=p,
                  budget_k=k, m=m, L=L, gqa_group=g, capacity=n + steps)
    prm = oracle.Params(d=d, p=p, k=k, m=m, L=L, g=g)
    sts = {s: oracle.OracleStream(prm, _np(K[s, :n]), _np(V[s, :n]), _np(U), n_cap=n + steps)
           for s in (0, S - 1)}
    gen = torch.Generator().manual_seed(8)
    for t in range(steps):
        qt = torch.randn(S * g, d, generator=gen).to(torch.bfloat16)
        pg, npg, out, tk = idx.decode_step(K[:, n + t].contiguous().to(dev),
                                            V[:, n + t].contiguous().to(dev), qt.to(dev),
                                            with_topk=True)
        torch.cuda.synchronize()
        for s, st in sts.items():
            st.insert(_np(K[s, n + t]), _np(V[s, n + t]))
            q_s = _np(qt[s * g:(s + 1) * g])
            r = st.query(q_s)
            _check_query(idx, st, s, r, pg, npg, tk, out[s * g:(s + 1) * g], q_s)
    for s, st in sts.items():
        _check_index(idx, st, s, n + steps)


def test_capacity_error(B):
    dev = torch.device("cuda")
    K, V, q, _ = _inputs(1, 40, 128, 1, 4, 13, "bf16")
    U = W.directions(4, 128, 13, "bf16").to(dev)
    idx = B.Index(K[:, :39].contiguous().to(dev), V[:, :39].contiguous().to(dev), U,
                  page_size=16, budget_k=32, m=2, L=2, capacity=40)
    idx.insert(K[:, 39].contiguous().to(dev), V[:, 39].contiguous().to(dev))
    with pytest.raises(B.IceError) as e:
        idx.insert(K[:, 39].contiguous().to(dev), V[:, 39].contiguous().to(dev))
    assert e.value.status == B.ICE_ERR_CAPACITY


def test_needle_131k_full_layer_sampled(B):
    """Full-size layer of the 131,072-token batch-4 needle workload (32 streams):
    every stream's needle tokens land in selected pages; two sampled streams
    are checked stage by stage against the oracle."""
    w = W.WORKLOADS["llama8b_needle_131k_b4"]
    dev = torch.device("cuda")
    print("[case] needle 131k full layer", flush=True)
    K, V, q, U, p0 = W.layer_inputs(w, layer=0, device=dev)
    idx = B.Index(K, V, U, page_size=w.p, budget_k=w.k, m=w.m, L=w.L, gqa_group=w.g,
                  capacity=w.n + 128)
    page_ids, n_pages, topk = idx.query_pages(q, with_topk=True)
    out = idx.sparse_attn(q, page_ids, n_pages)
    torch.cuda.synchronize()
    loc = idx.view("loc")
    for s in range(w.streams):
        sel = set(page_ids[s, :int(n_pages[s])].tolist())
        needle_pages = set((loc[s, p0[s]:p0[s] + w.needle] // w.p).tolist())
        assert needle_pages <= sel, s
    prm = oracle.Params(d=w.d, p=w.p, k=w.k, m=w.m, L=w.L, g=w.g)
    for s in (5, 26):
        print(f"[case] needle 131k stream {s} vs oracle", flush=True)
        st = oracle.OracleStream(prm, _np(K[s]), _np(V[s]), _np(U), n_cap=w.n + 128)
        _check_index(idx, st, s, w.n)
        q_s = _np(q[s * w.g:(s + 1) * w.g])
        r = st.query(q_s, literal=False)
        _check_query(idx, st, s, r, page_ids, n_pages, topk, out[s * w.g:(s + 1) * w.g], q_s)


@pytest.mark.parametrize("S,n,g,p,k,m,L,k0", [
    (2, 20011, 2, 16, 1024, 6, 6, 0),   # union up to 6,144 tokens per stream
    (1, 30000, 1, 16, 4800, 4, 2, 0),   # top-k of 4,800 ranks: several rank windows, 300 pages
    (2, 9000, 4, 32, 256, 4, 4, 1500),  # k0 above the budget: few pages, large union
])
def test_large_union(B, S, n, g, p, k, m, L, k0):
    """L * k0 above 4,096: the union stays in global memory and is ranked in windows."""
    run_case(B, S=S, n=n, g=g, p=p, k=k, m=m, L=L, k0=k0, seed=40 + L, literal=False)


def test_large_union_fewer_tokens_than_k0(B):
    """L * k0 above 4,096 with fewer tokens than k0: every composite returns
    all tokens and the union is the whole stream; then inserts grow it."""
    run_case(B, S=2, n=700, inserts=30, g=2, p=16, k=1024, m=3, L=6, seed=42, literal=False)


def test_identical_keys_large_union(B):
    """Every score equal and a union of 4,608 tokens: one score bucket larger
    than a rank window, ranked by token."""
    S, n, d, g = 1, 6000, 128, 1
    K = torch.full((S, n, d), 0.5, dtype=torch.bfloat16)
    V = torch.randn(S, n, d, generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    q = torch.randn(S * g, d, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    run_case(B, S=S, n=n, d=d, g=g, p=16, k=4608, m=3, L=2, keys=(K, V, q), seed=41,
             literal=False)


def test_large_union_walk_past_the_first_window(B):
    """1,500 near-copies of 60 times the query direction, far above every other
    score, fill whole pages of 32: the first 1,024 ranks hold at most 32 distinct
    pages, fewer than the 64 the budget selects, so the large-union page walk
    goes on into its next rank window.  Pages, top-k and attention against
    the oracle, with and without the top-k asked (its windows differ)."""
    S, n, d, g, p, k, m, L = 2, 20000, 128, 1, 32, 2048, 4, 4
    K, V, _, _ = _inputs(S, n, d, g, 64, 95, "bf16")
    gen = torch.Generator().manual_seed(96)
    u = torch.randn(d, generator=gen)
    u = u / u.norm()
    K[:, 5000:6500] = (60.0 * u + 0.5 * torch.randn(S, 1500, d, generator=gen)).to(torch.bfloat16)
    q = u.repeat(S * g, 1).to(torch.bfloat16)
    idx = run_case(B, S=S, n=n, d=d, g=g, p=p, k=k, m=m, L=L, keys=(K, V, q), seed=95,
                   literal=False)
    prm = oracle.Params(d=d, p=p, k=k, m=m, L=L, g=g)
    st = oracle.OracleStream(prm, _np(K[0]), _np(V[0]), _np(W.directions(m * L, d, 95, "bf16")),
                             n_cap=n)
    r = st.query(_np(q[:g]), literal=False)
    assert L * k > 4096  # the large-union finaliser (chosen by L * k0)
    assert len(np.unique(st.page_of[r["ranked"][:1024]])) < k // p  # the case is what it says
    dev = torch.device("cuda")
    pg, npg, _ = idx.query_pages(q.to(dev))  # the page walk alone: walk-only windows
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pg[0, :int(npg[0])].cpu().numpy(), r["page_ids"])


def test_qwen3_4b_262k_full_layer_sampled(B):
    """Full-size layer of the 262,144-token Qwen3-4B-shaped workload (8 streams,
    power-law cluster sizes, L * k0 = 12,288): two sampled streams checked
    stage by stage against the oracle."""
    w = W.WORKLOADS["qwen3_4b_262k"]
    dev = torch.device("cuda")
    print("[case] qwen3_4b_262k full layer", flush=True)
    K, V, q, U, _ = W.layer_inputs(w, layer=0, device=dev)
    idx = B.Index(K, V, U, page_size=w.p, budget_k=w.k, m=w.m, L=w.L, gqa_group=w.g,
                  capacity=w.n + 64)
    page_ids, n_pages, topk = idx.query_pages(q, with_topk=True)
    out = idx.sparse_attn(q, page_ids, n_pages)
    torch.cuda.synchronize()
    assert torch.all(n_pages == w.k // w.p)
    prm = oracle.Params(d=w.d, p=w.p, k=w.k, m=w.m, L=w.L, g=w.g)
    for s in (2, 7):
        print(f"[case] qwen3_4b_262k stream {s} vs oracle", flush=True)
        st = oracle.OracleStream(prm, _np(K[s]), _np(V[s]), _np(U), n_cap=w.n + 64)
        _check_index(idx, st, s, w.n)
        q_s = _np(q[s * w.g:(s + 1) * w.g])
        r = st.query(q_s, literal=False)
        _check_query(idx, st, s, r, page_ids, n_pages, topk, out[s * w.g:(s + 1) * w.g], q_s)


# ---------------------------------------------------------------- visit budget k1

@pytest.mark.parametrize("k1", [1, 7, 500, 3001, 9000, 15999, 16000, 1 << 40])
def test_visit_budget(B, k1):
    """Walks bounded at k1 list entries per composite (m * n = 16,000 here):
    from no completed token (k1 = 1) to the unbounded result (k1 >= m * n)."""
    idx = run_case(B, S=2, n=4000, g=2, p=16, k=256, m=4, L=2, k1=k1, seed=41)
    cc = idx.view("cand_count").cpu().numpy()
    if k1 <= 500:  # the budget, not k0 = 256, ends every walk
        assert cc.max() < 256
    if k1 == 1:  # a token needs all m = 4 of its entries visited
        assert cc.max() == 0


def test_visit_budget_llama8b_layer_36k(B):
    """A bounded walk (k1 = m*n/3 visits per composite) on the full 36,864-token
    layer: the visit-budget passes with the scan and collect grids of that size
    (1,280-token blocks), two heads against the oracle's literal walk."""
    w = W.WORKLOADS["llama8b_layer_36k"]
    K, V, q, U, _ = W.layer_inputs(w, layer=3)
    k1 = w.m * w.n // 3
    dev = torch.device("cuda")
    print(f"[case] llama8b_layer_36k k1={k1}", flush=True)
    idx = B.Index(K.to(dev), V.to(dev), U.to(dev), page_size=w.p, budget_k=w.k, m=w.m, L=w.L,
                  gqa_group=w.g, k1=k1, capacity=w.n + 8)
    qd = q.to(dev)
    page_ids, n_pages, topk = idx.query_pages(qd, with_topk=True)
    out = idx.sparse_attn(qd, page_ids, n_pages)
    torch.cuda.synchronize()
    prm = oracle.Params(d=w.d, p=w.p, k=w.k, m=w.m, L=w.L, g=w.g, k1=k1)
    for s in (1, 6):
        st = oracle.OracleStream(prm, _np(K[s]), _np(V[s]), _np(U), n_cap=w.n + 8)
        q_s = _np(q[s * w.g:(s + 1) * w.g])
        r = st.query(q_s)
        _check_query(idx, st, s, r, page_ids, n_pages, topk, out[s * w.g:(s + 1) * w.g], q_s)


def test_visit_budget_ragged_fp32_inserts(B):
    run_case(B, S=3, n=2333, g=1, p=8, k=128, m=3, L=3, dtype="f32", inserts=4, k1=2500,
             seed=42)


def test_visit_budget_identical_keys(B):
    """Every key equal: every entry of a composite ties at one distance, so the
    k1-th entry is found by token and list order alone."""
    S, n, d, g = 2, 700, 128, 2
    K = torch.full((S, n, d), 0.5, dtype=torch.bfloat16)
    V = torch.randn(S, n, d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    q = torch.randn(S * g, d, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    for k1 in (1, 4, 5, 999, 1001, 2799):
        run_case(B, S=S, n=n, d=d, g=g, p=16, k=64, m=4, L=2, keys=(K, V, q), k1=k1, seed=10)


def test_visit_budget_few_distinct_keys(B):
    """Keys drawn from four points: long runs of equal distances around the
    k1-th entry in every composite."""
    S, n, d, g = 2, 3000, 64, 1
    gen = torch.Generator().manual_seed(8)
    pts = torch.randn(4, d, generator=gen)
    K = pts[torch.randint(0, 4, (S, n), generator=gen)].to(torch.bfloat16)
    V = torch.randn(S, n, d, generator=gen).to(torch.bfloat16)
    q = torch.randn(S * g, d, generator=gen).to(torch.bfloat16)
    for k1 in (2000, 6001, 11999):
        run_case(B, S=S, n=n, d=d, g=g, p=16, k=128, m=4, L=2, keys=(K, V, q), k1=k1, seed=11)


def test_visit_budget_large_union(B):
    """L * k0 = 6,000 takes the large-union finaliser."""
    for k1 in (20000, 45000):
        run_case(B, S=1, n=12000, g=2, p=16, k=1024, m=4, L=2, k0=3000, k1=k1, seed=43,
                 literal=False)


def test_visit_budget_decode_step(B):
    """ice_decode_step with a bounded walk equals the oracle after every step."""
    S, n, steps, g, d, p, m, L, k, k1 = 2, 2500, 3, 2, 128, 16, 4, 2, 128, 3000
    dev = torch.device("cuda")
    K, V, _, _ = _inputs(S, n + steps, d, g, 24, 44, "bf16")
    U = W.directions(m * L, d, 44, "bf16")
    print(f"[case] decode_step k1={k1}", flush=True)
    a = B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U.to(dev),
                page_size=p, budget_k=k, m=m, L=L, gqa_group=g, k1=k1, capacity=n + steps)
    prm = oracle.Params(d=d, p=p, k=k, m=m, L=L, g=g, k1=k1)
    sts = [oracle.OracleStream(prm, _np(K[s, :n]), _np(V[s, :n]), _np(U), n_cap=n + steps)
           for s in range(S)]
    gen = torch.Generator().manual_seed(6)
    for t in range(steps):
        qt = torch.randn(S * g, d, generator=gen).to(torch.bfloat16)
        pa, na, oa, ta = a.decode_step(K[:, n + t].contiguous().to(dev),
                                       V[:, n + t].contiguous().to(dev), qt.to(dev),
                                       with_topk=True)
        torch.cuda.synchronize()
        for s in range(S):
            sts[s].insert(_np(K[s, n + t]), _np(V[s, n + t]))
            q_s = _np(qt[s * g:(s + 1) * g])
            r = sts[s].query(q_s, literal=True)
            _check_query(a, sts[s], s, r, pa, na, ta, oa[s * g:(s + 1) * g], q_s)


@pytest.mark.parametrize("k1", [0, 5000])
def test_high_threshold_bins_decode_step(B, k1):
    """Queries along the first direction (plus a little noise): on the first
    composite every distance lies above bin 255, so its threshold bin is not
    among the low bins the collect searches first (it reads the whole
    histogram), and with a visit budget the k1-th entry's distance is that
    high too; the other composites stay in the low bins.  ice_decode_step
    against the oracle after every step, unbounded and bounded walks."""
    S, n, steps, g, d, p, m, L, k = 2, 2500, 3, 2, 128, 16, 4, 3, 128
    dev = torch.device("cuda")
    K, V, _, _ = _inputs(S, n + steps, d, g, 24, 45, "bf16")
    U = W.directions(m * L, d, 45, "bf16")
    print(f"[case] high threshold bins decode_step k1={k1}", flush=True)
    a = B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U.to(dev),
                page_size=p, budget_k=k, m=m, L=L, gqa_group=g, k1=k1, capacity=n + steps)
    prm = oracle.Params(d=d, p=p, k=k, m=m, L=L, g=g, k1=k1)
    sts = [oracle.OracleStream(prm, _np(K[s, :n]), _np(V[s, :n]), _np(U), n_cap=n + steps)
           for s in range(S)]
    gen = torch.Generator().manual_seed(7)
    for t in range(steps):
        qt = (U[0, :d].float().repeat(S * g, 1)
              + 0.03 * torch.randn(S * g, d, generator=gen)).to(torch.bfloat16)
        pa, na, oa, ta = a.decode_step(K[:, n + t].contiguous().to(dev),
                                       V[:, n + t].contiguous().to(dev), qt.to(dev),
                                       with_topk=True)
        torch.cuda.synchronize()
        for s in range(S):
            sts[s].insert(_np(K[s, n + t]), _np(V[s, n + t]))
            q_s = _np(qt[s * g:(s + 1) * g])
            r = sts[s].query(q_s, literal=True)
            if t == 0 and s == 0:  # the case is what it says: composite 0 above bin 255
                c0 = sts[s].codes[:n + 1, :m].astype(np.int64)
                M0 = np.abs(c0 - r["qcode"][:m].astype(np.int64)).max(axis=1)
                assert (M0 >> 20).min() > 255
            _check_query(a, sts[s], s, r, pa, na, ta, oa[s * g:(s + 1) * g], q_s)


# ---------------------------------------------------------------- parameter ranges

@pytest.mark.parametrize("m,L,k", [(10, 4, 256), (12, 6, 256), (4, 32, 128)])
def test_inserts_many_directions(B, m, L, k):
    """Standalone inserts with more than 32 directions (the insert stages the
    directions 32 at a time: 40, 72 and 128 directions take two, three and
    four chunks), then the query; every array against the oracle."""
    run_case(B, S=2, n=2500, inserts=37, g=2, p=16, k=k, m=m, L=L, seed=50 + m)


@pytest.mark.parametrize("m,L", [(2, 8), (3, 8), (2, 20), (1, 32), (4, 32)])
def test_many_composites(B, m, L):
    """More than six composites: the scan's histogram goes straight to global
    memory, the collect reads M of composites 8 and up from memory, and above
    16 composites a finaliser wave serves several (L = 32, m = 4: the largest
    index, 128 directions)."""
    run_case(B, S=2, n=4100, g=2, p=16, k=128, m=m, L=L, seed=60 + L, inserts=5)


@pytest.mark.parametrize("g,d,dtype", [(8, 128, "bf16"), (16, 128, "bf16"), (16, 64, "f32"),
                                       (5, 128, "bf16")])
def test_wide_gqa_groups(B, g, d, dtype):
    """GQA groups above 4: the scan folds the heads four at a time, and the
    attention's matrix-core tiles carry up to 16 heads."""
    run_case(B, S=2, n=3300, g=g, d=d, p=16, k=256, m=4, L=3, dtype=dtype, seed=70 + g)


@pytest.mark.parametrize("g,L", [(16, 4), (8, 20)])
def test_decode_step_wide_groups_many_composites(B, g, L):
    """ice_decode_step (in-scan insert, fused attention) with 16 query heads
    and with 20 composites: identical to the separate calls, and the oracle."""
    S, n, d, p, m, k, steps = 2, 5000, 128, 16, 2, 128, 3
    dev = torch.device("cuda")
    K, V, _, _ = _inputs(S, n + steps, d, g, 24, 90 + g, "bf16")
    U = W.directions(m * L, d, 90 + g, "bf16").to(dev)
    print(f"[case] decode_step g={g} L={L}", flush=True)
    mk = lambda: B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U,
                         page_size=p, budget_k=k, m=m, L=L, gqa_group=g, capacity=n + steps)
    a, b = mk(), mk()
    gen = torch.Generator().manual_seed(17)
    for t in range(steps):
        qt = torch.randn(S * g, d, generator=gen).to(torch.bfloat16).to(dev)
        kn, vn = K[:, n + t].contiguous().to(dev), V[:, n + t].contiguous().to(dev)
        pa, na, oa, ta = a.decode_step(kn, vn, qt, with_topk=True)
        b.insert(kn, vn)
        pb, nb, tb = b.query_pages(qt, with_topk=True)
        ob = b.sparse_attn(qt, pb, nb)
        torch.cuda.synchronize()
        assert torch.equal(pa, pb) and torch.equal(na, nb) and torch.equal(ta, tb)
        assert torch.equal(oa, ob)
    prm = oracle.Params(d=d, p=p, k=k, m=m, L=L, g=g)
    for s in range(S):
        st = oracle.OracleStream(prm, _np(K[s, :n]), _np(V[s, :n]), _np(U), n_cap=n + steps)
        for t in range(steps):
            st.insert(_np(K[s, n + t]), _np(V[s, n + t]))
        q_s = _np(qt[s * g:(s + 1) * g])
        r = st.query(q_s)
        _check_index(a, st, s, n + steps)
        _check_query(a, st, s, r, pa, na, ta, oa[s * g:(s + 1) * g], q_s)


# ---------------------------------------------------------------- query statistics

def _check_stats(rec, st, r):
    """One stream's ice_query_stats against the oracle's walk: the visits of
    every composite, the union size, pages and attended tokens."""
    assert rec["visits"] == [int(v) for v in r["visits"]], (rec["visits"], r["visits"])
    assert rec["n_cand"] == len(r["C"])
    assert rec["n_pages"] == len(r["page_ids"])
    assert rec["n_tokens"] == int(st.page_len[r["page_ids"]].sum()) if len(r["page_ids"]) else \
        rec["n_tokens"] == 0


@pytest.mark.parametrize("case", [
    dict(S=2, n=4100, g=2, p=16, k=128, m=4, L=3, seed=101),
    dict(S=2, n=3000, g=1, p=16, k=128, m=4, L=2, k1=2500, seed=102),          # budget ends walks
    dict(S=2, n=3000, g=1, p=16, k=128, m=4, L=2, k1=9000, seed=103),          # mixed
    dict(S=1, n=100, g=2, p=16, k=256, m=4, L=2, seed=104),                    # n < k0
    dict(S=1, n=9000, g=2, p=16, k=1024, m=3, L=6, seed=105),                  # large union
    dict(S=2, n=2500, g=2, p=16, k=128, m=2, L=20, inserts=7, seed=106),       # 20 composites
    dict(S=1, n=0, g=1, p=16, k=32, m=2, L=2, inserts=3, seed=107),            # tiny
])
def test_query_stats(B, case):
    """ice_query_pages with the statistics output: every composite's visit
    count equals the oracle's literal walk, and |C|, pages and attended tokens
    equal the oracle's."""
    c = dict(d=128, k0=0, k1=0, inserts=0)
    c.update(case)
    dev = torch.device("cuda")
    S, n, ins = c["S"], c["n"], c["inserts"]
    K, V, q, _ = _inputs(S, n + ins, c["d"], c["g"], 24, c["seed"], "bf16")
    U = W.directions(c["m"] * c["L"], c["d"], c["seed"], "bf16")
    print(f"[case] stats {case}", flush=True)
    idx = B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U.to(dev),
                  page_size=c["p"], budget_k=c["k"], m=c["m"], L=c["L"], gqa_group=c["g"],
                  k0=c["k0"], k1=c["k1"], capacity=max(n + ins, 1))
    for t in range(ins):
        idx.insert(K[:, n + t].contiguous().to(dev), V[:, n + t].contiguous().to(dev))
    stats = B.stats_tensor(S, dev)
    qd = q.to(dev)
    pg, npg, tk = idx.query_pages(qd, with_topk=True, stats=stats)
    pg2, npg2, tk2 = idx.query_pages(qd, with_topk=True)  # statistics change nothing
    torch.cuda.synchronize()
    assert torch.equal(pg, pg2) and torch.equal(npg, npg2) and torch.equal(tk, tk2)
    recs = B.parse_stats(stats, c["L"])
    prm = oracle.Params(d=c["d"], p=c["p"], k=c["k"], m=c["m"], L=c["L"], g=c["g"], k0=c["k0"],
                        k1=c["k1"])
    for s in range(S):
        st = oracle.OracleStream(prm, _np(K[s, :n]), _np(V[s, :n]), _np(U), n_cap=max(n + ins, 1))
        for t in range(ins):
            st.insert(_np(K[s, n + t]), _np(V[s, n + t]))
        r = st.query(_np(q[s * c["g"]:(s + 1) * c["g"]]), literal=True)
        _check_stats(recs[s], st, r)


def test_decode_step_stats_llama8b_layer_36k(B):
    """ice_decode_step with statistics on the full 36,864-token layer (the
    benchmark's workload): visits, union, pages and tokens of all eight heads
    against the oracle's literal walk."""
    w = W.WORKLOADS["llama8b_layer_36k"]
    K, V, q, U, _ = W.layer_inputs(w, layer=2)
    kn, vn, qn = W.step_inputs(w, layer=2, step=0)
    dev = torch.device("cuda")
    print("[case] decode stats llama8b_layer_36k", flush=True)
    idx = B.Index(K.to(dev), V.to(dev), U.to(dev), page_size=w.p, budget_k=w.k, m=w.m, L=w.L,
                  gqa_group=w.g, capacity=w.n + 4)
    stats = B.stats_tensor(w.streams, dev)
    pg, npg, out, _ = idx.decode_step(kn.to(dev), vn.to(dev), qn.to(dev), stats=stats)
    torch.cuda.synchronize()
    recs = B.parse_stats(stats, w.L)
    prm = oracle.Params(d=w.d, p=w.p, k=w.k, m=w.m, L=w.L, g=w.g)
    for s in range(w.streams):
        st = oracle.OracleStream(prm, _np(K[s]), _np(V[s]), _np(U), n_cap=w.n + 4)
        st.insert(_np(kn[s]), _np(vn[s]))
        r = st.query(_np(qn[s * w.g:(s + 1) * w.g]))
        _check_stats(recs[s], st, r)
        np.testing.assert_array_equal(pg[s, :int(npg[s])].cpu().numpy(), r["page_ids"])


def test_blocked_dot_order_cases(B):
    """The query side's dot products take the blocked order on the GPU too: a
    query code that sits on a rounding tie under element order (the oracle
    pin's query: code 3, not 2) and keys whose scores tie only under the
    blocked order (ranked 0, 1, 2 by token), then every stage against the
    oracle."""
    d, n, m, L = 128, 300, 2, 2
    gen = torch.Generator().manual_seed(3)
    K = torch.randn(1, n, d, generator=gen) * 0.01
    K[0, :3] = 0.0
    K[0, :3, 0] = 1.0
    K[0, 0, 32] = K[0, 0, 48] = 2.0 ** -53
    K[0, 1, 1] = 2.0 ** -52
    K[0, 2, 16] = K[0, 2, 32] = 2.0 ** -53
    V = torch.randn(1, n, d, generator=gen)
    q = torch.ones(1, d)
    run_case(B, S=1, n=n, d=d, g=1, p=16, k=64, m=m, L=L, dtype="f32", k0=n, seed=5,
             keys=(K, V, q))
    # the query code case: q = e0 + 2^-40 (e32 + e48), direction 0 crafted
    dev = torch.device("cuda")
    U = W.directions(m * L, d, 6, "f32")
    U[0] = 0.0
    U[0, 0], U[0, 32], U[0, 48] = 5 * 2.0 ** -30, 2.0 ** -41, 2.0 ** -41
    qq = torch.zeros(1, d)
    qq[0, 0], qq[0, 32], qq[0, 48] = 1.0, 2.0 ** -40, 2.0 ** -40
    idx = B.Index(K.to(dev), V.to(dev), U.to(dev), page_size=16, budget_k=64, m=m, L=L,
                  capacity=n)
    idx.query_pages(qq.to(dev))
    torch.cuda.synchronize()
    _, qcode = oracle.query_prep(qq.numpy(), U.numpy())
    assert int(qcode[0]) == 3
    np.testing.assert_array_equal(idx.view("qcode")[0].cpu().numpy(), qcode)



# ---------------------------------------------------------------- GQA max mode

@pytest.mark.parametrize("case", [
    dict(S=2, n=5003, g=4, p=16, k=256, m=8, L=4, seed=201),             # 16 walks, 4,096 pooled
    dict(S=3, n=3001, g=2, p=16, k=128, m=4, L=2, seed=202, inserts=9),  # 4 walks, 512 pooled
    dict(S=2, n=2600, g=3, p=8, k=64, m=3, L=3, d=64, dtype="f32", seed=203),
    dict(S=2, n=4000, g=2, p=16, k=128, m=4, L=2, k1=5000, seed=204),     # bounded walks
    dict(S=1, n=150, g=4, p=16, k=256, m=4, L=2, seed=205),               # fewer tokens than k0
    # every head in one scan block: 48 directions (three code rounds), 16 walks
    dict(S=2, n=7001, g=4, p=16, k=64, m=12, L=4, seed=208),
    # 60 directions, 12 walks (the two-head block's limit)
    dict(S=3, n=4500, g=2, p=16, k=128, m=10, L=6, seed=209),
    # 1024-thread scan blocks, more of them than the device holds at once
    dict(S=96, n=6000, g=4, p=16, k=64, m=4, L=4, seed=210, check=(0, 47, 95)),
    # 24 and 32 walks: one scan pass per head, the collect's walks past its
    # 16 register slots read from memory
    dict(S=2, n=3000, g=4, p=16, k=64, m=3, L=6, seed=211),
    dict(S=2, n=2500, g=8, p=16, k=32, m=2, L=4, seed=212),
    # bounded walks with every head in one scan block (12 walks)
    dict(S=2, n=4000, g=4, p=16, k=128, m=4, L=3, k1=3000, seed=213),
])
def test_gqa_max(B, case):
    """GQA max mode: every head walks every composite with its own query codes,
    the pooled candidates are ranked by the largest head score; every walk's
    candidates, the query codes of every head, pages, top-k and attention
    against the oracle's max reading."""
    run_case(B, gqa="max", **case)


def test_gqa_max_one_head_is_mean(B):
    """With one head the max mode's pages, top-k and attention equal the mean
    mode's bit for bit."""
    S, n, d = 2, 4000, 128
    dev = torch.device("cuda")
    K, V, q, _ = _inputs(S, n, d, 1, 20, 206, "bf16")
    U = W.directions(8, d, 206, "bf16").to(dev)
    res = []
    for mode in ("mean", "max"):
        idx = B.Index(K.to(dev), V.to(dev), U, page_size=16, budget_k=128, m=4, L=2, gqa_group=1,
                      gqa_mode=mode)
        pg, npg, tk = idx.query_pages(q.to(dev), with_topk=True)
        out = idx.sparse_attn(q.to(dev), pg, npg)
        torch.cuda.synchronize()
        res.append((pg.cpu(), npg.cpu(), tk.cpu(), out.cpu()))
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_gqa_max_decode_step_and_stats(B):
    """A decode step in the max mode (the first head's pass inserts the token)
    equals insert + query + attention, and its statistics (visits of all
    g * L walks, |C|, pages, tokens) equal the oracle's literal walks."""
    S, n, g, d, p, m, L, k, steps = 2, 3000, 4, 128, 16, 4, 3, 128, 3
    dev = torch.device("cuda")
    K, V, _, _ = _inputs(S, n + steps, d, g, 24, 207, "bf16")
    U = W.directions(m * L, d, 207, "bf16").to(dev)
    mk = lambda: B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U,
                         page_size=p, budget_k=k, m=m, L=L, gqa_group=g, capacity=n + steps,
                         gqa_mode="max")
    a, b = mk(), mk()
    gen = torch.Generator().manual_seed(21)
    stats = B.stats_tensor(S, dev)
    for t in range(steps):
        qt = torch.randn(S * g, d, generator=gen).to(torch.bfloat16).to(dev)
        kn, vn = K[:, n + t].contiguous().to(dev), V[:, n + t].contiguous().to(dev)
        pa, na, oa, ta = a.decode_step(kn, vn, qt, with_topk=True, stats=stats)
        b.insert(kn, vn)
        pb, nb, tb = b.query_pages(qt, with_topk=True)
        ob = b.sparse_attn(qt, pb, nb)
        torch.cuda.synchronize()
        assert torch.equal(pa, pb) and torch.equal(na, nb) and torch.equal(ta, tb)
        assert torch.equal(oa, ob)
    recs = B.parse_stats(stats, g * L)
    prm = oracle.Params(d=d, p=p, k=k, m=m, L=L, g=g, gqa_max=True)
    for s in range(S):
        st = oracle.OracleStream(prm, _np(K[s, :n]), _np(V[s, :n]), _np(U), n_cap=n + steps)
        for t in range(steps):
            st.insert(_np(K[s, n + t]), _np(V[s, n + t]))
        q_s = _np(qt[s * g:(s + 1) * g])
        r = st.query(q_s, literal=True)
        _check_index(a, st, s, n + steps)
        _check_query(a, st, s, r, pa, na, ta, oa[s * g:(s + 1) * g], q_s)
        _check_stats(recs[s], st, r)


def test_gqa_max_llama8b_layer_36k(B):
    """The 36,864-token Llama-3.1-8B layer in the max mode (4 heads x 4
    composites = 16 walks per KV head): two heads against the oracle."""
    w = W.WORKLOADS["llama8b_layer_36k"]
    K, V, q, U, _ = W.layer_inputs(w, layer=5)
    dev = torch.device("cuda")
    print("[case] gqa max llama8b_layer_36k", flush=True)
    idx = B.Index(K.to(dev), V.to(dev), U.to(dev), page_size=w.p, budget_k=w.k, m=w.m, L=w.L,
                  gqa_group=w.g, capacity=w.n + 8, gqa_mode="max")
    qd = q.to(dev)
    page_ids, n_pages, topk = idx.query_pages(qd, with_topk=True)
    out = idx.sparse_attn(qd, page_ids, n_pages)
    torch.cuda.synchronize()
    prm = oracle.Params(d=w.d, p=w.p, k=w.k, m=w.m, L=w.L, g=w.g, gqa_max=True)
    for s in (2, 6):
        st = oracle.OracleStream(prm, _np(K[s]), _np(V[s]), _np(U), n_cap=w.n + 8)
        q_s = _np(q[s * w.g:(s + 1) * w.g])
        r = st.query(q_s, literal=False)
        _check_query(idx, st, s, r, page_ids, n_pages, topk, out[s * w.g:(s + 1) * w.g], q_s)



# ---------------------------------------------------------------- host-offloaded pool

@pytest.mark.parametrize("case", [
    dict(S=4, n=6000, g=4, p=16, k=256, m=8, L=4, gqa="mean", dtype="bf16"),
    dict(S=2, n=9000, g=2, p=16, k=1024, m=4, L=3, gqa="mean", dtype="bf16"),  # four splits
    dict(S=2, n=5000, g=4, p=16, k=256, m=8, L=4, gqa="max", dtype="bf16"),
    dict(S=2, n=3000, g=2, p=8, k=128, m=3, L=3, gqa="mean", dtype="f32", d=64),
    # the values alone in host memory, the keys resident
    dict(S=4, n=6000, g=4, p=16, k=256, m=8, L=4, gqa="mean", dtype="bf16", mode="values"),
    dict(S=2, n=9000, g=2, p=16, k=1024, m=4, L=3, gqa="mean", dtype="bf16", mode="values"),
    dict(S=2, n=3000, g=2, p=8, k=128, m=3, L=3, gqa="max", dtype="f32", d=64, mode="values"),
])
def test_offloaded_pool_equals_resident(B, case):
    """The page pool in pinned host memory (or its values alone, the keys
    resident): builds, inserts and decode steps write it over the host link,
    the rerank reads its key rows there (or in HBM), and the selected pages
    are staged in HBM for the attention.  Every index array,
    page, top-k and attention output equals the resident pool's bit for bit,
    step after step; the last step also against the oracle."""
    c = dict(d=128)
    c.update(case)
    S, n, g, d, steps = c["S"], c["n"], c["g"], c["d"], 3
    dev = torch.device("cuda")
    K, V, _, _ = _inputs(S, n + steps, d, g, 24, 301, c["dtype"])
    U = W.directions(c["m"] * c["L"], d, 301, c["dtype"]).to(dev)
    print(f"[case] offload {case}", flush=True)
    kw = dict(page_size=c["p"], budget_k=c["k"], m=c["m"], L=c["L"], gqa_group=g,
              capacity=n + steps + 2, gqa_mode=c["gqa"])
    mode = c.get("mode", True)
    a = B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U, offload=mode,
                **kw)
    b = B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U, **kw)
    assert a.layout()["offload"] == (2 if mode == "values" else 1) and b.layout()["offload"] == 0
    gen = torch.Generator().manual_seed(31)
    td = W.torch_dtype(c["dtype"])
    for t in range(steps):
        qt = torch.randn(S * g, d, generator=gen).to(td).to(dev)
        kn, vn = K[:, n + t].contiguous().to(dev), V[:, n + t].contiguous().to(dev)
        pa, na, oa, ta = a.decode_step(kn, vn, qt, with_topk=True)
        pb, nb, ob, tb = b.decode_step(kn, vn, qt, with_topk=True)
        torch.cuda.synchronize()
        assert torch.equal(pa, pb) and torch.equal(na, nb) and torch.equal(ta, tb)
        assert torch.equal(oa, ob)
    # the standalone attention over caller page lists, and an insert
    oa2 = a.sparse_attn(qt, pa, na)
    ob2 = b.sparse_attn(qt, pb, nb)
    torch.cuda.synchronize()
    assert torch.equal(oa2, ob2) and torch.equal(oa2, oa)
    nt = a.layout()["n_tokens"]
    npg = int(a.view("npages").max())
    assert torch.equal(a.view("npages"), b.view("npages"))
    for name in ("codes", "loc"):
        assert torch.equal(a.view(name)[:, :nt], b.view(name)[:, :nt]), name
    for name in ("page_tokens", "page_len"):
        assert torch.equal(a.view(name)[:, :npg], b.view(name)[:, :npg]), name
    filled = b.view("page_tokens") >= 0
    for name in ("pool_k", "pool_v"):
        assert torch.equal(a.view(name).cpu()[filled.cpu()], b.view(name).cpu()[filled.cpu()]), name
    prm = oracle.Params(d=d, p=c["p"], k=c["k"], m=c["m"], L=c["L"], g=g,
                        gqa_max=c["gqa"] == "max")
    st = oracle.OracleStream(prm, _np(K[0, :n]), _np(V[0, :n]), _np(U), n_cap=n + steps + 2)
    for t in range(steps):
        st.insert(_np(K[0, n + t]), _np(V[0, n + t]))
    q_s = _np(qt[:g])
    r = st.query(q_s, literal=False)
    _check_index(a, st, 0, n + steps)
    _check_query(a, st, 0, r, pa, na, ta, oa[:g], q_s)



# ---------------------------------------------------------------- list delta-merge

def test_merge_lists(B):
    """ice_merge_lists folds the inserted entries into the sorted lists: the
    stored lists then equal the oracle's (which inserts in place) with no
    re-sort, n_build becomes n, and queries are unchanged; a second round of
    inserts and merge, and a merge with nothing to merge, likewise."""
    S, n, g, d, p, m, L, k = 2, 3000, 2, 128, 16, 4, 3, 128
    dev = torch.device("cuda")
    K, V, q, _ = _inputs(S, n + 120, d, g, 24, 401, "bf16")
    U = W.directions(m * L, d, 401, "bf16")
    idx = B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U.to(dev),
                  page_size=p, budget_k=k, m=m, L=L, gqa_group=g, capacity=n + 120)
    prm = oracle.Params(d=d, p=p, k=k, m=m, L=L, g=g)
    sts = [oracle.OracleStream(prm, _np(K[s, :n]), _np(V[s, :n]), _np(U), n_cap=n + 120)
           for s in range(S)]
    qd = q.to(dev)
    nt = n
    for rnd, cnt in enumerate((77, 43)):
        for t in range(nt, nt + cnt):
            idx.insert(K[:, t].contiguous().to(dev), V[:, t].contiguous().to(dev))
            for s in range(S):
                sts[s].insert(_np(K[s, t]), _np(V[s, t]))
        nt += cnt
        before = idx.query_pages(qd, with_topk=True)
        torch.cuda.synchronize()
        assert idx.layout()["n_build"] == nt - cnt
        idx.merge_lists()
        assert idx.layout()["n_build"] == nt
        for s in range(S):
            lc, li = _stored_lists(idx, s)
            np.testing.assert_array_equal(lc, sts[s].lcode[:, :nt])
            np.testing.assert_array_equal(li, sts[s].lid[:, :nt])
        after = idx.query_pages(qd, with_topk=True)
        torch.cuda.synchronize()
        for x, y in zip(before, after):
            assert torch.equal(x, y)
    idx.merge_lists()  # nothing to merge
    assert idx.layout()["n_build"] == nt


def test_merge_lists_tail_limit(B):
    """More than 8,192 entries inserted since the last merge: UNSUPPORTED, and
    the index is untouched."""
    S, n, d = 1, 100, 64
    dev = torch.device("cuda")
    K, V, _, _ = _inputs(S, n + 8193, d, 1, 8, 402, "bf16")
    U = W.directions(4, d, 402, "bf16").to(dev)
    idx = B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U, page_size=16,
                  budget_k=32, m=2, L=2, capacity=n + 8193)
    Kd, Vd = K.to(dev), V.to(dev)
    for t in range(n, n + 8193):
        idx.insert(Kd[:, t].contiguous(), Vd[:, t].contiguous())
    with pytest.raises(B.IceError) as e:
        idx.merge_lists()
    assert e.value.status == B.ICE_ERR_UNSUPPORTED
    assert idx.layout()["n_build"] == n



# ---------------------------------------------------------------- reuse steps

@pytest.mark.parametrize("r,gqa", [(1, "mean"), (3, "mean"), (3, "max")])
def test_reuse_schedule(B, r, gqa):
    """A decode loop that queries every r steps and reuses the last selection in
    between (ice_decode_step_reuse): every step's attention equals the oracle
    attending over the same pages after the same inserts, reuse steps equal
    ice_insert + ice_sparse_attn up to the fp32 rounding of the new token's
    logit (one kernel), and the index after the loop equals the oracle's."""
    S, n, g, d, p, m, L, k, steps = 2, 3000, 4, 128, 16, 4, 3, 128, 7
    dev = torch.device("cuda")
    K, V, _, _ = _inputs(S, n + steps, d, g, 24, 501, "bf16")
    U = W.directions(m * L, d, 501, "bf16").to(dev)
    mk = lambda: B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U,
                         page_size=p, budget_k=k, m=m, L=L, gqa_group=g, capacity=n + steps,
                         gqa_mode=gqa)
    a, b = mk(), mk()
    prm = oracle.Params(d=d, p=p, k=k, m=m, L=L, g=g, gqa_max=gqa == "max")
    sts = [oracle.OracleStream(prm, _np(K[s, :n]), _np(V[s, :n]), _np(U), n_cap=n + steps)
           for s in range(S)]
    gen = torch.Generator().manual_seed(41)
    pg = npg = None
    for t in range(steps):
        qt = torch.randn(S * g, d, generator=gen).to(torch.bfloat16).to(dev)
        kn, vn = K[:, n + t].contiguous().to(dev), V[:, n + t].contiguous().to(dev)
        if t % r == 0:
            pg, npg, out, _ = a.decode_step(kn, vn, qt)
            b.decode_step(kn, vn, qt)
            torch.cuda.synchronize()
            for s in range(S):
                sts[s].insert(_np(K[s, n + t]), _np(V[s, n + t]))
                r_o = sts[s].query(_np(qt[s * g:(s + 1) * g]))
                np.testing.assert_array_equal(pg[s, :int(npg[s])].cpu().numpy(), r_o["page_ids"],
                                              err_msg=f"pages, stream {s} step {t}")
        else:
            out = a.decode_step_reuse(kn, vn, qt, pg, npg)
            b.insert(kn, vn)
            ob = b.sparse_attn(qt, pg, npg)
            torch.cuda.synchronize()
            # one kernel: equal up to the fp32 rounding of the new token's logit
            assert float((out - ob).abs().max()) <= 1e-5
            for s in range(S):
                sts[s].insert(_np(K[s, n + t]), _np(V[s, n + t]))
        for s in range(S):
            ref = sts[s].attend(_np(qt[s * g:(s + 1) * g]), pg[s, :int(npg[s])].cpu().numpy())
            err = float(np.max(np.abs(out[s * g:(s + 1) * g].cpu().numpy() - ref)))
            assert err <= ATTN_TOL, (t, s, err)
    for s in range(S):
        _check_index(a, sts[s], s, n + steps)


@pytest.mark.parametrize("dtype,d,p", [("bf16", 128, 8), ("f32", 64, 16)])
def test_reuse_step_one_kernel(B, dtype, d, p):
    """The one-kernel reuse step (a budget of one attention block, pool in
    HBM) against ice_insert + ice_sparse_attn on a twin index, over 24 steps
    whose page lists hold the new token's own page (found on the twin), twice
    on some steps, and a fresh page on the steps where the token opens one:
    the index arrays equal the twin's bit for bit; the attention equals the
    twin's up to the fp32 rounding of the new token's logit (1e-5), and the
    oracle's within the attention tolerance."""
    S, n, g, m, L, k, steps = 2, 2000, 2, 4, 2, 8 * p, 24
    dev = torch.device("cuda")
    K, V, _, _ = _inputs(S, n + steps, d, g, 16, 601, dtype)
    U = W.directions(m * L, d, 601, dtype).to(dev)
    mk = lambda: B.Index(K[:, :n].contiguous().to(dev), V[:, :n].contiguous().to(dev), U,
                         page_size=p, budget_k=k, m=m, L=L, gqa_group=g, capacity=n + steps)
    a, b = mk(), mk()
    assert a.layout()["n_tokens"] == n
    prm = oracle.Params(d=d, p=p, k=k, m=m, L=L, g=g)
    sts = [oracle.OracleStream(prm, _np(K[s, :n]), _np(V[s, :n]), _np(U), n_cap=n + steps)
           for s in range(S)]
    gen = torch.Generator().manual_seed(43)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q0 = torch.randn(S * g, d, generator=gen).to(tdt).to(dev)
    pg, npg, _ = a.query_pages(q0)
    torch.cuda.synchronize()
    P = k // p
    fresh = 0
    for t in range(steps):
        qt = torch.randn(S * g, d, generator=gen).to(tdt).to(dev)
        kn, vn = K[:, n + t].contiguous().to(dev), V[:, n + t].contiguous().to(dev)
        b.insert(kn, vn)
        torch.cuda.synchronize()
        loc = b.view("loc")[:, n + t].cpu()
        newpg = (loc // p).to(torch.int32)
        fresh += int(((loc % p) == 0).sum())
        pl = pg.clone().cpu()
        for s in range(S):  # the token's page first; twice on odd steps
            pl[s, 0] = newpg[s]
            if t % 2:
                pl[s, P - 1] = newpg[s]
        pl = pl.to(dev)
        npl = torch.full((S,), P, dtype=torch.int32, device=dev)
        out = a.decode_step_reuse(kn, vn, qt, pl, npl)
        ob = b.sparse_attn(qt, pl, npl)
        torch.cuda.synchronize()
        err_twin = float((out - ob).abs().max())
        assert err_twin <= 1e-5, (t, err_twin)
        for s in range(S):
            sts[s].insert(_np(K[s, n + t]), _np(V[s, n + t]))
            ref = sts[s].attend(_np(qt[s * g:(s + 1) * g]), pl[s].cpu().numpy())
            err = float(np.max(np.abs(out[s * g:(s + 1) * g].cpu().numpy() - ref)))
            assert err <= ATTN_TOL, (t, s, err)
    assert fresh > 0  # some step opened a page that its list held
    for name in ("codes", "list_code", "list_id", "loc", "page_tokens", "page_len", "page_cell",
                 "npages", "cell_count"):
        assert torch.equal(a.view(name), b.view(name)), name
    for s in range(S):  # the pools on their valid slots (the rest was never written)
        npg_s = int(a.view("npages")[s])
        plen = a.view("page_len")[s, :npg_s].cpu()
        ka, kb = a.view("pool_k")[s, :npg_s].cpu(), b.view("pool_k")[s, :npg_s].cpu()
        va, vb = a.view("pool_v")[s, :npg_s].cpu(), b.view("pool_v")[s, :npg_s].cpu()
        for j in range(npg_s):
            ln = int(plen[j])
            assert torch.equal(ka[j, :ln], kb[j, :ln]) and torch.equal(va[j, :ln], vb[j, :ln])
    for s in range(S):
        _check_index(a, sts[s], s, n + steps)
