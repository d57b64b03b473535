"""The no-allocation build (ice_build_index_noalloc), called through the C ABI,
against the plain build (ice_build_index) on the same inputs: two builds in a
row, the second smaller than the first, so the second runs on the fixed
scratch array with the first build's contents still in it.  Every index array
and the query's pages, top-k and attention must be identical."""
import pytest
import torch

from sparse_attention_dci_amd import workloads as W

pytestmark = pytest.mark.gpu

ARRAYS = ("norm_c", "codes", "list_code", "list_id", "loc", "page_tokens", "page_len",
          "page_cell", "npages", "cell_count")


def _inputs(S, n, d, g, seed):
    Ks, Vs, qs = [], [], []
    for s in range(S):
        K, V, q, _ = W.stream(n, d, 24, g, seed * 100 + s, "bf16")
        Ks.append(K)
        Vs.append(V)
        qs.append(q)
    return torch.stack(Ks), torch.stack(Vs), torch.cat(qs)


@pytest.mark.parametrize("calls", [((8, 36864), (3, 9001))])
def test_noalloc_build_equals_scratch_build(calls):
    from sparse_attention_dci_amd import binding as B
    dev = torch.device("cuda")
    d, g, p, k, m, L = 128, 4, 16, 256, 8, 4
    for i, (S, n) in enumerate(calls):
        print(f"[case] noalloc build call {i}: S={S} n={n}", flush=True)
        K, V, q = _inputs(S, n, d, g, 400 + i)
        U = W.directions(m * L, d, 400 + i, "bf16").to(dev)
        Kd, Vd, qd = K.to(dev), V.to(dev), q.to(dev)
        kw = dict(page_size=p, budget_k=k, m=m, L=L, gqa_group=g, capacity=n + 4)
        a = B.Index(Kd, Vd, U, noalloc=True, **kw)
        b = B.Index(Kd, Vd, U, **kw)
        torch.cuda.synchronize()
        a.release_build_buffers()
        b.release_build_buffers()
        for name in ARRAYS:
            ta, tb = a.view(name), b.view(name)
            if name in ("list_code", "list_id"):
                ta, tb = ta[:, :, :n], tb[:, :, :n]
            elif name in ("codes", "loc"):
                ta, tb = ta[:, :n], tb[:, :n]
            assert torch.equal(ta, tb), name
        npg = a.view("npages").cpu()
        filled = a.view("page_tokens") >= 0
        for name in ("pool_k", "pool_v"):
            assert torch.equal(a.view(name)[filled], b.view(name)[filled]), name
        assert int(npg.max()) > 0
        pa, na, ta_ = a.query_pages(qd, with_topk=True)
        oa = a.sparse_attn(qd, pa, na)
        pb, nb, tb_ = b.query_pages(qd, with_topk=True)
        ob = b.sparse_attn(qd, pb, nb)
        torch.cuda.synchronize()
        assert torch.equal(pa, pb) and torch.equal(na, nb) and torch.equal(ta_, tb_)
        assert torch.equal(oa, ob)
        del a, b
