"""Plain CPU oracle for the IceCache decode hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library and never imports it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, no FMA contraction); this
module holds the ctypes bindings and a per-stream driver that runs the steps in
the order the IceCache pages give them:

1. index the keys into the DCI-tree at prefill (IceCache paper page, Figure 2
   caption, step (1)): transform, project, sorted lists, cells, pages;
2. at decode, P-DCI finds the top-k tokens for q (Figure 2, step (2); the blog
   page's technical-details section: one tree and one P-DCI search per head);
3. the pages holding those tokens are selected and every token in them joins
   sparse attention with q (Figure 2, step (3)).

Every step has a pin in ``tests/test_oracle_*.py`` that checks it against
something other than itself (closed forms, invariants, brute force).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

MAX_TREE_DEPTH = 13


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-shared",
             "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.ora_key_norm_sq.argtypes = [P, i64, i32, P]
        L.ora_norm_bound.argtypes = [P, i64]
        L.ora_norm_bound.restype = f32
        L.ora_transform.argtypes = [P, i64, i32, f32, P]
        L.ora_project.argtypes = [P, i64, i32, P, i32, f32, i32, P, P]
        L.ora_sort_list.argtypes = [P, i64, i32, i32, P, P]
        L.ora_list_insert.argtypes = [P, P, i64, ctypes.c_int32, ctypes.c_int32]
        L.ora_tree.argtypes = [P, i64, i32, i32, P, P, P, P, P, i64]
        L.ora_tree.restype = i64
        L.ora_tree_append.argtypes = [i64, ctypes.c_uint32, i32, i64, P, P, P, P, P, i64]
        L.ora_tree_append.restype = i64
        L.ora_query_prep.argtypes = [P, i32, i32, P, i32, P, P]
        L.ora_pdci_literal.argtypes = [P, P, i64, i32, P, i64, i64, P, P]
        L.ora_pdci_literal.restype = i64
        L.ora_pdci_closed.argtypes = [P, i64, i32, i32, i32, P, i64, i64, P, P]
        L.ora_pdci_closed.restype = i64
        L.ora_dot_blocked.argtypes = [P, P, i32]
        L.ora_dot_blocked.restype = ctypes.c_double
        L.ora_score.argtypes = [P, i32, P, i64]
        L.ora_score.restype = ctypes.c_double
        L.ora_rerank.argtypes = [P, i32, P, P, i64, P, P]
        L.ora_rerank_max.argtypes = [P, i32, P, i32, P, i64, P, P]
        L.ora_select_pages.argtypes = [P, i64, P, i64, P]
        L.ora_select_pages.restype = i64
        L.ora_attention.argtypes = [P, i32, i32, P, P, i32, P, i64, P, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------- step wrappers

def key_norm_sq(K) -> np.ndarray:
    K = _f32(K)
    out = np.empty(K.shape[0], np.float64)
    lib().ora_key_norm_sq(_p(K), K.shape[0], K.shape[1], _p(out))
    return out


def norm_bound(K) -> float:
    nsq = key_norm_sq(K)
    return float(lib().ora_norm_bound(_p(nsq), nsq.shape[0]))


def transform(K, c: float) -> np.ndarray:
    K = _f32(K)
    out = np.empty((K.shape[0], K.shape[1] + 1), np.float64)
    lib().ora_transform(_p(K), K.shape[0], K.shape[1], c, _p(out))
    return out


def project(K, U, c: float, D: int):
    """codes [n][mL] int32 (2^29 fixed point) and cells [n] uint32."""
    K, U = _f32(K), _f32(U)
    n, d = K.shape
    mL = U.shape[0]
    assert U.shape[1] == d + 1
    codes = np.empty((n, mL), np.int32)
    cell = np.empty(n, np.uint32)
    lib().ora_project(_p(K), n, d, _p(U), mL, c, D, _p(codes), _p(cell))
    return codes, cell


def sort_list(codes: np.ndarray, t: int):
    codes = np.ascontiguousarray(codes, np.int32)
    n, mL = codes.shape
    oc = np.empty(n, np.int32)
    oi = np.empty(n, np.int32)
    lib().ora_sort_list(_p(codes), n, mL, t, _p(oc), _p(oi))
    return oc, oi


def query_prep(q, U):
    """q: [g][d].  Returns (qkv [d] fp32, qcode [mL] int32)."""
    q, U = _f32(q), _f32(U)
    g, d = q.shape
    mL = U.shape[0]
    qkv = np.empty(d, np.float32)
    qcode = np.empty(mL, np.int32)
    lib().ora_query_prep(_p(q), g, d, _p(U), mL, _p(qkv), _p(qcode))
    return qkv, qcode


def pdci_literal(lcode, lid, m: int, qcode_l, k0: int, k1: int = 0):
    """One composite: lcode/lid are its m sorted lists, [m][n]."""
    lcode = np.ascontiguousarray(lcode, np.int32)
    lid = np.ascontiguousarray(lid, np.int32)
    qcode_l = np.ascontiguousarray(qcode_l, np.int32)
    n = lcode.shape[1]
    S = np.empty(max(k0, 1), np.int32)
    v = ctypes.c_int64(0)
    ns = lib().ora_pdci_literal(_p(lcode), _p(lid), n, m, _p(qcode_l), k0, k1, _p(S),
                                ctypes.byref(v))
    return S[:ns].copy(), int(v.value)


def pdci_closed(codes, m: int, l: int, qcode, k0: int, k1: int = 0):
    codes = np.ascontiguousarray(codes, np.int32)
    qcode = np.ascontiguousarray(qcode, np.int32)
    n, mL = codes.shape
    S = np.empty(max(k0, 1), np.int32)
    v = ctypes.c_int64(0)
    ns = lib().ora_pdci_closed(_p(codes), n, mL, m, l, _p(qcode), k0, k1, _p(S),
                               ctypes.byref(v))
    return S[:ns].copy(), int(v.value)


def dot_blocked(a, b) -> float:
    """The query side's fp64 dot product in its fixed blocked order."""
    a, b = _f32(a), _f32(b)
    assert a.shape == b.shape and a.ndim == 1
    return float(lib().ora_dot_blocked(_p(a), _p(b), a.shape[0]))


def score(K, qkv, tok: int) -> float:
    K, qkv = _f32(K), _f32(qkv)
    return float(lib().ora_score(_p(K), K.shape[1], _p(qkv), tok))


def rerank(K, qkv, C):
    K, qkv = _f32(K), _f32(qkv)
    C = np.ascontiguousarray(C, np.int32)
    ranked = np.empty(max(len(C), 1), np.int32)
    scores = np.empty(max(len(C), 1), np.float64)
    lib().ora_rerank(_p(K), K.shape[1], _p(qkv), _p(C), len(C), _p(ranked), _p(scores))
    return ranked[:len(C)].copy(), scores[:len(C)].copy()


def rerank_max(K, Q, C):
    """GQA max reading: score_i = max over the heads of <q_h, k_i>."""
    K, Q = _f32(K), _f32(Q)
    C = np.ascontiguousarray(C, np.int32)
    ranked = np.empty(max(len(C), 1), np.int32)
    scores = np.empty(max(len(C), 1), np.float64)
    lib().ora_rerank_max(_p(K), K.shape[1], _p(Q), Q.shape[0], _p(C), len(C), _p(ranked),
                         _p(scores))
    return ranked[:len(C)].copy(), scores[:len(C)].copy()


def select_pages(ranked, page_of, P: int):
    ranked = np.ascontiguousarray(ranked, np.int32)
    page_of = np.ascontiguousarray(page_of, np.int32)
    out = np.empty(max(P, 1), np.int32)
    n = lib().ora_select_pages(_p(ranked), len(ranked), _p(page_of), P, _p(out))
    return out[:n].copy()


def attention(q, poolK, poolV, p: int, page_ids, page_len):
    """q [g][d]; pool [Pcap][p][d].  Returns out [g][d] fp64."""
    q, poolK, poolV = _f32(q), _f32(poolK), _f32(poolV)
    g, d = q.shape
    page_ids = np.ascontiguousarray(page_ids, np.int32)
    page_len = np.ascontiguousarray(page_len, np.int32)
    out = np.empty((g, d), np.float64)
    lib().ora_attention(_p(q), g, d, _p(poolK), _p(poolV), p, _p(page_ids), len(page_ids),
                        _p(page_len), _p(out))
    return out


# ---------------------------------------------------------------- readings

def tree_depth(n_build: int, p: int, mL: int) -> int:
    """READING: D = round(log2(n / (4p))) clamped to [1, min(mL, 13)], i.e. about
    four pages per cell at build.  Evaluated exactly in integers:
    round(log2 x) >= t  <=>  2^(2t-1) <= x^2."""
    t = 0
    for cand in range(1, 64):
        if (1 << (2 * cand - 1)) * (4 * p) ** 2 <= n_build * n_build:
            t = cand
    return max(1, min(t, mL, MAX_TREE_DEPTH))


def page_capacity(n_cap: int, p: int, D: int) -> int:
    """Each cell has at most one partial page: ceil(n/p) + 2^D pages suffice."""
    return -(-n_cap // p) + (1 << D)


@dataclass
class Params:
    d: int = 128
    p: int = 16           # page size
    k: int = 256          # token budget
    m: int = 8            # simple indices per composite
    L: int = 4            # composites
    g: int = 1            # query heads per KV head
    k0: int = 0           # candidates per composite (0 -> k)
    k1: int = 0           # visit budget per composite (0 -> unbounded)
    D: int = 0            # tree depth (0 -> derived at build)
    c: float = 0.0        # key-norm bound (0 -> derived at build)
    gqa_max: bool = False  # GQA reading: False = the heads' mean, True = per-head walks, max score

    @property
    def mL(self):
        return self.m * self.L

    @property
    def P(self):
        return self.k // self.p

    @property
    def k0_eff(self):
        return self.k0 if self.k0 > 0 else self.k


class OracleStream:
    """The whole index of one stream plus its queries, in plain steps.

    K, V: [n][d] float32 (bf16 keys are passed as their exact fp32 values);
    U: [mL][d+1] float32 directions (drawn by the caller, exactly as the GPU
    path receives them).
    """

    def __init__(self, prm: Params, K, V, U, n_cap: int | None = None):
        self.prm = prm
        K, V, U = _f32(K), _f32(V), _f32(U)
        n, d = K.shape
        assert d == prm.d and U.shape == (prm.mL, d + 1)
        self.U = U
        self.n = n
        self.n_cap = n_cap if n_cap is not None else n
        self.c = prm.c if prm.c > 0 else norm_bound(K)
        self.D = prm.D if prm.D > 0 else tree_depth(n, prm.p, prm.mL)
        self.Pcap = page_capacity(self.n_cap, prm.p, self.D)
        self.K = np.zeros((self.n_cap, d), np.float32)
        self.V = np.zeros((self.n_cap, d), np.float32)
        self.K[:n], self.V[:n] = K, V
        codes, cell = project(K, U, self.c, self.D)
        self.codes = np.zeros((self.n_cap, prm.mL), np.int32)
        self.cell = np.zeros(self.n_cap, np.uint32)
        self.codes[:n], self.cell[:n] = codes, cell
        # one sorted list per direction (published DCI index)
        self.lcode = np.zeros((prm.mL, self.n_cap), np.int32)
        self.lid = np.zeros((prm.mL, self.n_cap), np.int32)
        for t in range(prm.mL):
            self.lcode[t, :n], self.lid[t, :n] = sort_list(codes, t)
        # the lists as the build sorted them (before any insert), for tests that
        # check a stored build order without re-sorting it
        self.n_build = n
        self.lcode_build = self.lcode[:, :n].copy()
        self.lid_build = self.lid[:, :n].copy()
        # DCI-tree leaves as pages
        p = prm.p
        self.page_of = np.full(self.n_cap, -1, np.int32)
        self.slot_of = np.full(self.n_cap, -1, np.int32)
        self.page_tokens = np.empty((self.Pcap, p), np.int32)
        self.page_len = np.empty(self.Pcap, np.int32)
        self.page_cell = np.empty(self.Pcap, np.int32)
        cellc = np.ascontiguousarray(cell)
        self.npages = int(lib().ora_tree(_p(cellc), n, self.D, p, _p(self.page_of),
                                         _p(self.slot_of), _p(self.page_tokens),
                                         _p(self.page_len), _p(self.page_cell), self.Pcap))
        assert self.npages >= 0

    # ---------------------------------------------------------------- update
    def insert(self, k, v):
        """Append one token (blog page: no rebuild when a token arrives)."""
        prm = self.prm
        assert self.n < self.n_cap, "capacity exhausted"
        k = _f32(k).reshape(1, prm.d)
        codes, cell = project(k, self.U, self.c, self.D)
        i = self.n
        self.K[i], self.V[i] = k[0], _f32(v)
        self.codes[i], self.cell[i] = codes[0], cell[0]
        for t in range(prm.mL):
            lc = self.lcode[t]
            li = self.lid[t]
            lib().ora_list_insert(_p(lc), _p(li), i, int(codes[0, t]), i)
        self.npages = int(lib().ora_tree_append(
            i, int(cell[0]), prm.p, self.npages, _p(self.page_of), _p(self.slot_of),
            _p(self.page_tokens), _p(self.page_len), _p(self.page_cell), self.Pcap))
        assert self.npages >= 0
        self.n += 1

    # ---------------------------------------------------------------- views
    def pool(self):
        """Page pool [Pcap][p][d] for K and V (zero where a slot is empty)."""
        d, p = self.prm.d, self.prm.p
        pk = np.zeros((self.Pcap, p, d), np.float32)
        pv = np.zeros((self.Pcap, p, d), np.float32)
        tok = self.page_tokens
        ok = tok >= 0
        pk[ok] = self.K[tok[ok]]
        pv[ok] = self.V[tok[ok]]
        return pk, pv

    # ---------------------------------------------------------------- query
    def _walks(self, qcode, literal):
        """P-DCI over every composite for one set of query codes."""
        prm, n = self.prm, self.n
        S, visits = [], []
        for l in range(prm.L):
            if literal:
                sl = slice(l * prm.m, (l + 1) * prm.m)
                s, v = pdci_literal(self.lcode[sl, :n], self.lid[sl, :n], prm.m,
                                    qcode[sl], prm.k0_eff, prm.k1)
            else:
                s, v = pdci_closed(self.codes[:n], prm.m, l, qcode, prm.k0_eff, prm.k1)
            S.append(s)
            visits.append(v)
        return S, visits

    def query(self, q, literal: bool = True):
        """q: [g][d].  Returns a dict with every intermediate of the query.
        With gqa_max, S / visits / qcode hold one entry per (head, composite),
        head-major, and qkv is the heads themselves [g][d]."""
        prm = self.prm
        n = self.n
        if prm.gqa_max:
            q = _f32(q)
            S, visits, qcs, qks = [], [], [], []
            for h in range(q.shape[0]):
                qk, qc = query_prep(q[h:h + 1], self.U)
                s_h, v_h = self._walks(qc, literal)
                S += s_h
                visits += v_h
                qcs.append(qc)
                qks.append(qk)
            qkv, qcode = np.stack(qks), np.concatenate(qcs)
        else:
            qkv, qcode = query_prep(q, self.U)
            S, visits = self._walks(qcode, literal)
        C = np.unique(np.concatenate(S)) if S else np.empty(0, np.int32)
        C = C.astype(np.int32)
        if prm.gqa_max:
            ranked, scores = rerank_max(self.K[:n], qkv, C)
        else:
            ranked, scores = rerank(self.K[:n], qkv, C)
        topk = ranked[:prm.k]
        page_ids = select_pages(ranked, self.page_of[:n], prm.P)
        return dict(qkv=qkv, qcode=qcode, S=S, visits=visits, C=C, ranked=ranked,
                    scores=scores, topk=topk, page_ids=page_ids)

    def decode_reuse(self, k, v, q, page_ids):
        """READING of the pages' "IceCache (reuse)" variant (named with its
        accuracy only): a decode step that reuses an earlier step's page
        selection inserts its token, then attends over those pages."""
        self.insert(k, v)
        return self.attend(q, page_ids)

    def attend(self, q, page_ids):
        pk, pv = self.pool()
        return attention(q, pk, pv, self.prm.p, page_ids, self.page_len)
