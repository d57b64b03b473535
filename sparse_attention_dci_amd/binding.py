"""ctypes binding of libice.so (include/ice.h), argument marshalling only.

Torch supplies device memory and streams; every step of the hot path runs in
the library's HIP kernels.  There is no fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libice.so")

ICE_OK, ICE_ERR_INVALID_ARG, ICE_ERR_CAPACITY, ICE_ERR_UNSUPPORTED, ICE_ERR_WORKSPACE, \
    ICE_ERR_HIP, ICE_ERR_SCRATCH_LIMIT = 0, -1, -2, -3, -4, -5, -6
NOALLOC_SCRATCH_BYTES = 128 << 20  # ICE_NOALLOC_SCRATCH_BYTES
ICE_F32, ICE_BF16 = 0, 1
ICE_GQA_MEAN, ICE_GQA_MAX = 0, 1
TIMED_KERNELS = 9


class IceParams(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("budget_k", ctypes.c_int32), ("m", ctypes.c_int32), ("L", ctypes.c_int32),
                ("gqa_group", ctypes.c_int32), ("k0", ctypes.c_int32), ("k1", ctypes.c_int64),
                ("tree_depth", ctypes.c_int32), ("c", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("gqa_mode", ctypes.c_int32),
                ("offload", ctypes.c_int32)]


_LAYOUT_I64_HEAD = ["n_streams", "n_tokens", "n_build", "capacity_tokens", "page_capacity",
                    "n_cells"]
_LAYOUT_I32 = ["tree_depth", "mL", "k0", "elem_bytes", "Lq", "Gq", "offload"]
_LAYOUT_OFFS = ["norm_c", "codes", "list_code", "list_id", "loc", "page_tokens", "page_len",
                "page_cell", "npages", "cell_count", "pool_k", "pool_v", "qcode", "cand",
                "cand_count"]


class IceLayout(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_int64) for n in _LAYOUT_I64_HEAD]
                + [(n, ctypes.c_int32) for n in _LAYOUT_I32]
                + [(n, ctypes.c_int64) for n in _LAYOUT_OFFS]
                + [("workspace_bytes", ctypes.c_int64)])


class IceError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib().ice_status_string(status).decode()} ({status})")


_lib = None


def lib():
    """Load libice.so; raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "or python sparse_attention_dci_amd/build_lib.py")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        PP = ctypes.POINTER(IceParams)
        L.ice_workspace_bytes.argtypes = [PP, i32, i64, i64]
        L.ice_workspace_bytes.restype = ctypes.c_size_t
        L.ice_build_scratch_bytes.argtypes = [PP, i32, i64]
        L.ice_build_scratch_bytes.restype = ctypes.c_size_t
        L.ice_build_index.argtypes = [PP, i32, i64, i64, P, P, P, P, ctypes.c_size_t, P,
                                      ctypes.c_size_t, P, ctypes.POINTER(P)]
        L.ice_build_index.restype = ctypes.c_int
        L.ice_build_index_noalloc.argtypes = [PP, i32, i64, i64, P, P, P, P, ctypes.c_size_t,
                                              P, ctypes.POINTER(P)]
        L.ice_build_index_noalloc.restype = ctypes.c_int
        L.ice_host_pool_bytes.argtypes = [PP, i32, i64, i64]
        L.ice_host_pool_bytes.restype = ctypes.c_size_t
        L.ice_build_index_offload.argtypes = [PP, i32, i64, i64, P, P, P, P, ctypes.c_size_t, P,
                                              ctypes.c_size_t, P, ctypes.c_size_t, P,
                                              ctypes.POINTER(P)]
        L.ice_build_index_offload.restype = ctypes.c_int
        L.ice_merge_scratch_bytes.argtypes = [P]
        L.ice_merge_scratch_bytes.restype = ctypes.c_size_t
        L.ice_merge_lists.argtypes = [P, P, ctypes.c_size_t, P]
        L.ice_merge_lists.restype = ctypes.c_int
        L.ice_insert.argtypes = [P, P, P, P]
        L.ice_insert.restype = ctypes.c_int
        L.ice_query_pages.argtypes = [P, P, P, P, P, P, P]
        L.ice_query_pages.restype = ctypes.c_int
        L.ice_sparse_attn.argtypes = [P, P, P, P, P, P]
        L.ice_sparse_attn.restype = ctypes.c_int
        L.ice_decode_step.argtypes = [P, P, P, P, P, P, P, P, P, P]
        L.ice_decode_step.restype = ctypes.c_int
        L.ice_decode_step_reuse.argtypes = [P, P, P, P, P, P, P, P]
        L.ice_decode_step_reuse.restype = ctypes.c_int
        L.ice_destroy_index.argtypes = [P]
        L.ice_destroy_index.restype = None
        L.ice_status_string.argtypes = [ctypes.c_int]
        L.ice_status_string.restype = ctypes.c_char_p
        L.ice_index_layout.argtypes = [P, ctypes.POINTER(IceLayout)]
        L.ice_index_layout.restype = ctypes.c_int
        L.ice_timing_enable.argtypes = [P, ctypes.c_int]
        L.ice_timing_enable.restype = ctypes.c_int
        L.ice_timing_read.argtypes = [P, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_int64)]
        L.ice_timing_read.restype = ctypes.c_int
        L.ice_timing_name.argtypes = [ctypes.c_int]
        L.ice_timing_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


def make_params(d, page_size, budget_k, m, L, gqa_group=1, k0=0, k1=0, tree_depth=0, c=0.0,
                dtype=torch.bfloat16, gqa_mode="mean", offload=False) -> IceParams:
    dt = {torch.float32: ICE_F32, torch.bfloat16: ICE_BF16}[dtype]
    gm = {"mean": ICE_GQA_MEAN, "max": ICE_GQA_MAX}[gqa_mode]
    mode = 2 if offload == "values" else (1 if offload else 0)
    return IceParams(d, page_size, budget_k, m, L, gqa_group, k0, k1, tree_depth, c, dt, gm, mode)


STATS_MAX_L = 32
STATS_WORDS = STATS_MAX_L + 2  # int64 words of one ice_query_stats


def stats_tensor(S: int, device) -> torch.Tensor:
    """Device buffer for S ice_query_stats records ([S][34] int64)."""
    return torch.zeros(S, STATS_WORDS, dtype=torch.int64, device=device)


def parse_stats(t: torch.Tensor, L: int) -> list:
    """ice_query_stats records ([S][34] int64) as dicts."""
    a = t.cpu()
    out = []
    for s in range(a.shape[0]):
        tail = a[s, STATS_MAX_L:].contiguous().view(torch.int32).tolist()
        out.append({"visits": a[s, :L].tolist(), "n_cand": tail[0], "n_pages": tail[1],
                    "n_tokens": tail[2]})
    return out


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status, what):
    if status != ICE_OK:
        raise IceError(status, what)


def _dev_tensor(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    return t


class Index:
    """One IceCache index over S streams (KV heads), resident in a workspace tensor.

    K, V: [S][n][d] device tensors (bf16 or fp32); dirs: [m*L][d+1] of the same
    dtype.  The workspace and, during the build, a scratch tensor are allocated
    here with torch; the library itself never allocates.
    """

    def __init__(self, K, V, dirs, *, page_size, budget_k, m, L, gqa_group=1, k0=0, k1=0,
                 tree_depth=0, c=0.0, capacity=None, stream=None, noalloc=False,
                 gqa_mode="mean", offload=False):
        """offload: keep the page pool in a pinned host tensor (self.host_pool)
        instead of the workspace (ice_build_index_offload); "values": only its
        value pages there, the key pages in the workspace."""
        _dev_tensor(K, "K", ndim=3)
        _dev_tensor(V, "V", K.dtype, 3)
        _dev_tensor(dirs, "dirs", K.dtype, 2)
        S, n, d = K.shape
        if V.shape != K.shape:
            raise ValueError("K and V shapes differ")
        self.S, self.d = S, d
        self.dtype = K.dtype
        self.device = K.device
        self.capacity = int(capacity if capacity is not None else n)
        self.prm = make_params(d, page_size, budget_k, m, L, gqa_group, k0, k1, tree_depth, c,
                               K.dtype, gqa_mode, offload)
        L_ = lib()
        ws = L_.ice_workspace_bytes(ctypes.byref(self.prm), S, n, self.capacity)
        if ws == 0:
            # let the build report which argument is wrong
            ws = 256
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=K.device)
        h = ctypes.c_void_p()
        st = _stream(stream)
        self.host_pool = None
        if offload:  # the page pool in pinned host memory
            hb = L_.ice_host_pool_bytes(ctypes.byref(self.prm), S, n, self.capacity) or 256
            self.host_pool = torch.empty(hb, dtype=torch.uint8, pin_memory=True)
            sb = L_.ice_build_scratch_bytes(ctypes.byref(self.prm), S, n) or 256
            scratch = torch.empty(sb, dtype=torch.uint8, device=K.device)
            _check(L_.ice_build_index_offload(ctypes.byref(self.prm), S, n, self.capacity,
                                              _ptr(K), _ptr(V), _ptr(dirs), _ptr(self.workspace),
                                              ws, _ptr(scratch), sb, _ptr(self.host_pool), hb, st,
                                              ctypes.byref(h)), "ice_build_index_offload")
        elif noalloc:  # the library's fixed build scratch (ice_build_index_noalloc)
            scratch = None
            _check(L_.ice_build_index_noalloc(ctypes.byref(self.prm), S, n, self.capacity,
                                              _ptr(K), _ptr(V), _ptr(dirs), _ptr(self.workspace),
                                              ws, st, ctypes.byref(h)),
                   "ice_build_index_noalloc")
        else:
            sb = L_.ice_build_scratch_bytes(ctypes.byref(self.prm), S, n) or 256
            scratch = torch.empty(sb, dtype=torch.uint8, device=K.device)
            _check(L_.ice_build_index(ctypes.byref(self.prm), S, n, self.capacity, _ptr(K),
                                      _ptr(V), _ptr(dirs), _ptr(self.workspace), ws,
                                      _ptr(scratch), sb, st, ctypes.byref(h)), "ice_build_index")
        self._h = h
        # keep the scratch (and the build inputs) alive until the build has run
        self._pending = (scratch, K, V, dirs)
        self.P = budget_k // page_size
        self.k = budget_k
        self.g = gqa_group

    def release_build_buffers(self):
        """Drop the build scratch once the caller has synchronised the stream."""
        self._pending = None

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.ice_destroy_index(h)
            self._h = None

    # ------------------------------------------------------------ calls
    def insert(self, k_new, v_new, stream=None):
        _dev_tensor(k_new, "k_new", self.dtype, 2)
        _dev_tensor(v_new, "v_new", self.dtype, 2)
        if k_new.shape != (self.S, self.d) or v_new.shape != (self.S, self.d):
            raise ValueError("k_new, v_new must be [S][d]")
        _check(lib().ice_insert(self._h, _ptr(k_new), _ptr(v_new), _stream(stream)), "ice_insert")

    def merge_lists(self, stream=None):
        """Fold the inserted list entries into the sorted lists (ice_merge_lists);
        the scratch is freed when the call returns (after a synchronisation)."""
        nb = lib().ice_merge_scratch_bytes(self._h)
        scratch = torch.empty(nb, dtype=torch.uint8, device=self.device)
        _check(lib().ice_merge_lists(self._h, _ptr(scratch), nb, _stream(stream)),
               "ice_merge_lists")
        torch.cuda.synchronize(self.device)  # the scratch lives until the merge has run

    def query_pages(self, q, with_topk=False, page_ids=None, n_pages=None, topk=None,
                    stats=None, stream=None):
        """stats: an optional stats_tensor(S) that receives the query statistics."""
        _dev_tensor(q, "q", self.dtype, 2)
        if q.shape != (self.S * self.g, self.d):
            raise ValueError("q must be [S*g][d]")
        dev = self.device
        page_ids = page_ids if page_ids is not None else torch.empty(
            self.S, self.P, dtype=torch.int32, device=dev)
        n_pages = n_pages if n_pages is not None else torch.empty(self.S, dtype=torch.int32,
                                                                  device=dev)
        if with_topk and topk is None:
            topk = torch.empty(self.S, self.k, dtype=torch.int32, device=dev)
        if stats is not None:
            _dev_tensor(stats, "stats", torch.int64, 2)
            if stats.shape != (self.S, STATS_WORDS):
                raise ValueError("stats must be stats_tensor(S)")
        _check(lib().ice_query_pages(self._h, _ptr(q), _ptr(page_ids), _ptr(n_pages),
                                     _ptr(topk) if with_topk else None, _ptr(stats),
                                     _stream(stream)),
               "ice_query_pages")
        return page_ids, n_pages, (topk if with_topk else None)

    def sparse_attn(self, q, page_ids, n_pages, out=None, stream=None):
        _dev_tensor(q, "q", self.dtype, 2)
        _dev_tensor(page_ids, "page_ids", torch.int32, 2)
        _dev_tensor(n_pages, "n_pages", torch.int32, 1)
        out = out if out is not None else torch.empty(self.S * self.g, self.d,
                                                      dtype=torch.float32, device=self.device)
        _check(lib().ice_sparse_attn(self._h, _ptr(q), _ptr(page_ids), _ptr(n_pages), _ptr(out),
                                     _stream(stream)), "ice_sparse_attn")
        return out

    def decode_step(self, k_new, v_new, q, page_ids=None, n_pages=None, out=None,
                    with_topk=False, topk=None, stats=None, stream=None):
        """insert(k_new, v_new); query_pages(q); sparse_attn(q, ...) in one call."""
        for t, nm in ((k_new, "k_new"), (v_new, "v_new"), (q, "q")):
            _dev_tensor(t, nm, self.dtype, 2)
        if k_new.shape != (self.S, self.d) or v_new.shape != (self.S, self.d):
            raise ValueError("k_new, v_new must be [S][d]")
        if q.shape != (self.S * self.g, self.d):
            raise ValueError("q must be [S*g][d]")
        dev = self.device
        page_ids = page_ids if page_ids is not None else torch.empty(
            self.S, self.P, dtype=torch.int32, device=dev)
        n_pages = n_pages if n_pages is not None else torch.empty(self.S, dtype=torch.int32,
                                                                  device=dev)
        out = out if out is not None else torch.empty(self.S * self.g, self.d,
                                                      dtype=torch.float32, device=dev)
        if with_topk and topk is None:
            topk = torch.empty(self.S, self.k, dtype=torch.int32, device=dev)
        if stats is not None:
            _dev_tensor(stats, "stats", torch.int64, 2)
            if stats.shape != (self.S, STATS_WORDS):
                raise ValueError("stats must be stats_tensor(S)")
        _check(lib().ice_decode_step(self._h, _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(page_ids),
                                     _ptr(n_pages), _ptr(topk) if with_topk else None, _ptr(out),
                                     _ptr(stats), _stream(stream)), "ice_decode_step")
        return page_ids, n_pages, out, (topk if with_topk else None)

    def decode_step_reuse(self, k_new, v_new, q, page_ids, n_pages, out=None, stream=None):
        """insert(k_new, v_new); sparse_attn(q, page_ids, n_pages): a step that
        reuses an earlier selection (ice_decode_step_reuse)."""
        for t, nm in ((k_new, "k_new"), (v_new, "v_new"), (q, "q")):
            _dev_tensor(t, nm, self.dtype, 2)
        _dev_tensor(page_ids, "page_ids", torch.int32, 2)
        _dev_tensor(n_pages, "n_pages", torch.int32, 1)
        if k_new.shape != (self.S, self.d) or v_new.shape != (self.S, self.d):
            raise ValueError("k_new, v_new must be [S][d]")
        if q.shape != (self.S * self.g, self.d):
            raise ValueError("q must be [S*g][d]")
        out = out if out is not None else torch.empty(self.S * self.g, self.d,
                                                      dtype=torch.float32, device=self.device)
        _check(lib().ice_decode_step_reuse(self._h, _ptr(k_new), _ptr(v_new), _ptr(q),
                                           _ptr(page_ids), _ptr(n_pages), _ptr(out),
                                           _stream(stream)), "ice_decode_step_reuse")
        return out

    # ------------------------------------------------------------ timing
    def timing(self, enable: bool):
        _check(lib().ice_timing_enable(self._h, 1 if enable else 0), "ice_timing_enable")

    def timing_read(self) -> dict:
        """{kernel: (total_ms, launches)} since the last read; waits for the events."""
        n = TIMED_KERNELS
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        _check(lib().ice_timing_read(self._h, ms, cnt), "ice_timing_read")
        return {lib().ice_timing_name(k).decode(): (ms[k], cnt[k]) for k in range(n)}

    # ------------------------------------------------------------ inspection
    def layout(self) -> dict:
        y = IceLayout()
        _check(lib().ice_index_layout(self._h, ctypes.byref(y)), "ice_index_layout")
        return {f: getattr(y, f) for f, _ in IceLayout._fields_}

    def view(self, name: str):
        """A tensor view of one index array inside the workspace (see ice_index_layout)."""
        y = self.layout()
        S, ncap, pcap = y["n_streams"], y["capacity_tokens"], y["page_capacity"]
        mL, p, d = y["mL"], self.prm.page_size, self.d
        Lq, Gq = y["Lq"], y["Gq"]
        shapes = {
            "norm_c": (torch.float32, (S,)),
            "codes": (torch.int32, (S, (ncap + 63) // 64, mL, 64)),
            "list_code": (torch.int32, (S, mL, ncap)),
            "list_id": (torch.int32, (S, mL, ncap)),
            "loc": (torch.int32, (S, ncap)),
            "page_tokens": (torch.int32, (S, pcap, p)),
            "page_len": (torch.int32, (S, pcap)),
            "page_cell": (torch.int32, (S, pcap)),
            "npages": (torch.int32, (S,)),
            "cell_count": (torch.int32, (S, y["n_cells"])),
            "pool_k": (self.dtype, (S, pcap, p, d)),
            "pool_v": (self.dtype, (S, pcap, d, p)),
            "qcode": (torch.int32, (S, Gq * mL)),
            "cand": (torch.int32, (S, Lq, y["k0"])),
            "cand_count": (torch.int32, (S, Lq)),
        }
        dt, shape = shapes[name]
        off = y[name]
        nbytes = torch.empty((), dtype=dt).element_size()
        count = 1
        for s_ in shape:
            count *= s_
        base = self.workspace
        if y["offload"] and (name == "pool_v" or (name == "pool_k" and y["offload"] == 1)):
            base = self.host_pool  # offsets into the host pool
        raw = base[off:off + count * nbytes]
        t = raw.view(dt).view(shape)
        if name == "codes":  # tiles of 64 tokens -> [S][ncap][mL] (a copy)
            t = t.permute(0, 1, 3, 2).reshape(S, -1, mL)[:, :ncap]
        if name == "pool_v":  # element-major pages -> [S][pcap][p][d] (a view)
            t = t.permute(0, 1, 3, 2)
        return t
