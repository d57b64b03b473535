"""Decode-step benchmark of the IceCache hot path on one MI355X.

Default workload: one Llama-3.1-8B-shaped layer at 36,864 tokens of context
(8 KV heads, 32 query heads, head_dim 128, bf16 KV, page 16, budget 256
tokens, DCI m=8, L=4), synthetic mixture keys.  A decode step is the whole
decode-time path on that layer, one ice_decode_step call: insert the new
token's key/value into every head's index, query (P-DCI candidates, exact
rerank, page selection) and paged sparse attention.  The prefill build of the
index is timed separately (build_ms).

Several copies of the layer ("layers" with their own inputs) are built and the
steps rotate over them, so each step finds its index cold in the 256 MB
last-level cache, as in a real multi-layer decode.

--workload picks another configuration (the 32-layer decode, the 131k needle
batch); --copy-calibration times a plain device copy of known size instead
(the reference for the HBM byte counters); --write-traffic turns four
rocprofv3 counter runs (FETCH_SIZE and WRITE_SIZE of the decode kernels, the
same two of the copy) into profiles/traffic.json (no GPU needed).

Prints one JSON line (the last line of stdout).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "llama8b_layer_36k"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_attention_dci_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".cpp", ".h")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, kernel: str, visits: float, n_cand: float, attended: float,
                      fused: bool = True) -> float:
    """Bytes the decode path has to move per launch of `kernel` for one layer
    (S streams): the per-unit figures times the units one launch processes.
    `visits` is the mean sum over composites of the list entries a stream's
    P-DCI walk visits (sum_l V_l), `n_cand` the mean union size |C|,
    `attended` the mean tokens attended per stream, all measured (the query
    statistics of a decode step on the timed layers).

    qscan     the walk: 4 bytes per visited list entry (4 * sum_l V_l); the
              query prep: the g heads in (g*d*elem), the query codes and q_kv
              out (4*mL + 4*d), the fp32 directions once per layer
              ((d+1)*mL*4); the insert of the step's token: k and v in, their
              pool rows out (4*d*elem), mL codes and list entries out (12*mL)
    qcollect  the exact rerank: the key row of every candidate (d*elem * |C|)
    qfinal    (fused) the attention: K and V rows of every attended token
              (2*d*elem each), the g heads in and their fp32 outputs
    attn      (when the finaliser does not run the attention) as above
    insert    (the standalone ice_insert, not part of a decode step) the
              insert's bytes as above plus the directions
    """
    S, d, mL, g = w.streams, w.d, w.mL, w.g
    elem = 2 if w.dtype == "bf16" else 4
    att = attended * 2 * d * elem + g * d * (elem + 4)
    dirs = (d + 1) * mL * 4.0
    insert = 4.0 * d * elem + 12.0 * mL
    per_stream = {
        "insert": insert,
        "qscan": 4.0 * visits + g * d * elem + 4.0 * mL + 4.0 * d + insert,
        "qcollect": n_cand * d * elem,
        "qfinal": att if fused else 0.0,
        "attn": att,
        # the offloaded pool's staging copy: K and V rows of every attended token
        # in (over the host link) and out (to HBM)
        "fetch": attended * 2 * d * elem * 2,
    }
    per_layer = {"insert": dirs, "qscan": dirs}
    return S * per_stream.get(kernel, 0.0) + per_layer.get(kernel, 0.0)


def scan_code_bytes(w, ntok: float) -> float:
    """What the scan actually reads of the index: every token's m*L codes (it
    computes the walk's closed form in one pass instead of visiting entries)."""
    return w.streams * ntok * w.mL * 4.0


def cpu_baseline(w, K, V, q, U, k_new, v_new, reps: int):
    """The oracle, as it stands, on one layer's decode step for every stream,
    one stream per thread.  Returns (best step microseconds, build seconds,
    threads, mean union size |C|, mean sum_l V_l per stream)."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    oracle.build()
    prm = oracle.Params(d=w.d, p=w.p, k=w.k, m=w.m, L=w.L, g=w.g)
    Kn, Vn, qn, Un = (t.float().cpu().numpy() for t in (K, V, q, U))
    kn, vn = k_new.float().cpu().numpy(), v_new.float().cpu().numpy()
    threads = min(w.streams, os.cpu_count() or 1)

    def build(s):
        return oracle.OracleStream(prm, Kn[s], Vn[s], Un, n_cap=w.n + reps)

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:
        streams = list(ex.map(build, range(w.streams)))
    build_s = time.perf_counter() - t0

    def step(s):
        st = streams[s]
        st.insert(kn[s], vn[s])
        qs = np.ascontiguousarray(qn[s * w.g:(s + 1) * w.g])
        r = st.query(qs)
        st.attend(qs, r["page_ids"])
        return r

    times, res = [], []
    with cf.ThreadPoolExecutor(threads) as ex:
        for _ in range(reps):
            t0 = time.perf_counter()
            res = list(ex.map(step, range(w.streams)))
            times.append(time.perf_counter() - t0)
    sizes = [len(r["C"]) for r in res]
    visits = [float(sum(r["visits"])) for r in res]
    return min(times) * 1e6, build_s, threads, float(np.mean(sizes)), float(np.mean(visits))


def copy_calibration(args):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) of the profiled kernels."""
    import torch
    n = 256 << 20  # bytes
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": args.steps}), flush=True)


# decode kernels reported by the benchmark -> their names in rocprofv3 output
# (the library's own timing names both finalisers "qfinal")
PROFILED = {"qscan": ("k_qscan<",), "qcollect": ("k_qcollect<",),
            "qfinal": ("k_qfinal<", "k_qfinal_big<"), "attn": ("k_attn<",),
            "amerge": ("k_attn_merge",), "fetch": ("k_fetch_pages",)}


def _counter_means(directory: str, counter: str) -> dict:
    """Mean value of `counter` per dispatch, per kernel name, over every
    rocprofv3 counter_collection.csv under `directory`."""
    import csv
    sums = {}
    for root, _, files in os.walk(directory):
        for f in files:
            if not f.endswith("counter_collection.csv"):
                continue
            with open(os.path.join(root, f), newline="") as fh:
                for row in csv.DictReader(fh):
                    if row.get("Counter_Name") != counter:
                        continue
                    name = row["Kernel_Name"]
                    a, c = sums.get(name, (0.0, 0))
                    sums[name] = (a + float(row["Counter_Value"]), c + 1)
    if not sums:
        raise SystemExit(f"no {counter} rows under {directory}")
    return {k: a / c for k, (a, c) in sums.items()}


def counter_summary(directory: str) -> dict:
    """Every counter of every library kernel under `directory` (rocprofv3
    counter_collection.csv files): the mean over dispatches of the sum of a
    dispatch's rows, per kernel (its name without the namespace and template
    arguments) and counter."""
    import csv
    import re
    acc = {}
    for root, _, files in os.walk(directory):
        for f in files:
            if not f.endswith("counter_collection.csv"):
                continue
            with open(os.path.join(root, f), newline="") as fh:
                for row in csv.DictReader(fh):
                    m = re.search(r"ice::(\w+)", row["Kernel_Name"])
                    if not m:
                        continue
                    d = acc.setdefault((m.group(1), row["Counter_Name"]), {})
                    k = row["Dispatch_Id"]
                    d[k] = d.get(k, 0.0) + float(row["Counter_Value"])
    out = {}
    for (kern, ctr), d in sorted(acc.items()):
        out.setdefault(kern, {"dispatches": len(d)})[ctr] = sum(d.values()) / len(d)
    return out


def write_traffic(args):
    """HBM bytes per launch of each decode kernel: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled so that a plain device copy of known size
    reads and writes exactly its size."""
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.write_traffic
    copy_bytes = 256 << 20  # the --copy-calibration copy

    def copy_kib(d, counter):
        means = _counter_means(d, counter)
        return max(v for k, v in means.items() if "copy" in k.lower())

    fscale = copy_bytes / 1024.0 / copy_kib(cfetch_dir, "FETCH_SIZE")
    wscale = copy_bytes / 1024.0 / copy_kib(cwrite_dir, "WRITE_SIZE")
    fm = _counter_means(fetch_dir, "FETCH_SIZE")
    wm = _counter_means(write_dir, "WRITE_SIZE")
    per = {}
    for short, pats in PROFILED.items():
        fk = [v for k, v in fm.items() if any(p in k for p in pats)]
        wk = [v for k, v in wm.items() if any(p in k for p in pats)]
        if fk and wk:
            per[short] = int(round(1024.0 * (fk[0] * fscale + wk[0] * wscale)))
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    tr = {}
    if os.path.exists(tfile):
        with open(tfile) as fh:
            tr = json.load(fh)
    h = kernel_source_hash()
    if tr.get("source_hash") != h or abs(tr.get("fetch_scale", 0) - fscale) > 0.05:
        tr = {"workloads": {}}
    tr.update({"source_hash": h, "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
               "unit": "HBM bytes per launch (fetch + write)"})
    tr["workloads"][args.workload] = per
    with open(tfile, "w") as fh:
        json.dump(tr, fh, indent=1)
    print(json.dumps(tr), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=8,
                    help="index copies rotated (at least the layers of one step)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--gqa", choices=("mean", "max"), default="mean",
                    help="GQA query mode: the heads' mean, or per-head walks ranked by the max score")
    ap.add_argument("--offload", nargs="?", const="all", default=None, choices=("all", "values"),
                    help="page pool in pinned host memory (all; 'values': only the value pages, "
                         "the keys stay in HBM); the selected pages are staged in HBM")
    ap.add_argument("--pregen", type=int, default=0,
                    help="decode steps run on every layer copy before timing (a long generation)")
    ap.add_argument("--reuse", type=int, default=1,
                    help="query every REUSE decode steps of a layer; the steps between reuse "
                         "its last page selection (ice_decode_step_reuse)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--counter-summary", metavar="DIR",
                    help="print per-kernel means of every counter under a rocprofv3 --pmc "
                         "output directory (csv) and exit")
    ap.add_argument("--write-traffic", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args)
        return
    if args.counter_summary:
        print(json.dumps(counter_summary(args.counter_summary), indent=1), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the streams of different layers and heads are independent, so a multi-GPU "
              "run would shard whole layers with no exchange)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args)
        return
    if args.reuse < 1:
        print("--reuse must be at least 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_attention_dci_amd import binding, workloads as W

    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    # a decode step of the 32-layer workload runs every layer once
    layers_per_step = w.layers if args.workload == "llama8b_decode_36k" else 1
    R = max(args.layers, layers_per_step)
    passes = 2 if args.reuse == 1 else 5  # timed and kernel-timing passes
    total_calls = (args.warmup + passes * args.steps) * layers_per_step
    per_layer = (total_calls + R - 1) // R + 1
    cap = w.n + per_layer + args.pregen

    log(f"[bench] building {R} layers of {args.workload}")
    layers, build_ms = [], []
    keep = None
    for r in range(R):
        K, V, q, U, _ = W.layer_inputs(w, layer=r, device=dev)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        idx = binding.Index(K, V, U, page_size=w.p, budget_k=w.k, m=w.m, L=w.L, gqa_group=w.g,
                            capacity=cap, gqa_mode=args.gqa,
                            offload={None: False, "all": True, "values": "values"}[args.offload])
        e1.record()
        torch.cuda.synchronize()
        build_ms.append(e0.elapsed_time(e1))
        idx.release_build_buffers()
        layers.append(idx)
        if r == 0 and not args.no_cpu:
            keep = (K, V, q, U)
        del K, V
    log(f"[bench] build ms per layer: {[round(x, 2) for x in build_ms]}")
    if args.pregen:  # a long generation on every copy before anything is timed
        for r, idx in enumerate(layers):
            for t in range(args.pregen):
                k_new, v_new, q = W.step_inputs(w, layer=r, step=10 ** 6 + t, device=dev)
                idx.decode_step(k_new, v_new, q)
        torch.cuda.synchronize()
        log(f"[bench] {args.pregen} tokens generated on every layer copy")

    steps_in = [W.step_inputs(w, layer=t % R, step=t, device=dev) for t in range(4 * R)]
    # no page selected until a layer copy's first query
    outs = [(torch.zeros(w.streams, w.k // w.p, dtype=torch.int32, device=dev),
             torch.zeros(w.streams, dtype=torch.int32, device=dev),
             torch.empty(w.streams * w.g, w.d, dtype=torch.float32, device=dev))
            for _ in range(R)]
    call = [0]
    ncall = [0] * R  # decode steps run on each layer copy

    def step(reuse=args.reuse):
        """One decode step of every layer of the step.  With reuse r > 1 a layer
        queries on every r-th of its steps and reuses its last selection on
        the others (reuse=0: reuse only)."""
        for _ in range(layers_per_step):
            t = call[0]
            call[0] += 1
            r = t % R
            k_new, v_new, q = steps_in[t % len(steps_in)]
            pg, npg, out = outs[r]
            if reuse and ncall[r] % reuse == 0:
                layers[r].decode_step(k_new, v_new, q, page_ids=pg, n_pages=npg, out=out)
            else:
                layers[r].decode_step_reuse(k_new, v_new, q, pg, npg, out=out)
            ncall[r] += 1

    host_us = []  # host time to issue one step (argument marshalling and launches)

    def timed(reuse):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        h0 = time.perf_counter()
        for _ in range(args.steps):
            step(reuse)
        host_us.append((time.perf_counter() - h0) * 1e6 / args.steps)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    for _ in range(args.warmup):
        step(1)
    torch.cuda.synchronize()
    log("[bench] timing")
    ms_per_step = timed(args.reuse)
    reuse_res = None
    if args.reuse > 1:  # the two kinds of step the schedule mixes, timed alone
        q_ms, r_ms = timed(1), timed(0)
        reuse_res = {"r": args.reuse, "query_step_us": round(q_ms * 1e3, 2),
                     "reuse_step_us": round(r_ms * 1e3, 2)}
        log(f"[bench] reuse {reuse_res}")

    # per-kernel durations: HIP events the library records on the launch stream
    def kernel_times(reuse):
        for idx in layers:
            idx.timing(True)
        for _ in range(args.steps):
            step(reuse)
        torch.cuda.synchronize()
        tot = {}
        for idx in layers:
            for name, (ms, cnt) in idx.timing_read().items():
                a, b = tot.get(name, (0.0, 0))
                tot[name] = (a + ms, b + cnt)
            idx.timing(False)
        return tot, {k: 1e3 * ms / c for k, (ms, c) in tot.items() if c}

    # the kernel table is that of the query steps (every step queries)
    per_kernel, avg_us = kernel_times(1)
    log(f"[bench] per-kernel average us: { {k: round(v, 2) for k, v in avg_us.items()} }")
    if reuse_res is not None:
        _, r_us = kernel_times(0)
        reuse_res["reuse_step_kernels_us"] = {k: round(v, 3) for k, v in r_us.items()}

    # the work each stream's query did: the query statistics of one more decode
    # step on every layer copy (after everything timed)
    stats = binding.stats_tensor(w.streams, dev)
    vis, cands, toks = [], [], []
    walks = w.L * (w.g if args.gqa == "max" else 1)
    for r in range(R):
        k_new, v_new, q = steps_in[r]
        pg, npg, out = outs[r]
        layers[r].decode_step(k_new, v_new, q, page_ids=pg, n_pages=npg, out=out, stats=stats)
        for rec in binding.parse_stats(stats, walks):
            vis.append(float(sum(rec["visits"])))
            cands.append(float(rec["n_cand"]))
            toks.append(float(rec["n_tokens"]))
    visits, n_cand, attended = (sum(x) / len(x) for x in (vis, cands, toks))
    ntok = w.n + args.pregen + per_layer // 2  # mean tokens per stream over the timed steps
    log(f"[bench] per stream: sum_l V_l {visits:.0f} of {walks * w.m * ntok:.0f} entries, "
        f"|C| {n_cand:.1f}, attended {attended:.1f}")

    # page fill of the timed layers (fragmentation after a long generation) and,
    # after one, the list delta-merge of the generated tokens
    npg = torch.stack([ly.view("npages").cpu() for ly in layers]).float()
    fills, partial = [], []
    for ly in layers:
        nps, pl = ly.view("npages").cpu(), ly.view("page_len").cpu()
        for st_ in range(w.streams):
            lens = pl[st_, :int(nps[st_])].float()
            fills.append(float(lens.mean()))
            partial.append(float((lens < w.p).sum()))
    pages = {"tokens_per_stream": layers[0].layout()["n_tokens"],
             "pages_per_stream": round(float(npg.mean()), 1),
             "mean_fill": round(sum(fills) / len(fills), 3), "page_size": w.p,
             "partial_pages_per_stream": round(sum(partial) / len(partial), 1),
             "cells": layers[0].layout()["n_cells"]}
    tail = layers[0].layout()["n_tokens"] - layers[0].layout()["n_build"]
    if args.pregen and tail <= 8192:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nb = binding.lib().ice_merge_scratch_bytes(layers[0]._h)
        scratch = torch.empty(nb, dtype=torch.uint8, device=dev)
        e0.record()
        binding._check(binding.lib().ice_merge_lists(layers[0]._h, binding._ptr(scratch), nb,
                                                     binding._stream(None)), "ice_merge_lists")
        e1.record()
        torch.cuda.synchronize()
        pages["merge_tail"] = tail
        pages["merge_ms"] = round(e0.elapsed_time(e1), 3)
    log(f"[bench] pages: {pages}")

    cpu = None
    if not args.no_cpu and args.gqa == "max":
        log("[bench] no oracle baseline for the GQA max mode (the baseline times the mean mode)")
    elif not args.no_cpu and args.pregen:
        log("[bench] no oracle baseline after a long generation (the oracle holds the built layer)")
    if not args.no_cpu and not args.pregen:
        log("[bench] oracle cpu baseline")
        K, V, q, U = keep
        k_new, v_new, _ = W.step_inputs(w, layer=0, step=10 ** 6, device=dev)
        us, build_s, threads, o_cand, o_visits = cpu_baseline(w, K, V, q, U, k_new, v_new,
                                                              args.cpu_reps)
        cpu = {"value": round(us * layers_per_step, 1), "unit": "us",
               "cores": os.cpu_count(), "threads": threads, "kind": "oracle",
               "build_s": round(build_s, 2),
               "sample": f"one decode step (insert + literal P-DCI query + rerank + page "
                         f"selection + fp64 attention) of all {w.streams} KV heads of one "
                         f"{w.n}-token layer, one head per thread, best of {args.cpu_reps}"
                         + (f", times {layers_per_step} layers" if layers_per_step > 1 else "")
                         + f"; build_s: the oracle's index build of that layer",
               "oracle_visits": round(o_visits, 1), "oracle_union": round(o_cand, 1)}

    kernels = {}
    fused = "attn" not in avg_us
    for k, us in avg_us.items():
        # a layer step's bytes over its launches of the kernel (a kernel
        # launched more than once per layer step shares them)
        per_step = per_kernel[k][1] / float(args.steps * layers_per_step)
        alg = algorithmic_bytes(w, k, visits, n_cand, attended, fused) / max(per_step, 1.0)
        kernels[k] = {"avg_us": round(us, 3), "alg_bytes": int(alg),
                      "gbs": round(alg / (us * 1e-6) / 1e9, 1),
                      "frac": round(alg / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    if "qscan" in kernels:  # what the scan reads beyond the walk's entries
        kernels["qscan"]["code_bytes"] = int(scan_code_bytes(w, ntok))
    dominant = max(avg_us, key=avg_us.get)
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as fh:
            tr = json.load(fh)
        per_wl = tr.get("workloads", {}).get(args.workload, {})
        if tr.get("source_hash") == kernel_source_hash() and dominant in per_wl:
            traffic = per_wl[dominant]
    dk = kernels[dominant]
    roofline = {"bound": "hbm", "kernel": dominant, "achieved": dk["gbs"], "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": dk["frac"], "traffic": traffic, "avg_us": dk["avg_us"],
                "alg_bytes": dk["alg_bytes"]}
    step_alg = sum(algorithmic_bytes(w, k, visits, n_cand, attended, fused)
                   for k in ("qscan", "qcollect", "qfinal", "attn")
                   if k in avg_us) * layers_per_step
    step_gbs = step_alg / (ms_per_step * 1e-3) / 1e9

    res = {
        "metric": "decode-step us (P-DCI query + sparse paged attn) @36k ctx; achieved HBM GB/s",
        "value": round(ms_per_step * 1e3, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i32 codes, f64 rerank; attention on bf16 MFMA (fp32 accumulate, fp32 "
                 "probabilities as bf16 hi+lo pairs), fp32 softmax; bf16 KV",
        "data": "synthetic (seeded Gaussian-mixture keys, N(0,1) values)",
        "config": {"workload": args.workload, "kv_heads": w.streams,
                   "query_heads": w.streams * w.g, "context": w.n, "head_dim": w.d,
                   "page_size": w.p, "budget_k": w.k, "m": w.m, "L": w.L,
                   "layers_per_step": layers_per_step, "layers_rotated": R,
                   "generated_before_timing": args.pregen, "gqa": args.gqa,
                   "pool": {None: "HBM", "all": "host (pinned, staged per step)",
                            "values": "values in host memory (pinned, staged per step), keys in HBM"}[
                       args.offload],
                   "reuse": args.reuse,
                   "step": "ice_decode_step = insert + query_pages + sparse_attn"
                           + ("" if args.reuse == 1 else
                              f"; every {args.reuse}th step of a layer, the others "
                              "ice_decode_step_reuse = insert + sparse_attn over the "
                              "layer's last selection")},
        "build_ms": round(sorted(build_ms)[len(build_ms) // 2], 3),
        # host time to issue one step in the timed loop: below `value`, the
        # device is the bound and the launch queue never runs dry
        "host_us_per_step": round(host_us[0], 2),
        "step_alg_bytes": int(step_alg),
        "step_alg_gbs": round(step_gbs, 1),
        "step_frac": round(step_gbs / PEAK_HBM_GBS, 4),
        "pages": pages,
        "query_stats": {"visits": round(visits, 1), "union_size": round(n_cand, 1),
                        "attended": round(attended, 1), "tokens": ntok},
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if reuse_res is not None:
        res["reuse"] = reuse_res
    if args.offload and "fetch" in avg_us:  # what crosses the host link per layer step
        ways = 1 if args.offload == "values" else 2  # the values alone, or keys and values
        page_bytes = w.streams * attended * ways * w.d * (2 if w.dtype == "bf16" else 4)
        rows = (0 if args.offload == "values" else 1) * w.streams * n_cand * w.d * (
            2 if w.dtype == "bf16" else 4)
        res["offload"] = {"fetch_us": round(avg_us["fetch"], 2), "page_bytes": int(page_bytes),
                          "fetch_link_gbs": round(page_bytes / (avg_us["fetch"] * 1e-6) / 1e9, 1),
                          "rerank_row_bytes_over_link": int(rows),
                          "collect_us": round(avg_us.get("qcollect", 0.0), 2)}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
