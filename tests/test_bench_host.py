"""Host-side logic of bench.py (no GPU): the one-GPU contract, the HBM
traffic summary built from rocprofv3 counter CSVs, and the algorithmic-byte
accounting of the decode kernels."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_attention_dci_amd import workloads as W  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=FIELDS)
        wr.writeheader()
        for i, (name, value) in enumerate(rows):
            wr.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name,
                         "Counter_Name": counter, "Counter_Value": value})


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_counter_means_per_kernel(tmp_path):
    _write_counters(str(tmp_path), "FETCH_SIZE",
                    [("void ice::k_qscan<1, true, 2, 640>(ice::Dev)", 10.0),
                     ("void ice::k_qscan<1, true, 2, 640>(ice::Dev)", 30.0),
                     ("void ice::k_qcollect<1, 640>(ice::Dev)", 5.0)])
    m = bench._counter_means(str(tmp_path), "FETCH_SIZE")
    assert m["void ice::k_qscan<1, true, 2, 640>(ice::Dev)"] == 20.0
    assert m["void ice::k_qcollect<1, 640>(ice::Dev)"] == 5.0
    with pytest.raises(SystemExit):
        bench._counter_means(str(tmp_path), "WRITE_SIZE")


def test_write_traffic_scales_by_the_copy(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled so the
    256 MiB calibration copy reads and writes exactly 256 MiB."""
    copy_kib = 256 * 1024
    _write_counters(str(tmp_path / "cf"), "FETCH_SIZE",
                    [("__amd_rocclr_copyBuffer", copy_kib / 2), ("fill_kernel", 1.0)])
    _write_counters(str(tmp_path / "cw"), "WRITE_SIZE", [("__amd_rocclr_copyBuffer", copy_kib)])
    _write_counters(str(tmp_path / "f"), "FETCH_SIZE",
                    [("void ice::k_qscan<1, true, 2, 640>(x)", 100.0),
                     ("void ice::k_qfinal_big<1>(x)", 7.0)])
    _write_counters(str(tmp_path / "w"), "WRITE_SIZE",
                    [("void ice::k_qscan<1, true, 2, 640>(x)", 3.0),
                     ("void ice::k_qfinal_big<1>(x)", 1.0)])
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0123456789abcdef")

    class A:
        write_traffic = [str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                         str(tmp_path / "cw")]
        workload = "llama8b_layer_36k"
    bench.write_traffic(A)
    tr = json.load(open(prof / "traffic.json"))
    assert tr["fetch_scale"] == 2.0 and tr["write_scale"] == 1.0
    assert tr["source_hash"] == "0123456789abcdef"
    per = tr["workloads"]["llama8b_layer_36k"]
    assert per["qscan"] == int(1024 * (100.0 * 2 + 3.0))
    assert per["qfinal"] == int(1024 * (7.0 * 2 + 1.0))  # the large-union finaliser counts as qfinal
    assert "qcollect" not in per


def test_algorithmic_bytes_follow_the_walk():
    """The query's bytes are what the method moves: 4 bytes per list entry the
    P-DCI walk visits (not every code the scan happens to read), one key row
    per candidate for the exact rerank, and K and V rows of the attended
    tokens; per stream, times the layer's streams."""
    w = W.WORKLOADS["llama8b_layer_36k"]
    S, d, mL, g, elem = w.streams, w.d, w.mL, w.g, 2
    visits, cand, att = 819_000.0, 880.0, 256.0  # per stream
    scan = bench.algorithmic_bytes(w, "qscan", visits, cand, att)
    prep_insert = g * d * elem + 4 * mL + 4 * d + 4 * d * elem + 12 * mL
    assert scan == S * (4 * visits + prep_insert) + (d + 1) * mL * 4
    assert bench.algorithmic_bytes(w, "qcollect", visits, cand, att) == S * cand * d * elem
    fin = bench.algorithmic_bytes(w, "qfinal", visits, cand, att)
    assert fin == S * (att * 2 * d * elem + g * d * (elem + 4))
    # the attention is counted once: in the finaliser when it is fused, else
    # in the standalone kernel
    assert bench.algorithmic_bytes(w, "qfinal", visits, cand, att, fused=False) == 0.0
    assert bench.algorithmic_bytes(w, "attn", visits, cand, att, fused=False) == fin
    # the walk's bytes scale with the visits; the scan's code read does not
    assert bench.scan_code_bytes(w, 36865) == S * 36865 * mL * 4
    assert bench.algorithmic_bytes(w, "qscan", 2 * visits, cand, att) - scan == S * 4 * visits
