"""Host-side checks of the benchmark's accounting and its traffic bookkeeping."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import mla_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_attention_flop_per_pair_matches_the_footnote():
    # spke.com article, footnote 1: 2 * (576 + 512) = 2,176 FLOP per row and head
    assert bench.attn_flop_per_pair(1) == 2176
    assert bench.attn_flop_per_pair(64) == 64 * 2176


def test_pair_counts_by_brute_force():
    wl = mla_inputs.Workload("pc", (50, 7), (((0, 20), (40, 50)), ((3, 7),)), n_heads=8,
                             idx_heads=4, idx_dim=64, topk=16, kv_dtype="bf16", seed=0)
    causal = selected = 0
    for p in wl.q_pos():
        keys = list(range(p + 1))
        causal += len(keys)
        selected += min(len(keys), 16)
    pc = bench.pair_counts(wl)
    assert pc == {"causal": causal, "selected": selected}
    f = bench.workload_flops(wl)
    assert f["attention"] == selected * 8 * 2176
    assert f["indexer"] == causal * 2 * 4 * 64


def test_sparse32k_totals():
    wl = mla_inputs.WORKLOADS["sparse32k"]
    pc = bench.pair_counts(wl)
    n = 32768
    assert pc["causal"] == n * (n + 1) // 2
    assert pc["selected"] == sum(min(p + 1, 2048) for p in range(n))


def _write_csv(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_counter_ingestion_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    f_csv, w_csv = tmp_path / "f.csv", tmp_path / "w.csv"
    # the 64 MiB copy reads 2x its size by this counter, writes 1x; a small copy is ignored
    _write_csv(f_csv, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 64.0),
                       ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 2 * 65536.0),
                       ("mla::attn_f8_kernel<false>", "FETCH_SIZE", 1000.0),
                       ("mla::attn_f8_kernel<false>", "FETCH_SIZE", 3000.0)])
    _write_csv(w_csv, [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 65536.0),
                       ("mla::attn_f8_kernel<false>", "WRITE_SIZE", 10.0),
                       ("mla::attn_f8_kernel<false>", "WRITE_SIZE", 30.0)])
    rec = bench.ingest_counters(str(f_csv), str(w_csv), 64, "sparse32k", "fp8", "cmd")
    a = rec["kernels"]["attention"]
    assert rec["fetch_factor"] == pytest.approx(0.5)
    assert a["fetch_bytes"] == pytest.approx(2000 * 1024 * 0.5)
    assert a["write_bytes"] == pytest.approx(20 * 1024)
    assert bench.measured_traffic("sparse32k", "fp8", "attention") == pytest.approx(a["bytes"])
    assert bench.measured_traffic("sparse32k", "bf16", "attention") is None
    assert bench.measured_traffic("sparse32k", "fp8", "indexer") is None
    # fused path: the indexer and merge dispatches of a step add up
    _write_csv(f_csv, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 2 * 65536.0),
                       ("mla::indexer_kernel<128, 2, false, true>(x)", "FETCH_SIZE", 100.0),
                       ("mla::cand_select_kernel(x)", "FETCH_SIZE", 8.0),
                       ("mla::attn_f8_kernel<false>", "FETCH_SIZE", 1000.0)])
    _write_csv(w_csv, [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 65536.0),
                       ("mla::indexer_kernel<128, 2, false, true>(x)", "WRITE_SIZE", 4.0),
                       ("mla::cand_select_kernel(x)", "WRITE_SIZE", 2.0),
                       ("mla::attn_f8_kernel<false>", "WRITE_SIZE", 10.0)])
    rec = bench.ingest_counters(str(f_csv), str(w_csv), 64, "sparse32k", "fp8", "cmd", "bf16", "fused")
    f = rec["kernels"]["indexer_topk"]
    assert f["fetch_bytes"] == pytest.approx(108 * 1024 * 0.5)
    assert f["write_bytes"] == pytest.approx(6 * 1024)
    assert "indexer" not in rec["kernels"] and "topk" not in rec["kernels"]
    assert bench.measured_traffic("sparse32k", "fp8", "indexer_topk", "bf16", "fused") == \
        pytest.approx(f["bytes"])
    # two instances of one kernel per step (top-k rows of 512 and 1,024
    # threads): a launch's bytes are the sum of their per-dispatch means
    _write_csv(f_csv, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 2 * 65536.0),
                       ("mla::topk_kernel<1024>(x)", "FETCH_SIZE", 300.0),
                       ("mla::topk_kernel<512>(x)", "FETCH_SIZE", 20.0),
                       ("mla::topk_kernel<1024>(x)", "FETCH_SIZE", 100.0),
                       ("mla::topk_kernel<512>(x)", "FETCH_SIZE", 40.0)])
    _write_csv(w_csv, [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 65536.0),
                       ("mla::topk_kernel<1024>(x)", "WRITE_SIZE", 6.0),
                       ("mla::topk_kernel<512>(x)", "WRITE_SIZE", 2.0),
                       ("mla::topk_kernel<1024>(x)", "WRITE_SIZE", 6.0),
                       ("mla::topk_kernel<512>(x)", "WRITE_SIZE", 2.0)])
    rec = bench.ingest_counters(str(f_csv), str(w_csv), 64, "ragged", "fp8", "cmd")
    t = rec["kernels"]["topk"]
    assert t["fetch_bytes"] == pytest.approx((200 + 30) * 1024 * 0.5)
    assert t["write_bytes"] == pytest.approx(8 * 1024)
    # a changed kernel source invalidates the stored figure
    table = json.load(open(bench.TRAFFIC_FILE))
    table["sparse32k/fp8"]["kernels"]["attention"]["source_hash"] = "stale"
    json.dump(table, open(bench.TRAFFIC_FILE, "w"))
    assert bench.measured_traffic("sparse32k", "fp8", "attention") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_fp8_indexer_bytes_and_traffic_keys():
    """FP8 indexer inputs: 1-byte codes plus an fp32 scale per (query, head)
    row and per key, w as before; scores as before. The stored traffic of
    the FP8-indexer run sits under its own key."""
    wl = mla_inputs.WORKLOADS["sparse32k"]
    pc = bench.pair_counts(wl)
    b16 = bench.kernel_bytes(wl, "fp8", "bf16")["indexer"]
    b8 = bench.kernel_bytes(wl, "fp8", "fp8")["indexer"]
    assert b16 - b8 == wl.total_q * wl.idx_heads * (wl.idx_dim - 4) + wl.total_kv * (wl.idx_dim - 4)
    assert b8 == pc["causal"] * 4 + wl.total_q * wl.idx_heads * (wl.idx_dim + 8) \
        + wl.total_kv * (wl.idx_dim + 4)
    assert bench.kernel_bytes(wl, "fp8")["attention"] == bench.kernel_bytes(wl, "fp8", "fp8")["attention"]
    assert bench.traffic_key("sparse32k", "fp8") == "sparse32k/fp8"
    assert bench.traffic_key("sparse32k", "fp8", "fp8") == "sparse32k/fp8/indexer-fp8"
    assert bench.traffic_key("sparse32k", "fp8", "bf16", "fused") == "sparse32k/fp8/fused"


def test_fused_path_bytes_and_traffic():
    """The fused indexer + top-k moves the indexer's inputs and the indices,
    not the score matrix; its traffic sums the indexer and merge dispatches
    of a step and is stored under the fused key."""
    wl = mla_inputs.WORKLOADS["sparse32k"]
    pc = bench.pair_counts(wl)
    b = bench.kernel_bytes(wl, "fp8")
    assert b["indexer_topk"] == b["indexer"] - 4 * pc["causal"] + wl.total_q * wl.topk * 4


def test_resume64_is_a_few_query_workload():
    """resume64: 64 new tokens at the end of one 32,768-token sequence."""
    wl = mla_inputs.WORKLOADS["resume64"]
    assert wl.total_q == 64 and wl.total_kv == 32768
    assert list(wl.q_pos()) == list(range(32704, 32768))
    pc = bench.pair_counts(wl)
    assert pc["causal"] == sum(p + 1 for p in range(32704, 32768))
    assert pc["selected"] == 64 * 2048
