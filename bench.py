#!/usr/bin/env python3
"""Benchmark: sparse MLA prefill (indexer -> top-k -> absorbed sparse MLA) on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
mla_indexer_score, mla_topk_select and mla_sparse_prefill (or, for a dense
workload, mla_sparse_prefill alone). Inputs are resident in HBM before the
timed region starts. Prints one JSON line.

Default workload: 32,768-token sparse prefill, 64 heads, indexer 64 x 128
(bf16), top-2,048, FP8-E4M3 latent KV with a per-token scale.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

D_QK, D_V = 576, 512
DS656_ROW = 656
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}     # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0


# ------------------------------------------------------------- accounting --
# Algorithmic work only: causal pairs and selected pairs, never padded tiles.
def attn_flop_per_pair(n_heads: int) -> int:
    """FLOP per (query, attended key): every head does QK over 576 dims and PV
    over 512 (spke.com article, footnote 1: 2,176 FLOP per row and head)."""
    return 2 * (D_QK + D_V) * n_heads


def indexer_flop_per_pair(idx_heads: int, idx_dim: int) -> int:
    """MFMA FLOP per (query, earlier key) of the indexer GEMM."""
    return 2 * idx_heads * idx_dim


def sparse_query_bytes(n_heads: int, topk: int, row_bytes: int = 660) -> int:
    """Bytes one sparse-MLA query moves: topk gathered rows (KV row + 4-byte
    index) plus, per head, its bf16 query (576) and output (512)."""
    return topk * row_bytes + n_heads * 2 * (D_QK + D_V)


def kv_bytes_per_token(mla_layers=78, mla_row=656, idx_layers=21, idx_key=132, mtp=788) -> int:
    return mla_layers * mla_row + idx_layers * idx_key + mtp


def pair_counts(wl) -> dict:
    """Causal (query, key) pairs and selected pairs of a workload."""
    p = wl.q_pos().astype(np.int64)
    causal = int((p + 1).sum())
    selected = causal if wl.dense else int(np.minimum(p + 1, wl.topk).sum())
    return {"causal": causal, "selected": selected}


def workload_flops(wl) -> dict:
    pc = pair_counts(wl)
    f_idx = 0 if wl.dense else pc["causal"] * indexer_flop_per_pair(wl.idx_heads, wl.idx_dim)
    f_attn = pc["selected"] * attn_flop_per_pair(wl.n_heads)
    return {"indexer": f_idx, "attention": f_attn, **pc}


def kernel_bytes(wl, kv_dtype: str, idx_dtype: str = "bf16") -> dict:
    """Algorithmic HBM bytes per launch of each kernel (inputs read once,
    outputs written once; gathered rows counted per selected pair). FP8
    indexer inputs are 1-byte codes plus an fp32 scale per row."""
    pc = pair_counts(wl)
    row = D_QK + 4 if kv_dtype == "fp8" else 2 * D_QK      # 656-byte rows: attention reads bf16
    q_bytes = wl.total_q * wl.n_heads * (2 * D_QK + 2 * D_V + 4)
    out = {"attention": pc["selected"] * (row + (0 if wl.dense else 4)) + q_bytes}
    if kv_dtype == "ds656":
        out["kv_decode"] = wl.total_kv * (DS656_ROW + 2 * D_QK)
    if not wl.dense:
        if idx_dtype == "fp8":
            out["indexer"] = pc["causal"] * 4 + wl.total_q * wl.idx_heads * (wl.idx_dim + 8) \
                + wl.total_kv * (wl.idx_dim + 4)
        else:
            out["indexer"] = pc["causal"] * 4 + wl.total_q * wl.idx_heads * (2 * wl.idx_dim + 4) \
                + wl.total_kv * 2 * wl.idx_dim
        out["topk"] = pc["causal"] * 4 + wl.total_q * wl.topk * 4
        # fused: the indexer's inputs in, the indices out (no score matrix)
        out["indexer_topk"] = out["indexer"] - pc["causal"] * 4 + wl.total_q * wl.topk * 4
    return out


# ---------------------------------------------------------------- traffic --
# Measured HBM traffic per launch comes from two rocprofv3 counter passes over
# this script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by
# what the same counter reads for a device-to-device copy of known size run
# in the same process (--copy-calibration-mib). The figures are stored with a
# hash of the kernel's sources and reported only while the sources match.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {"attention": ("attention.hip", "attention_f8.hip", "attn_common.h"),
                  "indexer": ("indexer.hip", "attn_common.h", "cand_select.h"), "topk": ("topk.hip",),
                  "indexer_topk": ("indexer.hip", "attn_common.h", "cand_select.h", "topk.hip"),
                  "kv_decode": ("decode_ds656.hip",)}
KERNEL_SYMBOLS = {"attention": ("attn_bf16_kernel", "attn_f8_kernel"), "indexer": ("indexer_kernel",),
                  "topk": ("topk_kernel",), "indexer_topk": ("indexer_kernel", "cand_select_kernel"),
                  "kv_decode": ("ds656_decode_kernel",)}
PATH_KERNELS = {"fused": ("indexer_topk", "kv_decode", "attention"),
                "unfused": ("indexer", "topk", "kv_decode", "attention")}
COPY_SYMBOL = "copyBuffer"


def kernel_source_hash(name: str) -> str:
    csrc = os.path.join(ROOT, "sparse_mla_long_amd", "csrc")
    h = hashlib.sha256()
    for f in (*KERNEL_SOURCES[name], "common.h", "kernels.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _counter_rows(path: str, counter: str) -> list:
    with open(path, newline="") as fh:
        return [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]


def traffic_key(workload: str, kv_dtype: str, idx_dtype: str = "bf16", path: str = "unfused") -> str:
    key = "%s/%s" % (workload, kv_dtype)
    key = key if idx_dtype == "bf16" else key + "/indexer-" + idx_dtype
    return key if path == "unfused" else key + "/" + path


def ingest_counters(fetch_csv: str, write_csv: str, calib_mib: int, workload: str,
                    kv_dtype: str, command: str, idx_dtype: str = "bf16", path: str = "unfused") -> dict:
    """Turn the two counter passes into bytes per launch and store them (a
    kernel's launches: the sum over the dispatches of its symbols per step)."""
    n = calib_mib << 20
    rec = {"workload": workload, "kv_dtype": kv_dtype, "indexer_dtype": idx_dtype, "path": path,
           "calibration_bytes": n,
           "command": command, "kernels": {}}
    for key, csv_path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = _counter_rows(csv_path, counter)
        copies = [float(r["Counter_Value"]) for r in rows if COPY_SYMBOL in r["Kernel_Name"]]
        if not copies:
            raise SystemExit("no %s dispatch in %s" % (COPY_SYMBOL, csv_path))
        kib = max(copies)                      # the calibration copy is by far the largest
        factor = n / (kib * 1024.0)
        rec[key + "_factor"] = factor
        rec[key + "_copy_kib"] = kib
        for name in PATH_KERNELS[path]:
            # one list per kernel instance (full name): a call may launch several
            # (the top-k launches one per run of short or long sequences), so a
            # launch's bytes are the sum over instances of their per-dispatch mean
            per_inst = {}
            for r in rows:
                kn = r["Kernel_Name"]
                if any(sym + "<" in kn or sym + "(" in kn for sym in KERNEL_SYMBOLS[name]):
                    per_inst.setdefault(kn, []).append(float(r["Counter_Value"]))
            per_sym = list(per_inst.values())
            if per_sym:
                d = rec["kernels"].setdefault(name, {"source_hash": kernel_source_hash(name)})
                kib = float(sum(np.mean(v) for v in per_sym))
                d[key + "_kib_avg"] = kib
                d[key + "_bytes"] = kib * 1024.0 * factor
                d[key + "_dispatches"] = max(len(v) for v in per_sym)
    for d in rec["kernels"].values():
        d["bytes"] = d.get("fetch_bytes", 0.0) + d.get("write_bytes", 0.0)
    table = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            table = json.load(fh)
    table[traffic_key(workload, kv_dtype, idx_dtype, path)] = rec
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return rec


def measured_traffic(workload: str, kv_dtype: str, name: str, idx_dtype: str = "bf16",
                     path: str = "unfused"):
    """HBM bytes per launch of kernel `name` from the stored counter passes,
    or None when there are none or the kernel's sources changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        rec = json.load(fh).get(traffic_key(workload, kv_dtype, idx_dtype, path))
    d = rec and rec["kernels"].get(name)
    if not d or d["source_hash"] != kernel_source_hash(name) or "fetch_bytes" not in d \
            or "write_bytes" not in d:
        return None
    return d["bytes"]


# ------------------------------------------------------------------ bench --
def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def path_dtype(kv_dtype: str, idx_dtype: str, dense: bool) -> tuple:
    """Arithmetic types of the path: (short label, description)."""
    attn = ("e4m3 MFMA (Q and P*sigma as exact / 8-bit hi+lo E4M3 pairs: bf16 precision), "
            "fp32 accumulate" if kv_dtype == "fp8" else "bf16 MFMA, fp32 accumulate")
    if kv_dtype == "ds656":
        attn += ", on rows decoded from 656-byte E4M3 rows (bf16(code * tile scale))"
    parts = {"attention": attn}
    kinds = {"e4m3" if kv_dtype == "fp8" else "bf16"}
    if kv_dtype == "ds656":
        kinds.add("e4m3")
    if not dense:
        parts["indexer"] = ("e4m3 MFMA on E4M3 codes with fp32 scales" if idx_dtype == "fp8"
                            else "bf16 MFMA") + ", fp32 accumulate"
        parts["topk"] = "int32 radix select on fp32 score keys"
        kinds.add("e4m3" if idx_dtype == "fp8" else "bf16")
    return "+".join(sorted(kinds, reverse=True)), parts


def cpu_baseline(inp, wl, budget_s: float = 12.0, seed: int = 7) -> dict:
    """The fp64 oracle (indexer -> top-k -> attention) timed on the host cores
    on a sample of query rows, extrapolated to the whole workload by FLOP
    weight (row costs span orders of magnitude)."""
    import oracle
    rng = np.random.default_rng(seed)
    q_pos = wl.q_pos()
    fl_pair_i = indexer_flop_per_pair(wl.idx_heads, wl.idx_dim) if not wl.dense else 0
    fl_pair_a = attn_flop_per_pair(wl.n_heads)

    def run(rows):
        t0 = time.perf_counter()
        if wl.dense:
            oracle.attention_rows(inp, rows, None)
        else:
            sc = oracle.indexer_rows(inp, rows)
            idx = oracle.topk_rows(sc, q_pos[rows], wl.topk)
            oracle.attention_rows(inp, rows, idx)
        dt = time.perf_counter() - t0
        p = q_pos[rows].astype(np.int64)
        sel = p + 1 if wl.dense else np.minimum(p + 1, wl.topk)
        return dt, float(((p + 1) * fl_pair_i + sel * fl_pair_a).sum())

    oracle.lib()
    # grow the sample until it takes about budget_s (small samples are
    # dominated by fixed costs, so one calibration step undershoots)
    n = 8
    while True:
        rows = np.sort(rng.choice(wl.total_q, n, replace=False))
        dt, fl = run(rows)
        if dt >= 0.6 * budget_s or n >= wl.total_q:
            break
        n = int(min(wl.total_q, max(2 * n, n * budget_s / max(dt, 1e-3))))
    total_fl = sum(workload_flops(wl)[k] for k in ("indexer", "attention"))
    t_full = dt * total_fl / fl
    return {"value": wl.total_q / t_full, "unit": "query-tokens/s",
            "cores": oracle.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "%d uniformly drawn query rows of the same workload (whole path in fp64: "
                      "indexer over every earlier key, top-k, attention), %.1f s wall, "
                      "extrapolated by FLOP weight" % (n, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sparse32k")
    ap.add_argument("--kv-dtype", default=None,
                    help="override the workload's KV dtype: bf16, fp8 (576 E4M3 + one scale per "
                         "row) or ds656 (656-byte rows, decoded to bf16 before attention)")
    ap.add_argument("--split", type=int, default=None,
                    help="attention through mla_sparse_prefill_split with this many parts per "
                         "query (0: chosen from the CU count)")
    ap.add_argument("--path", default="unfused", choices=("fused", "unfused"),
                    help="unfused: mla_indexer_score, mla_topk_select, attention; fused: "
                         "mla_indexer_topk (indexer and top-k in one pass, no score matrix) then "
                         "attention. Identical indices; unfused measures faster at 32k")
    ap.add_argument("--indexer-dtype", default="bf16", choices=("bf16", "fp8"),
                    help="indexer queries and keys: bf16, or E4M3 codes with an fp32 scale per "
                         "row (mla_indexer_score_fp8)")
    ap.add_argument("--scrub-steps", type=int, default=10,
                    help="after the timed steps, this many more, each behind a 1 GiB fill that "
                         "evicts L2 and MALL (reported as 'scrubbed'; 0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device copy of this size before the steps (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="store per-launch traffic from two rocprofv3 counter CSVs and exit")
    ap.add_argument("--command", default="", help="with --ingest-counters: the profiling command")
    args = ap.parse_args()

    if args.ingest_counters:
        import mla_inputs
        wl = mla_inputs.WORKLOADS[args.workload]
        if args.copy_calibration_mib <= 0:
            raise SystemExit("--ingest-counters needs the --copy-calibration-mib of the runs")
        rec = ingest_counters(args.ingest_counters[0], args.ingest_counters[1],
                              args.copy_calibration_mib, wl.name, args.kv_dtype or wl.kv_dtype,
                              args.command, args.indexer_dtype,
                              "unfused" if wl.dense else args.path)
        print(json.dumps(rec, indent=1))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path "
              "(one GPU runs its own context-parallel share; see --workload cp131k).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mla_inputs
    import sparse_mla_long_amd as sm

    sm.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = mla_inputs.WORKLOADS[args.workload]
    kv_dtype = args.kv_dtype or wl.kv_dtype
    idx_dtype = args.indexer_dtype
    inp = mla_inputs.make_inputs(wl, dev, kv_dtype=kv_dtype, idx_dtype=idx_dtype)
    batch = sm.Batch.from_inputs(inp, dev)
    fused = args.path == "fused" and not wl.dense
    scores = None if wl.dense or fused else torch.empty((wl.total_q, wl.max_kv_len),
                                                        dtype=torch.float32, device=dev)
    topk_ws = sm.topk_workspace(batch, wl.topk) if fused else None
    indices = None if wl.dense else torch.empty((wl.total_q, wl.topk), dtype=torch.int32,
                                                device=dev)
    out = torch.empty((wl.total_q, wl.n_heads, D_V), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((wl.total_q, wl.n_heads), dtype=torch.float32, device=dev)
    names = (["attention"] if wl.dense else ["indexer_topk", "attention"] if fused
             else ["indexer", "topk", "attention"])
    kv_bf16 = None
    if kv_dtype == "ds656":
        names.insert(len(names) - 1, "kv_decode")
        kv_bf16 = torch.empty((wl.total_kv, D_QK), dtype=torch.bfloat16, device=dev)
    split_ws = None
    if args.split is not None:
        need = sm.load_library().mla_sparse_prefill_split_workspace_size(wl.total_q, wl.n_heads,
                                                                          args.split)
        split_ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        def attend(idx, at):
            kv = inp["kv"]
            if kv_bf16 is not None:
                sm.kv_decode_ds656(inp["kv"], out=kv_bf16)
                mark(at)
                at += 1
                kv = kv_bf16
            sm.sparse_prefill(batch, inp["q"], kv, inp["kv_scale"], idx, wl.sm_scale,
                              out=out, lse=lse, n_split=args.split, workspace=split_ws)
            mark(at)

        if wl.dense:
            mark(0)
            attend(None, 1)
            return
        mark(0)
        if fused:
            if idx_dtype == "fp8":
                sm.indexer_topk_fp8(batch, inp["q_idx"], inp["q_idx_scale"], inp["k_idx"],
                                    inp["k_idx_scale"], inp["w"], wl.topk, indices=indices,
                                    workspace=topk_ws)
            else:
                sm.indexer_topk(batch, inp["q_idx"], inp["k_idx"], inp["w"], wl.topk,
                                indices=indices, workspace=topk_ws)
            mark(1)
        else:
            if idx_dtype == "fp8":
                sm.indexer_score_fp8(batch, inp["q_idx"], inp["q_idx_scale"], inp["k_idx"],
                                     inp["k_idx_scale"], inp["w"], scores=scores)
            else:
                sm.indexer_score(batch, inp["q_idx"], inp["k_idx"], inp["w"], scores=scores)
            mark(1)
            sm.topk_select(batch, scores, wl.topk, indices=indices)
            mark(2)
        attend(indices, 2 if fused else 3)

    if args.copy_calibration_mib > 0:
        src = torch.ones(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    def kernel_times(evs):
        return {n: [e[i].elapsed_time(e[i + 1]) for e in evs] for i, n in enumerate(names)}

    warm = kernel_times(events)
    # per-kernel figures: the median over the timed steps (the mean beside it)
    per_kernel_ms = {n: float(np.median(v)) for n, v in warm.items()}
    per_kernel_mean = {n: float(np.mean(v)) for n, v in warm.items()}

    scrubbed = None
    if args.scrub_steps > 0:
        # 1 GiB written by a fill kernel before each step evicts L2 (4 MB per
        # XCD) and MALL (256 MB); the events bracket the path only
        scrub = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        sevents = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
                   for _ in range(args.scrub_steps)]
        for s in range(args.scrub_steps):
            scrub.fill_(float(s))
            step(sevents[s])
        torch.cuda.synchronize()
        st = kernel_times(sevents)
        steps_ms = [e[0].elapsed_time(e[-1]) for e in sevents]
        scrubbed = {"steps": args.scrub_steps, "step_ms_median": float(np.median(steps_ms)),
                    "query_tokens_per_s": wl.total_q / (float(np.median(steps_ms)) * 1e-3),
                    "kernel_ms_median": {n: float(np.median(v)) for n, v in st.items()},
                    "note": "each step behind a 1 GiB fill that evicts L2 and MALL; event time "
                            "of the path only (the fill is outside the events)"}
        del scrub

    fl = workload_flops(wl)
    fl["indexer_topk"] = fl["indexer"]
    byts = kernel_bytes(wl, kv_dtype, idx_dtype)
    # peak of the MFMA type each contraction runs on: the indexer's input
    # dtype; the attention's KV dtype (the FP8 kernel issues E4M3 MFMAs)
    peak_of = {"indexer": PEAK_TFLOPS[idx_dtype], "indexer_topk": PEAK_TFLOPS[idx_dtype],
               "attention": PEAK_TFLOPS["fp8" if kv_dtype == "fp8" else "bf16"]}
    kern = {}
    for n in names:
        t = per_kernel_ms[n] * 1e-3
        d = {"ms": per_kernel_ms[n], "ms_mean": per_kernel_mean[n]}
        if n in ("indexer", "indexer_topk", "attention"):
            tf = fl[n] / t / 1e12
            d.update({"tflops": tf, "bound": "mfma", "peak_tflops": peak_of[n],
                      "frac": tf / peak_of[n]})
            if n == "attention" and kv_dtype == "fp8":
                # each bf16-precision product is two E4M3 MFMAs (hi and lo),
                # so the kernel's own ceiling is half the FP8 peak
                d["bf16_equiv_peak_tflops"] = PEAK_TFLOPS["bf16"]
                d["bf16_equiv_frac"] = tf / PEAK_TFLOPS["bf16"]
        if n in byts:
            d["algo_bytes"] = byts[n]
            d["gbs"] = byts[n] / t / 1e9
        d["traffic"] = measured_traffic(wl.name, kv_dtype, n, idx_dtype, args.path)
        kern[n] = d
    kern["topk"] = kern.get("topk", {})
    if "topk" in per_kernel_ms:
        kern["topk"].update({"bound": "hbm", "peak_gbs": PEAK_HBM_GBS,
                             "frac": kern["topk"]["gbs"] / PEAK_HBM_GBS})
    else:
        kern.pop("topk")
    dominant = max(names, key=lambda n: per_kernel_ms[n])
    dk = kern[dominant]
    if dk.get("bound") == "mfma":
        roof = {"bound": "mfma", "kernel": dominant, "achieved": dk["tflops"],
                "peak": dk["peak_tflops"], "unit": "TFLOP/s", "frac": dk["frac"],
                "traffic": dk["traffic"]}
        if "bf16_equiv_frac" in dk:
            roof["ceiling"] = {"peak": dk["bf16_equiv_peak_tflops"], "frac": dk["bf16_equiv_frac"],
                               "note": "peak priced at FP8 (the MFMA the kernel issues); every "
                                       "QK and PV product is two E4M3 MFMAs (hi + lo) for bf16 "
                                       "precision, so the kernel's ceiling is the bf16 rate"}
    else:
        roof = {"bound": "hbm", "kernel": dominant, "achieved": dk["gbs"], "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": dk["frac"], "traffic": dk["traffic"]}

    ms_step = elapsed / args.steps * 1e3
    dtype_label, dtype_detail = path_dtype(kv_dtype, idx_dtype, wl.dense)
    t_kernels = sum(per_kernel_ms.values()) * 1e-3
    p_attn = PEAK_TFLOPS["fp8" if kv_dtype in ("fp8", "ds656") else "bf16"]
    mfma_frac = (fl["indexer"] / (PEAK_TFLOPS[idx_dtype] * 1e12) +
                 fl["attention"] / (p_attn * 1e12)) / (ms_step * 1e-3)
    res = {
        "metric": "prefill query-tokens/s on 1 MI355X + % MFMA peak (64 heads, top-k 2048)",
        "value": wl.total_q / (ms_step * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_label,
        "dtype_detail": dtype_detail,
        "data": "synthetic",
        "config": {"workload": wl.name, "path": None if wl.dense else args.path,
                   "seq_lens": list(wl.kv_lens), "total_q": wl.total_q,
                   "n_heads": wl.n_heads, "indexer": "%dx%d" % (wl.idx_heads, wl.idx_dim),
                   "indexer_dtype": None if wl.dense else idx_dtype,
                   "attention_split": args.split,
                   "topk": None if wl.dense else wl.topk, "kv_dtype": kv_dtype,
                   "dense": wl.dense, "parallelism": "single GPU"},
        "mfma_peak_frac": mfma_frac,
        "mfma_peak_frac_note": "(F_indexer/P_idx + F_attention/P_attn)/t_step, P_attn = fp8 peak "
                               "for FP8 KV whatever MFMA type the kernel uses, P_idx = the peak "
                               "of the indexer's input dtype",
        "flops": {"indexer": fl["indexer"], "attention": fl["attention"]},
        "kernels": kern,
        "kernel_sum_ms": t_kernels * 1e3,
        "roofline": roof,
        "kernel_time_stat": "median over the timed steps (HIP events on the launch stream)",
    }
    if scrubbed is not None:
        res["scrubbed"] = scrubbed
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, wl, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
