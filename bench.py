"""Benchmark of the QSA hot path on one MI355X.

A step is one pass of the whole path -- qsa_compress and qsa_index_logits_topk (as the one call
qsa_compress_index_logits_topk, a single scoring launch for a one-row batch such as this), then
qsa_sparse_gqa -- over one batch of the decode_32k workload: 64 requests at 32768 tokens of context, one query
row each; indexer 8 heads, compress ratio 4, budget 2048, bf16; attention 16 Q / 2 KV heads,
head_dim 128, page 16.  Inputs are seeded synthetic tensors resident in HBM.  Several copies of
the inputs are rotated step by step so that a step never finds its ~270 MB working set in the
256 MB Infinity Cache.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--separate-calls]

Prints one JSON line: rows/s for the whole step, the step's algorithmic HBM GB/s, per-call and
per-kernel times (each kernel alone, through the library call that launches only it), the
roofline of the dominant kernel, and the CPU oracle timed on the host beside it.
"""

from __future__ import annotations

import argparse
import copy
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, 8 TB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # MI355X dense matrix cores per dtype
MFMA_MIN_ROWS = 16      # bf16 requests with more rows are scored on the matrix cores
METRIC = "decode rows/sec + achieved HBM GB/s, QSA indexer+sparse GQA at 32k ctx"
# The kernels timed one by one (each through the call that launches only it), with the sources
# they are built from (a traffic record applies only while these are unchanged).
KERNELS = {
    "prep_compress_kernel": ("compress", ["qsa_internal.h", "prep_ops.h", "compress.hip"]),
    "prep_logits_kernel": ("prep_logits", ["qsa_internal.h", "prep_ops.h", "select.h",
                                           "logits_tile.h", "prep_logits.hip"]),
    "logits_valu_kernel": ("logits", ["qsa_internal.h", "select.h", "select.hip", "logits_tile.h",
                                      "logits.hip", "logits_list.hip", "logits_mfma.hip"]),
    "topk_kernel": ("block_topk", ["qsa_internal.h", "select.h", "select.hip", "topk.hip"]),
    "gqa_partial_kernel": ("gqa_partial", ["qsa_internal.h", "gqa.hip"]),
    "gqa_merge_kernel": ("gqa_merge", ["qsa_internal.h", "gqa.hip"]),
}
# The device kernels each of those calls launches (counter records group them per call).
CALL_KERNELS = {
    "prep_compress_kernel": ("prep_compress_kernel", "ring_store_kernel"),
    "prep_logits_kernel": ("prep_logits_kernel",),
    "logits_valu_kernel": ("logits_valu_kernel", "logits_valu_list_kernel", "logits_mfma_kernel"),
    "topk_kernel": ("topk_kernel",),
    "gqa_partial_kernel": ("gqa_partial_kernel", "gqa_rowtile_kernel"),
    "gqa_merge_kernel": ("gqa_merge_kernel",),
}
NUM_XCDS, NUM_SIMDS = 8, 1024        # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode_32k")
    p.add_argument("--rotate", type=int, default=4, help="input copies cycled through")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--index-agg", choices=("sum", "relu"), default="sum",
                   help="head aggregation of the indexer score (relu: the ReLU-sum switch)")
    p.add_argument("--max-logits-mb", type=float, default=0.0,
                   help="logits memory cap of qsa_index_logits_topk (MB; 0: none): the rows are "
                        "scored and selected in windows whose logits fit it")
    p.add_argument("--main-prepare", action="store_true",
                   help="also run the main-attention prepare inside qsa_compress (the attention "
                        "then uses the prepared Q and reads the gate in place) and report its "
                        "marginal cost")
    p.add_argument("--row-tiles", action="store_true",
                   help="qsa_sparse_gqa's opt-in row-tiled prefill attention (32-row tiles of "
                        "one request share each loaded K/V window)")
    p.add_argument("--separate-calls", action="store_true",
                   help="run qsa_compress and qsa_index_logits_topk as two calls even when the "
                        "batch qualifies for the combined call (its fused scoring launch)")
    p.add_argument("--graph", action="store_true",
                   help="also time the step captured in one HIP graph per input copy")
    p.add_argument("--profile-only", action="store_true",
                   help="warm up and run the timed steps only (for rocprofv3)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only copy MIB MiB device to device 5 times (counter calibration)")
    p.add_argument("--write-traffic", nargs="+",
                   metavar="DIR", help="FETCH_DIR WRITE_DIR CAL_DIR [BENCH_JSON]: record the "
                   "workload's HBM bytes per call in profiles/traffic.json and write "
                   "profiles/<workload>_traffic_counters.md, from rocprofv3 --pmc FETCH_SIZE and "
                   "WRITE_SIZE runs of --profile-only and of --copy-calibration (BENCH_JSON: the "
                   "workload's bench line, for the algorithmic bytes beside them)")
    p.add_argument("--write-mfma-counters", nargs="+", metavar="DIR",
                   help="PMC_DIR [BENCH_JSON]: write profiles/<workload>_mfma_counters.md from a "
                        "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                        "SQ_BUSY_CYCLES GRBM_GUI_ACTIVE run of --profile-only")
    return p.parse_args()


def clone_workload(wl):
    """An independent copy of every tensor of the workload (same contents)."""
    import torch
    c = copy.copy(wl)
    for k, v in vars(wl).items():
        if isinstance(v, torch.Tensor):
            setattr(c, k, v.clone())
    return c


def algorithmic_bytes(wl, packed, combined=False):
    """Bytes each call must move at minimum (read + write), from the workload's shapes and the
    selection it produced.  Compressed keys count once per request (every visible key, read
    once); K/V count once per selected token per KV head (the union of a request's rows'
    selections; one row per request here); partials, logits scratch and re-reads are not
    algorithmic.  `combined`: the step's first two calls are one (qsa_compress_index_logits_topk,
    whose scoring kernel computes q_idx instead of reading it; the top-k reads it)."""
    import numpy as np
    T, Hi, Hq, Hkv = wl.num_tokens, wl.index_heads, wl.q_heads, wl.kv_heads
    elt = 1 if wl.index_dtype == "fp8" else 2
    W = wl.output_width
    c = wl.compress_ratio
    lens = wl.seq_lens_host
    rows = wl.rows_host
    S = int(wl.ring.shape[1])
    groups = int(sum(L // c - (L - n) // c for L, n in zip(lens, rows)))
    b_compress = (T * Hi * 128 * 2 + T * 128 * 2          # q_proj, k_proj
                  + T * Hi * 128 * elt                     # q_idx written
                  + groups * 128 * elt                     # compressed rows written
                  + int(sum(min(S, n) for n in rows)) * 128 * 2)    # ring rows written
    b_logits = (int(sum(L // c for L in lens)) * 128 * elt  # every visible compressed key
                + T * Hi * 128 * elt + T * (W + 1) * 4)    # q_idx read, packed written
    pk = packed.cpu().numpy()
    req = wl.token_to_req.cpu().numpy()
    kv_tokens = 0
    for r in range(wl.num_requests):
        sel = pk[req == r]
        toks = set()
        for row in sel:
            toks.update(row[:row[W]].tolist())
        kv_tokens += len(toks)
    kv_row = 256 if getattr(wl, "kv_dtype", "bf16") == "fp8" else 512   # K + V bytes
    b_gqa = (kv_tokens * Hkv * kv_row                       # K and V rows of selected tokens
             + T * Hq * 128 * 2 * 3                         # q, gate read; out written
             + T * (W + 1) * 4)                             # packed read
    per_call = {"qsa_compress": b_compress, "qsa_index_logits_topk": b_logits,
                "qsa_sparse_gqa": b_gqa}
    b_packed = T * (W + 1) * 4
    b_qgo = T * Hq * 128 * 2
    per_kernel = {"prep_compress_kernel": b_compress,
                  "logits_valu_kernel": b_logits - b_packed,      # keys + q_idx (logits: scratch)
                  "topk_kernel": b_packed,                        # packed rows written
                  "gqa_partial_kernel": b_gqa - 2 * b_qgo,        # K/V, q, packed
                  "gqa_merge_kernel": 2 * b_qgo}                  # gate read, out written
    if combined:
        b_qidx = T * Hi * 128 * elt
        per_call = {"qsa_compress_index_logits_topk": b_compress + b_logits,
                    "qsa_sparse_gqa": b_gqa}
        per_kernel.pop("prep_compress_kernel")
        per_kernel.pop("logits_valu_kernel")
        per_kernel = {"prep_logits_kernel": b_compress + b_logits - b_packed - b_qidx,
                      "topk_kernel": b_packed + b_qidx, **{
                          k: v for k, v in per_kernel.items() if k.startswith("gqa")}}
    return per_call, per_kernel, int(np.int64(kv_tokens))


def mfma_logits_flop(wl, index_agg):
    """Causal-visible indexer logits of the requests the matrix-core kernel scores, as
    (executed, per_head) FLOP: the kernel folds the heads into Q and runs one contraction of 3 x
    128 (three bf16 terms of the folded Q) per (row, visible block), 2 * 384 FLOP; the per-head
    form (one contraction of 128 per head) would be 2 * Hi * 128."""
    if index_agg != "sum" or wl.index_heads > 16:
        return 0, 0
    c, pairs = wl.compress_ratio, 0
    for L, n in zip(wl.seq_lens_host.tolist(), wl.rows_host.tolist()):
        if n > MFMA_MIN_ROWS and n <= L:
            pairs += sum((x + 1) // c for x in range(L - n, L))
    return int(pairs * 2 * 3 * 128), int(pairs * 2 * wl.index_heads * 128)


def _source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNELS[kernel][1]:
        h.update(open(os.path.join(ROOT, "sparse_attention_qsa_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def traffic_record(kernel, workload):
    """Per-launch HBM bytes measured by rocprofv3 counters for the call timed as `kernel`, if the
    committed record holds this workload and was taken on the current kernel sources (else
    None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("workloads", {}).get(workload, {}).get(kernel)
    if not rec:
        return None
    return rec["bytes_per_launch"] if rec.get("source_sha256") == _source_hash(kernel) else None


def _counter_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def _per_dispatch(rows, counter):
    """{kernel name: (mean of the counter per dispatch, dispatches)}; a dispatch's value is the
    sum of its rows (one per XCD or agent instance)."""
    acc = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r.get("Dispatch_Id", ""))
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    by_name = {}
    for (name, _), v in acc.items():
        by_name.setdefault(name, []).append(v)
    return {k: (sum(v) / len(v), len(v)) for k, v in by_name.items()}


def _short(name):
    """A kernel's name without its namespace and argument list."""
    s = name.split("(anonymous namespace)::", 1)[-1].split("(qsa::")[0]
    return s.replace("qsa::(anonymous namespace)::", "").replace("void ", "")


def _call_of(name):
    for call, pats in CALL_KERNELS.items():
        if any(f"::{p}<" in name or f"::{p}(" in name for p in pats):
            return call
    return None


def _bench_line(path):
    if not path:
        return None
    return json.loads(open(path).read().strip().splitlines()[-1])


def write_traffic(dirs, cal_mib, workload):
    """profiles/traffic.json (this workload's entry) and profiles/<workload>_traffic_counters.md:
    HBM bytes per launch of each call, from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each
    scaled by the factor that maps the same counter on a plain copy of cal_mib MiB to its true
    size.  A call's launch sums its kernels' per-dispatch averages.  Both files are written from
    the same counter runs."""
    if len(dirs) not in (3, 4):
        raise SystemExit("--write-traffic FETCH_DIR WRITE_DIR CAL_DIR [BENCH_JSON]")
    fetch_dir, write_dir, cal_dir = dirs[:3]
    bench = _bench_line(dirs[3] if len(dirs) == 4 else None)
    true_bytes = cal_mib * 2**20
    cal = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        pk = _per_dispatch(_counter_rows(cal_dir), counter)
        copies = [v for k, (v, _) in pk.items() if "qsa::" not in k]
        if not copies:
            raise SystemExit("calibration run holds no copy kernel")
        cal[counter] = true_bytes / (max(copies) * 1024.0)
    fetch = _per_dispatch(_counter_rows(fetch_dir), "FETCH_SIZE")
    write = _per_dispatch(_counter_rows(write_dir), "WRITE_SIZE")
    entry = {}
    for kernel in KERNELS:
        names = sorted(k for k in fetch if _call_of(k) == kernel)
        if not names:
            continue
        fb = sum(fetch[k][0] for k in names) * 1024.0
        wb = sum(write.get(k, (0.0, 0))[0] for k in names) * 1024.0
        entry[kernel] = {"fetch_bytes": round(fb * cal["FETCH_SIZE"]),
                         "write_bytes": round(wb * cal["WRITE_SIZE"]),
                         "bytes_per_launch": round(fb * cal["FETCH_SIZE"] + wb * cal["WRITE_SIZE"]),
                         "kernels": names, "source_sha256": _source_hash(kernel)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    table = json.load(open(path)) if os.path.exists(path) else {}
    table = {"_note": "HBM bytes per launch of each call from rocprofv3 --pmc FETCH_SIZE and "
                      "WRITE_SIZE (KiB per dispatch), scaled by the factor that maps each counter "
                      f"on a plain {cal_mib} MiB device copy to its true size; written with "
                      "profiles/<workload>_traffic_counters.md from the same runs",
             "workloads": table.get("workloads", {})}
    table["workloads"][workload] = {"_calibration": cal, **entry}
    json.dump(table, open(path, "w"), indent=1)

    R = "$ROOT"
    lines = [f"# {workload}: HBM traffic counters per kernel", "",
             "Commands (on the MI355X box, from the repository root `$ROOT`; one counter per run):",
             "", "    cd /tmp && export TMPDIR=/tmp"]
    for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        lines.append(f"    timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d {R}/{d} "
                     f"-o run -- python3 {R}/bench.py --workload {workload} --profile-only "
                     "--steps 8 --warmup 2")
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        lines.append(f"    timeout -s KILL 120 rocprofv3 --pmc {c} --output-format csv -d "
                     f"{R}/{cal_dir}/{c} -o run -- python3 {R}/bench.py --copy-calibration "
                     f"{cal_mib}")
    lines += [f"    cd {R} && python3 bench.py --workload {workload} --write-traffic "
              + " ".join(dirs) + "   # writes this file and the workload's entry of "
              "profiles/traffic.json", "",
              f"Calibration: a {cal_mib} MiB device copy reads FETCH_SIZE x "
              f"{1 / cal['FETCH_SIZE']:.4f} and WRITE_SIZE x {1 / cal['WRITE_SIZE']:.4f} of its "
              f"true size; the scaled columns multiply by {cal['FETCH_SIZE']:.4f} and "
              f"{cal['WRITE_SIZE']:.4f}. Counter values are KiB per dispatch, averaged over the "
              "traced dispatches (the warm-up and timed steps of the profile-only run).", "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | "
              "scaled write MB |", "|---|---|---|---|---|---|"]
    for k in sorted((k for k in fetch if _call_of(k)), key=lambda k: -fetch[k][0]):
        f_kib, n = fetch[k]
        w_kib = write.get(k, (0.0, 0))[0]
        lines.append(f"| {_short(k)} | {n} | {f_kib:.1f} | {w_kib:.1f} | "
                     f"{f_kib * 1024 * cal['FETCH_SIZE'] / 1e6:.2f} | "
                     f"{w_kib * 1024 * cal['WRITE_SIZE'] / 1e6:.2f} |")
    lines += ["", "Per call, as profiles/traffic.json records them (the sum of its kernels' rows "
              "above; the bench's roofline.traffic for its dominant kernel): "
              + ", ".join(f"{k} {v['bytes_per_launch'] / 1e6:.2f} MB" for k, v in entry.items())
              + "."]
    if bench:
        ab = bench["per_kernel_algorithmic_bytes"]
        lines += ["", "Algorithmic bytes per launch (the bench line of the same tree): "
                  + ", ".join(f"{k} {v / 1e6:.2f} MB" for k, v in ab.items()) + "; measured / "
                  "algorithmic: " + ", ".join(
                      f"{k} {entry[k.split('+')[0]]['bytes_per_launch'] / v:.3f}"
                      for k, v in ab.items() if k.split('+')[0] in entry and v) + "."]
    out = os.path.join(ROOT, "profiles", f"{workload}_traffic_counters.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print(f"wrote {path} ({workload}) and {out}")


def write_mfma_counters(dirs, workload):
    """profiles/<workload>_mfma_counters.md: matrix-core counters per kernel.  Per dispatch:
    SQ_INSTS_VALU_MFMA_MOPS_BF16 counts bf16 matrix work in units of 512 flop,
    SQ_VALU_MFMA_BUSY_CYCLES the matrix-core busy cycles summed over the SIMDs, GRBM_GUI_ACTIVE
    the GPU's busy cycles summed over the XCDs.  Utilisation = busy / (active / XCDs x SIMDs)."""
    if len(dirs) not in (1, 2):
        raise SystemExit("--write-mfma-counters PMC_DIR [BENCH_JSON]")
    bench = _bench_line(dirs[1] if len(dirs) == 2 else None)
    rows = _counter_rows(dirs[0])
    cnt = {c: _per_dispatch(rows, c) for c in ("SQ_VALU_MFMA_BUSY_CYCLES",
                                               "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                                               "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")}
    names = sorted((k for k in cnt["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
                    if "qsa::" in k and cnt["SQ_INSTS_VALU_MFMA_MOPS_BF16"][k][0] > 0),
                   key=lambda k: -cnt["SQ_INSTS_VALU_MFMA_MOPS_BF16"][k][0])
    R = "$ROOT"
    lines = [f"# {workload}: matrix-core counters per kernel", "",
             "Commands (on the MI355X box, from the repository root `$ROOT`):", "",
             "    cd /tmp && export TMPDIR=/tmp",
             f"    timeout -s KILL 120 rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES "
             f"SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv -d "
             f"{R}/{dirs[0]} -o run -- python3 {R}/bench.py --workload {workload} --profile-only "
             "--steps 4 --warmup 1",
             f"    cd {R} && python3 bench.py --workload {workload} --write-mfma-counters "
             + " ".join(dirs) + "   # writes this file", "",
             "Per dispatch, averaged over the traced dispatches. SQ_INSTS_VALU_MFMA_MOPS_BF16 "
             "counts bf16 matrix work in units of 512 flop (both indexer dtypes run bf16 "
             "contractions); SQ_VALU_MFMA_BUSY_CYCLES is the matrix cores' busy cycles summed "
             f"over the {NUM_SIMDS} SIMDs; GRBM_GUI_ACTIVE is the GPU's busy cycles summed over "
             f"the {NUM_XCDS} XCDs, so the kernel's own cycles are GRBM_GUI_ACTIVE / {NUM_XCDS} "
             "(at 2.4 GHz that agrees with the traced durations). Matrix-core utilisation = "
             f"busy / (cycles x {NUM_SIMDS}); the rate = flop / (cycles / 2.4 GHz).", "",
             "| kernel | dispatches | MOPS_BF16 (x512 flop) | flop (GFLOP) | MFMA busy cycles | "
             "kernel cycles | MFMA utilisation | TFLOP/s at 2.4 GHz |",
             "|---|---|---|---|---|---|---|---|"]
    for k in names:
        mops, n = cnt["SQ_INSTS_VALU_MFMA_MOPS_BF16"][k]
        busy = cnt["SQ_VALU_MFMA_BUSY_CYCLES"].get(k, (0.0, 0))[0]
        cyc = cnt["GRBM_GUI_ACTIVE"].get(k, (0.0, 0))[0] / NUM_XCDS
        flop = mops * 512
        lines.append(f"| {_short(k)} | {n} | {mops:,.0f} | {flop / 1e9:.1f} | {busy:,.0f} | "
                     f"{cyc:,.0f} | {100 * busy / (cyc * NUM_SIMDS):.1f} % | "
                     f"{flop / (cyc / 2.4e9) / 1e12:.0f} |")
    if bench and "mfma_logits" in bench:
        m = bench["mfma_logits"]
        h = m["per_head_equivalent"]
        lines += ["", f"Algorithmic figures of the matrix-core logits (the bench line of the "
                  f"same tree): {m['flop'] / 1e9:.1f} GFLOP of the folded three-term "
                  f"contraction over the causal-visible (row, key) pairs (the counter's figure "
                  f"adds the tile padding at the causal edge); the per-head form would be "
                  f"{h['flop'] / 1e9:.1f} GFLOP. The logits call (this kernel with the max |k| "
                  f"pass) took {m['us']} us in the bench: {m['achieved']} TFLOP/s executed "
                  f"({100 * m['frac']:.1f} % of the 2.5 PFLOP/s bf16 peak), "
                  f"{h['tflops']} TFLOP/s per-head equivalent ({100 * h['frac']:.1f} %)."]
    out = os.path.join(ROOT, "profiles", f"{workload}_mfma_counters.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def copy_calibration(mib):
    """A plain device-to-device copy of mib MiB, 5 times, for counter calibration."""
    import torch
    a = torch.ones(mib * 2**20 // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib}))


_WORKER_WL = None


def _oracle_rows(args):
    """One task of the all-cores leg: the whole step restricted to a slice of the rows, on the
    worker's own host copy of the workload (built on its first task from the same generator;
    the worker was forked before the parent touched the GPU)."""
    global _WORKER_WL
    name, rows, agg = args
    from threadpoolctl import threadpool_limits

    from sparse_attention_qsa_amd.workloads import make_workload
    from tests.oracle_io import oracle_step
    with threadpool_limits(limits=1):
        if _WORKER_WL is None or _WORKER_WL.name != name:
            _WORKER_WL = make_workload(name, device="cpu")
        if rows is None:        # warm-up task: hold the worker so that every worker gets one
            time.sleep(1.0)
            return 0
        oracle_step(_WORKER_WL, rows=rows, agg=agg)
    return len(rows)


def oracle_pool():
    """Worker processes for the all-cores oracle leg, one per host core (at most 16), forked
    before anything in this process initialises the GPU."""
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    cores = max(1, min(int(cores or 1), 16))
    return mp.get_context("fork").Pool(cores), cores


def cpu_baseline(host_inputs, wl_meta, agg="sum", min_seconds=10.0, pool=None):
    """The oracle, as it stands, on the whole step of the same workload (host inputs taken
    before any GPU step): single-threaded, repeated until at least min_seconds have passed;
    then, with `pool`, the same step's rows dealt out to one process per host core."""
    from threadpoolctl import threadpool_limits

    from tests.oracle_io import oracle_step
    reps = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            oracle_step(host_inputs, agg=agg)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    out = {"value": round(reps * wl_meta.num_tokens / dt, 3), "unit": "rows/s", "cores": 1,
           "kind": "oracle",
           "sample": f"the whole step ({wl_meta.num_tokens} rows of {wl_meta.name}) {reps} times, "
                     f"{dt:.2f} s wall on one host core"}
    if pool is None:
        return out
    pool, cores = pool
    T = wl_meta.num_tokens
    cores = min(cores, T)
    slices = [list(range(T))[i::cores] for i in range(cores)]
    # Every worker builds its host copy first (not timed).
    pool.map(_oracle_rows, [(wl_meta.name, None, agg)] * (2 * cores), chunksize=1)
    t0 = time.perf_counter()
    done, passes = 0, 0
    while True:
        done += sum(pool.map(_oracle_rows, [(wl_meta.name, sl, agg) for sl in slices],
                             chunksize=1))
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds / 2:
            break
    out["all_cores"] = {"value": round(done / dt, 3), "unit": "rows/s", "cores": cores,
                        "hardware_concurrency": os.cpu_count(),
                        "sample": f"the whole step's {T} rows dealt to {cores} processes "
                                  f"(each holds a host copy of the workload drawn with the same "
                                  f"recipe and compresses the requests of its rows), {passes} "
                                  f"passes, {dt:.2f} s wall"}
    return out


def measured_ceilings():
    """Practical HBM read ceiling on this device, measured with the library's own probe
    (qsa_diag_read_bandwidth), cold (another 1 GiB buffer is read in between, so the Infinity
    Cache holds nothing useful and no dirty lines): a streaming read of 2 GiB in 4 KiB chunks
    (the compressed keys' page-sized runs), plus a device copy for reference.  The probe's
    gather mode (2 KiB chunks at random positions) is not used as a ceiling: its simple
    eight-chunks-in-flight loop reaches less than the attention kernel's own gather does."""
    import torch

    from sparse_attention_qsa_amd import binding as B
    n = 2 * 2**30
    a = torch.empty(n // 2, dtype=torch.bfloat16, device="cuda:0").normal_()
    b = torch.empty(n // 4, dtype=torch.bfloat16, device="cuda:0")
    flush = torch.empty(2**30 // 4, dtype=torch.float32, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn):
        best = None
        flush.fill_(1.0)
        for _ in range(5):
            flush.sum()   # a read: evicts the Infinity Cache with clean lines
            torch.cuda.synchronize()
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            t = ev[0].elapsed_time(ev[1]) * 1e-3
            best = t if best is None else min(best, t)
        return best
    t_read = timed(lambda: B.qsa_diag_read_bandwidth(a, 4096, sink, stream=stream))
    t_copy = timed(lambda: b.copy_(a[:n // 4]))
    res = {"stream_read_gbps": round(n / t_read / 1e9, 1),
           "copy_gbps": round(2 * (n // 2) / t_copy / 1e9, 1)}
    del a, b, flush
    torch.cuda.empty_cache()
    return res


def path_dtype(wl):
    """Arithmetic types of the path: the indexer's, then the attention's K/V."""
    idx = "e4m3" if wl.index_dtype == "fp8" else "bf16"
    kv = "e4m3" if getattr(wl, "kv_dtype", "bf16") == "fp8" else "bf16"
    return idx if idx == kv else f"{idx} indexer, {kv} attention"


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args.write_traffic, cal_mib=args.copy_calibration or 1024,
                      workload=args.workload)
        return
    if args.write_mfma_counters:
        write_mfma_counters(args.write_mfma_counters, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    pool = None
    if not args.no_cpu_baseline and not args.profile_only:
        pool = oracle_pool()                # forked before this process touches the GPU
    import torch

    from sparse_attention_qsa_amd.step import QsaStep
    from sparse_attention_qsa_amd.workloads import main_prepare_inputs, make_workload

    dev = "cuda:0"
    wl0 = make_workload(args.workload, device=dev)
    host = None
    if not args.no_cpu_baseline and not args.profile_only:
        host = clone_workload(wl0)          # pre-state for the oracle (moved to the host below)
        for k, v in vars(host).items():
            if isinstance(v, torch.Tensor):
                setattr(host, k, v.cpu())
    wls = [wl0] + [clone_workload(wl0) for _ in range(max(0, args.rotate - 1))]
    mains = [main_prepare_inputs(w) if args.main_prepare else None for w in wls]
    cap = int(args.max_logits_mb * 2**20)
    steps = [QsaStep(w, main=m, index_agg=args.index_agg, max_logits_bytes=cap)
             for w, m in zip(wls, mains)]
    for st in steps:
        st.g_args.row_tiles = 1 if args.row_tiles else 0
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # The combined prepare + selection call when the batch qualifies for its fused launch.
    combined = steps[0].fused and not args.separate_calls

    for i in range(args.warmup):
        steps[i % len(steps)].run(stream, combined=combined)
    torch.cuda.synchronize()

    # ---- the timed region: exactly K steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        steps[i % len(steps)].run(stream, combined=combined)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    if args.profile_only:
        print(json.dumps({"profile_only": True, "ms_per_step": ms_step}))
        return

    # ---- per-step distribution: the same K steps again, an event pair around each
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        steps[i % len(steps)].run(stream, combined=combined)
        b.record(stream)
    torch.cuda.synchronize()
    import numpy as np
    per_step_us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    step_dist = {"median": round(float(np.median(per_step_us)), 2),
                 "p10": round(float(np.percentile(per_step_us, 10)), 2),
                 "p90": round(float(np.percentile(per_step_us, 90)), 2)}

    # ---- per-call times (HIP events on the launch stream around each call)
    per_call = {}
    call_fns = ({"qsa_compress_index_logits_topk": "prep_topk", "qsa_sparse_gqa": "gqa"}
                if combined else
                {"qsa_compress": "compress", "qsa_index_logits_topk": "topk",
                 "qsa_sparse_gqa": "gqa"})
    for call, fn in call_fns.items():
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(evs):
            st = steps[i % len(steps)]
            a.record(stream)
            getattr(st, fn)(stream)
            b.record(stream)
        torch.cuda.synchronize()
        per_call[call] = sum(a.elapsed_time(b) for a, b in evs) / len(evs) * 1e3   # us

    # ---- per-kernel times: each kernel alone, through the call that launches only it (the
    # decode workloads run the VALU logits kernel only; prefill ones add the matrix-core one).
    # Launched back to back between two events (rotating the input copies), as in the step, so
    # that the average is the kernel's launch duration rather than launch latency plus kernel.
    def timed(fn_name):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(args.steps):
            getattr(steps[i % len(steps)], fn_name)(stream)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps * 1e3   # us
    import ctypes
    from sparse_attention_qsa_amd import binding as B
    uncapped = type(steps[0].t_args).from_buffer_copy(steps[0].t_args)
    uncapped.max_logits_bytes = 0
    windows = steps[0].t_ws.numel() < B.lib().qsa_index_logits_topk_workspace_size(
        ctypes.byref(uncapped))
    per_kernel = {}
    skip = ({"prep_compress_kernel", "logits_valu_kernel"} if combined
            else {"prep_logits_kernel"})
    for k, (fn, _) in KERNELS.items():
        if k in skip:
            continue    # the other form of the step's first two calls
        if windows and fn in ("logits", "block_topk"):
            continue    # the split top-k calls take one window only (the combined call is timed)
        per_kernel[k] = timed(fn)
    # The merge kernel runs only with several splits that are not merged in the workgroup.
    merge_kernel = B.lib().qsa_sparse_gqa_merge_kernel(ctypes.byref(steps[0].g_args)) == 1
    if not merge_kernel:
        per_kernel.pop("gqa_merge_kernel")

    graph_leg = None
    if args.graph:
        # The same K steps, each a replay of that input copy's captured step (no host launch
        # work between the kernels).  Reported beside the eager figure, not in its place.
        graphs = []
        for st in steps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                st.run(combined=combined)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % len(graphs)].replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(args.steps):
            graphs[i % len(graphs)].replay()
        b.record(stream)
        torch.cuda.synchronize()
        ms_g = a.elapsed_time(b) / args.steps
        graph_leg = {"ms_per_step": round(ms_g, 4),
                     "rows_per_s": round(wl0.num_tokens / (ms_g * 1e-3), 1)}
        del graphs

    main_leg = None
    if args.main_prepare:
        # The prepare's marginal cost: the same compress call without it.
        plain = [QsaStep(w, index_agg=args.index_agg) for w in wls]
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            plain[i % len(plain)].compress(stream)
            b.record(stream)
        torch.cuda.synchronize()
        us_plain = sum(a.elapsed_time(b) for a, b in evs) / len(evs) * 1e3
        elt = 1 if wl0.kv_dtype == "fp8" else 2
        Hq, Hkv, T = wl0.q_heads, wl0.kv_heads, wl0.num_tokens
        mbytes = T * (Hq * 128 * 2 + 2 * Hkv * 128 * 2          # q heads, K, V read
                      + Hq * 128 * 2 + 2 * Hkv * 128 * elt + 8)  # main Q, cache rows written
        marg = per_call["qsa_compress"] - us_plain
        main_leg = {"us_compress_with_main": round(per_call["qsa_compress"], 2),
                    "us_compress_without": round(us_plain, 2), "us_marginal": round(marg, 2),
                    "algorithmic_bytes": int(mbytes),
                    "gbps_over_call": round(mbytes / (per_call["qsa_compress"] * 1e-6) / 1e9, 1)}
        del plain

    alg, alg_k, kv_tokens = algorithmic_bytes(wl0, steps[0].packed, combined)
    if not merge_kernel:   # the attention kernel also reads the gate and writes the output
        alg_k["gqa_partial_kernel"] += alg_k.pop("gqa_merge_kernel")
    mfma_flop, mfma_flop_per_head = mfma_logits_flop(wl0, args.index_agg)
    if mfma_flop:
        # The logits call also launches the matrix-core kernel: name the entry for both (the
        # roofline of the pair is reported against the matrix cores in mfma_logits below).
        both = "logits_valu_kernel+logits_mfma_kernel"
        per_kernel = {both if k == "logits_valu_kernel" else k: v for k, v in per_kernel.items()}
        alg_k[both] = alg_k.pop("logits_valu_kernel")
    step_bytes = sum(alg.values())
    ceilings = measured_ceilings()
    rows_per_s = wl0.num_tokens / (ms_step * 1e-3)
    dom = max(per_kernel, key=per_kernel.get)      # the dominant kernel
    achieved = alg_k[dom] / (per_kernel[dom] * 1e-6) / 1e9
    traffic = traffic_record(dom, wl0.name) if dom in KERNELS else None

    out = {
        "metric": METRIC,
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": path_dtype(wl0),
        "data": "synthetic",
        "config": {"workload": wl0.name, "requests": wl0.num_requests,
                   "context": int(wl0.max_seq_len), "rows_per_request": int(wl0.rows_host[0]),
                   "index_heads": wl0.index_heads, "compress_ratio": wl0.compress_ratio,
                   "budget": wl0.budget, "index_dtype": wl0.index_dtype,
                   "q_heads": wl0.q_heads, "kv_heads": wl0.kv_heads, "head_dim": 128,
                   "page_size": int(wl0.kv_cache.shape[2]), "kv_dtype": getattr(wl0, "kv_dtype", "bf16"),
                   "input_copies_rotated": len(steps),
                   "main_prepare": bool(args.main_prepare), "index_agg": args.index_agg,
                   "max_logits_mb": args.max_logits_mb, "row_tiles": bool(args.row_tiles),
                   "topk_workspace_mb": round(steps[0].t_ws.numel() / 2**20, 1),
                   "combined_prepare_call": combined,
                   "gqa_splits": steps[0].num_splits,
                   "gqa_merge_kernel": merge_kernel},
        "hbm_gbps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "hbm_frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_us": step_dist,
        "measured_ceilings": ceilings,
        "hbm_frac_of_read_ceiling": round(step_bytes / (ms_step * 1e-3) / 1e9
                                          / ceilings["stream_read_gbps"], 4),
        "step_algorithmic_bytes": int(step_bytes),
        "per_call_us": {k: round(v, 2) for k, v in per_call.items()},
        "per_call_algorithmic_bytes": {k: int(v) for k, v in alg.items()},
        "per_kernel_us": {k: round(v, 2) for k, v in per_kernel.items()},
        "per_kernel_algorithmic_bytes": {k: int(alg_k[k]) for k in per_kernel},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "frac_of_read_ceiling": round(achieved / ceilings["stream_read_gbps"], 4)},
    }
    if mfma_flop and "logits_valu_kernel+logits_mfma_kernel" in per_kernel:
        # The logits call of a workload with matrix-core requests: logits_valu_kernel only takes
        # max |k| of their keys, logits_mfma_kernel scores them.  Timed together (one call), so
        # the rate is a lower bound of the matrix-core kernel's own.
        us = per_kernel["logits_valu_kernel+logits_mfma_kernel"]
        tf = mfma_flop / (us * 1e-6) / 1e12
        peak = MFMA_PEAK_TFLOPS["bf16"]      # both indexer dtypes run bf16 contractions
        tf_h = mfma_flop_per_head / (us * 1e-6) / 1e12
        out["mfma_logits"] = {"bound": "mfma", "dtype": "bf16",
                              "kernels": ["logits_valu_kernel (max |k| pass)",
                                          "logits_mfma_kernel"],
                              "us": round(us, 2), "flop": mfma_flop,
                              "achieved": round(tf, 1), "peak": peak,
                              "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                              "per_head_equivalent": {
                                  "flop": mfma_flop_per_head,
                                  "floor_us_at_peak": round(mfma_flop_per_head / peak / 1e6, 2),
                                  "tflops": round(tf_h, 1), "frac": round(tf_h / peak, 4)}}
    if main_leg is not None:
        out["main_prepare"] = main_leg
    if graph_leg is not None:
        out["graph_replay"] = graph_leg
    if host is not None:
        del steps, wls
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(host, wl0, args.index_agg, pool=pool)
    if pool is not None:
        pool[0].close()
        pool[0].join()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
