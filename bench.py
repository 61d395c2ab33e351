#!/usr/bin/env python3
"""Benchmark: samples/s of the sparse embedding + DIN attention forward on one
MI355X, on seeded synthetic Taobao-shaped inputs.

A step is one pass of the whole path over one batch already resident in HBM:
lengths -> offsets, sequence plan, sum-pooled embedding bags (16 tables,
3.14M rows), padding-free DIN attention (bf16 matrix cores, fp32 accumulate),
made as one rec_sparse_din_fwd call (three kernel launches).  The rest of the
MultiTowerDIN forward (deep tower + final MLP, rec_towers_fwd) is timed
beside it and reported under "towers"; it is not part of the timed step.  So are
the sparse backward with its AdaGrad step ("adagrad"), the DIN attention's
backward ("din_bwd"), the hash tables' rebuild and admission ("hash_rebuild",
"hash_admit"), the DLRM interaction layer at 217 x 96 ("dlrm_interaction")
and the DLRM forwards ("dlrm_forward", "dlrm_wide").  Kernel times come warm
and cold (1 GiB read before each step: "warm", "cold"), beside the chip's
measured copy rate ("copy_peak") and a leg whose inputs start in pinned host
memory ("host_inputs").
Four resident batches rotate (so the L2 does not keep one batch's rows); one
HIP graph holds a step for each of them and is replayed.  Within a step
everything runs on one stream: inside a graph, a fork/join to a second stream
costs more than the overlap it buys for the short plan (--side-stream to
compare).  Across steps, several batches are kept in flight: over the four
resident batches and over sixteen (--flight-batches), batch k on stream k
mod n (n = 2 and 4 are measured), one graph per stream, so one batch's
gathers run beside another's attention; `value` is the fastest of these
throughputs (config.streams and config.rotating_batches say which), and the
single-stream step is reported beside it.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--config 2]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "samples/s for embedding+DIN fwd at B=8192; HBM GB/s and MFMA util vs peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 matrix/vector

# algorithmic bytes (what the method must move) and flops per unit
INSERT_BYTES_PER_KEY = 8 + 64 + 8 + 1 + 64 + 8   # read key + values; write key, digest, values, score
CLEAR_BYTES_PER_SLOT = 8 + 1 + 8                 # key, digest, score
EMB_BYTES_PER_ID = 8 + 64                  # raw id + one 64-byte row
EMB_BYTES_PER_BAG = 4 + 8 + 64             # length + offset + pooled output
DIN_BYTES_PER_POS = 3 * (8 + 64)           # three ids + three rows
PLAN_BYTES_PER_POS = 3 * 8 + 20            # the plan build: three ids in, 20 B of entries out
PLAN_BYTES_PER_SAMPLE = 4 + 4 + 8          # length in; packed start, sequence base out
DIN_BYTES_PER_SAMPLE = 4 + 8 + 4 + 192 + 192   # length, offset, packed start, query, output
DIN_BYTES_WEIGHTS = 256 * 192 * 2 + 64 * 256 * 2 + (256 + 64 + 64) * 4
DIN_FLOPS_PER_POS = 2 * (192 * 256 + 256 * 64 + 64)
# what the bf16 kernel executes per position: its first layer takes 144 inputs
# ((W1q + W1d) q + (W1s - W1d) s + W1m (q*s), the same sum)
DIN_EXEC_FLOPS_PER_POS = 2 * (144 * 256 + 256 * 64 + 64)
TOWER_FLOPS_PER_SAMPLE = 2 * (256 * 512 + 512 * 256 + 256 * 128 + 176 * 64 + 64)
TOWER_WEIGHT_BYTES = 2 * (256 * 512 + 512 * 256 + 256 * 128 + 176 * 64)
ADAGRAD_BYTES_PER_READ = 8 + 64            # raw id + the read's 64-byte output gradient
ADAGRAD_BYTES_PER_BAG = 4 + 8              # length + offset
ADAGRAD_BYTES_PER_ROW = 2 * (64 + 64)      # weights and accumulator, read and written


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=2)
    p.add_argument("--batches", type=int, default=4)
    p.add_argument("--flight-batches", type=int, default=16,
                   help="resident batches of the batches-in-flight legs (one graph per stream "
                        "over every stream-th batch: a graph of one step per stream was bound by "
                        "the host's replays)")
    p.add_argument("--range-positions", type=int, default=0)
    p.add_argument("--kernel-reps", type=int, default=100)
    p.add_argument("--cpu-seconds", type=float, default=8.0)
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--calls", action="store_true",
                   help="run a step as the four separate calls instead of one rec_sparse_din_fwd")
    p.add_argument("--side-stream", action="store_true",
                   help="run the sequence plan on a second stream (pays off when the plan is long, "
                        "e.g. hash-table sequence ids)")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-pcie", action="store_true", help="skip the host-resident-inputs leg")
    p.add_argument("--no-hash-rebuild", action="store_true",
                   help="skip timing the rebuild of the hash workload's tables (clear + insert)")
    p.add_argument("--no-dlrm", action="store_true",
                   help="skip the DLRM forward leg (the essay's example model, B=8192)")
    p.add_argument("--no-interaction", action="store_true",
                   help="skip the DLRM interaction leg (217 vectors of width 96 per sample)")
    p.add_argument("--no-two-streams", action="store_true",
                   help="skip the several-batches-in-flight measurements")
    p.add_argument("--no-din-bwd", action="store_true",
                   help="skip the DIN attention backward leg")
    p.add_argument("--no-adagrad", action="store_true",
                   help="skip the backward + sparse AdaGrad leg reported beside the step")
    p.add_argument("--no-towers", action="store_true",
                   help="skip the deep tower + final MLP measurement")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain 64 MiB elementwise copy (for counter scaling)")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="write profiles/traffic_*.json from two rocprofv3 --pmc counter CSVs "
                        "(FETCH_SIZE, WRITE_SIZE) of a --calibrate-copy run, then exit")
    p.add_argument("--profile-summary", metavar="DIR",
                   help="write profiles/step_kernels_<workload>.md (and traffic_*.json) from the "
                        "outputs of the rocprofv3 runs listed in it, found under DIR, then exit")
    return p.parse_args()


def src_hash(files=None) -> str:
    """Hash of kernel sources (all of csrc/, or the named files in it) with
    comments and blank space removed: stored traffic figures stay valid across
    edits of the comments only (the sources hold no string literal with a
    comment marker in it)."""
    h = hashlib.sha256()
    if files is None:
        paths = sorted(glob.glob(os.path.join(ROOT, "sparse_embedding_din_amd", "csrc", "*")))
    else:
        paths = [os.path.join(ROOT, "sparse_embedding_din_amd", "csrc", f) for f in sorted(files)]
    for f in paths:
        with open(f, encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip())
        h.update(os.path.basename(f).encode() + b"\0" + code.encode() + b"\0")
    return h.hexdigest()[:16]


# The sources each kernel's traffic depends on: its own file, the headers it
# includes and the host side that sizes its launch.  A stored figure is used
# only while these are unchanged.
_COMMON = ["rec_internal.h", "rec_abi.hip"]
_FWD = ["rec_din.hip", "rec_fwd.hip", "rec_embbag.hip", "rec_embbag_dev.h", "rec_scan.hip",
        "rec_scan_dev.h", "rec_mfma.h"] + _COMMON
_BWD = ["rec_bwd.hip"] + _COMMON
KERNEL_SOURCES = {"k_din_attn": _FWD, "k_embbag_fwd": _FWD, "k_fwd_gather": _FWD, "k_fwd_sums": _FWD,
                  "k_towers_bf16": ["rec_tower.hip", "rec_mfma.h"] + _COMMON,
                  "k_hash_insert": ["rec_hash.hip"] + _COMMON,
                  "k_hash_insert_winner": ["rec_hash.hip"] + _COMMON,
                  "k_hash_insert_values": ["rec_hash.hip"] + _COMMON,
                  "k_bwd_keys": _BWD, "k_sort_hist": _BWD, "k_sort_scan": _BWD, "k_sort_scatter": _BWD,
                  "k_bwd_chunks": _BWD, "k_bwd_cross": _BWD,
                  "k_dlrm_interact": ["rec_dlrm.hip", "rec_mfma.h"] + _COMMON,
                  "k_dlrm_fwd": ["rec_dlrm_fwd.hip", "rec_mfma.h"] + _COMMON}
for _k in ("k_dinb_prep", "k_dinb_map", "k_dinb_fwd", "k_dinb_soft", "k_dinb_bwdt",
           "k_dinb_gq", "k_dinb_wgrad", "k_dinb_reduce"):
    KERNEL_SOURCES[_k] = ["rec_din_bwd.hip"] + _COMMON


CAL_BYTES = 64 << 20            # bytes read (and written) by the calibration copy
COPY_PEAK_BYTES = 512 << 20     # bytes read (and written) by the measured copy rate
CAL_ROWS = 1 << 20              # random 64-byte rows read (and written) by the calibration gather
CAL_TABLE_ROWS = 3 << 20        # rows of its table (192 MiB, like the embedding tables)
KERNELS = {"k_din_attn": "k_din_attn",
           "k_embbag_fwd": "k_embbag_fwd<", "k_fwd_gather": "k_fwd_gather", "k_fwd_sums": "k_fwd_sums",
           "k_towers_bf16": "k_towers_bf16", "k_hash_insert": "k_hash_insert(",
           "k_hash_insert_winner": "k_hash_insert_winner", "k_hash_insert_values": "k_hash_insert_values",
           "k_bwd_keys": "k_bwd_keys", "k_sort_hist": "k_sort_hist", "k_sort_scan": "k_sort_scan",
           "k_sort_scatter": "k_sort_scatter", "k_bwd_chunks": "k_bwd_chunks",
           "k_bwd_cross": "k_bwd_cross", "k_dlrm_interact": "k_dlrm_interact",
           "k_dinb_prep": "k_dinb_prep",
           "k_dinb_map": "k_dinb_map", "k_dinb_fwd": "k_dinb_fwd", "k_dinb_soft": "k_dinb_soft",
           "k_dinb_bwdt": "k_dinb_bwdt", "k_dinb_gq": "k_dinb_gq", "k_dinb_wgrad": "k_dinb_wgrad",
           "k_dinb_reduce": "k_dinb_reduce", "copy": "MulFunctor", "gather_cal": "vectorized_gather_kernel",
           "k_dlrm_fwd": "k_dlrm_fwd<"}
# kernels whose reads are mostly random 64-byte rows: their FETCH_SIZE is scaled
# by the calibration gather's reading (random 64-byte rows), the others' by
# the calibration copy's (streaming)
RANDOM_ROW_KERNELS = {"k_din_attn", "k_embbag_fwd", "k_fwd_gather", "k_bwd_chunks", "k_bwd_cross",
                      "k_dlrm_fwd"}


def load_traffic(kernels, shash: str, config: str):
    """HBM bytes per launch (summed over `kernels`) from committed rocprofv3
    counter runs, if they were taken on the current kernel sources and this
    workload; else None."""
    tot = 0.0
    for k in kernels:
        path = os.path.join(ROOT, "profiles", f"traffic_{k}_{config}.json")
        if not os.path.exists(path):
            return None
        with open(path) as f:
            d = json.load(f)
        if d.get("src_hash") != src_hash(KERNEL_SOURCES[k]):
            return None
        tot += d["bytes_per_launch"]
    return tot


def traffic_from(fetch_csv: str, write_csv: str, config: str):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of each kernel, each
    scaled by the same counter's reading for the calibration copy (CAL_BYTES
    read, CAL_BYTES written)."""
    import csv

    def per_kernel(path, counter):
        acc = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                name = row["Kernel_Name"]
                for key, pat in KERNELS.items():
                    if pat in name:
                        acc.setdefault(key, []).append(float(row["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}

    fetch, nf = per_kernel(fetch_csv, "FETCH_SIZE")
    write, nw = per_kernel(write_csv, "WRITE_SIZE")
    f_cal = fetch["copy"] * 1024.0 / CAL_BYTES
    w_cal = write["copy"] * 1024.0 / CAL_BYTES
    g_cal = fetch["gather_cal"] * 1024.0 / (CAL_ROWS * 64) if "gather_cal" in fetch else None
    gw_cal = write["gather_cal"] * 1024.0 / (CAL_ROWS * 64) if "gather_cal" in write else None
    only = set(os.environ.get("TRAFFIC_KERNELS", "").split(",")) - {""}
    for k in KERNELS:
        if k in ("copy", "gather_cal") or k not in fetch or k not in write or (only and k not in only):
            continue
        raw = (fetch[k] + write[k]) * 1024.0
        by_copy = fetch[k] * 1024.0 / f_cal + write[k] * 1024.0 / w_cal
        by_gather = None if g_cal is None else fetch[k] * 1024.0 / g_cal + write[k] * 1024.0 / w_cal
        use_gather = k in RANDOM_ROW_KERNELS and by_gather is not None
        b = by_gather if use_gather else by_copy
        d = {"kernel": k, "config": config, "src_hash": src_hash(KERNEL_SOURCES[k]),
             "sources": KERNEL_SOURCES[k], "bytes_per_launch": b,
             "scaled_by": "calibration gather (random 64-byte rows)" if use_gather else "calibration copy",
             "bytes_raw": raw, "bytes_copy_scaled": by_copy, "bytes_gather_scaled": by_gather,
             "fetch_kib_raw": fetch[k], "write_kib_raw": write[k], "dispatches": [nf[k], nw[k]],
             "copy_scale": {"fetch": f_cal, "write": w_cal, "bytes": CAL_BYTES},
             "gather_scale": {"fetch": g_cal, "write": gw_cal, "rows": CAL_ROWS, "bytes": CAL_ROWS * 64}}
        with open(os.path.join(ROOT, "profiles", f"traffic_{k}_{config}.json"), "w") as f:
            json.dump(d, f, indent=1)
        print(f"{k}: {b / 1e6:.3f} MB per launch ({d['scaled_by']}; raw {raw / 1e6:.3f} MB: fetch "
              f"{fetch[k]:.0f} KiB, write {write[k]:.0f} KiB)")
    print(f"copy scale: fetch {f_cal:.3f}, write {w_cal:.3f}; gather scale: fetch {g_cal}, write {gw_cal}")


# The rocprofv3 runs whose summaries profiles/ holds, per workload; {c} is
# the --config number.  Each runs bench.py as it is committed.
PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats -d gpurun_out/prof_cfg{c} -o run --output-format csv "
             "-- python3 bench.py --config {c} --steps 40 --warmup 8 --no-cpu --kernel-reps 40",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_FETCH_SIZE_cfg{c} -o run --output-format csv "
             "-- python3 bench.py --config {c} --steps 8 --warmup 4 --no-cpu --no-graph --kernel-reps 8 "
             "--calibrate-copy",
    "write": "rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc_WRITE_SIZE_cfg{c} -o run --output-format csv "
             "-- python3 bench.py --config {c} --steps 8 --warmup 4 --no-cpu --no-graph --kernel-reps 8 "
             "--calibrate-copy",
    "mfma": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 "
            "SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_BUSY_CYCLES GRBM_GUI_ACTIVE -d gpurun_out/pmc_MFMA_cfg{c} -o run "
            "--output-format csv "
            "-- python3 bench.py --config {c} --steps 8 --warmup 4 --no-cpu --no-graph --kernel-reps 8",
    "lds": "rocprofv3 --pmc SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS GRBM_GUI_ACTIVE "
           "-d gpurun_out/pmc_LDS_cfg{c} -o run --output-format csv "
           "-- python3 bench.py --config {c} --steps 8 --warmup 4 --no-cpu --no-graph --kernel-reps 8",
    "ldsbw": "rocprofv3 --pmc SQ_INSTS_LDS_LOAD_BANDWIDTH -d gpurun_out/pmc_LDSBW_cfg{c} -o run "
             "--output-format csv -- python3 bench.py --config {c} --steps 8 --warmup 4 --no-cpu --no-graph "
             "--kernel-reps 8",
}
CLOCK_HZ = 2.4e9                # MI355X peak engine clock
CUS = 256
# kernels whose LDS counters the summary reports (the matrix-core kernels
# that stream their weights or staged inputs through LDS)
LDS_KERNELS = ("k_din_attn", "k_towers_bf16", "k_dinb_fwd", "k_dinb_bwdt", "k_dinb_wgrad")
SIMDS = 1024                    # 256 CUs x 4 SIMDs


def _kernel_key(name: str):
    for key, pat in KERNELS.items():
        if pat in name:
            return key
    return None


def _stats_line(v):
    import statistics
    return (len(v), statistics.fmean(v), statistics.median(v), min(v), max(v))


def profile_summary(root: str, c: int, workload: str) -> str:
    """profiles/step_kernels_<workload>.md from the outputs of PROFILE_COMMANDS
    under `root` (the runs' -d folders): per-kernel durations of the whole
    run (rocprofv3 --stats), the bench's warm kernel leg picked out of the
    trace by its two spin-kernel markers, HBM traffic per launch (FETCH_SIZE
    and WRITE_SIZE, calibrated) and the MFMA counters of the bf16 kernels."""
    import csv
    d = {k: os.path.join(root, f"{n}_cfg{c}") for k, n in
         (("trace", "prof"), ("fetch", "pmc_FETCH_SIZE"), ("write", "pmc_WRITE_SIZE"), ("mfma", "pmc_MFMA"),
          ("lds", "pmc_LDS"), ("ldsbw", "pmc_LDSBW"))}
    have_lds = all(os.path.exists(os.path.join(d[k], "run_counter_collection.csv")) for k in ("lds", "ldsbw"))
    cmd = {k: v.format(c=c) for k, v in PROFILE_COMMANDS.items()}
    out = [f"# Kernel durations, HBM traffic, MFMA and LDS counters: {workload}", "",
           "Made by `python3 bench.py --config %d --profile-summary gpurun_out` from the outputs of" % c,
           "these runs (each on one MI355X, bench.py as committed):", "", "```"]
    out += [cmd[k] for k in ("trace", "fetch", "write", "mfma") + (("lds", "ldsbw") if have_lds else ())]
    out += ["```", ""]

    rows = list(csv.DictReader(open(os.path.join(d["trace"], "run_kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    spins = [i for i, r in enumerate(rows) if "spin_kernel" in r["Kernel_Name"]]
    leg = {}
    if len(spins) >= 2:
        for r in rows[spins[0] + 1: spins[1]]:
            k = _kernel_key(r["Kernel_Name"])
            if k:
                leg.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out += ["## Warm kernel leg", "",
            "The launches between the run's first two spin kernels: the leg whose attention launches",
            "bench.py times with HIP events bound to the dispatch (`roofline.avg_launch_us`), back to",
            "back over the resident batches (us):", "",
            "| kernel | launches | mean | median | min | max |", "|---|---|---|---|---|---|"]
    for k, v in leg.items():
        n, m, md, lo, hi = _stats_line(v)
        out.append(f"| {k} | {n} | {m:.2f} | {md:.2f} | {lo:.2f} | {hi:.2f} |")
    out += ["", "## Every launch of the run (rocprofv3 --stats)", "",
            "All launches of each kernel: the graph-replayed steps, the two- and four-stream legs",
            "(where launches of different batches overlap and each runs longer), the warm and cold",
            "(1 GiB read before each step) kernel legs and the side workloads (us):", "",
            "| kernel | calls | avg | min | max |", "|---|---|---|---|---|"]
    for r in csv.DictReader(open(os.path.join(d["trace"], "run_kernel_stats.csv"))):
        n = r["Name"]
        if "rec::" not in n:
            continue
        short = re.sub(r"\(.*$", "", n.replace("rec::(anonymous namespace)::", "")).replace("void ", "")
        out.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")

    fetch_csv = os.path.join(d["fetch"], "run_counter_collection.csv")
    write_csv = os.path.join(d["write"], "run_counter_collection.csv")
    out += ["", "## HBM traffic per launch", "",
            "FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged over the run's dispatches), each",
            "divided by what the same counter reads for a calibration kernel of known traffic: a",
            f"streaming copy ({CAL_BYTES >> 20} MiB read and written) for most kernels, a gather of",
            f"{CAL_ROWS} random 64-byte rows of a {CAL_TABLE_ROWS * 64 >> 20} MiB table for the kernels whose reads",
            "are mostly random embedding rows.  The figures are written to `traffic_<kernel>_" + workload + ".json`",
            "beside this file with the hash of the kernel's sources; bench.py reports them only while",
            "the sources are unchanged.", ""]
    lines = []
    import contextlib
    import io
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        traffic_from(fetch_csv, write_csv, workload)
    lines = buf.getvalue().splitlines()
    out += ["```"] + lines + ["```"]

    acc = {}
    dur = {}
    for r in csv.DictReader(open(os.path.join(d["mfma"], "run_counter_collection.csv"))):
        k = _kernel_key(r["Kernel_Name"])
        if k not in ("k_din_attn", "k_towers_bf16", "k_dinb_fwd", "k_dinb_bwdt", "k_dinb_wgrad"):
            continue
        acc.setdefault(k, {}).setdefault(r["Counter_Name"], {})[r["Dispatch_Id"]] = float(r["Counter_Value"])
        dur.setdefault(k, {})[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    out += ["", "## MFMA counters", "",
            "Means per dispatch.  One v_mfma_f32_16x16x32_bf16 counts 32 in SQ_INSTS_VALU_MFMA_MOPS_BF16",
            "(units of 512 flops) and 16 busy cycles in SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs), so",
            "the busy fraction is busy / (1024 SIMDs x 2.4 GHz x duration); `warm` uses the warm leg's",
            "mean duration above (the counter run's own where the kernel is not in that leg), `counted`",
            "the counter run's own (counter collection serialises dispatches and lengthens them).  The",
            "attention backward's tiles (`k_dinb_*`) run fp32 products: their executed flops come from",
            "SQ_INSTS_VALU_MFMA_MOPS_F32.  GRBM_GUI_ACTIVE is recorded as rocprofv3 reports it.", "",
            "| kernel | dispatches | executed GFLOP | busy cycles | SQ_BUSY_CYCLES | GRBM_GUI_ACTIVE | counted us | busy frac (counted) | busy frac (warm) |",
            "|---|---|---|---|---|---|---|---|---|"]
    for k, cn in acc.items():
        def mean(name):
            v = list(cn.get(name, {}).values())
            return sum(v) / len(v) if v else float("nan")
        busy = mean("SQ_VALU_MFMA_BUSY_CYCLES")
        mops = mean("SQ_INSTS_VALU_MFMA_MOPS_F32" if k.startswith("k_dinb") else "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        du = sum(dur[k].values()) / len(dur[k])
        warm = statistics_mean(leg.get(k)) or du
        frac_c = busy / (SIMDS * CLOCK_HZ * du * 1e-6)
        frac_w = busy / (SIMDS * CLOCK_HZ * warm * 1e-6) if warm else float("nan")
        out.append(f"| {k} | {len(dur[k])} | {mops * 512 / 1e9:.3f} | {busy:.0f} | {mean('SQ_BUSY_CYCLES'):.0f} | "
                   f"{mean('GRBM_GUI_ACTIVE'):.0f} | {du:.2f} | {frac_c:.4f} | {frac_w:.4f} |")
    if have_lds:
        lacc, ldur = {}, {}
        for key in ("lds", "ldsbw"):
            for r in csv.DictReader(open(os.path.join(d[key], "run_counter_collection.csv"))):
                k = _kernel_key(r["Kernel_Name"])
                if k not in LDS_KERNELS:
                    continue
                lacc.setdefault(k, {}).setdefault(r["Counter_Name"], {})[r["Dispatch_Id"]] = \
                    float(r["Counter_Value"])
                if key == "lds":
                    ldur.setdefault(k, {})[r["Dispatch_Id"]] = \
                        (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        out += ["", "## LDS counters", "",
                "Means per dispatch, from two counter runs (the LDS load bytes in a run of their own).",
                "SQ_INSTS_LDS_LOAD_BANDWIDTH counts 64-byte units loaded from LDS, SQ_LDS_IDX_ACTIVE the",
                "cycles the LDS of a CU is busy (summed over the CUs), SQ_LDS_BANK_CONFLICT the cycles of",
                "those stalled on bank conflicts.  Active fraction = active / (256 CUs x 2.4 GHz x",
                "duration); bytes per CU-cycle = loaded bytes / (256 x 2.4 GHz x duration); `warm` uses the",
                "warm leg's mean duration where the kernel is in it, else the counter run's own.", "",
                "| kernel | dispatches | LDS instructions | loaded MB | active cycles | bank-conflict cycles | "
                "counted us | active frac (counted) | active frac (warm) | loaded B per CU-cycle (warm) |",
                "|---|---|---|---|---|---|---|---|---|---|"]
        for k in LDS_KERNELS:
            if k not in lacc:
                continue
            cn = lacc[k]

            def lmean(name):
                v = list(cn.get(name, {}).values())
                return sum(v) / len(v) if v else float("nan")
            du = sum(ldur[k].values()) / len(ldur[k])
            warm = statistics_mean(leg.get(k)) or du
            act = lmean("SQ_LDS_IDX_ACTIVE")
            loaded = lmean("SQ_INSTS_LDS_LOAD_BANDWIDTH") * 64
            cyc_c = CUS * CLOCK_HZ * du * 1e-6
            cyc_w = CUS * CLOCK_HZ * warm * 1e-6
            out.append(f"| {k} | {len(ldur[k])} | {lmean('SQ_INSTS_LDS'):.0f} | {loaded / 1e6:.1f} | {act:.0f} | "
                       f"{lmean('SQ_LDS_BANK_CONFLICT'):.0f} | {du:.2f} | {act / cyc_c:.4f} | {act / cyc_w:.4f} | "
                       f"{loaded / cyc_w:.1f} |")
    text = "\n".join(out) + "\n"
    with open(os.path.join(ROOT, "profiles", f"step_kernels_{workload}.md"), "w") as f:
        f.write(text)
    return text


def statistics_mean(v):
    return sum(v) / len(v) if v else None


_CPU = {}


def _cpu_worker(args):
    """One CPU worker: the oracle forward over its share of batch 0's samples,
    repeated for `seconds`; returns (samples done, seconds)."""
    i, workers, seconds = args
    import numpy as np

    import oracle
    model, batch = _CPU["model"], _CPU["batch"]
    shard = np.arange(i, batch.B, workers, dtype=np.int64)
    orc = oracle.get()
    t0 = time.perf_counter()
    done = 0
    while True:
        oracle.forward(model, batch, samples=shard, orc=orc)
        done += shard.size
        if time.perf_counter() - t0 >= seconds:
            break
    return done, time.perf_counter() - t0


def cpu_model_name() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_leg(cfg, model, batch, seconds: float, max_workers: int = 16):
    """The oracle as it stands (fp64 C) timed on this host, before the GPU is
    touched (the worker pool forks): on one thread over batch 0's samples,
    then on min(usable cores, max_workers) processes, each over its share of
    the samples (the oracle's work is independent per sample)."""
    import multiprocessing as mp

    import numpy as np

    import oracle
    _CPU["model"], _CPU["batch"] = model, batch
    nproc = os.cpu_count() or 1
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else nproc
    workers = max(1, min(usable, max_workers))
    orc = oracle.get()
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.forward(model, batch, orc=orc)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 20:
            break
    one = reps * batch.B / el
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        t1 = time.perf_counter()
        res = pool.map(_cpu_worker, [(i, workers, seconds) for i in range(workers)])
        wall = time.perf_counter() - t1
    done = sum(r[0] for r in res)
    many = done / max(r[1] for r in res)
    print(f"[bench] oracle: {one:.0f} samples/s on 1 thread, {many:.0f} on {workers} processes",
          file=sys.stderr, flush=True)
    return {"value": round(many, 1), "unit": "samples/s", "cores": workers, "kind": "oracle",
            "single_thread": round(one, 1), "nproc": nproc, "usable_cores": usable,
            "cpu_model": cpu_model_name(),
            "sample": f"the oracle forward (fp64 C: offsets, embedding bags, DIN attention) of "
                      f"batch 0 ({batch.B} samples) of {cfg.name}: {reps} passes on one thread "
                      f"in {el:.1f} s; then {workers} processes, each over every {workers}-th "
                      f"sample for about {seconds:.0f} s ({done} samples, {wall:.1f} s wall)"}


def main():
    a = parse()
    if a.profile_summary:
        import synth
        print(profile_summary(a.profile_summary, a.config, synth.WORKLOADS[a.config].name))
        return
    if a.traffic_from:
        import synth
        traffic_from(a.traffic_from[0], a.traffic_from[1], synth.WORKLOADS[a.config].name)
        return
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {a.gpus} is not supported "
              "(the forward is data-parallel over samples with replicated tables and needs no "
              "collective; multi-GPU runs are not part of it)", file=sys.stderr)
        sys.exit(2)
    import numpy as np

    import synth
    cfg = synth.WORKLOADS[a.config]
    B = cfg.B
    t_gen = time.perf_counter()
    model = synth.make_model(cfg)
    batches = [synth.make_batch(model, batch_index=i) for i in range(a.batches)]
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)
    # the CPU leg runs first: its worker pool forks, which must happen before
    # this process touches the GPU
    cpu = None if a.no_cpu else cpu_leg(cfg, model, batches[0], a.cpu_seconds)

    import torch

    from sparse_embedding_din_amd import pipeline as PL
    from sparse_embedding_din_amd import rec as R

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    R.lib()
    dev = torch.device("cuda")
    tabs = PL.DeviceTables(model.tables, dev)
    mlp = PL.DeviceMLP(model, dev)
    # one set of buffers (offsets, plan, outputs) per resident batch, so any
    # call can be replayed for any batch without stale bookkeeping
    dbs = [PL.DeviceBatch(b, dev) for b in batches]
    fwds = [PL.SparseDinForward(tabs, mlp, B, cfg.max_len, dev, range_positions=a.range_positions)
            for _ in dbs]
    nb = len(dbs)
    tw = None if a.no_towers else PL.DeviceTowers(model.towers, dev)
    if tw is not None:
        tw_deep = torch.empty(B, 128, dtype=torch.float32, device=dev)
        tw_logit = torch.empty(B, dtype=torch.float32, device=dev)
        tw_prob = torch.empty(B, dtype=torch.float32, device=dev)

    def towers_call(f, db):
        R.rec_towers_fwd(tw.desc, db.B, f.pooled, f.T * 16, f.att, tw_logit, deep_out=tw_deep,
                         prob=tw_prob)

    stream = torch.cuda.Stream()
    side = torch.cuda.Stream() if a.side_stream else None
    def step(f, db):
        if a.calls or side is not None:
            f.run(db, side=side)
        else:
            f.run_whole(db)

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for f, db in zip(fwds, dbs):
            step(f, db)
    torch.cuda.synchronize()

    # One graph holds one step per resident batch (the launch-bound loop of
    # `nb` forwards); the timed region replays it steps/nb times.
    graph = None
    if not a.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for f, db in zip(fwds, dbs):
                step(f, db)
        torch.cuda.synchronize()
        a.steps = (a.steps + nb - 1) // nb * nb      # whole replays in the timed region

    def run_steps(n):
        """n steps: whole replays of the graph (nb steps each), then any
        remainder as single steps."""
        k0 = 0
        if graph is not None:
            for _ in range(n // nb):
                graph.replay()
            k0 = n // nb * nb
        for k in range(k0, n):
            step(fwds[k % nb], dbs[k % nb])

    with torch.cuda.stream(stream):
        run_steps(a.warmup)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        run_steps(a.steps)
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / a.steps
    gpu_ms = e0.elapsed_time(e1) / a.steps
    ms_per_step = wall_ms
    print(f"[bench] timed {a.steps} steps: wall {wall_ms*1e3:.2f} us/step, "
          f"gpu {gpu_ms*1e3:.2f} us/step", file=sys.stderr, flush=True)

    # Batches in flight: the resident batches (the `nb` above, and a larger
    # set whose first `nb` are those) split over ns streams (batch k on stream
    # k mod ns), one graph per stream, replayed in turn, so that one batch's
    # gathers can run beside another's attention.  W warmup steps and exactly
    # K timed steps: whole rounds of the graphs, then the remainder as single
    # steps on their streams.  Reported beside the single-stream step.
    two_stream = None
    in_flight = {}
    nbf = max(a.flight_batches, nb)
    dbs_f, fwds_f = dbs, fwds
    if graph is not None and not a.no_two_streams and nbf > nb:
        extra = [synth.make_batch(model, batch_index=i) for i in range(nb, nbf)]
        dbs_f = dbs + [PL.DeviceBatch(b, dev) for b in extra]
        fwds_f = fwds + [PL.SparseDinForward(tabs, mlp, B, cfg.max_len, dev, range_positions=a.range_positions)
                         for _ in extra]
        del extra
        with torch.cuda.stream(stream):
            for f, db in zip(fwds_f[nb:], dbs_f[nb:]):
                step(f, db)
        torch.cuda.synchronize()
    legs = [(ns, nbl) for nbl in sorted({nb, nbf}) for ns in (2, 4)]
    for ns, nbl in legs:
        if graph is None or nbl % ns != 0 or a.no_two_streams:
            continue
        strs = [torch.cuda.Stream() for _ in range(ns)]
        graphs = [torch.cuda.CUDAGraph() for _ in range(ns)]
        for i in range(ns):
            with torch.cuda.graph(graphs[i], stream=strs[i]):
                for k in range(i, nbl, ns):
                    step(fwds_f[k], dbs_f[k])
        torch.cuda.synchronize()

        def run_n(n):
            for _ in range(n // nbl):
                for i in range(ns):
                    with torch.cuda.stream(strs[i]):
                        graphs[i].replay()
            for k in range(n - n // nbl * nbl):
                with torch.cuda.stream(strs[k % ns]):
                    step(fwds_f[k], dbs_f[k])

        run_n(a.warmup)
        torch.cuda.synchronize()
        s0, ea = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ends = [torch.cuda.Event() for _ in range(ns)]
        tw0 = time.perf_counter()
        s0.record(strs[0])
        for i in range(1, ns):
            strs[i].wait_event(s0)
        run_n(a.steps)
        for i in range(1, ns):
            ends[i].record(strs[i])
            strs[0].wait_event(ends[i])
        ea.record(strs[0])
        torch.cuda.synchronize()
        tw1 = time.perf_counter()
        n2 = a.steps
        leg = {"streams": ns, "ms_per_step": round((tw1 - tw0) * 1e3 / n2, 5),
               "gpu_ms_per_step": round(s0.elapsed_time(ea) / n2, 5),
               "samples_s": round(B / ((tw1 - tw0) / n2), 1), "steps": n2, "warmup": a.warmup,
               "rotating_batches": nbl, "layout": f"batch k on stream k mod {ns}, one graph per stream"}
        in_flight[(ns, nbl)] = leg
        print(f"[bench] {ns} streams, {nbl} batches: wall {leg['ms_per_step'] * 1e3:.2f} us/step",
              file=sys.stderr, flush=True)
        del graphs
    if in_flight:
        two_stream = min(in_flight.values(), key=lambda r: r["ms_per_step"])

    # Kernel durations: HIP events bound to the kernel's own dispatch
    # (rec_time_next_launch -> hipExtLaunchKernelGGL), so each is the
    # kernel's execution time alone, as a kernel trace measures it.  The
    # steps are enqueued one by one (events cannot be bound inside a graph)
    # on the same launch stream and resident batches as the timed region.
    # Warm: back to back.  Cold: a 1 GiB read before each step evicts the
    # L2s and the 256 MB MALL, so the tables (192 MB) come from HBM.
    def stats(v):
        v = np.asarray(v, np.float64)
        return dict(mean=float(v.mean()), median=float(np.median(v)),
                    p10=float(np.percentile(v, 10)), p90=float(np.percentile(v, 90)), n=int(v.size))

    def timed(enqueue, kinds, reps, flush=None):
        """enqueue(r) enqueues rep r; kinds: name -> REC_TIME_* (each kernel
        must launch once per rep).  Returns per-kernel stats (us) and the
        stats of events around each rep (us)."""
        evs = [{k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for k in list(kinds) + ["_rep"]} for _ in range(reps)]
        with torch.cuda.stream(stream):
            for e in evs:                          # create the HIP events
                for x, y in e.values():
                    x.record(stream)
                    y.record(stream)
            torch.cuda.synchronize()
            for r in range(reps):
                if flush is not None:
                    flush()
                for k, w in kinds.items():
                    R.rec_time_next_launch(w, *evs[r][k])
                evs[r]["_rep"][0].record(stream)
                enqueue(r)
                evs[r]["_rep"][1].record(stream)
            torch.cuda.synchronize()
        out = {k: stats([e[k][0].elapsed_time(e[k][1]) * 1e3 for e in evs]) for k in kinds}
        return out, stats([e["_rep"][0].elapsed_time(e["_rep"][1]) * 1e3 for e in evs])

    reps = a.kernel_reps
    step_kinds = {"sums": R.REC_TIME_SUMS, "gather": R.REC_TIME_GATHER, "din": R.REC_TIME_DIN_ATTN}
    # Two short spin kernels bracket this leg, so that a kernel trace of the
    # same command can pick out its launches (the first two spin kernels of
    # the run; the later legs' spins come after them).
    with torch.cuda.stream(stream):
        torch.cuda._sleep(1000)
    kern_us, _ = timed(lambda r: fwds[r % nb].run_whole(dbs[r % nb]), step_kinds, reps)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(1000)

    def calls_rep(r):
        f, db = fwds[r % nb], dbs[r % nb]
        f.offsets_step(db)
        f.plan_step(db)
        f.embbag_step(db)
        f.din_step(db)
    call_us, _ = timed(calls_rep, {"embbag": R.REC_TIME_GATHER, "din_plan": R.REC_TIME_DIN_ATTN}, reps)
    if tw is not None:
        kern_us["towers"] = timed(lambda r: towers_call(fwds[r % nb], dbs[r % nb]),
                                  {"towers": R.REC_TIME_TOWERS}, reps)[0]["towers"]
    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device=dev)     # 1 GiB
    flush_buf.fill_(1.0)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)

    def flush():
        torch.sum(flush_buf, dim=0, out=flush_out)
    cold_reps = max(10, reps // 4)
    cold_us, _ = timed(lambda r: fwds[r % nb].run_whole(dbs[r % nb]), step_kinds, cold_reps, flush)
    # the step's wall time, warm and cold, one graph replay per step (a graph
    # per resident batch), events around each replay
    if graph is not None:
        step_graphs = []
        for f, db in zip(fwds, dbs):
            g1 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g1, stream=stream):
                step(f, db)
            step_graphs.append(g1)
        torch.cuda.synchronize()
        _, warm_step = timed(lambda r: step_graphs[r % nb].replay(), {}, reps)
        _, cold_step = timed(lambda r: step_graphs[r % nb].replay(), {}, cold_reps, flush)
        del step_graphs
    else:
        _, warm_step = timed(lambda r: step(fwds[r % nb], dbs[r % nb]), {}, reps)
        _, cold_step = timed(lambda r: step(fwds[r % nb], dbs[r % nb]), {}, cold_reps, flush)
    cold_calls, _ = timed(calls_rep, {"embbag": R.REC_TIME_GATHER, "din_plan": R.REC_TIME_DIN_ATTN},
                          cold_reps, flush)
    del flush_buf
    # the chip's copy rate, measured: a device-to-device copy of COPY_PEAK_BYTES
    # (as many bytes read as written), so that the gathers' algorithmic GB/s
    # read against what a plain stream reaches as well as against the peak
    cp_src = torch.ones(COPY_PEAK_BYTES // 4, dtype=torch.float32, device=dev)
    cp_dst = torch.empty_like(cp_src)
    _, cp_us = timed(lambda r: cp_dst.copy_(cp_src), {}, 20)
    copy_gbs = 2 * COPY_PEAK_BYTES / (cp_us["median"] * 1e-6) / 1e9
    del cp_src, cp_dst
    copy_peak = {"gb_s": round(copy_gbs, 1), "hbm_frac": round(copy_gbs / HBM_PEAK_GBS, 4),
                 "bytes_read": COPY_PEAK_BYTES, "bytes_written": COPY_PEAK_BYTES, "us": cp_us,
                 "how": "torch copy_ between two device tensors, median of 20 (events around each copy)"}
    print(f"[bench] copy peak: {copy_gbs:.0f} GB/s ({COPY_PEAK_BYTES >> 20} MiB read and written)",
          file=sys.stderr, flush=True)
    print(f"[bench] kernel us (warm): " + ", ".join(f"{k}={v['mean']:.2f}" for k, v in kern_us.items())
          + f"; calls: embbag={call_us['embbag']['mean']:.2f} din={call_us['din_plan']['mean']:.2f}"
          + f"; cold: " + ", ".join(f"{k}={v['mean']:.2f}" for k, v in cold_us.items())
          + f", step {cold_step['mean']:.2f} (warm {warm_step['mean']:.2f})", file=sys.stderr, flush=True)
    step_timing = "one graph replay per step" if graph is not None else "one step enqueued per step"

    # algorithmic work of the average batch
    nnz = float(np.mean([b.values.size for b in batches]))
    P = float(np.mean([np.minimum(b.seq_lengths, cfg.max_len).sum() for b in batches]))
    emb_bytes = nnz * EMB_BYTES_PER_ID + synth.T * B * EMB_BYTES_PER_BAG
    plan_bytes = P * PLAN_BYTES_PER_POS + B * PLAN_BYTES_PER_SAMPLE
    din_bytes = P * DIN_BYTES_PER_POS + B * DIN_BYTES_PER_SAMPLE + DIN_BYTES_WEIGHTS
    din_flops = P * DIN_FLOPS_PER_POS
    bf16 = mlp.dtype in (R.REC_BF16, R.REC_BF16_PACKED)
    peak_mfma = BF16_PEAK_TFLOPS if bf16 else FP32_PEAK_TFLOPS
    shash = src_hash()

    def rates(ku, cu):
        din_t = ku["din"]["mean"] * 1e-6
        return {"din_tflops": round(din_flops / din_t / 1e12, 2),
                "din_mfma_frac": round(din_flops / din_t / 1e12 / peak_mfma, 4),
                "gather_gb_s": round((emb_bytes + plan_bytes) / (ku["gather"]["mean"] * 1e-6) / 1e9, 1),
                "gather_hbm_frac": round((emb_bytes + plan_bytes) / (ku["gather"]["mean"] * 1e-6)
                                         / 1e9 / HBM_PEAK_GBS, 4),
                "embbag_gb_s": round(emb_bytes / (cu["embbag"]["mean"] * 1e-6) / 1e9, 1),
                "embbag_hbm_frac": round(emb_bytes / (cu["embbag"]["mean"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "gather_copy_frac": round((emb_bytes + plan_bytes) / (ku["gather"]["mean"] * 1e-6)
                                          / 1e9 / copy_gbs, 4),
                "embbag_copy_frac": round(emb_bytes / (cu["embbag"]["mean"] * 1e-6) / 1e9 / copy_gbs, 4)}
    warm_rates, cold_rates = rates(kern_us, call_us), rates(cold_us, cold_calls)
    din_tflops = warm_rates["din_tflops"]
    roof = {"kernel": "k_din_attn (the attention launch of rec_sparse_din_fwd)", "bound": "mfma",
            "achieved": din_tflops, "peak": peak_mfma, "unit": "TFLOP/s",
            "frac": round(din_tflops / peak_mfma, 4),
            "traffic": load_traffic(["k_din_attn"], shash, cfg.name),
            "per_launch": {"flops": din_flops, "bytes": din_bytes, "positions": P, "samples": B,
                           "executed_flops": P * DIN_EXEC_FLOPS_PER_POS,
                           "flops_note": "flops = the attention MLP as the pages define it (192 inputs); "
                                         "the bf16 kernel executes executed_flops (144 inputs, the same "
                                         "sum factored)"},
            "avg_launch_us": round(kern_us["din"]["mean"], 3),
            "timing": "mean kernel execution time of the attention launch over "
                      f"{kern_us['din']['n']} warm steps (HIP events bound to the dispatch)"}

    # With host-resident inputs: batch 0's ids and lengths copied from pinned
    # host memory to its device buffers before each step (and, second figure,
    # the pooled output and the attention output copied back after it), on
    # the step's stream.  For the record: the boundary takes device buffers,
    # so `value` has inputs already in HBM.
    pcie = None
    if not a.no_pcie:
        db0, f0 = dbs[0], fwds[0]
        ins = [db0.values, db0.lengths, db0.seq_values, db0.seq_lengths]
        hins = [torch.empty(x.shape, dtype=x.dtype, pin_memory=True) for x in ins]
        for h, x in zip(hins, ins):
            h.copy_(x.cpu())
        houts = [torch.empty((B, f0.T * 16), dtype=torch.float32, pin_memory=True),
                 torch.empty((B, 48), dtype=torch.float32, pin_memory=True)]
        in_bytes = float(sum(x.numel() * x.element_size() for x in ins))
        out_bytes = float(sum(h.numel() * h.element_size() for h in houts))

        def h2d_step(r, back=False):
            for h, x in zip(hins, ins):
                x.copy_(h, non_blocking=True)
            step(f0, db0)
            if back:
                houts[0].copy_(f0.pooled[:B], non_blocking=True)
                houts[1].copy_(f0.att[:B], non_blocking=True)
        timed(h2d_step, {}, 5)
        _, pin_step = timed(h2d_step, {}, reps)
        _, pio_step = timed(lambda r: h2d_step(r, True), {}, reps)
        _, copy_only = timed(lambda r: [x.copy_(h, non_blocking=True) for h, x in zip(hins, ins)], {}, reps)
        pcie = {"inputs_bytes": in_bytes, "outputs_bytes": out_bytes,
                "step_with_inputs_us": pin_step, "step_with_inputs_and_outputs_us": pio_step,
                "inputs_copy_us": copy_only,
                "inputs_copy_gb_s": round(in_bytes / (copy_only["mean"] * 1e-6) / 1e9, 1),
                "samples_s_with_inputs": round(B / (pin_step["mean"] * 1e-6), 1),
                "samples_s_with_inputs_and_outputs": round(B / (pio_step["mean"] * 1e-6), 1),
                "note": "one stream, eager launches, batch 0; pinned host buffers"}
        print(f"[bench] with host inputs: {pin_step['mean']:.1f} us per step ({in_bytes / 1e6:.2f} MB in, "
              f"{pcie['inputs_copy_gb_s']} GB/s); with outputs back: {pio_step['mean']:.1f} us",
              file=sys.stderr, flush=True)
        del hins, houts

    # The whole MultiTowerDIN forward (sparse step + towers), graph-replayed
    # the same way, for the record; `value` stays the sparse step.
    towers = None
    if tw is not None:
        full_ms = None
        if graph is not None:
            g2 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g2, stream=stream):
                for f, db in zip(fwds, dbs):
                    step(f, db)
                    towers_call(f, db)
            with torch.cuda.stream(stream):
                for _ in range(a.warmup // nb):
                    g2.replay()
                torch.cuda.synchronize()
                f0 = torch.cuda.Event(enable_timing=True)
                f1 = torch.cuda.Event(enable_timing=True)
                f0.record(stream)
                for _ in range(a.steps // nb):
                    g2.replay()
                f1.record(stream)
                torch.cuda.synchronize()
            full_ms = f0.elapsed_time(f1) / a.steps
        tt = kern_us["towers"]["mean"] * 1e-6
        # workgroups of the launch: 32 samples each, 64 from 16384 samples on
        tower_groups = (B + 31) // 32 if B < 16384 else (B + 63) // 64
        tflops = TOWER_FLOPS_PER_SAMPLE * B / tt / 1e12
        towers = {"entry": "rec_towers_fwd (deep 256->512->256->128, concat att, 176->64->1)",
                  "avg_launch_us": round(kern_us["towers"]["mean"], 3),
                  "flops_per_launch": TOWER_FLOPS_PER_SAMPLE * B,
                  "achieved_tflops": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
                  "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                  "weight_stream_tb_s": round(TOWER_WEIGHT_BYTES * tower_groups / tt / 1e12, 2),
                  "bound": f"L2 -> CU weight stream: each workgroup of {B // tower_groups} samples "
                           f"reads all {TOWER_WEIGHT_BYTES // 1024} KiB of bf16 weights",
                  "traffic": load_traffic(["k_towers_bf16"], shash, cfg.name),
                  "full_forward_ms_per_step": None if full_ms is None else round(full_ms, 5),
                  "full_forward_samples_s": None if full_ms is None else round(B / (full_ms * 1e-3), 1)}

    rebuild = None
    if not a.no_hash_rebuild:
        # The start-up rebuild of the hash workload's tables ("集成 DynamicEmb"
        # §6.4: 5 tables, keys and values inserted from storage): clear each
        # table, then insert its stored pairs with STEP scores.
        hcfg = synth.WORKLOADS[5]
        hm = model if cfg.hash_keys else synth.make_model(hcfg)
        htabs = PL.DeviceTables([hm.tables[k] for k in hcfg.hash_keys], dev)
        hk, hv = [], []
        for k in hcfg.hash_keys:
            t = hm.tables[k]
            occ = np.nonzero(t["keys"] != R.REC_EMPTY_KEY)[0]
            hk.append(torch.from_numpy(t["keys"][occ]).to(dev))
            hv.append(torch.from_numpy(np.ascontiguousarray(t["values"][occ])).to(dev))
        nkeys = sum(x.numel() for x in hk)
        ins_wsb = max(R.rec_hash_insert_workspace_bytes(x.numel(), hcfg.hash_capacity) for x in hk)
        ins_ws = torch.empty(ins_wsb, dtype=torch.uint8, device=dev)

        def rebuild_tables(ev=None):
            for i in range(len(hk)):
                R.rec_hash_clear(htabs.desc[i], stream=stream)
                if ev is not None:
                    ev[i][0].record(stream)
                R.rec_hash_insert(htabs.desc[i], hk[i], hv[i], hk[i].numel(), R.REC_SCORE_STEP, 1,
                                  None, ins_ws, ins_wsb, stream=stream)
                if ev is not None:
                    ev[i][1].record(stream)

        with torch.cuda.stream(stream):
            for _ in range(3):
                rebuild_tables()
            torch.cuda.synchronize()
            reps_r = 10
            r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    for _ in hk] for _ in range(reps_r)]
            torch.cuda._sleep(20_000_000)
            r0.record(stream)
            for r in range(reps_r):
                rebuild_tables(evs[r])
            r1.record(stream)
            torch.cuda.synchronize()
        total_us = r0.elapsed_time(r1) * 1e3 / reps_r
        ins = np.array([[s_.elapsed_time(e_) * 1e3 for s_, e_ in row] for row in evs])
        ins_us = float(ins.mean())
        per_table = nkeys / len(hk)
        ins_gbs = INSERT_BYTES_PER_KEY * per_table / (ins_us * 1e-6) / 1e9
        rebuild = {"entry": "rec_hash_clear + rec_hash_insert (STEP scores), per table",
                   "tables": len(hk), "capacity": hcfg.hash_capacity, "keys": int(nkeys),
                   "us_all_tables": round(total_us, 2),
                   "keys_per_s": round(nkeys / (total_us * 1e-6), 1),
                   "insert_call_us": round(ins_us, 3),
                   "insert_launches": ["k_hash_insert", "k_hash_insert_winner", "k_hash_insert_values"],
                   "insert_algorithmic_gb_s": round(ins_gbs, 1),
                   "insert_hbm_frac": round(ins_gbs / HBM_PEAK_GBS, 4),
                   "bytes_per_key": INSERT_BYTES_PER_KEY,
                   "traffic": load_traffic(["k_hash_insert", "k_hash_insert_winner", "k_hash_insert_values"],
                                          shash, cfg.name),
                   "pages": "about 100-500 ms for 1.5M keys on the GPU (context, another machine)"}
        print(f"[bench] hash rebuild: {nkeys} keys in {total_us:.1f} us ({ins_us:.2f} us per insert call)",
              file=sys.stderr, flush=True)

    admit = None
    if not a.no_hash_rebuild:
        # One admission step on the hash workload's first table ("集成
        # DynamicEmb" §4.1, §4.2): capacity 300,000 holding 210,000 ids, a batch
        # of 20,000 stored ids and 40,000 new ids seen twice, threshold 2, STEP
        # scores, at most 210,000 ids -- so 40,000 admissions evict as many of
        # the oldest entries.  Each timed call starts from a fresh copy.
        hcfg = synth.WORKLOADS[5]
        hm5 = model if cfg.hash_keys else synth.make_model(hcfg)
        t0_ = hm5.tables[hcfg.hash_keys[0]]
        rng_a = np.random.default_rng(31)
        st_ = t0_["keys"] != R.REC_EMPTY_KEY
        olds = t0_["keys"][st_]
        fresh = np.unique(rng_a.integers(-2**62, 2**62, size=45000, dtype=np.int64))
        fresh = fresh[~np.isin(fresh, olds)][:40000]
        akeys = np.concatenate([rng_a.choice(olds, 20000, replace=False), fresh, fresh])
        akeys = akeys[rng_a.permutation(akeys.size)]
        ak = torch.from_numpy(akeys).to(dev)
        av = torch.from_numpy((rng_a.standard_normal((akeys.size, 16)) * 0.05).astype(np.float32)).to(dev)
        base_sc = np.zeros(int(t0_["rows"]), np.uint64)
        base_sc[st_] = np.arange(int(st_.sum()), dtype=np.uint64) % 1000
        src_t = PL.DeviceTables([dict(t0_, scores=base_sc)], dev)
        work_t = PL.DeviceTables([dict(t0_, scores=base_sc)], dev)
        cap_ = int(t0_["rows"])
        ck_ = torch.empty(1 << 18, dtype=torch.int64, device=dev)
        cc_ = torch.empty(1 << 18, dtype=torch.int64, device=dev)
        a_wsb = R.rec_hash_admit_workspace_bytes(akeys.size, cap_, R.REC_SCORE_STEP)
        a_ws = torch.empty(a_wsb, dtype=torch.uint8, device=dev)
        a_cnt = torch.empty(3, dtype=torch.int64, device=dev)

        def reset_tables():
            for x, y in zip(work_t.tensors[0], src_t.tensors[0]):
                x.copy_(y)
            ck_.fill_(-1)
            cc_.zero_()

        def admit_call():
            R.rec_hash_admit(work_t.desc[0], 210000, ck_, cc_, 1 << 18, ak, av, akeys.size, 2,
                             R.REC_SCORE_STEP, 5000, None, a_cnt, a_ws, a_wsb, stream=stream)
        with torch.cuda.stream(stream):
            reps_ad = 10
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(reps_ad)]
            for r in range(reps_ad + 2):
                reset_tables()
                if r >= 2:
                    evs[r - 2][0].record(stream)
                admit_call()
                if r >= 2:
                    evs[r - 2][1].record(stream)
            torch.cuda.synchronize()
        d_ad = np.array([x.elapsed_time(y) * 1e3 for x, y in evs])
        admit = {"entry": "rec_hash_admit (STEP, threshold 2, max_keys 210,000, full table)",
                 "ids": int(akeys.size), "admitted_evicted_left": [int(x) for x in a_cnt.cpu().tolist()],
                 "call_us": float(d_ad.mean()), "ids_per_s": round(akeys.size / (d_ad.mean() * 1e-6), 1)}
        print(f"[bench] hash admission: {d_ad.mean():.1f} us per call ({akeys.size} ids, "
              f"{admit['admitted_evicted_left']})", file=sys.stderr, flush=True)
        del src_t, work_t, a_ws

    adagrad = None
    if not a.no_adagrad:
        # The sparse half of a training step, beside the forward: gradients of
        # the pooled bags and of the sequence rows (random, as the dense
        # backward would deliver them) summed per row, then one AdaGrad step
        # ("当前现状分析" run-config table), on copies of the tables.
        rng = np.random.default_rng(4242)
        T = synth.T
        rows = [int(t["rows"]) for t in model.tables]
        aw = [torch.from_numpy(np.asarray(t["values"], np.float32)).to(dev) for t in model.tables]
        aa = [torch.zeros(r, 16, dtype=torch.float32, device=dev) for r in rows]
        akd = [(torch.from_numpy(t["keys"]).to(dev), torch.from_numpy(t["digests"]).to(dev))
               if t["kind"] == "hash" else (None, None) for t in model.tables]
        atabs = [R.adagrad_table(aw[t], aa[t], rows[t],
                                 R.REC_HASH if akd[t][0] is not None else R.REC_DIRECT, *akd[t])
                 for t in range(T)]

        def flat_rows(t, raw):
            tab = model.tables[t]
            if tab["kind"] != "hash":
                return np.mod(raw, rows[t]) + sum(rows[:t])
            occ = np.nonzero(tab["keys"] != R.REC_EMPTY_KEY)[0]
            order = np.argsort(tab["keys"][occ])
            sk, ss = tab["keys"][occ][order], occ[order]
            at = np.minimum(np.searchsorted(sk, raw), sk.size - 1)
            hit = sk[at] == raw
            return ss[at][hit] + sum(rows[:t])
        legs = []
        for b_, db in zip(batches, dbs):
            P_ = int(b_.seq_lengths.sum())
            off = np.concatenate([[0], np.cumsum(b_.lengths.astype(np.int64))[:-1]])
            legs.append(dict(
                db=db, P=P_, off=torch.from_numpy(off).to(dev),
                gp=torch.from_numpy(rng.standard_normal((B, T * 16)).astype(np.float32)).to(dev),
                gs=torch.from_numpy(rng.standard_normal((3, P_, 16)).astype(np.float32)).to(dev)))
        wsb = max(R.rec_embbag_adagrad_workspace_bytes(T, B, L["db"].nnz, L["P"]) for L in legs)
        aws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        st = list(synth.SEQ_KEYS)

        def adagrad_call(L):
            db = L["db"]
            R.rec_embbag_adagrad(atabs, T, B, db.values, db.lengths, L["off"], db.nnz, L["gp"], st,
                                 db.seq_values, db.seq_stride, L["P"], L["gs"], 1e-3, 1e-10, aws,
                                 wsb, stream=stream)

        reps_a = 40
        with torch.cuda.stream(stream):
            for r in range(4):
                adagrad_call(legs[r % nb])
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(reps_a)]
            torch.cuda._sleep(40_000_000)
            for r in range(reps_a):
                evs[r][0].record(stream)
                adagrad_call(legs[r % nb])
                evs[r][1].record(stream)
            torch.cuda.synchronize()
        d = np.array([s_.elapsed_time(e_) * 1e3 for s_, e_ in evs])
        # algorithmic work of the average batch: reads, bags and distinct rows
        reads, touched = [], []
        for b_ in batches:
            starts = np.concatenate([[0], np.cumsum(b_.lengths.astype(np.int64))])
            keys = []
            for t in range(T):
                keys.append(flat_rows(t, b_.values[starts[t * B]: starts[(t + 1) * B]]))
            Pb = int(b_.seq_lengths.sum())
            for k, t in enumerate(st):
                keys.append(flat_rows(t, b_.seq_values[k, :Pb]))
            keys = np.concatenate(keys)
            reads.append(keys.size)
            touched.append(np.unique(keys).size)
        n_reads, n_rows = float(np.mean(reads)), float(np.mean(touched))
        a_bytes = (n_reads * ADAGRAD_BYTES_PER_READ + T * B * ADAGRAD_BYTES_PER_BAG
                   + n_rows * ADAGRAD_BYTES_PER_ROW)
        a_us = float(d.mean())
        total_rows = sum(rows)
        passes = (int(total_rows).bit_length() + 7) // 8       # the sort covers 0 .. total_rows
        adagrad = {"entry": "rec_embbag_adagrad (row keys, radix sort, chunk sums + AdaGrad, "
                            "cross-chunk runs)",
                   "avg_call_us": round(a_us, 3), "median_call_us": round(float(np.median(d)), 3),
                   "reads": n_reads, "distinct_rows": n_rows,
                   "algorithmic_bytes": a_bytes,
                   "algorithmic_gb_s": round(a_bytes / (a_us * 1e-6) / 1e9, 1),
                   "hbm_frac": round(a_bytes / (a_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "traffic": load_traffic(["k_bwd_keys", "k_bwd_chunks", "k_bwd_cross"]
                                           + ["k_sort_hist", "k_sort_scan", "k_sort_scatter"] * passes,
                                           shash, cfg.name),
                   "sort_passes": passes}
        print(f"[bench] backward + AdaGrad: {a_us:.2f} us per call ({n_reads:.0f} reads, "
              f"{n_rows:.0f} rows)", file=sys.stderr, flush=True)
        del aw, aa, akd, aws, legs

    din_bwd = None
    if not a.no_din_bwd:
        # The attention's backward beside the step: random output gradients
        # [B,48] through rec_din_attn_bwd (query and sequence-row gradients and
        # the six MLP weight gradients), plain (unpacked) weights.
        rng = np.random.default_rng(777)
        b0, db0, f0 = batches[0], dbs[0], fwds[0]
        Pb = int(b0.seq_lengths.sum())
        offs0 = torch.from_numpy(np.concatenate([[0], np.cumsum(b0.seq_lengths.astype(np.int64))[:-1]])).to(dev)
        mlp_plain = PL.DeviceMLP(model, dev, packed=False)
        gatt = torch.from_numpy(rng.standard_normal((B, 48)).astype(np.float32)).to(dev)
        gq = torch.empty(B, 48, dtype=torch.float32, device=dev)
        gs = torch.empty(3, max(db0.seq_stride, 1), 16, dtype=torch.float32, device=dev)
        wg = [torch.empty(sh, dtype=torch.float32, device=dev)
              for sh in ((256, 192), (256,), (64, 256), (64,), (64,), (1,))]
        wsb_d = R.rec_din_attn_bwd_workspace_bytes(db0.seq_stride, True)
        ws_d = torch.empty(wsb_d, dtype=torch.uint8, device=dev)
        seq_arr = tabs.array(list(synth.SEQ_KEYS))

        def din_bwd_call():
            R.rec_din_attn_bwd(seq_arr, db0.seq_values, db0.seq_stride, offs0, db0.seq_lengths,
                               cfg.max_len, B, f0.pooled, f0.T * 16, synth.QUERY_COL, mlp_plain.desc,
                               gatt, gq, gs, *wg, workspace=ws_d, workspace_bytes=wsb_d,
                               stream=stream)

        with torch.cuda.stream(stream):
            for _ in range(2):
                din_bwd_call()
            torch.cuda.synchronize()
            reps_d = 10
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(reps_d)]
            torch.cuda._sleep(20_000_000)
            for r in range(reps_d):
                evs[r][0].record(stream)
                din_bwd_call()
                evs[r][1].record(stream)
            torch.cuda.synchronize()
        d = np.array([s_.elapsed_time(e_) * 1e3 for s_, e_ in evs])
        d_us = float(d.mean())
        Pv = float(np.minimum(b0.seq_lengths, cfg.max_len).sum())
        # per position: the forward once (kept for the backward), the
        # backward's two products, and the weight-gradient products
        d_flops = Pv * (DIN_FLOPS_PER_POS + 2 * (64 * 256 + 256 * 192) + 2 * (256 * 193 + 64 * 257 + 65))
        din_bwd = {"entry": "rec_din_attn_bwd (query, sequence-row and MLP weight gradients)",
                   "avg_call_us": round(d_us, 2), "positions": Pv, "samples": B,
                   "flops_per_call": d_flops, "achieved_tflops": round(d_flops / (d_us * 1e-6) / 1e12, 2),
                   "peak": FP32_PEAK_TFLOPS, "frac": round(d_flops / (d_us * 1e-6) / 1e12 / FP32_PEAK_TFLOPS, 4),
                   "bound": "fp32 matrix cores (v_mfma_f32_16x16x4f32): 32 positions per workgroup, "
                            "weight gradients as LDS-tiled vector products",
                   "traffic": load_traffic(["k_dinb_prep", "k_dinb_map",
                                            "k_dinb_fwd", "k_dinb_soft", "k_dinb_bwdt", "k_dinb_gq",
                                            "k_dinb_wgrad", "k_dinb_reduce"], shash, cfg.name)}
        print(f"[bench] DIN attention backward: {d_us:.1f} us per call ({Pv:.0f} positions)",
              file=sys.stderr, flush=True)
        del gatt, gq, gs, wg, ws_d

    interaction = None
    if not a.no_interaction:
        # The DLRM interaction layer at the pages' measured shape (the DLRM
        # essay §3.1: 217 vectors of width 96 per sample; 1.8 ms per forward on
        # a V100 with the batch not given, context only), over 4096 samples.
        Bi, Fi, di = 4096, 217, 96
        npairs = Fi * (Fi + 1) // 2
        zi = torch.randn(Bi, Fi, di, dtype=torch.float32, device=dev)
        oi = torch.empty(Bi, npairs, dtype=torch.float32, device=dev)
        with torch.cuda.stream(stream):
            for _ in range(3):
                R.rec_dlrm_interact(zi, Bi, Fi, di, oi, stream=stream)
            torch.cuda.synchronize()
        i_us = timed(lambda r: R.rec_dlrm_interact(zi, Bi, Fi, di, oi, stream=stream),
                     {"interact": R.REC_TIME_DLRM_INTERACT}, 20)[0]["interact"]["mean"]
        i_flops = 2.0 * di * npairs * Bi
        i_bytes = 4.0 * (Fi * di + npairs) * Bi
        interaction = {"entry": "rec_dlrm_interact (upper triangle with the diagonal of Z Z^T)",
                       "samples": Bi, "vectors": Fi, "width": di, "avg_call_us": round(i_us, 3),
                       "us_per_sample": round(i_us / Bi, 4),
                       "achieved_tflops": round(i_flops / (i_us * 1e-6) / 1e12, 2),
                       "fp32_peak_tflops": FP32_PEAK_TFLOPS,
                       "mfma_frac": round(i_flops / (i_us * 1e-6) / 1e12 / FP32_PEAK_TFLOPS, 4),
                       "algorithmic_gb_s": round(i_bytes / (i_us * 1e-6) / 1e9, 1),
                       "hbm_frac": round(i_bytes / (i_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                       "traffic": load_traffic(["k_dlrm_interact"], shash, cfg.name),
                       "pages": "1.8 ms per forward on a V100, batch not given (context, another machine)"}
        print(f"[bench] DLRM interaction: {i_us:.1f} us for {Bi} samples of {Fi} x {di}",
              file=sys.stderr, flush=True)
        del zi, oi

    dlrm = None
    if not a.no_dlrm:
        # The DLRM essay's example model (§4.2: 13 dense features, 8 tables of
        # 100000 .. 500 rows, width 96, bottom 13-128-96, top 45-128-64-1) over
        # B = 8192 samples with bags of 1-5 ids, by rec_dlrm_fwd.
        dcfg = synth.DLRM_WORKLOADS[1]
        dm = synth.make_dlrm(dcfg)
        dbt = synth.make_dlrm_batch(dm)
        to = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # noqa: E731
        keep = [to(t) for t in dm.tables] + [to(getattr(dm, k)) for k in
                                            ("wb1", "bb1", "wb2", "bb2", "wt1", "bt1", "wt2", "bt2", "wt3")]
        S_, d_ = len(dm.tables), dcfg.dim
        dmlp = R.dlrm_mlp(dcfg.n_dense, d_, S_, *keep[S_:], dm.bt3)
        dtabs = [R.table(R.REC_DIRECT, t.shape[0], keep[i], dim=d_) for i, t in enumerate(dm.tables)]
        Bd = dbt.B
        doff = to(np.concatenate([[0], np.cumsum(dbt.lengths.astype(np.int64))[:-1]]))
        dd, dv, dl = to(dbt.dense), to(dbt.values), to(dbt.lengths)
        zbuf = torch.empty(Bd, S_ + 1, d_, dtype=torch.float32, device=dev)
        lg, pr = torch.empty(Bd, dtype=torch.float32, device=dev), torch.empty(Bd, dtype=torch.float32, device=dev)

        def dlrm_call(r=0):
            R.rec_dlrm_fwd(dmlp, dtabs, list(dm.modes), Bd, dd, dv, dl, doff, zbuf, None, lg, pr,
                           stream=stream)
        with torch.cuda.stream(stream):
            for _ in range(3):
                dlrm_call()
            torch.cuda.synchronize()
        dk, dcall = timed(dlrm_call, {"fwd": R.REC_TIME_DLRM_FWD}, 40)
        nnz_d = float(dbt.values.size)
        F_ = S_ + 1
        np_ = F_ * (F_ + 1) // 2
        # algorithmic bytes: ids, rows, lengths and offsets, dense inputs, z out,
        # logit and probability out (the weights, read once, are negligible)
        d_bytes = (nnz_d * (8 + 4 * d_) + S_ * Bd * (4 + 8) + Bd * dcfg.n_dense * 4
                   + Bd * F_ * d_ * 4 + Bd * 8)
        d_flops = Bd * 2.0 * (dcfg.n_dense * 128 + 128 * d_ + np_ * d_ + np_ * 128 + 128 * 64 + 64)
        fwd_us = dk["fwd"]["mean"]
        dlrm = {"entry": "rec_dlrm_fwd (bags of width 96, bottom MLP, interaction, top MLP: one launch)",
                "workload": f"{dcfg.name}: B={Bd}, 13 dense, tables {list(dcfg.sizes)} of width {d_}, "
                            f"bags 1-{dcfg.bag_max} ids, sum pooling",
                "call_us": dcall, "kernel_us": dk["fwd"],
                "samples_s": round(Bd / (fwd_us * 1e-6), 1),
                "algorithmic_bytes": d_bytes, "flops": d_flops,
                "gb_s": round(d_bytes / (fwd_us * 1e-6) / 1e9, 1),
                "hbm_frac": round(d_bytes / (fwd_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "tflops": round(d_flops / (fwd_us * 1e-6) / 1e12, 2),
                "bound": "HBM (random 384-byte rows) and the per-workgroup weight stream from L2",
                "traffic": load_traffic(["k_dlrm_fwd"], shash, cfg.name)}
        print(f"[bench] DLRM forward: {fwd_us:.1f} us per launch ({dcall['mean']:.1f} us per call), "
              f"{dlrm['gb_s']:.0f} GB/s of algorithmic bytes", file=sys.stderr, flush=True)
        del keep, zbuf

    dlrm_wide = None
    if not a.no_dlrm:
        # The interaction's measured shape as a whole model: 216 tables of width
        # 96 and the dense vector (217 features), B = 4096; z and the
        # interaction output go through memory.
        wcfg = synth.DLRM_WORKLOADS[3]
        wm = synth.make_dlrm(wcfg)
        wb = synth.make_dlrm_batch(wm)
        to = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # noqa: E731
        wkeep = [to(t) for t in wm.tables] + [to(getattr(wm, k)) for k in
                                              ("wb1", "bb1", "wb2", "bb2", "wt1", "bt1", "wt2", "bt2", "wt3")]
        Sw, dw = len(wm.tables), wcfg.dim
        Fw = Sw + 1
        npw = Fw * (Fw + 1) // 2
        wmlp = R.dlrm_mlp(wcfg.n_dense, dw, Sw, *wkeep[Sw:], wm.bt3)
        wtabs = [R.table(R.REC_DIRECT, t.shape[0], wkeep[i], dim=dw) for i, t in enumerate(wm.tables)]
        Bw = wb.B
        woff = to(np.concatenate([[0], np.cumsum(wb.lengths.astype(np.int64))[:-1]]))
        wd, wv, wl = to(wb.dense), to(wb.values), to(wb.lengths)
        wz = torch.empty(Bw, Fw, dw, dtype=torch.float32, device=dev)
        wi = torch.empty(Bw, npw, dtype=torch.float32, device=dev)
        wlg, wpr = torch.empty(Bw, dtype=torch.float32, device=dev), torch.empty(Bw, dtype=torch.float32, device=dev)

        def wide_call(r=0):
            R.rec_dlrm_fwd(wmlp, wtabs, list(wm.modes), Bw, wd, wv, wl, woff, wz, wi, wlg, wpr,
                           stream=stream)
        with torch.cuda.stream(stream):
            for _ in range(2):
                wide_call()
            torch.cuda.synchronize()
        wk, wcall = timed(wide_call, {"top": R.REC_TIME_DLRM_FWD}, 10)
        w_flops = Bw * 2.0 * (wcfg.n_dense * 128 + 128 * dw + npw * dw + npw * 128 + 128 * 64 + 64)
        dlrm_wide = {"entry": "rec_dlrm_fwd, wide model (z and the interaction through memory)",
                     "workload": f"{wcfg.name}: B={Bw}, 216 tables of {wcfg.sizes[0]} rows, width {dw}, "
                                 f"bags 1-{wcfg.bag_max} ids, {npw} pairs per sample",
                     "call_us": wcall, "top_mlp_us": wk["top"],
                     "samples_s": round(Bw / (wcall["mean"] * 1e-6), 1),
                     "flops": w_flops, "tflops": round(w_flops / (wcall["mean"] * 1e-6) / 1e12, 2),
                     "pages": "1.8 ms per forward of the 217 x 96 interaction on a V100, batch not given "
                              "(context, another machine)"}
        print(f"[bench] DLRM wide (217 features): {wcall['mean']:.1f} us per call of {Bw} samples "
              f"(top MLP {wk['top']['mean']:.1f} us)", file=sys.stderr, flush=True)
        del wkeep, wz, wi

    # `value` is whole-job throughput: with batches in flight on several
    # streams when that is faster (every step is still one whole pass over one
    # resident batch).
    single = {"ms_per_step": round(ms_per_step, 5), "gpu_ms_per_step": round(gpu_ms, 5),
              "samples_s": round(B / (ms_per_step * 1e-3), 1)}
    streams, rotating = 1, len(dbs)
    if two_stream is not None and two_stream["ms_per_step"] < ms_per_step:
        streams = two_stream["streams"]
        rotating = two_stream["rotating_batches"]
        ms_per_step = two_stream["ms_per_step"]
        gpu_ms = two_stream["gpu_ms_per_step"]
    value = B / (ms_per_step * 1e-3)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic: seeded Taobao-shaped ids, tables N(0,0.05), Xavier MLP",
        "config": {"workload": f"{cfg.name}: {synth.describe(cfg)}",
                   "global_batch": B, "parallelism": "single GPU",
                   "graph_replay": graph is not None, "rotating_batches": rotating,
                   "streams": streams,
                   "plan_on_side_stream": side is not None,
                   "entry": "separate calls" if (a.calls or side is not None) else "rec_sparse_din_fwd"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "gpu_ms_per_step": round(gpu_ms, 5),
        "single_stream": single,
        "batches_in_flight": list(in_flight.values()),
        "kernels_us": kern_us,
        "calls_us": call_us,
        "warm": {"step_us": warm_step, "step_timing": step_timing, **warm_rates},
        "host_inputs": pcie,
        "cold": {"step_us": cold_step, "kernels_us": cold_us, "calls_us": cold_calls, **cold_rates,
                 "flush": "1 GiB read before each step (L2s and the 256 MB MALL evicted)"},
        "copy_peak": copy_peak,
        "algorithmic": {"gather_bytes": emb_bytes + plan_bytes, "embbag_bytes": emb_bytes,
                        "plan_bytes": plan_bytes, "din_bytes": din_bytes, "din_flops": din_flops},
        "towers": towers,
        "hash_rebuild": rebuild,
        "hash_admit": admit,
        "adagrad": adagrad,
        "din_bwd": din_bwd,
        "dlrm_interaction": interaction,
        "dlrm_forward": dlrm,
        "dlrm_wide": dlrm_wide,
        "src_hash": shash,
    }
    if a.calibrate_copy:
        # counter calibration: a streaming copy (CAL_BYTES read, CAL_BYTES
        # written) and a gather of CAL_ROWS random 64-byte rows of a 192 MB
        # table (CAL_ROWS * 64 bytes read, as many written)
        src = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        g = torch.Generator(device="cpu").manual_seed(5)
        table = torch.rand(CAL_TABLE_ROWS, 16, generator=g).to(dev)
        idx = torch.randint(0, CAL_TABLE_ROWS, (CAL_ROWS,), generator=g).to(dev)
        rows_out = torch.empty(CAL_ROWS, 16, dtype=torch.float32, device=dev)
        for _ in range(3):
            torch.index_select(table, 0, idx, out=rows_out)
        torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
