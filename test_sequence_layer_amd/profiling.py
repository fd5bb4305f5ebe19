"""Summarise rocprofv3 output for one kernel into profiles/.

Given the CSV directories of three rocprofv3 runs of the same benchmark command
(kernel trace with --stats, then --pmc FETCH_SIZE, then --pmc WRITE_SIZE), each
run also executing a plain device copy of known size (bench.py
--copy-calibration: 1 GiB read + 1 GiB written), this writes

  profiles/<kernel>__<workload>.md   average launch time, HBM bytes per launch
  profiles/traffic.json              bytes per launch, keyed by kernel|workload,
                                     with a hash of the kernel's source files so
                                     a stale figure is never reported.

The HBM byte counters are scaled by what they read for the copy kernel:
factor = known bytes / counter bytes (per counter).

    python -m test_sequence_layer_amd.profiling --stats D1 --fetch D2 --write D3 \
        --kernel ttt_linear_mfma_d64b16 --workload l1p3b --algorithmic-bytes N \
        --command "..."
    python -m test_sequence_layer_amd.profiling --counters D --kernel K --workload W \
        --algorithmic-flops F --command "..."      (SQ counter summary)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30

# source files that define each kernel (a change to any of them invalidates its counters)
KERNEL_SOURCES = {
    "ttt_linear_mfma_d64b16": ["linear_mfma.hip", "mfma_common.h", "wave_prio.h", "args_linear.h", "ttt_common.h"],
    "ttt_linear_mfma_head_maps": ["linear_mfma.hip", "mfma_common.h", "wave_prio.h", "args_linear.h", "ttt_common.h"],
    "ttt_linear_mfma_f32_d64b16": ["linear_mfma_f32.hip", "mfma_common.h", "args_linear.h", "ttt_common.h"],
    "ttt_linear_generic_kernel": ["linear_generic.hip", "args_linear.h", "ttt_common.h"],
    "ttt_linear_bwd_d64b16": ["linear_bwd_mfma.hip", "mfma_common.h", "wave_prio.h", "args_bwd.h", "ttt_common.h"],
    "ttt_linear_bwd_generic_kernel": ["linear_bwd_generic.hip", "args_bwd.h", "ttt_common.h"],
    "ttt_linear_ln_bwd_d64b16": ["linear_ln_bwd_mfma.hip", "mfma_common.h", "wave_prio.h", "args_bwd.h", "ttt_common.h"],
    "ttt_linear_ln_bwd_fp32": ["linear_ln_bwd.hip", "args_bwd.h", "ttt_common.h"],
    "ttt_mlp_fwd_d64h256b16": ["mlp.hip", "gelu.h", "mfma_common.h", "wave_prio.h", "args_mlp.h", "ttt_common.h"],
    "ttt_mlp_primal_d64h256": ["mlp_primal.hip", "gelu.h", "mfma_common.h", "args_primal.h", "ttt_common.h"],
    "ttt_mlp_ln_primal_d64h256": ["mlp_primal.hip", "gelu.h", "mfma_common.h", "args_primal.h", "ttt_common.h"],
    "ttt_mlp_bwd_d64h256": ["mlp_bwd.hip", "mfma_common.h", "args_mlp_bwd.h", "ttt_common.h"],
    "ttt_mlp_bwd_d64h256b16": ["mlp_bwd_mfma.hip", "mfma_common.h", "args_mlp_bwd.h", "ttt_common.h"],
    "ttt_linear_primal_kernel": ["linear_primal.hip", "args_primal.h", "ttt_common.h"],
    "ttt_linear_ln_primal_kernel": ["linear_primal.hip", "args_primal.h", "ttt_common.h"],
    "ttt_linear_chunk_scan": ["linear_chunked.hip", "args_linear.h", "ttt_common.h"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel.split("<")[0], []):
        with open(os.path.join(PKG, "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _one(d: str, pattern: str) -> str:
    files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if len(files) != 1:
        raise FileNotFoundError(f"expected one {pattern} under {d}, found {files}")
    return files[0]


def kernel_stats(stats_dir: str, kernel: str):
    """(calls, average ns, min ns) of the kernel from *_kernel_stats.csv."""
    for r in csv.DictReader(open(_one(stats_dir, "*_kernel_stats.csv"))):
        if kernel in r["Name"]:
            return int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), r["Name"]
    raise KeyError(kernel)


def last_launches_avg_ns(stats_dir: str, kernel: str, count: int):
    """Average duration (ns) of the last ``count`` dispatches of the kernel in
    the kernel trace: the launches a benchmark's timed region covers."""
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            for r in sorted(csv.DictReader(open(_one(stats_dir, "*_kernel_trace.csv"))),
                            key=lambda r: int(r["Start_Timestamp"]))
            if kernel in r["Kernel_Name"]]
    if not durs:
        raise KeyError(kernel)
    tail = durs[-count:] if count > 0 else durs
    return sum(tail) / len(tail), len(tail)


def counter_kib(pmc_dir: str, name_substr: str, counter: str):
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(_one(pmc_dir, "*_counter_collection.csv")))
            if name_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise KeyError((name_substr, counter))
    return vals


def summarize(stats_dir, fetch_dir, write_dir, kernel, workload, algorithmic_bytes, command, out_dir=PROFILES,
              timed=0, match=None):
    """``match``: the substring that picks the kernel's rows in the CSVs (default:
    ``kernel``), e.g. a template argument list when one run launches several
    instantiations of one kernel."""
    match = match or kernel
    calls, avg_ns, min_ns, full_name = kernel_stats(stats_dir, match)
    timed_ns, ntimed = last_launches_avg_ns(stats_dir, match, timed)
    fetch = counter_kib(fetch_dir, match, "FETCH_SIZE")
    write = counter_kib(write_dir, match, "WRITE_SIZE")
    cf = counter_kib(fetch_dir, COPY_KERNEL, "FETCH_SIZE")
    cw = counter_kib(write_dir, COPY_KERNEL, "WRITE_SIZE")
    f_fetch = COPY_BYTES / (statistics.median(cf) * 1024)
    f_write = COPY_BYTES / (statistics.median(cw) * 1024)
    rd = statistics.median(fetch) * 1024 * f_fetch
    wr = statistics.median(write) * 1024 * f_write
    total = rd + wr
    os.makedirs(out_dir, exist_ok=True)
    base = f"{kernel}__{workload}"
    md = os.path.join(out_dir, base + ".md")
    with open(md, "w") as fh:
        fh.write(f"# {kernel} -- {workload}\n\n")
        fh.write(f"Kernel symbol: `{full_name}`\n\n")
        fh.write("Commands (run from /tmp with TMPDIR=/tmp; $R is the repository root):\n\n")
        for c in command:
            fh.write(f"    {c}\n")
        fh.write("\n| quantity | value |\n|---|---|\n")
        fh.write(f"| launches traced | {calls} |\n")
        fh.write(f"| average launch duration | {avg_ns / 1e3:.1f} us |\n")
        fh.write(f"| fastest launch | {min_ns / 1e3:.1f} us |\n")
        fh.write(f"| average of the last {ntimed} launches (the benchmark's timed steps) | {timed_ns / 1e3:.1f} us |\n")
        fh.write(f"| FETCH_SIZE per launch (median, raw) | {statistics.median(fetch):.0f} KiB |\n")
        fh.write(f"| WRITE_SIZE per launch (median, raw) | {statistics.median(write):.0f} KiB |\n")
        fh.write(f"| copy calibration (1 GiB copy) FETCH / WRITE raw | "
                 f"{statistics.median(cf):.0f} / {statistics.median(cw):.0f} KiB |\n")
        fh.write(f"| scale factors FETCH / WRITE | {f_fetch:.4f} / {f_write:.4f} |\n")
        fh.write(f"| HBM bytes read per launch | {rd:.4e} |\n")
        fh.write(f"| HBM bytes written per launch | {wr:.4e} |\n")
        fh.write(f"| HBM traffic per launch | {total:.4e} B |\n")
        fh.write(f"| algorithmic bytes per launch | {algorithmic_bytes:.4e} B |\n")
        fh.write(f"| traffic / algorithmic | {total / algorithmic_bytes:.4f} |\n")
        fh.write(f"| achieved (algorithmic bytes / average of the timed launches) | "
                 f"{algorithmic_bytes / timed_ns:.1f} GB/s |\n")
        fh.write(f"| kernel source hash | {source_hash(kernel)} |\n")
    tj = os.path.join(out_dir, "traffic.json")
    db = json.load(open(tj)) if os.path.exists(tj) else {}
    db[f"{kernel}|{workload}"] = {"bytes_per_launch": round(total), "read": round(rd), "write": round(wr),
                                  "avg_launch_us": round(avg_ns / 1e3, 2),
                                  "timed_avg_launch_us": round(timed_ns / 1e3, 2),
                                  "source_hash": source_hash(kernel)}
    with open(tj, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)
    return md


def _kernel_id(symbol: str) -> str:
    """The kernel's own name in a demangled symbol (namespaces, template
    arguments and parameters stripped)."""
    return re.search(r"(ttt_\w+)", symbol.split("(ttt::")[0].replace("(anonymous namespace)", "")).group(1)


def summarize_call(stats_dir, fetch_dir, write_dir, name, parts, algorithmic_bytes, command, out_dir=PROFILES,
                   timed=0):
    """profiles/<name>.md for an entry point that launches several kernels per
    call (``parts``: (label, substring) pairs, one per launch in a call): each
    launch's average duration and scaled HBM bytes, their sums per call, and the
    call's algorithmic bytes over the summed time of the timed calls."""
    cf = counter_kib(fetch_dir, COPY_KERNEL, "FETCH_SIZE")
    cw = counter_kib(write_dir, COPY_KERNEL, "WRITE_SIZE")
    f_fetch = COPY_BYTES / (statistics.median(cf) * 1024)
    f_write = COPY_BYTES / (statistics.median(cw) * 1024)
    rows, t_sum, rd_sum, wr_sum = [], 0.0, 0.0, 0.0
    for label, match in parts:
        calls, avg_ns, _, full_name = kernel_stats(stats_dir, match)
        timed_ns, ntimed = last_launches_avg_ns(stats_dir, match, timed)
        rd = statistics.median(counter_kib(fetch_dir, match, "FETCH_SIZE")) * 1024 * f_fetch
        wr = statistics.median(counter_kib(write_dir, match, "WRITE_SIZE")) * 1024 * f_write
        rows.append((label, full_name, calls, avg_ns, timed_ns, ntimed, rd, wr))
        t_sum, rd_sum, wr_sum = t_sum + timed_ns, rd_sum + rd, wr_sum + wr
    os.makedirs(out_dir, exist_ok=True)
    md = os.path.join(out_dir, name + ".md")
    with open(md, "w") as fh:
        fh.write(f"# {name}\n\n")
        fh.write("Commands (run from /tmp with TMPDIR=/tmp; $R is the repository root):\n\n")
        for c in command:
            fh.write(f"    {c}\n")
        fh.write(f"\nCopy calibration (1 GiB copy) FETCH / WRITE raw: {statistics.median(cf):.0f} / "
                 f"{statistics.median(cw):.0f} KiB; scale factors {f_fetch:.4f} / {f_write:.4f}.\n\n")
        fh.write("| launch | kernel symbol | launches traced | average | average of the timed launches "
                 "| HBM read | HBM written |\n|---|---|---|---|---|---|---|\n")
        for label, full_name, calls, avg_ns, timed_ns, ntimed, rd, wr in rows:
            fh.write(f"| {label} | `{full_name}` | {calls} | {avg_ns / 1e3:.1f} us | {timed_ns / 1e3:.1f} us "
                     f"(last {ntimed}) | {rd:.4e} B | {wr:.4e} B |\n")
        fh.write(f"\n| per call | value |\n|---|---|\n")
        fh.write(f"| summed launch time (timed launches) | {t_sum / 1e3:.1f} us |\n")
        fh.write(f"| HBM traffic | {rd_sum + wr_sum:.4e} B |\n")
        fh.write(f"| algorithmic bytes | {algorithmic_bytes:.4e} B |\n")
        fh.write(f"| traffic / algorithmic | {(rd_sum + wr_sum) / algorithmic_bytes:.4f} |\n")
        fh.write(f"| achieved (algorithmic bytes / summed launch time) | {algorithmic_bytes / t_sum:.1f} GB/s |\n")
        kernels = sorted({_kernel_id(r[1]) for r in rows})
        fh.write(f"| kernel source hashes | {', '.join(f'{k} {source_hash(k)}' for k in kernels)} |\n")
    return md


COUNTER_SET = ("MfmaUtil", "VALUBusy", "LDSBankConflict", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE")


def summarize_counters(pmc_dir, kernel, workload, algorithmic_flops, command, out_dir=PROFILES):
    """Write profiles/<kernel>__<workload>__counters.md from one rocprofv3 --pmc
    run of COUNTER_SET: medians per dispatch, and the MFMA work the kernel
    performed (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts the MFMA's add and multiply
    operations / 512, so x 512 is flops) against its algorithmic flops."""
    med = {}
    for c in COUNTER_SET:
        v = counter_kib(pmc_dir, kernel, c)
        med[c] = statistics.median(v)
    performed = med["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    md = os.path.join(out_dir, f"{kernel}__{workload}__counters.md")
    with open(md, "w") as fh:
        fh.write(f"# {kernel} -- {workload}: SQ counters\n\n")
        fh.write("Commands (run from /tmp with TMPDIR=/tmp; $R is the repository root):\n\n")
        for c in command:
            fh.write(f"    {c}\n")
        fh.write("\n| counter (median per dispatch) | value |\n|---|---|\n")
        fh.write(f"| MfmaUtil (MFMA busy / (GPU active x SIMDs)) | {med['MfmaUtil']:.1f} % |\n")
        fh.write(f"| VALUBusy (VALU instruction cycles / (GPU active x CUs)) | {med['VALUBusy']:.1f} % |\n")
        fh.write(f"| LDSBankConflict (bank-conflict stall / (GPU active x CUs)) | {med['LDSBankConflict']:.1f} % |\n")
        fh.write(f"| GRBM_GUI_ACTIVE (summed over the 8 XCDs) | {med['GRBM_GUI_ACTIVE']:.4e} cycles |\n")
        fh.write(f"| SQ_INSTS_VALU_MFMA_MOPS_BF16 | {med['SQ_INSTS_VALU_MFMA_MOPS_BF16']:.4e} |\n")
        fh.write(f"| bf16 MFMA flops performed (MOPS x 512) | {performed:.4e} |\n")
        fh.write(f"| algorithmic flops | {algorithmic_flops:.4e} |\n")
        fh.write(f"| performed / algorithmic (split passes, padding) | {performed / algorithmic_flops:.2f} |\n")
        fh.write(f"| kernel source hash | {source_hash(kernel)} |\n")
    record_counters(kernel, workload, med, out_dir)
    return md


def record_counters(kernel, workload, med, out_dir=PROFILES, source=None):
    """Keep the medians of one counter run in profiles/counters.json, keyed by
    kernel|workload with the kernel's source hash (bench.py reports the MFMA
    flops performed only while that hash is current)."""
    cj = os.path.join(out_dir, "counters.json")
    db = json.load(open(cj)) if os.path.exists(cj) else {}
    db[f"{kernel}|{workload}"] = {"mfma_util_pct": round(med["MfmaUtil"], 2), "valu_busy_pct": round(med["VALUBusy"], 2),
                                  "lds_bank_conflict_pct": round(med["LDSBankConflict"], 2),
                                  "grbm_gui_active": round(med["GRBM_GUI_ACTIVE"]),
                                  "mfma_flops_performed": round(med["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512),
                                  "source_hash": source or source_hash(kernel)}
    with open(cj, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--counters", help="summarise one --pmc run of COUNTER_SET instead")
    ap.add_argument("--algorithmic-flops", type=float)
    ap.add_argument("--stats")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--kernel")
    ap.add_argument("--workload")
    ap.add_argument("--call", help="summarise every launch of one multi-kernel call into profiles/CALL.md")
    ap.add_argument("--part", action="append", default=[], help="LABEL=SUBSTRING, one per launch of the call")
    ap.add_argument("--algorithmic-bytes", type=float)
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--timed", type=int, default=200, help="launches in the benchmark's timed region")
    ap.add_argument("--match", help="substring that picks the kernel's rows (default: --kernel)")
    a = ap.parse_args()
    if a.call:
        parts = [tuple(p.split("=", 1)) for p in a.part]
        print(summarize_call(a.stats, a.fetch, a.write, a.call, parts, a.algorithmic_bytes, a.command,
                             timed=a.timed))
        return
    if not a.kernel or not a.workload:
        ap.error("--kernel and --workload are required")
    if a.counters:
        print(summarize_counters(a.counters, a.kernel, a.workload, a.algorithmic_flops, a.command))
        return
    print(summarize(a.stats, a.fetch, a.write, a.kernel, a.workload, a.algorithmic_bytes, a.command,
                    timed=a.timed, match=a.match))


if __name__ == "__main__":
    main()
