"""Summaries of rocprofv3 output for the tuning step, and the HBM-traffic
figure the benchmark reports.

    python -m post_weight_quantization_autoround_amd.profiling kernel-stats \\
        RUN_kernel_stats.csv --cmd "<rocprofv3 command>" > profiles/<name>.txt
    python -m post_weight_quantization_autoround_amd.profiling traffic \\
        FETCH_counter_collection.csv WRITE_counter_collection.csv \\
        --cmd-fetch "<command>" --cmd-write "<command>" > profiles/<name>.txt
    python -m post_weight_quantization_autoround_amd.profiling counters \\
        A_counter_collection.csv B_counter_collection.csv \\
        --cmd-a "<command>" --cmd-b "<command>" > profiles/<name>.txt

Traffic: rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE give KiB per dispatch.  Each
counter is scaled by the ratio between the known size of a plain 256 MiB
device copy (which bench.py runs after its timed region) and what the same
counter reads for that copy.  The summary records a hash of the sources the
tuning-step kernels are built from; bench.py reports the traffic only while
those sources still match.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CALIB_KIB = 256 * 1024          # the benchmark's calibration copy: 256 MiB read and written


# the files the tuning step's kernels and their launch configuration come from
STEP_SOURCES = ("ar_internal.h", "gemm_tiles.h", "gemm_kernels.hip", "qdq_kernels.hip", "tune_kernels.hip",
                "runtime.hip")


def kernel_source_hash() -> str:
    """SHA-256 (first 16 hex digits) over the sources of the tuning-step kernels."""
    h = hashlib.sha256()
    for p in [os.path.join(PKG, "csrc", f) for f in STEP_SOURCES]:
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def role(kernel_name: str) -> str:
    """Name of the tuning-step kernel a demangled symbol implements."""
    m = re.search(r"gemm_(bf16|f32)(_dma)?_kernel<([^>]*)>", kernel_name)
    if m:
        # template arguments: BM, BN, BK, NWM, NWN, [STAGES,] EPI[, KPRE]
        epi = int(m.group(3).split(",")[6 if m.group(2) else 5])
        return {0: "gemm_store (reference output / weight gradient)", 1: "gemm_fwd_loss",
                2: "gemm_wgrad_ste_update"}.get(epi, "gemm")
    for key, name in [("qdq_kernel", "qdq_fwd"), ("ste_seg_kernel", "ste_bwd"), ("ste_group_kernel", "ste_bwd"),
                      ("signsgd_kernel", "signsgd_update"), ("loss_decide_kernel", "loss_decide"),
                      ("swiglu_fwd_kernel", "swiglu_fwd"), ("swiglu_bwd_kernel", "swiglu_bwd"),
                      ("transpose_pool_kernel", "transpose"), ("transpose_b16_kernel", "transpose"),
                      ("transpose2d_kernel", "transpose"), ("w4a16_gemm_kernel", "w4a16_gemm"),
                      ("w4a16_skinny_kernel", "w4a16_gemm_decode"), ("rmsnorm_fwd_kernel", "rmsnorm_fwd"),
                      ("rmsnorm_bwd_kernel", "rmsnorm_bwd"), ("rope_fwd_kernel", "rope_fwd"),
                      ("rope_bwd_kernel", "rope_bwd"), ("attn_fwd_kernel", "attn_fwd"),
                      ("attn_prep_bwd_kernel", "attn_bwd_prep"), ("attn_bwd_dq_kernel", "attn_bwd_dq"),
                      ("attn_bwd_dkdv_kernel", "attn_bwd_dkdv"), ("yref_combine_kernel", "loss_target"),
                      ("add_rows_kernel", "add_rows"), ("w4a16_decode_kernel", "w4a16_gemm_decode"),
                      ("rmsnorm_fwd_vec_kernel", "rmsnorm_fwd"), ("rmsnorm_bwd_vec_kernel", "rmsnorm_bwd"),
                      ("swiglu_fwd_vec_kernel", "swiglu_fwd"), ("swiglu_bwd_vec_kernel", "swiglu_bwd"),
                      ("yref_combine_vec_kernel", "loss_target")]:
        if key in kernel_name:
            return name
    return ""


def kernel_stats_summary(path: str, cmd: str, top: int = 14, trace: str | None = None) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["# rocprofv3 kernel trace summary (--kernel-trace --stats)", f"# command: {cmd}",
           "# avg_us  calls  share%  step-kernel  symbol"]
    for r in rows[:top]:
        out.append(f"{float(r['AverageNs']) / 1e3:9.2f} {int(r['Calls']):6d} {float(r['Percentage']):6.2f}  "
                   f"{role(r['Name']) or '-':<24s} {r['Name'][:110]}")
    if trace:
        out += context_durations(trace)
    return "\n".join(out) + "\n"


def context_durations(trace_csv: str) -> list:
    """Durations of the two kernels of the layer step split by context, from
    the per-dispatch kernel trace: "in-step" launches alternate with the other
    step kernel (the graph-replayed steps), "repeated" launches follow or
    precede a launch of the same kernel (the benchmark's per-kernel timing:
    a graph of back-to-back launches of one kernel)."""
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    seq = [(role(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows]
    step = ("gemm_fwd_loss", "gemm_wgrad_ste_update")
    durs = collections.defaultdict(list)
    for i, (k, t0, t1) in enumerate(seq):
        if k not in step:
            continue
        nb = [seq[j][0] for j in (i - 1, i + 1) if 0 <= j < len(seq)]
        ctx = "repeated" if k in nb else ("in-step" if any(n in step for n in nb) else "other")
        durs[(k, ctx)].append((t1 - t0) / 1e3)
    out = ["# per-context durations of the step kernels (from the per-dispatch trace)",
           "# step-kernel  context  launches  mean_us  median_us  min_us  max_us"]
    for (k, ctx), v in sorted(durs.items()):
        v = sorted(v)
        out.append(f"context {k} {ctx} {len(v)} {sum(v) / len(v):.2f} {v[len(v) // 2]:.2f} {v[0]:.2f} {v[-1]:.2f}")
    return out


# counter sets of the two --pmc passes (at most 8 SQ counters each) and the
# derived figures, per dispatch, following rocprofv3's own metric
# definitions (MfmaUtil, VALUBusy, LDSBankConflict) with 1024 SIMDs and
# 256 CUs on MI355X
COUNTER_PASSES = {
    "A": ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_WAVES",
          "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"],
    "B": ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS",
          "SQ_LDS_ADDR_CONFLICT", "SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_INSTS_SALU", "GRBM_GUI_ACTIVE"],
}
SIMDS, CUS, XCCS = 1024, 256, 8     # GRBM_GUI_ACTIVE arrives summed over the 8 XCDs


def _counter_means(path: str):
    """{kernel symbol: {counter: mean over dispatches}} (each counter's value
    summed over its dimensions within a dispatch), the dispatch counts and
    the mean dispatch durations in us."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    dur = collections.defaultdict(list)
    seen = set()
    for r in csv.DictReader(open(path)):
        # one symbol serves several problem shapes: keep them apart by grid size
        name = f"{r['Kernel_Name']} [grid {r['Grid_Size']}]"
        per[(name, r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
        if (name, r["Dispatch_Id"]) not in seen:
            seen.add((name, r["Dispatch_Id"]))
            dur[name].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for (name, _), vals in per.items():
        for c, v in vals.items():
            agg[name][c].append(v)
    return {n: {c: sum(v) / len(v) for c, v in cs.items()} for n, cs in agg.items()}, \
        {n: len(next(iter(cs.values()))) for n, cs in agg.items()}, {n: sum(v) / len(v) for n, v in dur.items()}


def _short(name: str, width: int = 90) -> str:
    """A symbol cut to `width` characters, keeping its grid-size suffix."""
    i = name.rfind(" [grid")
    sym, grid = name[:i], name[i:]
    return sym + grid if len(sym) <= width else sym[:width] + "..." + grid


def counter_summary(csv_a: str, csv_b: str, cmd_a: str, cmd_b: str) -> str:
    ma, na, ta = _counter_means(csv_a)
    mb, _, _ = _counter_means(csv_b)
    out = ["# rocprofv3 --pmc counters per dispatch (two passes, means over dispatches)",
           f"# command (pass A: {' '.join(COUNTER_PASSES['A'])}): {cmd_a}",
           f"# command (pass B: {' '.join(COUNTER_PASSES['B'])}): {cmd_b}",
           f"source_hash {kernel_source_hash()}",
           "# cycles = GRBM_GUI_ACTIVE / 8 XCDs; mfma_busy% = SQ_VALU_MFMA_BUSY_CYCLES / (cycles * 1024 SIMDs);"
           " valu_busy% = SQ_ACTIVE_INST_VALU / (256 CUs * cycles) (rocprofv3 VALUBusy); coexec% ="
           " SQ_VALU_MFMA_COEXEC_CYCLES / MFMA busy; lds_bank_conflict% = SQ_LDS_BANK_CONFLICT / (256 CUs * cycles)"
           " (LDSBankConflict);"
           " conflicts/access = SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT);"
           " lds_wait% = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES and lds_active% = SQ_ACTIVE_INST_LDS / SQ_WAVE_CYCLES"
           " (share of the waves' resident cycles spent waiting to issue, and issuing, LDS instructions);"
           " any_active% = SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES",
           "# step-kernel  dispatches  us_per_dispatch  mfma_busy%  valu_busy%  coexec%  lds_bank_conflict%  "
           "conflicts/access  valu_insts/wave  mfma_insts/wave  lds_insts/wave  lds_wait%  lds_active%  any_active%"
           "  symbol"]
    for name in sorted(ma, key=lambda n: -ma[n].get("GRBM_GUI_ACTIVE", 0)):
        r = role(name)
        if not r or name not in mb:
            continue
        a, b = ma[name], mb[name]
        # busy cycles of the dispatch: GRBM_GUI_ACTIVE per XCD (rocprofv3's metrics take its maximum)
        gui_a, gui_b = (a.get("GRBM_GUI_ACTIVE", 0) or XCCS) / XCCS, (b.get("GRBM_GUI_ACTIVE", 0) or XCCS) / XCCS
        waves = a.get("SQ_WAVES", 0) or 1
        mfma = 100 * a.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / (gui_a * SIMDS)
        valu = 100 * a.get("SQ_ACTIVE_INST_VALU", 0) / (CUS * gui_a)
        coex = 100 * a.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0) / max(a.get("SQ_VALU_MFMA_BUSY_CYCLES", 0), 1)
        bank = 100 * b.get("SQ_LDS_BANK_CONFLICT", 0) / (CUS * gui_b)
        cpa = b.get("SQ_LDS_BANK_CONFLICT", 0) / max(b.get("SQ_LDS_IDX_ACTIVE", 0) - b.get("SQ_LDS_BANK_CONFLICT", 0), 1)
        wc = max(b.get("SQ_WAVE_CYCLES", 0), 1)
        lwait = 100 * b.get("SQ_WAIT_INST_LDS", 0) / wc
        lact = 100 * b.get("SQ_ACTIVE_INST_LDS", 0) / wc
        anyact = 100 * b.get("SQ_ACTIVE_INST_ANY", 0) / wc
        out.append(f"kernel {r.split(' ')[0]} {na[name]} {ta[name]:.1f} {mfma:.1f} {valu:.1f} {coex:.1f} {bank:.2f} {cpa:.4f} "
                   f"{a.get('SQ_INSTS_VALU', 0) / waves:.0f} {a.get('SQ_INSTS_MFMA', 0) / waves:.0f} "
                   f"{a.get('SQ_INSTS_LDS', 0) / waves:.0f} {lwait:.1f} {lact:.1f} {anyact:.1f} {_short(name)}")
    return "\n".join(out) + "\n"


def _per_kernel(path: str, counter: str):
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    agg = collections.defaultdict(list)
    for r in rows:
        agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    # the calibration copy is the last device-to-device copy dispatch of the
    # run (torch's same-dtype copy_ of 256 MiB, executed by the runtime's
    # copy kernel after the timed region)
    copies = [float(r["Counter_Value"]) for r in rows if r["Kernel_Name"].startswith("__amd_rocclr_copyBuffer")]
    calib = copies[-1] if copies else None
    return agg, calib


def traffic_summary(fetch_csv: str, write_csv: str, cmd_fetch: str, cmd_write: str) -> str:
    fa, fcal = _per_kernel(fetch_csv, "FETCH_SIZE")
    wa, wcal = _per_kernel(write_csv, "WRITE_SIZE")
    fs = CALIB_KIB / fcal if fcal else 1.0
    ws = CALIB_KIB / wcal if wcal else 1.0
    out = ["# HBM traffic per dispatch from rocprofv3 --pmc (one counter per run)",
           f"# command (FETCH_SIZE): {cmd_fetch}", f"# command (WRITE_SIZE): {cmd_write}",
           f"# calibration: 256 MiB device copy read FETCH_SIZE {fcal} KiB, WRITE_SIZE {wcal} KiB",
           f"fetch_scale {fs:.4f}", f"write_scale {ws:.4f}", f"source_hash {kernel_source_hash()}",
           "# step-kernel  dispatches  fetch_KiB  write_KiB  scaled_MB_read  scaled_MB_written  symbol"]
    for name in sorted(fa, key=lambda n: -sum(fa[n]) / len(fa[n])):
        r = role(name)
        if not r or name not in wa:
            continue
        f = sum(fa[name]) / len(fa[name])
        w = sum(wa[name]) / len(wa[name])
        out.append(f"kernel {r.split(' ')[0]} {len(fa[name])} {f:.1f} {w:.1f} {f * fs * 1024 / 1e6:.2f} "
                   f"{w * ws * 1024 / 1e6:.2f} {name[:100]}")
    return "\n".join(out) + "\n"


def read_traffic(path: str, kernel: str):
    """Scaled HBM bytes per launch (read + written) of `kernel` from a committed
    traffic summary, or None when it is missing or the sources have changed."""
    if not os.path.exists(path):
        return None
    src_hash = None
    for line in open(path):
        parts = line.split()
        if not parts or parts[0].startswith("#"):
            continue
        if parts[0] == "source_hash":
            src_hash = parts[1]
        if parts[0] == "kernel" and parts[1] == kernel:
            if src_hash != kernel_source_hash():
                return None
            return (float(parts[5]) + float(parts[6])) * 1e6
    return None


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("kernel-stats")
    a.add_argument("csv")
    a.add_argument("--cmd", required=True)
    a.add_argument("--top", type=int, default=14)
    a.add_argument("--trace", help="the run's kernel_trace.csv: adds per-context durations of the step kernels")
    c = sub.add_parser("counters")
    c.add_argument("csv_a")
    c.add_argument("csv_b")
    c.add_argument("--cmd-a", required=True)
    c.add_argument("--cmd-b", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("--cmd-fetch", required=True)
    b.add_argument("--cmd-write", required=True)
    args = ap.parse_args(argv)
    if args.what == "kernel-stats":
        sys.stdout.write(kernel_stats_summary(args.csv, args.cmd, args.top, args.trace))
    elif args.what == "counters":
        sys.stdout.write(counter_summary(args.csv_a, args.csv_b, args.cmd_a, args.cmd_b))
    else:
        sys.stdout.write(traffic_summary(args.fetch_csv, args.write_csv, args.cmd_fetch, args.cmd_write))


if __name__ == "__main__":
    main()
