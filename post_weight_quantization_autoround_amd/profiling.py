"""Summaries of rocprofv3 output for the tuning step, and the HBM-traffic
figure the benchmark reports.

    python -m post_weight_quantization_autoround_amd.profiling kernel-stats \\
        RUN_kernel_stats.csv --cmd "<rocprofv3 command>" > profiles/<name>.txt
    python -m post_weight_quantization_autoround_amd.profiling traffic \\
        FETCH_counter_collection.csv WRITE_counter_collection.csv \\
        --cmd-fetch "<command>" --cmd-write "<command>" > profiles/<name>.txt

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


def kernel_stats_summary(path: str, cmd: str, top: int = 14) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["# rocprofv3 kernel trace summary (--kernel-trace --stats)", f"# command: {cmd}",
           "# avg_us  calls  share%  step-kernel  symbol"]
    for r in rows[:top]:
        out.append(f"{float(r['AverageNs']) / 1e3:9.2f} {int(r['Calls']):6d} {float(r['Percentage']):6.2f}  "
                   f"{role(r['Name']) or '-':<24s} {r['Name'][:110]}")
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
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("--cmd-fetch", required=True)
    b.add_argument("--cmd-write", required=True)
    args = ap.parse_args(argv)
    if args.what == "kernel-stats":
        sys.stdout.write(kernel_stats_summary(args.csv, args.cmd, args.top))
    else:
        sys.stdout.write(traffic_summary(args.fetch_csv, args.write_csv, args.cmd_fetch, args.cmd_write))


if __name__ == "__main__":
    main()
