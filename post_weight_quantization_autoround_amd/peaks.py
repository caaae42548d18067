"""Measured peaks of the GPU (libarpeaks, include/ar_peaks.h): a streaming
device copy, a read-only stream and a register-only bf16 MFMA loop, each
timed with HIP events.
They are the on-box denominators shown beside AMD's published peaks (HBM3E
8 TB/s, dense bf16 MFMA 2.5 PFLOP/s) for the benchmark's roofline fractions.

    python -m post_weight_quantization_autoround_amd.peaks          # peaks
    python -m post_weight_quantization_autoround_amd.peaks --blas   # library GEMM yardstick
"""
from __future__ import annotations

import ctypes
import json
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
PROBE_PATH = os.path.join(_PKG, "libarpeaks.so")


def _lib() -> ctypes.CDLL:
    if not os.path.exists(PROBE_PATH):
        raise ImportError(f"{PROBE_PATH} is missing: build it with `python post_weight_quantization_autoround_amd/build.py`")
    lib = ctypes.CDLL(PROBE_PATH)
    lib.ar_peak_copy_gbs.restype = ctypes.c_int
    lib.ar_peak_copy_gbs.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(ctypes.c_double)]
    lib.ar_peak_read_gbs.restype = ctypes.c_int
    lib.ar_peak_read_gbs.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(ctypes.c_double)]
    lib.ar_peak_mfma_tflops.restype = ctypes.c_int
    lib.ar_peak_mfma_tflops.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_double)]
    return lib


def copy_gbs(nbytes: int = 1 << 30, reps: int = 20) -> float:
    """GB/s of bytes read plus bytes written by a device copy of `nbytes`."""
    out = ctypes.c_double(0.0)
    rc = _lib().ar_peak_copy_gbs(nbytes, reps, ctypes.byref(out))
    if rc != 0:
        raise RuntimeError(f"ar_peak_copy_gbs failed with HIP error {rc}")
    return out.value


def read_gbs(nbytes: int = 1 << 30, reps: int = 20) -> float:
    """GB/s of bytes read by a read-only stream over `nbytes`."""
    out = ctypes.c_double(0.0)
    rc = _lib().ar_peak_read_gbs(nbytes, reps, ctypes.byref(out))
    if rc != 0:
        raise RuntimeError(f"ar_peak_read_gbs failed with HIP error {rc}")
    return out.value


def mfma_tflops(iters: int = 20000) -> float:
    """TFLOP/s of back-to-back v_mfma_f32_32x32x16_bf16 on every SIMD."""
    out = ctypes.c_double(0.0)
    rc = _lib().ar_peak_mfma_tflops(iters, ctypes.byref(out))
    if rc != 0:
        raise RuntimeError(f"ar_peak_mfma_tflops failed with HIP error {rc}")
    return out.value


def measure() -> dict:
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("the peak probe needs a GPU")
    return {"copy_GB/s": round(copy_gbs(), 1), "read_GB/s": round(read_gbs(), 1),
            "mfma_bf16_TFLOP/s": round(mfma_tflops(), 1),
            "copy": "1 GiB device copy, nontemporal 16-byte loads/stores, 16 workgroups per CU, mean of 20; read + written bytes",
            "read": "1 GiB read-only stream, global_load_lds_dwordx4 into LDS, one 512-thread workgroup per CU, mean of 20",
            "mfma": "v_mfma_f32_32x32x16_bf16, 4 independent accumulators per wavefront, 2 wavefronts per SIMD, register operands"}


# GEMM shapes (M, N, K) of the tuning steps, C[M, N] = A[M, K] B[K, N]: the
# 4096 x 4096 layer's forward and weight gradient at 2048 tokens, the
# 70B-shaped block's gate/up forward, dh2 and gate weight gradient at 1024
# tokens, the 7B-shaped block's gate/up forward, and a square reference.
YARDSTICK_SHAPES = [(2048, 4096, 4096), (4096, 4096, 2048), (1024, 57344, 8192), (1024, 8192, 57344),
                    (28672, 8192, 1024), (2048, 22016, 4096), (8192, 8192, 8192)]


def blas_yardstick(reps: int = 20) -> list:
    """The vendor library's bf16 GEMM (torch.mm, contiguous operands, no
    epilogue) on the tuning steps' shapes, for comparison only: it is never
    on the library's path.  Mean of `reps` launches between HIP events."""
    import torch

    out = []
    for m, n, k in YARDSTICK_SHAPES:
        a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16)
        c = torch.mm(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.mm(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out.append({"M": m, "N": n, "K": k, "us": round(us, 1), "PFLOP/s": round(2.0 * m * n * k / us * 1e-9, 3)})
        del a, b, c
    return out


if __name__ == "__main__":
    import sys

    if "--blas" in sys.argv:
        print(json.dumps(blas_yardstick()), flush=True)
    else:
        print(json.dumps(measure()), flush=True)
