"""Measured peaks of the GPU (libarpeaks, include/ar_peaks.h): a streaming
device copy, a read-only stream and a register-only bf16 MFMA loop, each
timed with HIP events.
They are the on-box denominators shown beside AMD's published peaks (HBM3E
8 TB/s, dense bf16 MFMA 2.5 PFLOP/s) for the benchmark's roofline fractions.

    python -m post_weight_quantization_autoround_amd.peaks
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


if __name__ == "__main__":
    print(json.dumps(measure()), flush=True)
