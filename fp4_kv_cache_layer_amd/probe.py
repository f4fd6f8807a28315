"""Measured peaks for the roofline figures (libcsa2_probe.so, include/csa2_probe.h).

The vendor peaks (8 TB/s HBM, 5.0 PFLOP/s dense FP8) are what a kernel's
fraction is quoted against; these probes measure what plain kernels of known
work reach on the same part, so the fraction can also be stated against
what is achievable.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2_probe.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "csa2_probe.h")
MFMA_FLOP = 2 * 16 * 16 * 128          # one V_MFMA_SCALE_F32_16X16X128_F8F6F4

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m fp4_kv_cache_layer_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.csa2_probe_mfma_fp8.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_void_p]
        lib.csa2_probe_mfma_fp8.restype = ctypes.c_int32
        lib.csa2_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p,
                                               ctypes.c_void_p]
        lib.csa2_probe_stream_read.restype = ctypes.c_int32
        _lib = lib
    return _lib


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise RuntimeError(f"{fn} returned hipError {rc}")


def _best_ms(launch, reps: int) -> float:
    """Shortest of `reps` event-timed launches on the current stream (after one warm-up)."""
    from . import ops                                  # timing events without the system-scope fence
    launch()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = ops.HipEvent(), ops.HipEvent()
        e0.record()
        launch()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_ms(e1))
    return best


def mfma_fp8_tflops(epilogue: bool = False, waves_per_simd: int = 4, iters: int = 4096, reps: int = 5) -> float:
    """FP8 MFMA rate in TFLOP/s: 4 waves per workgroup (one per SIMD),
    waves_per_simd workgroups per CU, `iters` MFMAs per wave."""
    lib = load()
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    blocks = cus * waves_per_simd
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def launch():
        _check("csa2_probe_mfma_fp8", lib.csa2_probe_mfma_fp8(blocks, iters, int(epilogue), sink.data_ptr(), stream))

    ms = _best_ms(launch, reps)
    return blocks * 4 * iters * MFMA_FLOP / (ms * 1e-3) / 1e12


def stream_read_gbps(buf: torch.Tensor, nbytes: int, rotate: int = 1, reps: int = 8) -> float:
    """HBM read rate in GB/s over `nbytes` of the uint8 device buffer `buf`;
    with rotate > 1, successive launches read successive nbytes slices of it
    (the first rotate * nbytes bytes), so no launch finds its data in the
    last-level cache."""
    lib = load()
    assert buf.is_cuda and buf.dtype == torch.uint8 and buf.numel() >= rotate * nbytes and nbytes % 16 == 0
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    state = {"i": 0}

    def launch():
        src = buf.data_ptr() + (state["i"] % rotate) * nbytes
        state["i"] += 1
        _check("csa2_probe_stream_read", lib.csa2_probe_stream_read(src, nbytes, cus * 16, sink.data_ptr(), stream))

    ms = _best_ms(launch, reps)
    return nbytes / (ms * 1e-3) / 1e9
