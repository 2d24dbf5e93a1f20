"""ctypes binding of libstarpeaks.so (include/star_peaks.h): the measured
peaks that bench.py reads the attention kernels against, beside the published
ones. Argument marshalling only; the probes are HIP kernels.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .binding import StarAttnError

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libstarpeaks.so")
SINK_BYTES = 4096

EXPORTS = ("star_peak_mfma_bf16", "star_peak_hbm_read", "star_peak_exp")

# published MI355X figures the probes are read against
SPEC_BF16_TFLOPS = 2500.0          # dense bf16 MFMA at 2.4 GHz
CHIP_FLOP_PER_CLOCK = 256 * 4 * 1024  # CUs x SIMDs x bf16 FLOP per SIMD per clock

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libstarpeaks.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m long_context_attention_phase1_amd.build`")
    lib = ctypes.CDLL(path)
    I32, P, D, Z = ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), \
        ctypes.POINTER(ctypes.c_size_t)
    for name, args in (("star_peak_mfma_bf16", [I32, I32, P, D, P]),
                       ("star_peak_hbm_read", [P, ctypes.c_size_t, I32, P, D, Z, P]),
                       ("star_peak_exp", [I32, I32, P, D, P])):
        f = getattr(lib, name)
        f.restype, f.argtypes = ctypes.c_int, args
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise StarAttnError(status, where)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _sink(device):
    return torch.empty(SINK_BYTES // 4, dtype=torch.int32, device=device)


def mfma_bf16_tflops(iters: int = 4096, reps: int = 10, device="cuda") -> float:
    sink, out = _sink(device), ctypes.c_double()
    _check(load_library().star_peak_mfma_bf16(iters, reps, ctypes.c_void_p(sink.data_ptr()),
                                              ctypes.byref(out), _stream()),
           "star_peak_mfma_bf16")
    return out.value


def hbm_read_gbs(buf: torch.Tensor, reps: int = 20):
    """(GB/s, bytes read) of a non-temporal read stream over `buf` (device)."""
    if not buf.is_cuda:
        raise ValueError("buf must be a device tensor")
    sink, out, nb = _sink(buf.device), ctypes.c_double(), ctypes.c_size_t()
    _check(load_library().star_peak_hbm_read(ctypes.c_void_p(buf.data_ptr()),
                                             buf.numel() * buf.element_size(), reps,
                                             ctypes.c_void_p(sink.data_ptr()), ctypes.byref(out),
                                             ctypes.byref(nb), _stream()),
           "star_peak_hbm_read")
    return out.value, nb.value


def exp_gps(iters: int = 4096, reps: int = 10, device="cuda") -> float:
    sink, out = _sink(device), ctypes.c_double()
    _check(load_library().star_peak_exp(iters, reps, ctypes.c_void_p(sink.data_ptr()),
                                        ctypes.byref(out), _stream()),
           "star_peak_exp")
    return out.value


def measure(device="cuda", nbytes: int = 1 << 30) -> dict:
    """All three probes. The read stream runs over a buffer of `nbytes` (1 GiB
    by default: four times the 256 MB last-level cache, so HBM serves it)."""
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    tf = mfma_bf16_tflops(device=buf.device)
    gbs, nb = hbm_read_gbs(buf)
    return {
        "mfma_bf16": {"value": tf, "unit": "TFLOP/s",
                      "probe": "v_mfma_f32_32x32x16_bf16, register operands, 8 waves per CU"},
        "mfma_clock_ghz": tf * 1e12 / CHIP_FLOP_PER_CLOCK / 1e9,
        "hbm_read": {"value": gbs, "unit": "GB/s", "bytes": nb,
                     "probe": "non-temporal 16-byte loads, 4 waves per CU"},
        "v_exp_f32": {"value": exp_gps(device=buf.device), "unit": "G/s"},
    }
