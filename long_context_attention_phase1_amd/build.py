"""Builds the native libraries in-tree for gfx950 with hipcc.

``python -m long_context_attention_phase1_amd.build`` (or
``__graft_entry__.build()``) compiles
  * ``csrc/star_host.cpp`` + ``csrc/star_kernels.hip`` into ``libstarattn.so``
    (the attention path, include/star_attn.h);
  * ``csrc/star_peaks.hip`` into ``libstarpeaks.so`` (the peak probes that
    bench.py reads the kernels against, include/star_peaks.h).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libstarattn.so")
PEAKS_LIB = os.path.join(PKG, "libstarpeaks.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["star_host.cpp", "star_kernels.hip"]
PEAKS_SOURCES = ["star_peaks.hip"]

# Device code: no packed fp32 ALU ops; IEEE mode off and no NaN operands
# (lets max chains fold into v_max3_f32 without canonicalizing every MFMA
# result). Host code keeps full IEEE semantics (its argument checks test NaN).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Xarch_device", "-mno-amdgpu-ieee", "-Xarch_device", "-fno-honor-nans"]


def command(out: str = LIB, extra=(), sources=SOURCES) -> list:
    return ([HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]
            + DEVICE_FLAGS + list(extra)
            + ["-I", os.path.join(PKG, "..", "include")]
            + [os.path.join(CSRC, s) for s in sources] + ["-o", out])


def _compile(lib: str, sources, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = command(tmp, sources=sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile both libraries (always rebuilds); return the attention library's path."""
    _compile(PEAKS_LIB, PEAKS_SOURCES, verbose)
    return _compile(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
