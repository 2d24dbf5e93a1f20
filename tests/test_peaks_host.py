"""libstarpeaks.so on the CPU: it exports every function include/star_peaks.h
declares, and each probe rejects bad arguments before launching anything
(no kernel runs here)."""
import ctypes
import os
import re
import subprocess

from long_context_attention_phase1_amd import binding as B
from long_context_attention_phase1_amd import peaks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "star_peaks.h")


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(star_[a-z0-9_]+)\s*\(", text)))


def test_peaks_library_exports_every_declared_symbol():
    lib = peaks.load_library()
    names = _declared_functions()
    assert set(names) == set(peaks.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", peaks.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported


def test_peak_probes_validate_before_launching():
    lib = peaks.load_library()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation
    d, z = ctypes.c_double(), ctypes.c_size_t()
    E = B.STAR_ERR_INVALID_ARG
    assert lib.star_peak_mfma_bf16(0, 1, fake, ctypes.byref(d), None) == E
    assert lib.star_peak_mfma_bf16(1, 0, fake, ctypes.byref(d), None) == E
    assert lib.star_peak_mfma_bf16(1, 1, None, ctypes.byref(d), None) == E
    assert lib.star_peak_mfma_bf16(1, 1, fake, None, None) == E
    assert lib.star_peak_exp(0, 1, fake, ctypes.byref(d), None) == E
    assert lib.star_peak_exp(1, 1, None, ctypes.byref(d), None) == E
    big = 64 << 20
    assert lib.star_peak_hbm_read(None, big, 1, fake, ctypes.byref(d), ctypes.byref(z), None) == E
    assert lib.star_peak_hbm_read(fake, (16 << 20) - 1, 1, fake, ctypes.byref(d),
                                  ctypes.byref(z), None) == E
    assert lib.star_peak_hbm_read(fake, big, 0, fake, ctypes.byref(d), ctypes.byref(z), None) == E
    assert lib.star_peak_hbm_read(fake, big, 1, None, ctypes.byref(d), ctypes.byref(z), None) == E
    assert lib.star_peak_hbm_read(fake, big, 1, fake, None, ctypes.byref(z), None) == E
