"""The peak probes on the GPU return rates inside what MI355X can do: the
bf16 MFMA probe at most the 2.5 PFLOP/s spec and above a third of it, the
non-temporal read stream at most the 8 TB/s spec and above 2 TB/s, and the
exp probe a positive rate; the stream reads whole chunks inside the buffer."""
import pytest
import torch

from long_context_attention_phase1_amd import peaks

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")


def test_peak_probes_are_plausible():
    _need_gpu()
    nbytes = 1 << 30
    m = peaks.measure(device="cuda", nbytes=nbytes)
    tf, gbs = m["mfma_bf16"]["value"], m["hbm_read"]["value"]
    print(f"mfma {tf:.0f} TFLOP/s (clock {m['mfma_clock_ghz']:.2f} GHz), "
          f"read {gbs:.0f} GB/s over {m['hbm_read']['bytes']} B, "
          f"exp {m['v_exp_f32']['value']:.0f} G/s")
    assert peaks.SPEC_BF16_TFLOPS / 3 < tf <= peaks.SPEC_BF16_TFLOPS * 1.01
    assert 0.5 < m["mfma_clock_ghz"] <= 2.45
    assert 2000.0 < gbs <= 8000.0 * 1.01
    assert nbytes // 2 < m["hbm_read"]["bytes"] <= nbytes
    assert m["hbm_read"]["bytes"] % (64 * 16 * 16) == 0
    assert m["v_exp_f32"]["value"] > 0.0
