"""Three workloads run at once from three host threads, each on its own stream
(default priority), give bit-identical results to the same workloads run one
after the other on the default stream: every entry point runs on the stream
it is given, and the library keeps no state between calls."""
import contextlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from long_context_attention_phase1_amd import synthetic as syn
from long_context_attention_phase1_amd.pipeline import Pipeline

pytestmark = pytest.mark.gpu

W = syn.Workload
WORKLOADS = [
    # balanced decode plan with an unaligned context (the slice-split path)
    W("streams_a", 1, 8, 2, 128, 2172, 1024, 300, 8, 4, "bf16", seed=31),
    # blockwise plan, d = 64, two sequences, GQA 8:1, a wide query step
    W("streams_b", 2, 16, 2, 64, 700, 64, 64, 40, 4, "bf16", seed=32),
    # fp32 on the matrix cores: two-wave workgroups at d = 128
    W("streams_f32", 1, 4, 2, 128, 500, 128, 100, 6, 3, "f32", seed=33),
]


def _run(w, stream=None):
    ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
    with ctx:
        p = Pipeline(w, threads=1)
        p.write_context()
        o1 = p.phase1().float().cpu().numpy()
        to, tl = p.run_tail(fused=True)
        torch.cuda.current_stream().synchronize()
    return o1, to, tl


def test_concurrent_streams_match_sequential_runs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")
    ref = [_run(w) for w in WORKLOADS]
    streams = [torch.cuda.Stream() for _ in WORKLOADS]
    with ThreadPoolExecutor(len(WORKLOADS)) as ex:
        got = list(ex.map(lambda a: _run(*a), zip(WORKLOADS, streams)))
    torch.cuda.synchronize()
    for w, r, g in zip(WORKLOADS, ref, got):
        for a, b in zip(r, g):
            assert np.array_equal(a, b, equal_nan=True), w.name
