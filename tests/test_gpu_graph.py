"""The decode step inside a HIP graph: eight star_attn_decode_step calls
(each one append + split partials + merge: two launches in bf16, three in
fp32) captured once and replayed three times, with eager work and
synchronisation between replays, give bit-identical outputs to the eager
calls every time. The library
allocates nothing, synchronises nothing and issues no memset, so a serving
loop can capture its decode steps."""
import numpy as np
import pytest
import torch

from long_context_attention_phase1_amd import synthetic as syn
from long_context_attention_phase1_amd.pipeline import Pipeline

pytestmark = pytest.mark.gpu

STEPS = 8


GRAPH_WORKLOADS = {
    "bf16": syn.Workload("graph", 1, 8, 2, 128, 1536, 512, 256, 4, STEPS, "bf16", seed=41),
    # fp32: the append, the matrix-core partials (four-wave workgroups at d = 64), the merge
    "f32": syn.Workload("graph_f32", 1, 4, 2, 64, 600, 256, 128, 4, STEPS, "f32", seed=42),
}


@pytest.mark.parametrize("dtype", list(GRAPH_WORKLOADS))
def test_decode_steps_replay_in_a_graph(dtype):
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")
    w = GRAPH_WORKLOADS[dtype]
    p = Pipeline(w, threads=1)
    p.write_context()
    p.query_step()
    eager = []
    for t in range(STEPS):
        o, lse = p.decode_step_fused(t)
        eager.append((o.float().cpu().numpy(), lse.cpu().numpy()))
    torch.cuda.synchronize()

    # every step's workspace exists now; the graph copies each step's output
    # into buffers of its own (steps with the same split count share one)
    o_cp = [torch.empty_like(p.decode_step_fused(t)[0]) for t in range(STEPS)]
    l_cp = [torch.empty_like(p.decode_step_fused(t)[1]) for t in range(STEPS)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(STEPS):
            o, lse = p.decode_step_fused(t)
            o_cp[t].copy_(o)
            l_cp[t].copy_(lse)
    for rep in range(3):
        for t in range(STEPS):
            o_cp[t].fill_(float("nan"))
            l_cp[t].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for t in range(STEPS):
            assert np.array_equal(o_cp[t].float().cpu().numpy(), eager[t][0]), (rep, t)
            assert np.array_equal(l_cp[t].cpu().numpy(), eager[t][1]), (rep, t)
        # eager work between replays
        p.decode_step_fused(STEPS - 1)
        torch.cuda.synchronize()
