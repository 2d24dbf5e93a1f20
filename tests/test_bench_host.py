"""Host-side pieces of bench.py: the algorithmic work figures and the oracle's
CPU baseline (run here on tiny budgets; no GPU)."""
import pytest

import bench
from long_context_attention_phase1_amd import synthetic as syn


def test_phase1_flops_counts_visible_pairs():
    # 128K workload: 8 blocks of 16K, anchor 16K -> 4*d per visible pair, 32 heads
    w = syn.workload("llama8b_128k_peaked")
    b, a, n = w.block_len, w.anchor_len, w.n_blocks
    pairs = n * b * (b + 1) // 2 + (n - 1) * a * b
    assert bench.phase1_flops(w) == 4.0 * w.head_dim * pairs * w.n_q_heads
    assert abs(bench.phase1_flops(w) / 4.84e13 - 1) < 5e-3


def test_decode_bytes_is_dominated_by_the_cache():
    w = syn.workload("llama8b_128k_peaked")
    kv_len = w.ctx_len + w.n_query + 1
    cache = 2.0 * w.n_kv_heads * kv_len * w.head_dim * 2
    got = bench.decode_bytes(w, kv_len)
    assert cache < got < cache * 1.002


@pytest.mark.parametrize("name", ["tiny_f32", "llama8b_32k"])
def test_cpu_baseline_reports_both_legs(name):
    w = syn.workload(name)
    inputs = syn.make_inputs(w)
    cb = bench.cpu_baseline(w, inputs, budget_s=0.2, decode_budget_s=0.2)
    assert cb["kind"] == "oracle" and cb["unit"] == "ctx tokens/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    d = cb["decode"]
    assert d["unit"] == "µs/token" and d["value"] > 0 and d["cores"] >= 1
    assert "decode tokens" in d["sample"]


def test_bench_config_of_a_command():
    from long_context_attention_phase1_amd.profiling import bench_config
    assert bench_config("python3 /root/repo/bench.py --steps 1 --no-cpu-baseline") == {
        "workload": "llama8b_128k_peaked", "paged": False, "rope": "none"}
    assert bench_config("python bench.py --workload llama8b_1m --paged --rope adjacent") == {
        "workload": "llama8b_1m", "paged": True, "rope": "adjacent"}


def test_traffic_is_only_attached_to_the_measured_configuration():
    import json
    doc = json.load(open(bench.TRAFFIC_FILE))
    cfg = doc["_bench_config"]
    kernel = next(k for k in doc if not k.startswith("_"))
    other = dict(cfg, workload="llama8b_32k" if cfg["workload"] != "llama8b_32k" else "llama8b_1m")
    assert bench.load_traffic(other, kernel) is None
    assert bench.load_traffic(dict(cfg, paged=not cfg["paged"]), kernel) is None


def test_query_step_work_and_bound():
    # 32K and 128K sit below the ridge (HBM-bound), 1M well below, the
    # four-sequence 64-head shape above it (MFMA-bound)
    for name, bound in (("llama8b_32k", "hbm"), ("llama8b_128k_peaked", "hbm"),
                        ("llama8b_1m", "hbm"), ("llama70b_256k_b4", "mfma")):
        w = syn.workload(name)
        flop, nbytes = bench.query_work(w)
        T, L = w.n_query, w.ctx_len
        assert flop == 4.0 * w.head_dim * w.batch * w.n_q_heads * sum(L + j + 1 for j in range(T))
        cache = 2.0 * w.batch * w.n_kv_heads * (L + T) * w.head_dim * 2
        assert cache < nbytes < cache * 1.2  # plus the replies of 64 rows x 9-33 hosts
        r = bench.query_roofline(w, 1.0)
        assert r["bound"] == bound
        t_bound = max(flop / 2.5e15, nbytes / 8e12)
        assert abs(r["frac"] - t_bound / 1e-3) < 1e-12
        assert r["frac_other_bound"] <= r["frac"]
