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


def test_cpu_baseline_records_host_and_compares_gpu_outputs():
    """The oracle leg states the host (cores available, CPU model, BLAS) and,
    given a run's outputs, their max-abs error on the sampled rows: zero for
    the oracle's own outputs, the planted offset for shifted ones."""
    import numpy as np

    from oracle import star_oracle as orc
    w = syn.workload("tiny_f32")
    x = {k: syn.to_f64(v, w.dtype) for k, v in syn.make_inputs(w).items()}
    sc = orc.resolve_scale(w.head_dim, 0.0)
    o1 = orc.phase1(x["q_ctx"], x["k_ctx"], x["v_ctx"], w.block_len, w.anchor_len, sc)[0]
    ro, rl = orc.decode_loop(x["q_tail"], x["k_ctx"], x["v_ctx"], x["k_tail"], x["v_tail"],
                             w.n_query, sc)
    exact = {"o_ctx": o1, "o_last": ro[0, -1], "lse_last": rl[0, -1]}
    inputs = syn.make_inputs(w)
    cb = bench.cpu_baseline(w, inputs, budget_s=0.2, decode_budget_s=0.2, gpu=exact)
    h = cb["host"]
    assert h["cores_available"] >= 1 and h["cpu_count"] >= h["cores_available"]
    assert h["blas"] and cb["cores"] >= 1 and cb["achieved_parallelism"] > 0
    par = cb["parity"]
    assert par["phase1_rows"] >= 1
    assert par["phase1_max_abs"] < 1e-12 and par["last_decode_max_abs"] < 1e-12
    assert par["last_decode_lse_max_abs"] < 1e-12
    shifted = {"o_ctx": o1 + 1e-3, "o_last": ro[0, -1] - 2e-3, "lse_last": rl[0, -1] + 3e-3}
    par = bench.cpu_baseline(w, inputs, budget_s=0.2, decode_budget_s=0.2, gpu=shifted)["parity"]
    assert abs(par["phase1_max_abs"] - 1e-3) < 1e-9
    assert abs(par["last_decode_max_abs"] - 2e-3) < 1e-9
    assert abs(par["last_decode_lse_max_abs"] - 3e-3) < 1e-9


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


def test_clock_sampler_reports_why_it_has_no_clock_without_a_gpu():
    # on a host without the GPU driver the record names the reason instead of
    # failing the bench line
    rec = bench.gfx_clock_during(lambda: None, 1)
    assert set(rec) == {"error"} and rec["error"]


def test_flag_spellings_of_the_bench_record(monkeypatch, capsys):
    # --config, --reps and --seed are spellings the bench record documents;
    # --gpus above 1 stops before anything touches a GPU
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2", "--config", "llama8b_32k",
                                     "--reps", "3", "--seed", "7", "--no-clock"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def test_counter_summary_is_per_dispatch(tmp_path):
    # two dispatches of one kernel in a run: the summary reports one
    # dispatch's counters, so the engine clock (active cycles over the
    # dispatch duration) does not grow with the number of launches
    from long_context_attention_phase1_amd import profiling
    k = "void star::(anonymous namespace)::attn_wide_kernel<128, 8, 1, true, false, 0, false>(WideArgs)"
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp"]
    for disp in (1, 2):
        t0 = disp * 10**9
        # 8 XCDs x 2.0e6 active cycles over 1 ms: a 2.0 GHz clock
        rows.append(f'{disp},"{k}",GRBM_GUI_ACTIVE,{8 * 2.0e6},{t0},{t0 + 10**6}')
        rows.append(f'{disp},"{k}",SQ_INSTS_MFMA,1000,{t0},{t0 + 10**6}')
        rows.append(f'{disp},"{k}",SQ_INSTS_VALU,5800,{t0},{t0 + 10**6}')
    d = tmp_path / "run"
    d.mkdir()
    (d / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    out = tmp_path / "c.txt"
    profiling.counters(str(out), [str(d)], "cmd")
    text = out.read_text()
    assert "SQ_INSTS_MFMA                    1.000000e+03" in text
    assert "effective engine clock (active / duration) 2.000 GHz" in text
    assert "non-MFMA VALU instructions per MFMA        4.80" in text


def test_mfma_peak_follows_the_workload_type():
    """fp32 workloads run on the fp32 matrix cores: their MFMA roofline is
    the dense fp32 peak (157.3 TFLOP/s), not the bf16 one."""
    import bench
    f32, bf16 = syn.workload("tiny_f32"), syn.workload("llama8b_32k")
    assert bench.mfma_peak(f32) == 157.3 and bench.mfma_peak(bf16) == 2500.0
    # a query step made MFMA-bound at fp32 is priced against the fp32 peak
    r = bench.query_roofline(f32.__class__(**{**f32.__dict__, "n_query": 256, "ctx_len": 4096,
                                              "block_len": 1024, "anchor_len": 1024}), 1.0)
    assert r["bound"] == "mfma" and r["peak"] == 157.3, r
