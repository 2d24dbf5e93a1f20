"""Benchmark of the Star Attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
context KV write, phase 1 (blockwise-local causal attention with the anchor),
the phase-2 query step (KV append, split partials, LSE merge) and the
autoregressive decode loop (n_decode steps of append + partials + merge).

Prints ONE JSON line. ``value`` is the phase-1 context throughput (tokens/s)
measured inside the timed steps; the decode figure (µs per step and per
token) is reported beside it. ``roofline`` is for the dominant kernel
(phase 1, MFMA-bound, against the dense MFMA peak of the workload's type),
from HIP events recorded on the launch stream around every phase-1 launch in
the timed steps; ``roofline_query`` is for the query step against the larger
of its two bounds; ``roofline_phase2`` is for the decode step (HBM-bound),
from events around the whole decode loop (every step's launches: append and
partials in one, then the merge; fp32: append, partials, merge) divided by
the steps. ``cpu_baseline`` is the fp64 oracle timed on a bounded sample on
the host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
(NAME: a workload of the scope table, default the 128K one, or a sweep
variant: sweep_128k_b32k, sweep_128k_b8k, sweep_128k_b4k, sweep_128k_a4k_b16k,
sweep_125k_ragged)
"""
from __future__ import annotations

import argparse
import json
import os
import resource
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "phase-1 ctx tokens/s + phase-2 decode µs/token at 128K, % of roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def phase1_flops(w) -> float:
    """Algorithmic FLOPs of phase 1: 4*d per visible (query, key) pair, per head."""
    pairs = 0
    for i in range(w.n_blocks):
        bl = min(w.block_len, w.ctx_len - i * w.block_len)
        pairs += bl * (bl + 1) // 2 + (w.anchor_len * bl if i > 0 else 0)
    return 4.0 * w.head_dim * pairs * w.batch * w.n_q_heads


def decode_bytes(w, kv_len: int) -> float:
    """Algorithmic HBM bytes of one decode step: the new token's K/V row
    written, K+V rows [0, kv_len) and the query read once, every host's reply
    (one fp32 vector and one scalar per query head, for each context block
    and the tail) written and read back by the aggregation, the output row
    and its LSE written. The kernels' finer split partials are not counted:
    they are this implementation's choice, not the method's."""
    elt = 2 if w.dtype == "bf16" else 4
    append = 2.0 * w.batch * w.n_kv_heads * w.head_dim * elt
    kv = 2.0 * w.batch * w.n_kv_heads * kv_len * w.head_dim * elt
    q = w.batch * w.n_q_heads * w.head_dim * elt
    hosts = w.n_blocks + 1
    parts = 2.0 * w.batch * w.n_q_heads * hosts * (w.head_dim + 1) * 4
    out = w.batch * w.n_q_heads * (w.head_dim * elt + 4)
    return append + kv + q + parts + out


def query_work(w):
    """Algorithmic (FLOP, HBM bytes) of the query step: the n_query tokens'
    K/V rows written, K+V rows [0, ctx_len + n_query) and the queries read
    once, every host's reply (one fp32 vector and one scalar per query row
    and head, for each context block and the tail) written and read back,
    the outputs and their LSEs written. FLOP: 4*d per visible (query, key)
    pair; query j sees rows [0, ctx_len + j]."""
    elt = 2 if w.dtype == "bf16" else 4
    T, L = w.n_query, w.ctx_len
    pairs = T * L + T * (T + 1) // 2
    flop = 4.0 * w.head_dim * pairs * w.batch * w.n_q_heads
    append = 2.0 * w.batch * T * w.n_kv_heads * w.head_dim * elt
    kv = 2.0 * w.batch * w.n_kv_heads * (L + T) * w.head_dim * elt
    q = w.batch * T * w.n_q_heads * w.head_dim * elt
    parts = 2.0 * w.batch * T * w.n_q_heads * (w.n_blocks + 1) * (w.head_dim + 1) * 4
    out = w.batch * T * w.n_q_heads * (w.head_dim * elt + 4)
    return flop, append + kv + q + parts + out


def mfma_peak(w) -> float:
    """The dense MFMA peak of the workload's arithmetic type, TFLOP/s."""
    return PEAK_F32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS


def query_roofline(w, q_ms: float) -> dict:
    """The query step against the larger of its two bounds (MFMA time of its
    FLOP at the MFMA peak of its type, HBM time of its bytes at 8 TB/s)."""
    flop, nbytes = query_work(w)
    t_mfma = flop / (mfma_peak(w) * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    t = q_ms * 1e-3
    if t_hbm >= t_mfma:
        r = {"bound": "hbm", "achieved": nbytes / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": flop / t / 1e12, "peak": mfma_peak(w),
             "unit": "TFLOP/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r["frac_other_bound"] = min(t_mfma, t_hbm) / t
    r["kernel"] = "query step: kv_write + partials + merge"
    r["algorithmic"] = (f"{flop:.4e} FLOP (4*d per visible pair) and {nbytes:.4e} B "
                        f"(K+V rows read once, n_query K/V rows written, replies, outputs)")
    return r


def host_info():
    """The host the oracle runs on: cores available to this process, CPU model,
    numpy's BLAS library and its thread count."""
    import numpy as np
    from threadpoolctl import threadpool_info
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    try:
        dep = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas_name = f"{dep.get('name')} {dep.get('version')}"
    except Exception:  # older numpy: no dict form
        blas_name = blas[0]["internal_api"] if blas else None
    return {"cores_available": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(),
            "cpu_model": model, "blas": blas_name,
            "blas_threads": blas[0]["num_threads"] if blas else None}


def cpu_baseline(w, inputs, budget_s: float = 12.0, decode_budget_s: float = 6.0, gpu=None):
    """The oracle (as it stands) on a bounded sample of the same workload:
    phase-1 context rows (the headline unit), then decode tokens.

    ``gpu``: optional GPU results of the timed run (``o_ctx`` for sequence 0
    and ``o_last``, the last decode step's output) that the sampled oracle
    rows are also compared with, element by element (max-abs error)."""
    import numpy as np

    from long_context_attention_phase1_amd import synthetic as syn
    from oracle import star_oracle as orc

    rng = np.random.default_rng(0)
    G = w.group
    sc = orc.resolve_scale(w.head_dim, 0.0)
    rows = rng.integers(0, w.ctx_len, size=4096)
    # exact widening of the inputs, outside the timed region
    wide = (syn.bf16_bits_to_f32 if w.dtype == "bf16" else np.asarray)
    Ks = [wide(inputs["k_ctx"][0, :, g]) for g in range(w.n_kv_heads)]
    Vs = [wide(inputs["v_ctx"][0, :, g]) for g in range(w.n_kv_heads)]
    t0, c0 = time.perf_counter(), time.process_time()
    done, ref1 = 0, []
    for r in rows:
        r = int(r)
        outs = []
        for g in range(w.n_kv_heads):
            q = wide(inputs["q_ctx"][0, r:r + 1, g * G:(g + 1) * G])
            outs.append(orc.phase1_rows_one_head(q, Ks[g], Vs[g], [r], w.block_len, w.anchor_len,
                                                 sc))
        ref1.append((r, outs))
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    wall = time.perf_counter() - t0
    cpu = time.process_time() - c0

    # decode tokens of sequence 0 in order: each attends to the context and
    # the tail rows up to itself (the dense definition of a phase-2 row)
    Kall = [np.concatenate([Ks[g], wide(inputs["k_tail"][0, :, g])]) for g in range(w.n_kv_heads)]
    Vall = [np.concatenate([Vs[g], wide(inputs["v_tail"][0, :, g])]) for g in range(w.n_kv_heads)]
    del Ks, Vs
    t1, c1 = time.perf_counter(), time.process_time()
    steps = 0
    for t in range(w.n_decode):
        row = w.n_query + t
        for g in range(w.n_kv_heads):
            q = wide(inputs["q_tail"][0, row:row + 1, g * G:(g + 1) * G])
            orc.phase2_rows_one_head(q, Kall[g], Vall[g], [w.ctx_len + row], sc)
        steps += 1
        if time.perf_counter() - t1 > decode_budget_s:
            break
    dwall = time.perf_counter() - t1
    dcpu = time.process_time() - c1
    parity = None
    if gpu is not None:
        # the GPU's outputs of the timed run against the sampled oracle rows
        e1 = 0.0
        for r, outs in ref1:
            o = gpu["o_ctx"][r]  # [Hq, d] float64
            for g, ref in enumerate(outs):
                e1 = max(e1, float(np.abs(o[g * G:(g + 1) * G] - ref[0]).max()))
        row = w.n_query + w.n_decode - 1
        e2, el = 0.0, 0.0
        for g in range(w.n_kv_heads):
            q = wide(inputs["q_tail"][0, row:row + 1, g * G:(g + 1) * G])
            ro, rl = orc.phase2_rows_one_head(q, Kall[g], Vall[g], [w.ctx_len + row], sc)
            e2 = max(e2, float(np.abs(gpu["o_last"][g * G:(g + 1) * G] - ro[0]).max()))
            el = max(el, float(np.abs(gpu["lse_last"][g * G:(g + 1) * G] - rl[0]).max()))
        parity = {"phase1_max_abs": e1, "phase1_rows": len(ref1),
                  "last_decode_max_abs": e2, "last_decode_lse_max_abs": el,
                  "sample": f"sequence 0: the {len(ref1)} timed phase-1 rows (all heads) and the "
                            f"last decode token (all heads) of the timed run against the fp64 "
                            f"oracle"}
    info = host_info()
    return {"value": done / wall, "unit": "ctx tokens/s", "cores": info["blas_threads"]
            or info["cores_available"],
            "achieved_parallelism": cpu / wall, "host": info, "parity": parity,
            "kind": "oracle",
            "sample": f"phase-1 fp64 oracle on {done} context rows drawn uniformly (seed 0) "
                      f"from sequence 0, all {w.n_q_heads} query heads, {wall:.1f} s wall",
            "decode": {"value": dwall * 1e6 / steps, "unit": "µs/token",
                       "cores": info["blas_threads"] or info["cores_available"],
                       "achieved_parallelism": dcpu / dwall,
                       "sample": f"dense fp64 oracle rows of the first {steps} decode tokens "
                                 f"of sequence 0, all {w.n_q_heads} query heads, "
                                 f"{dwall:.1f} s wall"}}


def load_traffic(config: dict, *kernels):
    """HBM bytes per launch, summed over the given kernels, from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE summary, if it was taken on the current
    native library source (csrc/) and on this bench configuration (workload,
    cache, rotary mode: the launch shapes depend on it); else None."""
    try:
        doc = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if doc.get("_bench_config") != config:
        return None
    from long_context_attention_phase1_amd.profiling import source_sha
    sha = source_sha()
    total = 0.0
    for k in kernels:
        ent = doc.get(k)
        if not ent or ent.get("source_sha256_16") != sha:
            return None
        total += ent["bytes_per_launch"]
    return total


def copy_calibration():
    """A plain device copy of COPY_BYTES (read once, written once): the
    reference volume that scales the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    from long_context_attention_phase1_amd.profiling import COPY_BYTES
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


class _Rows:
    """Rows of a device tensor, fetched one at a time as float64 host arrays."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, r):
        return self.t[r].double().cpu().numpy()


def decode_flushed(p, w, stream):
    """The decode loop with the KV cache evicted from the 256 MB last-level
    cache (MALL) before every step: a 512 MiB device read (a sum) before each
    step. A read leaves no dirty lines behind, so the step pays no write-back
    of the flush buffer. Timed as a loop of (flush, step) against a loop of
    the flushes alone, each bracketed by HIP events on the launch stream with
    the queue never idle; the difference over the steps is the step time on a
    cold MALL."""
    import numpy as np
    import torch
    flush = torch.ones(128 << 20, dtype=torch.float32, device=p.k_cache.device)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def loop(with_steps: bool) -> float:
        e0, e1 = ev(), ev()
        e0.record(stream)
        for t in range(w.n_decode):
            flush.sum()
            if with_steps:
                row = w.n_query + t
                kv_len = w.ctx_len + row + 1
                n_split, o_part, lse_part, o, lse = p.workspace(kv_len, 1)
                p.decode_call(kv_len, row, o_part, lse_part, o, lse)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    loop(True)  # warm-up
    both = [loop(True) for _ in range(3)]
    flushes = [loop(False) for _ in range(3)]
    us = (float(np.median(both)) - float(np.median(flushes))) * 1e3 / w.n_decode
    nbytes = sum(decode_bytes(w, w.ctx_len + w.n_query + t + 1) for t in range(w.n_decode))
    gbs = nbytes / w.n_decode / (us * 1e-6) / 1e9
    del flush
    return {"us_per_step": us, "achieved_GBs": gbs, "frac_of_8TBs": gbs / PEAK_HBM_GBS,
            "method": "median of 3 loops of (512 MiB read, decode step) minus median of 3 "
                      "loops of the reads alone, over the steps"}


def gfx_clock_during(fn, launch_ms: float, device: int = 0, busy_s: float = 1.5,
                     period_s: float = 0.05):
    """The graphics clock of each XCD while fn (one launch of launch_ms) runs
    back to back for about busy_s, read from the SMU's metrics table through
    amdsmi by a host thread. The table refreshes about once a second, so only
    the samples of the second half of the busy window count. A record with an
    "error" field when amdsmi or the device's handle is not available."""
    import math
    import threading

    import numpy as np
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception as e:  # no amdsmi, or no access to the driver's interface
        return {"error": f"amdsmi unavailable: {e}"}
    try:
        hs = amdsmi.amdsmi_get_processor_handles()
        prop = torch.cuda.get_device_properties(device)
        bdf = f"{prop.pci_domain_id:04x}:{prop.pci_bus_id:02x}:{prop.pci_device_id:02x}"
        match = [h for h in hs if amdsmi.amdsmi_get_gpu_device_bdf(h).lower().startswith(bdf)]
        h = match[0] if match else (hs[0] if len(hs) == 1 else None)
        if h is None:
            return {"error": f"no amdsmi handle for the GPU at {bdf}"}
        samples = []  # (seconds since the launches were enqueued, per-XCD MHz, socket W)
        stop = threading.Event()

        def sample(t0):
            while not stop.is_set():
                try:
                    m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                    clks = [float(c) for c in m.get("current_gfxclks", []) if isinstance(c, int)]
                    if not clks and isinstance(m.get("current_gfxclk"), int):
                        clks = [float(m["current_gfxclk"])]
                    pw = m.get("current_socket_power")
                    samples.append((time.perf_counter() - t0, clks,
                                    float(pw) if isinstance(pw, int) else None))
                except Exception:
                    pass
                stop.wait(period_s)

        n = max(3, min(4000, math.ceil(busy_s * 1e3 / max(launch_ms, 1e-3))))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        th = threading.Thread(target=sample, args=(t0,), daemon=True)
        th.start()
        torch.cuda.synchronize()
        busy = time.perf_counter() - t0
        stop.set()
        th.join()
        late = [(c, w) for t, c, w in samples if busy / 2 <= t <= busy and c]
        if not late:
            return {"error": f"no clock sample in the second half of a {busy:.2f} s busy window"}
        per_xcd = np.median(np.array([c for c, _ in late]), axis=0)
        power = [w for _, w in late if w is not None]
        return {"xcd_mhz": [round(float(x)) for x in per_xcd],
                "mean_mhz": float(per_xcd.mean()), "min_mhz": float(per_xcd.min()),
                "max_mhz": float(per_xcd.max()),
                "socket_power_w": float(np.median(power)) if power else None,
                "samples": len(late),
                "method": f"amdsmi metrics (current_gfxclks per XCD), {len(late)} samples in the "
                          f"second half of {n} back-to-back phase-1 launches ({busy:.2f} s), after "
                          f"the timed steps"}
    except Exception as e:
        return {"error": f"amdsmi clock query failed: {e}"}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", "--reps", dest="steps", type=int, default=10,
                    help="timed steps (one step: context write, phase 1, query step, "
                         "decode loop)")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", "--config", dest="workload", default="llama8b_128k_peaked",
                    help="a workload of synthetic.WORKLOADS or synthetic.SWEEPS")
    ap.add_argument("--seed", type=int, default=None,
                    help="seed of the synthetic inputs (default: the workload's, 0)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock record (about 1.5 s of back-to-back phase-1 launches "
                         "after the timed steps), e.g. under a kernel trace whose per-kernel "
                         "averages should cover the bench's own launches only")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the peak probes (libstarpeaks.so) run after the timed steps")
    ap.add_argument("--threads", type=int, default=None)
    ap.add_argument("--rope", choices=["none", "original", "adjacent"], default="none",
                    help="phase 1 with the rotary embedding fused (K rotated by the context "
                         "write, the query in phase 1), anchor position ids as named")
    ap.add_argument("--paged", action="store_true",
                    help="phase 2 (query step and decode loop) on a paged cache through a "
                         "block table; the context is written into the pages too")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--flush-mall", action="store_true",
                    help="after the timed steps, time the decode loop with the 256 MB "
                         "last-level cache (MALL) flushed before each step (a 512 MiB buffer "
                         "read between steps; the reads alone are timed and taken off)")
    args = ap.parse_args()
    if args.paged and args.rope != "none":
        ap.error("--paged writes the context unrotated into the pages: use it without --rope")
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the path is measured on one GPU's share "
              f"(--gpus {args.gpus} is not supported)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import long_context_attention_phase1_amd as sa
    from long_context_attention_phase1_amd import synthetic as syn
    from long_context_attention_phase1_amd.pipeline import PagedPipeline, Pipeline

    w = syn.workload(args.workload)
    if args.seed is not None:
        w = w.replace(seed=args.seed)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
    t_gen = time.perf_counter()
    inputs = syn.make_inputs(w, args.threads)
    p = (PagedPipeline if args.paged else Pipeline)(w, inputs=inputs, fill_nan=False)
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    p1_events, dec_bytes, q_events = [], [], []
    rope = None
    if args.rope != "none":
        rope = p.rope(sa.STAR_ROPE_ADJACENT if args.rope == "adjacent" else sa.STAR_ROPE_ORIGINAL)

    def step(record: bool):
        if rope is None:
            p.write_context()
        else:
            p.write_context_rope(rope)
        e0, e1 = ev(), ev()
        e0.record(stream)
        if rope is None:
            p.phase1()
        else:
            p.phase1_rope(rope)
        e1.record(stream)
        if record:
            p1_events.append((e0, e1))
        q0, q1 = ev(), ev()
        q0.record(stream)
        p.query_step()
        q1.record(stream)
        if record:
            q_events.append((q0, q1))
        d0 = ev()
        d0.record(stream)
        for t in range(w.n_decode):
            row = w.n_query + t
            kv_len = w.ctx_len + row + 1
            n_split, o_part, lse_part, o, lse = p.workspace(kv_len, 1)
            # append the token's K/V + split partials (one launch), then the
            # merge (a second launch): star_attn_decode_step[_paged]
            p.decode_call(kv_len, row, o_part, lse_part, o, lse)
            if record:
                dec_bytes.append(decode_bytes(w, kv_len))
        d1 = ev()
        d1.record(stream)
        return d0, d1

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    dec_loops = []
    t0 = time.perf_counter()
    s0 = ev()
    s0.record(stream)
    for _ in range(args.steps):
        dec_loops.append(step(True))
    s1 = ev()
    s1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    gpu_ms = s0.elapsed_time(s1)
    assert torch.isfinite(p.o_ctx.float()).all(), "non-finite phase-1 output"

    p1_ms = float(np.median([a.elapsed_time(b) for a, b in p1_events]))
    p1_avg_ms = float(np.mean([a.elapsed_time(b) for a, b in p1_events]))
    q_ms = float(np.median([a.elapsed_time(b) for a, b in q_events]))
    loop_ms = np.array([a.elapsed_time(b) for a, b in dec_loops])
    dec_loop_ms = float(np.median(loop_ms))
    ctx_tok_s = w.batch * w.ctx_len / (p1_ms * 1e-3)
    flops = phase1_flops(w)
    p1_tflops = flops / (p1_avg_ms * 1e-3) / 1e12
    dec_gbs = float(np.sum(dec_bytes) / (np.sum(loop_ms) * 1e-3) / 1e9)
    step_us = dec_loop_ms * 1e3 / w.n_decode

    pg = "true" if args.paged else "false"
    rp = {"none": 0, "original": 1, "adjacent": 2}[args.rope]
    if w.dtype == "f32":
        # fp32 runs on the matrix-core fp32 kernel; its decode step is three
        # launches: the append, the partials, the merge
        kname1 = f"attn_f32m_kernel<{w.head_dim}, true, false, {rp}>"
        kname2 = (f"kv_write_kernel<float, {w.head_dim}, {pg}, false>",
                  f"attn_f32m_kernel<{w.head_dim}, false, {pg}, 0>",
                  f"lse_merge_kernel<{w.head_dim}>")
    else:
        kname1 = f"attn_wide_kernel<{w.head_dim}, 8, 1, true, false, {rp}, false>"
        # the decode kernel's instantiation that splits a 32-key slice at a
        # host boundary serves contexts and blocks off the slice grid
        mid = "true" if (w.ctx_len % 32 or w.block_len % 32) else "false"
        kname2 = (f"attn_decode_kernel<{w.head_dim}, true, {pg}, {mid}>",
                  f"lse_merge_kernel<{w.head_dim}>")
    pk = mfma_peak(w)
    bcfg = {"workload": args.workload, "paged": bool(args.paged), "rope": args.rope}
    t1, t2 = load_traffic(bcfg, kname1), load_traffic(bcfg, *kname2)
    # the shader clock phase 1 runs at (outside the timed region)
    clock = None if args.no_clock else gfx_clock_during(
        p.phase1 if rope is None else (lambda: p.phase1_rope(rope)), p1_ms)
    # measured peaks (after the timed region): the rates each roofline is also
    # read against, beside the published peaks
    measured = None
    if not args.no_peaks:
        from long_context_attention_phase1_amd import peaks
        measured = peaks.measure(device=p.k_cache.device)
        torch.cuda.synchronize()
    out = {
        "metric": METRIC,
        "value": ctx_tok_s,
        "unit": "ctx tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": max(wall_ms, gpu_ms) / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "ctx_len": w.ctx_len,
                   "block_len": w.block_len, "anchor_len": w.anchor_len,
                   "n_query": w.n_query, "n_decode": w.n_decode, "seed": w.seed,
                   "peaked_k_rows": w.peak_frac, "peak_factor": w.peak_factor,
                   "phase2_cache": "paged" if args.paged else "contiguous",
                   "rope": args.rope},
        "phase1_ms": p1_ms,
        "phase1_ctx_tokens_per_s": ctx_tok_s,
        "query_step_ms": q_ms,
        "decode_us_per_step": step_us,
        "decode_us_per_token": step_us / w.batch,
        "roofline": {"bound": "mfma", "achieved": p1_tflops, "peak": pk,
                     "unit": "TFLOP/s", "frac": p1_tflops / pk,
                     "traffic": t1, "kernel": kname1,
                     "algorithmic": f"{flops:.4e} FLOP per launch (4*d per visible pair)"},
        "roofline_phase2": {"bound": "hbm", "achieved": dec_gbs, "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": dec_gbs / PEAK_HBM_GBS, "traffic": t2,
                            "kernel": " + ".join(kname2),
                            "algorithmic": "per decode step: K+V rows [0, kv_len) and q read, "
                                           "new K/V row written, one fp32 reply per host "
                                           "written and re-read, output row written"},
        "roofline_query": query_roofline(w, q_ms),
        "gfx_clock_phase1": clock,
    }
    if measured is not None:
        out["measured_peaks"] = measured
        if w.dtype == "bf16":
            out["roofline"]["frac_of_measured"] = p1_tflops / measured["mfma_bf16"]["value"]
        out["roofline_phase2"]["frac_of_measured"] = dec_gbs / measured["hbm_read"]["value"]
        rq = out["roofline_query"]
        if rq["bound"] == "hbm":
            rq["frac_of_measured"] = rq["achieved"] / measured["hbm_read"]["value"]
        elif w.dtype == "bf16":
            rq["frac_of_measured"] = rq["achieved"] / measured["mfma_bf16"]["value"]
    if args.flush_mall:
        out["decode_mall_flushed"] = decode_flushed(p, w, stream)
    if not args.no_cpu_baseline:
        row = w.n_query + w.n_decode - 1
        _, _, _, o_last, lse_last = p.workspace(w.ctx_len + row + 1, 1)
        gpu = {"o_ctx": _Rows(p.o_ctx[0]),
               "o_last": o_last[0, 0].double().cpu().numpy(),
               "lse_last": lse_last[0, 0].double().cpu().numpy()}
        out["cpu_baseline"] = cpu_baseline(w, inputs, gpu=gpu)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
