"""Summaries of rocprofv3 CSV output for the committed profile records.

``python -m long_context_attention_phase1_amd.profiling stats DIR OUT.txt [BENCH.json] -- CMD``
    formats the kernel_stats.csv of a ``rocprofv3 --kernel-trace --stats
    --output-format csv`` run (per-kernel calls, total/avg/min/max duration)
    and, given the JSON line that the profiled bench.py printed, the figures
    of that same run measured with HIP events.

``python -m long_context_attention_phase1_amd.profiling traffic FETCH_DIR WRITE_DIR OUT.json OUT.txt -- CMD``
    reads two ``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs of
    ``bench.py --copy-calibration`` and writes, per kernel and launch shape,
    the HBM bytes per launch. Both counters are in KiB per dispatch; each is
    scaled by what it reads on the plain device-to-device copy of known size
    that the calibration run performs first (``COPY_BYTES`` read and written
    once), so the figures are in the same units as the algorithmic bytes.
    The bench configuration the runs measured (workload, cache, rotary mode:
    ``bench_config`` of their command) is recorded beside the figures, which
    hold for that configuration only.

``python -m long_context_attention_phase1_amd.profiling counters OUT.txt DIR... -- CMD``
    sums the SQ_* / GRBM_GUI_ACTIVE counters of the given ``rocprofv3 --pmc``
    runs per kernel and derives MFMA utilisation (MFMA-busy cycles over
    active cycles x SIMDs), LDS utilisation, VALU and co-issue figures and
    the effective engine clock (active cycles over the kernel duration).

Host-only text processing; no GPU work.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

COPY_BYTES = 1 << 30
PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")


# the attention library's sources: a change to any of them (kernels,
# launchers, planner) can change what a launch does
LIB_SOURCES = ("star_host.cpp", "star_internal.hpp", "star_kernels.hip")


def source_sha() -> str:
    """sha256[:16] over the attention library's sources."""
    h = hashlib.sha256()
    for name in sorted(LIB_SOURCES):
        h.update(name.encode() + b"\0" + open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    """Demangled kernel name without namespaces and argument lists."""
    n = name.replace("star::(anonymous namespace)::", "")
    n = re.sub(r"\((?:[^()]|\([^()]*\))*\)\s*$", "", n).strip()
    if n.startswith("void "):
        n = n[5:]
    return n


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def _bench_lines(path: str):
    d = json.loads(open(path).read().strip().splitlines()[-1])
    r1, r2 = d["roofline"], d["roofline_phase2"]
    return ["# bench.py line printed by the same profiled run (HIP events on the launch stream):",
            f"#   phase 1 {r1['kernel']}: {r1['achieved']:.1f} TFLOP/s -> "
            f"{d['phase1_ms']:.2f} ms per launch (median of the timed launches)",
            f"#   decode loop: {d['decode_us_per_step']:.2f} us per step ({r2['kernel']}), "
            f"{r2['achieved']:.0f} GB/s",
            "# raw line: " + json.dumps(d)]


def stats(d: str, out: str, command: str, bench_json: str = None) -> None:
    rows = list(csv.DictReader(open(_find(d, "kernel_stats.csv"))))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {command}",
             f"# native source (csrc/) sha256[:16]: {source_sha()}",
             f"{'kernel':58s} {'calls':>6s} {'total ms':>10s} {'avg us':>10s} "
             f"{'min us':>10s} {'max us':>10s} {'%':>6s}"]
    for r in rows:
        lines.append(f"{short_name(r['Name'])[:58]:58s} {int(r['Calls']):6d} "
                     f"{float(r['TotalDurationNs']) / 1e6:10.3f} "
                     f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                     f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}")
    if bench_json:
        lines += _bench_lines(bench_json)
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _dispatches(d: str, counter: str):
    """{dispatch id: (kernel short name, grid size, counter value in KiB)}."""
    out = {}
    for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
        if r["Counter_Name"] == counter:
            out[int(r["Dispatch_Id"])] = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]),
                                          float(r["Counter_Value"]))
    return out


def _calibration(disp, counter: str) -> float:
    """Scale that turns the counter into bytes: COPY_BYTES over its mean value
    on the device-to-device copies of COPY_BYTES (runtime blit kernel) that the
    calibration run issues."""
    vals = [v for k, _, v in disp.values() if k == "__amd_rocclr_copyBuffer"]
    if counter == "WRITE_SIZE":
        vals = [v for v in vals if abs(v * 1024 - COPY_BYTES) < 0.01 * COPY_BYTES]
    vals = [v for v in vals if v * 1024 > COPY_BYTES / 8]
    if not vals:
        raise RuntimeError("calibration copy not found in the counter run")
    return COPY_BYTES / (sum(vals) / len(vals) * 1024)


def bench_config(command: str) -> dict:
    """The workload options of a bench.py command line (its defaults where
    absent): the launch shapes, hence the traffic, depend on them."""
    import shlex

    args = shlex.split(command)
    cfg = {"workload": "llama8b_128k_peaked", "paged": "--paged" in args, "rope": "none"}
    for i, a in enumerate(args[:-1]):
        if a == "--workload":
            cfg["workload"] = args[i + 1]
        elif a == "--rope":
            cfg["rope"] = args[i + 1]
    return cfg


def traffic(fetch_dir: str, write_dir: str, out_json: str, out_txt: str, commands) -> None:
    fetch = _dispatches(fetch_dir, "FETCH_SIZE")
    write = _dispatches(write_dir, "WRITE_SIZE")
    f_scale, w_scale = _calibration(fetch, "FETCH_SIZE"), _calibration(write, "WRITE_SIZE")
    # library kernels only, grouped by (kernel, grid): one group per launch shape
    groups = defaultdict(list)
    for i, (k, grid, fv) in fetch.items():
        if i in write and write[i][0] == k and "_kernel<" in k and not k.startswith("at::"):
            groups[(k, grid)].append((fv, write[i][2]))
    sha = source_sha()
    cfgs = [bench_config(c.split(" -- ", 1)[-1]) for c in commands]
    if any(c != cfgs[0] for c in cfgs):
        raise ValueError("the FETCH_SIZE and WRITE_SIZE runs measured different bench configurations")
    doc = {"_calibration": {"copy_bytes": COPY_BYTES, "fetch_scale": f_scale,
                            "write_scale": w_scale, "copy_kernel": "__amd_rocclr_copyBuffer",
                            "commands": list(commands)},
           "_bench_config": cfgs[0]}
    lines = ["# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch)",
             *[f"# command: {c}" for c in commands],
             f"# bench configuration: {json.dumps(cfgs[0])} (the figures hold for it only)",
             f"# calibration: device-to-device copy of {COPY_BYTES} B (runtime blit kernel) -> "
             f"bytes = FETCH_SIZE KiB x 1024 x {f_scale:.4f} + WRITE_SIZE KiB x 1024 x "
             f"{w_scale:.4f}",
             f"# native source (csrc/) sha256[:16]: {sha}",
             f"{'kernel':40s} {'grid':>9s} {'disp':>5s} {'FETCH KiB':>12s} {'WRITE KiB':>12s} "
             f"{'bytes/launch':>13s}"]
    best = {}
    for (k, grid), vals in sorted(groups.items()):
        fv = sum(v[0] for v in vals) / len(vals)
        wv = sum(v[1] for v in vals) / len(vals)
        b = fv * 1024 * f_scale + wv * 1024 * w_scale
        lines.append(f"{k[:40]:40s} {grid:9d} {len(vals):5d} {fv:12.1f} {wv:12.1f} {b:13.4e}")
        # per kernel: the launch shape issued most often (the decode loop's)
        if k not in best or len(vals) > best[k]["dispatches"]:
            best[k] = {"grid": grid, "dispatches": len(vals), "fetch_kib": fv, "write_kib": wv,
                       "bytes_per_launch": b, "source_sha256_16": sha}
    doc.update(best)
    json.dump(doc, open(out_json, "w"), indent=1)
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


SIMDS, CUS, XCDS = 1024, 256, 8


def counters(out_txt: str, dirs, command: str, kernels=None) -> None:
    """Per-kernel counters per dispatch over the given --pmc runs: each run's
    total for a kernel over the number of its dispatches in that run. A
    counter taken in several runs (the GRBM_GUI_ACTIVE reference) is averaged
    over them."""
    vals = defaultdict(lambda: defaultdict(list))  # kernel -> counter -> per-run means
    durs = defaultdict(list)                        # kernel -> dispatch durations (s)
    for d in dirs:
        run = defaultdict(lambda: defaultdict(float))
        spans = {}
        for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
            k = short_name(r["Kernel_Name"])
            if kernels and k not in kernels:
                continue
            run[k][r["Counter_Name"]] += float(r["Counter_Value"])
            spans[(k, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        n_disp = defaultdict(int)
        for (k, _), t in spans.items():
            durs[k].append(t)
            n_disp[k] += 1
        for k, c in run.items():
            for name, v in c.items():
                vals[k][name].append(v / n_disp[k])
    lines = ["# rocprofv3 --pmc counters per kernel and dispatch (summed over the XCDs and shader",
             "# engines, averaged over the kernel's dispatches; GRBM_GUI_ACTIVE averaged over the",
             "# runs that took it)",
             f"# command: {command}",
             f"# native source (csrc/) sha256[:16]: {source_sha()}"]
    for k, cl in vals.items():
        c = {name: sum(v) / len(v) for name, v in cl.items()}
        gui = c.get("GRBM_GUI_ACTIVE", 0.0) / XCDS  # active cycles of one XCD
        lines.append(f"{k}")
        for name in sorted(c):
            lines.append(f"    {name:32s} {c[name]:.6e}")
        if gui <= 0:
            continue
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            lines.append(f"    MFMA busy / (active cycles x SIMDs)        {c['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui * SIMDS):.3f}")
        if "SQ_LDS_IDX_ACTIVE" in c:
            lines.append(f"    LDS active / (active cycles x CUs)         {c['SQ_LDS_IDX_ACTIVE'] / (gui * CUS):.3f}")
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in c:
            lines.append(f"    MFMA+VALU co-issue / (active x SIMDs)      {c['SQ_VALU_MFMA_COEXEC_CYCLES'] / (gui * SIMDS):.3f}")
        if "SQ_INSTS_MFMA" in c and "SQ_INSTS_VALU" in c:
            lines.append(f"    non-MFMA VALU instructions per MFMA        {(c['SQ_INSTS_VALU'] - c['SQ_INSTS_MFMA']) / c['SQ_INSTS_MFMA']:.2f}")
        if durs[k]:
            t = sum(durs[k]) / len(durs[k])
            lines.append(f"    mean dispatch duration                     {t * 1e3:.3f} ms")
            lines.append(f"    effective engine clock (active / duration) {gui / t / 1e9:.3f} GHz")
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _main(argv):
    if argv[:1] == ["stats"] and "--" in argv:
        i = argv.index("--")
        stats(argv[1], argv[2], " ".join(argv[i + 1:]), argv[3] if i > 3 else None)
    elif argv[:1] == ["counters"] and "--" in argv:
        i = argv.index("--")
        counters(argv[1], argv[2:i], " ".join(argv[i + 1:]),
                 kernels={"attn_wide_kernel<128, 8, 1, true, false, 0, false>"})
    elif argv[:1] == ["traffic"] and "--" in argv:
        i = argv.index("--")
        cmds = " ".join(argv[i + 1:]).split(" ;; ")
        traffic(argv[1], argv[2], argv[3], argv[4], cmds)
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(_main(sys.argv[1:]))
