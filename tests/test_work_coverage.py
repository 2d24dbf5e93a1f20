"""Host replay of the kernels' workgroup -> work mapping at full size.

tests/host/coverage_driver.cpp walks every workgroup, wave and lane of each
launch (phase 1, the phase-2 query step and decode steps) through the same
mapping functions the kernels call on blockIdx (csrc/star_internal.hpp) and
checks that every output and every split partial is written exactly once,
that every work item is taken once, that the key tiles of each workgroup are
exactly its rows' key sets (hotaipapers.com podcast, Phase 1 description:
every block is processed, each row attending to the anchor and to its own
block causally; Phase 2 description: every host's cached rows answer the
query), and that every loaded row lies inside the cache buffer and below the
rows already written.

Shapes: the five workloads of the scope table, the sweep variants at full
size, and seeded small shapes that reach the other branches of the maps
(several head sub-groups and query tiles, ragged blocks, the blockwise decode
plan, head_dim 64). Host code only: built with g++ under ASan and UBSan."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from long_context_attention_phase1_amd import synthetic as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _line(name, B, Hq, Hkv, d, L, b, a, Tq, Td, f32=False):
    return f"{name} {B} {Hq} {Hkv} {d} {L} {b} {a} {Tq} {Td} {1 if f32 else 0}"


def _shapes():
    lines = []
    for w in list(syn.WORKLOADS.values()) + list(syn.SWEEPS.values()):
        lines.append(_line(w.name, w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx_len,
                           w.block_len, w.anchor_len, w.n_query, w.n_decode, w.dtype == "f32"))
    rng = np.random.default_rng(2024)
    for k in range(60):
        Hkv = int(rng.integers(1, 9))
        G = int(rng.choice([1, 2, 3, 4, 6, 8]))
        B = int(rng.integers(1, 5))
        L = int(rng.integers(1, 6000))
        b = int(rng.integers(1, L + 1))
        a = int(rng.integers(1, b + 1))
        Tq = int(rng.integers(1, 300))
        Td = int(rng.integers(1, 40))
        d = 64 if k % 3 == 0 else 128
        lines.append(_line(f"random_{k}", B, Hkv * G, Hkv, d, L, b, a, Tq, Td))
    # branches the random draws may miss: 8 kv-head groups of 2 sub-groups
    # with several query tiles (phase 2's kv-head-major map), many more
    # groups than XCDs, blocks shorter than a decode range (blockwise plan)
    lines.append(_line("kv_major", 2, 32, 4, 128, 4096, 1024, 1024, 300, 8))
    lines.append(_line("many_groups", 8, 16, 8, 64, 2048, 512, 512, 40, 4))
    lines.append(_line("short_blocks", 1, 8, 2, 128, 70000, 100, 60, 5, 6))
    lines.append(_line("unaligned", 3, 12, 3, 128, 9001, 777, 333, 70, 9))
    # query steps of at most half a query tile (four and two heads per workgroup)
    lines.append(_line("short_tile_g4", 1, 8, 2, 128, 2100, 512, 300, 24, 2))
    lines.append(_line("short_tile_g2", 2, 4, 2, 64, 3000, 700, 200, 40, 3))
    # fp32 shapes (the fp32 matrix-core kernel): ragged blocks, blocks shorter
    # than a 32-row group, GQA, several column groups per kv head
    lines.append(_line("f32_ragged", 2, 4, 2, 64, 333, 100, 37, 5, 2, f32=True))
    lines.append(_line("f32_short_blocks", 1, 8, 2, 128, 200, 20, 7, 70, 3, f32=True))
    lines.append(_line("f32_g1", 1, 3, 3, 64, 97, 97, 97, 40, 2, f32=True))
    return "\n".join(lines) + "\n"


def test_every_work_item_once_and_every_address_in_bounds(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "coverage_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "long_context_attention_phase1_amd", "csrc"),
           os.path.join(ROOT, "long_context_attention_phase1_amd", "csrc", "star_host.cpp"),
           os.path.join(ROOT, "tests", "host", "coverage_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    shapes = _shapes()
    r = subprocess.run([exe], input=shapes, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    n = shapes.count("\n")
    assert f"all checks passed ({n} shapes)" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
