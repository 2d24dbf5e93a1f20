"""The seeded input generator: determinism, seekability, rounding, peaked rows."""
import numpy as np
import pytest
import torch

from long_context_attention_phase1_amd import synthetic as syn


def _small(**kw):
    w = syn.Workload("t", 2, 4, 2, 8, 9000, 4096, 4096, 3, 2, "bf16")
    return w.replace(**kw)


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -3.0e-39, 65504.0, 0.0, -0.0],
                                 dtype=np.float32)])
    ours = syn.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = syn.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_seekable_rows_equal_full_tensor():
    w = _small()
    full = syn.full_tensor(w, syn.T_K, threads=4)
    assert full.shape == (2, 9000, 2, 8) and full.dtype == np.uint16
    for s, a, b in ((0, 0, 5), (1, 4090, 4100), (1, 8999, 9000), (0, 8192, 9000)):
        assert np.array_equal(syn.rows(w, syn.T_K, s, a, b), full[s, a:b])
    again = syn.full_tensor(w, syn.T_K, threads=1)
    assert np.array_equal(full, again)


def test_streams_are_distinct_and_normal():
    w = _small()
    q = syn.to_f64(syn.full_tensor(w, syn.T_QCTX), "bf16")
    k = syn.to_f64(syn.full_tensor(w, syn.T_K), "bf16")
    assert not np.array_equal(q[:, :, :2], k)
    assert abs(q.mean()) < 0.01 and abs(q.std() - 1.0) < 0.01
    assert not np.array_equal(q[0], q[1])


def test_peaked_rows():
    w = _small(peak_frac=0.01, peak_factor=8.0)
    plain = syn.full_tensor(w.replace(peak_frac=0.0), syn.T_K)
    peaked = syn.full_tensor(w, syn.T_K)
    pk = syn.peaked_rows(w, 1)
    assert pk.shape == (2, 90)
    for g in range(2):
        assert len(set(pk[g].tolist())) == 90
        a = syn.to_f64(plain[1, :, g], "bf16")
        b = syn.to_f64(peaked[1, :, g], "bf16")
        changed = np.nonzero(np.any(a != b, axis=1))[0]
        assert set(changed.tolist()) <= set(pk[g].tolist())
        np.testing.assert_array_equal(b[pk[g]], 8.0 * a[pk[g]])


def test_f32_workload_values():
    w = syn.WORKLOADS["tiny_f32"]
    x = syn.full_tensor(w, syn.T_V)
    assert x.dtype == np.float32 and x.shape == (1, 512, 1, 64)
    t = syn.full_tensor(w, syn.T_QTAIL)
    assert t.shape == (1, 24, 1, 64)


def test_sweeps_vary_only_the_intended_sizes():
    """Each sweep variant is the 128K workload with only its block sizes (or
    context length) changed and 64 decode steps; lookup by name covers both
    tables."""
    base = syn.WORKLOADS["llama8b_128k_peaked"]
    changed = {
        "sweep_128k_b32k": {"block_len": 32768, "anchor_len": 32768},
        "sweep_128k_b8k": {"block_len": 8192, "anchor_len": 8192},
        "sweep_128k_b4k": {"block_len": 4096, "anchor_len": 4096},
        "sweep_128k_a4k_b16k": {"anchor_len": 4096},
        "sweep_125k_ragged": {"ctx_len": 125003},
    }
    assert set(changed) == set(syn.SWEEPS)
    for name, kw in changed.items():
        w = syn.workload(name)
        assert w == base.replace(name=name, n_decode=64, **kw)
        assert w.anchor_len <= w.block_len
    r = syn.workload("sweep_125k_ragged")
    assert r.ctx_len % r.block_len != 0 and r.ctx_len % 64 != 0 and r.n_blocks == 8
    assert syn.workload("llama8b_32k") is syn.WORKLOADS["llama8b_32k"]
    with pytest.raises(KeyError):
        syn.workload("nope")
