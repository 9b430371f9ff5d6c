"""Seeded generator: determinism, layout, poison placement (no GPU)."""
import numpy as np

import workloads
from workloads import CONFIGS, custom_spec, make_workload


def test_same_seed_same_arrays():
    a = make_workload("c1")
    b = make_workload("c1")
    for x, y in [(a.q, b.q), (a.k_cache, b.k_cache), (a.v_cache, b.v_cache),
                 (a.block_tables, b.block_tables), (a.k_new, b.k_new)]:
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_chunking_does_not_depend_on_threads(monkeypatch):
    spec = custom_spec(2, 2, 1, 64, 16, "bf16", ctx=[5000, 3000])
    a = make_workload(spec, seed=3)
    monkeypatch.setattr(workloads, "_threads", lambda: 1)
    b = make_workload(spec, seed=3)
    assert np.array_equal(a.k_cache, b.k_cache)
    assert np.array_equal(a.v_cache, b.v_cache)


def test_config1_layout():
    w = make_workload("c1")
    s = CONFIGS["c1"]
    assert w.k_cache.shape == (40, 16, 2, 64) and w.k_cache.dtype == np.float32
    assert list(w.context_lens) == [17, 64, 100, 255]
    assert w.block_tables.shape == (4, 16)
    used = (w.block_tables >= 0).sum()
    assert used == 2 + 5 + 7 + 16  # ceil((ctx + 1) / 16) per sequence
    ids = w.block_tables[w.block_tables >= 0]
    assert len(set(ids.tolist())) == len(ids)
    assert abs(w.scale - 1 / 8) < 1e-9 and s.max_blocks_per_seq == 16


def test_poison_marks_exactly_unattended_slots():
    w = make_workload("c1")
    nan_k = np.isnan(w.k_cache).all(axis=(2, 3))
    attended = np.zeros_like(nan_k)
    for b in range(4):
        for t in range(int(w.context_lens[b])):
            attended[w.block_tables[b, t // 16], t % 16] = True
    assert np.array_equal(~nan_k, attended)
    assert np.isnan(w.k_cache).any(axis=(2, 3)).sum() == nan_k.sum()


def test_slot_mapping_points_at_next_position():
    w = make_workload("c1")
    for b in range(4):
        L = int(w.context_lens[b])
        assert w.slot_mapping[b] == w.block_tables[b, L // 16] * 16 + L % 16


def test_bf16_is_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.4e38], dtype=np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    # 1 + 2^-8 is a tie -> even (1.0); 1 + 3*2^-8 is a tie -> even (1 + 2^-6)
    assert list(bits[:4]) == [0x3F80, 0x3F80, 0x3F82, 0xC020]
    assert np.array_equal(workloads.bf16_bits_to_f32(bits[:4]),
                          np.array([1.0, 1.0, 1.015625, -2.5], np.float32))


def test_accounting_c3_expectation():
    s = CONFIGS["c3"]
    w = make_workload(custom_spec(2, 64, 8, 128, 16, "bf16", ctx=[1024, 8192]))
    assert workloads.kv_read_bytes(w) == (1024 + 8192) * 4096
    assert workloads.algorithmic_flops(w) == 2 * 64 * 256 * (1024 + 8192)
    assert s.max_blocks_per_seq == 513
