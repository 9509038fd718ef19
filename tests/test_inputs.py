"""The seeded generators: determinism, shapes, and the structure each workload promises."""

import numpy as np

import mla_inputs as MI


def test_tiny_shapes_and_determinism():
    a, b = MI.tiny(), MI.tiny()
    assert np.array_equal(a.kv_rows, b.kv_rows) and np.array_equal(a.w_uv, b.w_uv)
    assert a.seq_lens.tolist() == [37, 100]
    assert a.q_nope.shape == (2, 1, 16, 128) and a.q_pe.shape == (2, 1, 16, 64)
    assert a.w_uk_t.shape == (16, 128, 512) and a.w_uv.shape == (16, 512, 128)
    assert a.kv_rows.shape == (16, 64, 576)


def test_block_tables_are_distinct_pages():
    w = MI.make_workload("t", 5, 2, 4, [1, 64, 65, 300, 0], 20, MI.KV_BF16, False, 3)
    used = w.block_table[w.block_table >= 0]
    assert len(set(used.tolist())) == used.size and used.max() < w.num_pages
    for b, s in enumerate(w.seq_lens):
        n = (int(s) + 63) // 64
        assert np.all(w.block_table[b, :n] >= 0) and np.all(w.block_table[b, n:] == -1)


def test_new_slots_point_at_last_positions():
    w = MI.make_workload("t", 3, 2, 4, [5, 64, 130], 8, MI.KV_BF16, False, 4)
    for b in range(3):
        for t in range(2):
            pos = int(w.seq_lens[b]) - 2 + t
            slot = w.new_slots[b * 2 + t]
            assert slot == w.block_table[b, pos // 64] * 64 + pos % 64


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 3.0e38], np.float32)
    bits = MI.to_bf16_bits(x)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F62]


def test_named_workload_sizes():
    w = MI.spec_long()
    assert w.q_len == 2 and w.N == 128 and w.num_pages == 5100
    assert w.seq_lens.tolist() == [131072, 65536, 32768, 16384, 8192, 4096, 2048, 1024]


def test_random_fp8_rows_have_no_nan_codes():
    rows = MI.random_fp8_rows(np.random.default_rng(0), 100)
    codes = rows[:, :576]
    assert not np.any((codes & 0x7F) == 0x7F)
    assert rows.shape == (100, 584)
