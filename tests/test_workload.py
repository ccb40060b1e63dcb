"""Seeded input generator and byte accounting (CPU only)."""

import json
import os

import numpy as np
import pytest

from decode_phase_attention_paged_amd.workload import (CONFIGS, Config, generate, kv_read_bytes,
                                                     prefill_flops, prefill_rows)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_kv_bytes_reproduce_the_xllm_memory_table():
    """xLLM README memory table: the KV-cache row prints 30 (GiB) for llama2-7B."""
    with open(os.path.join(GOLDEN, "xllm_kv_memory_table.json")) as f:
        g = json.load(f)
    p = g["params"]
    tokens = -(-(p["s"] + p["n"]) // p["granule_tokens"]) * p["granule_tokens"]
    # h1 = Hkv * D with the Llama-2-7B head shape (32 heads of 128).
    per_layer = kv_read_bytes([tokens] * p["b"], 32, p["h1"] // 32, p["dtype_bytes"])
    assert per_layer * p["L"] / 2**30 == pytest.approx(g["printed_kv_cache_G"], abs=0.05)


def test_kv_bytes_int8_counts_row_scales():
    assert kv_read_bytes([3, 5], 2, 128, 1, 4) == 8 * 2 * 2 * (128 + 4)


SMALL = Config(0, "small", batch=5, n_q_heads=4, n_kv_heads=2, head_dim=128, block_size=16,
               len_lo=1, len_hi=100, kv_dtype="fp16")


def test_same_seed_same_arrays():
    a, b = generate(SMALL, seed=3), generate(SMALL, seed=3)
    for name in ("q", "k_pages", "v_pages", "block_table", "seq_lens"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    c = generate(SMALL, seed=4)
    assert not np.array_equal(a.k_pages, c.k_pages) or not np.array_equal(a.seq_lens, c.seq_lens)


@pytest.mark.parametrize("extra", [0, 5])
def test_block_table_is_a_partition_of_the_pool(extra):
    w = generate(SMALL, seed=1, extra_pages=extra)
    bs = SMALL.block_size
    used = []
    for b in range(SMALL.batch):
        nb = -(-int(w.seq_lens[b]) // bs)
        assert np.all(w.block_table[b, :nb] >= 0)
        assert np.all(w.block_table[b, nb:] == -1)
        used.extend(w.block_table[b, :nb].tolist())
    assert len(set(used)) == len(used)
    assert w.num_pages == len(used) + extra
    assert max(used) < w.num_pages
    assert SMALL.len_lo <= w.seq_lens.min() and w.seq_lens.max() <= SMALL.len_hi


def test_config_shapes_and_presets():
    assert [CONFIGS[i].max_blocks_per_seq for i in range(1, 6)] == [16, 36, 256, 8192, 34]
    w = generate(CONFIGS[1])
    assert w.k_pages.shape == (16, 8, 16, 128) and w.k_pages.dtype == np.float16
    assert np.array_equal(w.block_table[0], np.arange(16))
    assert w.seq_lens.tolist() == [256]
    assert w.scale == np.float32(1 / np.sqrt(128))


def test_int8_preset_ranges():
    w = generate(CONFIGS[5])
    assert w.k_pages.dtype == np.int8 and w.k_scale.dtype == np.float32
    assert w.k_pages.min() >= -127 and w.v_pages.min() >= -127
    assert w.k_pages.max() <= 127
    assert 0.005 <= w.k_scale.min() and w.v_scale.max() <= 0.02
    assert w.block_table.shape == (200, 34)
    assert 18 <= w.seq_lens.min() and w.seq_lens.max() <= 530


def test_peaky_rows_scaled_by_eight():
    cfg = CONFIGS[4].with_(len_lo=4096, len_hi=4096)
    w = generate(cfg)
    plain = generate(cfg.with_(peaky_fraction=0.0))
    # Same draws up to the peaky rows: scaled rows are exactly 8x (fp16 of 8x fp32).
    ratio_rows = np.any(w.k_pages != plain.k_pages, axis=-1)      # [NP, Hkv, bs]
    assert ratio_rows.sum(axis=(0, 2)).tolist() == [round(0.01 * 4096)] * cfg.n_kv_heads
    sel = ratio_rows
    big = w.k_pages[sel].astype(np.float32)
    small = plain.k_pages[sel].astype(np.float32)
    np.testing.assert_allclose(big, 8 * small, rtol=2e-3, atol=1e-2)


def test_poison_marks_only_unowned_slots():
    w = generate(SMALL, seed=2, extra_pages=3, poison=True)
    bs = SMALL.block_size
    valid = np.zeros(w.k_pages.shape[:3], dtype=bool)  # [NP, Hkv, bs]
    for b in range(SMALL.batch):
        for t in range(int(w.seq_lens[b])):
            valid[w.block_table[b, t // bs], :, t % bs] = True
    nan_rows = np.isnan(w.k_pages).all(axis=-1)
    assert np.array_equal(nan_rows, ~valid)


def test_bf16_and_fp8_presets_draw_the_stated_values():
    from decode_phase_attention_paged_amd.workload import CONFIGS
    wb = generate(CONFIGS[6].with_(batch=4), seed=6)
    assert wb.q.dtype == np.uint16 and wb.k_pages.dtype == np.uint16 and wb.k_scale is None
    vals = (wb.k_pages.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isfinite(vals)) and 0.9 < vals.std() < 1.1
    wf = generate(CONFIGS[7].with_(batch=4), seed=7)
    assert wf.k_pages.dtype == np.uint8 and wf.k_scale.dtype == np.float32
    codes = np.concatenate([wf.k_pages.ravel(), wf.v_pages.ravel()])
    assert not np.isin(codes, [0x7F, 0xFF]).any()
    assert len(np.unique(codes)) == 254
    assert wf.k_scale.min() >= 0.005 * 127 / 448 * 0.999 and wf.k_scale.max() <= 0.02 * 127 / 448
    assert wf.kv_bytes == int(wf.seq_lens.sum()) * 32 * 2 * (128 + 4)
    assert wb.kv_bytes == int(wb.seq_lens.sum()) * 32 * 2 * 256


def test_prefill_flops_count_every_visible_pair():
    # Brute force: every (chunk row, visible token) pair costs 4 D flops per query head.
    lens = np.array([5, 1, 9, 16], dtype=np.int32)
    q_start = np.array([0, 3, 4, 13, 13], dtype=np.int32)      # chunks 3, 1, 9, 0
    pairs = 0
    for b, n in enumerate(lens):
        c = int(q_start[b + 1] - q_start[b])
        for i in range(c):
            pairs += sum(1 for t in range(n) if t <= n - c + i)
    assert prefill_flops(lens, q_start, 6, 8) == pairs * 6 * 4 * 8


def test_prefill_rows_layout_and_formats():
    w = generate(CONFIGS[8].with_(batch=3, len_lo=20, len_hi=900))
    q, q_start = prefill_rows(w)
    assert q.dtype == np.float16 and q_start.dtype == np.int32
    np.testing.assert_array_equal(np.diff(q_start), np.minimum(w.seq_lens, 512))
    assert q.shape == (int(q_start[-1]), 32, 128)
    wb = generate(CONFIGS[8].with_(batch=3, len_lo=20, len_hi=900, kv_dtype="bf16"))
    qb, _ = prefill_rows(wb)
    assert qb.dtype == np.uint16                     # bf16 bit patterns for a bf16 cache
    # Drawn from their own stream: the workload's arrays are the same with or without them.
    w2 = generate(CONFIGS[8].with_(batch=3, len_lo=20, len_hi=900))
    np.testing.assert_array_equal(w.k_pages, w2.k_pages)
    np.testing.assert_array_equal(q, prefill_rows(w2)[0])
