"""Pins for the chunked-prefill oracle (oracle/prefill.py), none of which re-types it:

* a library routine: torch's scaled_dot_product_attention in float64 with an explicit
  causal mask anchored at each sequence's chunk start, over a cache the test writes
  logically and only then scatters into pages;
* brute force: scalar loops over the flat pool on tiny inputs;
* special cases: a one-token chunk is the decode oracle's result, and the last row of
  every chunk sees the whole sequence, also the decode result;
* causality: changing the cache after a row's position leaves that row unchanged;
* planted mistakes (a mask one token short, a mask anchored at 0, a chunk's rows
  reversed) must fail at least one pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import prefill as prefill_mod
from decode_phase_attention_paged_amd.workload import Config, generate

TINY = Config(0, "tiny_prefill", batch=3, n_q_heads=4, n_kv_heads=2, head_dim=8, block_size=4,
              len_lo=5, len_hi=30, kv_dtype="fp16")


def chunked(cfg, seed, chunks=None):
    """A workload plus chunk sizes C_b <= L_b (at least one full-length chunk, one of 1)
    and the stacked query rows for them."""
    w = generate(cfg, seed=seed)
    rng = np.random.default_rng(seed)
    lens = w.seq_lens
    if chunks is None:
        chunks = np.array([rng.integers(1, int(n) + 1) for n in lens])
        chunks[0] = lens[0]
        chunks[-1] = 1
    q_start = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = rng.standard_normal((int(q_start[-1]), cfg.n_q_heads, cfg.head_dim)).astype(np.float16)
    return w, q, q_start


def run(w, q, q_start, **kw):
    return oracle.prefill_attention(q, w.k_pages, w.v_pages, w.block_table, w.seq_lens,
                                    q_start, w.scale, w.k_scale, w.v_scale, **kw)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_matches_torch_sdpa_with_causal_mask(seed):
    w, q, q_start = chunked(TINY, seed)
    out, _ = run(w, q, q_start, out_dtype=np.float64)
    bs, g = TINY.block_size, TINY.n_q_heads // TINY.n_kv_heads
    for b in range(TINY.batch):
        n = int(w.seq_lens[b])
        c = int(q_start[b + 1] - q_start[b])
        # Logical K/V read token by token from the pages, then repeated over the group.
        k = np.stack([w.k_pages[w.block_table[b, t // bs], :, t % bs] for t in range(n)], 1)
        v = np.stack([w.v_pages[w.block_table[b, t // bs], :, t % bs] for t in range(n)], 1)
        kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(g, 0)
        vt = torch.from_numpy(v.astype(np.float64)).repeat_interleave(g, 0)
        qt = torch.from_numpy(q[q_start[b]:q_start[b + 1]].astype(np.float64)).transpose(0, 1)
        mask = torch.tensor([[j <= n - c + i for j in range(n)] for i in range(c)])
        want = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, scale=float(np.float32(w.scale)))
        np.testing.assert_allclose(out[q_start[b]:q_start[b + 1]],
                                   want.transpose(0, 1).numpy(), rtol=1e-10, atol=1e-12)


def test_brute_force_scalar_loops():
    w, q, q_start = chunked(TINY.with_(block_size=2, len_hi=12), 4)
    c = w.config
    out, lse = run(w, q, q_start, out_dtype=np.float64)
    kf = w.k_pages.astype(np.float64).ravel().tolist()
    vf = w.v_pages.astype(np.float64).ravel().tolist()
    sigma = float(np.float32(w.scale))
    g, d, bs, hkv = c.n_q_heads // c.n_kv_heads, c.head_dim, c.block_size, c.n_kv_heads
    for b in range(c.batch):
        n = int(w.seq_lens[b])
        for row in range(int(q_start[b]), int(q_start[b + 1])):
            pos = n - (int(q_start[b + 1]) - row)
            for h in range(c.n_q_heads):
                flat = [((int(w.block_table[b][t // bs]) * hkv + h // g) * bs + t % bs)
                        for t in range(pos + 1)]
                s = [sigma * math.fsum(float(q[row, h, i]) * kf[r * d + i] for i in range(d))
                     for r in flat]
                top = max(s)
                e = [math.exp(x - top) for x in s]
                tot = math.fsum(e)
                assert lse[row, h] == pytest.approx(top + math.log(tot), abs=1e-12)
                for i in range(d):
                    want = math.fsum(p * vf[r * d + i] for p, r in zip(e, flat)) / tot
                    assert out[row, h, i] == pytest.approx(want, abs=1e-12)


def test_one_token_chunks_are_decode_attention():
    w = generate(TINY, seed=5)
    q_start = np.arange(TINY.batch + 1, dtype=np.int32)
    out, lse = run(w, w.q, q_start, out_dtype=np.float64)
    want, want_lse = oracle.decode_attention(w.q, w.k_pages, w.v_pages, w.block_table,
                                             w.seq_lens, w.scale, out_dtype=np.float64)
    assert np.array_equal(out, want) and np.array_equal(lse, want_lse)


def test_last_chunk_row_sees_the_whole_sequence():
    w, q, q_start = chunked(TINY, 6)
    out, lse = run(w, q, q_start, out_dtype=np.float64)
    last = q_start[1:] - 1
    want, want_lse = oracle.decode_attention(q[last], w.k_pages, w.v_pages, w.block_table,
                                             w.seq_lens, w.scale, out_dtype=np.float64)
    np.testing.assert_allclose(out[last], want, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[last], want_lse, rtol=1e-12, atol=1e-14)


def test_future_tokens_do_not_leak():
    w, q, q_start = chunked(TINY, 7, chunks=np.array([6, 4, 1]))
    base, _ = run(w, q, q_start, out_dtype=np.float64)
    bs = TINY.block_size
    for b in range(TINY.batch):
        n = int(w.seq_lens[b])
        c = int(q_start[b + 1] - q_start[b])
        for i in range(c - 1):
            pos = n - c + i
            k2, v2 = w.k_pages.copy(), w.v_pages.copy()
            for t in range(pos + 1, n):
                k2[w.block_table[b, t // bs], :, t % bs] = 50.0
                v2[w.block_table[b, t // bs], :, t % bs] = -50.0
            got, _ = oracle.prefill_attention(q, k2, v2, w.block_table, w.seq_lens, q_start,
                                              w.scale, out_dtype=np.float64)
            row = int(q_start[b]) + i
            assert np.array_equal(got[row], base[row])
            assert not np.array_equal(got[row + 1:q_start[b + 1]], base[row + 1:q_start[b + 1]])


def test_rejects_bad_chunk_layouts():
    w, q, q_start = chunked(TINY, 8)
    with pytest.raises(ValueError):
        run(w, q, q_start[::-1].copy())
    bad = q_start.copy()
    bad[1] = w.seq_lens[0] + 1
    bad[2:] += bad[1] - q_start[1]
    qq = np.zeros((int(bad[-1]),) + q.shape[1:], dtype=np.float16)
    with pytest.raises(ValueError):
        run(w, qq, bad)


# --------------------------------------------------------------------------- planted mistakes

_REAL_ATTEND = prefill_mod.attend


def pins_pass():
    checks = [lambda: test_matches_torch_sdpa_with_causal_mask(1),
              test_brute_force_scalar_loops, test_one_token_chunks_are_decode_attention,
              test_last_chunk_row_sees_the_whole_sequence, test_future_tokens_do_not_leak]
    for check in checks:
        try:
            check()
        except AssertionError:
            return False
    return True


def test_pins_pass_on_the_real_oracle():
    assert pins_pass()


def _short_by_one(q, keys, values, scale):
    n = keys.shape[0]
    return _REAL_ATTEND(q, keys[:max(n - 1, 1)], values[:max(n - 1, 1)], scale)


def _mutant(row_position, row_query):
    """The oracle's loop with the row -> position and row -> query maps replaced."""
    def prefill(q, k_pages, v_pages, block_table, seq_lens, q_start, scale, k_scale=None,
                v_scale=None, out_dtype=np.float32):
        n_kv, bs = k_pages.shape[1], k_pages.shape[2]
        g = q.shape[1] // n_kv
        out = np.zeros(q.shape, dtype=np.float64)
        lse = np.full(q.shape[:2], -np.inf)
        for b in range(len(seq_lens)):
            n = int(seq_lens[b])
            c = int(q_start[b + 1] - q_start[b])
            keys = oracle.gather_sequence(k_pages, block_table[b], n, bs).astype(np.float64)
            vals = oracle.gather_sequence(v_pages, block_table[b], n, bs).astype(np.float64)
            for i in range(c):
                row = int(q_start[b]) + i
                vis = row_position(n, c, i) + 1
                for h in range(q.shape[1]):
                    o, l, _ = oracle.attend(q[row_query(q_start, b, c, i), h].astype(np.float64),
                                            keys[h // g, :vis], vals[h // g, :vis],
                                            float(np.float32(scale)))
                    out[row, h], lse[row, h] = o, l
        return out.astype(out_dtype), lse
    return prefill


MUTANTS = {
    "mask anchored at 0": _mutant(lambda n, c, i: i, lambda qs, b, c, i: int(qs[b]) + i),
    "rows of a chunk reversed": _mutant(lambda n, c, i: n - c + i,
                                        lambda qs, b, c, i: int(qs[b]) + c - 1 - i),
}


def test_mutant_harness_is_faithful():
    # With the right maps the rewritten loop agrees with the oracle, so the mutants below
    # differ from it only in the planted map.
    w, q, q_start = chunked(TINY, 9)
    good = _mutant(lambda n, c, i: n - c + i, lambda qs, b, c, i: int(qs[b]) + i)
    a = good(q, w.k_pages, w.v_pages, w.block_table, w.seq_lens, q_start, w.scale,
             out_dtype=np.float64)
    b = run(w, q, q_start, out_dtype=np.float64)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-13, atol=1e-15)


def test_planted_short_mask_fails_a_pin(monkeypatch):
    monkeypatch.setattr(prefill_mod, "attend", _short_by_one)
    assert not pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail_a_pin(monkeypatch, name):
    monkeypatch.setattr(oracle, "prefill_attention", MUTANTS[name])
    assert not pins_pass(), f"planted mistake not caught: {name}"


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
def test_one_token_chunks_are_decode_attention_in_every_format(kv):
    # The prefill and decode oracles decode the stored formats through the same pinned
    # routines; one-token chunks must give the decode result bit for bit in each format.
    cfg = TINY.with_(kv_dtype=kv)
    w = generate(cfg, seed=8)
    q_start = np.arange(cfg.batch + 1, dtype=np.int32)
    out, lse = run(w, w.q, q_start, out_dtype=np.float64)
    want, want_lse = oracle.decode_attention(w.q, w.k_pages, w.v_pages, w.block_table,
                                             w.seq_lens, w.scale, w.k_scale, w.v_scale,
                                             out_dtype=np.float64)
    assert np.array_equal(out, want) and np.array_equal(lse, want_lse)


@pytest.mark.parametrize("kv", ["int8", "fp8"])
def test_coded_rows_equal_their_dequantised_values(kv):
    # A coded cache with row scales gives the prefill result of a float64 cache holding
    # code x scale, row by row: pins that each row takes its own scale, K's for K and V's
    # for V.
    cfg = TINY.with_(kv_dtype=kv)
    w, _, q_start = chunked(cfg, 9)
    rng = np.random.default_rng(9)
    q = rng.standard_normal((int(q_start[-1]), cfg.n_q_heads, cfg.head_dim)).astype(np.float16)
    out, lse = run(w, q, q_start, out_dtype=np.float64)
    kd = oracle.element_values(w.k_pages) * w.k_scale[..., None].astype(np.float64)
    vd = oracle.element_values(w.v_pages) * w.v_scale[..., None].astype(np.float64)
    want, want_lse = oracle.prefill_attention(q, kd, vd, w.block_table, w.seq_lens, q_start,
                                              w.scale, out_dtype=np.float64)
    np.testing.assert_allclose(out, want, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, want_lse, rtol=1e-13, atol=1e-15)
    swapped, _ = oracle.prefill_attention(q, w.k_pages, w.v_pages, w.block_table, w.seq_lens,
                                          q_start, w.scale, w.v_scale, w.k_scale,
                                          out_dtype=np.float64)
    assert not np.allclose(swapped, want, rtol=1e-6, atol=1e-9)
