"""Pins for the storage-format decoders of the oracle (oracle/formats.py) and for
attention over BF16 and FP8 caches, none of which re-types the decoders:

* library routines: torch's own bfloat16 and float8_e4m3fn conversions on the CPU,
  over every bit pattern;
* values the formats' definitions fix: 1.0, the largest finite E4M3 magnitude 448,
  the smallest normal 2^-6 and subnormal 2^-9, signed zeros, the NaN codes, the
  bf16 infinity and smallest subnormal;
* brute force: the scalar-loop attention of test_oracle.py over pools decoded by
  torch, against the oracle over the raw bit patterns;
* cross-format identities: a BF16 cache whose values fp16 holds exactly gives the
  fp16 result bit for bit, and an FP8 cache whose codes decode to small integers
  gives the INT8 result on those integers and scales bit for bit;
* planted mistakes in the decoders must fail at least one pin.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import decode as decode_mod
from oracle import formats as fmt
from decode_phase_attention_paged_amd.workload import Config, Workload, generate

from test_oracle import brute_force

TINY_BF16 = Config(0, "tiny_bf16", batch=2, n_q_heads=4, n_kv_heads=2, head_dim=8,
                   block_size=4, len_lo=1, len_hi=40, kv_dtype="bf16")
TINY_FP8 = TINY_BF16.with_(name="tiny_fp8", kv_dtype="fp8", n_kv_heads=4)


def torch_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def torch_e4m3(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def same(a, b):
    """Equal values, NaN where the other is NaN, and equal signs of zero."""
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    nan = np.isnan(a)
    return (np.array_equal(nan, np.isnan(b)) and np.array_equal(a[~nan], b[~nan])
            and np.array_equal(np.signbit(a[~nan]), np.signbit(b[~nan])))


# --------------------------------------------------------------------------- decoders

def test_bf16_matches_torch_on_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    assert same(fmt.bf16_to_float64(bits), torch_bf16(bits))


def test_e4m3_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    assert same(fmt.e4m3_to_float64(codes), torch_e4m3(codes))


def test_e4m3_fixed_points():
    v = fmt.e4m3_to_float64(np.array([0x38, 0xB8, 0x7E, 0xFE, 0x08, 0x01, 0x07, 0x00, 0x80,
                                      0x7F, 0xFF, 0x40, 0x30], dtype=np.uint8))
    assert v[:9].tolist() == [1.0, -1.0, 448.0, -448.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9,
                              0.0, 0.0]
    assert not np.signbit(v[7]) and np.signbit(v[8])
    assert np.isnan(v[9]) and np.isnan(v[10])
    assert v[11] == 2.0 and v[12] == 0.5


def test_e4m3_positive_codes_increase_and_sign_mirrors():
    pos = fmt.e4m3_to_float64(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    neg = fmt.e4m3_to_float64((np.arange(0x7F) | 0x80).astype(np.uint8))
    assert np.array_equal(neg[1:], -pos[1:])


def test_bf16_fixed_points():
    v = fmt.bf16_to_float64(np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x4049],
                                     dtype=np.uint16))
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == np.inf and v[3] == -np.inf
    assert v[4] == 2.0 ** -133
    assert v[5] == 0 and np.signbit(v[5])
    assert v[6] == 3.140625


def test_element_values_passes_fp16_and_int8_through():
    x = np.array([1.5, -2.25], dtype=np.float16)
    assert fmt.element_values(x).tolist() == [1.5, -2.25]
    assert fmt.element_values(np.array([-127, 5], dtype=np.int8)).tolist() == [-127.0, 5.0]
    with pytest.raises(TypeError):
        fmt.element_values(np.array([1], dtype=np.int32))


# --------------------------------------------------------------------------- attention

def decoded(w):
    """The same workload with every stored element replaced by torch's decode of it."""
    dec = torch_bf16 if w.config.kv_dtype == "bf16" else torch_e4m3
    q = torch_bf16(w.q) if w.config.kv_dtype == "bf16" else w.q
    return Workload(w.config, w.seed, q, dec(w.k_pages), dec(w.v_pages), w.k_scale,
                    w.v_scale, w.block_table, w.seq_lens, w.scale)


def run(w, **kw):
    return oracle.decode_attention(w.q, w.k_pages, w.v_pages, w.block_table, w.seq_lens,
                                   w.scale, w.k_scale, w.v_scale, **kw)


@pytest.mark.parametrize("cfg", [TINY_BF16, TINY_FP8], ids=["bf16", "fp8"])
@pytest.mark.parametrize("seed", [1, 2])
def test_brute_force_over_torch_decoded_pools(cfg, seed):
    w = generate(cfg, seed=seed)
    out, lse = run(w, out_dtype=np.float64)
    want, want_lse = brute_force(decoded(w))
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, want_lse, rtol=1e-12, atol=1e-12)


def test_bf16_of_fp16_values_equals_fp16_bitwise():
    # Values k / 64 with |k| < 256 are exact in both fp16 and bf16.
    w = generate(TINY_BF16, seed=3)
    rng = np.random.default_rng(3)
    vals = [rng.integers(-255, 256, size=a.shape) / 64.0 for a in (w.q, w.k_pages, w.v_pages)]
    as_bf16 = [(v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16) for v in vals]
    assert all(np.array_equal(fmt.bf16_to_float64(b), v) for b, v in zip(as_bf16, vals))
    got = oracle.decode_attention(as_bf16[0], as_bf16[1], as_bf16[2], w.block_table, w.seq_lens,
                                  w.scale, out_dtype=np.float64)
    want = oracle.decode_attention(*(v.astype(np.float16) for v in vals), w.block_table,
                                   w.seq_lens, w.scale, out_dtype=np.float64)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_fp8_of_small_integers_equals_int8_bitwise():
    # E4M3 codes for the integers -16..16 (exact in E4M3), found through torch's decode.
    table = torch_e4m3(np.arange(256, dtype=np.uint8))
    code_of = {int(v): c for c, v in enumerate(table)
               if np.isfinite(v) and v == int(v) and abs(v) <= 16 and not (v == 0 and c)}
    assert sorted(code_of) == list(range(-16, 17))
    w = generate(TINY_FP8, seed=4)
    rng = np.random.default_rng(4)
    ints = [rng.integers(-16, 17, size=w.k_pages.shape) for _ in range(2)]
    codes = [np.vectorize(code_of.get)(i).astype(np.uint8) for i in ints]
    got = oracle.decode_attention(w.q, codes[0], codes[1], w.block_table, w.seq_lens, w.scale,
                                  w.k_scale, w.v_scale, out_dtype=np.float64)
    want = oracle.decode_attention(w.q, ints[0].astype(np.int8), ints[1].astype(np.int8),
                                   w.block_table, w.seq_lens, w.scale, w.k_scale, w.v_scale,
                                   out_dtype=np.float64)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_poisoned_bf16_and_fp8_slots_are_never_read():
    for cfg in (TINY_BF16, TINY_FP8):
        w = generate(cfg, seed=5, poison=True, extra_pages=3)
        out, lse = run(w)
        assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse[w.seq_lens > 0]))


# --------------------------------------------------------------------------- planted mistakes

def _e4m3_bias_8(codes):
    return fmt_real_e4m3(codes) / 2.0


def _e4m3_subnormals_as_normals(codes):
    c = np.asarray(codes).astype(np.int64)
    e, m = (c >> 3) & 0xF, (c & 7).astype(np.float64)
    mag = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    mag = np.where((e == 0xF) & (m == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def _bf16_low_half(bits):
    return np.asarray(bits).astype(np.uint32).view(np.float32).astype(np.float64)


fmt_real_e4m3 = fmt.e4m3_to_float64
fmt_real_bf16 = fmt.bf16_to_float64


def pins_pass():
    checks = [test_bf16_matches_torch_on_every_pattern, test_e4m3_matches_torch_on_every_code,
              test_e4m3_fixed_points, test_bf16_fixed_points,
              test_e4m3_positive_codes_increase_and_sign_mirrors,
              lambda: test_brute_force_over_torch_decoded_pools(TINY_BF16, 1),
              lambda: test_brute_force_over_torch_decoded_pools(TINY_FP8, 1),
              test_bf16_of_fp16_values_equals_fp16_bitwise,
              test_fp8_of_small_integers_equals_int8_bitwise]
    for check in checks:
        try:
            check()
        except AssertionError:
            return False
    return True


def test_pins_pass_on_the_real_decoders():
    assert pins_pass()


@pytest.mark.parametrize("name,target,mutant", [
    ("e4m3 bias 8", "e4m3_to_float64", _e4m3_bias_8),
    ("e4m3 subnormals decoded as normals", "e4m3_to_float64", _e4m3_subnormals_as_normals),
    ("bf16 taken as the low half", "bf16_to_float64", _bf16_low_half),
])
def test_planted_decoder_mistakes_fail_a_pin(monkeypatch, name, target, mutant):
    monkeypatch.setattr(fmt, target, mutant)
    assert not pins_pass(), f"planted mistake not caught: {name}"


def test_planted_dropped_fp8_scale_fails_a_pin(monkeypatch):
    real = decode_mod.dequantize_rows
    monkeypatch.setattr(decode_mod, "dequantize_rows",
                        lambda rows, scales: real(rows, np.ones_like(scales))
                        if rows.dtype == np.float64 and np.any(rows != np.round(rows))
                        else real(rows, scales))
    assert not pins_pass()
