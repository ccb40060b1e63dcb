"""Pins for the K/V-append oracle (oracle/append.py), none of which re-types it:
closed forms of the per-row INT8 and FP8 rules, their rounding bounds, torch's
own float32 -> float8_e4m3fn rounding, a brute-force page walk on a flat pool,
untouched-memory invariants, agreement with the attention oracle over the grown
cache, and planted mistakes that must fail at least one pin."""

import numpy as np
import pytest
import torch

import oracle
from oracle import append as app
from oracle import formats as fmt


F32 = np.float32


# ------------------------------------------------------------------ per-row INT8 rule

def test_single_nonzero_element_maps_to_127():
    for a in (1.0, -3.5, 1e-3, 6.0e4):
        x = np.zeros(128, dtype=np.float16)
        x[17] = a
        codes, s = oracle.quantize_row(x)
        assert s == F32(abs(F32(np.float16(a)))) / F32(127)
        assert codes[17] == (127 if a > 0 else -127)
        assert np.count_nonzero(codes) == 1


def test_zero_row_stores_zero_scale_and_codes():
    codes, s = oracle.quantize_row(np.zeros(128, dtype=np.float16))
    assert s == 0 and not codes.any() and codes.dtype == np.int8


def test_integer_multiples_of_a_power_of_two_are_exact():
    rng = np.random.default_rng(3)
    for c in (2.0 ** -6, 2.0 ** -2, 1.0, 4.0):
        k = rng.integers(-127, 128, size=128)
        k[5] = -127                      # max |k| = 127, so s = 127 c / 127 = c exactly
        x = (k * c).astype(np.float16)
        assert np.array_equal(x.astype(np.float64), k * c)
        codes, s = oracle.quantize_row(x)
        assert s == F32(c)
        assert np.array_equal(codes, k.astype(np.int8))


def test_ties_round_to_even():
    # max |x| = 127 makes s = 1, so x / s is x itself and the ties are exact.
    x = np.zeros(128, dtype=np.float16)
    x[:8] = [127, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 126.5]
    codes, s = oracle.quantize_row(x)
    assert s == 1
    assert codes[:8].tolist() == [127, 2, 4, -2, 0, 2, 0, 126]


def test_rounding_error_bound_and_full_range():
    # Round to nearest: every dequantised value is within s / 2 of the input, plus the
    # fp32 rounding of x / s (below 127 * 2^-24 code units), and the largest magnitude maps
    # to exactly 127.
    rng = np.random.default_rng(4)
    for _ in range(200):
        x = (rng.standard_normal(128) * rng.uniform(0.01, 100)).astype(np.float16)
        codes, s = oracle.quantize_row(x)
        err = np.abs(codes.astype(np.float64) * float(s) - x.astype(np.float64))
        assert err.max() <= float(s) * (0.5 + 1e-5)
        assert np.abs(codes).max() == 127


# ------------------------------------------------------------------ per-row FP8 rule

def torch_e4m3_codes(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def e4m3_grid():
    return torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_rounding_matches_torch():
    rng = np.random.default_rng(11)
    grid = e4m3_grid()
    mids = (grid[1:] + grid[:-1]) / 2                      # every tie between neighbours
    rand = rng.uniform(-1, 1, size=20000) * np.exp2(rng.uniform(-12, 8.8, size=20000))
    v = np.concatenate([mids, -mids, grid, -grid, rand, [0.0, -0.0]]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    assert np.array_equal(oracle.e4m3_from_float32(v), torch_e4m3_codes(v))


def test_e4m3_codes_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(oracle.e4m3_from_float32(vals), codes)


def test_fp8_single_element_maps_to_448():
    for a in (1.0, -3.5, 1e-3, 6.0e4):
        x = np.zeros(128, dtype=np.float16)
        x[3] = a
        codes, s = oracle.quantize_row_fp8(x)
        assert s == F32(abs(F32(np.float16(a)))) / F32(448)
        assert codes[3] == (0x7E if a > 0 else 0xFE)
        assert np.count_nonzero(codes) == 1


def test_fp8_zero_row_and_exact_rows():
    codes, s = oracle.quantize_row_fp8(np.zeros(128, dtype=np.float16))
    assert s == 0 and not codes.any() and codes.dtype == np.uint8
    # Rows of E4M3 values times a power of two c, with one element at 448 c: s = c exactly,
    # so the codes come back unchanged.
    rng = np.random.default_rng(12)
    grid = e4m3_grid()
    for c in (2.0 ** -8, 2.0 ** -3, 1.0):
        idx = rng.integers(0, 0x7F, size=128)
        sign = rng.integers(0, 2, size=128)
        idx[9], sign[9] = 0x7E, 1
        x = (np.where(sign, -1, 1) * grid[idx] * c).astype(np.float16)
        assert np.array_equal(x.astype(np.float64), np.where(sign, -1, 1) * grid[idx] * c)
        codes, s = oracle.quantize_row_fp8(x)
        assert s == F32(c)
        want = (idx | np.where(sign, 0x80, 0)).astype(np.uint8)
        nz = grid[idx] != 0
        assert np.array_equal(codes[nz], want[nz])


def test_fp8_rounding_error_bound():
    # Nearest rounding: relative error at most 2^-4 in the normal range, absolute at most
    # 2^-10 (half a subnormal step) below 2^-6, both in units of the row scale, plus the
    # fp32 rounding of x / s.
    rng = np.random.default_rng(13)
    for _ in range(200):
        x = (rng.standard_normal(128) * rng.uniform(0.01, 100)).astype(np.float16)
        codes, s = oracle.quantize_row_fp8(x)
        deq = fmt.e4m3_to_float64(codes) * float(s)
        xa = x.astype(np.float64)
        bound = np.maximum(np.abs(xa) * 2.0 ** -4, 2.0 ** -10 * float(s)) * (1 + 1e-6)
        assert np.all(np.abs(deq - xa) <= bound)
        assert np.abs(fmt.e4m3_to_float64(codes)).max() == 448


# ------------------------------------------------------------------ page placement

def small_cache(int8, rng, np_=7, hkv=2, bs=4, d=8, kind=None):
    kind = kind or ("int8" if int8 else "fp16")
    if kind == "fp8":
        k = rng.integers(0, 0x7F, size=(np_, hkv, bs, d)).astype(np.uint8)
        v = rng.integers(0x80, 0xFF, size=(np_, hkv, bs, d)).astype(np.uint8)
        ks = rng.uniform(0.1, 1, size=(np_, hkv, bs)).astype(np.float32)
        vs = rng.uniform(0.1, 1, size=(np_, hkv, bs)).astype(np.float32)
        return k, v, ks, vs
    if kind == "bf16":
        k = rng.integers(0, 1 << 16, size=(np_, hkv, bs, d)).astype(np.uint16)
        v = rng.integers(0, 1 << 16, size=(np_, hkv, bs, d)).astype(np.uint16)
        return k, v, None, None
    if int8:
        k = rng.integers(-127, 128, size=(np_, hkv, bs, d)).astype(np.int8)
        v = rng.integers(-127, 128, size=(np_, hkv, bs, d)).astype(np.int8)
        ks = rng.uniform(0.1, 1, size=(np_, hkv, bs)).astype(np.float32)
        vs = rng.uniform(0.1, 1, size=(np_, hkv, bs)).astype(np.float32)
    else:
        k = rng.standard_normal((np_, hkv, bs, d)).astype(np.float16)
        v = rng.standard_normal((np_, hkv, bs, d)).astype(np.float16)
        ks = vs = None
    return k, v, ks, vs


@pytest.mark.parametrize("kind", ["fp16", "int8", "bf16", "fp8"])
def test_brute_force_on_a_flat_pool(kind):
    # The flat pool is addressed as ((page * Hkv + g) * bs + slot) * D + d, with
    # page = table[b][p // bs] and slot = p % bs; rows with p < 0 are skipped. FP8 codes
    # come from torch's float32 -> float8_e4m3fn rounding of x / s.
    rng = np.random.default_rng(5)
    int8 = kind in ("int8", "fp8")
    k, v, ks, vs = small_cache(int8, rng, kind=kind)
    np_, hkv, bs, d = k.shape
    table = np.array([[6, 2, 0], [1, 4, 3], [5, 5, 5]], dtype=np.int32)
    positions = np.array([9, 3, -1], dtype=np.int32)      # page 0 slot 1; page 1 slot 3
    if kind == "bf16":
        k_new = rng.integers(0, 1 << 16, size=(3, hkv, d)).astype(np.uint16)
        v_new = rng.integers(0, 1 << 16, size=(3, hkv, d)).astype(np.uint16)
    else:
        k_new = rng.standard_normal((3, hkv, d)).astype(np.float16)
        v_new = rng.standard_normal((3, hkv, d)).astype(np.float16)
    top = 448 if kind == "fp8" else 127
    got = oracle.append_kv(k, v, table, positions, k_new, v_new, bs, ks, vs)

    flat_k, flat_v = k.reshape(-1).copy(), v.reshape(-1).copy()
    flat_ks = ks.reshape(-1).copy() if int8 else None
    flat_vs = vs.reshape(-1).copy() if int8 else None
    for b in range(3):
        p = int(positions[b])
        if p < 0:
            continue
        page = int(table[b][p // bs])
        for g in range(hkv):
            row = (page * hkv + g) * bs + p % bs
            for src, flat, flat_s in ((k_new, flat_k, flat_ks), (v_new, flat_v, flat_vs)):
                vals = [float(src[b, g, i]) for i in range(d)]
                if int8:
                    m = max(abs(t) for t in vals)
                    s = F32(F32(m) / F32(top))
                    flat_s[row] = s
                    for i in range(d):
                        if m == 0:
                            flat[row * d + i] = 0
                        elif kind == "fp8":
                            flat[row * d + i] = torch_e4m3_codes([F32(vals[i]) / s])[0]
                        else:
                            flat[row * d + i] = int(np.rint(F32(vals[i]) / s))
                elif kind == "bf16":
                    for i in range(d):
                        flat[row * d + i] = src[b, g, i]
                else:
                    for i in range(d):
                        flat[row * d + i] = vals[i]
    assert np.array_equal(got[0].reshape(-1), flat_k)
    assert np.array_equal(got[1].reshape(-1), flat_v)
    if int8:
        assert np.array_equal(got[2].reshape(-1), flat_ks)
        assert np.array_equal(got[3].reshape(-1), flat_vs)


def test_inputs_untouched_and_only_target_rows_change():
    rng = np.random.default_rng(6)
    k, v, ks, vs = small_cache(True, rng)
    keep = [a.copy() for a in (k, v, ks, vs)]
    table = np.array([[3, 1]], dtype=np.int32)
    k_new = rng.standard_normal((1, 2, 8)).astype(np.float16)
    out = oracle.append_kv(k, v, table, np.array([6], dtype=np.int32), k_new, k_new, 4, ks, vs)
    for a, b in zip((k, v, ks, vs), keep):
        assert np.array_equal(a, b)
    for new, old in zip(out, keep):
        diff = np.argwhere(new != old) if new.ndim == 3 else np.argwhere(np.any(new != old, axis=-1))
        assert {(int(r[0]), int(r[2])) for r in diff} <= {(1, 2)}   # page 1, slot 2 only


# ------------------------------------------------------------------ agreement with attention

def test_attention_over_the_grown_cache():
    # Append each sequence's token at position L_b; attention with L_b + 1 tokens must equal
    # attention over the gathered cache with the new row concatenated (fp16 rows are stored
    # exactly).
    from decode_phase_attention_paged_amd.workload import CONFIGS, generate
    cfg = CONFIGS[1].with_(batch=3, n_q_heads=4, n_kv_heads=2, len_lo=5, len_hi=40)
    w = generate(cfg, seed=9, extra_pages=0)
    lens = w.seq_lens.copy()
    lens[0] = 47                  # position 47 lands in slot 15 of the table's last page
    table = w.block_table.copy()
    pools_k, pools_v = w.k_pages, w.v_pages
    # Give every sequence a page for its new token where the table has none yet.
    free = pools_k.shape[0]
    need = []
    for b in range(cfg.batch):
        j = int(lens[b]) // cfg.block_size
        if table[b, j] < 0:
            table[b, j] = free + len(need)
            need.append(b)
    zk = np.zeros((len(need),) + pools_k.shape[1:], dtype=pools_k.dtype)
    pools_k = np.concatenate([pools_k, zk])
    pools_v = np.concatenate([pools_v, zk])
    rng = np.random.default_rng(10)
    k_new = rng.standard_normal((cfg.batch, cfg.n_kv_heads, 128)).astype(np.float16)
    v_new = rng.standard_normal((cfg.batch, cfg.n_kv_heads, 128)).astype(np.float16)
    gk, gv, _, _ = oracle.append_kv(pools_k, pools_v, table, lens, k_new, v_new, cfg.block_size)
    # w.q / scale are the generator's; lengths grow by one
    out, lse = oracle.decode_attention(w.q, gk, gv, table, lens + 1, w.scale)
    G = cfg.n_q_heads // cfg.n_kv_heads
    for b in range(cfg.batch):
        kb = oracle.gather_sequence(pools_k, table[b], int(lens[b]), cfg.block_size)
        vb = oracle.gather_sequence(pools_v, table[b], int(lens[b]), cfg.block_size)
        for h in range(cfg.n_q_heads):
            g = h // G
            keys = np.concatenate([kb[g], k_new[b, g][None]]).astype(np.float64)
            vals = np.concatenate([vb[g], v_new[b, g][None]]).astype(np.float64)
            o, l, _ = oracle.attend(w.q[b, h].astype(np.float64), keys, vals,
                                    float(np.float64(np.float32(w.scale))))
            np.testing.assert_allclose(out[b, h], o, rtol=1e-6, atol=1e-7)
            np.testing.assert_allclose(lse[b, h], l, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ planted mistakes

def pins_pass():
    tests = [test_single_nonzero_element_maps_to_127, test_zero_row_stores_zero_scale_and_codes,
             test_integer_multiples_of_a_power_of_two_are_exact, test_ties_round_to_even,
             test_rounding_error_bound_and_full_range,
             lambda: test_brute_force_on_a_flat_pool("fp16"),
             lambda: test_brute_force_on_a_flat_pool("int8"),
             lambda: test_brute_force_on_a_flat_pool("bf16"),
             lambda: test_brute_force_on_a_flat_pool("fp8"),
             test_e4m3_rounding_matches_torch, test_e4m3_codes_round_trip,
             test_fp8_single_element_maps_to_448, test_fp8_zero_row_and_exact_rows,
             test_fp8_rounding_error_bound,
             test_inputs_untouched_and_only_target_rows_change]
    for t in tests:
        try:
            t()
        except (AssertionError, IndexError, ValueError, ZeroDivisionError, FloatingPointError):
            return False
    return True


def test_pins_pass_on_the_real_oracle():
    assert pins_pass()


def _quantize_scale_128(x):
    x32 = np.asarray(x, dtype=F32)
    m = F32(np.max(np.abs(x32)))
    if m == 0:
        return np.zeros(x32.shape, dtype=np.int8), F32(0)
    s = F32(m / F32(128))
    return np.clip(np.rint(x32 / s), -127, 127).astype(np.int8), s


def _quantize_half_up(x):
    x32 = np.asarray(x, dtype=F32)
    m = F32(np.max(np.abs(x32)))
    if m == 0:
        return np.zeros(x32.shape, dtype=np.int8), F32(0)
    s = F32(m / F32(127))
    return np.clip(np.floor(x32 / s + F32(0.5)), -127, 127).astype(np.int8), s


def _quantize_truncate(x):
    x32 = np.asarray(x, dtype=F32)
    m = F32(np.max(np.abs(x32)))
    if m == 0:
        return np.zeros(x32.shape, dtype=np.int8), F32(0)
    s = F32(m / F32(127))
    return np.clip(np.trunc(x32 / s), -127, 127).astype(np.int8), s


def _append_wrong_slot(k_pages, v_pages, block_table, positions, k_new, v_new, block_size,
                       k_scale=None, v_scale=None):
    shifted = np.where(positions >= 0, positions + 1, positions).astype(np.int32)
    return ORIG_APPEND(k_pages, v_pages, block_table, shifted, k_new, v_new, block_size,
                       k_scale, v_scale)


def _append_swapped_kv(k_pages, v_pages, block_table, positions, k_new, v_new, block_size,
                       k_scale=None, v_scale=None):
    return ORIG_APPEND(k_pages, v_pages, block_table, positions, v_new, k_new, block_size,
                       k_scale, v_scale)


def _fp8_max_240(x):
    x32 = np.asarray(x, dtype=F32)
    m = F32(np.max(np.abs(x32)))
    if m == 0:
        return np.zeros(x32.shape, dtype=np.uint8), F32(0)
    s = F32(m / F32(240))
    return fmt.e4m3_from_float32(x32 / s), s


def _e4m3_ties_away(v):
    v = np.asarray(v, dtype=np.float32)
    grid = fmt.e4m3_to_float64(np.arange(0x7F, dtype=np.uint8))
    a = np.abs(v.astype(np.float64))
    hi = np.clip(np.searchsorted(grid, a), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    code = np.where(np.abs(grid[hi] - a) <= np.abs(a - grid[lo]), hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def _e4m3_truncate(v):
    v = np.asarray(v, dtype=np.float32)
    grid = fmt.e4m3_to_float64(np.arange(0x7F, dtype=np.uint8))
    a = np.abs(v.astype(np.float64))
    code = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 126).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


ORIG_APPEND = app.append_kv


@pytest.mark.parametrize("name,target,mutant", [
    ("scale over 128", "quantize_row", _quantize_scale_128),
    ("ties rounded up", "quantize_row", _quantize_half_up),
    ("codes truncated", "quantize_row", _quantize_truncate),
    ("slot off by one", "append_kv", _append_wrong_slot),
    ("K and V swapped", "append_kv", _append_swapped_kv),
    ("fp8 scale over 240", "quantize_row_fp8", _fp8_max_240),
    ("fp8 ties away from zero", "e4m3_from_float32", _e4m3_ties_away),
    ("fp8 codes truncated", "e4m3_from_float32", _e4m3_truncate),
])
def test_planted_mistakes_fail_a_pin(monkeypatch, name, target, mutant):
    monkeypatch.setattr(app, target, mutant)
    monkeypatch.setattr(oracle, target, mutant)
    if hasattr(fmt, target):
        monkeypatch.setattr(fmt, target, mutant)
    assert not pins_pass(), f"planted mistake not caught: {name}"
