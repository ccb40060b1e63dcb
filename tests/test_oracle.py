"""Pins for the fp64 oracle, each against something other than the oracle itself.

* brute force: pure-Python scalar loops that address the flat page pool by
  ((page * Hkv + head) * bs + slot) * D + d, never through the oracle's gather;
* a library routine: torch's scaled_dot_product_attention in float64 on the
  CPU, over a cache the test writes logically first and only then scatters
  into pages;
* closed forms: identical keys, q = 0, a single token, two tokens (logistic
  weights), one dominant key;
* invariants: page permutation, NaN in unused slots, GQA as repeated MHA,
  shift of every key by one vector, affine V, INT8 with unit scales, scale
  folding, and the split/merge identity of Flash-Decoding;
* planted mistakes: each plausible slip in the oracle (wrong GQA index, a
  transposed gather, a dropped max in the lse, a flipped exponent sign, a
  dropped softmax scale, a swapped dequant scale) is planted by monkeypatching
  and must make at least one pin fail.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import decode as oracle_mod
from decode_phase_attention_paged_amd.workload import Config, generate

TINY = Config(0, "tiny", batch=2, n_q_heads=4, n_kv_heads=2, head_dim=8, block_size=4,
              len_lo=1, len_hi=40, kv_dtype="fp16")
TINY_INT8 = TINY.with_(kv_dtype="int8", n_kv_heads=4)


# --------------------------------------------------------------------------- helpers

def brute_force(w, scale=None):
    """Scalar-loop decode attention straight off the flat pool (float64 Python)."""
    c = w.config
    bs, hkv, d = c.block_size, c.n_kv_heads, c.head_dim
    group = c.n_q_heads // hkv
    sigma = float(np.float32(w.scale if scale is None else scale))
    kf = w.k_pages.astype(np.float64).ravel().tolist()
    vf = w.v_pages.astype(np.float64).ravel().tolist()
    ks = w.k_scale.astype(np.float64).ravel().tolist() if w.k_scale is not None else None
    vs = w.v_scale.astype(np.float64).ravel().tolist() if w.v_scale is not None else None
    qf = w.q.astype(np.float64)
    out = np.zeros((c.batch, c.n_q_heads, d))
    lse = np.full((c.batch, c.n_q_heads), -math.inf)
    for b in range(c.batch):
        length = int(w.seq_lens[b])
        for h in range(c.n_q_heads):
            g = h // group
            rows = []
            for t in range(length):
                page = int(w.block_table[b][t // bs])
                row = (page * hkv + g) * bs + t % bs
                rows.append(row)
            scores = []
            for row in rows:
                kscale = ks[row] if ks is not None else 1.0
                scores.append(sigma * math.fsum(qf[b, h, i] * kf[row * d + i] * kscale
                                                for i in range(d)))
            if not rows:
                continue
            top = max(scores)
            weights = [math.exp(s - top) for s in scores]
            total = math.fsum(weights)
            lse[b, h] = top + math.log(total)
            for i in range(d):
                out[b, h, i] = math.fsum(
                    wt * vf[row * d + i] * (vs[row] if vs is not None else 1.0)
                    for wt, row in zip(weights, rows)) / total
    return out, lse


def scatter_to_pages(logical_k, logical_v, lengths, block_size, rng, extra_pages=0):
    """Write per-sequence contiguous caches [Hkv, L_b, D] into a shuffled page pool."""
    hkv, d = logical_k[0].shape[0], logical_k[0].shape[2]
    n_blocks = [-(-int(n) // block_size) for n in lengths]
    n_pages = sum(n_blocks) + extra_pages
    perm = rng.permutation(n_pages)
    mb = max(n_blocks + [1])
    table = np.full((len(lengths), mb), -1, dtype=np.int32)
    kp = np.zeros((n_pages, hkv, block_size, d), dtype=logical_k[0].dtype)
    vp = np.zeros_like(kp)
    off = 0
    for b, nb in enumerate(n_blocks):
        table[b, :nb] = perm[off:off + nb]
        off += nb
        for t in range(int(lengths[b])):
            kp[table[b, t // block_size], :, t % block_size, :] = logical_k[b][:, t, :]
            vp[table[b, t // block_size], :, t % block_size, :] = logical_v[b][:, t, :]
    return kp, vp, table


def run_oracle(w, **kw):
    return oracle.decode_attention(w.q, w.k_pages, w.v_pages, w.block_table, w.seq_lens,
                                   w.scale, w.k_scale, w.v_scale, **kw)


# --------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", [1, 2, 3])
def test_brute_force_fp16(seed):
    w = generate(TINY, seed=seed)
    out, lse = run_oracle(w, out_dtype=np.float64)
    ref_out, ref_lse = brute_force(w)
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [4, 5])
def test_brute_force_int8(seed):
    w = generate(TINY_INT8, seed=seed)
    out, lse = run_oracle(w, out_dtype=np.float64)
    ref_out, ref_lse = brute_force(w)
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_brute_force_block_size_2_and_empty():
    cfg = TINY.with_(block_size=2, n_q_heads=6, n_kv_heads=3)
    w = generate(cfg, seed=7, seq_lens=np.array([0, 5]))
    out, lse = run_oracle(w, out_dtype=np.float64)
    ref_out, ref_lse = brute_force(w)
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-12)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    np.testing.assert_allclose(lse[1], ref_lse[1], rtol=1e-12)


# --------------------------------------------------------------------------- library routine

@pytest.mark.parametrize("group", [1, 4])
def test_matches_torch_sdpa_float64(group):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11 + group)
    hkv, d, bs = 2, 16, 4
    hq = hkv * group
    lengths = [1, 9, 16, 23]
    lk = [rng.standard_normal((hkv, n, d)) for n in lengths]
    lv = [rng.standard_normal((hkv, n, d)) for n in lengths]
    q = rng.standard_normal((len(lengths), hq, d))
    kp, vp, table = scatter_to_pages(lk, lv, lengths, bs, rng, extra_pages=3)
    scale = float(np.float32(0.3))
    out, lse = oracle.decode_attention(q, kp, vp, table, np.array(lengths), scale,
                                       out_dtype=np.float64)
    for b, n in enumerate(lengths):
        qt = torch.from_numpy(q[b]).reshape(1, hq, 1, d)
        kt = torch.from_numpy(lk[b]).repeat_interleave(group, dim=0).unsqueeze(0)
        vt = torch.from_numpy(lv[b]).repeat_interleave(group, dim=0).unsqueeze(0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        np.testing.assert_allclose(out[b], ref[0, :, 0, :].numpy(), rtol=1e-12, atol=1e-13)
        ref_lse = torch.logsumexp(scale * (kt[0] @ qt[0].transpose(1, 2))[..., 0], dim=-1)
        np.testing.assert_allclose(lse[b], ref_lse.numpy(), rtol=1e-12)


# --------------------------------------------------------------------------- closed forms

def _single(q, keys, values, scale=1.0, bs=4):
    """Run the oracle on one sequence given as [L, D] arrays (one head)."""
    n = keys.shape[0]
    rng = np.random.default_rng(n)
    kp, vp, table = scatter_to_pages([keys[None]], [values[None]], [n], bs, rng)
    out, lse, probs = oracle.decode_attention(q[None, None], kp, vp, table, np.array([n]),
                                              scale, return_probs=True, out_dtype=np.float64)
    return out[0, 0], lse[0, 0], probs[(0, 0)]


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(3)
    k = np.tile(rng.standard_normal(8), (13, 1))
    v = rng.standard_normal((13, 8))
    out, lse, p = _single(rng.standard_normal(8), k, v)
    np.testing.assert_allclose(out, v.mean(axis=0), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(p, np.full(13, 1 / 13), rtol=1e-13)


def test_zero_query_gives_mean_and_log_length():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((21, 8))
    out, lse, _ = _single(np.zeros(8), rng.standard_normal((21, 8)), v)
    np.testing.assert_allclose(out, v.mean(axis=0), rtol=1e-13, atol=1e-14)
    assert lse == pytest.approx(math.log(21), rel=1e-14)


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(5)
    k, v, q = rng.standard_normal((1, 8)), rng.standard_normal((1, 8)), rng.standard_normal(8)
    out, lse, p = _single(q, k, v, scale=0.75)
    assert np.array_equal(out, v[0]) and p.tolist() == [1.0]
    assert lse == pytest.approx(0.75 * float(k[0] @ q), rel=1e-14)


def test_two_tokens_logistic_weights():
    rng = np.random.default_rng(6)
    k, v, q = rng.standard_normal((2, 8)), rng.standard_normal((2, 8)), rng.standard_normal(8)
    scale = 0.875
    s0, s1 = scale * float(k[0] @ q), scale * float(k[1] @ q)
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    out, lse, p = _single(q, k, v, scale=scale)
    np.testing.assert_allclose(p, [w0, 1 - w0], rtol=1e-13)
    np.testing.assert_allclose(out, w0 * v[0] + (1 - w0) * v[1], rtol=1e-12, atol=1e-14)
    assert lse == pytest.approx(s0 + math.log1p(math.exp(s1 - s0)), rel=1e-13)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(8)
    q = rng.standard_normal(8)
    k = 0.1 * rng.standard_normal((30, 8))
    v = rng.standard_normal((30, 8))
    j = 17
    k[j] = 40.0 * q / np.linalg.norm(q)
    out, _, p = _single(q, k, v)
    s = k @ q
    bound = sum(math.exp(s[t] - s[j]) * np.abs(v[t] - v[j]).max() for t in range(30) if t != j)
    assert np.abs(out - v[j]).max() <= bound + 1e-15
    assert bound < 1e-6
    assert p.argmax() == j


def test_weights_sum_to_one():
    w = generate(TINY, seed=9)
    _, _, probs = run_oracle(w, return_probs=True)
    for (b, _h), p in probs.items():
        assert len(p) == w.seq_lens[b]
        assert math.fsum(p) == pytest.approx(1.0, abs=1e-12)
        assert np.all(p >= 0)


# --------------------------------------------------------------------------- invariants

def test_page_permutation_is_bitwise_invariant():
    w = generate(TINY, seed=10, extra_pages=3)
    out, lse = run_oracle(w)
    rng = np.random.default_rng(0)
    perm = rng.permutation(w.num_pages)          # new position of each old page
    kp = np.empty_like(w.k_pages)
    vp = np.empty_like(w.v_pages)
    kp[perm] = w.k_pages
    vp[perm] = w.v_pages
    table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1)
    out2, lse2 = oracle.decode_attention(w.q, kp, vp, table, w.seq_lens, w.scale)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("cfg", [TINY, TINY_INT8])
def test_nan_in_unused_slots_and_pages_is_never_read(cfg):
    clean = generate(cfg, seed=12, extra_pages=4)
    dirty = generate(cfg, seed=12, extra_pages=4, poison=True)
    if cfg.kv_dtype == "fp16":
        assert np.isnan(dirty.k_pages).any()
    else:
        assert np.isnan(dirty.k_scale).any()
    a, la = run_oracle(clean)
    b, lb = run_oracle(dirty)
    assert np.isfinite(b).all() and np.array_equal(a, b) and np.array_equal(la, lb)


def test_gqa_equals_mha_with_repeated_kv_heads():
    w = generate(TINY, seed=13)
    group = TINY.n_q_heads // TINY.n_kv_heads
    out, lse = run_oracle(w, out_dtype=np.float64)
    kr = np.repeat(w.k_pages, group, axis=1)
    vr = np.repeat(w.v_pages, group, axis=1)
    out2, lse2 = oracle.decode_attention(w.q, kr, vr, w.block_table, w.seq_lens, w.scale,
                                         out_dtype=np.float64)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_shift_of_all_keys_leaves_output_unchanged():
    w = generate(TINY, seed=14)
    kp = w.k_pages.astype(np.float64)
    vp = w.v_pages.astype(np.float64)
    u = np.random.default_rng(1).standard_normal(TINY.head_dim)
    out, lse = oracle.decode_attention(w.q, kp, vp, w.block_table, w.seq_lens, w.scale,
                                       out_dtype=np.float64)
    out2, lse2 = oracle.decode_attention(w.q, kp + u, vp, w.block_table, w.seq_lens,
                                         w.scale, out_dtype=np.float64)
    np.testing.assert_allclose(out2, out, rtol=1e-11, atol=1e-12)
    shift = float(np.float32(w.scale)) * (w.q.astype(np.float64) @ u)
    np.testing.assert_allclose(lse2 - lse, shift, rtol=1e-10, atol=1e-11)


def test_affine_values_map_affinely():
    w = generate(TINY, seed=15)
    kp = w.k_pages.astype(np.float64)
    vp = w.v_pages.astype(np.float64)
    a, c = -2.5, 0.75
    out, _ = oracle.decode_attention(w.q, kp, vp, w.block_table, w.seq_lens, w.scale,
                                     out_dtype=np.float64)
    out2, _ = oracle.decode_attention(w.q, kp, a * vp + c, w.block_table, w.seq_lens,
                                      w.scale, out_dtype=np.float64)
    np.testing.assert_allclose(out2, a * out + c, rtol=1e-12, atol=1e-12)


def test_int8_with_unit_scales_equals_fp16_on_same_integers():
    w = generate(TINY_INT8, seed=16)
    ones = np.ones_like(w.k_scale)
    out, lse = oracle.decode_attention(w.q, w.k_pages, w.v_pages, w.block_table, w.seq_lens,
                                       w.scale, ones, ones)
    kh = w.k_pages.astype(np.float16)
    vh = w.v_pages.astype(np.float16)
    out2, lse2 = oracle.decode_attention(w.q, kh, vh, w.block_table, w.seq_lens, w.scale)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_int8_scale_folding():
    w = generate(TINY_INT8, seed=17)
    c = 4.0  # a power of two, so scale * c and k_scale * c stay exact in fp32
    out, lse = run_oracle(w, out_dtype=np.float64)
    out_k, lse_k = oracle.decode_attention(w.q, w.k_pages, w.v_pages, w.block_table,
                                           w.seq_lens, w.scale * c,
                                           w.k_scale, w.v_scale, out_dtype=np.float64)
    out_k2, lse_k2 = oracle.decode_attention(w.q, w.k_pages, w.v_pages, w.block_table,
                                             w.seq_lens, w.scale, w.k_scale * c,
                                             w.v_scale, out_dtype=np.float64)
    np.testing.assert_allclose(out_k2, out_k, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_k2, lse_k, rtol=1e-12)
    out_v, lse_v = oracle.decode_attention(w.q, w.k_pages, w.v_pages, w.block_table,
                                           w.seq_lens, w.scale, w.k_scale,
                                           w.v_scale * np.float32(c), out_dtype=np.float64)
    np.testing.assert_allclose(out_v, c * out, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(lse_v, lse)


def merge_partials(parts):
    """Flash-Decoding merge, written here from its definition: weights exp(lse_s - M)."""
    lses = np.array([l for _, l in parts])
    if np.all(np.isneginf(lses)):
        return np.zeros_like(parts[0][0]), -np.inf
    top = lses.max()
    wts = np.exp(lses - top)
    out = sum(wt * o for wt, (o, _) in zip(wts, parts)) / wts.sum()
    return out, top + math.log(wts.sum())


@pytest.mark.parametrize("pages_per_split", [1, 2, 3, 7])
def test_split_merge_identity(pages_per_split):
    """Partial attention over page-aligned token ranges, merged, equals the whole."""
    cfg = TINY.with_(len_lo=0, len_hi=40)
    w = generate(cfg, seed=20 + pages_per_split)
    bs = cfg.block_size
    full, full_lse = run_oracle(w, out_dtype=np.float64)
    mb = cfg.max_blocks_per_seq
    for b in range(cfg.batch):
        length = int(w.seq_lens[b])
        parts = []
        for j0 in range(0, mb, pages_per_split):
            sub_len = max(0, min(length, (j0 + pages_per_split) * bs) - j0 * bs)
            sub_table = w.block_table[b:b + 1, j0:]
            o, l = oracle.decode_attention(w.q[b:b + 1], w.k_pages, w.v_pages, sub_table,
                                           np.array([sub_len]), w.scale, out_dtype=np.float64)
            parts.append((o[0], l[0]))
        for h in range(cfg.n_q_heads):
            o, l = merge_partials([(po[h], pl[h]) for po, pl in parts])
            np.testing.assert_allclose(o, full[b, h], rtol=1e-12, atol=1e-13)
            if length:
                assert l == pytest.approx(full_lse[b, h], rel=1e-13)
            else:
                assert np.isneginf(l) and np.isneginf(full_lse[b, h])


# --------------------------------------------------------------------------- planted mistakes

def _pins_pass():
    """Run a selection of the pins above; True when all of them hold."""
    checks = [
        lambda: test_brute_force_fp16(1),
        lambda: test_brute_force_int8(4),
        lambda: test_two_tokens_logistic_weights(),
        lambda: test_split_merge_identity(2),
        lambda: test_int8_scale_folding(),
    ]
    try:
        import torch  # noqa: F401
        checks.append(lambda: test_matches_torch_sdpa_float64(4))
    except ImportError:  # pragma: no cover
        pass
    for check in checks:
        try:
            check()
        except AssertionError:
            return False
    return True


def _attend_flipped_sign(q, keys, values, scale):
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1]), -np.inf, np.zeros(0)
    s = scale * (keys @ q)
    e = np.exp(s.max() - s)
    return (e / e.sum()) @ values, float(s.max() + np.log(e.sum())), e / e.sum()


def _attend_lse_without_max(q, keys, values, scale):
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1]), -np.inf, np.zeros(0)
    s = scale * (keys @ q)
    e = np.exp(s - s.max())
    return (e / e.sum()) @ values, float(np.log(e.sum())), e / e.sum()


_REAL_ATTEND = oracle_mod.attend


def _attend_unscaled(q, keys, values, scale):
    return _REAL_ATTEND(q, keys, values, 1.0)


def _gather_transposed(pages, table_row, seq_len, block_size):
    seq_len = int(seq_len)
    n_kv = pages.shape[1]
    if seq_len == 0:
        return np.empty((n_kv, 0) + pages.shape[3:], dtype=pages.dtype)
    nb = -(-seq_len // block_size)
    tiles = pages[np.asarray(table_row[:nb], dtype=np.int64)]
    return tiles.reshape((n_kv, nb * block_size) + pages.shape[3:])[:, :seq_len]


MUTANTS = {
    "gqa index h % Hkv": ("kv_head_of", lambda h, g: h % 2),
    "exp(max - s)": ("attend", _attend_flipped_sign),
    "lse without the max": ("attend", _attend_lse_without_max),
    "scale dropped": ("attend", _attend_unscaled),
    "gather without head/page transpose": ("gather_sequence", _gather_transposed),
    "v dequantised with k scales": ("dequantize_rows", None),
}


def test_pins_hold_on_the_real_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    original = getattr(oracle_mod, attr)
    if name == "v dequantised with k scales":
        calls = {"n": 0}

        def fn(rows, scales):  # noqa: F811 - the second call of each pair (V) reuses the first's scales
            calls["n"] += 1
            if calls["n"] % 2 == 1:
                calls["k"] = scales
                return original(rows, scales)
            return original(rows, calls["k"])
    monkeypatch.setattr(oracle_mod, attr, fn)
    assert not _pins_pass(), f"no pin caught the planted mistake: {name}"
