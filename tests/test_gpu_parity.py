"""GPU parity: the HIP library against the fp64 oracle on the same seeded inputs.

Bar (the decode-attention tolerance for fp32 outputs): elementwise
|gpu - oracle| <= 2e-3 + 1e-2 * |oracle|. Every call goes through the C ABI.
"""

import os

import numpy as np
import pytest

import oracle
from decode_phase_attention_paged_amd.workload import CONFIGS, Config, generate

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need an MI355X"
    return t


@pytest.fixture(scope="module")
def lib(torch):
    from decode_phase_attention_paged_amd import binding
    return binding


def dev_tensor(torch, a):
    """A host array on the GPU; bf16 bit patterns (uint16) become bfloat16 tensors and E4M3
    codes (uint8) float8_e4m3fn tensors."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    t = torch.from_numpy(a).to("cuda:0")
    return t.view(torch.float8_e4m3fn) if a.dtype == np.uint8 else t


def to_dev(torch, w):
    t = lambda a: dev_tensor(torch, a)
    return dict(q=t(w.q), k_pages=t(w.k_pages), v_pages=t(w.v_pages), k_scale=t(w.k_scale),
                v_scale=t(w.v_scale), block_table=t(w.block_table), seq_lens=t(w.seq_lens))


def gpu_run(torch, lib, w, num_workgroups=0, lse=True, dev_inputs=None, num_splits=0):
    d = dev_inputs or to_dev(torch, w)
    lse_out = torch.empty(w.q.shape[:2], dtype=torch.float32, device="cuda:0") if lse else None
    out = lib.decode_attn_ex(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["seq_lens"],
                             w.scale, k_scale=d["k_scale"], v_scale=d["v_scale"],
                             lse_out=lse_out, num_workgroups=num_workgroups,
                             num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse_out.cpu().numpy() if lse else None)


def assert_parity(got, ref, what=""):
    diff = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    bound = ATOL + RTOL * np.abs(ref.astype(np.float64))
    bad = ~(diff <= bound)
    print(f"{what}: max|d|={np.nanmax(diff) if diff.size else 0:.3e}", flush=True)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance, "
                           f"max|d|={np.nanmax(diff):.3e}")


def assert_lse(got, ref, what=""):
    empty = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), empty), what
    np.testing.assert_allclose(got[~empty], ref[~empty], rtol=1e-4, atol=1e-3, err_msg=what)


def oracle_run(w):
    return oracle.decode_attention(w.q, w.k_pages, w.v_pages, w.block_table, w.seq_lens, w.scale,
                                   w.k_scale, w.v_scale)


SMALL = Config(0, "small_gqa", batch=3, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
               len_lo=1, len_hi=300, kv_dtype="fp16")


# ------------------------------------------------------------------ small, every kernel variant

# Plans exercised: the library's own; stream mode on several grids (64 workgroups give
# 256 workers for ~100 units, so most are empty and some sit between the pieces of a cut
# (sequence, head) pair); segment mode on its own grid and on one and two workgroups (every
# workgroup then runs several segments back to back); split mode with three partitions.
PLANS = [dict(), dict(num_workgroups=1), dict(num_workgroups=3), dict(num_workgroups=64),
         dict(num_splits=1), dict(num_splits=1, num_workgroups=1),
         dict(num_splits=1, num_workgroups=2), dict(num_splits=3)]
PLAN_IDS = ["auto", "wg1", "wg3", "wg64", "seg", "seg-wg1", "seg-wg2", "split3"]


KVS = ["fp16", "int8", "bf16", "fp8"]


@pytest.mark.parametrize("kv", KVS)
@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("plan", PLANS, ids=PLAN_IDS)
def test_small_all_variants(torch, lib, kv, group, plan):
    cfg = SMALL.with_(kv_dtype=kv, n_q_heads=2 * group, n_kv_heads=2)
    w = generate(cfg, seed=100 + group)
    print(f"case kv={kv} G={group} plan={plan} lens={w.seq_lens.tolist()}", flush=True)
    ref, ref_lse = oracle_run(w)
    got, lse = gpu_run(torch, lib, w, **plan)
    assert_parity(got, ref, f"{kv} G={group} {plan}")
    assert_lse(lse, ref_lse, "lse")


@pytest.mark.parametrize("plan", [dict(num_workgroups=n) for n in (1, 2, 3, 7, 19, 64, 300)]
                         + [dict(num_splits=n) for n in (1, 2, 3, 7, 19, 75)]
                         + [dict(num_splits=1, num_workgroups=n) for n in (1, 2, 5, 6, 7)],
                         ids=lambda p: "-".join(f"{k}{v}" for k, v in p.items()))
def test_plans_and_determinism(torch, lib, plan):
    w = generate(SMALL.with_(len_hi=1200), seed=7)
    ref, ref_lse = oracle_run(w)
    d = to_dev(torch, w)
    a, la = gpu_run(torch, lib, w, dev_inputs=d, **plan)
    b, lb = gpu_run(torch, lib, w, dev_inputs=d, **plan)
    assert_parity(a, ref, f"{plan}")
    assert_lse(la, ref_lse, "lse")
    assert np.array_equal(a, b) and np.array_equal(la, lb), "same inputs, same plan: not bitwise equal"


EDGE_PLANS = [dict(num_workgroups=1), dict(num_workgroups=4), dict(num_workgroups=19),
              dict(num_workgroups=100), dict(num_splits=1), dict(num_splits=1, num_workgroups=1),
              dict(num_splits=1, num_workgroups=5), dict(num_splits=4), dict(num_splits=19)]


@pytest.mark.parametrize("kv", KVS)
def test_edge_lengths_and_nan_canaries(torch, lib, kv):
    # Empty, single-token, page-boundary and full caches in one batch; every slot no token
    # owns (and 5 pages nobody references) holds NaN.
    lens = np.array([0, 1, 15, 16, 17, 31, 32, 33, 299, 300, 0, 2], dtype=np.int32)
    cfg = SMALL.with_(kv_dtype=kv, batch=len(lens), len_lo=0)
    w = generate(cfg, seed=11, seq_lens=lens, extra_pages=5, poison=True)
    print(f"case edge kv={kv}", flush=True)
    ref, ref_lse = oracle_run(w)
    assert np.isfinite(ref).all()
    for plan in EDGE_PLANS:
        got, lse = gpu_run(torch, lib, w, **plan)
        assert np.isfinite(got).all(), f"{plan}: a NaN canary leaked into the output"
        assert_parity(got, ref, f"edge {kv} {plan}")
        assert_lse(lse, ref_lse, "lse")
        assert np.all(got[lens == 0] == 0)


@pytest.mark.parametrize("case", range(16))
def test_seeded_random_shapes(torch, lib, case):
    # Seeded draws over formats, group sizes, KV head counts, batch sizes, length mixes
    # (empty caches included), softmax scales, unreferenced pages and plans, every slot no
    # token owns holding NaN.
    rng = np.random.default_rng(700 + case)
    kv = KVS[case % 4]
    group = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.integers(1, 5))
    batch = int(rng.integers(1, 41))
    hi = int(rng.integers(1, 1200))
    cfg = SMALL.with_(kv_dtype=kv, batch=batch, n_q_heads=group * hkv, n_kv_heads=hkv,
                      len_lo=0, len_hi=hi, scale=float(rng.uniform(0.02, 0.3)))
    # Lengths: uniform, with about one in six empty and one in six a whole number of pages.
    lens = rng.integers(0, hi + 1, size=batch)
    pick = rng.random(batch)
    lens = np.where(pick < 1 / 6, 0, np.where(pick < 2 / 6, 16 * (lens // 16), lens))
    w = generate(cfg, seed=800 + case, poison=True, extra_pages=int(rng.integers(0, 4)),
                 seq_lens=lens.astype(np.int32))
    plan = PLANS[int(rng.integers(0, len(PLANS)))]
    print(f"case decode random {case}: {kv} G={group} Hkv={hkv} B={batch} "
          f"lens={w.seq_lens.tolist()} plan={plan}", flush=True)
    ref, ref_lse = oracle_run(w)
    got, lse = gpu_run(torch, lib, w, **plan)
    assert np.isfinite(got).all(), f"{plan}: a NaN canary leaked into the output"
    assert_parity(got, ref, f"random case {case}")
    assert_lse(lse, ref_lse, f"random case {case}")
    assert np.all(got[w.seq_lens == 0] == 0)


@pytest.mark.parametrize("kv,group", [("fp16", 1), ("fp16", 2), ("int8", 4), ("fp8", 8)])
def test_segment_mode_full_and_partial_rounds(torch, lib, kv, group):
    # 160 segments dealt in a snake over grids that leave the last round full, partial or a
    # single segment, and over one round; lengths from a small set (ties, empty caches).
    n_kv = 4
    cfg = SMALL.with_(kv_dtype=kv, batch=40, n_q_heads=n_kv * group, n_kv_heads=n_kv,
                      len_lo=0, len_hi=700)
    rng = np.random.default_rng(40 + group)
    lens = rng.choice(np.array([0, 1, 16, 17, 64, 65, 300, 700], dtype=np.int32), size=cfg.batch)
    w = generate(cfg, seed=41, seq_lens=lens, extra_pages=2, poison=True)
    print(f"case segment rounds kv={kv} G={group}", flush=True)
    ref, ref_lse = oracle_run(w)
    d = to_dev(torch, w)
    for grid in (3, 7, 31, 53, 80, 159, 160, 161):
        got, lse = gpu_run(torch, lib, w, dev_inputs=d, num_splits=1, num_workgroups=grid)
        assert np.isfinite(got).all(), f"grid {grid}: a NaN canary leaked into the output"
        assert_parity(got, ref, f"segment rounds {kv} G={group} grid {grid}")
        assert_lse(lse, ref_lse, "lse")


@pytest.mark.parametrize("batch", [255, 256, 257])
@pytest.mark.parametrize("grid", [0, 3, 1000])
@pytest.mark.parametrize("caches", ["short", "long"])
def test_segment_mode_order_and_grids(torch, lib, batch, grid, caches):
    # Segment mode ranks batches of up to 256 sequences by decreasing length inside every
    # workgroup (ties by index) and takes larger batches in index order (lengths then come
    # through scalar loads); segments are dealt out in a snake over the grid. Short and
    # long (over 64 pages) caches.
    # Lengths from a small set make ties common; empty caches rank last. Grids: the
    # library's, 3 workgroups (about 170 segments each, so query rows are restaged in LDS
    # many times), and more workgroups than segments.
    choices = [0, 1, 16, 17, 40, 64] + ([1100, 1025] if caches == "long" else [])
    lens = np.random.default_rng(batch).choice(choices, size=batch)
    cfg = SMALL.with_(batch=batch, len_lo=0, len_hi=max(choices))
    w = generate(cfg, seed=30, seq_lens=lens.astype(np.int32), poison=True)
    print(f"case segment order batch={batch} grid={grid} caches={caches}", flush=True)
    ref, ref_lse = oracle_run(w)
    got, lse = gpu_run(torch, lib, w, num_splits=1, num_workgroups=grid)
    assert_parity(got, ref, f"batch {batch} grid {grid}")
    assert_lse(lse, ref_lse, "lse")


@pytest.mark.parametrize("grid", [1, 2, 3])
@pytest.mark.parametrize("kv", ["fp16", "int8"])
def test_segment_mode_very_long_segments(torch, lib, grid, kv):
    # Segment mode over caches of 4096, 4097, 4375 and 8750 pages, with short and empty
    # caches between; on one workgroup they all run back to back.
    lens = np.array([140000, 65536, 100, 65537, 0, 70000, 17], dtype=np.int32)
    cfg = SMALL.with_(kv_dtype=kv, batch=len(lens), n_q_heads=4, n_kv_heads=2, len_lo=0,
                      len_hi=int(lens.max()))
    w = generate(cfg, seed=62, seq_lens=lens, poison=True, extra_pages=3)
    print(f"case segment chunks kv={kv} grid={grid}", flush=True)
    ref, ref_lse = oracle_run(w)
    got, lse = gpu_run(torch, lib, w, num_splits=1, num_workgroups=grid)
    assert_parity(got, ref, f"segment chunks {kv} grid {grid}")
    assert_lse(lse, ref_lse, "lse")


@pytest.mark.parametrize("kv", KVS)
def test_stream_mode_query_rows_beyond_lds(torch, lib, kv):
    # Stream mode stages a workgroup's query rows in LDS when they fit in 16 KiB; one
    # workgroup over 80 (sequence, KV head) segments of G = 8 (2 KiB of query rows each)
    # takes them from global memory instead, as does every workgroup of a 3-workgroup grid.
    cfg = SMALL.with_(kv_dtype=kv, batch=40, n_q_heads=16, n_kv_heads=2, len_lo=1, len_hi=70)
    w = generate(cfg, seed=60)
    print(f"case stream global queries kv={kv}", flush=True)
    ref, ref_lse = oracle_run(w)
    for grid in (1, 3):
        got, lse = gpu_run(torch, lib, w, num_workgroups=grid)
        assert_parity(got, ref, f"{kv} grid {grid}")
        assert_lse(lse, ref_lse, "lse")


@pytest.mark.parametrize("longest", [40000, 70000])
def test_split_mode_partitions_beyond_one_table_chunk(torch, lib, longest):
    # A split workgroup stages its partition's table entries in LDS 1024 pages at a time;
    # two partitions of 40000 or 70000 tokens (1250 or 2188 pages each) need two or three
    # chunks; the shorter sequence ends inside its second chunk.
    cfg = SMALL.with_(batch=2, n_q_heads=4, n_kv_heads=1, len_lo=1, len_hi=longest)
    lens = np.array([longest, 2049 * 16 + 5], dtype=np.int32)
    w = generate(cfg, seed=61, seq_lens=lens, poison=True)
    print(f"case split chunks longest={longest}", flush=True)
    ref, ref_lse = oracle_run(w)
    got, lse = gpu_run(torch, lib, w, num_splits=2)
    assert_parity(got, ref, f"longest {longest}")
    assert_lse(lse, ref_lse, "lse")


@pytest.mark.parametrize("kv", KVS)
def test_segment_mode_long_caches(torch, lib, kv):
    # Eight (sequence, KV head) segments of up to 9000 tokens (563 pages) on one, two or
    # eight workgroups: long runs of pages per wave across several segments, including a
    # single-token one.
    cfg = SMALL.with_(kv_dtype=kv, batch=4, n_q_heads=4, n_kv_heads=2, len_lo=1, len_hi=9000)
    lens = np.array([9000, 1, 4097, 8191], dtype=np.int32)
    w = generate(cfg, seed=50, seq_lens=lens, poison=True)
    print(f"case long caches kv={kv}", flush=True)
    ref, ref_lse = oracle_run(w)
    for grid in (1, 2, 8):
        got, lse = gpu_run(torch, lib, w, num_splits=1, num_workgroups=grid)
        assert_parity(got, ref, f"{kv} grid {grid}")
        assert_lse(lse, ref_lse, "lse")


@pytest.mark.parametrize("kv", KVS)
@pytest.mark.parametrize("group", [1, 4, 8])
def test_segment_mode_restages_query_rows(torch, lib, kv, group):
    # One or two workgroups over 90 (sequence, KV head) segments: more than one LDS chunk of
    # query rows (64 / G segments) per workgroup, with lengths that leave some waves without
    # a page in many segments.
    cfg = SMALL.with_(kv_dtype=kv, batch=45, n_q_heads=2 * group, n_kv_heads=2, len_lo=1,
                      len_hi=90)
    w = generate(cfg, seed=40 + group)
    print(f"case restage kv={kv} G={group}", flush=True)
    ref, ref_lse = oracle_run(w)
    for grid in (1, 2):
        got, lse = gpu_run(torch, lib, w, num_splits=1, num_workgroups=grid)
        assert_parity(got, ref, f"{kv} G={group} grid {grid}")
        assert_lse(lse, ref_lse, "lse")


@pytest.mark.parametrize("kv", ["fp16", "int8"])
@pytest.mark.parametrize("group", [1, 4])
def test_batches_beyond_4096_sequences(torch, lib, kv, group):
    # 4500 sequences of 0-100 tokens (ties and empty caches common; the unused slots of
    # each last page and the spare pages hold NaN). Past 4096 sequences segment mode takes
    # the segments in index order with lengths through scalar loads; it runs on the library's
    # grid and on 3 workgroups (3000 segments each), and split mode on two partitions.
    # Stream mode keeps the batch's page counts in LDS and refuses such a batch.
    batch = 4500
    choices = np.array([0, 1, 16, 17, 40, 64, 100], dtype=np.int32)
    lens = np.random.default_rng(batch + group).choice(choices, size=batch)
    cfg = SMALL.with_(kv_dtype=kv, batch=batch, n_q_heads=2 * group, n_kv_heads=2, len_lo=0,
                      len_hi=int(choices.max()))
    w = generate(cfg, seed=70 + group, seq_lens=lens, poison=True, extra_pages=2)
    print(f"case batch {batch} kv={kv} G={group}", flush=True)
    ref, ref_lse = oracle_run(w)
    d = to_dev(torch, w)
    for name, plan in (("auto", {}), ("segment grid 3", dict(num_splits=1, num_workgroups=3)),
                       ("split 2", dict(num_splits=2))):
        got, lse = gpu_run(torch, lib, w, dev_inputs=d, **plan)
        assert np.isfinite(got).all(), f"{name}: a NaN canary leaked into the output"
        assert_parity(got, ref, f"batch {batch} {kv} G={group} {name}")
        assert_lse(lse, ref_lse, name)
    with pytest.raises(lib.DecodeAttnError) as err:
        gpu_run(torch, lib, w, dev_inputs=d, num_workgroups=64)
    assert err.value.status == 2    # DECODE_ATTN_ERR_UNSUPPORTED


@pytest.mark.parametrize("plan", [dict(num_workgroups=2), dict(num_splits=2),
                                  dict(num_splits=1, num_workgroups=2)],
                         ids=["wg2", "split2", "seg2"])
def test_all_sequences_empty(torch, lib, plan):
    cfg = SMALL.with_(len_lo=0, len_hi=40)
    w = generate(cfg, seed=3, seq_lens=np.zeros(cfg.batch, dtype=np.int32))
    w.k_pages = np.zeros((1,) + w.k_pages.shape[1:], dtype=np.float16)
    w.v_pages = w.k_pages.copy()
    got, lse = gpu_run(torch, lib, w, **plan)
    assert np.all(got == 0) and np.all(np.isneginf(lse))


def test_bad_lengths_and_page_ids_give_nan_not_faults(torch, lib):
    # The kernels range-check every length and every page id they read; a bad one turns
    # that sequence's output into NaN and reads nothing through it. Other sequences are
    # exact.
    w = generate(SMALL.with_(batch=6, len_hi=400), seed=21)
    ref, _ = oracle_run(w)
    mb = SMALL.with_(len_hi=400).max_blocks_per_seq
    lens = w.seq_lens.copy()
    lens[1] = mb * 16 + 1          # longer than the table allows
    lens[4] = -3                   # negative
    table = w.block_table.copy()
    nb3 = -(-int(lens[3]) // 16)
    table[3, nb3 - 1] = w.num_pages        # one past the pool
    table[5, 0] = -7
    w.seq_lens, w.block_table = lens, table
    for plan in (dict(num_workgroups=1), dict(num_workgroups=5), dict(num_workgroups=40),
                 dict(num_splits=1), dict(num_splits=1, num_workgroups=1),
                 dict(num_splits=1, num_workgroups=4), dict(num_splits=4)):
        got, lse = gpu_run(torch, lib, w, **plan)
        for b in (1, 3, 4, 5):
            assert np.isnan(got[b]).all() and np.isnan(lse[b]).all(), (plan, b)
        for b in (0, 2):
            assert_parity(got[b], ref[b], f"clean sequence {b} {plan}")


@pytest.mark.parametrize("plan", [dict(num_workgroups=2), dict(num_splits=2),
                                  dict(num_splits=1, num_workgroups=2)],
                         ids=["wg2", "split2", "seg2"])
def test_page_permutation_is_bitwise_invariant(torch, lib, plan):
    w = generate(SMALL, seed=12, extra_pages=3)
    a, _ = gpu_run(torch, lib, w, **plan)
    perm = np.random.default_rng(0).permutation(w.num_pages)
    k2 = np.empty_like(w.k_pages)
    v2 = np.empty_like(w.v_pages)
    k2[perm] = w.k_pages
    v2[perm] = w.v_pages
    w.k_pages, w.v_pages = k2, v2
    w.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    b, _ = gpu_run(torch, lib, w, **plan)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("kv", KVS)
@pytest.mark.parametrize("group", [1, 4, 8])
@pytest.mark.parametrize("scale", [-0.2, 0.0, 2.0])
def test_softmax_scale_extremes(torch, lib, kv, group, scale):
    """A negative scale (the smallest products get the largest weights), a zero scale (the
    mean of V) and a sharp one (near one-hot weights), on both consumes (vector G = 1,
    matrix cores G >= 4 over fp16, INT8, FP8) and every plan kind."""
    cfg = SMALL.with_(kv_dtype=kv, n_q_heads=2 * group, n_kv_heads=2, len_lo=1, len_hi=400)
    w = generate(cfg, seed=50 + group)
    w.scale = float(np.float32(scale))
    print(f"case scale {scale} kv={kv} G={group}", flush=True)
    ref, ref_lse = oracle_run(w)
    d = to_dev(torch, w)
    for plan in (dict(num_splits=1), dict(num_workgroups=3), dict(num_splits=3)):
        got, lse = gpu_run(torch, lib, w, dev_inputs=d, **plan)
        assert_parity(got, ref, f"scale {scale} {kv} G={group} {plan}")
        assert_lse(lse, ref_lse, "lse")


@pytest.mark.parametrize("kv", ["fp16", "int8"])
@pytest.mark.parametrize("group", [1, 4, 8])
def test_running_max_rises_every_page(torch, lib, kv, group):
    """Scores that grow along each cache (key t = (t / 64) u, with every query head equal
    to u), so the running max keeps moving: by about 4 log2 units per page, past the matrix-
    core consume's lazy threshold every two pages; the weights end up on the last few
    tokens."""
    cfg = SMALL.with_(kv_dtype=kv, n_q_heads=2 * group, n_kv_heads=2, len_lo=200, len_hi=400)
    w = generate(cfg, seed=70 + group)
    rng = np.random.default_rng(71)
    u = rng.standard_normal(128).astype(np.float32)
    w.q[...] = u.astype(np.float16)
    bs = cfg.block_size
    for b in range(cfg.batch):
        for t in range(int(w.seq_lens[b])):
            page, slot = int(w.block_table[b, t // bs]), t % bs
            c = t / 64.0
            if kv == "fp16":
                w.k_pages[page, :, slot, :] = (c * u).astype(np.float16)
            else:
                w.k_pages[page, :, slot, :] = np.clip(np.rint(u * 30.0), -127, 127).astype(np.int8)
                w.k_scale[page, :, slot] = np.float32(c / 30.0)
    print(f"case rising max kv={kv} G={group}", flush=True)
    ref, ref_lse = oracle_run(w)
    d = to_dev(torch, w)
    for plan in (dict(num_splits=1), dict(num_workgroups=3), dict(num_splits=3)):
        got, lse = gpu_run(torch, lib, w, dev_inputs=d, **plan)
        assert_parity(got, ref, f"rising max {kv} G={group} {plan}")
        assert_lse(lse, ref_lse, "lse")


def test_gqa_matches_repeated_mha(torch, lib):
    """G = 4 against the same heads as MHA (K/V repeated per query head). The G = 4 build
    runs on the matrix cores, which take each softmax weight rounded to fp16 (relative error
    at most 2^-11; the normaliser sums the unrounded weights), while G = 1 keeps fp32
    weights: the outputs may differ by at most 2^-11 max|V| per row, plus fp16 underflow of
    weights below 2^-14 (at most 2^-25 each, L <= 300 of them here)."""
    w = generate(SMALL, seed=13)
    a, lse_a = gpu_run(torch, lib, w, num_workgroups=1)
    group = SMALL.n_q_heads // SMALL.n_kv_heads
    w.k_pages = np.repeat(w.k_pages, group, axis=1)
    w.v_pages = np.repeat(w.v_pages, group, axis=1)
    b, lse_b = gpu_run(torch, lib, w, num_workgroups=1)
    vmax = float(np.abs(w.v_pages.astype(np.float64)).max())
    bound = 2.0 ** -11 * vmax + SMALL.len_hi * 2.0 ** -25 * vmax + 1e-6
    np.testing.assert_allclose(a, b, rtol=0, atol=bound)
    np.testing.assert_allclose(lse_a, lse_b, rtol=1e-6, atol=1e-5)


def test_int8_unit_scales_match_fp16_on_same_integers(torch, lib):
    cfg = SMALL.with_(kv_dtype="int8")
    w = generate(cfg, seed=14)
    w.scale = 0.001  # raw int8 dot products are ~1e3; keep the softmax soft
    w.k_scale = np.ones_like(w.k_scale)
    w.v_scale = np.ones_like(w.v_scale)
    a, _ = gpu_run(torch, lib, w, num_workgroups=1)
    w.k_pages = w.k_pages.astype(np.float16)
    w.v_pages = w.v_pages.astype(np.float16)
    w.k_scale = w.v_scale = None
    b, _ = gpu_run(torch, lib, w, num_workgroups=1)
    np.testing.assert_allclose(a, b, rtol=1e-5, atol=1e-5)


def test_fp8_small_integers_match_int8_bitwise(torch, lib):
    # E4M3 codes whose values are the integers -16..16 decode to the same exact fp16 pairs
    # as those integers stored as INT8, so with the same row scales both paths do identical
    # arithmetic.
    table = oracle.e4m3_to_float64(np.arange(256, dtype=np.uint8))
    code_of = {int(v): c for c, v in enumerate(table)
               if np.isfinite(v) and v == int(v) and abs(v) <= 16 and not (v == 0 and c)}
    cfg = SMALL.with_(kv_dtype="int8", n_q_heads=8, n_kv_heads=2)
    w = generate(cfg, seed=17)
    rng = np.random.default_rng(17)
    ints = [rng.integers(-16, 17, size=w.k_pages.shape) for _ in range(2)]
    w.k_pages, w.v_pages = (i.astype(np.int8) for i in ints)
    for plan in (dict(), dict(num_workgroups=3), dict(num_splits=1), dict(num_splits=3)):
        a, la = gpu_run(torch, lib, w, **plan)
        w8 = generate(cfg, seed=17)
        w8.k_pages, w8.v_pages = (np.vectorize(code_of.get)(i).astype(np.uint8) for i in ints)
        b, lb = gpu_run(torch, lib, w8, **plan)
        assert np.array_equal(a, b) and np.array_equal(la, lb), f"{plan}"
    assert_parity(a, oracle_run(w)[0], "int8 integers")


def test_fp8_and_int8_small_integers_agree_on_the_vector_consume(torch, lib):
    # With one query head per KV head the vector consume runs: FP8 widens its codes to the
    # exact integers, INT8 carries them as 1152 + x and takes the offset off per load and
    # per segment. Both must agree to rounding (the offset's fp32 rounding is far below the
    # parity tolerance), in every plan mode, and both must match the oracle.
    table = oracle.e4m3_to_float64(np.arange(256, dtype=np.uint8))
    code_of = {int(v): c for c, v in enumerate(table)
               if np.isfinite(v) and v == int(v) and abs(v) <= 16 and not (v == 0 and c)}
    cfg = SMALL.with_(kv_dtype="int8", n_q_heads=4, n_kv_heads=4)
    w = generate(cfg, seed=19)
    rng = np.random.default_rng(19)
    ints = [rng.integers(-16, 17, size=w.k_pages.shape) for _ in range(2)]
    w.k_pages, w.v_pages = (i.astype(np.int8) for i in ints)
    ref = oracle_run(w)[0]
    for plan in (dict(), dict(num_workgroups=3), dict(num_splits=1), dict(num_splits=3)):
        a, la = gpu_run(torch, lib, w, **plan)
        w8 = generate(cfg, seed=19)
        w8.k_pages, w8.v_pages = (np.vectorize(code_of.get)(i).astype(np.uint8) for i in ints)
        b, lb = gpu_run(torch, lib, w8, **plan)
        np.testing.assert_allclose(a, b, rtol=1e-4, atol=1e-4, err_msg=f"{plan}")
        np.testing.assert_allclose(la, lb, rtol=1e-4, atol=1e-4, err_msg=f"{plan}")
        assert_parity(a, ref, f"int8 integers, {plan}")


@pytest.mark.parametrize("plan", [dict(), dict(num_splits=1), dict(num_workgroups=64)],
                         ids=["auto", "segment", "stream"])
def test_int8_offset_over_a_long_cache(torch, lib, plan):
    # The INT8 vector consume adds w (v + 1152) and takes 1152 Σw off once per segment, so
    # its fp32 rounding grows with the cache: at most about 2^-24 · 1152 · √L of a row
    # scale per output, 3.5e-4 here (65 536 tokens, scales at their largest, 0.02), against
    # the 2e-3 absolute bound (measured: below 1e-5 in every mode). One sequence per KV head
    # runs as one segment, as partitions or as stream runs.
    cfg = Config(0, "long_int8_mha", batch=1, n_q_heads=4, n_kv_heads=4, head_dim=128,
                 block_size=16, len_lo=65536, len_hi=65536, kv_dtype="int8")
    w = generate(cfg, seed=23)
    w.k_scale = np.full_like(w.k_scale, 0.02)
    w.v_scale = np.full_like(w.v_scale, 0.02)
    got, lse = gpu_run(torch, lib, w, **plan)
    ref, ref_lse = oracle_run(w)
    assert_parity(got, ref, f"int8, 65536 tokens, {plan}")
    assert np.abs(got.astype(np.float64) - ref).max() < 1e-3
    assert_lse(lse, ref_lse, f"int8, 65536 tokens, {plan}")


def test_fp8_subnormal_codes_are_not_flushed(torch, lib):
    # One key per sequence made of subnormal codes (exponent field 0, values m/8 * 2^-6)
    # with a large row scale, so its score dominates only if the subnormals survive the
    # conversion; the values of that token are subnormal codes too.
    cfg = SMALL.with_(kv_dtype="fp8", n_q_heads=2, n_kv_heads=2, len_lo=20, len_hi=40)
    w = generate(cfg, seed=18)
    w.q = np.abs(w.q)
    rng = np.random.default_rng(18)
    for b in range(cfg.batch):
        page = w.block_table[b, 0]
        w.k_pages[page, :, 3, :] = rng.integers(1, 8, size=(2, 128))      # +m/8 * 2^-6
        w.v_pages[page, :, 3, :] = rng.integers(1, 8, size=(2, 128)) | 0x80
        w.k_scale[page, :, 3] = 400.0
        w.v_scale[page, :, 3] = 64.0
    ref, ref_lse = oracle_run(w)
    got, lse = gpu_run(torch, lib, w)
    assert_parity(got, ref, "fp8 subnormals")
    assert_lse(lse, ref_lse, "lse")
    assert np.all(ref < 0), "the subnormal token must dominate the reference"


def test_output_guard_words_untouched(torch, lib):
    w = generate(SMALL, seed=15)
    d = to_dev(torch, w)
    n = w.q.size
    buf = torch.full((n + 2 * 64,), 12345.0, dtype=torch.float32, device="cuda:0")
    out = buf[64:64 + n].view(w.q.shape)
    lib.decode_attn_ex(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["seq_lens"],
                       w.scale, out=out, num_workgroups=3)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert np.all(host[:64] == 12345.0) and np.all(host[64 + n:] == 12345.0)
    assert_parity(host[64:64 + n].reshape(w.q.shape), oracle_run(w)[0], "guarded")


def test_library_owned_workspace_entry_point(torch, lib):
    w = generate(SMALL.with_(len_hi=2000), seed=16)
    d = to_dev(torch, w)
    out = lib.decode_attn(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["seq_lens"],
                          w.scale)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy(), oracle_run(w)[0], "decode_attn")
    ex, _ = gpu_run(torch, lib, w, num_workgroups=0, lse=False, dev_inputs=d)
    assert np.array_equal(out.cpu().numpy(), ex)


def test_one_hip_runtime_and_native_library(torch, lib):
    lib.load_library()
    maps = open("/proc/self/maps").read().splitlines()
    hip = {ln.split()[-1] for ln in maps if "libamdhip64" in ln}
    ours = {ln.split()[-1] for ln in maps if "libdecode_attn.so" in ln}
    assert len(hip) == 1, f"more than one HIP runtime mapped: {hip}"
    assert len(ours) == 1 and next(iter(ours)).startswith(os.path.dirname(lib.__file__))


# ------------------------------------------------------------------ the preset workloads

@pytest.mark.parametrize("index", [1, 2, 3, 4, 5, 6, 7, 9, 10, 11])
def test_preset_workload_full_size(torch, lib, index):
    """Each preset at its full size, in the launch configuration the benchmark times
    (library-chosen grid), compared elementwise on every output."""
    w = generate(CONFIGS[index])
    print(f"case preset {index} ({CONFIGS[index].name}) pages={w.num_pages}", flush=True)
    got, lse = gpu_run(torch, lib, w, num_workgroups=0)
    ref, ref_lse = oracle_run(w)
    assert_parity(got, ref, f"preset {index}")
    assert_lse(lse, ref_lse, "lse")
