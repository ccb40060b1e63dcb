"""GPU parity of decode_attn_prefill (chunked-prefill attention on the matrix cores) against
the fp64 oracle: every chunk row within |gpu - oracle| <= 2e-3 + 1e-2 |oracle|. Chunks of
every size class (whole prompts, single decode tokens, page-crossing, more rows than one
workgroup block), every group size, a grid smaller than the chunks, NaN canaries in every
slot no token owns, bad device values, and the full-size preset on sampled sequences.
Every call goes through the C ABI."""

import numpy as np
import pytest

import oracle
from decode_phase_attention_paged_amd.workload import CONFIGS, Config, generate, prefill_rows

from test_gpu_parity import assert_parity, dev_tensor

pytestmark = pytest.mark.gpu

SMALL = Config(0, "small_prefill", batch=5, n_q_heads=8, n_kv_heads=2, head_dim=128,
               block_size=16, len_lo=1, len_hi=200, kv_dtype="fp16")


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need an MI355X"
    return t


@pytest.fixture(scope="module")
def lib(torch):
    from decode_phase_attention_paged_amd import binding
    return binding


def chunk_layout(lens, rng, kinds=("full", "one", "rand")):
    sizes = []
    for i, n in enumerate(lens):
        kind = kinds[i % len(kinds)]
        n = int(n)
        sizes.append(n if kind == "full" else 1 if kind == "one" else int(rng.integers(1, n + 1)))
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def draw_q(rng, rows, cfg):
    """Chunk rows ~ N(0, 1): fp16, or bf16 bit patterns (uint16) for a bf16 cache."""
    q32 = rng.standard_normal((rows, cfg.n_q_heads, 128)).astype(np.float32)
    if cfg.kv_dtype == "bf16":
        return (q32.view(np.uint32) >> 16).astype(np.uint16)
    return q32.astype(np.float16)


def run(torch, lib, w, q, q_start, max_chunk=None, out=None):
    t = lambda a: dev_tensor(torch, a)
    got = lib.decode_attn_prefill(t(q), t(q_start), t(w.k_pages), t(w.v_pages), t(w.block_table),
                                  t(w.seq_lens), w.scale, k_scale=t(w.k_scale),
                                  v_scale=t(w.v_scale), max_chunk=max_chunk, out=out)
    torch.cuda.synchronize()
    return got.cpu().numpy()


def reference(w, q, q_start):
    return oracle.prefill_attention(q, w.k_pages, w.v_pages, w.block_table, w.seq_lens,
                                    q_start, w.scale, w.k_scale, w.v_scale)[0]


@pytest.mark.parametrize("kv", ["fp16", "bf16", "int8", "fp8"])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("seed", [1, 2])
def test_small_mixed_chunks(torch, lib, kv, group, seed):
    # NaN canaries sit in every slot no token owns, scales included.
    cfg = SMALL.with_(n_q_heads=2 * group, n_kv_heads=2, kv_dtype=kv)
    w = generate(cfg, seed=200 + seed, poison=True, extra_pages=3)
    rng = np.random.default_rng(seed)
    q_start = chunk_layout(w.seq_lens, rng)
    q = draw_q(rng, int(q_start[-1]), cfg)
    print(f"case prefill {kv} G={group} seed={seed} lens={w.seq_lens.tolist()} "
          f"chunks={np.diff(q_start).tolist()}", flush=True)
    got = run(torch, lib, w, q, q_start)
    assert np.isfinite(got).all(), "a NaN canary leaked"
    assert_parity(got, reference(w, q, q_start), f"prefill {kv} G={group}")


@pytest.mark.parametrize("max_chunk", [1, 7, 64, 10000])
def test_grid_smaller_than_the_chunks(torch, lib, max_chunk):
    # The grid is sized from max_chunk; workgroups loop over the remaining row blocks.
    cfg = SMALL.with_(batch=3, len_lo=150, len_hi=300)
    w = generate(cfg, seed=210)
    rng = np.random.default_rng(210)
    q_start = chunk_layout(w.seq_lens, rng, kinds=("full",))
    q = rng.standard_normal((int(q_start[-1]), cfg.n_q_heads, 128)).astype(np.float16)
    print(f"case prefill max_chunk={max_chunk}", flush=True)
    got = run(torch, lib, w, q, q_start, max_chunk=max_chunk)
    assert_parity(got, reference(w, q, q_start), f"max_chunk {max_chunk}")


def test_one_token_chunks_match_decode(torch, lib):
    # A batch of one-token chunks is a decode step: same results as decode_attn within the
    # tolerance (the two kernels round differently).
    w = generate(SMALL, seed=211)
    q_start = np.arange(SMALL.batch + 1, dtype=np.int32)
    got = run(torch, lib, w, w.q, q_start)
    t = lambda a: dev_tensor(torch, a)
    dec = lib.decode_attn(t(w.q), t(w.k_pages), t(w.v_pages), t(w.block_table), t(w.seq_lens),
                          w.scale)
    torch.cuda.synchronize()
    ref = oracle.decode_attention(w.q, w.k_pages, w.v_pages, w.block_table, w.seq_lens, w.scale)[0]
    assert_parity(got, ref, "one-token chunks")
    assert_parity(dec.cpu().numpy(), ref, "decode")


def test_bad_values_give_nan_and_leave_other_rows(torch, lib):
    cfg = SMALL.with_(batch=4, len_lo=40, len_hi=90)
    w = generate(cfg, seed=212)
    rng = np.random.default_rng(212)
    q_start = chunk_layout(w.seq_lens, rng, kinds=("rand",))
    q = rng.standard_normal((int(q_start[-1]) + 5, cfg.n_q_heads, 128)).astype(np.float16)
    table = w.block_table.copy()
    table[1, 1] = w.num_pages + 7                   # a bad page id for sequence 1
    lens = w.seq_lens.copy()
    lens[2] = int(q_start[3] - q_start[2]) - 1       # sequence 2: chunk longer than L_b
    t = lambda a: dev_tensor(torch, a)
    out = torch.full(q.shape, 777.0, dtype=torch.float32, device="cuda:0")
    lib.decode_attn_prefill(t(q), t(q_start), t(w.k_pages), t(w.v_pages), t(table), t(lens),
                            w.scale, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isnan(got[q_start[1]:q_start[2]]).all()
    assert np.isnan(got[q_start[2]:q_start[3]]).all()
    assert np.all(got[q_start[-1]:] == 777.0), "rows outside every chunk were written"
    keep = np.r_[q_start[0]:q_start[1], q_start[3]:q_start[4]]
    ref = reference(w, q[:q_start[-1]], q_start)
    assert_parity(got[keep], ref[keep], "good sequences")


def test_full_size_preset_every_sequence(torch, lib):
    """The prefill preset at full size, in the launch the benchmark times, against the
    oracle on every row of all eight sequences."""
    cfg = CONFIGS[8]
    w = generate(cfg)
    q, q_start = prefill_rows(w)
    print(f"case prefill preset rows={q.shape[0]}", flush=True)
    got = run(torch, lib, w, q, q_start, max_chunk=cfg.chunk)
    ref = oracle.prefill_attention(q, w.k_pages, w.v_pages, w.block_table, w.seq_lens, q_start,
                                   w.scale)[0]
    for b in range(cfg.batch):
        rows = slice(int(q_start[b]), int(q_start[b + 1]))
        assert_parity(got[rows], ref[rows], f"preset sequence {b} (L={int(w.seq_lens[b])})")


@pytest.mark.parametrize("batch,hkv", [(4, 2), (8, 1), (3, 8)])
def test_work_orders(torch, lib, batch, hkv):
    # Pair counts that are multiples of 8 run every row block of a (sequence, KV head) on
    # one die; the others run in rank order only. Lengths with ties check the ranking.
    cfg = SMALL.with_(batch=batch, n_q_heads=4 * hkv, n_kv_heads=hkv, len_lo=20, len_hi=330)
    rng = np.random.default_rng(300 + batch)
    lens = rng.integers(20, 331, size=batch).astype(np.int32)
    lens[batch // 2] = lens[0]
    w = generate(cfg, seed=301, poison=True, seq_lens=lens)
    q_start = chunk_layout(w.seq_lens, rng)
    q = rng.standard_normal((int(q_start[-1]), cfg.n_q_heads, 128)).astype(np.float16)
    print(f"case prefill order batch={batch} hkv={hkv} lens={w.seq_lens.tolist()}", flush=True)
    got = run(torch, lib, w, q, q_start, max_chunk=int(np.diff(q_start).max()))
    assert_parity(got, reference(w, q, q_start), f"order {batch}x{hkv}")


def test_batch_beyond_the_ranked_order(torch, lib):
    # More than 256 sequences: the workgroups take pairs in index order.
    cfg = SMALL.with_(batch=300, n_q_heads=4, n_kv_heads=1, len_lo=1, len_hi=40)
    w = generate(cfg, seed=302)
    rng = np.random.default_rng(302)
    q_start = chunk_layout(w.seq_lens, rng)
    q = rng.standard_normal((int(q_start[-1]), cfg.n_q_heads, 128)).astype(np.float16)
    print("case prefill batch 300", flush=True)
    got = run(torch, lib, w, q, q_start)
    assert_parity(got, reference(w, q, q_start), "batch 300")


@pytest.mark.parametrize("scale", [-0.0883883, 0.0, 0.5])
def test_scales(torch, lib, scale):
    # A negative scale runs as |scale| on -q; a zero scale gives uniform weights; a large
    # one makes peaky rows whose reference max moves often.
    cfg = SMALL.with_(batch=3, n_q_heads=8, n_kv_heads=2, len_lo=60, len_hi=260, scale=scale)
    w = generate(cfg, seed=303)
    rng = np.random.default_rng(303)
    q_start = chunk_layout(w.seq_lens, rng)
    q = rng.standard_normal((int(q_start[-1]), cfg.n_q_heads, 128)).astype(np.float16)
    print(f"case prefill scale={scale}", flush=True)
    got = run(torch, lib, w, q, q_start)
    assert_parity(got, reference(w, q, q_start), f"scale {scale}")


def test_graph_replays_match_eager(torch, lib):
    # The prefill launches one kernel and allocates nothing, so a captured call replays: with
    # new chunk rows copied in before each replay and an eager call in between, every replay
    # must give the eager call's bit pattern and match the oracle.
    cfg = SMALL.with_(batch=4, len_lo=30, len_hi=300)
    w = generate(cfg, seed=304, poison=True)
    rng = np.random.default_rng(304)
    q_start = chunk_layout(w.seq_lens, rng)
    shape = (int(q_start[-1]), cfg.n_q_heads, 128)
    t = lambda a: dev_tensor(torch, a)
    d = dict(q=t(rng.standard_normal(shape).astype(np.float16)), q_start=t(q_start),
             k_pages=t(w.k_pages), v_pages=t(w.v_pages), block_table=t(w.block_table),
             seq_lens=t(w.seq_lens))
    out = torch.zeros(shape, dtype=torch.float32, device="cuda:0")
    eager = torch.empty_like(out)

    def call(dst):
        lib.decode_attn_prefill(d["q"], d["q_start"], d["k_pages"], d["v_pages"],
                                d["block_table"], d["seq_lens"], w.scale, out=dst)

    print("case prefill graph", flush=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out)                                    # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out)
    torch.cuda.synchronize()
    for replay in range(3):
        q_new = rng.standard_normal(shape).astype(np.float16)
        d["q"].copy_(t(q_new))
        graph.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        call(eager)                                  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(got, eager.cpu().numpy()), f"replay {replay}: out differs"
        assert_parity(got, reference(w, q_new, q_start), f"prefill graph replay {replay}")


def test_deterministic(torch, lib):
    # The same inputs give the same bits: the kernel has no atomics and a fixed order.
    cfg = SMALL.with_(batch=6, len_lo=50, len_hi=400, n_q_heads=16, n_kv_heads=4)
    w = generate(cfg, seed=305)
    rng = np.random.default_rng(305)
    q_start = chunk_layout(w.seq_lens, rng)
    q = rng.standard_normal((int(q_start[-1]), cfg.n_q_heads, 128)).astype(np.float16)
    print("case prefill determinism", flush=True)
    first = run(torch, lib, w, q, q_start)
    second = run(torch, lib, w, q, q_start)
    assert np.array_equal(first, second)


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
def test_formats_at_the_preset_shape(torch, lib, kv):
    """The prefill preset's shapes over the other storage formats, in the launch the
    benchmark times, against the oracle on every row of all eight sequences."""
    cfg = CONFIGS[8].with_(kv_dtype=kv)
    w = generate(cfg)
    q, q_start = prefill_rows(w)
    print(f"case prefill preset {kv} rows={q.shape[0]}", flush=True)
    got = run(torch, lib, w, q, q_start, max_chunk=cfg.chunk)
    ref = oracle.prefill_attention(q, w.k_pages, w.v_pages, w.block_table, w.seq_lens, q_start,
                                   w.scale, w.k_scale, w.v_scale)[0]
    for b in range(cfg.batch):
        rows = slice(int(q_start[b]), int(q_start[b + 1]))
        assert_parity(got[rows], ref[rows], f"preset {kv} sequence {b} (L={int(w.seq_lens[b])})")


@pytest.mark.parametrize("kv", ["int8", "fp8"])
def test_coded_one_token_chunks_match_decode(torch, lib, kv):
    # One-token chunks over a coded cache: the prefill (dequantised on staging, fp16 matrix
    # cores) and decode (codes in registers, scales on scores and weights) both within the
    # tolerance of the oracle.
    cfg = SMALL.with_(kv_dtype=kv)
    w = generate(cfg, seed=306)
    q_start = np.arange(cfg.batch + 1, dtype=np.int32)
    got = run(torch, lib, w, w.q, q_start)
    ref = oracle.decode_attention(w.q, w.k_pages, w.v_pages, w.block_table, w.seq_lens, w.scale,
                                  w.k_scale, w.v_scale)[0]
    assert_parity(got, ref, f"{kv} one-token chunks")


def test_empty_chunks_and_empty_sequences(torch, lib):
    # Sequences with no chunk rows (C_b = 0, some of them with L_b = 0 too) sit between real
    # chunks: they write nothing and leave the other sequences' rows exact.
    cfg = SMALL.with_(batch=6, len_lo=1, len_hi=120)
    lens = np.array([0, 57, 33, 0, 120, 9], dtype=np.int32)
    w = generate(cfg, seed=307, poison=True, seq_lens=lens)
    sizes = np.array([0, 57, 0, 0, 40, 9])
    q_start = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rng = np.random.default_rng(307)
    q = draw_q(rng, int(q_start[-1]), cfg)
    print("case prefill empty chunks", flush=True)
    t = lambda a: dev_tensor(torch, a)
    out = torch.full(q.shape, 777.0, dtype=torch.float32, device="cuda:0")
    got = run(torch, lib, w, q, q_start, out=out)
    assert np.isfinite(got).all()
    assert_parity(got, reference(w, q, q_start), "empty chunks")


@pytest.mark.parametrize("case", range(12))
def test_seeded_random_shapes(torch, lib, case):
    # Seeded draws over formats, group sizes, batch sizes, lengths and chunk layouts
    # (including chunks longer than one workgroup's 128 rows and grids sized below them).
    rng = np.random.default_rng(400 + case)
    kv = ["fp16", "bf16", "int8", "fp8"][case % 4]
    group = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.integers(1, 4))
    batch = int(rng.integers(1, 7))
    hi = int(rng.integers(16, 400))
    cfg = SMALL.with_(batch=batch, n_q_heads=group * hkv, n_kv_heads=hkv, len_lo=1, len_hi=hi,
                      kv_dtype=kv, scale=float(rng.uniform(0.02, 0.2)))
    w = generate(cfg, seed=500 + case, poison=True, extra_pages=int(rng.integers(0, 3)))
    sizes = np.array([int(rng.integers(0, n + 1)) for n in w.seq_lens])
    q_start = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    q = draw_q(rng, int(q_start[-1]), cfg)
    max_chunk = int(rng.choice([1, 16, max(1, int(sizes.max()))]))
    print(f"case prefill random {case}: {kv} G={group} Hkv={hkv} lens={w.seq_lens.tolist()} "
          f"chunks={sizes.tolist()} max_chunk={max_chunk}", flush=True)
    got = run(torch, lib, w, q, q_start, max_chunk=max_chunk)
    assert np.isfinite(got).all(), "a NaN canary leaked"
    assert_parity(got, reference(w, q, q_start), f"random case {case}")
