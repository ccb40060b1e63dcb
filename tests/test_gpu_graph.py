"""HIP-graph capture of the library's calls, and workspace reuse.

A decode step is launch-bound at small batch, so a serving loop captures it once and
replays it. Every entry point launches kernels only (no memset, copy or allocation), so
captures work: each replay, with new inputs copied into the captured buffers and eager
work in between, must give the bit pattern the same call gives eagerly. The workspace is
scratch: one workspace full of garbage serves calls of any shape and partition count.
Every call goes through the C ABI.
"""

import numpy as np
import pytest

import oracle
from decode_phase_attention_paged_amd.workload import Config, generate

from test_gpu_parity import assert_parity, dev_tensor, oracle_run, to_dev

pytestmark = pytest.mark.gpu

SMALL = Config(0, "small_gqa", batch=6, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
               len_lo=1, len_hi=700, kv_dtype="fp16")


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need an MI355X"
    return t


@pytest.fixture(scope="module")
def lib(torch):
    from decode_phase_attention_paged_amd import binding
    return binding


def workspace_for(torch, lib, w, **plan):
    c = w.config
    need = lib.plan(c.batch, c.max_blocks_per_seq, c.n_q_heads, c.n_kv_heads, 16, c.kv_dtype,
                    num_cus=torch.cuda.get_device_properties(0).multi_processor_count,
                    **plan).workspace_bytes
    return torch.full((max(need, 256),), 0x5A, dtype=torch.uint8, device="cuda:0")


def call(lib, d, w, out, ws, lse=None, **plan):
    return lib.decode_attn_ex(d["q"], d["k_pages"], d["v_pages"], d["block_table"],
                              d["seq_lens"], w.scale, k_scale=d["k_scale"], v_scale=d["v_scale"],
                              out=out, lse_out=lse, workspace=ws, **plan)


PLANS = [dict(num_splits=1), dict(num_splits=3), dict(num_workgroups=5), dict()]
IDS = ["segment", "split3", "stream5", "auto"]


@pytest.mark.parametrize("kv", ["fp16", "int8"])
@pytest.mark.parametrize("plan", PLANS, ids=IDS)
def test_graph_replays_match_eager(torch, lib, kv, plan):
    cfg = SMALL.with_(kv_dtype=kv)
    w = generate(cfg, seed=90)
    d = to_dev(torch, w)
    shape = w.q.shape
    out = torch.zeros(shape, dtype=torch.float32, device="cuda:0")
    lse = torch.zeros(shape[:2], dtype=torch.float32, device="cuda:0")
    ws = workspace_for(torch, lib, w, **plan)
    print(f"case graph kv={kv} plan={plan}", flush=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(lib, d, w, out, ws, lse, **plan)           # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(lib, d, w, out, ws, lse, **plan)
    torch.cuda.synchronize()

    eager_out = torch.empty_like(out)
    eager_lse = torch.empty_like(lse)
    eager_ws = workspace_for(torch, lib, w, **plan)
    rng = np.random.default_rng(91)
    for replay in range(3):
        q_new = rng.standard_normal(shape).astype(np.float16)
        d["q"].copy_(dev_tensor(torch, q_new))
        graph.replay()
        torch.cuda.synchronize()
        got, got_lse = out.cpu().numpy(), lse.cpu().numpy()
        call(lib, d, w, eager_out, eager_ws, eager_lse, **plan)   # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(got, eager_out.cpu().numpy()), f"replay {replay}: out differs"
        assert np.array_equal(got_lse, eager_lse.cpu().numpy()), f"replay {replay}: lse differs"
        w.q = q_new
        assert_parity(got, oracle_run(w)[0], f"graph {kv} {plan} replay {replay}")


def test_graph_of_a_decode_step(torch, lib):
    # Append each sequence's new K/V rows, then attend over the grown cache: one graph per
    # decode step, replayed for three steps with new rows and positions each time.
    cfg = SMALL.with_(kv_dtype="int8", len_lo=5, len_hi=60)
    w = generate(cfg, seed=92)
    table = w.block_table.copy()
    lens = w.seq_lens.copy()
    extra = 0
    for b in range(cfg.batch):
        for p in range(int(lens[b]), int(lens[b]) + 3):
            if table[b, p // 16] < 0:
                table[b, p // 16] = w.num_pages + extra
                extra += 1
    shape = (extra,) + w.k_pages.shape[1:]
    k_pages = np.concatenate([w.k_pages, np.zeros(shape, dtype=np.int8)])
    v_pages = np.concatenate([w.v_pages, np.zeros(shape, dtype=np.int8)])
    k_scale = np.concatenate([w.k_scale, np.zeros(shape[:3], dtype=np.float32)])
    v_scale = np.concatenate([w.v_scale, np.zeros(shape[:3], dtype=np.float32)])
    t = lambda a: dev_tensor(torch, a)
    d = dict(q=t(w.q), k_pages=t(k_pages), v_pages=t(v_pages), k_scale=t(k_scale),
             v_scale=t(v_scale), block_table=t(table), seq_lens=t(lens))
    rows = (cfg.batch, cfg.n_kv_heads, 128)
    k_new = torch.zeros(rows, dtype=torch.float16, device="cuda:0")
    v_new = torch.zeros_like(k_new)
    pos = torch.zeros(cfg.batch, dtype=torch.int32, device="cuda:0")
    out = torch.zeros(w.q.shape, dtype=torch.float32, device="cuda:0")
    ws = workspace_for(torch, lib, w, num_splits=2)
    print("case graph decode step", flush=True)

    def step():
        lib.decode_attn_append(k_new, v_new, d["block_table"], pos, d["k_pages"], d["v_pages"],
                               k_scale=d["k_scale"], v_scale=d["v_scale"])
        call(lib, d, w, out, ws, num_splits=2)

    # Capture with positions that skip every row (p < 0), so the warm-up and the capture
    # leave the cache as it is.
    pos.fill_(-1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    ref = [k_pages, v_pages, k_scale, v_scale]
    rng = np.random.default_rng(93)
    for s in range(3):
        new = [rng.standard_normal(rows).astype(np.float16) for _ in range(2)]
        p = (lens + s).astype(np.int32)
        k_new.copy_(t(new[0]))
        v_new.copy_(t(new[1]))
        pos.copy_(t(p))
        d["seq_lens"].copy_(t(p + 1))
        graph.replay()
        torch.cuda.synchronize()
        ref = list(oracle.append_kv(ref[0], ref[1], table, p, new[0], new[1], 16, ref[2], ref[3]))
        assert np.array_equal(d["k_pages"].cpu().numpy(), ref[0]), f"step {s}: K pool"
        assert np.array_equal(d["v_scale"].cpu().numpy(), ref[3]), f"step {s}: V scales"
        want, _ = oracle.decode_attention(w.q, ref[0], ref[1], table, p + 1, w.scale, ref[2],
                                          ref[3])
        assert_parity(out.cpu().numpy(), want, f"decode step {s}")


@pytest.mark.parametrize("kv", ["fp16", "bf16"])
def test_split_workspace_serves_many_calls(torch, lib, kv):
    # One workspace, filled with garbage once, through calls with different inputs, batch
    # sizes and partition counts: each must match the oracle.
    ws = torch.full((16 << 20,), 0x5A, dtype=torch.uint8, device="cuda:0")
    for i, (splits, batch) in enumerate(((2, 6), (7, 6), (3, 2), (19, 9), (2, 6))):
        cfg = SMALL.with_(kv_dtype=kv, len_hi=2000, batch=batch)
        w = generate(cfg, seed=94 + i, poison=True, extra_pages=2)
        assert workspace_for(torch, lib, w, num_splits=splits).numel() <= ws.numel()
        d = to_dev(torch, w)
        out = torch.empty(w.q.shape, dtype=torch.float32, device="cuda:0")
        print(f"case split reuse kv={kv} splits={splits}", flush=True)
        call(lib, d, w, out, ws, num_splits=splits)
        torch.cuda.synchronize()
        assert_parity(out.cpu().numpy(), oracle_run(w)[0], f"call {i} splits {splits}")


def test_library_workspace_growth_keeps_earlier_graphs_valid(torch, lib):
    # decode_attn owns its workspace and replaces it by a larger buffer when a call needs
    # more. A graph captured from an earlier, smaller call keeps the old buffer's address,
    # so that buffer must stay allocated: capture a small split-mode call, grow the
    # workspace with an eager stream-mode call over a 64/8-head batch (the largest
    # workspace the library's plans use), allocate and scribble over fresh memory, then
    # replay the small graph.
    small = SMALL.with_(len_hi=700)
    w = generate(small, seed=95)
    d = to_dev(torch, w)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    p = lib.plan(small.batch, small.max_blocks_per_seq, small.n_q_heads, small.n_kv_heads, 16,
                 "fp16", num_cus=cus)
    assert p.mode == lib.MODE_SPLIT and p.workspace_bytes > 0
    out = torch.zeros(w.q.shape, dtype=torch.float32, device="cuda:0")
    print("case workspace growth: small split call", flush=True)

    def small_call():
        lib.decode_attn(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["seq_lens"],
                        w.scale, out=out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        small_call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        small_call()
    torch.cuda.synchronize()

    # 320 (sequence, KV head) pairs of G = 2 over INT8 caches: the library plans stream mode,
    # whose piece slots need more workspace than the small call's partitions.
    big = Config(0, "int8_g2_stream", batch=40, n_q_heads=16, n_kv_heads=8, head_dim=128,
                 block_size=16, len_lo=1100, len_hi=2000, kv_dtype="int8")
    bp = lib.plan(big.batch, big.max_blocks_per_seq, big.n_q_heads, big.n_kv_heads, 16, "int8",
                  num_cus=cus)
    assert bp.mode == lib.MODE_STREAM and bp.workspace_bytes > p.workspace_bytes
    wb = generate(big, seed=96)
    db = to_dev(torch, wb)
    print("case workspace growth: large stream call", flush=True)
    big_out = lib.decode_attn(db["q"], db["k_pages"], db["v_pages"], db["block_table"],
                              db["seq_lens"], wb.scale, k_scale=db["k_scale"], v_scale=db["v_scale"])
    torch.cuda.synchronize()
    assert_parity(big_out.cpu().numpy(), oracle_run(wb)[0], "large call that grew the workspace")
    junk = torch.full((64 << 20,), 0x7F, dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()
    rng = np.random.default_rng(97)
    for replay in range(2):
        q_new = rng.standard_normal(w.q.shape).astype(np.float16)
        d["q"].copy_(dev_tensor(torch, q_new))
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        w.q = q_new
        assert_parity(out.cpu().numpy(), oracle_run(w)[0], f"small graph replay {replay} after growth")
    del junk
