"""decode_attn_noalloc: the entry point for callers that cannot allocate.

It runs decode_attn_ex's kernels with the library's static per-device scratch array as
the workspace. Two calls in a row through the C ABI, the second with a smaller input, must
each give decode_attn_ex's bits under the same plan request (and so match the fp64
oracle within the decode-attention tolerance), whatever the previous call left in the
shared array.
"""

import numpy as np
import pytest

from decode_phase_attention_paged_amd.workload import Config, generate

from test_gpu_parity import assert_lse, assert_parity, oracle_run, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need an MI355X"
    return t


@pytest.fixture(scope="module")
def lib(torch):
    from decode_phase_attention_paged_amd import binding
    return binding


LONG = Config(0, "noalloc_long", batch=2, n_q_heads=32, n_kv_heads=8, head_dim=128,
              block_size=16, len_lo=9000, len_hi=20000, kv_dtype="fp16")
SHORT = Config(0, "noalloc_short", batch=3, n_q_heads=8, n_kv_heads=2, head_dim=128,
               block_size=16, len_lo=1, len_hi=700, kv_dtype="fp16")

# (config, plan request): the first call of each pair leaves a larger workspace behind
# than the second one needs.
PAIRS = [
    ((LONG, dict(num_splits=24)), (SHORT, dict(num_splits=5))),          # split, split
    ((LONG.with_(kv_dtype="int8"), dict(num_workgroups=40)),              # stream, stream
     (SHORT.with_(kv_dtype="int8"), dict(num_workgroups=3))),
    ((LONG, dict()), (SHORT.with_(batch=2), dict())),                     # the library's plans
]


def run_both(torch, lib, w, plan):
    d = to_dev(torch, w)
    shape = w.q.shape
    out_ex = torch.full(shape, np.nan, dtype=torch.float32, device="cuda:0")
    lse_ex = torch.full(shape[:2], np.nan, dtype=torch.float32, device="cuda:0")
    lib.decode_attn_ex(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["seq_lens"],
                       w.scale, k_scale=d["k_scale"], v_scale=d["v_scale"], out=out_ex,
                       lse_out=lse_ex, **plan)
    out_na = torch.full(shape, np.nan, dtype=torch.float32, device="cuda:0")
    lse_na = torch.full(shape[:2], np.nan, dtype=torch.float32, device="cuda:0")
    lib.decode_attn_noalloc(d["q"], d["k_pages"], d["v_pages"], d["block_table"],
                            d["seq_lens"], w.scale, k_scale=d["k_scale"], v_scale=d["v_scale"],
                            out=out_na, lse_out=lse_na, **plan)
    torch.cuda.synchronize()
    return (out_ex.cpu().numpy(), lse_ex.cpu().numpy(), out_na.cpu().numpy(),
            lse_na.cpu().numpy())


@pytest.mark.parametrize("pair", range(len(PAIRS)), ids=["split", "stream", "auto"])
def test_noalloc_matches_ex_on_two_calls_second_smaller(torch, lib, pair):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    needs = []
    for step, (cfg, plan) in enumerate(PAIRS[pair]):
        p = lib.plan(cfg.batch, cfg.max_blocks_per_seq, cfg.n_q_heads, cfg.n_kv_heads, 16,
                     cfg.kv_dtype, num_cus=cus, **plan)
        assert 0 < p.workspace_bytes <= lib.STATIC_SCRATCH_BYTES
        needs.append(p.workspace_bytes)
        w = generate(cfg, seed=200 + 10 * pair + step, poison=True, extra_pages=3)
        print(f"case noalloc pair={pair} call={step} {cfg.name} {cfg.kv_dtype} plan={plan} "
              f"workspace={p.workspace_bytes}", flush=True)
        out_ex, lse_ex, out_na, lse_na = run_both(torch, lib, w, plan)
        assert np.array_equal(out_na, out_ex, equal_nan=True), f"call {step}: out differs from decode_attn_ex"
        assert np.array_equal(lse_na, lse_ex, equal_nan=True), f"call {step}: lse differs from decode_attn_ex"
        ref, ref_lse = oracle_run(w)
        assert_parity(out_na, ref, f"noalloc pair {pair} call {step}")
        assert_lse(lse_na, ref_lse, f"noalloc pair {pair} call {step} lse")
    assert needs[1] < needs[0]


def test_noalloc_refuses_plans_beyond_its_scratch(torch, lib):
    cfg = SHORT
    w = generate(cfg, seed=230)
    d = to_dev(torch, w)
    p = lib.plan(cfg.batch, cfg.max_blocks_per_seq, cfg.n_q_heads, cfg.n_kv_heads, 16, "fp16",
                 num_workgroups=20000)
    assert p.workspace_bytes > lib.STATIC_SCRATCH_BYTES
    out = torch.zeros(w.q.shape, dtype=torch.float32, device="cuda:0")
    with pytest.raises(lib.DecodeAttnError) as err:
        lib.decode_attn_noalloc(d["q"], d["k_pages"], d["v_pages"], d["block_table"],
                                d["seq_lens"], w.scale, out=out, num_workgroups=20000)
    assert err.value.status == 5
    torch.cuda.synchronize()
    assert not out.cpu().numpy().any(), "a refused call must not write"
