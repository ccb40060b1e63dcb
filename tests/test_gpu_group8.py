"""GPU parity of the library's own plans for G = 8 (64 query heads over 8 KV heads, the
Llama-3-70B head shape) on long caches, where the plan takes split mode, in every storage
format, against the fp64 oracle: |gpu - oracle| <= 2e-3 + 1e-2 |oracle| elementwise, and
the lse to 1e-3 + 1e-4 |lse|. Every call goes through the C ABI."""

import numpy as np
import pytest

from decode_phase_attention_paged_amd.workload import Config, generate

from test_gpu_parity import assert_parity, gpu_run, oracle_run

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


@pytest.mark.parametrize("kv", ["fp16", "bf16", "int8", "fp8"])
@pytest.mark.parametrize("batch,length", [(1, 32768), (3, 5000)])
def test_group8_long_caches_library_plan(torch, lib, kv, batch, length):
    cfg = Config(0, "g8_long", batch, 64, 8, 128, 16, length // 2, length, kv)
    w = generate(cfg, seed=600 + batch, poison=True)
    print(f"case G=8 {kv} batch={batch} lens={w.seq_lens.tolist()}", flush=True)
    got, got_lse = gpu_run(torch, lib, w)
    ref, ref_lse = oracle_run(w)
    assert_parity(got, ref, f"G=8 {kv} batch {batch}")
    np.testing.assert_allclose(got_lse, ref_lse, rtol=1e-4, atol=1e-3)
