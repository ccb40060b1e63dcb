"""Host-side logic of bench.py and the build (no GPU): timing statistics, the counter
arithmetic of the profile summariser on synthetic rocprofv3 output, and the build's reading
of the compiler's resource remarks."""

import csv
import json
import os

import pytest

import bench
from decode_phase_attention_paged_amd import build


def test_window_statistics():
    stats = bench.window_stats([10.0, 12.0, 11.0, 30.0, 9.0], steps=10)
    assert stats == {"median_ms": 1.1, "min_ms": 0.9, "max_ms": 3.0}
    # At least five windows and at least 100 steps in all.
    assert bench.default_windows(400) == 5
    assert bench.default_windows(20) == 5
    assert bench.default_windows(7) == 15
    assert bench.default_windows(0) == 100


def test_read_bytes_by_request_size():
    ctr = {"TCC_EA0_RDREQ_32B_sum": [1.0, 3.0], "TCC_EA0_RDREQ_64B_sum": [10.0],
           "TCC_EA0_RDREQ_128B_sum": [100.0, 100.0]}
    assert bench.read_bytes_by_request_size(ctr) == 2 * 32 + 10 * 64 + 100 * 128
    assert bench.read_bytes_by_request_size({"TCC_EA0_RDREQ_32B_sum": [1.0]}) is None


def test_derived_counters_formulas():
    # One XCD's busy cycles are an eighth of GRBM_GUI_ACTIVE; SQ cycle counters count
    # quad-cycles summed over all waves.
    cycles = 1000.0
    ctr = {
        "GRBM_GUI_ACTIVE": [cycles * bench.N_XCD],
        "SQ_WAVE_CYCLES": [3.0 * cycles * bench.N_CU / 4],       # 3 resident waves per CU
        "SQ_ACTIVE_INST_VALU": [0.25 * cycles * bench.N_SIMD / 4],  # VALU busy a quarter
        "SQ_VALU_MFMA_BUSY_CYCLES": [0.5 * cycles * bench.N_SIMD],
        "SQ_WAIT_ANY": [0.3 * 3.0 * cycles * bench.N_CU / 4],
        "SQ_WAVES": [1024.0],
        "SQ_INSTS_VALU": [2048.0],
        "TCC_HIT_sum": [1.0], "TCC_MISS_sum": [3.0],
        "TCC_EA0_RDREQ_sum": [10.0], "TCC_EA0_RDREQ_128B_sum": [9.0],
    }
    got = dict(bench.derived_counters(ctr, 1.0))
    assert got["gpu_busy_cycles_of_the_profiled_dispatch"] == "1000"
    assert got["mean_resident_waves_per_cu"] == "3.00"
    assert got["valu_busy_fraction_per_simd"] == "0.250"
    assert got["mfma_busy_fraction_per_simd"] == "0.500"
    assert got["sq_wait_any_over_wave_cycles"] == "0.300"
    assert got["sq_insts_valu_per_wave"] == "2.0"
    assert got["l2_hit_fraction"] == "0.250"
    assert got["share_of_128_byte_read_requests"] == "0.9000"


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _pmc_rows(kernel, values):
    return [{"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": name,
             "Counter_Value": v}
            for i, per in enumerate(values) for name, v in per.items()]


def test_summarize_profile_on_synthetic_output(tmp_path, monkeypatch):
    """A fake profiled run: two launches of one kernel of 1000 ns each, reading 2 MB of
    which 1.5 MB algorithmic, writing 0.5 MB; the copy reads 1 GiB but FETCH_SIZE shows half
    of it, as on gfx950. The summary must scale the fetch by 2, name the dominant kernel and
    its timed average, and agree with the request-size cross-check."""
    d = tmp_path / "prof"
    tag = "cfgX"
    kernel = "void dattn::seg_kernel<(dattn::KvType)0, 1>(dattn::Args)"
    alg = 1_500_000
    rec = {"metric": bench.METRIC, "argv": ["--config", "2"], "steps": 2, "repeats": 1,
           "us_per_step": 1.0,
           "config": {"workload": "synthetic_case", "kv_bytes_per_step": alg, "batch": 2,
                      "n_q_heads": 4, "head_dim": 128}}
    d.mkdir()
    (d / f"trace_{tag}.json").write_text("progress line\n" + json.dumps(rec) + "\n")
    trace = [{"Kernel_Name": kernel, "Start_Timestamp": 100 * i, "End_Timestamp": 100 * i + 1000,
              "VGPR_Count": 128, "Accum_VGPR_Count": 0, "SGPR_Count": 96, "LDS_Block_Size": 0,
              "Scratch_Size": 0, "Grid_Size_X": 65536, "Workgroup_Size_X": 256}
             for i in range(2)]
    _write_csv(str(d / f"trace_{tag}" / "run_kernel_trace.csv"), trace)
    copy = "__amd_rocclr_copyBuffer"
    _write_csv(str(d / "pmc_FETCH_SIZE_copy" / "run_counter_collection.csv"),
               _pmc_rows(copy, [{"FETCH_SIZE": (1 << 30) / 1024 / 2}]))
    _write_csv(str(d / "pmc_WRITE_SIZE_copy" / "run_counter_collection.csv"),
               _pmc_rows(copy, [{"WRITE_SIZE": (1 << 30) / 1024}]))
    fetch_kib = 2_000_000 / 1024 / 2
    write_kib = 500_000 / 1024
    _write_csv(str(d / f"pmc_FETCH_SIZE_{tag}" / "run_counter_collection.csv"),
               _pmc_rows(kernel, [{"FETCH_SIZE": fetch_kib}] * 2))
    _write_csv(str(d / f"pmc_WRITE_SIZE_{tag}" / "run_counter_collection.csv"),
               _pmc_rows(kernel, [{"WRITE_SIZE": write_kib}] * 2))
    _write_csv(str(d / f"pmc_rdreq_{tag}" / "run_counter_collection.csv"),
               _pmc_rows(kernel, [{"TCC_EA0_RDREQ_32B_sum": 0.0, "TCC_EA0_RDREQ_64B_sum": 0.0,
                                   "TCC_EA0_RDREQ_128B_sum": 2_000_000 / 128,
                                   "TCC_EA0_RDREQ_sum": 2_000_000 / 128}] * 2))
    # Another workload's passes in the same directory, whose tag ends like this one's.
    _write_csv(str(d / f"pmc_FETCH_SIZE_append_{tag}" / "run_counter_collection.csv"),
               _pmc_rows("void dattn::append_kernel(dattn::AppendArgs)", [{"FETCH_SIZE": 1.0}]))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    bench.summarize_profile(str(d), tag)
    text = (tmp_path / "decode_attn_synthetic_case.txt").read_text()
    fields = {}
    for line in text.splitlines():
        if ": " in line and not line.startswith("#") and not line.startswith(" "):
            k, v = line.split(": ", 1)
            fields[k] = v
    assert "command_pmc_FETCH_SIZE_append" not in fields
    assert "command_pmc_rdreq" in fields
    assert fields["dominant_kernel"] == kernel
    assert float(fields["dominant_kernel_timed_avg_ns"]) == 1000.0
    assert float(fields["fetch_scale"]) == pytest.approx(2.0)
    assert float(fields["write_scale"]) == pytest.approx(1.0)
    assert float(fields["traffic_bytes_per_launch"]) == pytest.approx(2_500_000, rel=1e-6)
    assert float(fields["traffic_over_algorithmic"]) == pytest.approx(2_500_000 / alg, abs=1e-4)
    assert float(fields["read_bytes_by_request_size_per_launch"]) == pytest.approx(2_000_000)
    assert float(fields["read_plus_write_bytes_over_algorithmic"].split()[0]) == pytest.approx(
        2_500_000 / alg, abs=1e-4)
    qo = 2 * 4 * 128 * (2 + 4)
    assert float(fields["traffic_over_kv_plus_q_and_out"].split()[0]) == pytest.approx(
        2_500_000 / (alg + qo), abs=1e-4)
    # 1.5 MB in 1000 ns = 1500 GB/s.
    assert float(fields["achieved_gbs_at_trace_timed_avg"]) == pytest.approx(1500.0)
    assert fields["kernel_source_sha256"] == bench.kernel_source_hash(bench.SOURCES_OF_OP["attn"])


def test_source_hash_ignores_comments_only():
    code = 'int f(int x) {  // doubled\n  return 2 * x; /* no overflow\n here */\n}\n'
    same = '/* header */\nint f(int x) {\n\n  return 2 * x;   // other words\n}\n'
    other = 'int f(int x) {\n  return 3 * x;\n}\n'
    assert bench.strip_comments(code) == bench.strip_comments(same)
    assert bench.strip_comments(code) != bench.strip_comments(other)
    assert bench.strip_comments('const char* s = "a // b"; char c = \'/\';') == \
        'const char* s = "a // b"; char c = \'/\';'


def test_build_reads_scratch_from_resource_remarks():
    remarks = "\n".join([
        "kernels.hip:10:1: remark: Function Name: _Z3fooPf [-Rpass-analysis=kernel-resource-usage]",
        "kernels.hip:10:1: remark:     VGPRs: 40 [-Rpass-analysis=kernel-resource-usage]",
        "kernels.hip:10:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "kernels.hip:20:1: remark: Function Name: _Z3barPf [-Rpass-analysis=kernel-resource-usage]",
        "kernels.hip:20:1: remark:     ScratchSize [bytes/lane]: 24 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert build.scratch_use(remarks) == {"_Z3fooPf": 0, "_Z3barPf": 24}
    assert build.scratch_use("no remarks here") == {}


def test_summarize_hbm_reference_on_synthetic_output(tmp_path, monkeypatch):
    """A fake `bench.py --op hbm` run under the kernel trace: the summary groups launches
    by (kernel, grid), copies the event-timed rates and the best ones, and names the
    command and the source hash of the reference kernels."""
    d = tmp_path / "prof"
    d.mkdir()
    tag = "hbm"
    rec = {"metric": "HBM reference read rate", "argv": ["--op", "hbm", "--steps", "10"],
           "best_gather_gbs": 6700.0, "best_stream_gbs": 7100.0,
           "best_gather_frac_of_peak": 0.8375, "best_stream_frac_of_peak": 0.8875,
           "config": {"workload": "synthetic_case", "gather_bytes_per_launch": 8192,
                      "tile_pairs_per_launch": 1, "stream_bytes_per_launch": 4096},
           "gather": [{"depth": 2, "nontemporal": True, "grid": 512, "us_per_launch": 1.0,
                       "gbs": 6700.0, "gbs_min_max": [6600.0, 6750.0]}],
           "stream": [{"depth": 8, "nontemporal": False, "grid": 1024, "us_per_launch": 2.0,
                       "gbs": 7100.0, "gbs_min_max": [7000.0, 7150.0]}]}
    (d / f"trace_{tag}.json").write_text("progress\n" + json.dumps(rec) + "\n")
    gk = "void dattn::(anonymous namespace)::ref_gather_kernel<2, true>(...)"
    sk = "void dattn::(anonymous namespace)::ref_stream_kernel<8, false>(...)"
    rows = [{"Kernel_Name": gk, "Start_Timestamp": 0, "End_Timestamp": 1000, "Grid_Size_X": 512 * 256},
            {"Kernel_Name": gk, "Start_Timestamp": 0, "End_Timestamp": 3000, "Grid_Size_X": 512 * 256},
            {"Kernel_Name": gk, "Start_Timestamp": 0, "End_Timestamp": 5000, "Grid_Size_X": 256 * 256},
            {"Kernel_Name": sk, "Start_Timestamp": 0, "End_Timestamp": 2000, "Grid_Size_X": 1024 * 256},
            {"Kernel_Name": "__amd_rocclr_fillBufferAligned", "Start_Timestamp": 0,
             "End_Timestamp": 9, "Grid_Size_X": 64}]
    _write_csv(str(d / f"trace_{tag}" / "run_kernel_trace.csv"), rows)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    bench.summarize_profile(str(d), tag)
    text = (tmp_path / "hbm_reference_synthetic_case.txt").read_text()
    assert "ref_gather_kernel<2, true> grid 512: calls 2  avg_ns 2000.0" in text
    assert "ref_gather_kernel<2, true> grid 256: calls 1  avg_ns 5000.0" in text
    assert "ref_stream_kernel<8, false> grid 1024: calls 1  avg_ns 2000.0" in text
    assert "rocclr" not in text
    assert "gather depth 2 nontemporal 1 grid 512: 1.0 us  6700.0 GB/s  (windows 6600.0-6750.0)" in text
    assert "best_stream_gbs: 7100.0" in text
    assert "-- python3 $REPO/bench.py --op hbm --steps 10" in text
    assert f"kernel_source_sha256: {bench.kernel_source_hash(bench.HBM_SOURCES)}" in text


@pytest.mark.parametrize("index", [2, 3, 5, 10])
def test_reference_gather_reads_each_tile_of_a_step_once(index):
    """The reference gather's index list is exactly the set of (page, KV head) tiles one
    decode step of the workload touches: every page of every sequence's table, for every
    KV head, once."""
    import numpy as np
    from decode_phase_attention_paged_amd.workload import CONFIGS, layout
    cfg = CONFIGS[index]
    tiles, pool_tiles = bench.decode_step_tiles(cfg, np)
    lens, table, num_pages = layout(cfg)
    hkv = cfg.n_kv_heads
    assert pool_tiles == num_pages * hkv
    expect = {int(table[b, j]) * hkv + g for b in range(cfg.batch)
              for j in range(-(-int(lens[b]) // cfg.block_size)) for g in range(hkv)}
    assert tiles.dtype == np.int32 and len(tiles) == len(expect)
    assert set(tiles.tolist()) == expect
    assert tiles.min() >= 0 and tiles.max() < pool_tiles
    # the workloads use every page of their pool
    assert len(expect) == pool_tiles
