"""The C ABI on the host: the library loads, exports what include/decode_attn.h
declares, plans deterministically, and rejects bad arguments before any HIP call
(no GPU needed)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decode_attn.h")


@pytest.fixture(scope="module")
def binding():
    from decode_phase_attention_paged_amd import binding as b
    if not os.path.exists(b.LIB_PATH):
        from decode_phase_attention_paged_amd import build
        build.build(verbose=False)
    return b


@pytest.fixture(scope="module")
def lib(binding):
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w\s\*]*?\b(decode_attn\w*)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "decode_attn", "decode_attn_append", "decode_attn_ex", "decode_attn_hbm_reference",
        "decode_attn_noalloc", "decode_attn_plan", "decode_attn_prefill",
        "decode_attn_status_string", "decode_attn_version"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_plan_struct_matches_the_header(binding):
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} decode_attn_plan_t;", text, re.S).group(1)
    fields = re.findall(r"^\s*(int|size_t)\s+(\w+);", body, flags=re.M)
    assert [name for _, name in fields] == [f[0] for f in binding.Plan._fields_]


def test_version_and_status_strings(lib):
    assert lib.decode_attn_version() >> 16 == 6 and lib.decode_attn_version() & 0xFFFF >= 4
    names = [lib.decode_attn_status_string(i).decode() for i in range(6)]
    assert names == ["DECODE_ATTN_OK", "DECODE_ATTN_ERR_INVALID_ARGUMENT",
                     "DECODE_ATTN_ERR_UNSUPPORTED", "DECODE_ATTN_ERR_WORKSPACE",
                     "DECODE_ATTN_ERR_HIP", "DECODE_ATTN_ERR_SCRATCH_LIMIT"]
    assert lib.decode_attn_status_string(99) == b"DECODE_ATTN_UNKNOWN_STATUS"


# Fake device addresses: never dereferenced, because every case below fails host-side
# validation (or enqueues nothing) before the first HIP call.
A = 1 << 20
GOOD = dict(q=A, k=2 * A, v=3 * A, ks=None, vs=None, bt=4 * A, sl=5 * A, batch=2, mb=8,
            np_=16, hq=8, hkv=2, d=128, bs=16, kv=0, scale=0.088, out=6 * A)


def call(lib, **over):
    a = dict(GOOD, **over)
    return lib.decode_attn(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"], a["sl"], a["batch"],
                           a["mb"], a["np_"], a["hq"], a["hkv"], a["d"], a["bs"], a["kv"],
                           a["scale"], a["out"], None)


def call_ex(lib, wgs, splits, ws, ws_bytes, **over):
    a = dict(GOOD, **over)
    return lib.decode_attn_ex(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"], a["sl"],
                              a["batch"], a["mb"], a["np_"], a["hq"], a["hkv"], a["d"], a["bs"],
                              a["kv"], a["scale"], a["out"], None, wgs, splits, ws, ws_bytes, None)


@pytest.mark.parametrize("over,status", [
    (dict(hq=6, hkv=4), 1),            # Hq % Hkv != 0
    (dict(d=64), 2),                   # head_dim other than 128
    (dict(bs=32), 2),                  # block_size other than 16
    (dict(hq=6, hkv=2), 2),            # G = 3
    (dict(hq=32, hkv=2), 2),           # G = 16
    (dict(kv=1), 1),                   # int8 without row scales
    (dict(ks=7 * A, vs=8 * A), 1),     # fp16 with row scales
    (dict(kv=1, ks=7 * A), 1),         # int8 with only one scale array
    (dict(kv=3), 1),                   # fp8 without row scales
    (dict(kv=3, vs=8 * A), 1),         # fp8 with only one scale array
    (dict(kv=2, ks=7 * A, vs=8 * A), 1),   # bf16 with row scales
    (dict(kv=5), 1),                   # unknown storage type
    (dict(kv=-1), 1),
    (dict(q=None), 1),
    (dict(out=None), 1),
    (dict(bt=None), 1),
    (dict(q=A + 8), 1),                # q not 16-byte aligned
    (dict(k=2 * A + 4), 1),            # pages not 16-byte aligned
    (dict(out=6 * A + 4), 1),          # out not 16-byte aligned
    (dict(kv=1, ks=7 * A + 4, vs=8 * A), 1),   # int8 row scales not 8-byte aligned
    (dict(mb=1 << 20, hkv=4096, hq=4096), 2),  # unit count beyond 32 bits
    (dict(batch=-1), 1),
    (dict(mb=0), 1),
    (dict(np_=0), 1),
    (dict(hkv=0), 1),
    (dict(batch=0, q=None, k=None, v=None, bt=None, sl=None, out=None), 0),  # empty batch
])
def test_host_validation(lib, over, status):
    assert call(lib, **over) == status


def plan(lib, binding, batch, mb, hq, hkv, wgs=0, splits=0, cus=256, kv=0):
    p = binding.Plan()
    st = lib.decode_attn_plan(batch, mb, hq, hkv, 16, kv, wgs, splits, cus, ctypes.byref(p))
    assert st == 0, st
    return p


def test_explicit_plans_need_no_device_and_check_the_workspace(lib, binding):
    # Stream mode on 4 workgroups: 16 workers x 2 piece slots x G heads of 129 floats, plus
    # a 16-byte record per worker, each array 256-byte aligned.
    p = plan(lib, binding, 2, 8, 8, 2, wgs=4)
    rows = 16 * 2 * 4
    assert p.mode == binding.MODE_STREAM and p.num_workgroups == 4
    assert p.workspace_bytes == rows * 128 * 4 + 512 + 256
    need = p.workspace_bytes
    assert call_ex(lib, 4, 0, None, 0) == 3
    assert call_ex(lib, 4, 0, 9 * A, need - 1) == 3
    assert call_ex(lib, 4, 0, 9 * A + 16, need) == 3   # not 256-byte aligned
    assert call_ex(lib, -1, 0, None, 0) == 1
    assert call_ex(lib, 4, 3, None, 0) == 1            # a grid with several partitions
    assert call_ex(lib, 4, 0, 9 * A, need, hq=6, hkv=4) == 1
    # Split mode with 3 partitions of 3 pages: partial rows B x Hq x S.
    s = plan(lib, binding, 2, 8, 8, 2, splits=3)
    assert (s.mode, s.num_splits, s.pages_per_split, s.num_workgroups) == (
        binding.MODE_SPLIT, 3, 3, 3 * 2 * 2)
    assert s.workspace_bytes == 2 * 8 * 3 * 128 * 4 + 256
    assert call_ex(lib, 0, 3, 9 * A, s.workspace_bytes - 1) == 3
    # Segment mode on an explicit grid: no workspace, any grid size.
    g = plan(lib, binding, 2, 8, 8, 2, wgs=7, splits=1)
    assert (g.mode, g.num_workgroups, g.num_splits, g.pages_per_split, g.workspace_bytes) == (
        binding.MODE_SEGMENT, 7, 1, 0, 0)


def call_noalloc(lib, wgs, splits, **over):
    a = dict(GOOD, **over)
    return lib.decode_attn_noalloc(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"], a["sl"],
                                   a["batch"], a["mb"], a["np_"], a["hq"], a["hkv"], a["d"],
                                   a["bs"], a["kv"], a["scale"], a["out"], None, wgs, splits,
                                   None)


def test_noalloc_checks_arguments_and_its_scratch_limit_before_any_hip_call(lib, binding):
    # Stream mode on 20000 workgroups needs 80000 workers x 2 slots x G = 4 rows of 129
    # floats, far beyond the 32 MiB static scratch array; 4 workgroups fit.
    assert binding.STATIC_SCRATCH_BYTES == 32 << 20
    assert plan(lib, binding, 2, 8, 8, 2, wgs=20000).workspace_bytes > binding.STATIC_SCRATCH_BYTES
    assert plan(lib, binding, 2, 8, 8, 2, wgs=4).workspace_bytes < binding.STATIC_SCRATCH_BYTES
    assert call_noalloc(lib, 20000, 0) == 5
    assert call_noalloc(lib, 20000, 0, hq=6, hkv=4) == 1     # arguments are checked first
    assert call_noalloc(lib, 4, 3) == 1                      # a grid with several partitions
    assert call_noalloc(lib, 4, 0, d=64) == 2
    assert call_noalloc(lib, 4, 0, batch=0, q=None, k=None, v=None, bt=None, sl=None,
                        out=None) == 0                       # empty batch: nothing enqueued


def test_stream_mode_refuses_batches_beyond_the_lds_scan(lib, binding):
    p = binding.Plan()
    assert lib.decode_attn_plan(4097, 4, 8, 8, 16, 0, 8, 0, 0, ctypes.byref(p)) == 2
    auto = plan(lib, binding, 4097, 4, 8, 8)
    assert auto.mode == binding.MODE_SEGMENT
    assert plan(lib, binding, 4097, 100, 8, 8, kv=1).mode == binding.MODE_SEGMENT


def test_split_requests_round_to_whole_partitions(lib, binding):
    got = lambda req: (plan(lib, binding, 1, 16, 8, 8, splits=req).num_splits,
                       plan(lib, binding, 1, 16, 8, 8, splits=req).pages_per_split)
    assert got(1) == (1, 0)       # one partition is segment mode
    assert plan(lib, binding, 1, 16, 8, 8, splits=1).mode == binding.MODE_SEGMENT
    assert plan(lib, binding, 1, 1, 8, 8, splits=4).mode == binding.MODE_SEGMENT
    assert got(3) == (3, 6)
    assert got(7) == (6, 3)       # ceil(16 / ceil(16 / 7))
    assert got(100) == (16, 1)
    for mb in (1, 2, 15, 36, 256, 8192):
        for req in (1, 2, 3, 5, 64):
            p = plan(lib, binding, 3, mb, 8, 4, splits=req)
            if p.mode == binding.MODE_SEGMENT:
                assert p.num_splits == 1 and (req == 1 or mb == 1)
                continue
            assert p.num_splits * p.pages_per_split >= mb
            assert (p.num_splits - 1) * p.pages_per_split < mb


def test_auto_plan_for_the_preset_shapes(lib, binding):
    # (batch, MB, Hq, Hkv) of the preset workloads on a 256-CU device.
    p1 = plan(lib, binding, 1, 16, 8, 8)
    p2 = plan(lib, binding, 48, 36, 32, 32)
    p3 = plan(lib, binding, 160, 256, 32, 8)
    p4 = plan(lib, binding, 1, 8192, 32, 8)
    p5 = plan(lib, binding, 200, 34, 32, 32, kv=1)
    # Many (sequence, head) pairs over short caches: segment mode, one workgroup per
    # compute unit for 16-bit caches with G = 1 and three for INT8 (the workgroups resident
    # at each build's occupancy), no workspace.
    assert (p2.mode, p2.num_splits, p2.num_workgroups) == (binding.MODE_SEGMENT, 1, 256)
    assert (p5.mode, p5.num_splits, p5.num_workgroups) == (binding.MODE_SEGMENT, 1, 768)
    assert p2.workspace_bytes == 0 and p5.workspace_bytes == 0
    # Never more workgroups than segments; every format takes segment mode for many short
    # caches, G = 8 included.
    assert plan(lib, binding, 3, 8, 1, 1, cus=4).num_workgroups == 3
    assert plan(lib, binding, 3, 8, 8, 8, cus=30).num_workgroups == 24
    assert plan(lib, binding, 3, 8, 8, 8, cus=20).num_workgroups == 20
    assert plan(lib, binding, 300, 8, 8, 1, cus=2).mode == binding.MODE_SEGMENT
    assert plan(lib, binding, 300, 8, 8, 1, cus=2, kv=1).mode == binding.MODE_SEGMENT
    assert plan(lib, binding, 300, 8, 8, 1, cus=2, kv=3).mode == binding.MODE_SEGMENT
    assert plan(lib, binding, 300, 8, 8, 4, cus=2).mode == binding.MODE_SEGMENT
    # Many pairs over long caches: segment mode while every workgroup gets two segments or
    # more (1280 pairs, 256 workgroups for G = 4); between one and two pairs per CU the
    # 1-byte vector-ALU builds (G <= 2) take the balanced stream, every other build keeps
    # segment mode.
    assert p3.mode == binding.MODE_SEGMENT and p3.num_workgroups == 256
    s3 = plan(lib, binding, 10, 256, 32, 32, kv=1)
    assert s3.mode == binding.MODE_STREAM and s3.num_workgroups == 512
    assert plan(lib, binding, 10, 256, 32, 32, kv=3).mode == binding.MODE_STREAM
    assert plan(lib, binding, 10, 256, 32, 32).mode == binding.MODE_SEGMENT        # fp16, G = 1
    assert plan(lib, binding, 10, 256, 32, 32, kv=2).mode == binding.MODE_SEGMENT  # BF16, G = 1
    m3 = plan(lib, binding, 60, 256, 32, 8)
    assert (m3.mode, m3.num_workgroups) == (binding.MODE_SEGMENT, 256)
    assert plan(lib, binding, 40, 256, 64, 8, kv=3).mode == binding.MODE_SEGMENT  # FP8, G = 8
    assert plan(lib, binding, 60, 256, 32, 8, kv=2).mode == binding.MODE_SEGMENT  # BF16, G = 4
    # Fewer pairs than CUs over long caches: partitions for about one workgroup per CU,
    # rounded; more than half as many pairs as CUs is segment mode.
    assert plan(lib, binding, 24, 256, 32, 8).mode == binding.MODE_SEGMENT          # 192 pairs
    p96 = plan(lib, binding, 12, 256, 32, 8)
    assert (p96.mode, p96.num_splits) == (binding.MODE_SPLIT, 3)                     # 96 pairs
    p32 = plan(lib, binding, 4, 256, 32, 8)
    assert (p32.mode, p32.num_splits) == (binding.MODE_SPLIT, 8)                     # 32 pairs
    # 64 x 8 pairs of G = 8 over 256-page INT8 caches (two pairs per CU): segment mode, with
    # the grid cut from the two workgroups per CU the build keeps resident to one, so that
    # each workgroup still gets two segments; 160 x 8 INT8 pairs keep both.
    p10 = plan(lib, binding, 64, 256, 64, 8, kv=1)
    assert (p10.mode, p10.num_workgroups) == (binding.MODE_SEGMENT, 256)
    p11 = plan(lib, binding, 160, 256, 32, 8, kv=1)
    assert (p11.mode, p11.num_workgroups) == (binding.MODE_SEGMENT, 512)
    # Few long caches: split mode, about one workgroup per CU.
    assert (p4.mode, p4.num_splits, p4.pages_per_split, p4.num_workgroups) == (
        binding.MODE_SPLIT, 32, 256, 256)
    # Few pairs over caches of at most 16 pages: segment mode (one workgroup per pair);
    # longer caches: split mode.
    assert (p1.mode, p1.num_workgroups) == (binding.MODE_SEGMENT, 8)
    assert plan(lib, binding, 1, 1, 8, 8).mode == binding.MODE_SEGMENT
    p17 = plan(lib, binding, 1, 17, 8, 8)
    assert p17.mode == binding.MODE_SPLIT and p17.num_splits == 17
    assert plan(lib, binding, 160, 256, 32, 8, cus=80).num_workgroups == 80


def test_plan_rejects_bad_arguments(lib, binding):
    p = binding.Plan()
    assert lib.decode_attn_plan(1, 0, 8, 8, 16, 0, 0, 0, 256, ctypes.byref(p)) == 1
    assert lib.decode_attn_plan(1, 8, 8, 8, 16, 0, -2, 0, 256, ctypes.byref(p)) == 1
    assert lib.decode_attn_plan(1, 8, 8, 8, 16, 0, 2, 2, 256, ctypes.byref(p)) == 1
    assert lib.decode_attn_plan(1, 8, 6, 4, 16, 0, 0, 0, 256, ctypes.byref(p)) == 1
    assert lib.decode_attn_plan(1, 8, 8, 8, 16, 4, 0, 0, 256, ctypes.byref(p)) == 1   # kv type
    assert lib.decode_attn_plan(1, 8, 8, 8, 16, 0, 0, 0, 256, None) == 1


def test_binding_plan_helper_matches_the_c_call(lib, binding):
    # The Python helper forwards every argument in the C order.
    p = binding.plan(200, 34, 32, 32, 16, kv_dtype="int8", num_workgroups=0, num_splits=0,
                     num_cus=256)
    q = plan(lib, binding, 200, 34, 32, 32, kv=1)
    assert (p.mode, p.num_workgroups, p.num_splits, p.workspace_bytes) == (
        q.mode, q.num_workgroups, q.num_splits, q.workspace_bytes)
    s = binding.plan(3, 8, 8, 2, num_workgroups=5, num_splits=1, num_cus=256)
    assert (s.mode, s.num_workgroups) == (binding.MODE_SEGMENT, 5)
    t = binding.plan(3, 8, 8, 2, num_workgroups=5, num_cus=256)
    assert (t.mode, t.num_workgroups) == (binding.MODE_STREAM, 5)


# decode_attn_append: fake device addresses again; every case fails host-side validation
# (or enqueues nothing) before the first HIP call.
APPEND = dict(k=A, v=2 * A, bt=3 * A, pos=4 * A, batch=2, mb=8, np_=16, hkv=2, d=128, bs=16,
              kv=0, kp=5 * A, vp=6 * A, ks=None, vs=None)


def call_append(lib, **over):
    a = dict(APPEND, **over)
    return lib.decode_attn_append(a["k"], a["v"], a["bt"], a["pos"], a["batch"], a["mb"],
                                  a["np_"], a["hkv"], a["d"], a["bs"], a["kv"], a["kp"],
                                  a["vp"], a["ks"], a["vs"], None)


@pytest.mark.parametrize("over,status", [
    (dict(kv=1), 1),                         # int8 without row scales
    (dict(ks=7 * A, vs=8 * A), 1),           # fp16 with row scales
    (dict(kv=3), 1),                         # fp8 without row scales
    (dict(kv=2, ks=7 * A, vs=8 * A), 1),     # bf16 with row scales
    (dict(kv=4), 1),                         # unknown storage type
    (dict(k=None), 1),
    (dict(kp=None), 1),
    (dict(pos=None), 1),
    (dict(k=A + 8), 1),                      # new rows not 16-byte aligned
    (dict(kp=5 * A + 4), 1),                 # pools not 16-byte aligned
    (dict(kv=1, ks=7 * A + 2, vs=8 * A), 1), # scales not 4-byte aligned
    (dict(batch=-1), 1),
    (dict(mb=0), 1),
    (dict(np_=0), 1),
    (dict(hkv=0), 1),
    (dict(d=64), 2),
    (dict(bs=8), 2),
    (dict(batch=1 << 20, hkv=4096), 2),      # batch * Hkv beyond 31 bits
    (dict(batch=0, k=None, v=None, bt=None, pos=None, kp=None, vp=None), 0),
])
def test_append_host_validation(lib, over, status):
    assert call_append(lib, **over) == status


# decode_attn_prefill: fake device addresses; every case fails host-side validation (or
# enqueues nothing).
PREFILL = dict(q=A, qs=2 * A, k=3 * A, v=4 * A, ks=None, vs=None, bt=5 * A, sl=6 * A, batch=2,
               total=10, mb=8, np_=16, hq=8, hkv=2, d=128, bs=16, kv=0, chunk=8, scale=0.088,
               out=7 * A)


def call_prefill(lib, **over):
    a = dict(PREFILL, **over)
    return lib.decode_attn_prefill(a["q"], a["qs"], a["k"], a["v"], a["ks"], a["vs"], a["bt"],
                                   a["sl"], a["batch"], a["total"], a["mb"], a["np_"], a["hq"],
                                   a["hkv"], a["d"], a["bs"], a["kv"], a["chunk"], a["scale"],
                                   a["out"], None)


@pytest.mark.parametrize("over,status", [
    (dict(hq=6, hkv=4), 1),                  # Hq % Hkv != 0
    (dict(hq=6, hkv=2), 2),                  # G = 3
    (dict(kv=1), 1),                         # int8 pools without row scales
    (dict(kv=3, ks=8 * A), 1),               # fp8 with only one of the two scale arrays
    (dict(kv=2, ks=8 * A, vs=9 * A), 1),     # bf16 pools with row scales
    (dict(kv=0, vs=9 * A), 1),               # fp16 pools with a row scale
    (dict(kv=1, ks=8 * A + 2, vs=9 * A), 1), # row scales not 4-byte aligned
    (dict(kv=7), 1),                         # unknown storage type
    (dict(d=64), 2),
    (dict(bs=8), 2),
    (dict(chunk=0), 1),
    (dict(total=-1), 1),
    (dict(qs=None), 1),
    (dict(q=None), 1),
    (dict(out=None), 1),
    (dict(q=A + 8), 1),                      # q not 16-byte aligned
    (dict(out=7 * A + 4), 1),
    (dict(batch=1 << 23), 2),                # batch x Hkv = 2^24: beyond the grid
    (dict(batch=-1), 1),
    (dict(batch=0, q=None, qs=None, k=None, v=None, bt=None, sl=None, out=None), 0),
    (dict(total=0, q=None, out=None, batch=0), 0),
])
def test_prefill_host_validation(lib, over, status):
    assert call_prefill(lib, **over) == status


def call_hbm(lib, **over):
    a = dict(kind=1, depth=2, nt=1, a=A, b=2 * A, asc=5 * A, bsc=6 * A, tiles=3 * A,
             count=100, num_tiles=64, grid=8, sink=4 * A)
    a.update(over)
    return lib.decode_attn_hbm_reference(a["kind"], a["depth"], a["nt"], a["a"], a["b"],
                                         a["asc"], a["bsc"], a["tiles"], a["count"],
                                         a["num_tiles"], a["grid"], a["sink"], None)


@pytest.mark.parametrize("over", [
    dict(kind=3), dict(kind=-1), dict(depth=3), dict(depth=8), dict(kind=0, depth=2),
    dict(kind=0, depth=1), dict(kind=2, depth=16), dict(nt=2), dict(grid=0),
    dict(grid=65536), dict(count=-1), dict(num_tiles=-1), dict(a=None), dict(sink=None),
    dict(a=A + 4), dict(b=None), dict(tiles=None), dict(b=2 * A + 8), dict(tiles=3 * A + 2),
    dict(kind=2, asc=None), dict(kind=2, bsc=None), dict(kind=2, asc=5 * A + 32),
    dict(kind=2, bsc=6 * A + 16),
])
def test_hbm_reference_rejects_bad_arguments(lib, over):
    assert call_hbm(lib, **over) == 1     # DECODE_ATTN_ERR_INVALID_ARGUMENT


def test_hbm_reference_empty_enqueues_nothing(lib):
    # count 0 returns before any HIP call; a streaming read needs neither b nor tiles
    assert call_hbm(lib, count=0) == 0
    assert call_hbm(lib, kind=2, count=0) == 0
    # a streaming read needs neither b, tiles nor scales; a 4 KiB gather no scales
    assert call_hbm(lib, kind=0, depth=8, b=None, tiles=None, asc=None, bsc=None, count=0) == 0
    assert call_hbm(lib, kind=1, asc=None, bsc=None, count=0) == 0
