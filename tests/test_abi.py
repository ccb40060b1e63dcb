"""The C ABI on the host: the library loads, exports what include/decode_attn.h
declares, and rejects bad arguments before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decode_attn.h")


@pytest.fixture(scope="module")
def lib():
    from decode_phase_attention_paged_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from decode_phase_attention_paged_amd import build
        build.build(verbose=False)
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w\s\*]*?\b(decode_attn\w*)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "decode_attn", "decode_attn_ex", "decode_attn_plan", "decode_attn_workspace_size",
        "decode_attn_status_string", "decode_attn_version"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.decode_attn_version() >> 16 == 1
    names = [lib.decode_attn_status_string(i).decode() for i in range(5)]
    assert names == ["DECODE_ATTN_OK", "DECODE_ATTN_ERR_INVALID_ARGUMENT",
                     "DECODE_ATTN_ERR_UNSUPPORTED", "DECODE_ATTN_ERR_WORKSPACE",
                     "DECODE_ATTN_ERR_HIP"]
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


def call_ex(lib, splits, ws, ws_bytes, **over):
    a = dict(GOOD, **over)
    return lib.decode_attn_ex(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"], a["sl"],
                              a["batch"], a["mb"], a["np_"], a["hq"], a["hkv"], a["d"], a["bs"],
                              a["kv"], a["scale"], a["out"], None, splits, ws, ws_bytes, None)


@pytest.mark.parametrize("over,status", [
    (dict(hq=6, hkv=4), 1),            # Hq % Hkv != 0
    (dict(d=64), 2),                   # head_dim other than 128
    (dict(bs=32), 2),                  # block_size other than 16
    (dict(hq=6, hkv=2), 2),            # G = 3
    (dict(hq=32, hkv=2), 2),           # G = 16
    (dict(kv=1), 1),                   # int8 without row scales
    (dict(ks=7 * A, vs=8 * A), 1),     # fp16 with row scales
    (dict(kv=1, ks=7 * A), 1),         # int8 with only one scale array
    (dict(kv=5), 1),                   # unknown storage type
    (dict(q=None), 1),
    (dict(out=None), 1),
    (dict(bt=None), 1),
    (dict(q=A + 8), 1),                # q not 16-byte aligned
    (dict(k=2 * A + 4), 1),            # pages not 16-byte aligned
    (dict(batch=-1), 1),
    (dict(mb=0), 1),
    (dict(np_=0), 1),
    (dict(hkv=0), 1),
    (dict(batch=0, q=None, k=None, v=None, bt=None, sl=None, out=None), 0),  # empty batch
])
def test_host_validation(lib, over, status):
    assert call(lib, **over) == status


def test_explicit_workspace_checks(lib):
    # An explicit split request needs no device query; a missing or short workspace is
    # refused before anything is enqueued.
    need = lib.decode_attn_workspace_size(2, 8, 128, 4)
    assert need == 2 * 8 * 4 * 128 * 4 + 256
    assert call_ex(lib, 4, None, 0) == 3
    assert call_ex(lib, 4, 9 * A, need - 1) == 3
    assert call_ex(lib, 4, 9 * A + 16, need) == 3   # not 256-byte aligned
    assert call_ex(lib, -1, None, 0) == 1
    assert call_ex(lib, 4, 9 * A, need, hq=6, hkv=4) == 1


def plan(lib, batch, mb, hkv, requested=0, cus=256):
    s, p = ctypes.c_int(0), ctypes.c_int(0)
    assert lib.decode_attn_plan(batch, mb, hkv, 16, requested, cus, ctypes.byref(s),
                                ctypes.byref(p)) == 0
    return s.value, p.value


def test_plan_explicit_requests(lib):
    assert plan(lib, 1, 16, 8, requested=1) == (1, 16)
    assert plan(lib, 1, 16, 8, requested=3) == (3, 6)
    assert plan(lib, 1, 16, 8, requested=7) == (6, 3)      # ceil(16 / ceil(16 / 7))
    assert plan(lib, 1, 16, 8, requested=100) == (16, 1)
    assert plan(lib, 1, 8192, 8, requested=256) == (256, 32)


def test_plan_covers_every_page_once(lib):
    for mb in (1, 2, 15, 36, 256, 8192):
        for req in (0, 1, 2, 3, 5, 64):
            s, p = plan(lib, 3, mb, 4, requested=req)
            assert s * p >= mb and (s - 1) * p < mb and s >= 1


def test_plan_auto_for_the_preset_shapes(lib):
    # (batch, MB, Hkv) of the five preset workloads on a 256-CU device.
    shapes = {1: (1, 16, 8), 2: (48, 36, 32), 3: (160, 256, 8), 4: (1, 8192, 8), 5: (200, 34, 32)}
    got = {k: plan(lib, *v) for k, v in shapes.items()}
    assert got[2][0] == 1 and got[5][0] == 1          # batch x heads fills the GPU
    assert got[4][0] > 1 and got[3][0] > 1            # long caches are split
    for k, (b, mb, hkv) in shapes.items():
        s, p = got[k]
        assert p <= 64 or s == mb


def test_plan_rejects_bad_arguments(lib):
    s, p = ctypes.c_int(0), ctypes.c_int(0)
    assert lib.decode_attn_plan(1, 0, 8, 16, 0, 256, ctypes.byref(s), ctypes.byref(p)) == 1
    assert lib.decode_attn_plan(1, 8, 8, 16, -2, 256, ctypes.byref(s), ctypes.byref(p)) == 1
    assert lib.decode_attn_plan(1, 8, 8, 16, 0, 256, None, ctypes.byref(p)) == 1


def test_workspace_size_is_zero_without_splits(lib):
    assert lib.decode_attn_workspace_size(4, 32, 128, 1) == 0
    assert lib.decode_attn_workspace_size(4, 32, 128, 0) == 0
    assert lib.decode_attn_workspace_size(0, 32, 128, 8) == 0
