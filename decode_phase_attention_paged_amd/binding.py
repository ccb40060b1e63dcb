"""ctypes binding over the C ABI in include/decode_attn.h.

Argument marshalling only: torch tensors supply device pointers and the current
HIP stream; every step of the computation runs in the HIP library. There is no
fallback of any kind: if the library is missing or a call fails, this module
raises.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch has already mapped (both carry the soname
libamdhip64.so.7), and torch's stream handles are valid inside it.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdecode_attn.so")

KV_FP16 = 0
KV_INT8 = 1
KV_BF16 = 2
KV_FP8 = 3
KV_NAMES = {KV_FP16: "fp16", KV_INT8: "int8", KV_BF16: "bf16", KV_FP8: "fp8"}
_KV_CODES = {v: k for k, v in KV_NAMES.items()}
# Pool element type -> storage format; INT8 and FP8 rows carry fp32 scales.
_KV_OF_DTYPE = {torch.float16: KV_FP16, torch.int8: KV_INT8, torch.bfloat16: KV_BF16,
                torch.float8_e4m3fn: KV_FP8}
_SCALED = (KV_INT8, KV_FP8)


def _pool_format(k_pages, k_scale, v_scale):
    """Storage format of the pools, with the scale checks that go with it."""
    kv = _KV_OF_DTYPE.get(k_pages.dtype)
    if kv is None:
        raise ValueError("k_pages must be fp16, bf16, int8 or float8_e4m3fn")
    if kv in _SCALED:
        if k_scale is None or v_scale is None:
            raise ValueError(f"{KV_NAMES[kv]} caches need k_scale and v_scale")
        for t in (k_scale, v_scale):
            if t.dtype != torch.float32 or tuple(t.shape) != tuple(k_pages.shape[:3]):
                raise ValueError("row scales must be fp32 [num_pages, n_kv_heads, block_size]")
    elif k_scale is not None or v_scale is not None:
        raise ValueError("row scales are only for int8 and fp8 caches")
    return kv


def _row_dtype(kv):
    """Type of q and of new K/V rows for a storage format: bf16 for a bf16 cache, else fp16."""
    return torch.bfloat16 if kv == KV_BF16 else torch.float16
STATUS = {0: "DECODE_ATTN_OK", 1: "DECODE_ATTN_ERR_INVALID_ARGUMENT",
          2: "DECODE_ATTN_ERR_UNSUPPORTED", 3: "DECODE_ATTN_ERR_WORKSPACE",
          4: "DECODE_ATTN_ERR_HIP", 5: "DECODE_ATTN_ERR_SCRATCH_LIMIT"}
STATIC_SCRATCH_BYTES = 32 << 20   # DECODE_ATTN_STATIC_SCRATCH_BYTES

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t

MODE_STREAM = 0
MODE_SPLIT = 1
MODE_SEGMENT = 2
_MODE_NAMES = {MODE_STREAM: "stream", MODE_SPLIT: "split", MODE_SEGMENT: "segment"}


class Plan(ctypes.Structure):
    """Mirror of decode_attn_plan_t."""
    _fields_ = [("mode", _I), ("num_workgroups", _I), ("num_splits", _I),
                ("pages_per_split", _I), ("workspace_bytes", _SZ)]

    def __repr__(self):
        mode = _MODE_NAMES.get(self.mode, str(self.mode))
        return (f"Plan(mode={mode}, num_workgroups={self.num_workgroups}, "
                f"num_splits={self.num_splits}, pages_per_split={self.pages_per_split}, "
                f"workspace_bytes={self.workspace_bytes})")


_SIGNATURES = {
    "decode_attn": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P]),
    "decode_attn_ex": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P,
                            _P, _I, _I, _P, _SZ, _P]),
    "decode_attn_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                                 _P, _P, _I, _I, _P]),
    "decode_attn_plan": (_I, [_I, _I, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(Plan)]),
    "decode_attn_append": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P]),
    "decode_attn_prefill": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                 _I, _I, _F, _P, _P]),
    "decode_attn_hbm_reference": (_I, [_I, _I, _I, _P, _P, _P, _P, _P, ctypes.c_longlong,
                                       ctypes.c_longlong, _I, _P, _P]),
    "decode_attn_status_string": (ctypes.c_char_p, [_I]),
    "decode_attn_version": (_I, []),
}

_lib = None


class DecodeAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {STATUS.get(status, status)}")


def load_library(path: str = LIB_PATH):
    """Load (once) and return the ctypes handle of libdecode_attn.so."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m decode_phase_attention_paged_amd.build` "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DecodeAttnError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _validate(q, k_pages, v_pages, block_table, seq_lens, k_scale, v_scale, out):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("decode_attn runs on the GPU only; q is on " + str(dev))
    named = dict(q=q, k_pages=k_pages, v_pages=v_pages, block_table=block_table,
                 seq_lens=seq_lens, out=out)
    if k_scale is not None or v_scale is not None:
        named.update(k_scale=k_scale, v_scale=v_scale)
    for name, t in named.items():
        if t is None:
            raise ValueError(f"{name} is required")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k_pages.dim() != 4 or v_pages.shape != k_pages.shape or v_pages.dtype != k_pages.dtype:
        raise ValueError("k_pages and v_pages must both be [num_pages, n_kv_heads, block_size, head_dim]")
    kv = _pool_format(k_pages, k_scale, v_scale)
    if q.dtype != _row_dtype(kv) or q.dim() != 3:
        raise ValueError(f"q must be {_row_dtype(kv)} [batch, n_q_heads, head_dim] for a "
                         f"{KV_NAMES[kv]} cache")
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise ValueError("block_table must be int32 [batch, max_blocks_per_seq]")
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (q.shape[0],):
        raise ValueError("seq_lens must be int32 [batch]")
    if block_table.shape[0] != q.shape[0]:
        raise ValueError("block_table rows must equal batch")
    if out.dtype != torch.float32 or tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must be fp32 [batch, n_q_heads, head_dim]")
    if k_pages.shape[3] != q.shape[2]:
        raise ValueError("head_dim of q and the pages differ")
    return kv


def _common(q, k_pages, v_pages, block_table, seq_lens, k_scale, v_scale, out):
    kv = _validate(q, k_pages, v_pages, block_table, seq_lens, k_scale, v_scale, out)
    batch, n_q, head_dim = q.shape
    num_pages, n_kv, block_size, _ = k_pages.shape
    return (kv, batch, block_table.shape[1], num_pages, n_q, n_kv, head_dim, block_size)


def decode_attn(q, k_pages, v_pages, block_table, seq_lens, scale, *, k_scale=None,
                v_scale=None, out=None):
    """Decode attention with the library's own split plan and workspace.

    Returns ``out`` (fp32 [batch, n_q_heads, head_dim]); the work is enqueued on
    torch's current stream of q's device.
    """
    lib = load_library()
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    kv, batch, mb, np_, n_q, n_kv, d, bs = _common(q, k_pages, v_pages, block_table, seq_lens,
                                                   k_scale, v_scale, out)
    with torch.cuda.device(q.device):
        st = lib.decode_attn(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                             _ptr(v_scale), _ptr(block_table), _ptr(seq_lens), batch, mb, np_,
                             n_q, n_kv, d, bs, kv, float(scale), _ptr(out), _stream(q.device))
    _check(st, "decode_attn")
    return out


def plan(batch: int, max_blocks_per_seq: int, n_q_heads: int, n_kv_heads: int,
         block_size: int = 16, kv_dtype: str = "fp16", num_workgroups: int = 0,
         num_splits: int = 0, num_cus: int = 0) -> Plan:
    """The plan the library uses for these shapes and requests (see decode_attn_plan);
    kv_dtype is "fp16", "bf16", "int8" or "fp8"."""
    lib = load_library()
    out = Plan()
    kv = _KV_CODES[kv_dtype]
    _check(lib.decode_attn_plan(batch, max_blocks_per_seq, n_q_heads, n_kv_heads, block_size,
                                kv, num_workgroups, num_splits, num_cus, ctypes.byref(out)),
           "decode_attn_plan")
    return out


def decode_attn_ex(q, k_pages, v_pages, block_table, seq_lens, scale, *, k_scale=None,
                   v_scale=None, out=None, lse_out=None, num_workgroups=0, num_splits=0,
                   workspace=None):
    """Decode attention with an explicit plan request and caller-owned workspace.

    ``num_splits`` = 1 asks for segment mode (on ``num_workgroups`` workgroups
    when that is > 0), ``num_splits`` > 1 for split mode with that many page
    partitions per (sequence, KV head), ``num_workgroups`` > 0 alone for stream
    mode on that grid; both 0 let the library choose. ``workspace`` (a uint8 device tensor)
    is allocated here, through torch, when not given. ``lse_out`` (fp32
    [batch, n_q_heads]) receives the natural-log log-sum-exp of the scores
    when given. Returns ``out``.
    """
    lib = load_library()
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    kv, batch, mb, np_, n_q, n_kv, d, bs = _common(q, k_pages, v_pages, block_table, seq_lens,
                                                   k_scale, v_scale, out)
    if lse_out is not None:
        if (lse_out.dtype != torch.float32 or tuple(lse_out.shape) != (batch, n_q)
                or not lse_out.is_contiguous() or lse_out.device != q.device):
            raise ValueError("lse_out must be contiguous fp32 [batch, n_q_heads] on q's device")
    cus = torch.cuda.get_device_properties(q.device).multi_processor_count
    need = plan(batch, mb, n_q, n_kv, bs, kv_dtype=KV_NAMES[kv],
                num_workgroups=num_workgroups, num_splits=num_splits,
                num_cus=cus).workspace_bytes
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = lib.decode_attn_ex(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                                _ptr(v_scale), _ptr(block_table), _ptr(seq_lens), batch, mb, np_,
                                n_q, n_kv, d, bs, kv, float(scale), _ptr(out), _ptr(lse_out),
                                num_workgroups, num_splits, _ptr(workspace), ws_bytes,
                                _stream(q.device))
    _check(st, "decode_attn_ex")
    return out


def decode_attn_noalloc(q, k_pages, v_pages, block_table, seq_lens, scale, *, k_scale=None,
                        v_scale=None, out, lse_out=None, num_workgroups=0, num_splits=0):
    """decode_attn_ex without a workspace argument: the library's static per-device
    scratch array serves as the workspace, and nothing is allocated (``out`` must be
    given). Plans needing more than STATIC_SCRATCH_BYTES of workspace raise
    DECODE_ATTN_ERR_SCRATCH_LIMIT. Calls that overlap on one device share the array and
    must not run concurrently. Returns ``out``."""
    lib = load_library()
    kv, batch, mb, np_, n_q, n_kv, d, bs = _common(q, k_pages, v_pages, block_table, seq_lens,
                                                   k_scale, v_scale, out)
    if lse_out is not None:
        if (lse_out.dtype != torch.float32 or tuple(lse_out.shape) != (batch, n_q)
                or not lse_out.is_contiguous() or lse_out.device != q.device):
            raise ValueError("lse_out must be contiguous fp32 [batch, n_q_heads] on q's device")
    with torch.cuda.device(q.device):
        st = lib.decode_attn_noalloc(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                                     _ptr(v_scale), _ptr(block_table), _ptr(seq_lens), batch, mb,
                                     np_, n_q, n_kv, d, bs, kv, float(scale), _ptr(out),
                                     _ptr(lse_out), num_workgroups, num_splits,
                                     _stream(q.device))
    _check(st, "decode_attn_noalloc")
    return out


def decode_attn_append(k_new, v_new, block_table, positions, k_pages, v_pages, *,
                       k_scale=None, v_scale=None):
    """Write each sequence's new K/V row (fp16 [batch, n_kv_heads, head_dim]; bf16 for a
    bf16 cache) into its page slot, in place: row (b, g) goes to page
    block_table[b, p // bs], slot p % bs, with p = positions[b] (int32; p < 0 skips b).
    INT8 and FP8 pools (with k_scale / v_scale) store per-row codes and scales (see
    decode_attn_append in include/decode_attn.h).
    The work is enqueued on torch's current stream of k_new's device."""
    lib = load_library()
    dev = k_new.device
    if dev.type != "cuda":
        raise ValueError("decode_attn_append runs on the GPU only; k_new is on " + str(dev))
    named = dict(k_new=k_new, v_new=v_new, block_table=block_table, positions=positions,
                 k_pages=k_pages, v_pages=v_pages)
    if k_scale is not None or v_scale is not None:
        named.update(k_scale=k_scale, v_scale=v_scale)
    for name, t in named.items():
        if t is None:
            raise ValueError(f"{name} is required")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k_pages.dim() != 4 or v_pages.shape != k_pages.shape or v_pages.dtype != k_pages.dtype:
        raise ValueError("k_pages and v_pages must both be [num_pages, n_kv_heads, block_size, head_dim]")
    kv = _pool_format(k_pages, k_scale, v_scale)
    row = _row_dtype(kv)
    if k_new.dtype != row or k_new.dim() != 3 or v_new.shape != k_new.shape \
            or v_new.dtype != row:
        raise ValueError(f"k_new and v_new must be {row} [batch, n_kv_heads, head_dim] for a "
                         f"{KV_NAMES[kv]} cache")
    batch, n_kv, head_dim = k_new.shape
    num_pages, pool_kv, block_size, pool_d = k_pages.shape
    if (pool_kv, pool_d) != (n_kv, head_dim):
        raise ValueError("the new rows' heads or head_dim differ from the pools'")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != batch:
        raise ValueError("block_table must be int32 [batch, max_blocks_per_seq]")
    if positions.dtype != torch.int32 or tuple(positions.shape) != (batch,):
        raise ValueError("positions must be int32 [batch]")
    with torch.cuda.device(dev):
        st = lib.decode_attn_append(_ptr(k_new), _ptr(v_new), _ptr(block_table), _ptr(positions),
                                    batch, block_table.shape[1], num_pages, n_kv, head_dim,
                                    block_size, kv, _ptr(k_pages), _ptr(v_pages), _ptr(k_scale),
                                    _ptr(v_scale), _stream(dev))
    _check(st, "decode_attn_append")


def decode_attn_prefill(q, q_start, k_pages, v_pages, block_table, seq_lens, scale, *,
                        k_scale=None, v_scale=None, max_chunk: Optional[int] = None, out=None):
    """Chunked-prefill attention (see decode_attn_prefill in include/decode_attn.h).

    ``q`` holds every sequence's chunk rows stacked ([T, n_q_heads, head_dim], fp16, or
    bf16 for a bf16 cache); sequence b's rows are ``q[q_start[b]:q_start[b+1]]`` (int32
    [batch + 1]) and sit at the end of its ``seq_lens[b]`` cached tokens. int8 and
    float8_e4m3fn pools take fp32 row scales, as for decode_attn. ``max_chunk`` bounds the
    chunk sizes for the grid (default: T, always safe). Returns ``out`` (fp32
    [T, n_q_heads, head_dim]), enqueued on torch's current stream of q's device."""
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("decode_attn_prefill runs on the GPU only; q is on " + str(dev))
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    named = dict(q=q, q_start=q_start, k_pages=k_pages, v_pages=v_pages,
                 block_table=block_table, seq_lens=seq_lens, out=out)
    if k_scale is not None or v_scale is not None:
        named.update(k_scale=k_scale, v_scale=v_scale)
    for name, t in named.items():
        if t is None:
            raise ValueError(f"{name} is required")
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k_pages.dim() != 4 or v_pages.shape != k_pages.shape or v_pages.dtype != k_pages.dtype:
        raise ValueError("k_pages and v_pages must both be [num_pages, n_kv_heads, block_size, head_dim]")
    kv = _pool_format(k_pages, k_scale, v_scale)
    if q.dtype != _row_dtype(kv) or q.dim() != 3:
        raise ValueError(f"q must be {_row_dtype(kv)} [total_rows, n_q_heads, head_dim] for a "
                         f"{KV_NAMES[kv]} cache")
    if out.dtype != torch.float32 or tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must be fp32 [total_rows, n_q_heads, head_dim]")
    batch = seq_lens.shape[0]
    if q_start.dtype != torch.int32 or tuple(q_start.shape) != (batch + 1,):
        raise ValueError("q_start must be int32 [batch + 1]")
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1:
        raise ValueError("seq_lens must be int32 [batch]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != batch:
        raise ValueError("block_table must be int32 [batch, max_blocks_per_seq]")
    total, n_q, head_dim = q.shape
    num_pages, n_kv, block_size, pool_d = k_pages.shape
    if pool_d != head_dim:
        raise ValueError("head_dim of q and the pages differ")
    chunk = max(1, total if max_chunk is None else int(max_chunk))
    with torch.cuda.device(dev):
        st = lib.decode_attn_prefill(_ptr(q), _ptr(q_start), _ptr(k_pages), _ptr(v_pages),
                                     _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
                                     _ptr(seq_lens), batch, total, block_table.shape[1],
                                     num_pages, n_q, n_kv, head_dim, block_size, kv, chunk,
                                     float(scale), _ptr(out), _stream(dev))
    _check(st, "decode_attn_prefill")
    return out


HBM_STREAM = 0
HBM_GATHER = 1          # 4 KiB tiles (16-bit K/V)
HBM_GATHER_SCALED = 2   # 2 KiB tiles plus 64-byte row-scale records (1-byte K/V)
_HBM_TILE_BYTES = {HBM_GATHER: 4096, HBM_GATHER_SCALED: 2048}


def hbm_reference(kind: int, a: torch.Tensor, sink: torch.Tensor, *, b=None, tiles=None,
                  a_scale=None, b_scale=None, depth: int = 2, nontemporal: bool = True,
                  grid: int = 512, count: Optional[int] = None) -> None:
    """Reference reads for the HBM roofline (decode_attn_hbm_reference): HBM_STREAM reads
    ``count`` 16-byte words of ``a`` (default: all of it); HBM_GATHER reads, for every entry
    t of ``tiles`` (int32), the 4 KiB tile t of ``a`` and of ``b``; HBM_GATHER_SCALED the
    2 KiB tile t of each and the 64-byte records t of ``a_scale`` and ``b_scale``. ``sink``
    is int32 [>= grid * 256]. Enqueued on torch's current stream of a's device."""
    lib = load_library()
    dev = a.device
    if dev.type != "cuda":
        raise ValueError("hbm_reference runs on the GPU only")
    if sink.dtype != torch.int32 or sink.numel() < grid * 256 or sink.device != dev:
        raise ValueError("sink must be int32 with at least grid * 256 elements on a's device")
    nbytes = lambda t: t.numel() * t.element_size()
    if kind == HBM_STREAM:
        n = nbytes(a) // 16 if count is None else int(count)
        b = tiles = a_scale = b_scale = None
        num_tiles = 0
    elif kind in _HBM_TILE_BYTES:
        if b is None or tiles is None or tiles.dtype != torch.int32:
            raise ValueError("a gather needs b and int32 tiles")
        if nbytes(b) != nbytes(a):
            raise ValueError("a and b must be pools of the same size")
        num_tiles = nbytes(a) // _HBM_TILE_BYTES[kind]
        if kind == HBM_GATHER_SCALED:
            if a_scale is None or b_scale is None:
                raise ValueError("a scaled gather needs a_scale and b_scale")
            if min(nbytes(a_scale), nbytes(b_scale)) < 64 * num_tiles:
                raise ValueError("a_scale and b_scale need 64 bytes per tile")
        else:
            a_scale = b_scale = None
        n = tiles.numel() if count is None else int(count)
    else:
        raise ValueError("kind must be HBM_STREAM, HBM_GATHER or HBM_GATHER_SCALED")
    with torch.cuda.device(dev):
        status = lib.decode_attn_hbm_reference(kind, depth, int(bool(nontemporal)), _ptr(a),
                                               _ptr(b), _ptr(a_scale), _ptr(b_scale),
                                               _ptr(tiles), n, num_tiles, grid, _ptr(sink),
                                               _stream(dev))
    _check(status, "decode_attn_hbm_reference")
