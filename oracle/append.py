"""Plain CPU oracle for writing a decode step's new K/V rows into the paged cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module; only ``tests/`` and ``__graft_entry__.smoke()`` use it.
It shares no code with the HIP library.

What it computes, and where the pages define it:

* Decode phase (page "Eine LLM-Inferenz-Engine von Grund auf mit C++ und CUDA
  bauen", section 1.1): every step appends the new token's key and value to the
  cache before attending.
* PagedAttention (swiftLLM README, feature list): the cache lives in fixed-size
  pages found through the block table, so token position p of sequence b goes
  to page ``block_table[b, p // bs]``, slot ``p % bs``.
* Per-row INT8 (xLLM README, optimisation list, quantisation): a stored row is
  one (token, KV head) vector of int8 codes with one fp32 scale, value =
  code * scale. The pages do not say how the codes are chosen; this oracle
  takes the symmetric max-abs rule with round-half-to-even, computed in fp32
  (the precision the kernel computes in, so both sides take the same integer
  decisions):
      s     = fp32(max_d |x_d|) / 127          (fp32 division)
      code  = rint(fp32(x_d) / s)              (fp32 division, ties to even)
  clamped to [-127, 127]; a row of zeros stores s = 0 and codes 0.
* FP8 E4M3 rows (C++/CUDA engine blog, section 4: FP8 cache quantisation;
  format as read in ``oracle/formats.py``) are quantised the same way with the
  format's largest magnitude in place of 127:
      s     = fp32(max_d |x_d|) / 448          (fp32 division)
      code  = e4m3(fp32(x_d) / s)              (fp32 division, nearest, ties to
                                                the even code)
  and a row of zeros stores s = 0 and codes 0x00. BF16 rows are stored as they
  are (the new rows of a BF16 cache are bf16 too).

Layout (the library's documented one): pools [NP, Hkv, bs, D] (fp16, bf16 bit
patterns as uint16, or int8 / E4M3 codes as uint8 with scales [NP, Hkv, bs]
fp32); new rows [B, Hkv, D] fp16 (bf16 bit patterns for a bf16 pool); block_table
[B, MB] int32; positions [B] int32, where a negative position means "no new
token for this sequence".

Pinned by ``tests/test_oracle_append.py``.
"""

from __future__ import annotations

import numpy as np

from .formats import e4m3_from_float32

__all__ = ["quantize_row", "quantize_row_fp8", "append_kv"]

_F32 = np.float32


def quantize_row(x: np.ndarray):
    """Per-row INT8 quantisation of one (token, KV head) row (see the module
    docstring for the rule). Returns (codes int8 [D], scale fp32)."""
    x32 = np.asarray(x, dtype=_F32)
    maxabs = _F32(np.max(np.abs(x32))) if x32.size else _F32(0)
    if maxabs == 0:
        return np.zeros(x32.shape, dtype=np.int8), _F32(0)
    s = _F32(maxabs / _F32(127))
    codes = np.rint(x32 / s)
    codes = np.clip(codes, -127, 127).astype(np.int8)
    return codes, s


def quantize_row_fp8(x: np.ndarray):
    """Per-row FP8 E4M3 quantisation of one (token, KV head) row (see the module
    docstring for the rule). Returns (codes uint8 [D], scale fp32)."""
    x32 = np.asarray(x, dtype=_F32)
    maxabs = _F32(np.max(np.abs(x32))) if x32.size else _F32(0)
    if maxabs == 0:
        return np.zeros(x32.shape, dtype=np.uint8), _F32(0)
    s = _F32(maxabs / _F32(448))
    return e4m3_from_float32(x32 / s), s


def append_kv(k_pages, v_pages, block_table, positions, k_new, v_new, block_size,
              k_scale=None, v_scale=None):
    """Write row (b, g) of ``k_new`` / ``v_new`` into page
    ``block_table[b, p // bs]``, slot ``p % bs``, head g, for every b with
    p = positions[b] >= 0. FP16 and BF16 pools take the row as it is; INT8 pools
    (int8, with ``k_scale`` / ``v_scale``) take ``quantize_row`` of it and FP8
    pools (uint8 codes, with scales) ``quantize_row_fp8``.

    Returns updated copies (k_pages, v_pages, k_scale, v_scale); the inputs are
    not modified. Positions must lie below MB * bs and their pages inside the
    pools (the caller's precondition; the library skips rows that violate it).
    """
    k_pages = np.array(k_pages, copy=True)
    v_pages = np.array(v_pages, copy=True)
    scaled = k_scale is not None
    quantize = quantize_row_fp8 if k_pages.dtype == np.uint8 else quantize_row
    if scaled:
        k_scale = np.array(k_scale, copy=True)
        v_scale = np.array(v_scale, copy=True)
    batch, n_kv_heads, _ = k_new.shape
    for b in range(batch):
        p = int(positions[b])
        if p < 0:
            continue
        page = int(block_table[b, p // block_size])
        slot = p % block_size
        for g in range(n_kv_heads):
            if scaled:
                k_pages[page, g, slot], k_scale[page, g, slot] = quantize(k_new[b, g])
                v_pages[page, g, slot], v_scale[page, g, slot] = quantize(v_new[b, g])
            else:
                k_pages[page, g, slot] = k_new[b, g]
                v_pages[page, g, slot] = v_new[b, g]
    return k_pages, v_pages, k_scale, v_scale
