"""Plain fp64 CPU oracle for decode-phase paged attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library: it reads the same documented memory layout and computes the plain
definition, slowly and in float64.

What it computes, and where the pages define it:

* Decode phase (page "Eine LLM-Inferenz-Engine von Grund auf mit C++ und CUDA
  bauen", section 1.1): each sequence contributes one new query token that
  attends over the keys and values cached for all of its earlier tokens.
* PagedAttention (swiftLLM README, feature list): the cache lives in
  fixed-size blocks, found through a per-sequence block table. The oracle
  first materialises each sequence's contiguous K and V from its pages and
  only then attends, so no paging trick reaches the arithmetic.
* GQA (xLLM README, optimisation list, "KV Cache"): several query heads share
  one KV head; query head h reads KV head h // G with G = Hq / Hkv.
* Per-row INT8 (xLLM README, optimisation list, quantisation): a stored row is
  one (token, KV head) vector of int8 values with one fp32 scale; its value is
  int8 * scale.
* BF16 caches (xLLM README, quantisation: "FP16, BF16") and FP8 E4M3 caches
  with per-row scales (C++/CUDA engine blog, section 4): elements are decoded
  to their exact values by ``oracle/formats.py`` before anything else.
* The online-normaliser softmax (xLLM README, SoftMax operator) and the
  split/merge of PagedAttention v2 / Flash-Decoding (swiftLLM feature list)
  are ways to reach this same result faster. The oracle uses neither: it is
  the naive softmax(scale * q K^T) V.

Memory layout read here (the pages leave it open; this is the library's
documented layout):
  q           [B, Hq, D]            fp16 (bf16 bit patterns, uint16, for a bf16 cache)
  k_pages     [NP, Hkv, bs, D]      fp16; bf16 as uint16 bit patterns; or int8 or
                                    E4M3 codes (uint8) with k_scale [NP, Hkv, bs] fp32
  v_pages     [NP, Hkv, bs, D]      same as k_pages
  block_table [B, MB]               int32; entry j of row b is the physical page
                                    holding tokens j*bs .. j*bs+bs-1 of sequence b
  seq_lens    [B]                   int32; 0 <= L_b <= MB*bs

Every function here is pinned by ``tests/test_oracle.py`` (brute force on tiny
inputs, a float64 library attention routine, closed forms and invariants).
"""

from __future__ import annotations

import numpy as np

from .formats import element_values

__all__ = [
    "gather_sequence",
    "dequantize_rows",
    "kv_head_of",
    "attend",
    "decode_attention",
]


def gather_sequence(pages: np.ndarray, table_row: np.ndarray, seq_len: int,
                    block_size: int) -> np.ndarray:
    """Materialise one sequence's contiguous cache from its pages.

    PagedAttention (swiftLLM feature list): logical block j of the sequence is
    the physical page ``table_row[j]``; token t sits in block t // bs at slot
    t % bs. Returns an array [Hkv, seq_len, ...] holding the sequence's tokens
    in order. Only the first ceil(seq_len / bs) table entries are read, and
    slots beyond seq_len in the last page are dropped.
    """
    seq_len = int(seq_len)
    n_kv = pages.shape[1]
    if seq_len == 0:
        return np.empty((n_kv, 0) + pages.shape[3:], dtype=pages.dtype)
    n_blocks = -(-seq_len // block_size)
    phys = np.asarray(table_row[:n_blocks], dtype=np.int64)
    tiles = pages[phys]                        # [nb, Hkv, bs, ...]
    per_head = np.swapaxes(tiles, 0, 1)        # [Hkv, nb, bs, ...]
    flat = per_head.reshape((n_kv, n_blocks * block_size) + pages.shape[3:])
    return flat[:, :seq_len]


def dequantize_rows(rows_int8: np.ndarray, row_scales: np.ndarray) -> np.ndarray:
    """Per-row INT8 (xLLM README, quantisation): value = int8 * row scale.

    ``rows_int8`` is [..., D] (int8 values, or the float64 values of decoded
    E4M3 codes, which take their row scale the same way); ``row_scales`` is
    [...] (one fp32 scale per row). Symmetric, no zero point, no clamping.
    Returns float64.
    """
    return rows_int8.astype(np.float64) * row_scales.astype(np.float64)[..., None]


def kv_head_of(q_head: int, group: int) -> int:
    """GQA (xLLM README, "KV Cache"): query head h reads KV head h // G."""
    return q_head // group


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """Attention of one query vector over L cached tokens, in float64.

    q [D], keys [L, D], values [L, Dv]. Scores s_t = scale * <q, k_t>;
    weights p = softmax(s); output sum_t p_t v_t; lse = log sum_t exp(s_t)
    (natural log). The max is subtracted before exp only to keep exp finite;
    it cancels exactly in p and is added back in lse. L = 0 gives a zero
    output and lse = -inf (the pages are silent on an empty cache; this is the
    reading taken for it).
    """
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1], dtype=np.float64), -np.inf, np.zeros(0)
    scores = scale * (keys @ q)
    peak = scores.max()
    e = np.exp(scores - peak)
    total = e.sum()
    p = e / total
    return p @ values, float(peak + np.log(total)), p


def decode_attention(q, k_pages, v_pages, block_table, seq_lens, scale,
                     k_scale=None, v_scale=None, return_probs=False,
                     out_dtype=np.float32):
    """Decode attention for a batch, over a paged KV cache, in float64.

    Arguments follow the layout in the module docstring. ``scale`` is taken as
    the fp32 value the library receives and then widened to float64, so both
    sides use the identical number. For INT8 caches ``k_scale``/``v_scale``
    hold the per-row scales and must both be given.

    Returns ``(out, lse)``: out [B, Hq, D] in ``out_dtype`` (by default the
    float64 result rounded to nearest float32, the library's output type; pass
    np.float64 to keep every bit), lse float64 [B, Hq] (natural log; -inf for
    an empty cache).
    With ``return_probs`` a third item is a dict {(b, h): p} of the softmax
    weights over the sequence's tokens, in token order.
    """
    q = np.asarray(q)
    batch, n_q, head_dim = q.shape
    n_kv = k_pages.shape[1]
    block_size = k_pages.shape[2]
    if n_q % n_kv != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    group = n_q // n_kv
    quantized = k_scale is not None
    if quantized != (v_scale is not None):
        raise ValueError("k_scale and v_scale go together")
    sigma = float(np.float32(scale))

    out = np.zeros((batch, n_q, v_pages.shape[3]), dtype=np.float64)
    lse = np.full((batch, n_q), -np.inf, dtype=np.float64)
    probs = {}
    for b in range(batch):
        length = int(seq_lens[b])
        keys = element_values(gather_sequence(k_pages, block_table[b], length, block_size))
        values = element_values(gather_sequence(v_pages, block_table[b], length, block_size))
        if quantized:
            keys = dequantize_rows(
                keys, gather_sequence(k_scale, block_table[b], length, block_size))
            values = dequantize_rows(
                values, gather_sequence(v_scale, block_table[b], length, block_size))
        q_b = element_values(q[b])
        for h in range(n_q):
            g = kv_head_of(h, group)
            o, l, p = attend(q_b[h], keys[g], values[g], sigma)
            out[b, h] = o
            lse[b, h] = l
            if return_probs:
                probs[(b, h)] = p
    result = (out.astype(out_dtype), lse)
    if return_probs:
        result = result + (probs,)
    return result
