"""Plain fp64 CPU oracle for chunked-prefill attention over the paged cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module; only ``tests/`` and ``bench.py``'s CPU-baseline leg use
it. It shares no code with the HIP library.

What it computes, and where the pages define it:

* The prefill phase runs a prompt's tokens through the model and fills the KV
  cache (page "Eine LLM-Inferenz-Engine von Grund auf mit C++ und CUDA bauen",
  section 1.1); handling several prompt tokens at once, with FlashAttention-
  style fused attention, is among that page's next steps (section 4); the
  swiftLLM README's feature list serves prefill chunks piggybacked on decode
  batches (SARATHI) with FlashAttention. Each new token attends causally: to
  every cached token up to and including its own position, and to none after.
* The cache is the same paged cache the decode oracle reads (swiftLLM feature
  list: PagedAttention), through the same block table; GQA maps query head h
  to KV head h // G (xLLM README, "KV Cache").

Reading taken where the pages are silent: a sequence's chunk is its last C_b
tokens, whose K/V rows are already in the cache (appended before the
attention, as in the decode step), so L_b counts them and chunk row i sits at
position L_b - C_b + i. A decode token is the chunk with C_b = 1, so a batch
may mix prefill chunks and decode tokens. Rows of all chunks are stacked:
sequence b's rows are q[q_start[b] : q_start[b + 1]].

Pinned by ``tests/test_oracle_prefill.py``.
"""

from __future__ import annotations

import numpy as np

from .decode import attend, dequantize_rows, gather_sequence, kv_head_of
from .formats import element_values

__all__ = ["prefill_attention"]


def prefill_attention(q, k_pages, v_pages, block_table, seq_lens, q_start, scale,
                      k_scale=None, v_scale=None, out_dtype=np.float32):
    """Causal attention of every chunk row over its sequence's cached prefix, in float64.

    q [T, Hq, D] (T = q_start[B]); q_start [B + 1] int, non-decreasing, q_start[0] = 0,
    with C_b = q_start[b + 1] - q_start[b] <= L_b = seq_lens[b]. Returns (out [T, Hq, D] in
    ``out_dtype``, lse float64 [T, Hq]).
    """
    q = np.asarray(q)
    q_start = np.asarray(q_start, dtype=np.int64)
    total, n_q, _ = q.shape
    batch = len(seq_lens)
    n_kv = k_pages.shape[1]
    block_size = k_pages.shape[2]
    if n_q % n_kv != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if q_start.shape != (batch + 1,) or q_start[0] != 0 or q_start[-1] != total \
            or np.any(np.diff(q_start) < 0):
        raise ValueError("q_start must run from 0 to T in non-decreasing steps")
    group = n_q // n_kv
    sigma = float(np.float32(scale))
    out = np.zeros((total, n_q, v_pages.shape[3]), dtype=np.float64)
    lse = np.full((total, n_q), -np.inf, dtype=np.float64)
    for b in range(batch):
        length = int(seq_lens[b])
        chunk = int(q_start[b + 1] - q_start[b])
        if chunk > length:
            raise ValueError("a chunk cannot be longer than its sequence")
        keys = element_values(gather_sequence(k_pages, block_table[b], length, block_size))
        values = element_values(gather_sequence(v_pages, block_table[b], length, block_size))
        if k_scale is not None:
            keys = dequantize_rows(keys, gather_sequence(k_scale, block_table[b], length,
                                                         block_size))
            values = dequantize_rows(values, gather_sequence(v_scale, block_table[b], length,
                                                             block_size))
        for i in range(chunk):
            row = int(q_start[b]) + i
            visible = length - chunk + i + 1          # tokens 0 .. position, inclusive
            q_row = element_values(q[row])
            for h in range(n_q):
                g = kv_head_of(h, group)
                o, l, _ = attend(q_row[h], keys[g, :visible], values[g, :visible], sigma)
                out[row, h] = o
                lse[row, h] = l
    return out.astype(out_dtype), lse
