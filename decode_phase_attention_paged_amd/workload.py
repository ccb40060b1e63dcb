"""Seeded synthetic workloads for decode-phase paged attention.

This module only draws inputs and lays them out in pages; it holds none of
the attention arithmetic. Both the oracle tests and the GPU path take their
inputs from here, so the two sides always see identical arrays.

The five presets stand in for the workloads the pages talk about: a
Llama-2-7B-shaped MHA batch and a Llama-3-8B-shaped GQA batch (xLLM README,
benchmark section; swiftLLM README, performance section), one very long
context (the long-context case of the C++/CUDA engine blog, section 3.4), and
a per-row INT8 cache (xLLM README, quantisation list). No weights, prompts or
datasets are involved: values are random with the stated distributions.

Draw order for a given seed is fixed:
  seq_lens -> page permutation -> q -> K -> V -> peaky rows -> (k_scale, v_scale)
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

__all__ = [
    "Config",
    "CONFIGS",
    "Workload",
    "generate",
    "kv_read_bytes",
    "other_bytes",
]


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    len_lo: int                 # seq_lens ~ integer uniform on [len_lo, len_hi]
    len_hi: int
    kv_dtype: str               # "fp16" or "int8"
    identity_table: bool = False
    peaky_fraction: float = 0.0  # fraction of each (sequence, KV head)'s keys scaled
    peaky_factor: float = 1.0
    scale: Optional[float] = None  # None -> 1/sqrt(head_dim)

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.len_hi // self.block_size)

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim))) if self.scale is None \
            else float(np.float32(self.scale))

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    1: Config(1, "tiny_mha", 1, 8, 8, 128, 16, 256, 256, "fp16", identity_table=True),
    2: Config(2, "llama2_7b_mha_b48", 48, 32, 32, 128, 16, 18, 563, "fp16"),
    3: Config(3, "llama3_8b_gqa_b160", 160, 32, 8, 128, 16, 64, 4096, "fp16"),
    4: Config(4, "long_ctx_gqa_131k", 1, 32, 8, 128, 16, 131072, 131072, "fp16",
              peaky_fraction=0.01, peaky_factor=8.0),
    5: Config(5, "int8_mha_b200", 200, 32, 32, 128, 16, 18, 530, "int8"),
}


@dataclass
class Workload:
    config: Config
    seed: int
    q: np.ndarray             # fp16 [B, Hq, D]
    k_pages: np.ndarray       # fp16 | int8 [NP, Hkv, bs, D]
    v_pages: np.ndarray
    k_scale: Optional[np.ndarray]   # fp32 [NP, Hkv, bs] for int8, else None
    v_scale: Optional[np.ndarray]
    block_table: np.ndarray   # int32 [B, MB], -1 past each sequence's last block
    seq_lens: np.ndarray      # int32 [B]
    scale: float              # fp32-representable softmax scale

    @property
    def num_pages(self) -> int:
        return self.k_pages.shape[0]

    @property
    def kv_bytes(self) -> int:
        c = self.config
        return kv_read_bytes(self.seq_lens, c.n_kv_heads, c.head_dim,
                             1 if c.kv_dtype == "int8" else 2,
                             4 if c.kv_dtype == "int8" else 0)


def kv_read_bytes(seq_lens, n_kv_heads: int, head_dim: int, elem_bytes: int,
                  row_scale_bytes: int = 0) -> int:
    """Algorithmic K+V bytes one decode-attention step must read.

    Every valid token of every sequence is read once for K and once for V, per
    KV head: sum_b L_b * Hkv * 2 * (D * elem + row_scale). This is the same
    accounting as the KV-cache row of the xLLM README's memory table
    (2 * b * h1 * tokens elements per layer, with h1 = Hkv * D).
    """
    tokens = int(np.asarray(seq_lens, dtype=np.int64).sum())
    return tokens * n_kv_heads * 2 * (head_dim * elem_bytes + row_scale_bytes)


def other_bytes(config: Config) -> int:
    """Non-KV algorithmic bytes of one step: q in, out out, table and lengths."""
    c = config
    return (c.batch * c.n_q_heads * c.head_dim * (2 + 4)
            + c.batch * c.max_blocks_per_seq * 4 + c.batch * 4)


def _poison_unused_slots(w: Workload, n_used_pages: int) -> None:
    """Fill every slot no valid token owns with NaN (fp16 values, int8 scales)."""
    bs = w.config.block_size
    for b in range(w.config.batch):
        length = int(w.seq_lens[b])
        nb = -(-length // bs)
        tail = length - (nb - 1) * bs if nb else bs
        if nb and tail < bs:
            page = w.block_table[b, nb - 1]
            if w.k_scale is None:
                w.k_pages[page, :, tail:, :] = np.float16(np.nan)
                w.v_pages[page, :, tail:, :] = np.float16(np.nan)
            else:
                w.k_scale[page, :, tail:] = np.float32(np.nan)
                w.v_scale[page, :, tail:] = np.float32(np.nan)
    unused = np.setdiff1d(np.arange(w.num_pages),
                          w.block_table[w.block_table >= 0], assume_unique=False)
    if unused.size:
        if w.k_scale is None:
            w.k_pages[unused] = np.float16(np.nan)
            w.v_pages[unused] = np.float16(np.nan)
        else:
            w.k_scale[unused] = np.float32(np.nan)
            w.v_scale[unused] = np.float32(np.nan)


def generate(config: Config, seed: Optional[int] = None, *, poison: bool = False,
             extra_pages: int = 0, seq_lens: Optional[np.ndarray] = None) -> Workload:
    """Draw one workload.

    ``seed`` defaults to 1000 + config.index. ``seq_lens`` overrides the drawn
    lengths (the draw still happens, so the rest of the stream is unchanged).
    ``extra_pages`` adds pages no sequence references; with ``poison`` those
    pages and every unused slot of each last page hold NaN (for int8 caches,
    their row scales do), so any stray read shows up in the output.
    """
    c = config
    seed = 1000 + c.index if seed is None else int(seed)
    rng = np.random.default_rng(seed)
    bs, hkv, d = c.block_size, c.n_kv_heads, c.head_dim

    lens = rng.integers(c.len_lo, c.len_hi + 1, size=c.batch).astype(np.int32)
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int32).copy()
        if lens.shape != (c.batch,):
            raise ValueError("seq_lens override must have shape [batch]")
    mb = c.max_blocks_per_seq
    if lens.size and (lens.min() < 0 or lens.max() > mb * bs):
        raise ValueError("seq_lens out of range for max_blocks_per_seq")
    n_blocks = -(-lens.astype(np.int64) // bs)
    n_used = int(n_blocks.sum())
    n_pages = n_used + int(extra_pages)

    perm = np.arange(n_pages) if c.identity_table else rng.permutation(n_pages)
    table = np.full((c.batch, mb), -1, dtype=np.int32)
    offset = 0
    for b in range(c.batch):
        nb = int(n_blocks[b])
        table[b, :nb] = perm[offset:offset + nb]
        offset += nb

    q = rng.standard_normal((c.batch, c.n_q_heads, d), dtype=np.float32).astype(np.float16)
    shape = (n_pages, hkv, bs, d)
    k_scale = v_scale = None
    if c.kv_dtype == "fp16":
        k32 = rng.standard_normal(shape, dtype=np.float32)
        v_pages = rng.standard_normal(shape, dtype=np.float32).astype(np.float16)
        if c.peaky_fraction > 0:
            for b in range(c.batch):
                length = int(lens[b])
                count = int(round(c.peaky_fraction * length))
                for g in range(hkv):
                    tokens = rng.choice(length, size=count, replace=False)
                    pages = table[b, tokens // bs]
                    k32[pages, g, tokens % bs, :] *= np.float32(c.peaky_factor)
        k_pages = k32.astype(np.float16)
        del k32
    elif c.kv_dtype == "int8":
        k_pages = rng.integers(-127, 128, size=shape, dtype=np.int8)
        v_pages = rng.integers(-127, 128, size=shape, dtype=np.int8)
        k_scale = rng.uniform(0.005, 0.02, size=shape[:3]).astype(np.float32)
        v_scale = rng.uniform(0.005, 0.02, size=shape[:3]).astype(np.float32)
    else:
        raise ValueError(f"unknown kv_dtype {c.kv_dtype!r}")

    w = Workload(c, seed, q, k_pages, v_pages, k_scale, v_scale, table, lens,
                 c.softmax_scale)
    if poison:
        _poison_unused_slots(w, n_used)
    return w
