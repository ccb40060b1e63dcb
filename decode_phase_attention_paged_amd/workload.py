"""Seeded synthetic workloads for decode-phase paged attention.

This module only draws inputs and lays them out in pages; it holds none of
the attention arithmetic. Both the oracle tests and the GPU path take their
inputs from here, so the two sides always see identical arrays.

The five first presets stand in for the workloads the pages talk about: a
Llama-2-7B-shaped MHA batch and a Llama-3-8B-shaped GQA batch (xLLM README,
benchmark section; swiftLLM README, performance section), one very long
context (the long-context case of the C++/CUDA engine blog, section 3.4), and
a per-row INT8 cache (xLLM README, quantisation list). Two more carry the other
storage formats the pages name: a BF16 cache (xLLM README, quantisation list:
"FP16, BF16") on the Llama-2-7B batch, and an FP8 E4M3 cache with per-row
scales (C++/CUDA engine blog, section 4) on the INT8 batch's shape. Three more take the
grouped-query shapes to the other group sizes and formats: 64 query heads over 8 KV heads
(G = 8, the Llama-3-70B head shape) in fp16 and per-row INT8, and the Llama-3-8B batch
(G = 4) over per-row INT8. No weights,
prompts or datasets are involved: values are random with the stated
distributions.

BF16 values are drawn as fp32 N(0, 1) and kept as the upper 16 bits of each
fp32 word (numpy has no bf16 type, so bf16 arrays hold uint16 bit patterns);
for a BF16 cache q is bf16 too. FP8 codes are uniform over the 254 finite E4M3
codes (every code but 0x7F and 0xFF), with row scales U(0.005, 0.02) * 127/448,
so that the largest code reaches the magnitude of the INT8 preset's largest.

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
    "prefill_rows",
    "prefill_flops",
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
    kv_dtype: str               # "fp16", "bf16", "int8" or "fp8"
    identity_table: bool = False
    peaky_fraction: float = 0.0  # fraction of each (sequence, KV head)'s keys scaled
    peaky_factor: float = 1.0
    scale: Optional[float] = None  # None -> 1/sqrt(head_dim)
    chunk: int = 0              # prefill presets: new tokens per sequence (C_b = min(chunk, L_b))

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
    6: Config(6, "llama2_7b_mha_b48_bf16", 48, 32, 32, 128, 16, 18, 563, "bf16"),
    7: Config(7, "fp8_mha_b200", 200, 32, 32, 128, 16, 18, 530, "fp8"),
    8: Config(8, "llama3_8b_gqa_prefill_c512", 8, 32, 8, 128, 16, 512, 4096, "fp16", chunk=512),
    9: Config(9, "llama3_70b_gqa8_b64", 64, 64, 8, 128, 16, 64, 4096, "fp16"),
    10: Config(10, "llama3_70b_gqa8_b64_int8", 64, 64, 8, 128, 16, 64, 4096, "int8"),
    11: Config(11, "llama3_8b_gqa_b160_int8", 160, 32, 8, 128, 16, 64, 4096, "int8"),
}

# Storage bytes per element and per row scale, by kv_dtype.
ELEM_BYTES = {"fp16": 2, "bf16": 2, "int8": 1, "fp8": 1}
SCALE_BYTES = {"fp16": 0, "bf16": 0, "int8": 4, "fp8": 4}


@dataclass
class Workload:
    config: Config
    seed: int
    q: np.ndarray             # fp16 [B, Hq, D]; bf16 bits (uint16) for a bf16 cache
    k_pages: np.ndarray       # fp16 | bf16 bits (uint16) | int8 | E4M3 codes (uint8)
    v_pages: np.ndarray       #   [NP, Hkv, bs, D]
    k_scale: Optional[np.ndarray]   # fp32 [NP, Hkv, bs] for int8 and fp8, else None
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
                             ELEM_BYTES[c.kv_dtype], SCALE_BYTES[c.kv_dtype])


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


_NAN = {np.dtype(np.float16): np.float16(np.nan), np.dtype(np.uint16): np.uint16(0x7FC0)}


def _poison_unused_slots(w: Workload, n_used_pages: int) -> None:
    """Fill every slot no valid token owns with NaN (fp16 and bf16 values, int8 and fp8
    row scales)."""
    bs = w.config.block_size
    for b in range(w.config.batch):
        length = int(w.seq_lens[b])
        nb = -(-length // bs)
        tail = length - (nb - 1) * bs if nb else bs
        if nb and tail < bs:
            page = w.block_table[b, nb - 1]
            if w.k_scale is None:
                w.k_pages[page, :, tail:, :] = _NAN[w.k_pages.dtype]
                w.v_pages[page, :, tail:, :] = _NAN[w.v_pages.dtype]
            else:
                w.k_scale[page, :, tail:] = np.float32(np.nan)
                w.v_scale[page, :, tail:] = np.float32(np.nan)
    unused = np.setdiff1d(np.arange(w.num_pages),
                          w.block_table[w.block_table >= 0], assume_unique=False)
    if unused.size:
        if w.k_scale is None:
            w.k_pages[unused] = _NAN[w.k_pages.dtype]
            w.v_pages[unused] = _NAN[w.v_pages.dtype]
        else:
            w.k_scale[unused] = np.float32(np.nan)
            w.v_scale[unused] = np.float32(np.nan)


def prefill_rows(w: "Workload", chunk: Optional[int] = None, seed: Optional[int] = None):
    """Chunk query rows for a prefill step over workload w: C_b = min(chunk, L_b) rows per
    sequence, stacked in sequence order. Returns (q [T, Hq, D] ~ N(0, 1), fp16, or bf16 bit
    patterns (uint16) for a bf16 cache, and q_start int32 [B + 1]). Drawn from their own
    stream (seed + 1), so w's draws are unchanged."""
    c = w.config
    chunk = c.chunk if chunk is None else int(chunk)
    sizes = np.minimum(np.asarray(w.seq_lens, dtype=np.int64), chunk)
    q_start = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rng = np.random.default_rng((w.seed if seed is None else int(seed)) + 1)
    q32 = rng.standard_normal((int(q_start[-1]), c.n_q_heads, c.head_dim), dtype=np.float32)
    q = _bf16_bits(q32) if c.kv_dtype == "bf16" else q32.astype(np.float16)
    return q, q_start


def prefill_flops(seq_lens, q_start, n_q_heads: int, head_dim: int) -> int:
    """Algorithmic flops of a prefill step: for every chunk row and query head, 2 D flops
    per visible token for q . k and 2 D for the weighted sum of V; row i of a chunk of C_b
    sees L_b - C_b + i + 1 tokens."""
    total = 0
    for b in range(len(seq_lens)):
        n = int(seq_lens[b])
        c = int(q_start[b + 1] - q_start[b])
        total += c * (n - c) + c * (c + 1) // 2
    return total * n_q_heads * 4 * head_dim


def _bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Draw bf16 values: keep the upper 16 bits of each fp32 word (uint16 patterns)."""
    return (np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _finite_e4m3_codes(rng, shape) -> np.ndarray:
    """Codes uniform over the 254 finite E4M3 codes (0x7F and 0xFF are NaN)."""
    u = rng.integers(0, 254, size=shape, dtype=np.int16)
    return (u + (u >= 0x7F)).astype(np.uint8)


def _draw_layout(c: Config, rng, seq_lens=None, extra_pages: int = 0):
    """The first draws of a workload: lengths, then the page permutation behind the block
    table. Returns (seq_lens, block_table, pages in use, pages in the pool)."""
    bs = c.block_size
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
    return lens, table, n_used, n_pages


def layout(config: Config, seed: Optional[int] = None):
    """(seq_lens, block_table, num_pages) of the workload generate(config, seed) draws,
    without drawing its tensors."""
    seed = 1000 + config.index if seed is None else int(seed)
    lens, table, _, n_pages = _draw_layout(config, np.random.default_rng(seed))
    return lens, table, n_pages


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
    lens, table, n_used, n_pages = _draw_layout(c, rng, seq_lens, extra_pages)

    q = rng.standard_normal((c.batch, c.n_q_heads, d), dtype=np.float32)
    q = _bf16_bits(q) if c.kv_dtype == "bf16" else q.astype(np.float16)
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
    elif c.kv_dtype == "bf16":
        k_pages = _bf16_bits(rng.standard_normal(shape, dtype=np.float32))
        v_pages = _bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    elif c.kv_dtype == "fp8":
        k_pages = _finite_e4m3_codes(rng, shape)
        v_pages = _finite_e4m3_codes(rng, shape)
        k_scale = (rng.uniform(0.005, 0.02, size=shape[:3]) * (127 / 448)).astype(np.float32)
        v_scale = (rng.uniform(0.005, 0.02, size=shape[:3]) * (127 / 448)).astype(np.float32)
    else:
        raise ValueError(f"unknown kv_dtype {c.kv_dtype!r}")

    w = Workload(c, seed, q, k_pages, v_pages, k_scale, v_scale, table, lens,
                 c.softmax_scale)
    if poison:
        _poison_unused_slots(w, n_used)
    return w
