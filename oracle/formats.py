"""Plain decoders for the 16-bit and 8-bit floating-point KV storage formats.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: nothing on the product
path imports it. It shares no code with the HIP library.

Where the pages name the formats, and the readings taken:

* BF16 (xLLM README, optimisation list, quantisation: "FP16, BF16" are the
  supported precisions). The pages do not define it; the reading is the usual
  one: a bf16 number is the upper half of an IEEE-754 binary32 (1 sign bit,
  8 exponent bits with bias 127, 7 fraction bits), so its value is that of the
  binary32 whose low 16 bits are zero. Arrays hold the raw bit patterns as
  uint16 (numpy has no bf16 type).
* FP8 (page "Eine LLM-Inferenz-Engine von Grund auf mit C++ und CUDA bauen",
  section 4: stronger quantisation of the cache with FP8 among the next
  steps). The pages name no FP8 encoding; the reading is E4M3 as the OCP 8-bit
  floating-point specification defines it (the "fn" variant): 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
  subnormals m/8 * 2^-6; the all-ones pattern S.1111.111 is NaN; there are no
  infinities, and the largest finite magnitude is 1.75 * 2^8 = 448. A row of
  an FP8 cache carries one fp32 scale, as a per-row INT8 row does (xLLM
  README, quantisation), so a stored value is decode(code) * scale. Arrays hold
  the raw codes as uint8.

Pinned by ``tests/test_oracle_formats.py``.
"""

from __future__ import annotations

import numpy as np

__all__ = ["bf16_to_float64", "e4m3_to_float64", "e4m3_from_float32", "element_values"]


def bf16_to_float64(bits: np.ndarray) -> np.ndarray:
    """Value of each bf16 bit pattern (uint16), exactly, as float64."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("bf16 values are passed as their uint16 bit patterns")
    widened = bits.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):       # signalling-NaN patterns widen to NaN
        return widened.view(np.float32).astype(np.float64)


def e4m3_to_float64(codes: np.ndarray) -> np.ndarray:
    """Value of each OCP E4M3 code (uint8), exactly, as float64; NaN for the
    two NaN codes."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("E4M3 values are passed as their uint8 codes")
    c = codes.astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exponent = (c >> 3) & 0xF
    mantissa = (c & 0x7).astype(np.float64)
    normal = (1.0 + mantissa / 8.0) * np.exp2(exponent.astype(np.float64) - 7.0)
    subnormal = (mantissa / 8.0) * 2.0 ** -6
    magnitude = np.where(exponent == 0, subnormal, normal)
    magnitude = np.where((exponent == 0xF) & ((c & 0x7) == 0x7), np.nan, magnitude)
    return sign * magnitude


def e4m3_from_float32(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code to each fp32 value, ties to the even code (even last mantissa
    bit), the sign kept (so -0.0 gives 0x80). Magnitudes above 448 saturate to 448: the
    pages fix no overflow rule, and the quantiser below never produces one. NaN is not
    accepted."""
    v = np.asarray(v, dtype=np.float32)
    if np.isnan(v).any():
        raise ValueError("NaN has no E4M3 code here")
    grid = e4m3_to_float64(np.arange(0x7F, dtype=np.uint8))   # codes 0..126, increasing
    a = np.abs(v.astype(np.float64))
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_hi, d_lo = np.abs(grid[hi] - a), np.abs(a - grid[lo])
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


def element_values(x: np.ndarray) -> np.ndarray:
    """Float64 values of stored elements, by storage type: fp16/fp32/fp64 and int8 as
    they are, uint16 as bf16 bit patterns, uint8 as E4M3 codes."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_float64(x)
    if x.dtype == np.uint8:
        return e4m3_to_float64(x)
    if x.dtype in (np.float16, np.float32, np.float64, np.int8):
        return x.astype(np.float64)
    raise TypeError(f"unsupported storage type {x.dtype}")
