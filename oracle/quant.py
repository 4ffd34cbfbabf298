"""Per-row integer codes for paged K/V (test infrastructure only).

What is computed, restated from the course page "Module 10. KV Caches and
Efficient Inference", project-exercise demo, Demo 2 (the teaching quantizer:
symmetric integer codes with one scale per row):

* for a row x of D values and a bit width `bits`, the largest code is
  limit = 2^(bits-1) - 1; the row's scale is max |x| / limit, or 1 for a
  row of zeros; each code is x / scale rounded to the nearest integer (ties
  to even, as numpy's rint) and clipped to [-limit, limit]; the row is
  reconstructed as code * scale.
* The page computes in float64; so does this module. The stored scale is
  float32 (the demo counts 4 bytes per scale), and a dequantized element is
  code * (that float32 scale widened to float64).

A paged cache in this format holds, per (block, KV head, slot), the D int8
codes of one token's K (or V) row and its float32 scale: codes
[num_blocks, Hkv, bs, D] int8, scales [num_blocks, Hkv, bs] float32.
"""

from __future__ import annotations

import numpy as np


def quantize_rows(x: np.ndarray, bits: int):
    """(codes int8, scale float64) of each row of x (last axis), as the page's
    quantizer: scale = max|x| / (2^(bits-1) - 1), 1 for all-zero rows."""
    if not 2 <= bits <= 8:
        raise ValueError("bits must be in [2, 8]")
    x = np.asarray(x, dtype=np.float64)
    limit = 2 ** (bits - 1) - 1
    scale = np.max(np.abs(x), axis=-1, keepdims=True) / limit
    scale = np.where(scale == 0, 1.0, scale)
    codes = np.clip(np.rint(x / scale), -limit, limit).astype(np.int8)
    return codes, scale[..., 0]


def fake_quantize_rows(x: np.ndarray, bits: int) -> np.ndarray:
    """The page's round trip: codes times scale, in float64."""
    codes, scale = quantize_rows(x, bits)
    return codes.astype(np.float64) * scale[..., None]


def cache_write_q(k_codes, v_codes, k_scales, v_scales, k_new64, v_new64, slots,
                  block_size: int, bits: int = 8) -> None:
    """Quantize each new (token, KV head) row and scatter codes and float32
    scales to the token's slot (slot -1: no write), in place.

    k_new64, v_new64: [T, Hkv, D] float64 (the new rows, widened exactly)."""
    kc, ks = quantize_rows(k_new64, bits)
    vc, vs = quantize_rows(v_new64, bits)
    for t, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        blk, off = divmod(s, block_size)
        k_codes[blk, :, off, :] = kc[t]
        v_codes[blk, :, off, :] = vc[t]
        k_scales[blk, :, off] = ks[t].astype(np.float32)
        v_scales[blk, :, off] = vs[t].astype(np.float32)


def dequantize_pool(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Float64 pool [num_blocks, Hkv, bs, D]: code * float32 scale."""
    return codes.astype(np.float64) * np.asarray(scales, np.float32).astype(np.float64)[..., None]
