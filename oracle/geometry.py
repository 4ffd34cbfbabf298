"""Payload, FLOP and waste counts from [KVNB §1, §2, §6] (test only).

* K+V bytes per token: 2 (K and V) * attention layers * KV heads * head dim
  * bytes per element ([KVNB §1] "Typed KV geometry and units").
* Payload of a batch: bytes per token * tokens * batch * scale, which must be
  a whole number of bytes ([KVNB §1] ``kv_payload_bytes``).
* Attention FLOPs (QK and AV, two per multiply-add) for ``queries`` causal
  suffix queries after ``cached_prefix`` keys: 4 * layers * Hq * D * pairs,
  pairs = queries * prefix + queries (queries + 1) / 2 ([KVNB §2]).
* Expected paged waste with a uniform remainder: ((bs-1)/2) / (avg +
  (bs-1)/2); naive reservation waste: (max - used) / max ([KVNB §6]).
"""

from __future__ import annotations

import math


def bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    for v in (layers, kv_heads, head_dim, elem_bytes):
        if isinstance(v, bool) or not isinstance(v, int) or v <= 0:
            raise ValueError("geometry sizes must be positive integers")
    return 2 * layers * kv_heads * head_dim * elem_bytes


def kv_payload_bytes(per_token: int, tokens: int, batch: int = 1, scale: float = 1.0) -> int:
    if isinstance(tokens, bool) or not isinstance(tokens, int) or tokens < 0:
        raise ValueError("tokens must be a non-negative integer")
    if isinstance(batch, bool) or not isinstance(batch, int) or batch <= 0:
        raise ValueError("batch must be a positive integer")
    if not math.isfinite(scale) or scale <= 0:
        raise ValueError("scale must be positive and finite")
    raw = per_token * tokens * batch * scale
    if abs(raw - round(raw)) > 1e-9:
        raise ValueError("scaled payload is not a whole number of bytes")
    return int(round(raw))


def attention_flops(layers: int, q_heads: int, head_dim: int, queries: int,
                    cached_prefix: int = 0) -> int:
    for v in (layers, q_heads, head_dim, queries, cached_prefix):
        if isinstance(v, bool) or not isinstance(v, int) or v < 0:
            raise ValueError("counts must be non-negative integers")
    if min(layers, q_heads, head_dim) == 0:
        raise ValueError("attention geometry must be positive")
    pairs = queries * cached_prefix + queries * (queries + 1) // 2
    return 4 * layers * q_heads * head_dim * pairs


def expected_paged_waste(avg_tokens: int, block_size: int) -> float:
    tail = (block_size - 1) / 2
    return tail / (avg_tokens + tail)


def naive_preallocation_waste(max_tokens: int, used_tokens: int) -> float:
    if used_tokens > max_tokens:
        raise ValueError("used exceeds maximum")
    return (max_tokens - used_tokens) / max_tokens
