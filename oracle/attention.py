"""Float64 oracle for the paged cache write and paged attention (test only).

What is computed, stated from the pages:

* Cache write ([NeuralOps] "Block Table", continuous-batching "slot
  mapping"): token t of a step carries a slot s; its key and value rows for
  every KV head land at physical block s // bs, offset s % bs. A slot of -1
  means "no write".

* Attention ([vLLM abstract]: attention over K/V kept in non-contiguous
  blocks; [KVNB demo] Demo 2 ``attention``: logits q.k scaled, the row
  maximum subtracted, exponentiated, normalised, then the weighted sum of
  values). For sequence b with context length L (the cache already holds
  this step's tokens), query index i of nq, and query head h:

  - the query sees n = L - nq + i + 1 keys ([KVNB §2] FLOP model: query j of
    a causal suffix sees cached_prefix + j + 1 keys; one decode query sees
    all L keys, itself included);
  - key/value t comes from block ``table[b][t // bs]`` at offset ``t % bs``
    and KV head g = h // (Hq / Hkv) (contiguous head groups);
  - s_t = sigma * sum_d q[d] k_t[d] with sigma the float32 scale widened to
    float64; m = max s_t; p_t = exp(s_t - m); l = sum p_t;
    out = sum p_t v_t / l; lse = m + ln l.

Every value is read in its storage dtype and widened exactly to float64.
The walk goes token by token through the block table, as the method does.

Split-K (long contexts): partition p covers logical tokens [pP, (p+1)P) of
the visible range and keeps (m_p, l_p, acc_p) with acc_p unnormalised; the
merge takes M = max m_p and returns sum e^(m_p-M) acc_p / sum e^(m_p-M) l_p.
The pages name only a "log-sum-exp merge"; this is its plainest form.
"""

from __future__ import annotations

import math

import numpy as np


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored elements.

    ``dtype`` "f32": ``x`` is float32. ``dtype`` "bf16": ``x`` holds the raw
    16-bit patterns (uint16 or int16); a bfloat16 number is the float32 whose
    upper 16 bits are these and whose lower 16 bits are zero.
    """
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x).view(np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f64":  # values already exact (e.g. a dequantized code pool)
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unsupported dtype {dtype!r}")


def cache_write(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray,
                v_new: np.ndarray, slots, block_size: int) -> None:
    """Scatter new rows into the pool in place.

    k_pool, v_pool: [num_blocks, Hkv, bs, D]; k_new, v_new: [T, Hkv, D];
    slots: T ints, -1 = skip. Element values are moved, never converted.
    """
    nb = k_pool.shape[0]
    for t, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        blk, off = divmod(s, block_size)
        if blk >= nb:
            raise IndexError("slot outside the pool")
        k_pool[blk, :, off, :] = k_new[t]
        v_pool[blk, :, off, :] = v_new[t]


def attend_row(q: np.ndarray, k_pool64: np.ndarray, v_pool64: np.ndarray,
               table, n: int, g: int, block_size: int, sigma: float):
    """One query row over its first ``n`` keys; returns (out, lse, p)."""
    if n <= 0:
        raise ValueError("a query must see at least one key")
    scores = []
    values = []
    for t in range(n):
        blk = int(table[t // block_size])
        off = t % block_size
        k_t = k_pool64[blk, g, off]
        scores.append(sigma * float(np.dot(q, k_t)))
        values.append(v_pool64[blk, g, off])
    m = max(scores)
    p = np.array([math.exp(s - m) for s in scores])
    l = float(p.sum())
    out = (p[:, None] * np.stack(values)).sum(axis=0) / l
    return out, m + math.log(l), p / l


def attention(q: np.ndarray, q_dtype: str, k_pool: np.ndarray,
              v_pool: np.ndarray, kv_dtype: str, block_tables, context_lens,
              scale: float, block_size: int):
    """Paged attention for a batch.

    q: [B, nq, Hq, D] in ``q_dtype`` storage; pools: [NB, Hkv, bs, D] in
    ``kv_dtype`` storage; block_tables: [B][>= ceil(L/bs)] ints;
    context_lens: [B]. Returns (out [B, nq, Hq, D], lse [B, nq, Hq]) float64.
    """
    B, nq, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    group = Hq // Hkv
    q64 = widen(q, q_dtype)
    k64 = widen(k_pool, kv_dtype)
    v64 = widen(v_pool, kv_dtype)
    sigma = float(np.float32(scale))
    out = np.zeros((B, nq, Hq, D))
    lse = np.zeros((B, nq, Hq))
    for b in range(B):
        L = int(context_lens[b])
        for i in range(nq):
            n = L - nq + i + 1
            for h in range(Hq):
                o, s, _ = attend_row(q64[b, i, h], k64, v64, block_tables[b], n,
                                     h // group, block_size, sigma)
                out[b, i, h] = o
                lse[b, i, h] = s
    return out, lse


def attention_weights(q_row: np.ndarray, q_dtype: str, k_pool, v_pool,
                      kv_dtype: str, table, n: int, g: int, scale: float,
                      block_size: int) -> np.ndarray:
    """The softmax weights p_t / l of one query row (for invariant checks)."""
    sigma = float(np.float32(scale))
    _, _, w = attend_row(widen(q_row, q_dtype), widen(k_pool, kv_dtype),
                         widen(v_pool, kv_dtype), table, n, g, block_size, sigma)
    return w


def partition_partials(q_row64: np.ndarray, k_pool64, v_pool64, table, n: int,
                       g: int, block_size: int, sigma: float, part: int):
    """Unnormalised (m_p, l_p, acc_p) for each partition of ``part`` tokens."""
    parts = []
    for start in range(0, n, part):
        stop = min(n, start + part)
        scores, values = [], []
        for t in range(start, stop):
            blk = int(table[t // block_size])
            off = t % block_size
            scores.append(sigma * float(np.dot(q_row64, k_pool64[blk, g, off])))
            values.append(v_pool64[blk, g, off])
        m = max(scores)
        p = np.array([math.exp(s - m) for s in scores])
        acc = (p[:, None] * np.stack(values)).sum(axis=0)
        parts.append((m, float(p.sum()), acc))
    return parts


def merge_partials(parts):
    """Log-sum-exp merge of partition partials; returns (out, lse)."""
    M = max(m for m, _, _ in parts)
    w = [math.exp(m - M) for m, _, _ in parts]
    num = sum(wi * acc for wi, (_, _, acc) in zip(w, parts))
    den = sum(wi * l for wi, (_, l, _) in zip(w, parts))
    return num / den, M + math.log(den)
