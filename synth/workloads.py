"""Workload shapes and seeded generators for the paged-attention hot path.

Recipe (the same for every workload, stated once):

* Seed: the course notebook's demo seed 20260801 ("Module 10 project-exercise
  demo", setup cell). Workload number ``i`` draws from
  ``numpy.random.default_rng(SEED + i)``.
* Draw order from that generator: first the free-stack permutation of the
  pool's physical block ids, then (variable-length workload only) the context
  lengths, then a 64-bit seed root from which the value streams are spawned.
* Values: standard normal, drawn in float32 by numpy (``standard_normal`` with
  ``dtype=float32``), one independent spawned stream per tensor and per chunk
  so that large tensors can be filled by several threads and still be
  reproducible. fp32 workloads use the draws as they are; bf16 workloads round
  them to nearest-even with ``torch.Tensor.to(torch.bfloat16)``.

Nothing here computes slots, block tables, cache contents or attention.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Sequence

import numpy as np

SEED = 20260801

# Bytes per element of the floating-point cache dtypes.
DTYPE_BYTES = {"f32": 4, "bf16": 2}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: the attention-layer geometry and batch shape."""

    index: int  # 1-based workload number; seeds the generator
    name: str
    dtype: str  # "f32" or "bf16"
    q_heads: int
    kv_heads: int
    head_dim: int
    block_size: int
    batch: int
    num_blocks: int  # physical blocks in the pool
    queries_per_seq: int = 1  # 1 = decode; K = speculative verify
    context: int | None = None  # equal context length for every sequence
    lengths: tuple[int, ...] | None = None  # explicit lengths (tiny workload)
    lognormal_median: float | None = None  # variable-length workload
    lognormal_sigma: float | None = None
    length_clip: tuple[int, int] | None = None
    partition_tokens: int = 0  # 0 = library's choice; -1 = balanced stream
    shared_prefix: int = 0  # prefix-sharing workload: tokens shared by all
    unique_suffix: int = 0  # prefix-sharing workload: private tokens per seq
    cache_write_in_step: bool = True
    # 8 or 3: the cache holds 8-bit (int8) or 3-bit (two per byte) per-row
    # codes with a float32 scale per row, written from `dtype` rows; 0: the
    # cache holds `dtype` itself
    kv_codes: int = 0

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def esize(self) -> int:
        return DTYPE_BYTES[self.dtype]

    @property
    def rng_seed(self) -> int:
        return SEED + self.index


WORKLOADS = {
    "tiny_f32": Workload(
        index=1, name="tiny_f32", dtype="f32", q_heads=4, kv_heads=2,
        head_dim=64, block_size=16, batch=4, num_blocks=16,
        lengths=(6, 9, 17, 33)),
    "llama3_8b_b32_8k": Workload(
        index=2, name="llama3_8b_b32_8k", dtype="bf16", q_heads=32,
        kv_heads=8, head_dim=128, block_size=16, batch=32, num_blocks=16384,
        context=8192),
    "llama3_8b_varlen_b256": Workload(
        index=3, name="llama3_8b_varlen_b256", dtype="bf16", q_heads=32,
        kv_heads=8, head_dim=128, block_size=16, batch=256, num_blocks=32768,
        lognormal_median=1024.0, lognormal_sigma=1.0, length_clip=(16, 8192),
        partition_tokens=-1),
    "llama33_70b_b4_128k": Workload(
        index=4, name="llama33_70b_b4_128k", dtype="bf16", q_heads=64,
        kv_heads=8, head_dim=128, block_size=16, batch=4, num_blocks=32768,
        context=131072, partition_tokens=512),
    "prefix_share_verify_k4": Workload(
        index=5, name="prefix_share_verify_k4", dtype="bf16", q_heads=32,
        kv_heads=8, head_dim=128, block_size=16, batch=64, num_blocks=4096,
        queries_per_seq=4, shared_prefix=2048, unique_suffix=512),
    # the 8K decode batch over a cache of 8-bit per-row codes
    "llama3_8b_b32_8k_q8": Workload(
        index=7, name="llama3_8b_b32_8k_q8", dtype="bf16", q_heads=32,
        kv_heads=8, head_dim=128, block_size=16, batch=32, num_blocks=16384,
        context=8192, kv_codes=8),
    # ... and over 3-bit codes (the notebook's 16 -> 3 bit storage scenario)
    "llama3_8b_b32_8k_q3": Workload(
        index=8, name="llama3_8b_b32_8k_q3", dtype="bf16", q_heads=32,
        kv_heads=8, head_dim=128, block_size=16, batch=32, num_blocks=16384,
        context=8192, kv_codes=3),
    # the variable-length batch over 8-bit codes (same seed, so the same
    # lengths and placement as the bf16 batch)
    "llama3_8b_varlen_b256_q8": Workload(
        index=3, name="llama3_8b_varlen_b256_q8", dtype="bf16", q_heads=32,
        kv_heads=8, head_dim=128, block_size=16, batch=256, num_blocks=32768,
        lognormal_median=1024.0, lognormal_sigma=1.0, length_clip=(16, 8192),
        partition_tokens=-1, kv_codes=8),
    # chunked prefill: each sequence's last 512-token prompt chunk over its
    # 7680 cached tokens (the notebook's 16 chunks of 512 for an 8K prompt)
    "llama3_8b_chunk512_b4_8k": Workload(
        index=6, name="llama3_8b_chunk512_b4_8k", dtype="bf16", q_heads=32,
        kv_heads=8, head_dim=128, block_size=16, batch=4, num_blocks=2560,
        queries_per_seq=512, context=8192),
}


def free_stack_permutation(rng: np.random.Generator, num_blocks: int) -> np.ndarray:
    """A seeded permutation of block ids, used as the pool's initial free stack."""
    return rng.permutation(num_blocks).astype(np.int32)


def draw_lengths(rng: np.random.Generator, w: Workload) -> np.ndarray:
    """Context lengths for a workload (after the permutation has been drawn).

    Variable-length workload: log-normal in natural-log space around the
    median, rounded to the nearest integer, clipped, and nudged off multiples
    of the block size so that every last block is partial.
    """
    if w.lengths is not None:
        return np.asarray(w.lengths, dtype=np.int32)
    if w.context is not None:
        return np.full(w.batch, w.context, dtype=np.int32)
    if w.lognormal_median is not None:
        lo, hi = w.length_clip
        raw = rng.normal(np.log(w.lognormal_median), w.lognormal_sigma, size=w.batch)
        lens = np.clip(np.rint(np.exp(raw)), lo, hi).astype(np.int64)
        on_boundary = lens % w.block_size == 0
        lens = np.where(on_boundary, np.where(lens >= hi, hi - 1, lens + 1), lens)
        return lens.astype(np.int32)
    if w.shared_prefix:
        return np.full(w.batch, w.shared_prefix + w.unique_suffix, dtype=np.int32)
    raise ValueError("workload has no length rule")


def _fill(seed_seq: np.random.SeedSequence, out: np.ndarray) -> None:
    rng = np.random.default_rng(seed_seq)
    rng.standard_normal(out.shape, dtype=np.float32, out=out)


def normal_array(root_seed: int, stream: int, shape: Sequence[int],
                 chunk_elems: int = 1 << 24, threads: int | None = None) -> np.ndarray:
    """Standard-normal float32 array of ``shape`` from stream ``stream``.

    The array is filled in chunks of ``chunk_elems`` along the flattened
    order, chunk ``c`` from ``SeedSequence(root_seed, spawn_key=(stream, c))``,
    so the result does not depend on how many threads fill it.
    """
    total = int(np.prod(shape)) if len(shape) else 1
    flat = np.empty(total, dtype=np.float32)
    n_chunks = max(1, (total + chunk_elems - 1) // chunk_elems)
    jobs = []
    for c in range(n_chunks):
        lo, hi = c * chunk_elems, min(total, (c + 1) * chunk_elems)
        ss = np.random.SeedSequence(root_seed, spawn_key=(stream, c))
        jobs.append((ss, flat[lo:hi]))
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if n_chunks == 1 or threads <= 1:
        for ss, view in jobs:
            _fill(ss, view)
    else:
        with concurrent.futures.ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda j: _fill(*j), jobs))
    return flat.reshape(shape)


def cast(x: np.ndarray, dtype: str):
    """Round float32 draws to the workload dtype; returns a CPU torch tensor."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "f32":
        return t.clone()
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError(f"unsupported dtype {dtype!r}")


def root_seed(rng: np.random.Generator) -> int:
    """Draw the 64-bit root from which value streams are spawned."""
    return int(rng.integers(0, 2**63 - 1, dtype=np.int64))
