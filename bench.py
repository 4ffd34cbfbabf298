#!/usr/bin/env python3
"""Paged-attention decode benchmark on one MI355X.

Default workload: one attention layer of Llama-3-8B geometry (32 query heads,
8 KV heads, head dim 128, bf16 K/V, 16-token blocks), 32 sequences at context
8192, one decode token each, physical blocks placed by a seeded permutation of
a 16384-block pool.

A step is the whole hot path for one batch: the slot-mapped cache write of
each sequence's new K/V token, then paged attention over all 8192 tokens
(one partition-kernel launch; when the launch plan splits contexts into
partitions, a log-sum-exp reduce launch follows). The host allocator ran before the
timed region (its cost is reported separately) and the block tables are
already resident in HBM.

Prints ONE JSON line. ``value`` is decode tokens/s (one token per sequence
per step) for the one GPU; ``roofline`` reports the attention call's achieved
HBM bandwidth from its algorithmic bytes and its event-timed duration;
``cpu_baseline`` times the float64 C oracle on the host cores.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, decimal GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
def kernel_sources(workload: str) -> list:
    """The sources whose code a workload's dominant kernel is built from: the
    bf16/fp32 partition kernel, or the matrix-core kernel over code caches."""
    from synth.workloads import WORKLOADS

    csrc = "paged_kv_cache_202_amd/csrc/"
    w = WORKLOADS[workload]
    if w.dtype == "bf16" and w.group * w.queries_per_seq > 16 and not w.shared_prefix:
        # the chunked-prefill row-tile kernel
        return [csrc + "decode_kernel.h", csrc + "verify_mfma.h", csrc + "shared_prefix.h",
                csrc + "shared_inst.hip", csrc + "decode.hip"]
    if w.shared_prefix:  # the one-pass shared-prefix kernel
        return [csrc + "decode_kernel.h", csrc + "verify_mfma.h", csrc + "shared_prefix.h",
                csrc + "group_decode.h", csrc + "shared_inst.hip", csrc + "decode.hip"]
    if w.kv_codes or mfma_decode(w.dtype, w.queries_per_seq, w.head_dim, w.partition_tokens):
        return [csrc + "decode_kernel.h", csrc + "verify_mfma.h", csrc + "decode_mfma.h",
                csrc + "decode_inst_mfma_d128.hip", csrc + "decode.hip"]
    return [csrc + "decode_kernel.h", csrc + "decode_inst_bf16_d128.hip", csrc + "decode.hip"]


def mfma_decode(dtype: str, nq: int, D: int, part: int) -> bool:
    """Whether the library plans a bf16 attention call on the MFMA decode
    kernel: one query token, head dim up to 128 (the stream plan,
    partition_tokens = -1, runs it in stream mode)."""
    return dtype == "bf16" and nq == 1 and D <= 128


def sources_sha256(workload: str) -> str:
    import hashlib

    h = hashlib.sha256()
    for src in kernel_sources(workload):
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profile_path(workload: str) -> str:
    """The committed counter summary of a workload's attention call, named for
    its dominant kernel."""
    from synth.workloads import WORKLOADS

    w = WORKLOADS[workload]
    if w.shared_prefix:
        kernel = "group_mfma_kernel"
    elif w.dtype == "bf16" and w.group * w.queries_per_seq > 16:  # a prefill chunk
        kernel = "chunk_mfma_kernel"
    else:
        kernel = "decode"
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}.json")


def prefix_unique_bytes(w) -> int:
    """Minimum bytes of one shared-prefix attention call: the shared prefix's
    K/V once per KV head, each sequence's private tokens (suffix and drafts)
    once, q read, fp32 out written, tables and lengths read."""
    B, nq = w.batch, w.queries_per_seq
    L = w.shared_prefix + w.unique_suffix + nq
    lens = np.full(B, L, dtype=np.int64)
    logical = algorithmic_bytes(B, nq, w.q_heads, w.kv_heads, w.head_dim, w.esize, lens,
                                -(-L // w.block_size))
    kv_logical = 2 * w.kv_heads * w.head_dim * w.esize * int(lens.sum())
    kv_unique = 2 * w.kv_heads * w.head_dim * w.esize * (w.shared_prefix + B * (L - w.shared_prefix))
    return logical - kv_logical + kv_unique


def profiled_traffic(workload: str):
    """HBM bytes per attention call from the committed rocprofv3 counter summary,
    or None when there is none or the kernel sources changed since it was taken."""
    path = profile_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    if sources_sha256(workload) != prof.get("kernel_sources_sha256"):
        return None
    return prof["traffic_bytes_per_launch"]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(B, nq, Hq, Hkv, D, es, lens, max_blocks, with_lse=False,
                      kv_row_bytes=None):
    """Bytes the attention call must move at minimum: every visible K and V
    element once per KV head, q read, fp32 out written, block-table entries
    and context lengths read. kv_row_bytes: bytes of one token's K (or V)
    row of one KV head, when it is not D * es (8-bit codes: D + 4)."""
    row = D * es if kv_row_bytes is None else kv_row_bytes
    kv = 2 * Hkv * row * int(np.sum(lens))
    q = B * nq * Hq * D * es
    out = B * nq * Hq * D * 4 + (B * nq * Hq * 4 if with_lse else 0)
    tables = 4 * int(np.sum(-(-np.asarray(lens) // 16)))
    return kv + q + out + tables + 4 * B


def is_chunk(wk) -> bool:
    """More than one 16-row tile of query rows per KV head: chunked prefill."""
    return wk.w.dtype == "bf16" and wk.Hq // wk.Hkv * wk.nq > 16


def chunk_flops(B, nq, Hq, D, lens) -> int:
    """Multiply-adds of a causal chunk call, counted as 2 FLOPs each: every
    row does q.k and p.v (2 D each) for each key it sees."""
    seen = 0
    for L in np.asarray(lens, dtype=np.int64):
        seen += int(np.sum(L - nq + np.arange(nq) + 1))
    return 4 * D * Hq * seen


def kernel_label(wk) -> str:
    """Which launches one attention call makes, as the library plans them."""
    tail = " + reduce_partitions_kernel" if wk.ws is not None else " (one launch per attention call)"
    if getattr(wk, "q8", False):
        kind = "int8" if wk.w.kv_codes == 8 else "3-bit"
        if wk.part == -1:
            return f"decode_mfma_kernel<{kind} codes> stream mode + reduce_stream_kernel"
        return f"decode_mfma_kernel<{kind} codes>" + tail
    if is_chunk(wk):
        return "chunk_mfma_kernel + reduce_partitions_kernel"
    mfma = wk.w.dtype == "bf16" and wk.nq > 1 and wk.Hq // wk.Hkv * wk.nq <= 16
    if getattr(wk, "share", False) and wk.groups.n_groups:
        return ("prefix_mfma_kernel + " + ("verify_mfma_kernel" if mfma else
                                           "decode_partition_kernel") +
                " + reduce_partitions_kernel")
    if wk.part == -1 and mfma_decode(wk.w.dtype, wk.nq, wk.D, wk.part):
        return "decode_mfma_kernel<bf16> stream mode + reduce_stream_kernel"
    if wk.part == -1 and not mfma:
        return "decode_stream_kernel + reduce_stream_kernel"
    if mfma_decode(wk.w.dtype, wk.nq, wk.D, wk.part):
        return "decode_mfma_kernel<bf16>" + tail
    main = "verify_mfma_kernel" if mfma else "decode_partition_kernel"
    return main + tail


class Workload:
    """Device state for one workload, built through the library only."""

    def __init__(self, name: str, rotate: int, device):
        import torch

        import paged_kv_cache_202_amd as pkv
        from synth import workloads as wl

        self.w = w = wl.WORKLOADS[name]
        self.torch, self.pkv = torch, pkv
        rng = np.random.default_rng(w.rng_seed)
        stack = wl.free_stack_permutation(rng, w.num_blocks)
        lens = wl.draw_lengths(rng, w)
        root = wl.root_seed(rng)
        self.stack, self.lens, self.root = stack, lens, root
        B, Hq, Hkv, D, bs, nq = w.batch, w.q_heads, w.kv_heads, w.head_dim, w.block_size, \
            w.queries_per_seq
        self.B, self.Hq, self.Hkv, self.D, self.bs, self.nq = B, Hq, Hkv, D, bs, nq
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.es = w.esize
        # context tokens cached before the step, then nq new tokens per sequence
        pre = lens - nq
        t0 = time.perf_counter()
        T = int(lens.sum())
        k_all = wl.cast(wl.normal_array(root, 0, (T, Hkv, D)), w.dtype)
        v_all = wl.cast(wl.normal_array(root, 1, (T, Hkv, D)), w.dtype)
        q = wl.cast(wl.normal_array(root, 2, (B, nq, Hq, D)), w.dtype)
        log(f"[bench] generated {T} tokens of K/V in {time.perf_counter() - t0:.1f}s")
        self.host_k, self.host_v, self.host_q = k_all, v_all, q
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
        pre_idx = np.concatenate([np.arange(s, s + n) for s, n in zip(starts, pre)])
        new_idx = np.concatenate([np.arange(s + n, s + n + nq) for s, n in zip(starts, pre)])

        pool = pkv.PagedKVPool(w.num_blocks, bs, stack)
        ids = list(range(B))
        for b in ids:
            pool.seq_create(b)
        t0 = time.perf_counter()
        pre_slots, cow = pool.alloc_batch(ids, pre.tolist())
        self.alloc_prefill_s = time.perf_counter() - t0
        t0 = time.perf_counter()
        step_slots, cow2 = pool.alloc_batch(ids, [nq] * B)
        self.alloc_step_s = time.perf_counter() - t0
        assert cow.shape[0] == 0 and cow2.shape[0] == 0
        self.max_blocks = int(max(-(-lens // bs)))
        tables, clens = pool.block_tables(ids, self.max_blocks)
        assert np.array_equal(clens, lens)
        self.pool = pool
        self.pre_slots, self.step_slots = pre_slots, step_slots
        dev = device
        shape = (w.num_blocks, Hkv, bs, D)
        self.q8 = w.kv_codes in (8, 3)  # a cache of per-row codes
        if self.q8:
            cls = pkv.Q8Cache if w.kv_codes == 8 else pkv.Q3Cache
            self.qc = [cls(w.num_blocks, Hkv, bs, D, dev) for _ in range(rotate)]
            self.write_q = (pkv.paged_cache_write_q8 if w.kv_codes == 8
                            else pkv.paged_cache_write_q3)
            self.decode_q = (pkv.paged_attention_decode_q8 if w.kv_codes == 8
                             else pkv.paged_attention_decode_q3)
        else:
            self.kc = [torch.empty(shape, dtype=tdt, device=dev) for _ in range(rotate)]
            self.vc = [torch.empty(shape, dtype=tdt, device=dev) for _ in range(rotate)]
        kpre = k_all[torch.from_numpy(pre_idx)].to(dev)
        vpre = v_all[torch.from_numpy(pre_idx)].to(dev)
        d_pre_slots = torch.from_numpy(pre_slots).to(dev)
        for i in range(rotate):
            if self.q8:
                self.write_q(kpre, vpre, self.qc[i], d_pre_slots)
            else:
                pkv.paged_cache_write(kpre, vpre, self.kc[i], self.vc[i], d_pre_slots)
        del kpre, vpre
        self.k_step = k_all[torch.from_numpy(new_idx)].to(dev)
        self.v_step = v_all[torch.from_numpy(new_idx)].to(dev)
        self.d_step_slots = torch.from_numpy(step_slots).to(dev)
        self.d_tables = torch.from_numpy(tables).to(dev)
        self.d_lens = torch.from_numpy(clens).to(dev)
        self.d_q = q.to(dev)
        self.tables_host = tables
        self.out = torch.empty((B, nq, Hq, D), dtype=torch.float32, device=dev)
        self.lse = None  # an optional [B, nq, Hq] float32 output (the parity tests set it)
        self.scale = 1.0 / math.sqrt(D)
        self.part = w.partition_tokens
        ws = pkv.paged_attention_workspace_size(B, nq, Hq, Hkv, D, self.max_blocks, bs,
                                                self.part)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev) if ws else None
        self.rotate = rotate
        torch.cuda.synchronize()

    def cache_write(self, i: int) -> None:
        r = i % self.rotate
        if self.q8:
            self.write_q(self.k_step, self.v_step, self.qc[r], self.d_step_slots)
            return
        self.pkv.paged_cache_write(self.k_step, self.v_step, self.kc[r], self.vc[r],
                                   self.d_step_slots)

    def attend(self, i: int) -> None:
        r = i % self.rotate
        if self.q8:
            self.decode_q(self.out, self.d_q, self.qc[r], self.d_tables, self.d_lens,
                          self.scale, partition_tokens=self.part, workspace=self.ws,
                          lse=self.lse)
            return
        self.pkv.paged_attention_decode(self.out, self.d_q, self.kc[r], self.vc[r],
                                        self.d_tables, self.d_lens, self.scale,
                                        partition_tokens=self.part, workspace=self.ws,
                                        lse=self.lse)

    def step(self, i: int) -> None:
        self.cache_write(i)
        self.attend(i)

    def attention_bytes(self) -> int:
        if self.q8:  # a code byte (or half a byte) per element and a 4-byte scale per row
            row = self.D + 4 if self.w.kv_codes == 8 else self.D // 2 + 4
            return algorithmic_bytes(self.B, self.nq, self.Hq, self.Hkv, self.D, self.es,
                                     self.lens, self.max_blocks, kv_row_bytes=row)
        return algorithmic_bytes(self.B, self.nq, self.Hq, self.Hkv, self.D, self.es,
                                 self.lens, self.max_blocks)

    def cache_write_bytes(self) -> int:
        return 2 * 2 * self.B * self.nq * self.Hkv * self.D * self.es + 4 * self.B * self.nq


class PrefixVerifyWorkload:
    """Prefix sharing + speculative verify, built through the library only.

    Sequence 0 writes the shared prefix; sequences 1..B-1 fork it (every
    prefix block referenced B times); every sequence then appends its own
    suffix in id order (a shared partial last block is copied on the first
    write into it), and finally its K draft tokens. The timed step is the
    cache write of the B*K draft tokens followed by one multi-query attention
    call (query i of K sees the first L - K + i + 1 tokens).
    """

    def __init__(self, name: str, device, prefix: int | None = None, share: bool = True,
                 rotate: int = 1):
        import torch

        import paged_kv_cache_202_amd as pkv
        from synth import workloads as wl

        self.w = w = wl.WORKLOADS[name]
        self.torch, self.pkv = torch, pkv
        rng = np.random.default_rng(w.rng_seed)
        stack = wl.free_stack_permutation(rng, w.num_blocks)
        root = wl.root_seed(rng)
        self.stack, self.root = stack, root
        B, Hq, Hkv, D, bs, K = w.batch, w.q_heads, w.kv_heads, w.head_dim, w.block_size, \
            w.queries_per_seq
        self.B, self.Hq, self.Hkv, self.D, self.bs, self.nq = B, Hq, Hkv, D, bs, K
        self.prefix = prefix if prefix is not None else w.shared_prefix
        self.suffix = w.unique_suffix
        self.es = w.esize
        tdt = torch.bfloat16
        # values: prefix rows, then per-sequence suffix rows, then draft rows
        self.k_pre = wl.cast(wl.normal_array(root, 0, (self.prefix, Hkv, D)), w.dtype)
        self.v_pre = wl.cast(wl.normal_array(root, 1, (self.prefix, Hkv, D)), w.dtype)
        self.k_suf = wl.cast(wl.normal_array(root, 2, (B * self.suffix, Hkv, D)), w.dtype)
        self.v_suf = wl.cast(wl.normal_array(root, 3, (B * self.suffix, Hkv, D)), w.dtype)
        self.k_dft = wl.cast(wl.normal_array(root, 4, (B * K, Hkv, D)), w.dtype)
        self.v_dft = wl.cast(wl.normal_array(root, 5, (B * K, Hkv, D)), w.dtype)
        self.host_q = wl.cast(wl.normal_array(root, 6, (B, K, Hq, D)), w.dtype)

        pool = pkv.PagedKVPool(w.num_blocks, bs, stack)
        ids = list(range(B))
        pool.seq_create(0)
        self.pre_slots, _ = pool.alloc(0, self.prefix)
        for s in ids[1:]:
            pool.fork(0, s, self.prefix)
        self.suf_slots, self.cow_pairs = pool.alloc_batch(ids, [self.suffix] * B)
        t0 = time.perf_counter()
        self.dft_slots, cow2 = pool.alloc_batch(ids, [K] * B)
        self.alloc_step_s = time.perf_counter() - t0
        assert cow2.shape[0] == 0
        self.pool = pool
        self.lens = np.array([pool.seq_length(s) for s in ids], dtype=np.int32)
        self.max_blocks = int(max(-(-self.lens // bs)))
        tables, clens = pool.block_tables(ids, self.max_blocks)
        self.tables_host = tables
        self.unique_tokens = self.prefix + B * (self.suffix + K)
        dev = device
        shape = (w.num_blocks, Hkv, bs, D)
        self.kc = torch.zeros(shape, dtype=tdt, device=dev)
        self.vc = torch.zeros(shape, dtype=tdt, device=dev)
        pkv.paged_cache_write(self.k_pre.to(dev), self.v_pre.to(dev), self.kc, self.vc,
                              torch.from_numpy(self.pre_slots).to(dev))
        if self.cow_pairs.shape[0]:
            pkv.paged_kv_copy_blocks(self.kc, self.vc, torch.from_numpy(self.cow_pairs).to(dev))
        pkv.paged_cache_write(self.k_suf.to(dev), self.v_suf.to(dev), self.kc, self.vc,
                              torch.from_numpy(self.suf_slots).to(dev))
        self.k_step = self.k_dft.to(dev)
        self.v_step = self.v_dft.to(dev)
        self.d_step_slots = torch.from_numpy(self.dft_slots).to(dev)
        self.d_tables = torch.from_numpy(tables).to(dev)
        self.d_lens = torch.from_numpy(clens).to(dev)
        self.d_q = self.host_q.to(dev)
        self.out = torch.empty((B, K, Hq, D), dtype=torch.float32, device=dev)
        self.lse = None  # an optional [B, K, Hq] float32 output (the parity tests set it)
        self.scale = 1.0 / math.sqrt(D)
        self.part = w.partition_tokens
        ws = pkv.paged_attention_workspace_size(B, K, Hq, Hkv, D, self.max_blocks, bs, self.part)
        # shared prefixes: groups found once from the host tables (they change
        # only on fork or free), each shared block then read once per KV head
        self.share = share
        self.groups_s = 0.0
        if share:
            t0 = time.perf_counter()
            self.groups = pkv.paged_kv_prefix_groups(tables, self.lens, K, bs)
            self.groups_s = time.perf_counter() - t0
            self.d_groups = self.groups.to_device(dev)
            ws = max(ws, pkv.paged_attention_shared_workspace_size(
                B, K, Hq, Hkv, D, self.max_blocks, bs, self.groups, self.part))
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev) if ws else None
        # pool copies used in turn (same contents, same tables): with two, the
        # working sets of successive calls (2 x 150 MB at the C5 sizes) do not
        # fit the 256 MB last-level cache, so repeats are read from HBM
        self.rotate = max(1, rotate)
        self.kcs = [self.kc] + [self.kc.clone() for _ in range(self.rotate - 1)]
        self.vcs = [self.vc] + [self.vc.clone() for _ in range(self.rotate - 1)]
        torch.cuda.synchronize()

    def cache_write(self, i: int) -> None:
        r = i % self.rotate
        self.pkv.paged_cache_write(self.k_step, self.v_step, self.kcs[r], self.vcs[r],
                                   self.d_step_slots)

    def attend(self, i: int) -> None:
        r = i % self.rotate
        if self.share:
            self.pkv.paged_attention_decode_shared(self.out, self.d_q, self.kcs[r], self.vcs[r],
                                                   self.d_tables, self.d_lens, self.scale,
                                                   self.groups, self.d_groups,
                                                   partition_tokens=self.part,
                                                   workspace=self.ws, lse=self.lse)
            return
        self.pkv.paged_attention_decode(self.out, self.d_q, self.kcs[r], self.vcs[r],
                                        self.d_tables, self.d_lens, self.scale,
                                        partition_tokens=self.part, workspace=self.ws,
                                        lse=self.lse)

    def step(self, i: int) -> None:
        self.cache_write(i)
        self.attend(i)

    def attention_bytes(self) -> int:
        """Logical bytes: every sequence's visible K/V once per KV head."""
        return algorithmic_bytes(self.B, self.nq, self.Hq, self.Hkv, self.D, self.es,
                                 self.lens, self.max_blocks)

    def unique_attention_bytes(self) -> int:
        """Bytes with each shared physical block counted once."""
        kv = 2 * self.Hkv * self.D * self.es * self.unique_tokens
        return kv + self.attention_bytes() - 2 * self.Hkv * self.D * self.es * int(self.lens.sum())


def cpu_baseline(wk: Workload, budget_s: float = 20.0) -> dict:
    """The float64 C oracle on the host cores, on its own allocator and pool."""
    from oracle import attention as oatt
    from oracle import native
    from oracle.pool import PagedPool

    w = wk.w
    threads = len(os.sched_getaffinity(0))
    native.build(force=False)
    t0 = time.perf_counter()
    opool = PagedPool(w.num_blocks, wk.bs, wk.stack.tolist())
    slots = []
    for b, n in enumerate(wk.lens.tolist()):
        opool.create(b)
        slots += opool.append(b, n)[0]
    tables, lens = opool.block_tables(range(wk.B), wk.max_blocks)
    npdt = np.uint16 if w.dtype == "bf16" else np.float32
    shape = (w.num_blocks, wk.Hkv, wk.bs, wk.D)
    kp = np.zeros(shape, npdt)
    vp = np.zeros(shape, npdt)

    def st(t):
        t = t.contiguous()
        return t.view(wk.torch.int16).numpy().view(np.uint16) if w.dtype == "bf16" else t.numpy()

    oatt.cache_write(kp, vp, st(wk.host_k), st(wk.host_v), slots, wk.bs)
    q = st(wk.host_q)
    log(f"[bench] oracle pool built in {time.perf_counter() - t0:.1f}s")
    tables = np.array(tables, np.int32)
    lens = np.array(lens, np.int32)
    rows_total = wk.B * wk.nq * wk.Hq
    # time one sequence's rows first, then size the sample to the budget
    probe = np.arange(wk.nq * wk.Hq, dtype=np.int64)
    t0 = time.perf_counter()
    native.attention(q, w.dtype, kp, vp, w.dtype, tables, lens, wk.scale, wk.bs, rows=probe,
                     threads=threads)
    t_seq = time.perf_counter() - t0
    n_seq = int(max(1, min(wk.B, budget_s / 3 / max(t_seq, 1e-6))))
    rows = np.arange(n_seq * wk.nq * wk.Hq, dtype=np.int64)
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        native.attention(q, w.dtype, kp, vp, w.dtype, tables, lens, wk.scale, wk.bs, rows=rows,
                         threads=threads)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    tok_s = n_seq * wk.nq / med
    return {"value": tok_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 C oracle walking block tables token by token, OpenMP over "
                      f"rows; {n_seq} of {wk.B} sequences (all {wk.Hq} heads, full context), "
                      f"median of 3 runs of {med:.2f}s; rows {len(rows)} of {rows_total}",
            "python_oracle_small": python_oracle_c1()}


def python_oracle_c1() -> dict:
    """The pure-Python float64 oracle timed on the small fp32 configuration
    (4 sequences of 6, 9, 17 and 33 tokens, 4 query heads over 2 KV heads,
    head dim 64): its cost per token is that of a walk over block tables one
    token at a time, which only the small case can afford."""
    from oracle import attention as oatt
    from oracle.pool import PagedPool
    from synth import workloads as wl

    w = wl.WORKLOADS["tiny_f32"]
    rng = np.random.default_rng(w.rng_seed)
    stack = wl.free_stack_permutation(rng, w.num_blocks)
    lens = wl.draw_lengths(rng, w)
    root = wl.root_seed(rng)
    pool = PagedPool(w.num_blocks, w.block_size, stack.tolist())
    slots = []
    for b, n in enumerate(lens.tolist()):
        pool.create(b)
        slots += pool.append(b, n)[0]
    tables, clens = pool.block_tables(range(w.batch), -(-int(lens.max()) // w.block_size))
    T = int(lens.sum())
    shape = (w.num_blocks, w.kv_heads, w.block_size, w.head_dim)
    kp = np.zeros(shape, np.float32)
    vp = np.zeros(shape, np.float32)
    k = wl.cast(wl.normal_array(root, 0, (T, w.kv_heads, w.head_dim)), "f32")
    v = wl.cast(wl.normal_array(root, 1, (T, w.kv_heads, w.head_dim)), "f32")
    q = wl.cast(wl.normal_array(root, 2, (w.batch, 1, w.q_heads, w.head_dim)), "f32")
    oatt.cache_write(kp, vp, k, v, slots, w.block_size)
    scale = 1.0 / math.sqrt(w.head_dim)
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        oatt.attention(q, "f32", kp, vp, "f32", tables, clens, scale, w.block_size)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    return {"value": w.batch / med, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "seconds": med,
            "sample": "pure-Python float64 oracle, whole small fp32 batch (4 sequences, "
                      "lengths 6/9/17/33, 4 query heads, 2 KV heads, head dim 64), "
                      "median of 3 runs"}


def copy_probe(mib: int, dev) -> int:
    """Copy `mib` MiB of K and of V blocks (src -> dst halves of a fresh pool)."""
    import torch

    import paged_kv_cache_202_amd as pkv

    Hkv, bs, D = 8, 16, 128
    block = Hkv * bs * D * 2
    n = mib * (1 << 20) // block
    kc = torch.zeros((2 * n, Hkv, bs, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    pairs = torch.stack([torch.arange(n), torch.arange(n, 2 * n)], 1).to(torch.int32).to(dev)
    for _ in range(3):
        pkv.paged_kv_copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": 2 * n * block, "copy_probe_bytes_written": 2 * n * block,
                      "launches": 3}), flush=True)
    return 0


def read_probe(mib: int, dev, chunk: int = 4096) -> int:
    """Read ceilings of this machine: a buffer of `mib` MiB (well past the 256 MB
    last-level cache) read as `chunk`-byte chunks -- 4 KiB: the K (or V) run
    of one 16-token, 128-dim bf16 tile; 1 KiB: the same for 3-bit codes;
    2 KiB: 8-bit codes -- in sequence and in a seeded random order,
    with the decode kernels' loads: to registers (plain and non-temporal; four
    workgroups of eight wavefronts a CU) and through the non-temporal
    direct-to-LDS rings (one workgroup a CU; 16, 8 and 4 KiB in flight a
    wavefront, as far as a ring holds one chunk).
    Prints one JSON line; each figure is the median of 5 timed launches."""
    import torch

    import paged_kv_cache_202_amd as pkv

    n = mib * (1 << 20) // chunk
    buf = torch.randint(0, 256, (n * chunk,), dtype=torch.uint8, device=dev)
    orders = {"sequential": torch.arange(n, dtype=torch.int32, device=dev),
              "random": torch.from_numpy(np.random.default_rng(20260801).permutation(n)
                                         .astype(np.int32)).to(dev)}
    modes = {"registers": (0, 1024, 16384), "registers_nt": (1, 1024, 16384),
             "lds_rings_nt": (2, 256, 16384)}
    for ring in (8192, 4096):
        if ring >= chunk:
            modes[f"lds_rings_nt_{ring // 1024}k"] = (2, 256, ring)
    out = {"read_probe_bytes": n * chunk, "chunk_bytes": chunk}
    for oname, order in orders.items():
        for mname, (mode, n_wg, ring) in modes.items():
            sink = torch.zeros(n_wg, dtype=torch.int32, device=dev)
            pkv.paged_kv_read_probe(buf, order, sink, chunk, mode, ring)
            times = []
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                pkv.paged_kv_read_probe(buf, order, sink, chunk, mode, ring)
                b.record()
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b) * 1e-3)
            gbs = n * chunk / statistics.median(times) / 1e9
            out[f"{oname}_{mname}_GBs"] = gbs
            log(f"[bench] read probe {oname:10s} {mname:13s} {gbs:7.0f} GB/s")
    print(json.dumps(out), flush=True)
    return 0


def _csv_rows(d: str, suffix: str):
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _counter_per_dispatch(d: str, counter: str, kernel_re: str):
    """Mean over dispatches of a kernel of one rocprofv3 --pmc counter."""
    per = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if r["Counter_Name"] == counter and re.search(kernel_re, r["Kernel_Name"]):
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for /{kernel_re}/ under {d}")
    return statistics.mean(per.values()), len(per)


def merge_sq_counters(args) -> int:
    """Add one rocprofv3 pass of SQ counters (LDS use, bank conflicts, wave
    residency, instruction mix: whichever the pass holds) to the workload's
    committed summary, with the command that took them. SQ_WAVE_CYCLES is
    read as counting 4-cycle units (per shader engine), SQ_BUSY_CYCLES as
    cycles; the machine has 32 shader engines of 32 SIMDs."""
    path = profile_path(args.workload)
    with open(path) as f:
        out = json.load(f)
    rows = [r for r in _csv_rows(args.sq_dir, "counter_collection.csv")
            if re.search(args.kernel_regex, r["Kernel_Name"])]
    per = {}
    for r in rows:
        per.setdefault(r["Dispatch_Id"], {}).setdefault(r["Counter_Name"], 0.0)
        per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"/{args.kernel_regex}/ matches no dispatch in {args.sq_dir}")
    names = sorted(next(iter(per.values())))
    avg = {c: sum(d[c] for d in per.values()) / len(per) for c in names}
    derived = {}
    if "SQ_WAVE_CYCLES" in avg and "SQ_BUSY_CYCLES" in avg:
        derived["resident_waves_per_simd"] = 4 * avg["SQ_WAVE_CYCLES"] / avg["SQ_BUSY_CYCLES"] / 32
    if "SQ_LDS_BANK_CONFLICT" in avg and "SQ_INSTS_LDS" in avg:
        derived["bank_conflict_cycles_per_lds_instruction"] = (avg["SQ_LDS_BANK_CONFLICT"] /
                                                               avg["SQ_INSTS_LDS"])
    if "SQ_LDS_BANK_CONFLICT" in avg and "SQ_LDS_IDX_ACTIVE" in avg:
        derived["bank_conflict_share_of_lds_active"] = (avg["SQ_LDS_BANK_CONFLICT"] /
                                                        avg["SQ_LDS_IDX_ACTIVE"])
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        derived["share_of_mfma_busy_with_valu_coexecuting"] = (
            avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / avg["SQ_VALU_MFMA_BUSY_CYCLES"])
    if "SQ_INSTS_VALU" in avg and "SQ_WAVES" in avg:
        w = avg["SQ_WAVES"]
        derived["per_wave"] = {c[len("SQ_INSTS_"):].lower(): avg[c] / w
                               for c in names if c.startswith("SQ_INSTS_")}
    key = args.sq_key or "sq_counters"
    out[key] = {"counters_per_dispatch": avg, "dispatches": len(per), "derived": derived,
                "command": args.sq_command or "",
                "kernel_sources_sha256": sources_sha256(args.workload)}
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out[key], indent=1))
    return 0


def summarize_profile(args) -> int:
    """Condense rocprofv3 output into profiles/decode_<workload>.json: the
    kernel's average duration (--kernel-trace --stats), its HBM bytes per
    dispatch (--pmc FETCH_SIZE, WRITE_SIZE) scaled by what the same counters
    read for a plain copy of known size (--copy-probe), and a hash of the
    kernel sources they were taken on."""
    kre = args.kernel_regex
    if args.sq_dir and not args.trace_dir:
        return merge_sq_counters(args)
    stats = [r for r in _csv_rows(args.trace_dir, "kernel_stats.csv") if re.search(kre, r["Name"])]
    if len(stats) != 1:
        raise SystemExit(f"/{kre}/ matches {len(stats)} kernels in the trace")
    st = stats[0]
    fetch, nd = _counter_per_dispatch(args.fetch_dir, "FETCH_SIZE", kre)
    write, _ = _counter_per_dispatch(args.write_dir, "WRITE_SIZE", kre)
    cfetch, _ = _counter_per_dispatch(args.copy_fetch_dir, "FETCH_SIZE", "copy_blocks")
    cwrite, _ = _counter_per_dispatch(args.copy_write_dir, "WRITE_SIZE", "copy_blocks")
    moved = 2 * args.copy_mib * 2**20  # K and V, read once and written once
    ffac, wfac = moved / (cfetch * 1024), moved / (cwrite * 1024)
    from synth.workloads import WORKLOADS

    from synth import workloads as wl

    w = WORKLOADS[args.workload]
    if w.shared_prefix:
        lens = np.full(w.batch, w.shared_prefix + w.unique_suffix + w.queries_per_seq,
                       dtype=np.int64)
    elif w.context is None:  # the seeded lengths, drawn as the workload draws them
        rng = np.random.default_rng(w.rng_seed)
        wl.free_stack_permutation(rng, w.num_blocks)
        lens = wl.draw_lengths(rng, w).astype(np.int64)
    else:
        lens = np.full(w.batch, w.context, dtype=np.int64)
    out = {
        "kernel": st["Name"],
        "workload": args.workload,
        "kernel_sources_sha256": sources_sha256(args.workload),
        "trace": {"calls": int(st["Calls"]), "avg_ns": float(st["AverageNs"]),
                  "min_ns": float(st["MinNs"]), "max_ns": float(st["MaxNs"])},
        "pmc": {"FETCH_SIZE_kib_per_dispatch": fetch, "WRITE_SIZE_kib_per_dispatch": write,
                "dispatches": nd},
        "calibration": {"probe": f"paged_kv_copy_blocks copying {args.copy_mib} MiB of K and "
                                 f"{args.copy_mib} MiB of V",
                        "bytes_read": moved, "bytes_written": moved,
                        "FETCH_SIZE_kib": cfetch, "WRITE_SIZE_kib": cwrite,
                        "fetch_factor": ffac, "write_factor": wfac},
        "fetch_bytes_per_launch": fetch * 1024 * ffac,
        "write_bytes_per_launch": write * 1024 * wfac,
        "traffic_bytes_per_launch": fetch * 1024 * ffac + write * 1024 * wfac,
        "algorithmic_bytes_per_launch": prefix_unique_bytes(w) if w.shared_prefix else
        algorithmic_bytes(
            w.batch, w.queries_per_seq, w.q_heads, w.kv_heads, w.head_dim, w.esize, lens,
            -(-int(lens.max()) // w.block_size),
            kv_row_bytes={8: w.head_dim + 4, 3: w.head_dim // 2 + 4}.get(w.kv_codes)),
    }
    if w.shared_prefix:
        out["algorithmic_bytes_note"] = ("unique bytes: every shared block once per KV head, "
                                         "each sequence's private tokens once")
    path = profile_path(args.workload)
    if os.path.exists(path):  # SQ counter passes merged earlier keep their own commands
        with open(path) as f:
            old = json.load(f)
        out.update({k: v for k, v in old.items()
                    if isinstance(v, dict) and "counters_per_dispatch" in v})
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="llama3_8b_b32_8k")
    ap.add_argument("--rotate", type=int, default=2,
                    help="pool copies used in turn so repeats cannot hit the 256 MB cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-share", action="store_true",
                    help="prefix-sharing workloads: attend with the plain kernels, reading "
                         "every shared block once per sequence")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run paged_kv_copy_blocks over MIB MiB of K and of V (a plain "
                         "copy of known size, to calibrate HBM byte counters), then exit")
    ap.add_argument("--read-probe", type=int, default=0, metavar="MIB",
                    help="only measure read ceilings over MIB MiB (sequential and random "
                         "chunks, with the decode kernels' loads), then exit")
    ap.add_argument("--read-probe-chunk", type=int, default=4096, choices=(1024, 2048, 4096),
                    help="chunk bytes of --read-probe")
    ap.add_argument("--summarize-profile", action="store_true",
                    help="no GPU work: condense rocprofv3 output (the --*-dir options) into "
                         "profiles/decode_<workload>.json")
    ap.add_argument("--kernel-regex", default="decode_(partition|mfma)_kernel")
    ap.add_argument("--trace-dir")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--copy-fetch-dir")
    ap.add_argument("--copy-write-dir")
    ap.add_argument("--copy-mib", type=int, default=512)
    ap.add_argument("--sq-dir", help="with --summarize-profile and no --trace-dir: merge this "
                                     "rocprofv3 --pmc pass of SQ counters into the summary")
    ap.add_argument("--sq-key", help="name of the merged section (default sq_counters)")
    ap.add_argument("--sq-command", help="the rocprofv3 command that took the pass")
    args = ap.parse_args()
    if args.summarize_profile:
        return summarize_profile(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each GPU would run its own pool and sequences with no exchange).",
              file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.copy_probe:
        return copy_probe(args.copy_probe, dev)
    if args.read_probe:
        return read_probe(args.read_probe, dev, args.read_probe_chunk)
    if args.workload.startswith("prefix_share"):
        wk = PrefixVerifyWorkload(args.workload, dev, share=not args.no_share,
                                  rotate=args.rotate)
    else:
        wk = Workload(args.workload, args.rotate, dev)
    log(f"[bench] workload {args.workload} ready; max_blocks {wk.max_blocks}")

    for i in range(args.warmup):
        wk.step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        wk.step(i)
    end.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_step * 1e3:.1f} us/step")

    # per-call durations with events on the launch stream (same steps again)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        a, b, c = ev[i]
        a.record()
        wk.cache_write(i)
        b.record()
        wk.attend(i)
        c.record()
    torch.cuda.synchronize()
    attn_ms = statistics.mean(b.elapsed_time(c) for a, b, c in ev)
    write_ms = statistics.mean(a.elapsed_time(b) for a, b, c in ev)
    # the shared-prefix path's minimum is every physical block once; the plain
    # path's is every sequence's visible K/V
    attn_bytes = wk.unique_attention_bytes() if getattr(wk, "share", False) else \
        wk.attention_bytes()
    achieved = attn_bytes / (attn_ms * 1e-3) / 1e9
    log(f"[bench] attention {attn_ms * 1e3:.1f} us -> {achieved:.0f} GB/s; cache write "
        f"{write_ms * 1e3:.1f} us")

    result = {
        "metric": "paged-attn decode tokens/s + achieved HBM GB/s (% of peak), 1 MI355X",
        "value": wk.B * wk.nq / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wk.w.dtype,
        "data": "synthetic",
        "config": {"workload": wk.w.name, "batch": wk.B, "context": int(wk.lens.max()),
                   "q_heads": wk.Hq, "kv_heads": wk.Hkv, "head_dim": wk.D,
                   "block_size": wk.bs, "queries_per_seq": wk.nq,
                   "kv_dtype": (f"{wk.w.kv_codes}-bit codes + f32 row scales"
                                if getattr(wk, "q8", False) else wk.w.dtype),
                   "pool_blocks": wk.w.num_blocks,
                   "placement": "seeded permutation", "pool_rotation": args.rotate},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": profiled_traffic(wk.w.name),
                     "kernel": kernel_label(wk),
                     "algorithmic_bytes": attn_bytes, "avg_duration_us": attn_ms * 1e3},
        "step_breakdown_us": {"cache_write": write_ms * 1e3, "attention": attn_ms * 1e3},
        "host_alloc_us": {"step_alloc": wk.alloc_step_s * 1e6},
    }
    if getattr(wk, "share", False):
        result["host_alloc_us"]["prefix_groups"] = wk.groups_s * 1e6
    if is_chunk(wk):
        # a prefill chunk is a dense contraction: priced against bf16 MFMA
        fl = chunk_flops(wk.B, wk.nq, wk.Hq, wk.D, wk.lens)
        tf = fl / (attn_ms * 1e-3) / 1e12
        result["value"] = wk.B * wk.nq / (ms_step * 1e-3)
        result["roofline"].update({
            "bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": tf / MFMA_BF16_PEAK_TFLOPS, "algorithmic_flops": fl,
            "hbm_achieved_GBs": achieved})
        result["roofline"].pop("algorithmic_bytes")
        result["roofline"]["algorithmic_bytes_hbm"] = attn_bytes
    if hasattr(wk, "unique_attention_bytes"):
        ub, lb = wk.unique_attention_bytes(), wk.attention_bytes()
        result["roofline"]["unique_bytes"] = ub
        result["roofline"]["achieved_unique"] = ub / (attn_ms * 1e-3) / 1e9
        result["roofline"]["logical_bytes"] = lb
        result["roofline"]["achieved_logical"] = lb / (attn_ms * 1e-3) / 1e9
    if (not args.no_cpu_baseline and not hasattr(wk, "unique_attention_bytes")
            and not getattr(wk, "q8", False) and not is_chunk(wk)):
        result["cpu_baseline"] = cpu_baseline(wk)
        log(f"[bench] cpu baseline {result['cpu_baseline']['value']:.1f} tokens/s")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
