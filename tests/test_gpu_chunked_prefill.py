"""GPU parity for chunked prefill: more than 16 query rows per KV head.

A chunk of nq prompt tokens attends over the cached prefix plus the chunk
itself (query i of the chunk sees the first L - nq + i + 1 tokens; the chunk
decomposition of the course notebook, section 7). The library runs it on
the MFMA row-tile kernel and the partition reduce; the C oracle walks the
same tables token by token in float64. Caches start filled with NaN bit
patterns, so stale slots past a context's end would show up in the output.
"""

import os

import numpy as np
import pytest
import torch

import paged_kv_cache_202_amd as pkv
from oracle import native
from scenario import Case, tolerance

pytestmark = pytest.mark.gpu

CASES = [
    # lens, Hq, Hkv, D, nq (chunk), partition_tokens
    ((164,), 32, 8, 128, 64, 0),          # 256 rows per KV head: two row tiles per wavefront
    ((40, 57), 8, 8, 64, 40, 0),          # G = 1: a first chunk (L == nq) and a short prefix
    ((550, 300), 64, 8, 256, 33, 0),      # G = 8, D = 256, ragged last row tile
    ((2048, 1212), 16, 8, 128, 512, 0),   # G = 2, 1024 rows per KV head
    ((2000, 1111, 515), 32, 8, 128, 128, 64),  # explicit 64-token partitions
    ((999,), 32, 8, 128, 77, 16),         # 16-token partitions, odd chunk
    ((300, 18), 32, 32, 128, 17, 0),      # G = 1, 17 rows: a 1-row second tile
    ((777,), 32, 8, 64, 200, -1),         # -1 asks for the library's choice here
    # one KV head (multi-query attention): more than 16 rows per KV head even
    # for one query token, so decode itself runs on the row-tile kernel
    ((600, 2100, 1), 32, 1, 128, 1, 0),   # G = 32, one query token, a 1-token context
    ((1500, 90), 64, 1, 64, 3, 0),        # G = 64, three query tokens
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_chunk_matches_oracle(ci, device):
    lens, Hq, Hkv, D, nq, part = CASES[ci]
    print(f"chunked prefill case {ci}: lens {lens} Hq {Hq} Hkv {Hkv} D {D} nq {nq} "
          f"part {part}", flush=True)
    case = Case(lens, Hq, Hkv, D, 16, "bf16", nq=nq, seed=900 + ci, stack_seed=ci,
                device=device, partition_tokens=part)
    out, lse = case.run_gpu()
    ref, ref_lse = case.run_oracle()
    err = np.abs(out - ref).max()
    print(f"  max-abs error {err:.3e}", flush=True)
    assert np.isfinite(out).all() and err <= tolerance("bf16")
    assert np.abs(lse - ref_lse).max() <= 1e-2


@pytest.mark.parametrize("bs", [32, 64])
def test_chunk_larger_blocks(bs, device):
    """Blocks of 32 and 64 tokens: the row-tile kernel's tiles start inside
    blocks, chunk and cached prefix alike."""
    print(f"chunked prefill, block size {bs}", flush=True)
    case = Case((700, 1300), 32, 8, 128, bs, "bf16", nq=96, seed=950 + bs, stack_seed=bs,
                device=device, partition_tokens=0)
    out, lse = case.run_gpu()
    ref, ref_lse = case.run_oracle()
    err = np.abs(out - ref).max()
    print(f"  max-abs error {err:.3e}", flush=True)
    assert np.isfinite(out).all() and err <= tolerance("bf16")
    assert np.abs(lse - ref_lse).max() <= 1e-2


def test_rows_without_keys_and_bad_tables_give_nan(device):
    """A sequence shorter than its chunk, and one whose table points outside
    the pool, produce NaN rows; the others are unaffected."""
    case = Case((5, 100, 90), 32, 8, 128, 16, "bf16", nq=20, seed=7, stack_seed=7,
                device=device)
    tables = case.d_tables.clone()
    tables[2, 1] = case.num_blocks + 3  # a block of sequence 2 past the pool
    out = torch.full((3, 20, 32, 128), 0.0, dtype=torch.float32, device=device)
    ws = torch.empty(pkv.paged_attention_workspace_size(3, 20, 32, 8, 128, case.max_blocks, 16),
                     dtype=torch.uint8, device=device)
    pkv.paged_attention_decode(out, case.d_q, case.k_cache, case.v_cache, tables, case.d_lens,
                               case.scale, workspace=ws)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.isnan(out[0]).all()
    # sequence 2 reads block entry 1 (tokens 16..31) in every row
    assert np.isnan(out[2]).all()
    rows = np.array([(1 * 20 + i) * 32 + h for i in range(20) for h in range(32)], np.int64)
    ref, _ = case.run_oracle(rows=rows)
    err = np.abs(out[1].reshape(-1, 128) - ref).max()
    assert err <= tolerance("bf16")


def test_fp32_chunks_are_refused(device):
    case = Case((64,), 32, 8, 64, 16, "f32", nq=8, seed=3, stack_seed=3, device=device)
    out = torch.empty((1, 8, 32, 64), dtype=torch.float32, device=device)
    with pytest.raises(pkv.InvalidArgument):
        pkv.paged_attention_decode(out, case.d_q, case.k_cache, case.v_cache, case.d_tables,
                                   case.d_lens, case.scale)


def test_chunk_full_size_sampled(device):
    """Four sequences at context 8192, each attending its last 512-token chunk
    (Llama-3-8B layer geometry), in the launch configuration bench.py times:
    slots and tables bit for bit, sampled rows against the C oracle."""
    import bench
    from test_gpu_full_size import oracle_side

    name = "llama3_8b_chunk512_b4_8k"
    print(f"chunked prefill full size: {name}", flush=True)
    wk = bench.Workload(name, 1, device)
    pre_slots, step_slots, tables, lens, kp, vp = oracle_side(wk)
    assert np.array_equal(wk.pre_slots, pre_slots)
    assert np.array_equal(wk.step_slots, step_slots)
    assert np.array_equal(wk.tables_host, tables)
    wk.step(0)  # the timed step: the chunk's cache write, then attention
    torch.cuda.synchronize()
    out = wk.out.cpu().numpy()
    B, nq, Hq, D = out.shape
    rng = np.random.default_rng(5)
    pick = np.unique(np.concatenate([rng.choice(B * nq * Hq, 160, replace=False),
                                     [0, Hq - 1, nq * Hq, B * nq * Hq - 1]])).astype(np.int64)
    q = wk.host_q.view(torch.int16).numpy().view(np.uint16)
    ref, _ = native.attention(q, "bf16", kp, vp, "bf16", tables, lens, wk.scale, wk.bs,
                              rows=pick, threads=min(16, len(os.sched_getaffinity(0))))
    err = np.abs(out.reshape(-1, D)[pick] - ref).max()
    print(f"  max-abs error {err:.3e} over {len(pick)} rows", flush=True)
    assert np.isfinite(out).all() and err <= tolerance("bf16")
