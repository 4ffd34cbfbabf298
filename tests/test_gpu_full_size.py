"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The GPU side is bench.py's own setup (library allocator, cache-write kernel,
the timed step: cache write of the new tokens then attention). The oracle
side builds its own allocator state and host pool from the same synthetic
inputs and walks the block tables in float64 (C oracle, OpenMP). Slots and
tables must match bit for bit; every output and lse must be within max-abs
1e-2 (bf16 caches) and within a tight bound that a dropped tile would break.
"""

import os
import sys

import numpy as np
import pytest
import torch

import bench
from oracle import attention as oatt
from oracle import native
from oracle.pool import PagedPool
from scenario import TIGHT

pytestmark = pytest.mark.gpu


def oracle_side(wk):
    opool = PagedPool(wk.w.num_blocks, wk.bs, wk.stack.tolist())
    pre = (wk.lens - wk.nq).tolist()
    pre_slots, step_slots = [], []
    for b in range(wk.B):
        opool.create(b)
    for b in range(wk.B):
        s, cow = opool.append(b, pre[b])
        assert not cow
        pre_slots += s
    for b in range(wk.B):
        s, cow = opool.append(b, wk.nq)
        assert not cow
        step_slots += s
    tables, lens = opool.block_tables(range(wk.B), wk.max_blocks)
    shape = (wk.w.num_blocks, wk.Hkv, wk.bs, wk.D)
    kp = np.zeros(shape, np.uint16)
    vp = np.zeros(shape, np.uint16)
    k = wk.host_k.view(torch.int16).numpy().view(np.uint16)
    v = wk.host_v.view(torch.int16).numpy().view(np.uint16)
    # the logical token order is sequence-major, the same order the slots cover
    starts = np.concatenate([[0], np.cumsum(wk.lens)[:-1]])
    order_pre = np.concatenate([np.arange(s, s + n) for s, n in zip(starts, pre)])
    order_new = np.concatenate([np.arange(s + n, s + n + wk.nq) for s, n in zip(starts, pre)])
    oatt.cache_write(kp, vp, k[order_pre], v[order_pre], pre_slots, wk.bs)
    oatt.cache_write(kp, vp, k[order_new], v[order_new], step_slots, wk.bs)
    return (np.array(pre_slots, np.int32), np.array(step_slots, np.int32),
            np.array(tables, np.int32), np.array(lens, np.int32), kp, vp)


# Tight bounds on out and lse beside the 1e-2 contract bound (see
# tests/scenario.py: far below what one dropped or repeated 16-token tile
# moves at these sizes).
BOUND = {"llama3_8b_b32_8k": TIGHT["decode"], "llama3_8b_varlen_b256": TIGHT["decode"],
         "llama33_70b_b4_128k": TIGHT["decode_128k"]}


@pytest.mark.parametrize("name", ["llama3_8b_b32_8k", "llama3_8b_varlen_b256",
                                  "llama33_70b_b4_128k"])
def test_full_size_workload(name, device):
    print(f"full-size workload {name}", flush=True)
    wk = bench.Workload(name, 1, device)
    pre_slots, step_slots, tables, lens, kp, vp = oracle_side(wk)
    assert np.array_equal(wk.pre_slots, pre_slots)
    assert np.array_equal(wk.step_slots, step_slots)
    assert np.array_equal(wk.tables_host, tables)
    assert np.array_equal(wk.lens, lens)
    wk.lse = torch.full((wk.B, wk.nq, wk.Hq), float("nan"), dtype=torch.float32, device=device)
    wk.step(0)  # the timed step: new-token cache write, then attention
    torch.cuda.synchronize()
    out = wk.out.cpu().numpy()
    lse = wk.lse.cpu().numpy()
    q = wk.host_q.view(torch.int16).numpy().view(np.uint16)
    ref, ref_lse = native.attention(q, "bf16", kp, vp, "bf16", tables, lens, wk.scale, wk.bs,
                                    threads=min(16, len(os.sched_getaffinity(0))))
    err = np.abs(out - ref).max()
    lerr = np.abs(lse - ref_lse).max()
    out_bound, lse_bound = BOUND[name]
    print(f"  {name}: max-abs error out {err:.3e}, lse {lerr:.3e} over {out.size} outputs "
          f"(tight bounds {out_bound:.0e}, {lse_bound:.0e})", flush=True)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert err <= 1e-2 and lerr <= 1e-2  # the contract
    assert err <= out_bound and lerr <= lse_bound
