"""GPU parity for prefix sharing + speculative verify (MFMA multi-query tile).

The GPU side is bench.py's PrefixVerifyWorkload (library allocator with
fork and copy-on-write, block copy and cache-write kernels, then the
multi-query attention step). The oracle builds the same state with its own
pool, copies and cache writes from the same synthetic inputs and walks the
tables in float64 with the causal multi-query rule.
"""

import os

import numpy as np
import pytest
import torch

import bench
from oracle import attention as oatt
from oracle import native
from oracle.pool import PagedPool
from scenario import TIGHT

pytestmark = pytest.mark.gpu

# Tight bounds on out and lse beside the 1e-2 contract bound (see
# tests/scenario.py): the multi-query tiles round the softmax weights to bf16
# for the p.v product, so out errors sit near 4e-4 here; one dropped or
# repeated 16-token tile of these ~2.5K-token contexts moves out by >= 3e-3
# and lse by >= 4e-3.
OUT_BOUND, LSE_BOUND = TIGHT["multi_query"]


def bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("prefix,expect_copies", [(2048, 0), (2056, 63)])
def test_prefix_share_verify(prefix, expect_copies, device):
    print(f"prefix-share verify: prefix {prefix}", flush=True)
    wk = bench.PrefixVerifyWorkload("prefix_share_verify_k4", device, prefix=prefix)
    B, K, bs = wk.B, wk.nq, wk.bs
    # oracle state from the same inputs
    opool = PagedPool(wk.w.num_blocks, bs, wk.stack.tolist())
    opool.create(0)
    pre_slots, _ = opool.append(0, prefix)
    for s in range(1, B):
        opool.share_prefix(0, s, prefix)
    suf_slots, pairs = [], []
    for s in range(B):
        sl, cw = opool.append(s, wk.suffix)
        suf_slots += sl
        pairs += cw
    dft_slots = []
    for s in range(B):
        sl, cw = opool.append(s, K)
        assert not cw
        dft_slots += sl
    assert len(pairs) == expect_copies
    assert wk.pre_slots.tolist() == pre_slots
    assert wk.suf_slots.tolist() == suf_slots
    assert [tuple(p) for p in wk.cow_pairs.tolist()] == pairs
    assert wk.dft_slots.tolist() == dft_slots
    tables, lens = opool.block_tables(range(B), wk.max_blocks)
    assert wk.tables_host.tolist() == tables
    shape = (wk.w.num_blocks, wk.Hkv, bs, wk.D)
    kp = np.zeros(shape, np.uint16)
    vp = np.zeros(shape, np.uint16)
    oatt.cache_write(kp, vp, bits(wk.k_pre), bits(wk.v_pre), pre_slots, bs)
    for src, dst in pairs:
        kp[dst] = kp[src]
        vp[dst] = vp[src]
    oatt.cache_write(kp, vp, bits(wk.k_suf), bits(wk.v_suf), suf_slots, bs)
    oatt.cache_write(kp, vp, bits(wk.k_dft), bits(wk.v_dft), dft_slots, bs)
    wk.lse = torch.full((B, K, wk.Hq), float("nan"), dtype=torch.float32, device=device)
    wk.step(0)  # the timed step: draft cache write, then verify attention
    torch.cuda.synchronize()
    out = wk.out.cpu().numpy()
    lse = wk.lse.cpu().numpy()
    ref, ref_lse = native.attention(bits(wk.host_q), "bf16", kp, vp, "bf16",
                                    np.array(tables, np.int32), np.array(lens, np.int32),
                                    wk.scale, bs, threads=min(16, len(os.sched_getaffinity(0))))
    err = np.abs(out - ref).max()
    lerr = np.abs(lse - ref_lse).max()
    print(f"  max-abs error out {err:.3e}, lse {lerr:.3e} over {out.size} outputs "
          f"(tight bounds {OUT_BOUND:.0e}, {LSE_BOUND:.0e})", flush=True)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert err <= 1e-2 and lerr <= 1e-2  # the contract
    assert err <= OUT_BOUND and lerr <= LSE_BOUND
    # 128 (or 129) shared blocks + each sequence's private blocks: 2240 either way
    assert wk.pool.stats()["allocated_blocks"] == 2240
