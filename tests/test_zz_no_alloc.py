"""GPU: the decode entry point that allocates nothing, against the one that
takes a caller workspace.

paged_attention_decode_noalloc keeps its partials in the library's own
per-GPU scratch array. Called through the C ABI, twice in a row -- first a
split-K call over long contexts that fills 5.9 MB of partials, then a
smaller balanced-stream call over mixed lengths, which reuses the array
holding the first call's contents -- it must give, bit for bit, what
paged_attention_decode gives with a fresh workspace on the same inputs (the
same kernels in the same launch plan), and match the float64 oracle.
Sizes past the array are refused before anything is launched.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_202_amd as pkv
from scenario import TIGHT, Case

pytestmark = pytest.mark.gpu


def run_both(case: Case, part: int):
    dev = case.device
    shape = (case.B, case.nq, case.Hq, case.D)
    outs = []
    for noalloc in (True, False):
        out = torch.full(shape, float("nan"), device=dev)
        lse = torch.full(shape[:3], float("nan"), device=dev)
        if noalloc:
            pkv.paged_attention_decode_noalloc(out, case.d_q, case.k_cache, case.v_cache,
                                               case.d_tables, case.d_lens, case.scale,
                                               partition_tokens=part, lse=lse)
        else:
            n = pkv.paged_attention_workspace_size(case.B, case.nq, case.Hq, case.Hkv, case.D,
                                                   case.max_blocks, case.bs, part)
            assert n > 0  # both calls use partials
            ws = torch.empty(n, dtype=torch.uint8, device=dev)
            pkv.paged_attention_decode(out, case.d_q, case.k_cache, case.v_cache,
                                       case.d_tables, case.d_lens, case.scale,
                                       partition_tokens=part, workspace=ws, lse=lse)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    return outs


@pytest.mark.parametrize("second", [False, True])
def test_noalloc_matches_workspace_entry_point(device, second):
    if not second:
        # 70B layer geometry, 512-token partitions: 3 x 64 rows x 59 partials
        print("no-alloc decode: split-K over (30000, 9000, 3001) tokens", flush=True)
        case = Case((30000, 9000, 3001), 64, 8, 128, 16, "bf16", seed=31, stack_seed=31)
        part = 512
        need = pkv.paged_attention_workspace_size(3, 1, 64, 8, 128, case.max_blocks, 16, part)
        assert need >= 192 * 59 * (128 + 2) * 4  # acc, m and l of every row and partition
    else:
        # smaller, after the first: the balanced stream over mixed lengths
        print("no-alloc decode: stream plan over 7 mixed lengths", flush=True)
        case = Case((700, 33, 1500, 5, 260, 16, 17), 32, 8, 128, 16, "bf16", seed=32,
                    stack_seed=32)
        part = -1
    (o_na, l_na), (o_ws, l_ws) = run_both(case, part)
    assert np.array_equal(o_na, o_ws) and np.array_equal(l_na, l_ws)
    ref, ref_lse = case.run_oracle()
    out_bound, lse_bound = TIGHT["decode"]
    assert np.abs(o_na - ref).max() <= out_bound and np.abs(l_na - ref_lse).max() <= lse_bound


def test_noalloc_refuses_sizes_past_its_array(device):
    case = Case((40, 40), 8, 2, 128, 16, "bf16", seed=33, stack_seed=33)
    out = torch.empty(2, 1, 8, 128, device=device)
    # 16-token partitions over contexts of 2^20 tokens: far past 64 MiB
    big = torch.full((2,), 1 << 20, dtype=torch.int32, device=device)
    tables = torch.zeros(2, (1 << 20) // 16, dtype=torch.int32, device=device)
    with pytest.raises(pkv.InvalidArgument, match="no-allocation"):
        pkv.paged_attention_decode_noalloc(out, case.d_q, case.k_cache, case.v_cache, tables,
                                           big, case.scale, partition_tokens=16)
