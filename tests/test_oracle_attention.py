"""Pins for the attention oracles (Python walk and C walk) -- CPU only.

The oracles are checked against things outside themselves:

* torch's float64 ``scaled_dot_product_attention`` (a library routine) on the
  logical, contiguous K/V -- the paged layout never enters that side, so a
  wrong block index, offset, head map or causal limit in the walk fails;
* invariance under a different physical placement (another free-stack
  permutation), which must give bit-identical results;
* weights summing to one, and lse equal to torch's ``logsumexp``;
* closed forms: one key => its value; zero query => mean of the visible
  values; identical keys => mean of the values; the one-hot construction of
  the course notebook's Demo 2 stays finite and picks the right value;
* split-K: partitions merged by log-sum-exp equal the unpartitioned result;
* speculative verify: nq causal queries equal nq separate decodes;
* chunked prefill: the chunks' rows equal the one-shot prefill's rows.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as pyo
from oracle import native
from oracle.pool import PagedPool
from synth import workloads as wl


def _as_storage(t: torch.Tensor) -> np.ndarray:
    """Storage view of a CPU tensor: float32 array or bf16 bit patterns."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def build_case(seed, lens, Hq, Hkv, D, bs, dtype, nq=1, num_blocks=None, stack_seed=None):
    """Logical K/V per sequence, scattered into a pool by the oracle allocator."""
    rng = np.random.default_rng(seed)
    nblk = num_blocks or sum(-(-n // bs) for n in lens) + 3
    stack = None
    if stack_seed is not None:
        stack = np.random.default_rng(stack_seed).permutation(nblk).tolist()
    pool = PagedPool(nblk, bs, initial_free_stack=stack)
    B = len(lens)
    logical_k = [wl.cast(rng.standard_normal((n, Hkv, D), dtype=np.float32), dtype) for n in lens]
    logical_v = [wl.cast(rng.standard_normal((n, Hkv, D), dtype=np.float32), dtype) for n in lens]
    q = wl.cast(rng.standard_normal((B, nq, Hq, D), dtype=np.float32), dtype)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    k_pool = torch.zeros((nblk, Hkv, bs, D), dtype=tdt)
    v_pool = torch.zeros((nblk, Hkv, bs, D), dtype=tdt)
    kp, vp = _as_storage(k_pool), _as_storage(v_pool)
    for b, n in enumerate(lens):
        pool.create(b)
        slots, cow = pool.append(b, n)
        assert not cow
        pyo.cache_write(kp, vp, _as_storage(logical_k[b]), _as_storage(logical_v[b]), slots, bs)
    maxb = max(-(-n // bs) for n in lens)
    tables, L = pool.block_tables(range(B), maxb)
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, tables=np.array(tables, np.int32),
                lens=np.array(L, np.int32), lk=logical_k, lv=logical_v, pool=pool)


def sdpa_reference(case, scale, nq):
    """torch float64 SDPA over the logical K/V (GQA by repeating KV heads)."""
    q = case["q"].double()
    B, _, Hq, D = q.shape
    outs, lses = [], []
    for b in range(B):
        k = case["lk"][b].double().transpose(0, 1)  # [Hkv, n, D]
        v = case["lv"][b].double().transpose(0, 1)
        Hkv, n, _ = k.shape
        k = k.repeat_interleave(Hq // Hkv, dim=0)
        v = v.repeat_interleave(Hq // Hkv, dim=0)
        qb = q[b].transpose(0, 1)  # [Hq, nq, D]
        # query i sees keys [0, n - nq + i]
        mask = torch.arange(n)[None, :] <= (n - nq + torch.arange(nq))[:, None]
        sigma = float(np.float32(scale))
        o = F.scaled_dot_product_attention(qb, k, v, attn_mask=mask, scale=sigma)
        logits = (qb @ k.transpose(-1, -2)) * sigma
        logits = logits.masked_fill(~mask, -math.inf)
        outs.append(o.transpose(0, 1))
        lses.append(torch.logsumexp(logits, dim=-1).transpose(0, 1))
    return torch.stack(outs).numpy(), torch.stack(lses).numpy()


def run_oracle(kind, case, dtype, scale, bs):
    q, kp, vp = _as_storage(case["q"]), _as_storage(case["k_pool"]), _as_storage(case["v_pool"])
    if kind == "python":
        return pyo.attention(q, dtype, kp, vp, dtype, case["tables"], case["lens"], scale, bs)
    return native.attention(q, dtype, kp, vp, dtype, case["tables"], case["lens"], scale, bs)


KINDS = ["python", "c"]

CASES = [
    # lens, Hq, Hkv, D, bs, dtype, nq
    ((6, 9, 17, 33), 4, 2, 64, 16, "f32", 1),
    ((1, 5, 16, 40), 8, 2, 32, 4, "bf16", 1),
    ((7, 12, 30), 4, 4, 16, 8, "f32", 3),
    ((20, 45), 8, 1, 16, 16, "bf16", 4),
    # chunked prefill: a whole first chunk (L == nq) and a chunk over a prefix
    ((40, 57), 4, 2, 16, 16, "bf16", 40),
]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("ci", range(len(CASES)))
def test_matches_sdpa_on_logical_kv(kind, ci):
    lens, Hq, Hkv, D, bs, dtype, nq = CASES[ci]
    scale = 1.0 / math.sqrt(D)
    case = build_case(100 + ci, lens, Hq, Hkv, D, bs, dtype, nq=nq, stack_seed=ci)
    out, lse = run_oracle(kind, case, dtype, scale, bs)
    ref_out, ref_lse = sdpa_reference(case, scale, nq)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind", KINDS)
def test_placement_invariance_is_bitwise(kind):
    lens, Hq, Hkv, D, bs, dtype, nq = CASES[1]
    a = build_case(7, lens, Hq, Hkv, D, bs, dtype, stack_seed=1, num_blocks=40)
    b = build_case(7, lens, Hq, Hkv, D, bs, dtype, stack_seed=2, num_blocks=40)
    assert not np.array_equal(a["tables"], b["tables"])
    oa, la = run_oracle(kind, a, dtype, 0.125, bs)
    ob, lb = run_oracle(kind, b, dtype, 0.125, bs)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_weights_sum_to_one():
    lens, Hq, Hkv, D, bs, dtype, nq = CASES[0]
    case = build_case(3, lens, Hq, Hkv, D, bs, dtype)
    q = _as_storage(case["q"])
    for b, n in enumerate(lens):
        for h in range(Hq):
            w = pyo.attention_weights(q[b, 0, h], dtype, _as_storage(case["k_pool"]),
                                      _as_storage(case["v_pool"]), dtype,
                                      case["tables"][b], n, h // (Hq // Hkv), 0.125, bs)
            assert len(w) == n and abs(w.sum() - 1.0) < 1e-12 and (w > 0).all()


@pytest.mark.parametrize("kind", KINDS)
def test_closed_forms(kind):
    bs, D, Hkv, Hq = 4, 8, 1, 2
    lens = (1, 5, 9)
    case = build_case(11, lens, Hq, Hkv, D, bs, "f32")
    # zero query for head 1 of every sequence => uniform weights
    case["q"][:, :, 1, :] = 0.0
    out, _ = run_oracle(kind, case, "f32", 0.3, bs)
    for b, n in enumerate(lens):
        v = case["lv"][b].double().numpy()[:, 0, :]
        np.testing.assert_allclose(out[b, 0, 1], v.mean(axis=0), rtol=0, atol=1e-14)
    # a single visible key => exactly its value
    np.testing.assert_array_equal(out[0, 0, 0], case["lv"][0].double().numpy()[0, 0])
    # identical keys => mean of the values, whatever the query
    case2 = build_case(12, (7,), Hq, Hkv, D, bs, "f32")
    k_same = case2["lk"][0][0:1].clone()
    kp = case2["k_pool"]
    for t in range(7):
        blk = case2["tables"][0][t // bs]
        kp[blk, 0, t % bs] = k_same[0, 0]
    out2, _ = run_oracle(kind, case2, "f32", 0.5, bs)
    v = case2["lv"][0].double().numpy()[:, 0, :]
    np.testing.assert_allclose(out2[0, 0, 0], v.mean(axis=0), rtol=0, atol=1e-14)


@pytest.mark.parametrize("kind", KINDS)
def test_one_hot_keys_stay_finite(kind):
    """[KVNB demo] Demo 2 construction: 128 keys, one-hot at positions 0 and 90."""
    n, d, bs = 128, 32, 16
    pool = PagedPool(8, bs)
    pool.create(0)
    slots, _ = pool.append(0, n)
    k = np.zeros((n, 1, d), np.float32)
    k[0, 0, 0] = 12
    k[90, 0, 1] = 12
    v = np.zeros((n, 1, d), np.float32)
    v[0, 0, 0] = 1
    v[90, 0, 1] = 1
    kp = np.zeros((8, 1, bs, d), np.float32)
    vp = np.zeros_like(kp)
    pyo.cache_write(kp, vp, k, v, slots, bs)
    tables, lens = pool.block_tables([0], 8)
    for target, scale in ((0, 40.0), (1, 40.0), (0, 1.0 / math.sqrt(d))):
        q = np.zeros((1, 1, 1, d), np.float32)
        q[0, 0, 0, target] = 4
        if kind == "python":
            out, lse = pyo.attention(q, "f32", kp, vp, "f32", tables, lens, scale, bs)
        else:
            out, lse = native.attention(q, "f32", kp, vp, "f32", np.array(tables, np.int32),
                                        np.array(lens, np.int32), scale, bs)
        assert np.isfinite(out).all() and np.isfinite(lse).all()
        hot = 0 if target == 0 else 90
        logits = np.zeros(n)
        logits[hot] = 48.0 * float(np.float32(scale))
        w = np.exp(logits - logits.max())
        w /= w.sum()
        assert abs(out[0, 0, 0, target] - w[hot]) < 1e-12


def test_split_k_merge_equals_single_pass():
    lens, Hq, Hkv, D, bs, dtype, nq = (70,), 2, 1, 16, 4, "f32", 1
    case = build_case(21, lens, Hq, Hkv, D, bs, dtype)
    q64 = pyo.widen(_as_storage(case["q"]), dtype)
    k64 = pyo.widen(_as_storage(case["k_pool"]), dtype)
    v64 = pyo.widen(_as_storage(case["v_pool"]), dtype)
    sigma = float(np.float32(0.25))
    full, lse_full, _ = pyo.attend_row(q64[0, 0, 0], k64, v64, case["tables"][0], 70, 0, bs, sigma)
    for part in (1, 3, 16, 64, 70, 128):
        parts = pyo.partition_partials(q64[0, 0, 0], k64, v64, case["tables"][0], 70, 0, bs,
                                       sigma, part)
        assert len(parts) == -(-70 // part)
        out, lse = pyo.merge_partials(parts)
        np.testing.assert_allclose(out, full, rtol=0, atol=1e-14)
        assert abs(lse - lse_full) < 1e-13


@pytest.mark.parametrize("kind", KINDS)
def test_verify_equals_sequential_decodes(kind):
    lens, Hq, Hkv, D, bs, dtype, K = (19, 33), 4, 2, 16, 4, "bf16", 4
    case = build_case(31, lens, Hq, Hkv, D, bs, dtype, nq=K)
    out, lse = run_oracle(kind, case, dtype, 0.25, bs)
    for i in range(K):
        single = dict(case)
        single["q"] = case["q"][:, i:i + 1].contiguous()
        single["lens"] = case["lens"] - (K - 1 - i)
        o1, l1 = run_oracle(kind, single, dtype, 0.25, bs)
        assert np.array_equal(out[:, i], o1[:, 0]) and np.array_equal(lse[:, i], l1[:, 0])


@pytest.mark.parametrize("kind", KINDS)
def test_chunks_equal_one_shot_prefill(kind):
    """Chunked prefill ([KVNB s7] chunk decomposition): the rows of chunk c,
    attended with the context cut at the chunk's end, are the one-shot
    prefill's rows c*C .. c*C + C - 1, bit for bit."""
    lens, Hq, Hkv, D, bs, dtype, C = (48, 48), 4, 2, 16, 16, "bf16", 16
    case = build_case(41, lens, Hq, Hkv, D, bs, dtype, nq=48)
    out, lse = run_oracle(kind, case, dtype, 0.25, bs)
    for c in range(3):
        chunk = dict(case)
        chunk["q"] = case["q"][:, c * C:(c + 1) * C].contiguous()
        chunk["lens"] = np.full_like(case["lens"], (c + 1) * C)
        oc, lc = run_oracle(kind, chunk, dtype, 0.25, bs)
        assert np.array_equal(out[:, c * C:(c + 1) * C], oc)
        assert np.array_equal(lse[:, c * C:(c + 1) * C], lc)


def test_bf16_widening_matches_torch():
    x = torch.randn(4096, dtype=torch.float32).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy()
    assert np.array_equal(pyo.widen(bits, "bf16"), x.double().numpy())


def test_cache_write_reads_back_through_tables():
    lens = (5, 16, 23)
    case = build_case(41, lens, 2, 2, 8, 4, "bf16", stack_seed=5)
    for b, n in enumerate(lens):
        for t in range(n):
            blk = case["tables"][b][t // 4]
            assert torch.equal(case["k_pool"][blk, :, t % 4], case["lk"][b][t])
            assert torch.equal(case["v_pool"][blk, :, t % 4], case["lv"][b][t])


def test_c_oracle_rejects_bad_tables():
    case = build_case(51, (9,), 2, 1, 8, 4, "f32")
    bad = case["tables"].copy()
    bad[0, 1] = 999
    with pytest.raises(ValueError):
        native.attention(_as_storage(case["q"]), "f32", _as_storage(case["k_pool"]),
                         _as_storage(case["v_pool"]), "f32", bad, case["lens"], 0.5, 4)
