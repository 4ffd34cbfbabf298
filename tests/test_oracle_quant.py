"""Pins for the per-row integer-code oracle (oracle/quant.py) and the
attention walk over a code pool (C and Python).

Sources: the course page "Module 10. KV Caches and Efficient Inference",
project-exercise demo, Demo 2 (teaching quantizer: symmetric codes, one
scale per row; its 8-bit output-error bound and the all-zero case), and the
notebook's section 8 compression scenario (16 -> 3 bits per coordinate).
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as pyo
from oracle import native
from oracle import quant
from oracle.geometry import bytes_per_token
from oracle.pool import PagedPool

SEED = 20260801  # the notebook's demo seed


def softmax_attention(q, k, v):
    """torch float64 attention with the scale 1/sqrt(width) of the demo."""
    out = F.scaled_dot_product_attention(torch.from_numpy(q)[None], torch.from_numpy(k)[None],
                                         torch.from_numpy(v)[None])
    return out[0].numpy()


def test_demo2_eight_bit_error_bound_and_zero_rows():
    """The demo's experiment: 128 keys and values of width 32, 12 queries
    drawn from the seed + 10 stream; 8-bit codes keep the relative output
    error under 0.03; an all-zero row reconstructs to zeros."""
    rng = np.random.default_rng(SEED + 10)
    n, d = 128, 32
    keys = rng.normal(size=(n, d))
    values = rng.normal(size=(n, d))
    queries = rng.normal(size=(12, d))
    ref = softmax_attention(queries, keys, values)
    errs = {}
    for bits in (8, 3):
        out = softmax_attention(queries, quant.fake_quantize_rows(keys, bits),
                                quant.fake_quantize_rows(values, bits))
        errs[bits] = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert errs[8] < 0.03
    assert errs[3] > errs[8]  # fewer bits, larger error
    np.testing.assert_array_equal(quant.fake_quantize_rows(np.zeros((2, 4)), 3), 0)
    codes, scale = quant.quantize_rows(np.zeros((2, 4)), 8)
    assert not codes.any() and (scale == 1.0).all()


@pytest.mark.parametrize("bits", [8, 4, 3])
def test_codes_closed_forms(bits):
    rng = np.random.default_rng(3)
    x = rng.normal(size=(200, 48)) * rng.uniform(0.01, 100, size=(200, 1))
    codes, scale = quant.quantize_rows(x, bits)
    limit = 2 ** (bits - 1) - 1
    assert codes.dtype == np.int8 and np.abs(codes).max() <= limit
    # the largest magnitude of every row maps to +-limit exactly
    i = np.argmax(np.abs(x), axis=1)
    top = codes[np.arange(200), i]
    assert (np.abs(top) == limit).all() and (np.sign(top) == np.sign(x[np.arange(200), i])).all()
    # reconstruction error at most half a step per element
    err = np.abs(codes * scale[:, None] - x)
    assert (err <= scale[:, None] / 2 * (1 + 1e-12)).all()


def test_codes_brute_force_nearest():
    """Each code is the integer of [-limit, limit] nearest to x / scale (ties
    to the even one), found by trying them all."""
    rng = np.random.default_rng(4)
    x = rng.normal(size=(30, 8))
    # exact ties at 3 bits: max 3 -> scale 1, so 1.5, -0.5, 2.5 and -1.5 sit halfway
    x[0] = [3.0, 1.5, -0.5, 2.5, 0.25, -1.5, 0.0, 1.0]
    for bits in (3, 8):
        codes, scale = quant.quantize_rows(x, bits)
        limit = 2 ** (bits - 1) - 1
        cand = np.arange(-limit, limit + 1)
        for r in range(x.shape[0]):
            for c in range(x.shape[1]):
                y = x[r, c] / scale[r]
                dist = np.abs(y - cand)
                best = cand[dist == dist.min()]
                want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
                assert codes[r, c] == want


def test_three_bit_storage_scenario():
    """Section 8: 16 -> 3 bits per coordinate takes Llama-3-8B's 128 KiB of
    K/V per token to 24 KiB (codes only, scales aside)."""
    per_token = bytes_per_token(layers=32, kv_heads=8, head_dim=128, elem_bytes=2)
    assert per_token == 131072
    assert per_token * 3 / 16 == 24 * 1024


def build_q8_case(seed, lens, Hq, Hkv, D, bs, nq=1):
    rng = np.random.default_rng(seed)
    B = len(lens)
    nb = sum(-(-n // bs) for n in lens) + 3
    pool = PagedPool(nb, bs, rng.permutation(nb).tolist())
    slots = []
    for b, n in enumerate(lens):
        pool.create(b)
        s, _ = pool.append(b, n)
        slots += s
    T = sum(lens)
    k_new = rng.normal(size=(T, Hkv, D)) * rng.uniform(0.1, 3.0, size=(T, Hkv, 1))
    v_new = rng.normal(size=(T, Hkv, D))
    kc = np.zeros((nb, Hkv, bs, D), np.int8)
    vc = np.zeros_like(kc)
    ks = np.ones((nb, Hkv, bs), np.float32)
    vs = np.ones_like(ks)
    quant.cache_write_q(kc, vc, ks, vs, k_new, v_new, slots, bs)
    maxb = max(-(-n // bs) for n in lens)
    tables, L = pool.block_tables(range(B), maxb)
    q = rng.normal(size=(B, nq, Hq, D)).astype(np.float32)
    return dict(q=q, kc=kc, vc=vc, ks=ks, vs=vs, tables=np.array(tables, np.int32),
                lens=np.array(L, np.int32), k_new=k_new, v_new=v_new, slots=slots)


def test_cache_write_reads_back_quantized_rows():
    c = build_q8_case(5, (7, 20, 33), 4, 2, 16, 8)
    kc_ref, ks_ref = quant.quantize_rows(c["k_new"], 8)
    t = 0
    for b, n in enumerate(c["lens"]):
        for i in range(n):
            blk = c["tables"][b][i // 8]
            assert np.array_equal(c["kc"][blk, :, i % 8], kc_ref[t])
            assert np.array_equal(c["ks"][blk, :, i % 8], ks_ref[t].astype(np.float32))
            t += 1


@pytest.mark.parametrize("nq", [1, 3])
def test_q8_walk_matches_dequantized_pool(nq):
    """The C walk over codes equals the Python walk over the dequantized
    pool, and torch float64 SDPA over the logical dequantized rows."""
    Hq, Hkv, D, bs = 8, 2, 16, 8
    c = build_q8_case(6, (9, 25, 40), Hq, Hkv, D, bs, nq=nq)
    out, lse = native.attention_q8(c["q"], "f32", c["kc"], c["vc"], c["ks"], c["vs"],
                                   c["tables"], c["lens"], 0.25, bs)
    kd = quant.dequantize_pool(c["kc"], c["ks"])
    vd = quant.dequantize_pool(c["vc"], c["vs"])
    po, pl = pyo.attention(c["q"], "f32", kd, vd, "f64", c["tables"], c["lens"], 0.25, bs)
    np.testing.assert_allclose(out, po, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, pl, rtol=0, atol=1e-12)
    # logical rows: token t of sequence b at its slot
    start = 0
    for b, n in enumerate(c["lens"]):
        ks = np.stack([kd[s // bs, :, s % bs] for s in c["slots"][start:start + n]])
        vs_ = np.stack([vd[s // bs, :, s % bs] for s in c["slots"][start:start + n]])
        start += n
        k = torch.from_numpy(ks).transpose(0, 1).repeat_interleave(Hq // Hkv, 0)
        v = torch.from_numpy(vs_).transpose(0, 1).repeat_interleave(Hq // Hkv, 0)
        qb = torch.from_numpy(c["q"][b].astype(np.float64)).transpose(0, 1)
        mask = torch.arange(n)[None, :] <= (n - nq + torch.arange(nq))[:, None]
        ref = F.scaled_dot_product_attention(qb, k, v, attn_mask=mask,
                                             scale=float(np.float32(0.25)))
        np.testing.assert_allclose(out[b], ref.transpose(0, 1).numpy(), rtol=0, atol=1e-12)
