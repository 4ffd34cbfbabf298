"""The tight parity bounds can see a dropped or repeated tile -- CPU only.

A kernel that skipped one 16-token tile of a context, or counted one twice,
would still meet the 1e-2 contract bound at long contexts: at 8192 tokens
the outputs are themselves only a few 1e-2 in size. The GPU parity tests
therefore also hold out and lse to the tight bounds of tests/scenario.py.
This file computes, in float64 on the CPU, how far the smallest such mistake
moves the result at each workload's geometry -- inputs N(0, 1) cast to bf16
as in every workload, scale 1/sqrt(head dim): for each tile of a (sequence,
KV head), the largest change over its query rows and dims when that tile is
dropped (or repeated); then the smallest of those over all tiles. Each tight
bound must sit well below it. (The softmax with and without a tile is
written out directly, no kernel is involved.)
"""

import numpy as np
import pytest
import torch

from scenario import TIGHT


def bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


def smallest_tile_effect(n, G, D=128, units=2, seed=0):
    """min over tiles and units of (max |d out|, max |d lse|) for a dropped
    tile and for a repeated one."""
    rng = np.random.default_rng(seed)
    scale = float(np.float32(1 / np.sqrt(D)))
    best = np.inf, np.inf
    for _ in range(units):
        q = bf16(rng.standard_normal((G, D)))
        k = bf16(rng.standard_normal((n, D)))
        v = bf16(rng.standard_normal((n, D)))
        s = (q @ k.T) * scale
        p = np.exp(s - s.max(axis=1, keepdims=True))
        l = p.sum(axis=1)
        acc = p @ v
        nt = n // 16
        p_t = p[:, :nt * 16].reshape(G, nt, 16)
        acc_t = np.einsum("gtk,tkd->gtd", p_t, v[:nt * 16].reshape(nt, 16, D))
        l_t = p_t.sum(axis=2)
        for sign in (-1.0, 1.0):
            l2 = l[:, None] + sign * l_t
            out2 = (acc[:, None, :] + sign * acc_t) / l2[:, :, None]
            d_out = np.abs(out2 - (acc / l[:, None])[:, None, :]).max(axis=(0, 2)).min()
            d_lse = np.abs(np.log(l2) - np.log(l)[:, None]).max(axis=0).min()
            best = min(best[0], d_out), min(best[1], d_lse)
    return best


@pytest.mark.parametrize("name,n,G,margin", [
    # the 8K batch (and the longest sequences of the variable-length batch)
    ("decode", 8192, 4, 8),
    # the 128K split-K workload (64 query heads over 8 KV heads)
    ("decode_128k", 131072, 8, 5),
    # prefix sharing + 4-draft verify: 2564-token contexts, shortest row 2561
    ("multi_query", 2561, 4, 3),
    # caches of codes: rows of contexts of at least 4096 tokens, and the
    # longest context below that
    ("codes_long", 8192, 4, 5),
    ("codes_short", 4095, 4, 2),
])
def test_tight_bound_sees_one_tile(name, n, G, margin):
    out_bound, lse_bound = TIGHT[name]
    d_out, d_lse = smallest_tile_effect(n, G)
    print(f"{name}: one tile moves out by >= {d_out:.2e}, lse by >= {d_lse:.2e}; "
          f"bounds {out_bound:.0e}, {lse_bound:.0e}")
    assert d_out >= margin * out_bound and d_lse >= margin * lse_bound
