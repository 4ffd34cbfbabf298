"""Pins for ``oracle.geometry`` against the course notebook's printed values."""

import json
import os

import pytest

from oracle.geometry import attention_flops, bytes_per_token, kv_payload_bytes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kvnb_contract.json")


@pytest.fixture(scope="module")
def contract():
    with open(GOLDEN) as f:
        return json.load(f)


GEOMETRY = {  # [KVNB §1] geometry table: layers, KV heads, head dim, bytes
    "70B MHA-equivalent (H=64)": (80, 64, 128, 2),
    "LLaMA-3.3-70B GQA": (80, 8, 128, 2),
    "Llama-3-8B GQA": (32, 8, 128, 2),
}


def test_bytes_per_token_ladder(contract):
    for name, geo in GEOMETRY.items():
        assert bytes_per_token(*geo) == contract["kv_ladder"][name]["bytes_per_token"]
    # one attention layer of each decode geometry used here: 4096 bytes/token
    assert bytes_per_token(1, 8, 128, 2) == 4096


def test_context_payload_70b(contract):
    per_tok = bytes_per_token(*GEOMETRY["LLaMA-3.3-70B GQA"])
    for tokens, expect in contract["context_memory_70b_gqa"].items():
        assert kv_payload_bytes(per_tok, int(tokens)) == expect["bytes"]
    with pytest.raises(ValueError):
        kv_payload_bytes(per_tok, -1)
    with pytest.raises(ValueError):
        kv_payload_bytes(per_tok, 1, 1, 1 / 3)


def test_attention_flops_brute_force_and_chunks():
    # brute force: count visible (query, key) pairs one by one
    for q, prefix in ((1, 0), (1, 7), (4, 10), (5, 0)):
        pairs = sum(prefix + j + 1 for j in range(q))
        assert attention_flops(1, 3, 8, q, prefix) == 4 * 3 * 8 * pairs
    # [KVNB §7]: 16 chunks of 512 hold the same causal pairs as 8192 at once
    chunks = [attention_flops(32, 32, 128, 512, p) for p in range(0, 8192, 512)]
    assert sum(chunks) == attention_flops(32, 32, 128, 8192)
    assert chunks[-1] > chunks[0]
    with pytest.raises(ValueError):
        attention_flops(32, 32, 128, -1)
