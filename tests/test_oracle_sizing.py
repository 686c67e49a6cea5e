"""Pins of the oracle's size arithmetic against the pages' worked examples."""

import json
import os

import pytest

from oracle import sizing

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_sizes.json"),
                      encoding="utf-8"))


@pytest.mark.parametrize("case", GOLD["cases"], ids=lambda c: c["name"])
def test_printed_examples(case):
    got = sizing.kv_bytes_total(case["layers"], case["kv_heads"], case["seq_len"],
                                case["head_dim"], case["dtype_bytes"])
    assert got == case["exact"]
    if "printed_gb" in case:      # the page rounds to decimal GB
        assert round(got / 1e9, 2 if got < 1e10 else 1) == case["printed_gb"]
    if "printed_mib" in case:
        assert round(got / 2**20, 2) == case["printed_mib"]


def test_concurrent_example():
    c = GOLD["concurrent"]
    got = c["requests"] * sizing.kv_bytes_total(c["layers"], c["kv_heads"], c["seq_len"],
                                                c["head_dim"], c["dtype_bytes"])
    assert got == c["exact"]
    assert round(got / 1e9) == c["printed_gb"]


def test_per_layer_linear_in_seq_len():
    # 4096 x seq_len bytes per layer for the 70B shape, for every length
    for L in (1, 15, 16, 33, 4096, 5120, 32768):
        assert sizing.kv_bytes_per_layer(8, L, 128, 2) == 4096 * L


def test_paged_pool_equals_formula_when_blocks_are_full():
    # a pool holding exactly the blocks of one 4096-token request (16-token
    # blocks) has the size the per-request formula gives
    nb = sizing.blocks_for_tokens(4096, 16)
    assert nb == 256
    assert sizing.paged_pool_bytes(80, nb, 16, 8, 128, 2) == 1342177280
    nb32k = sizing.blocks_for_tokens(32768, 16)
    assert sizing.paged_pool_bytes(80, nb32k, 16, 8, 128, 2) == 10737418240
    assert sizing.paged_pool_bytes(80, 100 * nb, 16, 8, 128, 2) == 134217728000


def test_quantised_storage_halves_bytes():
    # FP8 / INT8 storage halves the K/V bytes ("KV Cache 原理与 PagedAttention",
    # §四 table); per-token-head scales add 4 bytes per (token, head) for K and V
    bf16 = sizing.paged_pool_bytes(1, 1024, 32, 8, 128, 2)
    fp8 = sizing.paged_pool_bytes(1, 1024, 32, 8, 128, 1)
    int8 = sizing.paged_pool_bytes(1, 1024, 32, 8, 128, 1, per_token_head_scales=True)
    assert fp8 * 2 == bf16
    assert int8 - fp8 == 2 * 1024 * 32 * 8 * 4


def test_blocks_for_tokens_waste_bound():
    for B in (8, 16, 32):
        for n in range(0, 200):
            nb = sizing.blocks_for_tokens(n, B)
            assert nb * B >= n
            assert nb * B - n <= B - 1
