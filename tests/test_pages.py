"""Pins of the oracle's byte arithmetic to the numbers the pages print.

Every expected value below comes from tests/golden/page_arithmetic.json,
whose entries cite the page and section that print it."""

import json
import os

import pytest

from oracle import kvbytes

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "page_arithmetic.json")))


@pytest.mark.parametrize("case", GOLD["payload"], ids=lambda c: str(c["bytes"]))
def test_payload_eq_21_2(case):
    assert kvbytes.payload_bytes(*case["args"]) == case["bytes"]


@pytest.mark.parametrize("case", GOLD["tensor_values"], ids=lambda c: str(c["values"]))
def test_single_tensor_values(case):
    # one layer, one tensor (K alone): Eq. 21.2 without the factor 2, s=1 -> values
    vals = kvbytes.payload_bytes(1, 1, case["kv_heads"], case["positions"],
                                 case["head_dim"], 1) // 2
    assert vals == case["values"]
    if "bytes_at_2" in case:
        assert vals * 2 == case["bytes_at_2"]


@pytest.mark.parametrize("case", GOLD["growth_per_token"], ids=lambda c: str(c["bytes"]))
def test_growth_eq_21_3(case):
    assert kvbytes.growth_bytes_per_token(*case["args"]) == case["bytes"]


def test_growth_sequence_section_21_6():
    # 1280 -> 1536 -> 1792 -> 2048, +256 per processed position
    seq = [kvbytes.payload_bytes(2, 1, 4, t, 8, 2) for t in range(5, 9)]
    assert seq == [1280, 1536, 1792, 2048]
    assert all(b - a == kvbytes.growth_bytes_per_token(2, 1, 4, 8, 2)
               for a, b in zip(seq, seq[1:]))


def test_growth_example_21_1_selection_before_append():
    # 24 bytes after a 3-token prompt; 32 once token four is processed
    before = kvbytes.payload_bytes(1, 1, 1, 3, 2, 2)
    after = kvbytes.payload_bytes(1, 1, 1, 4, 2, 2)
    assert (before, after) == (24, 32)
    assert after - before == kvbytes.growth_bytes_per_token(1, 1, 1, 2, 2)


@pytest.mark.parametrize("case", GOLD["gib"], ids=lambda c: str(c["gib"]))
def test_kv_cache_gib(case):
    assert kvbytes.kv_cache_gib(*case["args"]) == case["gib"]


def test_pool_capacity_page_2():
    g = GOLD["pool_capacity"]
    pool = g["pool_gib"] * kvbytes.GIB
    for tokens, histories in g["histories"]:
        assert pool // (tokens * g["per_token_bytes"]) == histories
    assert g["block_tokens"] * g["per_token_bytes"] == g["block_bytes_all_layers"]
    assert pool // g["block_bytes_all_layers"] == g["blocks_in_pool"]
    assert kvbytes.blocks_for_tokens(32768, g["block_tokens"]) == g["blocks_for_32768_tokens"]
    # the per-token figure itself is Eq. 21.3 with B = 1 for the 8B-style model
    assert kvbytes.growth_bytes_per_token(32, 1, 8, 128, 2) == g["per_token_bytes"]


def test_prefix_sharing_saving_page_2():
    g = GOLD["prefix_sharing"]
    per = g["per_token_bytes"]
    bs = 16
    n = g["seq_tokens"]
    nshared = g["shared_tokens"] // bs
    nblk = kvbytes.blocks_for_tokens(n, bs)
    # two tables: private copies vs the first 16,384 tokens mapped to shared blocks
    copies = [list(range(0, nblk)), list(range(nblk, 2 * nblk))]
    shared = [list(range(0, nblk)),
              list(range(0, nshared)) + list(range(nblk, nblk + nblk - nshared))]
    blk_bytes = bs * per
    assert kvbytes.unique_block_bytes(copies, [n, n], bs, blk_bytes) == g["copies_gib"] * kvbytes.GIB
    assert kvbytes.unique_block_bytes(shared, [n, n], bs, blk_bytes) == g["shared_gib"] * kvbytes.GIB
    assert (g["copies_gib"] - g["shared_gib"]) == g["saving_gib"]


def test_shared_prefix_flow_page_3():
    g = GOLD["shared_prefix_flow"]
    assert kvbytes.blocks_for_tokens(g["prefix_tokens"], g["block_size"]) == g["prefix_blocks"]
    assert kvbytes.tail_waste_slots(g["prefix_tokens"], g["block_size"]) == 0
    # a fresh block every 16 tokens: the block count grows exactly at multiples of 16
    steps = [kvbytes.blocks_for_tokens(1200 + i, 16) - kvbytes.blocks_for_tokens(1200 + i - 1, 16)
             for i in range(1, 65)]
    assert [i + 1 for i, s in enumerate(steps) if s] == [1, 17, 33, 49]
    # fragmentation under one block per sequence
    assert all(kvbytes.tail_waste_slots(n, 16) < 16 for n in range(1, 2000))


def test_checkpoint_cached_positions():
    g = GOLD["checkpoint"]
    # selection does not append: the cache holds the processed prompt only
    assert g["cached_positions_at_first_selection"] == g["prompt_tokens"]
    assert kvbytes.blocks_for_tokens(g["prompt_tokens"], 4) == 2


@pytest.mark.parametrize("case", GOLD["transfer_floor"])
def test_transfer_floor_page_2(case):
    t = kvbytes.transfer_floor_s(case["bytes"], case["bytes_per_s"])
    assert round(t, case["digits"]) == case["seconds_rounded"]
    # the 4 GiB is the 32,768-token prefix of the same page (Eq. 21.2)
    assert case["bytes"] == kvbytes.payload_bytes(32, 1, 8, 32768, 128, 2)
