"""Pins of the oracle's block-pool model to the Table 21.1 walk (page 1,
section 21.5) and to the pages' release and copy-on-write rules."""

import json
import os

import pytest

from oracle import blockpool, paged

WALK = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "table_21_1_walk.json")))


def _initial_state():
    pool = blockpool.BlockPool(WALK["num_blocks"], WALK["block_size"], WALK["free_order"])
    rows = {}
    for name in ("A", "B"):
        spec = WALK["initial"][name]
        row = []
        for pos in range(spec["tokens"]):
            pool.prepare_append(row, pos)
        assert row == spec["blocks"], name
        rows[name] = row
    return pool, rows


def test_table_21_1_initial_and_reads():
    pool, rows = _initial_state()
    assert list(pool.free)[0] == 5
    for r in WALK["reads"]:
        assert paged.slot_of(rows[r["request"]], r["position"], WALK["block_size"]) == (r["block"], r["slot"])


def test_table_21_1_walk():
    pool, rows = _initial_state()
    for a in WALK["appends"]:
        row = rows[a["request"]]
        nb = len(row)
        blk, slot = pool.prepare_append(row, a["position"])
        assert (blk, slot) == (a["block"], a["slot"])
        assert (len(row) > nb) == a["new_block"]
        # the read of the just-written position goes through the same mapping
        assert paged.slot_of(row, a["position"], WALK["block_size"]) == (blk, slot)
    sh = WALK["share"]
    rows[sh["to"]] = pool.share_prefix(rows[sh["from"]], sh["blocks"])
    assert pool.refcount[sh["block"]] == sh["refcount_after"]

    free_before = set(pool.free)
    pool.release(rows.pop("A"))
    ra = WALK["release_A"]
    assert set(pool.free) - free_before == set(ra["freed"])
    assert pool.refcount[7] == ra["refcount_7"] and pool.refcount[9] == ra["refcount_9"]

    free_before = set(pool.free)
    pool.release(rows.pop("C"))
    assert set(pool.free) - free_before == set(WALK["release_C"]["freed"])
    free_before = set(pool.free)
    pool.release(rows.pop("B"))
    assert set(pool.free) - free_before == set(WALK["release_B"]["freed"])
    assert pool.num_free() == WALK["num_blocks"]


def test_release_order_is_fifo_tail():
    pool, rows = _initial_state()
    pool.release(rows["A"])          # 7 then 2 released, pushed behind the others
    assert list(pool.free)[-2:] == [7, 2]


def test_shared_partial_block_refuses_write():
    # copy-on-write paragraph: a partly filled shared block needs a private copy
    pool, rows = _initial_state()
    c = pool.share_prefix(rows["A"], 2)          # shares block 2 (2 of 4 slots)
    with pytest.raises(blockpool.SharedBlock):
        pool.prepare_append(rows["A"], 6)
    with pytest.raises(blockpool.SharedBlock):
        pool.prepare_append(c, 6)


def test_exhaustion_and_bad_blocks():
    pool = blockpool.BlockPool(2, 4)
    a = pool.alloc()
    pool.alloc()
    with pytest.raises(blockpool.OutOfBlocks):
        pool.alloc()
    pool.decref(a)
    with pytest.raises(blockpool.BadBlock):
        pool.decref(a)              # already free
    with pytest.raises(blockpool.BadBlock):
        pool.incref(a)              # cannot share a free block
    with pytest.raises(blockpool.BadBlock):
        pool.decref(7)              # not in the pool


def test_checkpoint_block_freed_only_after_last_reference():
    # page 1, chapter checkpoint: a block still referenced by another request
    # cannot be freed
    pool, rows = _initial_state()
    c = pool.share_prefix(rows["B"], 1)
    pool.release(rows["B"])
    assert 9 not in pool.free
    pool.release(c)
    assert 9 in pool.free


def test_pool_walk_32gib_exhaustion_page_2():
    # 16,384 block-equivalents; pin: allocation succeeds exactly 16,384 times
    pool = blockpool.BlockPool(16384, 16)
    for _ in range(16384):
        pool.alloc()
    with pytest.raises(blockpool.OutOfBlocks):
        pool.alloc()


def test_copy_on_write_keeps_the_other_view():
    # page 1, section 21.5, copy-on-write paragraph: C shares A's partly
    # filled block 2 (2 of 4 slots); A's next write must go to a private copy
    pool, rows = _initial_state()
    c = pool.share_prefix(rows["A"], 2)
    assert pool.refcount[2] == 2
    with pytest.raises(blockpool.SharedBlock):
        pool.prepare_append(list(rows["A"]), 6)
    blk, slot, src = pool.prepare_append_cow(rows["A"], 6)
    assert (blk, slot, src) == (5, 2, 2)          # the only free id of Table 21.1 is 5
    assert rows["A"] == [7, 5] and c == [7, 2]
    assert pool.refcount[2] == 1 and pool.refcount[5] == 1 and pool.refcount[7] == 2
    # C, now the only holder of block 2, appends in place
    assert pool.prepare_append_cow(c, 6) == (2, 2, None)
    # a full pool refuses the copy and changes nothing
    p2 = blockpool.BlockPool(2, 4)
    r1 = []
    for pos in range(2):
        p2.prepare_append(r1, pos)
    r2 = p2.share_prefix(r1, 1)
    p2.alloc()
    with pytest.raises(blockpool.OutOfBlocks):
        p2.prepare_append_cow(r1, 2)
    assert r1 == r2 and p2.refcount[r1[0]] == 2


def test_copy_on_write_data_flow():
    # the copy preserves every earlier position of both requests, and only the
    # writer sees its new token
    import numpy as np

    from oracle import paged
    rng = np.random.default_rng(0)
    pool = blockpool.BlockPool(8, 4)
    a = []
    for pos in range(6):
        pool.prepare_append(a, pos)
    c = pool.share_prefix(a, 2)
    kc = rng.standard_normal((8, 1, 4, 2)).astype(np.float32)
    vc = rng.standard_normal((8, 1, 4, 2)).astype(np.float32)
    before_a = paged.gather_head(kc, "f32", None, a, 6, 0, 4)
    blk, slot, src = pool.prepare_append_cow(a, 6)
    kc, vc, _, _ = paged.copy_blocks(kc, vc, [(src, blk)])
    new = np.full((1, 1, 2), 9.0, dtype=np.float32)
    kc, vc = paged.append(kc, vc, "f32", new, new, "f32", np.array([a]), np.array([7]), 4)
    after_a = paged.gather_head(kc, "f32", None, a, 7, 0, 4)
    after_c = paged.gather_head(kc, "f32", None, c, 6, 0, 4)
    assert np.array_equal(after_a[:6], before_a)
    assert np.array_equal(after_a[6], [9.0, 9.0])
    assert np.array_equal(after_c, before_a)
