"""One interface over the oracle's pool model and the library's host pool,
so that a walk written once runs on both and their states can be compared.
Rows are handled as Python lists on the outside."""

from __future__ import annotations

import ctypes as C

import paged_kv_cache_105_amd as pkv
from oracle import blockpool


class OracleDriver:
    OutOfBlocks = blockpool.OutOfBlocks

    def __init__(self, num_blocks, block_size, free_order=None):
        self.p = blockpool.BlockPool(num_blocks, block_size, free_order)
        self.block_size = block_size

    def new_row(self, cap):
        return []

    def blocks(self, row):
        return list(row)

    def open_blocks(self, row, n_new):
        """Take n_new more blocks for a row whose positions fill whole blocks."""
        for _ in range(n_new):
            self.p.prepare_append(row, len(row) * self.block_size)

    def append_positions(self, row, ctx_before, n):
        for t in range(ctx_before, ctx_before + n):
            self.p.prepare_append(row, t)

    def match(self, hashes, cap):
        return self.p.match_prefix(hashes)

    def cache(self, row, ctx_len, hashes):
        return self.p.cache_blocks(row, ctx_len, hashes)

    def release(self, row):
        self.p.release(row)
        row.clear()

    def lookup(self, h):
        b = self.p.lookup(h)
        return -1 if b is None else b

    def alloc(self):
        return self.p.alloc()

    def stats(self):
        return dict(queried=self.p.queried, hits=self.p.hits, evictions=self.p.evictions,
                    cached_idle=self.p.num_cached_idle(), hashed=len(self.p.hash_of))

    def num_free(self):
        return self.p.num_free()

    def free_queue(self):
        return list(self.p.free)

    def refcount(self, b):
        return self.p.refcount[b]


class _LibRow:
    def __init__(self, cap):
        self.arr = (C.c_int32 * cap)()
        self.n = 0


class LibDriver:
    OutOfBlocks = pkv.PkvError

    def __init__(self, num_blocks, block_size, free_order=None):
        self.p = pkv.BlockPool(num_blocks, block_size, free_order)
        self.block_size = block_size

    def new_row(self, cap):
        return _LibRow(cap)

    def blocks(self, row):
        return list(row.arr[:row.n])

    def open_blocks(self, row, n_new):
        for _ in range(n_new):
            row.n, _, _ = self.p.prepare_append(row.arr, row.n, row.n * self.block_size)

    def append_positions(self, row, ctx_before, n):
        for t in range(ctx_before, ctx_before + n):
            row.n, _, _ = self.p.prepare_append(row.arr, row.n, t)

    def match(self, hashes, cap):
        row = _LibRow(cap)
        row.n = self.p.match_prefix(b"".join(hashes), row.arr)
        return row

    def cache(self, row, ctx_len, hashes):
        return self.p.cache_blocks(row.arr, row.n, ctx_len, b"".join(hashes))

    def release(self, row):
        self.p.release(row.arr, row.n)
        row.n = 0

    def lookup(self, h):
        return self.p.lookup(h)

    def alloc(self):
        return self.p.alloc()

    def stats(self):
        return self.p.prefix_stats()

    def num_free(self):
        return self.p.num_free()

    def free_queue(self):
        return self.p.free_queue()

    def refcount(self, b):
        return self.p.refcount(b)


DRIVERS = {"oracle": OracleDriver, "library": LibDriver}
