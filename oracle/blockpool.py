"""Block pool model: free queue, reference counts, immediate release.

Page 1, "KV cache: Generation state, latency, and allocation", section 21.5,
Table 21.1 and the five numbered steps after it:

* the pool is a fixed set of physical block ids, each with ``block_size``
  position slots (page 2, section "Why PagedAttention allocates KV in
  blocks": the pool is initialised up front with a free-block queue);
* allocation takes a free block and records it in the request's table
  (step 2);
* sharing a complete block into another table raises its reference count
  (step 3, count two);
* releasing a request removes its references; a block whose count reaches
  zero returns to the free pool at once (step 4, "immediate-release
  policy"), while a block still referenced stays live (step 4, block 7);
* a shared block that is only partly filled must not be written in place
  (copy-on-write paragraph after the walk): ``prepare_append`` reports that
  case as an error, ``prepare_append_cow`` moves the writer to a fresh block
  and names the block whose contents must be copied into it.

The free pool is a FIFO queue: ``alloc`` pops the head, a release pushes to
the tail.  The pages call it a "free pool", a "free-block queue" (page 2) and
a "free list" (page 3) without fixing an order; FIFO is the plain reading.

Prefix retention (page 1 section 21.5 step 5, and the exercise answer at the
end of that chapter: after its last reference a block is either kept as an
evictable prefix entry or freed; page 2 "KV Cache Explained", sections "Why
PagedAttention allocates KV in blocks" and "Follow the 32 GiB pool until it
cannot allocate one more block": a free-block queue plus a hash-to-block
lookup; a cached block with no running reference stays available for
eviction; allocation uses empty blocks first and then reclaims the oldest
idle cached ones):

* ``cache_blocks`` gives complete blocks of a row their identity
  (``oracle.prefix``); an identity already held by another block leaves the
  new block without one;
* a block whose count reaches zero keeps its identity and joins the queue
  tail like any other free block, so the queue order is the eviction order;
* ``alloc`` pops the head; if that block has an identity the identity is
  dropped (an eviction);
* ``match_prefix`` takes a reference on the block of each leading identity
  that is present, stopping at the first one that is not; a hit on a block
  in the queue takes it out of the queue.
"""

from __future__ import annotations

from collections import deque


class PoolError(Exception):
    """Base class; ``code`` mirrors the status names of the C library."""
    code = "error"


class OutOfBlocks(PoolError):
    code = "out_of_blocks"


class BadBlock(PoolError):
    code = "bad_block"


class SharedBlock(PoolError):
    code = "shared_block"


class InvalidArg(PoolError):
    code = "invalid_arg"


class BlockPool:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise InvalidArg("num_blocks and block_size must be positive")
        if free_order is None:
            free_order = list(range(num_blocks))
        free_order = [int(x) for x in free_order]
        if sorted(free_order) != list(range(num_blocks)):
            raise InvalidArg("free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(free_order)
        self.refcount = [0] * num_blocks
        self.hash_of = {}        # block -> identity
        self.block_of = {}       # identity -> block
        self.queried = 0         # identities asked for by match_prefix
        self.hits = 0            # of those, blocks reused
        self.evictions = 0       # identities dropped by alloc

    # ---- block level -----------------------------------------------------
    def alloc(self) -> int:
        if not self.free:
            raise OutOfBlocks("no free block")
        b = self.free.popleft()
        if b in self.hash_of:
            del self.block_of[self.hash_of.pop(b)]
            self.evictions += 1
        self.refcount[b] = 1
        return b

    def alloc_n(self, n: int) -> list:
        """n blocks from the queue head, or none at all (OutOfBlocks) when
        fewer are free: a request brought back from host memory needs all of
        its blocks (page 3, "End-to-end flow": the victim resumes when blocks
        free up)."""
        if n < 0:
            raise InvalidArg("n must be >= 0")
        if n > len(self.free):
            raise OutOfBlocks(f"{n} blocks needed, {len(self.free)} free")
        return [self.alloc() for _ in range(n)]

    def _check(self, b: int):
        if not (0 <= b < self.num_blocks) or self.refcount[b] == 0:
            raise BadBlock(f"block {b} is not live")

    def incref(self, b: int):
        self._check(b)
        self.refcount[b] += 1

    def decref(self, b: int):
        self._check(b)
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free.append(b)

    def num_free(self) -> int:
        return len(self.free)

    def num_used(self) -> int:
        return self.num_blocks - len(self.free)

    def num_cached_idle(self) -> int:
        """Free blocks that still hold an identity (evictable prefix entries)."""
        return sum(1 for b in self.hash_of if self.refcount[b] == 0)

    def lookup(self, h: bytes):
        return self.block_of.get(bytes(h))

    # ---- sequence level --------------------------------------------------
    def prepare_append(self, table_row: list, ctx_before: int) -> tuple:
        """Make room for the position ``ctx_before`` (zero-based) of one
        request whose table row is ``table_row`` (a Python list that grows).

        Returns (physical block, slot) of the new position.  A new block is
        taken iff the position opens a new logical block (page 1, section
        21.5, step 2); writing into a block with refcount > 1 is refused
        (copy-on-write paragraph)."""
        bs = self.block_size
        j, r = divmod(ctx_before, bs)
        if r == 0:
            if len(table_row) != j:
                raise InvalidArg("table row length does not match ctx_before")
            table_row.append(self.alloc())
        else:
            if len(table_row) != j + 1:
                raise InvalidArg("table row length does not match ctx_before")
        b = table_row[j]
        if self.refcount[b] > 1:
            raise SharedBlock(f"block {b} is shared (refcount {self.refcount[b]})")
        return b, r

    def prepare_append_cow(self, table_row: list, ctx_before: int) -> tuple:
        """Like ``prepare_append``, but a shared target block is not refused:
        the writer gets a private copy first (page 1, section 21.5, the
        copy-on-write paragraph after the walk: shared state is copied before
        a writer changes it, so the other requests keep their view).

        Returns (physical block, slot, source block to copy or None).  The
        new block is taken before the shared one loses this row's reference,
        so an empty pool leaves everything unchanged."""
        bs = self.block_size
        j, r = divmod(ctx_before, bs)
        if r == 0 or len(table_row) != j + 1 or self.refcount[table_row[j]] <= 1:
            b, slot = self.prepare_append(table_row, ctx_before)
            return b, slot, None
        src = table_row[j]
        dst = self.alloc()
        self.decref(src)
        table_row[j] = dst
        return dst, r, src

    def share_prefix(self, src_row: list, n_full_blocks: int) -> list:
        """Map the first ``n_full_blocks`` complete blocks of ``src_row`` into
        a new table row (page 1, section 21.5, step 3)."""
        if n_full_blocks > len(src_row):
            raise InvalidArg("not that many blocks in the source row")
        dst = []
        for j in range(n_full_blocks):
            self.incref(src_row[j])
            dst.append(src_row[j])
        return dst

    def release(self, table_row: list):
        """Drop one reference to every block of a finished request (page 1,
        section 21.5, steps 4 and 5)."""
        for b in table_row:
            self.decref(b)

    # ---- prefix retention ------------------------------------------------
    def match_prefix(self, hashes) -> list:
        """Reuse the longest run of leading identities that are present: one
        more reference on each matched block, a queued block leaves the queue.
        Returns the new table row (the matched blocks, in order)."""
        row = []
        for h in hashes:
            b = self.block_of.get(bytes(h))
            if b is None:
                break
            if self.refcount[b] == 0:
                self.free.remove(b)
            self.refcount[b] += 1
            row.append(b)
        self.queried += len(hashes)
        self.hits += len(row)
        return row

    def cache_blocks(self, table_row: list, ctx_len: int, hashes) -> int:
        """Give the complete blocks of a row (the first ctx_len // block_size,
        at most len(hashes)) their identities.  Returns how many blocks got a
        new identity.  A block that already has a different identity is an
        error (a complete block's contents do not change); checks happen
        before any change."""
        n = min(len(hashes), ctx_len // self.block_size, len(table_row))
        for j in range(n):
            b = table_row[j]
            self._check(b)
            if b in self.hash_of and self.hash_of[b] != bytes(hashes[j]):
                raise InvalidArg(f"block {b} already holds another identity")
        added = 0
        for j in range(n):
            b, h = table_row[j], bytes(hashes[j])
            if b in self.hash_of or h in self.block_of:
                continue
            self.hash_of[b] = h
            self.block_of[h] = b
            added += 1
        return added
