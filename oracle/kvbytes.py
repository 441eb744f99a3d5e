"""Cache payload arithmetic, written out from the pages' formulas.

Page 1, "KV cache: Generation state, latency, and allocation", section 21.1:
Eq. 21.2 gives the ideal payload across layers as the product of 2 (keys and
values), layers, requests B, KV heads, stored positions T, head width d_h and
bytes per stored scalar s.  Eq. 21.3 gives the growth for one more processed
position in every request of the batch.  Page 2, "KV Cache Explained",
section "How much GPU memory does the KV cache use?", states the same
per-token figure without the batch factor.

All arithmetic is exact Python integers; GiB conversions divide by 1024**3.
"""

from __future__ import annotations

from math import ceil

GIB = 1024 ** 3
MIB = 1024 ** 2
KIB = 1024


def payload_bytes(layers: int, batch: int, kv_heads: int, positions: int,
                  head_dim: int, bytes_per_scalar: int) -> int:
    """Eq. 21.2: every stored K and V scalar counted once."""
    return 2 * layers * batch * kv_heads * positions * head_dim * bytes_per_scalar


def growth_bytes_per_token(layers: int, batch: int, kv_heads: int,
                           head_dim: int, bytes_per_scalar: int) -> int:
    """Eq. 21.3: payload added when each of ``batch`` requests processes one
    more position (use batch=1 for a single request)."""
    return payload_bytes(layers, batch, kv_heads, 1, head_dim, bytes_per_scalar)


def kv_cache_gib(layers: int, batch: int, kv_heads: int, seq_len: int,
                 head_dim: int, bytes_per_value: int = 2) -> float:
    """The page-1 estimate in GiB: Eq. 21.2 divided by 1024**3.

    Page 1, section 21.1, "Code example: A simple KV-cache memory estimate"
    (re-derived from the formula, not transcribed)."""
    return payload_bytes(layers, batch, kv_heads, seq_len, head_dim,
                         bytes_per_value) / GIB


def blocks_for_tokens(tokens: int, block_size: int) -> int:
    """Number of fixed-size blocks that hold ``tokens`` processed positions
    (page 1, section 21.5: logical block of position t is floor(t / bs), so
    positions 0..tokens-1 touch blocks 0..ceil(tokens / bs) - 1)."""
    if tokens <= 0:
        return 0
    return ceil(tokens / block_size)


def tail_waste_slots(tokens: int, block_size: int) -> int:
    """Unused slots in a request's last block (page 3: fragmentation is under
    one block per sequence)."""
    return blocks_for_tokens(tokens, block_size) * block_size - tokens


def decode_step_kv_read_bytes(context_lens, kv_heads: int, head_dim: int,
                              bytes_per_scalar: int) -> int:
    """KV bytes one decode step reads for one layer: Eq. 21.2 applied per
    request with T = n_b (its processed positions after the append) and
    layers = 1, summed over the batch."""
    return sum(payload_bytes(1, 1, kv_heads, int(n), head_dim, bytes_per_scalar)
               for n in context_lens)


def unique_block_bytes(block_tables, context_lens, block_size: int,
                       bytes_per_block: int) -> int:
    """Bytes of distinct physical blocks referenced by the given requests.

    A physical block shared by several tables is counted once (page 2,
    section "Prefix reuse saves prefill, while decode still needs the
    history": one physical copy of the common prefix)."""
    seen = set()
    for row, n in zip(block_tables, context_lens):
        for j in range(blocks_for_tokens(int(n), block_size)):
            seen.add(int(row[j]))
    return len(seen) * bytes_per_block


def transfer_floor_s(nbytes: int, bytes_per_s: float) -> float:
    """Lower bound on the time to move ``nbytes`` between memory tiers at an
    effective rate (page 2 "KV Cache Explained", section "What changes when KV
    moves off the GPU": bytes divided by the link rate; staging, connector and
    contention costs come on top)."""
    if bytes_per_s <= 0:
        raise ValueError("rate must be positive")
    return nbytes / bytes_per_s
