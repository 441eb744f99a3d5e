"""Chained block identities for prefix reuse.

Test infrastructure only: the library never imports this module.

Page 1, "KV cache: Generation state, latency, and allocation", section 21.4:
the identity of block i combines the identity of block i-1 with the exact
token ids of block i, starting from an identity h_0 of the compatible
configuration, so h_i = hash(h_{i-1}, tokens_i).  Only complete blocks get
an identity (the same section: the documented design reuses full blocks).
Page 2, "KV Cache Explained", section "Cache identity is a correctness
boundary": SHA-256 is the documented hash; every identity field (model,
adapter, position settings, isolation salt) belongs in the key.

Byte encoding (the pages fix none; this is the reading used by both sides):

* h_0 = SHA-256(identity bytes), where the caller's identity bytes name the
  configuration and any isolation salt;
* h_i = SHA-256(h_{i-1} || tokens_i), h_{i-1} as its 32 digest bytes and
  the block's ``block_size`` token ids as little-endian int32.

``hashlib.sha256`` is the hash primitive; the tests pin it to the FIPS 180-4
example digests.
"""

from __future__ import annotations

import hashlib
import struct

DIGEST_BYTES = 32


def root(identity: bytes) -> bytes:
    """h_0 of a configuration / isolation domain."""
    return hashlib.sha256(bytes(identity)).digest()


def block_hash(parent: bytes, block_tokens) -> bytes:
    """h_i = hash(h_{i-1}, tokens_i) for one complete block."""
    if len(parent) != DIGEST_BYTES:
        raise ValueError("parent identity must be 32 bytes")
    toks = [int(t) for t in block_tokens]
    return hashlib.sha256(bytes(parent) + struct.pack(f"<{len(toks)}i", *toks)).digest()


def block_hashes(parent: bytes, tokens, block_size: int) -> list:
    """Identities of every complete block of ``tokens``, in order; a trailing
    partial block has none."""
    if block_size <= 0:
        raise ValueError("block_size must be positive")
    toks = [int(t) for t in tokens]
    out = []
    h = bytes(parent)
    for j in range(len(toks) // block_size):
        h = block_hash(h, toks[j * block_size:(j + 1) * block_size])
        out.append(h)
    return out
