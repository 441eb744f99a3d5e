"""Algorithmic byte counts of one decode step (measurement arithmetic).

The bytes a decode step must move at minimum, independent of how the
kernels are written: each request reads its n_b cached positions of K and V
for every KV head (page 1 "KV cache: Generation state, latency, and
allocation", Eq. 21.2 per request with T = n_b and one layer; page 3
"xf_kv_cache": decode time is, to first order, cache bytes read divided by
memory bandwidth), plus the query, the output, the block-table entries, the
fp8 scales of the blocks read, and the append (new K/V read, one slot
written).  Workspace traffic of split partitions is implementation overhead
and is not counted.
"""

from __future__ import annotations

DTYPE_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}


def _ceil_div(a, b):
    return -(-a // b)


def attention_bytes(lens, H_Q, H_KV, d_h, block_size, kv_dtype, q_dtype) -> dict:
    s = DTYPE_BYTES[kv_dtype]
    sq = DTYPE_BYTES[q_dtype]
    lens = [int(n) for n in lens]
    kv = sum(2 * H_KV * n * d_h * s for n in lens)
    blocks = sum(_ceil_div(n, block_size) for n in lens)
    scales = 2 * H_KV * blocks * 4 if kv_dtype == "fp8_e4m3" else 0
    B = len(lens)
    q = B * H_Q * d_h * sq
    out = B * H_Q * d_h * 4
    table = blocks * 4 + B * 4
    return dict(kv=kv, scales=scales, q=q, out=out, table=table,
                total=kv + scales + q + out + table)


def cascade_attention_bytes(lens, shared_blocks, H_Q, H_KV, d_h, block_size, kv_dtype,
                            q_dtype) -> dict:
    """The step's bytes when every request's table starts with the same
    ``shared_blocks`` blocks and every context covers them: the shared
    positions are read once for the batch (page 2 "KV Cache Explained",
    section "Prefix reuse saves prefill, while decode still needs the
    history": one physical copy serves every request), each request's
    other positions once for itself.  Same other terms as
    ``attention_bytes`` (the shared table entries read once)."""
    s = DTYPE_BYTES[kv_dtype]
    sq = DTYPE_BYTES[q_dtype]
    lens = [int(n) for n in lens]
    shared = shared_blocks * block_size
    if any(n <= shared for n in lens):
        raise ValueError("every context must cover the shared blocks")
    positions = shared + sum(n - shared for n in lens)
    kv = 2 * H_KV * positions * d_h * s
    blocks = shared_blocks + sum(_ceil_div(n, block_size) - shared_blocks for n in lens)
    scales = 2 * H_KV * blocks * 4 if kv_dtype == "fp8_e4m3" else 0
    B = len(lens)
    q = B * H_Q * d_h * sq
    out = B * H_Q * d_h * 4
    table = blocks * 4 + B * 4
    return dict(kv=kv, scales=scales, q=q, out=out, table=table,
                total=kv + scales + q + out + table)


def append_bytes(B, H_KV, d_h, kv_dtype, in_dtype, block_size=None) -> int:
    s = DTYPE_BYTES[kv_dtype]
    si = DTYPE_BYTES[in_dtype]
    scales = 2 * B * H_KV * 4 if kv_dtype == "fp8_e4m3" else 0
    # new K, V read + one slot of K, V written + table entry + length
    return 2 * B * H_KV * d_h * (si + s) + scales + 8 * B
