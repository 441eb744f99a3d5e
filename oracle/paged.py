"""Paged attention for decode steps and chunks of new tokens: slot mapping,
append, gather, exact attention (float64).

Sources on the pages (page 1 = "KV cache: Generation state, latency, and
allocation"; page 3 = "xf_kv_cache"):

* Slot mapping -- page 1, section 21.5: position t of a request lies in
  logical block floor(t / bs) at slot t mod bs, and the request's block table
  gives the physical block.
* Append -- page 1, section 21.6, Eq. 21.6: each decode pass appends the
  consumed token's K and V to the cache, keeping logical order; section
  21.1: the new query reads the cached keys *and its own new key*.  So the
  append happens first and attention covers n_b positions, where n_b counts
  the positions after the append.
* Validity -- page 1, section 21.1 (after Eq. 21.1): unused slots must never
  be read as keys; section 21.5: occupancy marks valid slots.  Positions
  >= n_b are never gathered.
* Grouped heads -- page 1, section 21.1: H_Q must be divisible by H_KV and
  every query head keeps its own scores.  Query head hq reads KV head
  floor(hq / g), g = H_Q / H_KV (contiguous groups; the pages leave the
  assignment open).
* Attention -- page 1, section 21.1: scores are normalised and mix the
  values.  With scale c: s_t = c * q . k_t, w_t = exp(s_t - max s),
  out = sum_t w_t v_t / sum_t w_t.  Subtracting the maximum changes nothing
  mathematically and keeps exp() in range.
* Chunks of new tokens -- page 1, section 21.3 (chunked prefill): a prompt
  may be processed in portions; later portions keep the positions and the
  cached state of the earlier ones.  A chunk of n new tokens of a request
  whose cache holds ctx positions after the chunk's append occupies
  positions ctx - n .. ctx - 1, and its query i, at position
  p = ctx - n + i, reads every position up to and including p (section
  21.1: a query reads the cached keys of earlier positions and its own).
  Page 3, "End-to-end flow": the new tokens of a prefix hit attend to the
  shared prefix through the same block table.  A decode step is the chunk
  of one token.

Storage formats (``kv_dtype``): "f32" (float32 arrays), "bf16" (uint16 bit
patterns), "fp8_e4m3" (uint8 codes with one float32 scale per (physical
block, KV head); stored value = code value * scale).  Query and new-token
inputs are "f32" or "bf16".  Pools are laid out [num_blocks, H_KV, bs, d_h]
for K and V separately.
"""

from __future__ import annotations

import numpy as np

from . import codecs

F32, BF16, FP8 = "f32", "bf16", "fp8_e4m3"


def _in_to_f64(x, dtype: str) -> np.ndarray:
    if dtype == F32:
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return codecs.bf16_bits_to_f64(x)
    raise ValueError(f"unsupported input dtype {dtype}")


def slot_of(block_table_row, position: int, block_size: int) -> tuple:
    """(physical block, slot) holding zero-based logical ``position``."""
    j, r = divmod(int(position), int(block_size))
    return int(block_table_row[j]), r


def append(k_cache, v_cache, kv_dtype: str, k_new, v_new, in_dtype: str,
           block_table, context_lens, block_size: int,
           k_scale=None, v_scale=None, inplace=False):
    """Write each request's new K, V into slot (n_b - 1); return the pools
    (new copies unless ``inplace``).

    Stored form: the same bits for f32 -> f32 and bf16 -> bf16; for fp8, the
    E4M3FN code of fp32(x) / scale[p, h] (see ``codecs``).  Every other pool
    byte is left untouched."""
    kc = k_cache if inplace else np.array(k_cache, copy=True)
    vc = v_cache if inplace else np.array(v_cache, copy=True)
    num_blocks = kc.shape[0]
    B, H_KV, _ = np.shape(k_new)
    for b in range(B):
        n = int(context_lens[b])
        if n < 1:
            raise ValueError("context length after append must be >= 1")
        p, r = slot_of(block_table[b], n - 1, block_size)
        if not 0 <= p < num_blocks:
            raise ValueError(f"block id {p} outside the pool")
        for h in range(H_KV):
            for src, dst, sc in ((k_new, kc, k_scale), (v_new, vc, v_scale)):
                x = np.asarray(src[b, h])
                if kv_dtype == in_dtype:
                    dst[p, h, r, :] = x
                elif kv_dtype == FP8:
                    xf = _in_to_f64(x, in_dtype).astype(np.float32)  # exact
                    dst[p, h, r, :] = codecs.e4m3_quantize(xf, np.float32(sc[p, h]))
                else:
                    raise ValueError(f"unsupported append {in_dtype} -> {kv_dtype}")
    return kc, vc


def _chunk_bounds(query_start, B):
    qs = [int(x) for x in query_start]
    if len(qs) != B + 1 or qs[0] != 0 or any(qs[b + 1] < qs[b] for b in range(B)):
        raise ValueError("query_start must be a non-decreasing prefix sum starting at 0")
    return qs


def append_chunk(k_cache, v_cache, kv_dtype: str, k_new, v_new, in_dtype: str,
                 block_table, context_lens, query_start, block_size: int,
                 k_scale=None, v_scale=None, inplace=False):
    """Write each request's chunk of new K, V rows: row query_start[b] + i of
    k_new / v_new ([total, H_KV, d_h]) goes to position ctx_b - n_b + i,
    n_b = query_start[b + 1] - query_start[b].  Stored form as in
    ``append``; every other pool byte is left untouched."""
    kc = k_cache if inplace else np.array(k_cache, copy=True)
    vc = v_cache if inplace else np.array(v_cache, copy=True)
    num_blocks = kc.shape[0]
    B = len(context_lens)
    qs = _chunk_bounds(query_start, B)
    H_KV = np.shape(k_new)[1]
    for b in range(B):
        n_new, ctx = qs[b + 1] - qs[b], int(context_lens[b])
        if n_new > ctx:
            raise ValueError("a chunk cannot be longer than the context after it")
        for i in range(n_new):
            p, r = slot_of(block_table[b], ctx - n_new + i, block_size)
            if not 0 <= p < num_blocks:
                raise ValueError(f"block id {p} outside the pool")
            for h in range(H_KV):
                for src, dst, sc in ((k_new, kc, k_scale), (v_new, vc, v_scale)):
                    x = np.asarray(src[qs[b] + i, h])
                    if kv_dtype == in_dtype:
                        dst[p, h, r, :] = x
                    elif kv_dtype == FP8:
                        xf = _in_to_f64(x, in_dtype).astype(np.float32)  # exact
                        dst[p, h, r, :] = codecs.e4m3_quantize(xf, np.float32(sc[p, h]))
                    else:
                        raise ValueError(f"unsupported append {in_dtype} -> {kv_dtype}")
    return kc, vc


def copy_blocks(k_cache, v_cache, pairs, k_scale=None, v_scale=None):
    """Copy-on-write block copies: block dst takes every stored byte (all KV
    heads, all slots) and the scales of block src, for each (src, dst) pair.
    Returns new arrays (the inputs are not modified)."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    ks = None if k_scale is None else np.array(k_scale, copy=True)
    vs = None if v_scale is None else np.array(v_scale, copy=True)
    for src, dst in pairs:
        kc[dst] = k_cache[src]
        vc[dst] = v_cache[src]
        if ks is not None:
            ks[dst] = k_scale[src]
            vs[dst] = v_scale[src]
    return kc, vc, ks, vs


# ---- swap to host and back -------------------------------------------------
#
# Page 1, section 21.3: offloading moves retained cache state to another
# memory tier (CPU memory) and a later operation brings the needed blocks
# back; it changes placement and data movement, not which positions a query
# reads.  Page 3, "End-to-end flow": a preempted request's blocks are swapped
# to pinned host memory and copied back when blocks free up, instead of being
# recomputed.  Page 2, section "What changes when KV moves off the GPU": the
# byte count sets the transfer floor.
#
# Record of one block in the host buffer (the pages fix no format; this is
# the layout both sides use): the block's K bytes (all KV heads, all slots,
# [H_KV][bs][d_h] as stored), then its V bytes, then for fp8 caches the
# block's K scales and V scales ([H_KV] float32 each); the record is padded
# with unspecified bytes to a multiple of 256.

SWAP_ALIGN = 256


def swap_record_bytes(kv_dtype: str, H_KV: int, d_h: int, block_size: int) -> tuple:
    """(bytes of one block's K (or V), bytes of one padded record)."""
    elem = {F32: 4, BF16: 2, FP8: 1}[kv_dtype]
    blk = H_KV * block_size * d_h * elem
    rec = 2 * blk + (2 * H_KV * 4 if kv_dtype == FP8 else 0)
    return blk, -(-rec // SWAP_ALIGN) * SWAP_ALIGN


def swap_out(k_cache, v_cache, kv_dtype: str, blocks, k_scale=None, v_scale=None):
    """Host records of the listed blocks, in list order: uint8 [n, record]
    (padding bytes zero here; the library leaves them unspecified)."""
    nb, H_KV, bs, d_h = k_cache.shape
    blk, rec = swap_record_bytes(kv_dtype, H_KV, d_h, bs)
    out = np.zeros((len(blocks), rec), dtype=np.uint8)
    for i, b in enumerate(blocks):
        if not 0 <= int(b) < nb:
            raise ValueError(f"block id {b} outside the pool")
        out[i, :blk] = np.ascontiguousarray(k_cache[b]).view(np.uint8).reshape(-1)
        out[i, blk:2 * blk] = np.ascontiguousarray(v_cache[b]).view(np.uint8).reshape(-1)
        if kv_dtype == FP8:
            o = 2 * blk
            out[i, o:o + 4 * H_KV] = np.asarray(k_scale[b], dtype="<f4").view(np.uint8)
            out[i, o + 4 * H_KV:o + 8 * H_KV] = np.asarray(v_scale[b], dtype="<f4").view(np.uint8)
    return out


def swap_in(k_cache, v_cache, kv_dtype: str, blocks, records, k_scale=None, v_scale=None):
    """Write record i into block blocks[i]; returns new (k, v, k_scale,
    v_scale) arrays (the inputs are not modified)."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    ks = None if k_scale is None else np.array(k_scale, copy=True)
    vs = None if v_scale is None else np.array(v_scale, copy=True)
    nb, H_KV, bs, d_h = kc.shape
    blk, rec = swap_record_bytes(kv_dtype, H_KV, d_h, bs)
    for i, b in enumerate(blocks):
        if not 0 <= int(b) < nb:
            raise ValueError(f"block id {b} outside the pool")
        r = np.asarray(records[i], dtype=np.uint8)
        kc[b] = r[:blk].view(kc.dtype).reshape(kc.shape[1:])
        vc[b] = r[blk:2 * blk].view(vc.dtype).reshape(vc.shape[1:])
        if kv_dtype == FP8:
            o = 2 * blk
            ks[b] = r[o:o + 4 * H_KV].view("<f4")
            vs[b] = r[o + 4 * H_KV:o + 8 * H_KV].view("<f4")
    return kc, vc, ks, vs


def decode_stored(pool_slice, kv_dtype: str, scale=None) -> np.ndarray:
    """Stored scalars -> float64 values (exact)."""
    if kv_dtype == F32:
        return np.asarray(pool_slice, dtype=np.float32).astype(np.float64)
    if kv_dtype == BF16:
        return codecs.bf16_bits_to_f64(pool_slice)
    if kv_dtype == FP8:
        return codecs.e4m3_decode(pool_slice) * float(scale)
    raise ValueError(f"unsupported kv dtype {kv_dtype}")


def gather_head(cache, kv_dtype: str, scale, table_row, n: int, h: int,
                block_size: int) -> np.ndarray:
    """Dense float64 [n, d_h] keys (or values) of KV head ``h`` of one request,
    in logical order, read through its table: the paged form turned back into
    Eq. 21.1's layout for B = 1 and T = n."""
    t = np.arange(n)
    p = np.asarray(table_row, dtype=np.int64)[t // block_size]   # physical block per position
    r = t % block_size                                           # slot per position
    if kv_dtype == FP8:
        return codecs.e4m3_decode(cache[p, h, r]) * np.asarray(scale, np.float64)[p, h][:, None]
    return decode_stored(cache[p, h, r], kv_dtype)


def attend_one(q_rows, K, V, softmax_scale: float) -> np.ndarray:
    """Exact softmax attention of several query rows over one key/value set.

    q_rows [g, d], K [n, d], V [n, d] (float64) -> [g, d]."""
    s = (q_rows @ K.T) * softmax_scale                      # [g, n]
    w = np.exp(s - s.max(axis=1, keepdims=True))
    return (w @ V) / w.sum(axis=1, keepdims=True)


def attend(q, q_dtype: str, k_cache, v_cache, kv_dtype: str, block_table,
           context_lens, block_size: int, softmax_scale: float,
           k_scale=None, v_scale=None, requests=None) -> np.ndarray:
    """float64 output [B, H_Q, d_h] of one decode query per request.

    ``requests`` optionally restricts the computation to some request
    indices (the others are left as NaN), for sampled checks at full size."""
    qf = _in_to_f64(q, q_dtype)
    B, H_Q, d_h = qf.shape
    H_KV = k_cache.shape[1]
    if H_Q % H_KV:
        raise ValueError("H_Q must be divisible by H_KV")
    g = H_Q // H_KV
    out = np.full((B, H_Q, d_h), np.nan, dtype=np.float64)
    for b in (range(B) if requests is None else requests):
        n = int(context_lens[b])
        for h in range(H_KV):
            K = gather_head(k_cache, kv_dtype, k_scale, block_table[b], n, h, block_size)
            V = gather_head(v_cache, kv_dtype, v_scale, block_table[b], n, h, block_size)
            out[b, h * g:(h + 1) * g] = attend_one(qf[b, h * g:(h + 1) * g], K, V,
                                                    softmax_scale)
    return out


def attend_chunk(q, q_dtype: str, k_cache, v_cache, kv_dtype: str, block_table,
                 context_lens, query_start, block_size: int, softmax_scale: float,
                 k_scale=None, v_scale=None, requests=None) -> np.ndarray:
    """float64 output [total, H_Q, d_h] of every new query of every chunk:
    query row query_start[b] + i (position p = ctx_b - n_b + i) attends to
    positions 0..p of request b.  ``requests`` restricts the computation to
    some requests (the other rows are NaN)."""
    qf = _in_to_f64(q, q_dtype)
    total, H_Q, d_h = qf.shape
    H_KV = k_cache.shape[1]
    if H_Q % H_KV:
        raise ValueError("H_Q must be divisible by H_KV")
    g = H_Q // H_KV
    B = len(context_lens)
    qs = _chunk_bounds(query_start, B)
    if qs[B] != total:
        raise ValueError("query_start[B] must equal the number of query rows")
    out = np.full((total, H_Q, d_h), np.nan, dtype=np.float64)
    for b in (range(B) if requests is None else requests):
        n_new, ctx = qs[b + 1] - qs[b], int(context_lens[b])
        if n_new == 0:
            continue
        if n_new > ctx:
            raise ValueError("a chunk cannot be longer than the context after it")
        for h in range(H_KV):
            K = gather_head(k_cache, kv_dtype, k_scale, block_table[b], ctx, h, block_size)
            V = gather_head(v_cache, kv_dtype, v_scale, block_table[b], ctx, h, block_size)
            for i in range(n_new):
                p = ctx - n_new + i
                out[qs[b] + i, h * g:(h + 1) * g] = attend_one(
                    qf[qs[b] + i, h * g:(h + 1) * g], K[:p + 1], V[:p + 1], softmax_scale)
    return out


def chunk_step(q, q_dtype, k_new, v_new, k_cache, v_cache, kv_dtype, block_table,
               context_lens, query_start, block_size, softmax_scale, k_scale=None,
               v_scale=None, requests=None, inplace=False):
    """Append every request's chunk, then attend with every new query.

    Returns (k_cache_after, v_cache_after, out)."""
    kc, vc = append_chunk(k_cache, v_cache, kv_dtype, k_new, v_new, q_dtype, block_table,
                          context_lens, query_start, block_size, k_scale, v_scale, inplace)
    out = attend_chunk(q, q_dtype, kc, vc, kv_dtype, block_table, context_lens, query_start,
                       block_size, softmax_scale, k_scale, v_scale, requests)
    return kc, vc, out


def decode_step(q, q_dtype, k_new, v_new, k_cache, v_cache, kv_dtype,
                block_table, context_lens, block_size, softmax_scale,
                k_scale=None, v_scale=None, requests=None, inplace=False):
    """Append, then attend (page 1, section 21.1 and Eq. 21.6).

    Returns (k_cache_after, v_cache_after, out)."""
    kc, vc = append(k_cache, v_cache, kv_dtype, k_new, v_new, q_dtype,
                    block_table, context_lens, block_size, k_scale, v_scale, inplace)
    out = attend(q, q_dtype, kc, vc, kv_dtype, block_table, context_lens,
                 block_size, softmax_scale, k_scale, v_scale, requests)
    return kc, vc, out
