"""Paged KV-cache decode attention for MI355X (gfx950).

A thin Python layer over the C ABI of ``libpkv.so`` (include/pkv.h).  The
functions below only read shapes and raw pointers off torch tensors and pass
them on with the current HIP stream; all work runs in the library's HIP
kernels and host pool.  Importing the package does not load the library;
the first call does, and fails loudly if it has not been built.
"""

from __future__ import annotations

import ctypes as C

from . import _lib
from ._lib import (PKV_BF16, PKV_F32, PKV_FP8_E4M3, PKV_VARIANT_AUTO, PKV_VARIANT_GENERIC,
                   PKV_VARIANT_MFMA, PKV_VARIANT_MFMA_PARTITION, PkvError, check, load)

__all__ = ["kv_append", "copy_blocks", "decode_plan", "decode_workspace_size", "decode_step_noalloc", "cascade_partitions", "paged_decode_attention", "decode_partitions",
           "combine_partitions", "set_decode_variant", "BlockPool", "PkvError", "load",
           "prefix_root", "block_hashes", "DIGEST_BYTES", "kv_append_chunk",
           "paged_chunk_attention", "swap_record_bytes", "swap_out", "swap_in", "decode_step",
           "cascade_plan", "decode_step_cascade",
           "PKV_F32", "PKV_BF16", "PKV_FP8_E4M3", "PKV_VARIANT_AUTO", "PKV_VARIANT_GENERIC",
           "PKV_VARIANT_MFMA", "PKV_VARIANT_MFMA_PARTITION", "dtype_code"]


DIGEST_BYTES = _lib.PKV_DIGEST_BYTES


def prefix_root(identity: bytes) -> bytes:
    """h_0: SHA-256 of the configuration / isolation identity bytes
    (pkv_prefix_root)."""
    lib = load()
    identity = bytes(identity)
    out = (C.c_uint8 * DIGEST_BYTES)()
    check(lib.pkv_prefix_root(identity, len(identity), out), "pkv_prefix_root")
    return bytes(out)


def block_hashes(parent: bytes, tokens, block_size: int) -> bytes:
    """Chained identities of the complete blocks of ``tokens`` (an int32
    sequence or numpy array), as one bytes object of 32 bytes per block
    (pkv_block_hashes)."""
    import numpy as np
    lib = load()
    toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    parent = bytes(parent)
    if len(parent) != DIGEST_BYTES:
        raise PkvError(-1, "pkv_block_hashes")
    nb = len(toks) // block_size if block_size > 0 else 0
    out = (C.c_uint8 * max(1, nb * DIGEST_BYTES))()
    n = C.c_int64()
    check(lib.pkv_block_hashes(parent, toks.ctypes.data_as(C.POINTER(C.c_int32)), len(toks),
                               block_size, out, nb, C.byref(n)), "pkv_block_hashes")
    return bytes(out)[:n.value * DIGEST_BYTES]


def dtype_code(t) -> int:
    """pkv_dtype of a tensor (float32, bfloat16, float8_e4m3fn / uint8)."""
    return _dtype_code(t)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return PKV_FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def kv_append(k_new, v_new, k_cache, v_cache, block_table, context_lens,
              k_scale=None, v_scale=None, stream=None):
    """pkv_kv_append: write k_new/v_new [B, H_KV, d_h] into slot
    context_lens[b] - 1 of each request (lengths after the append)."""
    B, H_KV, d_h = k_new.shape
    num_blocks, _, bs, _ = k_cache.shape
    check(load().pkv_kv_append(_ptr(k_new), _ptr(v_new), _dtype_code(k_new), _ptr(k_cache),
                               _ptr(v_cache), _dtype_code(k_cache), _ptr(k_scale),
                               _ptr(v_scale), _ptr(block_table), block_table.shape[1],
                               _ptr(context_lens), B, H_KV, d_h, bs, num_blocks,
                               _stream(stream)), "pkv_kv_append")


def kv_append_chunk(k_new, v_new, k_cache, v_cache, block_table, context_lens, query_start,
                    k_scale=None, v_scale=None, stream=None):
    """pkv_kv_append_chunk: rows of k_new/v_new [total, H_KV, d_h] go to the
    last n_b positions of request b (n_b from query_start [B + 1])."""
    total, H_KV, d_h = k_new.shape
    num_blocks, _, bs, _ = k_cache.shape
    B = context_lens.shape[0]
    check(load().pkv_kv_append_chunk(_ptr(k_new), _ptr(v_new), _dtype_code(k_new),
                                     _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache),
                                     _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
                                     block_table.shape[1], _ptr(context_lens),
                                     _ptr(query_start), B, total, H_KV, d_h, bs, num_blocks,
                                     _stream(stream)), "pkv_kv_append_chunk")


def paged_chunk_attention(out, q, k_cache, v_cache, block_table, context_lens, query_start,
                          max_q_len, max_context_len, softmax_scale, k_scale=None,
                          v_scale=None, stream=None):
    """pkv_paged_chunk_attention: out [total, H_Q, d_h] float32."""
    total, H_Q, d_h = q.shape
    num_blocks, H_KV, bs, _ = k_cache.shape
    B = context_lens.shape[0]
    check(load().pkv_paged_chunk_attention(_ptr(out), _ptr(q), _dtype_code(q), _ptr(k_cache),
                                           _ptr(v_cache), _dtype_code(k_cache), _ptr(k_scale),
                                           _ptr(v_scale), _ptr(block_table),
                                           block_table.shape[1], _ptr(context_lens),
                                           _ptr(query_start), B, total, max_q_len,
                                           max_context_len, H_Q, H_KV, d_h, bs, num_blocks,
                                           softmax_scale, _stream(stream)),
          "pkv_paged_chunk_attention")


def swap_record_bytes(kv_dtype: int, H_KV: int, d_h: int, block_size: int):
    """pkv_swap_record_bytes -> (block_bytes, record_bytes)."""
    blk, rec = C.c_size_t(), C.c_size_t()
    check(load().pkv_swap_record_bytes(kv_dtype, H_KV, d_h, block_size, C.byref(blk),
                                       C.byref(rec)), "pkv_swap_record_bytes")
    return blk.value, rec.value


def swap_out(k_cache, v_cache, blocks, records, k_scale=None, v_scale=None, stream=None):
    """pkv_swap_out: blocks is a device int32 tensor [n]; records a pinned
    host (or device) uint8 tensor of at least n * record_bytes."""
    num_blocks, H_KV, bs, d_h = k_cache.shape
    check(load().pkv_swap_out(_ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache), _ptr(k_scale),
                              _ptr(v_scale), _ptr(blocks), blocks.shape[0], H_KV, d_h, bs,
                              num_blocks, _ptr(records), _stream(stream)), "pkv_swap_out")


def swap_in(k_cache, v_cache, blocks, records, k_scale=None, v_scale=None, stream=None):
    """pkv_swap_in: the inverse of swap_out, into the listed blocks."""
    num_blocks, H_KV, bs, d_h = k_cache.shape
    check(load().pkv_swap_in(_ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache), _ptr(k_scale),
                             _ptr(v_scale), _ptr(blocks), blocks.shape[0], H_KV, d_h, bs,
                             num_blocks, _ptr(records), _stream(stream)), "pkv_swap_in")


def copy_blocks(k_cache, v_cache, pairs, k_scale=None, v_scale=None, stream=None):
    """pkv_copy_blocks: pairs is a device int32 tensor [n, 2] of (src, dst)."""
    num_blocks, H_KV, bs, d_h = k_cache.shape
    check(load().pkv_copy_blocks(_ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache),
                                 _ptr(k_scale), _ptr(v_scale), _ptr(pairs), pairs.shape[0], H_KV,
                                 d_h, bs, num_blocks, _stream(stream)), "pkv_copy_blocks")


def decode_plan(B, H_Q, H_KV, d_h, block_size, max_context_len, partition_tokens=0,
                q_dtype=PKV_BF16, kv_dtype=PKV_BF16):
    """pkv_decode_plan -> (partition_tokens, max_partitions, workspace_bytes).

    q_dtype / kv_dtype are pkv_dtype codes (see dtype_code)."""
    pt, parts, ws = C.c_int32(), C.c_int32(), C.c_size_t()
    check(load().pkv_decode_plan(B, H_Q, H_KV, d_h, block_size, max_context_len,
                                 partition_tokens, int(q_dtype), int(kv_dtype), C.byref(pt),
                                 C.byref(parts), C.byref(ws)),
          "pkv_decode_plan")
    return pt.value, parts.value, ws.value


def decode_workspace_size(B, H_Q, H_KV, d_h, block_size, max_context_len, partition_tokens=0,
                          q_dtype=PKV_BF16, kv_dtype=PKV_BF16):
    """pkv_decode_workspace_size -> bytes: enough for every kernel variant."""
    ws = C.c_size_t()
    check(load().pkv_decode_workspace_size(B, H_Q, H_KV, d_h, block_size, max_context_len,
                                           partition_tokens, int(q_dtype), int(kv_dtype),
                                           C.byref(ws)),
          "pkv_decode_workspace_size")
    return ws.value


def _attn_args(out, q, k_cache, v_cache, block_table, context_lens, max_context_len,
               softmax_scale, k_scale, v_scale, partition_tokens, workspace, stream):
    B, H_Q, d_h = q.shape
    num_blocks, H_KV, bs, _ = k_cache.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_ptr(out), _ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache),
            _dtype_code(k_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
            block_table.shape[1], _ptr(context_lens), int(max_context_len), B, H_Q, H_KV, d_h,
            bs, num_blocks, float(softmax_scale), int(partition_tokens), _ptr(workspace),
            ws_bytes, _stream(stream))


def paged_decode_attention(out, q, k_cache, v_cache, block_table, context_lens,
                           max_context_len, softmax_scale, k_scale=None, v_scale=None,
                           partition_tokens=0, workspace=None, stream=None):
    """pkv_paged_decode_attention: out [B, H_Q, d_h] fp32."""
    check(load().pkv_paged_decode_attention(*_attn_args(
        out, q, k_cache, v_cache, block_table, context_lens, max_context_len, softmax_scale,
        k_scale, v_scale, partition_tokens, workspace, stream)), "pkv_paged_decode_attention")


def decode_step(k_new, v_new, out, q, k_cache, v_cache, block_table, context_lens,
                max_context_len, softmax_scale, k_scale=None, v_scale=None, partition_tokens=0,
                workspace=None, stream=None):
    """pkv_decode_step: append k_new / v_new [B, H_KV, d_h], then attend."""
    check(load().pkv_decode_step(_ptr(k_new), _ptr(v_new), *_attn_args(
        out, q, k_cache, v_cache, block_table, context_lens, max_context_len, softmax_scale,
        k_scale, v_scale, partition_tokens, workspace, stream)), "pkv_decode_step")


def decode_step_noalloc(k_new, v_new, out, q, k_cache, v_cache, block_table, context_lens,
                        max_context_len, softmax_scale, k_scale=None, v_scale=None,
                        partition_tokens=0, stream=None):
    """pkv_decode_step_noalloc: pkv_decode_step with the library's static
    device workspace (no caller workspace, nothing allocated)."""
    args = _attn_args(out, q, k_cache, v_cache, block_table, context_lens, max_context_len,
                      softmax_scale, k_scale, v_scale, partition_tokens, None, stream)
    # drop the workspace pointer and size of the plain step's argument list
    args = args[:-3] + args[-1:]
    check(load().pkv_decode_step_noalloc(_ptr(k_new), _ptr(v_new), *args),
          "pkv_decode_step_noalloc")


def cascade_plan(B, H_Q, H_KV, d_h, block_size, max_context_len, shared_blocks,
                 q_dtype=PKV_BF16, kv_dtype=PKV_BF16):
    """pkv_cascade_plan -> (prefix splits, workspace_bytes)."""
    sp, ws = C.c_int32(), C.c_size_t()
    check(load().pkv_cascade_plan(B, H_Q, H_KV, d_h, block_size, max_context_len, shared_blocks,
                                  q_dtype, kv_dtype, C.byref(sp), C.byref(ws)),
          "pkv_cascade_plan")
    return sp.value, ws.value


def decode_step_cascade(k_new, v_new, out, q, k_cache, v_cache, block_table, context_lens,
                        max_context_len, softmax_scale, shared_blocks, k_scale=None,
                        v_scale=None, workspace=None, stream=None):
    """pkv_decode_step_cascade: k_new / v_new may be None (no append)."""
    B, H_Q, d_h = q.shape
    num_blocks, H_KV, bs, _ = k_cache.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(load().pkv_decode_step_cascade(
        _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(q), _dtype_code(q), _ptr(k_cache),
        _ptr(v_cache), _dtype_code(k_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
        block_table.shape[1], _ptr(context_lens), int(max_context_len), B, H_Q, H_KV, d_h, bs,
        num_blocks, softmax_scale, int(shared_blocks), _ptr(workspace), ws_bytes,
        _stream(stream)), "pkv_decode_step_cascade")


def cascade_partitions(out, q, k_cache, v_cache, block_table, context_lens, max_context_len,
                       softmax_scale, shared_blocks, k_scale=None, v_scale=None, workspace=None,
                       stream=None):
    """pkv_cascade_partitions: the cascade's attention kernel alone."""
    B, H_Q, d_h = q.shape
    num_blocks, H_KV, bs, _ = k_cache.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(load().pkv_cascade_partitions(
        _ptr(out), _ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(k_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_table), block_table.shape[1],
        _ptr(context_lens), int(max_context_len), B, H_Q, H_KV, d_h, bs, num_blocks,
        softmax_scale, int(shared_blocks), _ptr(workspace), ws_bytes, _stream(stream)),
        "pkv_cascade_partitions")


def decode_partitions(out, q, k_cache, v_cache, block_table, context_lens, max_context_len,
                      softmax_scale, k_scale=None, v_scale=None, partition_tokens=0,
                      workspace=None, stream=None):
    """pkv_decode_partitions: the partition kernel alone."""
    check(load().pkv_decode_partitions(*_attn_args(
        out, q, k_cache, v_cache, block_table, context_lens, max_context_len, softmax_scale,
        k_scale, v_scale, partition_tokens, workspace, stream)), "pkv_decode_partitions")


def combine_partitions(out, context_lens, max_context_len, H_KV, block_size,
                       partition_tokens=0, workspace=None, stream=None):
    """pkv_combine_partitions: the split-K combine kernel alone."""
    B, H_Q, d_h = out.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(load().pkv_combine_partitions(_ptr(out), _ptr(context_lens), int(max_context_len), B,
                                        H_Q, H_KV, d_h, block_size, int(partition_tokens),
                                        _ptr(workspace), ws_bytes, _stream(stream)),
          "pkv_combine_partitions")


def set_decode_variant(variant: int) -> int:
    """pkv_set_decode_variant; returns the previous value."""
    return load().pkv_set_decode_variant(int(variant))


class BlockPool:
    """The library's host block pool (pkv_pool_*, pkv_seq_*)."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        lib = load()
        h = C.c_void_p()
        arr = None
        if free_order is not None:
            free_order = [int(x) for x in free_order]
            arr = (C.c_int32 * len(free_order))(*free_order)
            if len(free_order) != num_blocks:
                raise PkvError(-1, "pkv_pool_create")
        check(lib.pkv_pool_create(num_blocks, block_size, arr, C.byref(h)), "pkv_pool_create")
        self._h = h
        self._lib = lib
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if self._h:
            self._lib.pkv_pool_destroy(self._h)
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self) -> int:
        b = C.c_int32()
        check(self._lib.pkv_pool_alloc(self._h, C.byref(b)), "pkv_pool_alloc")
        return b.value

    def alloc_n(self, n: int) -> list:
        ids = (C.c_int32 * max(1, n))()
        check(self._lib.pkv_pool_alloc_n(self._h, n, ids), "pkv_pool_alloc_n")
        return list(ids[:n])

    def incref(self, block: int):
        check(self._lib.pkv_pool_incref(self._h, block), "pkv_pool_incref")

    def decref(self, block: int):
        check(self._lib.pkv_pool_decref(self._h, block), "pkv_pool_decref")

    def refcount(self, block: int) -> int:
        r = C.c_int32()
        check(self._lib.pkv_pool_refcount(self._h, block, C.byref(r)), "pkv_pool_refcount")
        return r.value

    def num_free(self) -> int:
        r = C.c_int32()
        check(self._lib.pkv_pool_num_free(self._h, C.byref(r)), "pkv_pool_num_free")
        return r.value

    def num_used(self) -> int:
        r = C.c_int32()
        check(self._lib.pkv_pool_num_used(self._h, C.byref(r)), "pkv_pool_num_used")
        return r.value

    def free_queue(self) -> list:
        n = C.c_int32()
        buf = (C.c_int32 * max(1, self.num_blocks))()
        check(self._lib.pkv_pool_free_queue(self._h, buf, self.num_blocks, C.byref(n)),
              "pkv_pool_free_queue")
        return list(buf[:n.value])

    def prepare_append(self, row, n_blocks: int, ctx_before: int):
        """row: a ctypes int32 array (the host table row, updated in place).
        Returns (n_blocks_after, block, slot)."""
        nb, blk, slot = C.c_int32(n_blocks), C.c_int32(), C.c_int32()
        check(self._lib.pkv_seq_prepare_append(self._h, row, len(row), ctx_before,
                                               C.byref(nb), C.byref(blk), C.byref(slot)),
              "pkv_seq_prepare_append")
        return nb.value, blk.value, slot.value

    def prepare_append_cow(self, row, n_blocks: int, ctx_before: int):
        """Returns (n_blocks_after, block, slot, cow_src); cow_src is -1 unless
        a shared block had to be replaced by a private copy."""
        nb, blk, slot, src = C.c_int32(n_blocks), C.c_int32(), C.c_int32(), C.c_int32()
        check(self._lib.pkv_seq_prepare_append_cow(self._h, row, len(row), ctx_before,
                                                   C.byref(nb), C.byref(blk), C.byref(slot),
                                                   C.byref(src)),
              "pkv_seq_prepare_append_cow")
        return nb.value, blk.value, slot.value, src.value

    def share_prefix(self, src_row, n_full_blocks: int, dst_row):
        check(self._lib.pkv_seq_share_prefix(self._h, src_row, n_full_blocks, dst_row),
              "pkv_seq_share_prefix")

    def release(self, row, n_blocks: int):
        check(self._lib.pkv_seq_release(self._h, row, n_blocks), "pkv_seq_release")

    # ---- prefix identity and retention ------------------------------------
    def lookup(self, digest: bytes) -> int:
        b = C.c_int32()
        check(self._lib.pkv_pool_lookup(self._h, bytes(digest), C.byref(b)), "pkv_pool_lookup")
        return b.value

    def match_prefix(self, hashes: bytes, row) -> int:
        """hashes: concatenated 32-byte identities; row: ctypes int32 array
        (the new request's table row).  Returns the number of blocks matched."""
        hashes = bytes(hashes)
        n = C.c_int32()
        check(self._lib.pkv_pool_match_prefix(self._h, hashes, len(hashes) // DIGEST_BYTES, row,
                                              len(row), C.byref(n)), "pkv_pool_match_prefix")
        return n.value

    def cache_blocks(self, row, n_blocks: int, ctx_len: int, hashes: bytes) -> int:
        hashes = bytes(hashes)
        n = C.c_int32()
        check(self._lib.pkv_pool_cache_blocks(self._h, row, n_blocks, ctx_len, hashes,
                                              len(hashes) // DIGEST_BYTES, C.byref(n)),
              "pkv_pool_cache_blocks")
        return n.value

    def prefix_stats(self) -> dict:
        st = (C.c_int64 * 5)()
        check(self._lib.pkv_pool_prefix_stats(self._h, st), "pkv_pool_prefix_stats")
        return dict(queried=st[0], hits=st[1], evictions=st[2], cached_idle=st[3],
                    hashed=st[4])
