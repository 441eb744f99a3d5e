/*
 * pkv.h -- C ABI of the paged KV-cache decode library (MI355X / gfx950).
 *
 * One decode step for one layer: append each request's new key and value
 * to its slot, then let each query head attend over every cached position of
 * its request, reading the cache through a block table.  All terms follow
 * page 1, "KV cache: Generation state, latency, and allocation":
 *
 *   - K, V of one layer are B x H_KV x T x d_h (section 21.1, Eq. 21.1);
 *     here T is spread over fixed-size blocks of `block_size` slots;
 *   - H_Q must be divisible by H_KV; query head hq reads KV head hq / g,
 *     g = H_Q / H_KV, and keeps its own scores (section 21.1);
 *   - position t of a request lives in logical block t / block_size, slot
 *     t % block_size; the block table maps the logical block to a physical
 *     block of the pool (section 21.5, Table 21.1);
 *   - the new token's K and V are appended first and the query reads them
 *     too (section 21.1; section 21.6, Eq. 21.6), so `context_lens` counts
 *     positions AFTER the append;
 *   - blocks come from a pool with a free queue and reference counts, and a
 *     block returns to the pool when its last reference goes (section
 *     21.5, steps 2-5; page 2 "KV Cache Explained", section "Why
 *     PagedAttention allocates KV in blocks").
 *
 * Memory layout (device, caller-owned):
 *   k_cache, v_cache : [num_blocks][H_KV][block_size][d_h] of kv_dtype,
 *                      separate K and V arrays per layer
 *   k_scale, v_scale : [num_blocks][H_KV] float, fp8 only (stored value =
 *                      E4M3 code value * scale), NULL otherwise
 *   block_table      : [B][max_blocks_per_seq] int32, row-major; entries
 *                      past a request's last block are never read;
 *                      max_blocks_per_seq * block_size <= INT32_MAX
 *                      (positions are int32), else PKV_ERR_INVALID_ARG
 *   context_lens     : [B] int32, positions after the append, >= 1
 *   q                : [B][H_Q][d_h] of q_dtype
 *   k_new, v_new     : [B][H_KV][d_h] of q_dtype
 *   out              : [B][H_Q][d_h] float
 *
 * Conventions:
 *   - every function returns a pkv_status; nothing throws across the ABI;
 *   - device functions are asynchronous on `stream` (a hipStream_t, NULL =
 *     the default stream); argument checks happen on the host before any
 *     launch, and a failed check launches nothing;
 *   - the library never allocates device memory: the caller passes every
 *     device buffer, including the attention workspace;
 *   - device-side values are trusted to be in range; a block id outside
 *     [0, num_blocks) or a context length outside [1, max_blocks_per_seq *
 *     block_size] is clamped (attention) or skipped (append) so that no
 *     access leaves the caller's buffers, and the results for that request
 *     are unspecified;
 *   - the pool is host-only, never touches device memory and is not
 *     thread-safe: callers serialise access to one pool.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,   /* bad shape, pointer, dtype or size          */
  PKV_ERR_OUT_OF_BLOCKS = -2, /* pool has no free block                     */
  PKV_ERR_BAD_BLOCK = -3,     /* block id not live (free or out of range)   */
  PKV_ERR_SHARED_BLOCK = -4,  /* write into a block whose refcount > 1      */
  PKV_ERR_HIP = -5,           /* a HIP launch or runtime call failed        */
  PKV_ERR_WORKSPACE = -6,     /* workspace missing or too small             */
  PKV_ERR_UNSUPPORTED = -7    /* valid but not implemented (dtype pair ...) */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

typedef void* pkv_stream_t; /* hipStream_t */

/* Human-readable name of a status code (static string, never NULL). */
const char* pkv_status_string(int status);

/* ABI version of this header (bumped on incompatible change). */
int pkv_abi_version(void);

/* ------------------------------------------------------------------------
 * Host block pool (page 1 section 21.5 Table 21.1 and steps 1-5; page 2
 * "Why PagedAttention allocates KV in blocks"; page 3 "xf_kv_cache",
 * "End-to-end flow": private blocks return to the free list, shared ones
 * only lose a reference).
 *
 * The free pool is a FIFO queue: alloc pops the head, a block whose count
 * drops to zero is pushed to the tail.  All functions leave the pool
 * unchanged when they return an error.
 * ---------------------------------------------------------------------- */
typedef struct pkv_pool pkv_pool;

/* Create a pool of `num_blocks` blocks of `block_size` slots.  `free_order`
 * (nullable) is the initial queue order and must be a permutation of
 * 0..num_blocks-1; NULL means 0, 1, 2, ...  *out receives a handle owned by
 * the library (free it with pkv_pool_destroy).  INVALID_ARG on bad sizes or
 * a non-permutation. */
int pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                    pkv_pool** out);
void pkv_pool_destroy(pkv_pool* pool);

/* Pop the queue head, set its refcount to 1.  OUT_OF_BLOCKS if empty. */
int pkv_pool_alloc(pkv_pool* pool, int32_t* block_id);
/* Pop n blocks from the queue head into ids[0..n), each with refcount 1,
 * or none at all: OUT_OF_BLOCKS (and no change) if fewer than n are free.
 * For bringing a swapped-out request back, which needs all of its blocks
 * (page 3 "xf_kv_cache", "End-to-end flow"). */
int pkv_pool_alloc_n(pkv_pool* pool, int32_t n, int32_t* ids);
/* Map a live block into one more table (section 21.5 step 3).  BAD_BLOCK
 * if the block is free or out of range. */
int pkv_pool_incref(pkv_pool* pool, int32_t block_id);
/* Drop one reference; at zero the block goes to the queue tail (step 4).
 * BAD_BLOCK if the block is free or out of range. */
int pkv_pool_decref(pkv_pool* pool, int32_t block_id);
int pkv_pool_refcount(const pkv_pool* pool, int32_t block_id, int32_t* out);
int pkv_pool_num_free(const pkv_pool* pool, int32_t* out);
int pkv_pool_num_used(const pkv_pool* pool, int32_t* out);
/* Copy the current free queue, head first, into `ids` (capacity `cap`);
 * *count receives the queue length.  INVALID_ARG if cap is too small. */
int pkv_pool_free_queue(const pkv_pool* pool, int32_t* ids, int32_t cap, int32_t* count);

/* Make room for zero-based position `ctx_before` of one request whose host
 * table row holds *n_blocks entries (capacity max_blocks).  Takes a new
 * block iff ctx_before % block_size == 0 (section 21.5 step 2) and then
 * increments *n_blocks.  Returns the target physical block and slot in
 * *block_out / *slot_out.  INVALID_ARG if *n_blocks does not match
 * ctx_before or the row is full; OUT_OF_BLOCKS if no block is free;
 * SHARED_BLOCK if the target block has refcount > 1 (copy-on-write,
 * section 21.5, is not done by this call). */
int pkv_seq_prepare_append(pkv_pool* pool, int32_t* table_row, int32_t max_blocks,
                           int32_t ctx_before, int32_t* n_blocks, int32_t* block_out,
                           int32_t* slot_out);
/* Copy-on-write variant of pkv_seq_prepare_append (page 1 section 21.5, the
 * paragraph after the walk: shared state is copied before a writer changes
 * it, preserving the other requests' view).  When the target block is
 * partly filled and shared (refcount > 1), a new block replaces it in this
 * row, this row's reference moves from the shared block to the new one, and
 * *cow_src receives the shared block: the caller must copy its contents into
 * *block_out (pkv_copy_blocks, every layer) before appending.  Otherwise it
 * behaves like pkv_seq_prepare_append and sets *cow_src = -1.
 * OUT_OF_BLOCKS (and no change) if a copy is needed and no block is free. */
int pkv_seq_prepare_append_cow(pkv_pool* pool, int32_t* table_row, int32_t max_blocks,
                               int32_t ctx_before, int32_t* n_blocks, int32_t* block_out,
                               int32_t* slot_out, int32_t* cow_src);
/* Map the first n_blocks blocks of src_row into dst_row, one more reference
 * each (section 21.5 step 3; sharing a partly filled last block makes the
 * next writer of that block copy it, see above).  BAD_BLOCK if any is not
 * live. */
int pkv_seq_share_prefix(pkv_pool* pool, const int32_t* src_row, int32_t n_full_blocks,
                         int32_t* dst_row);
/* Drop one reference to each of the n_blocks blocks (steps 4-5).  Checks
 * all ids first; BAD_BLOCK (and no change) if any is not live, or if a
 * block appears more often than it has references. */
int pkv_seq_release(pkv_pool* pool, const int32_t* table_row, int32_t n_blocks);

/* ------------------------------------------------------------------------
 * Prefix identity and retention (page 1 section 21.4, the chained block
 * identities h_i = hash(h_{i-1}, tokens_i), and section 21.5 step 5; page 2
 * "KV Cache Explained", sections "Why PagedAttention allocates KV in
 * blocks", "Follow the 32 GiB pool until it cannot allocate one more block"
 * and "Cache identity is a correctness boundary").
 *
 * An identity is a 32-byte SHA-256 digest (FIPS 180-4):
 *   h_0 = SHA-256(identity bytes of the configuration and isolation salt)
 *   h_i = SHA-256(h_{i-1} || tokens of block i as little-endian int32)
 * Only complete blocks have an identity.
 *
 * A block of the pool may hold one identity; the pool maps each identity it
 * holds to one block.  A block keeps its identity after its last reference
 * and joins the free queue tail like any other block ("cached" is not
 * "pinned"); the queue order is therefore the eviction order.  When alloc
 * (or a prepare_append that opens a block, or a copy-on-write) takes a
 * block that still holds an identity, the identity is dropped (an eviction).
 * Blocks without identities behave exactly as in the plain pool above.
 * ---------------------------------------------------------------------- */
#define PKV_DIGEST_BYTES 32

/* out[32] = h_0 = SHA-256 of the n identity bytes.  The bytes should name
 * everything that makes cached K/V interchangeable (model revision,
 * adapter, position settings, cache dtype and layout, isolation salt). */
int pkv_prefix_root(const void* identity, size_t n, uint8_t* out);
/* Identities of the n_tokens / block_size complete blocks of `tokens`
 * (token ids), chained from `parent` (h_0, or the identity of the block
 * before the first one given).  out: [cap_blocks][32]; *n_out receives the
 * number of complete blocks.  INVALID_ARG (nothing written) if cap_blocks is
 * smaller than that.  A trailing partial block gets no identity. */
int pkv_block_hashes(const uint8_t* parent, const int32_t* tokens, int64_t n_tokens,
                     int32_t block_size, uint8_t* out, int64_t cap_blocks, int64_t* n_out);
/* Block that holds `digest`, or -1 in *block_id.  Changes nothing. */
int pkv_pool_lookup(const pkv_pool* pool, const uint8_t* digest, int32_t* block_id);
/* Start a request's table row from retained blocks: for j = 0, 1, ...
 * while j < min(n_hashes, max_blocks) and hashes[j] (of [n_hashes][32]) is
 * held by a block, take one reference on that block (an idle cached block
 * leaves the free queue) and write it to table_row[j].  Stops at the first
 * identity not held.  *n_hit receives the number of blocks matched, which
 * is the row's new block count; the caller continues with
 * pkv_seq_prepare_append from position n_hit * block_size.  Counts
 * n_hashes identities asked for and n_hit reused in the statistics. */
int pkv_pool_match_prefix(pkv_pool* pool, const uint8_t* hashes, int32_t n_hashes,
                          int32_t* table_row, int32_t max_blocks, int32_t* n_hit);
/* Give the complete blocks of a row their identities: for j <
 * min(n_hashes, ctx_len / block_size, n_blocks), block table_row[j] gets
 * hashes[j] unless it already holds it, or another block already holds
 * that identity (the block then stays without one).  *n_cached receives the
 * number of blocks that got an identity.  BAD_BLOCK if one of those blocks
 * is not live; INVALID_ARG if one already holds a different identity (a
 * complete block's contents do not change).  Both checks run first, and a
 * failed check changes nothing. */
int pkv_pool_cache_blocks(pkv_pool* pool, const int32_t* table_row, int32_t n_blocks,
                          int32_t ctx_len, const uint8_t* hashes, int32_t n_hashes,
                          int32_t* n_cached);
/* stats[5] = { identities asked for by match_prefix, blocks reused,
 * identities evicted, free blocks that hold an identity, blocks that hold
 * an identity }. */
int pkv_pool_prefix_stats(const pkv_pool* pool, int64_t* stats);

/* ------------------------------------------------------------------------
 * Device entry points
 * ---------------------------------------------------------------------- */

/* Append (page 1 section 21.6, Eq. 21.6; slot rule of section 21.5).
 * For every request b: t = context_lens[b] - 1, p = block_table[b][t /
 * block_size], r = t % block_size, and for every KV head h
 *   k_cache[p][h][r][:] = store(k_new[b][h][:]),  same for V.
 * store is a bit copy when in_dtype == kv_dtype (F32 or BF16), and for
 * kv_dtype FP8_E4M3 the OCP E4M3 code of fp32(x) / scale[p][h] rounded to
 * nearest even and saturated to +-448 (NaN stays NaN).  Supported
 * (in_dtype, kv_dtype): (F32, F32), (BF16, BF16), (BF16, FP8_E4M3),
 * (F32, FP8_E4M3).  Every other pool byte is left untouched.  Requests
 * whose slot is not writable (length or block id out of range) are
 * skipped.  Requests must not share the written block. */
int pkv_kv_append(const void* k_new, const void* v_new, int in_dtype, void* k_cache,
                  void* v_cache, int kv_dtype, const float* k_scale, const float* v_scale,
                  const int32_t* block_table, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, int32_t B, int32_t H_KV, int32_t d_h,
                  int32_t block_size, int32_t num_blocks, pkv_stream_t stream);

/* Block copies for copy-on-write (page 1 section 21.5): for each pair i of
 * `pairs` (device int32 [n_pairs][2] = (src, dst)), every stored byte of
 * physical block src -- all KV heads and slots of K and of V -- and, for
 * FP8_E4M3 caches, its k/v scales are copied to block dst.  No block may
 * appear in two pairs as a destination, or as both a source and a
 * destination.  Pairs with an id outside [0, num_blocks) are skipped. */
int pkv_copy_blocks(void* k_cache, void* v_cache, int kv_dtype, float* k_scale, float* v_scale,
                    const int32_t* pairs, int32_t n_pairs, int32_t H_KV, int32_t d_h,
                    int32_t block_size, int32_t num_blocks, pkv_stream_t stream);

/* Work split (split-K) planning for paged_decode_attention.  The attention
 * kernels cut each request's positions into pieces whose partial results a
 * combine kernel merges:
 *   - the MFMA kernel (default where it applies: d_h = 128, block_size = 16,
 *     BF16 query with a BF16 or FP8 cache, H_Q / H_KV <= 32, B <= 8192)
 *     splits the blocks of all (request, KV head) sequences into one equal
 *     chunk per wave the device holds at once, so every wave reads the same
 *     number of blocks whatever the length mix;
 *   - the generic kernel (and the MFMA kernel when forced with
 *     PKV_VARIANT_MFMA_PARTITION) cut each request into partitions of
 *     `partition_tokens` positions (a multiple of block_size; 0 picks the
 *     library default for this shape).
 * *partition_tokens_out receives the partition length used by the
 * partition kernels, *max_partitions_out = ceil(max_context_len /
 * partition_tokens), and *workspace_bytes the device workspace the
 * attention call needs for these shapes and dtypes on the current device
 * (0 when no partial results can arise).  The result depends on the
 * variant selected by pkv_set_decode_variant at the time of the call. */
int pkv_decode_plan(int32_t B, int32_t H_Q, int32_t H_KV, int32_t d_h, int32_t block_size,
                    int32_t max_context_len, int32_t partition_tokens, int q_dtype,
                    int kv_dtype, int32_t* partition_tokens_out, int32_t* max_partitions_out,
                    size_t* workspace_bytes);

/* Workspace size for pkv_paged_decode_attention, pkv_decode_partitions and
 * pkv_decode_step with these shapes and dtypes: the largest size any kernel
 * variant needs (the plan above gives the size of the variant selected at
 * the time of that call only), so a workspace of this size serves every
 * call with these arguments whatever pkv_set_decode_variant holds when it
 * runs.  Sizes are for the device current at the call (the balanced split
 * has one chunk per wave the device holds at once); a call on a device
 * that needs more returns PKV_ERR_WORKSPACE and launches nothing.
 * INVALID_ARG for invalid shapes or a NULL workspace_bytes; UNSUPPORTED if
 * no kernel takes the shapes. */
int pkv_decode_workspace_size(int32_t B, int32_t H_Q, int32_t H_KV, int32_t d_h,
                              int32_t block_size, int32_t max_context_len,
                              int32_t partition_tokens, int q_dtype, int kv_dtype,
                              size_t* workspace_bytes);

/* Paged decode attention (page 1 section 21.1: every query head normalises
 * its scores over the request's cached keys, its own new key included, and
 * mixes the values; section 21.5: attention follows the block table).  For
 * request b, query head hq, KV head h = hq / (H_Q / H_KV), n = context_lens[b]:
 *   s_t = softmax_scale * q[b][hq] . K_t   for t < n  (K_t read at the
 *         table's block and slot; fp8 values are code * k_scale[p][h])
 *   out[b][hq][:] = sum_t exp(s_t - max s) V_t / sum_t exp(s_t - max s)
 * computed in fp32.  Slots at positions >= n are never read as keys or
 * values (they may hold anything, NaN included).  `max_context_len` (a host
 * value) must be >= every context_lens[b]; it sizes the grid.  Supported
 * (q_dtype, kv_dtype): (F32, F32), (BF16, BF16), (BF16, FP8_E4M3).
 * softmax_scale must be finite and > 0 (the usual 1 / sqrt(d_h)), and q,
 * k_cache, v_cache, out and workspace 16-byte aligned (INVALID_ARG
 * otherwise).
 * `workspace` holds partial results of requests whose positions are split
 * over several waves; its size comes from pkv_decode_plan with the same
 * arguments (WORKSPACE if too small; it may be NULL when the plan says 0).
 * Launches the partition kernel and, when partial results can arise, the
 * combine kernel.  Calls that share one workspace must not overlap. */
int pkv_paged_decode_attention(float* out, const void* q, int q_dtype, const void* k_cache,
                               const void* v_cache, int kv_dtype, const float* k_scale,
                               const float* v_scale, const int32_t* block_table,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t max_context_len, int32_t B, int32_t H_Q, int32_t H_KV,
                               int32_t d_h, int32_t block_size, int32_t num_blocks,
                               float softmax_scale, int32_t partition_tokens, void* workspace,
                               size_t workspace_bytes, pkv_stream_t stream);

/* One decode step: pkv_kv_append of k_new / v_new ([B][H_KV][d_h] in the
 * query dtype) followed by pkv_paged_decode_attention, same arguments and
 * results (the pools end up byte for byte as after pkv_kv_append; k_cache
 * and v_cache are written).  Where the MFMA kernels run on a bf16 cache
 * with H_Q / H_KV <= 16, or on an fp8 cache with H_Q / H_KV > 16 and the
 * balanced split, the append is done inside the attention launch by the
 * wave that reads the request's last block, which uses the new row from
 * registers (one launch fewer); other cases launch the append kernel
 * first. */
int pkv_decode_step(const void* k_new, const void* v_new, float* out, const void* q, int q_dtype,
                    void* k_cache, void* v_cache, int kv_dtype, const float* k_scale,
                    const float* v_scale, const int32_t* block_table, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t max_context_len, int32_t B, int32_t H_Q,
                    int32_t H_KV, int32_t d_h, int32_t block_size, int32_t num_blocks,
                    float softmax_scale, int32_t partition_tokens, void* workspace,
                    size_t workspace_bytes, pkv_stream_t stream);

/* pkv_decode_step without a caller workspace, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * hosts that forbid allocation).  Same arguments and results as
 * pkv_decode_step minus workspace / workspace_bytes: the partial results go
 * to a static device array of PKV_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends; the call itself
 * allocates nothing.  Shapes whose workspace (pkv_decode_plan) exceeds that
 * size are refused with PKV_ERR_WORKSPACE before anything is launched.
 * Every call on one GPU uses that GPU's one array: calls that overlap in
 * time on one GPU (other streams, other threads) race on it, and the caller
 * must order them.  Nothing in the array has to start at any value (each
 * step writes the partial results and the header it reads back).
 * PKV_ERR_HIP if the array's device address cannot be obtained. */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int pkv_decode_step_noalloc(const void* k_new, const void* v_new, float* out, const void* q,
                            int q_dtype, void* k_cache, void* v_cache, int kv_dtype,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t max_context_len, int32_t B,
                            int32_t H_Q, int32_t H_KV, int32_t d_h, int32_t block_size,
                            int32_t num_blocks, float softmax_scale, int32_t partition_tokens,
                            pkv_stream_t stream);

/* Cascade decode step over a shared prefix (page 3 "xf_kv_cache",
 * "End-to-end flow": many requests map the same prefix blocks; page 1
 * section 21.5 step 3).  Contract: the first shared_blocks entries of every
 * request's table row are the same physical blocks, every request's
 * context covers them (context_lens[b] > shared_blocks * block_size, so its
 * new token lies past the prefix), and shared blocks are not written.  The
 * result equals pkv_decode_step's up to the order of additions: the shared
 * blocks are read once per (KV head, 32 query heads of the batch) by a
 * prefix kernel that scores every request's queries against them, the
 * flat decode kernel covers each request's private blocks (appending the
 * new token, fused for bf16 with H_Q / H_KV <= 16, else by the append
 * kernel first; k_new = v_new = NULL skips the append), and the combine
 * merges both with the log-sum-exp rule.  Needs the MFMA kernels' shapes
 * (bf16 queries, bf16 or fp8 cache, d_h 128, 16-slot blocks) and the
 * balanced split; UNSUPPORTED otherwise (use pkv_decode_step).
 * pkv_cascade_plan gives the workspace size (and the prefix kernel's split
 * count); INVALID_ARG if shared_blocks < 1 or the prefix is longer than
 * max_context_len. */
int pkv_cascade_plan(int32_t B, int32_t H_Q, int32_t H_KV, int32_t d_h, int32_t block_size,
                     int32_t max_context_len, int32_t shared_blocks, int q_dtype, int kv_dtype,
                     int32_t* splits_out, size_t* workspace_bytes);
int pkv_decode_step_cascade(const void* k_new, const void* v_new, float* out, const void* q,
                            int q_dtype, void* k_cache, void* v_cache, int kv_dtype,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t max_context_len, int32_t B,
                            int32_t H_Q, int32_t H_KV, int32_t d_h, int32_t block_size,
                            int32_t num_blocks, float softmax_scale, int32_t shared_blocks,
                            void* workspace, size_t workspace_bytes, pkv_stream_t stream);

/* The attention launch of pkv_decode_step_cascade alone (no append, no
 * combine), for timing that kernel: the same arguments without k_new /
 * v_new; it leaves the prefix pieces and the private pieces in the
 * workspace and writes nothing to `out` that the combine would not
 * overwrite.  The results are complete only after the combine, which only
 * pkv_decode_step_cascade launches. */
int pkv_cascade_partitions(float* out, const void* q, int q_dtype, const void* k_cache,
                           const void* v_cache, int kv_dtype, const float* k_scale,
                           const float* v_scale, const int32_t* block_table,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t max_context_len, int32_t B, int32_t H_Q, int32_t H_KV,
                           int32_t d_h, int32_t block_size, int32_t num_blocks,
                           float softmax_scale, int32_t shared_blocks, void* workspace,
                           size_t workspace_bytes, pkv_stream_t stream);

/* The two launches of pkv_paged_decode_attention, callable separately (for
 * timing each kernel).  decode_partitions runs the online softmax over each
 * piece (same arguments); it writes `out` directly for requests whose
 * positions one wave covers and partial (max, sum, unnormalised output)
 * triples to the workspace otherwise, with a header saying which layout it
 * used.  combine_partitions merges those partials with the log-sum-exp
 * rule: M = max_p m_p, out = sum_p o_p e^(m_p - M) / sum_p l_p e^(m_p - M).
 * Call it right after decode_partitions, on the same stream, with the same
 * context_lens, max_context_len, B, H_Q, H_KV, d_h, block size, partition
 * and workspace; with a NULL workspace it does nothing. */
int pkv_decode_partitions(float* out, const void* q, int q_dtype, const void* k_cache,
                          const void* v_cache, int kv_dtype, const float* k_scale,
                          const float* v_scale, const int32_t* block_table,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t max_context_len, int32_t B, int32_t H_Q, int32_t H_KV,
                          int32_t d_h, int32_t block_size, int32_t num_blocks,
                          float softmax_scale, int32_t partition_tokens, void* workspace,
                          size_t workspace_bytes, pkv_stream_t stream);
int pkv_combine_partitions(float* out, const int32_t* context_lens, int32_t max_context_len,
                           int32_t B, int32_t H_Q, int32_t H_KV, int32_t d_h,
                           int32_t block_size, int32_t partition_tokens, const void* workspace,
                           size_t workspace_bytes, pkv_stream_t stream);

/* ------------------------------------------------------------------------
 * Chunks of new tokens (page 1 section 21.3: a prompt processed in chunks
 * keeps the earlier chunks' positions and cached state; section 21.1: a
 * query reads the keys of earlier positions and its own; page 3 "xf_kv_cache",
 * "End-to-end flow": the new tokens after a prefix hit attend to the shared
 * prefix through the same table).
 *
 * Request b brings n_b = query_start[b + 1] - query_start[b] new tokens
 * (query_start: device int32 [B + 1], non-decreasing, query_start[0] = 0,
 * query_start[B] = total).  context_lens[b] counts positions after the
 * chunk's append, so the chunk occupies positions context_lens[b] - n_b ..
 * context_lens[b] - 1 and needs n_b <= context_lens[b].  Rows of k_new,
 * v_new ([total][H_KV][d_h]), q and out ([total][H_Q][d_h]) follow request
 * order.  A decode step is the case n_b = 1 for every request.  Device-side
 * entries out of range (n_b > context length, rows past `total`) make the
 * request write nothing.
 * ---------------------------------------------------------------------- */

/* Write every request's chunk of new K and V rows into their slots (same
 * stored forms as pkv_kv_append): row query_start[b] + i goes to position
 * context_lens[b] - n_b + i.  total_tokens = query_start[B] (host value). */
int pkv_kv_append_chunk(const void* k_new, const void* v_new, int in_dtype, void* k_cache,
                        void* v_cache, int kv_dtype, const float* k_scale, const float* v_scale,
                        const int32_t* block_table, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, const int32_t* query_start, int32_t B,
                        int32_t total_tokens, int32_t H_KV, int32_t d_h, int32_t block_size,
                        int32_t num_blocks, pkv_stream_t stream);
/* Causal attention of every new token: query row query_start[b] + i, at
 * position p = context_lens[b] - n_b + i, query head hq, KV head hq / g:
 *   out[row][hq][:] = sum_{t <= p} exp(s_t - max s) V_t / sum_{t <= p} exp(s_t - max s),
 *   s_t = softmax_scale * q[row][hq] . K_t,
 * in fp32.  max_q_len (host) >= every n_b sizes the grid; max_context_len
 * (host) >= every context length.  Same dtype pairs, alignment and
 * softmax_scale rule as pkv_paged_decode_attention; B and H_Q at most 65535.  No workspace: the
 * outputs are written directly.  Call after pkv_kv_append_chunk. */
int pkv_paged_chunk_attention(float* out, const void* q, int q_dtype, const void* k_cache,
                              const void* v_cache, int kv_dtype, const float* k_scale,
                              const float* v_scale, const int32_t* block_table,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              const int32_t* query_start, int32_t B, int32_t total_q,
                              int32_t max_q_len, int32_t max_context_len, int32_t H_Q,
                              int32_t H_KV, int32_t d_h, int32_t block_size, int32_t num_blocks,
                              float softmax_scale, pkv_stream_t stream);

/* ------------------------------------------------------------------------
 * Swap to host memory and back (page 1 section 21.3: offloading moves
 * retained cache state to CPU memory and brings the needed blocks back;
 * page 3 "xf_kv_cache", "End-to-end flow": a preempted request's blocks go
 * to pinned host memory and are copied back when it resumes; page 2
 * "KV Cache Explained", section "What changes when KV moves off the GPU":
 * bytes / link rate is the floor of such a transfer).
 *
 * Record i of a record buffer holds one block: its K bytes ([H_KV][bs][d_h]
 * as stored, block_bytes of them), then its V bytes, then for FP8_E4M3 its
 * K scales and V scales ([H_KV] float each); records are record_bytes
 * apart (a multiple of 256), padding bytes untouched.  The buffer may be
 * pinned host memory (hipHostMalloc, torch pin_memory) or device memory;
 * pageable host memory is refused (INVALID_ARG).  The kernels read or write
 * it directly; the call is asynchronous on `stream`, so the caller
 * synchronises before reading a swapped-out buffer on the host, and may
 * release or reuse the blocks as soon as later work on the same stream is
 * what overwrites them.
 * ---------------------------------------------------------------------- */

/* Sizes of one block's K (or V) bytes and of one padded record. */
int pkv_swap_record_bytes(int kv_dtype, int32_t H_KV, int32_t d_h, int32_t block_size,
                          size_t* block_bytes, size_t* record_bytes);
/* Copy blocks[0..n) (device int32) into records 0..n-1 of `records`.  A
 * record whose block id is outside [0, num_blocks) is skipped. */
int pkv_swap_out(const void* k_cache, const void* v_cache, int kv_dtype, const float* k_scale,
                 const float* v_scale, const int32_t* blocks, int32_t n, int32_t H_KV,
                 int32_t d_h, int32_t block_size, int32_t num_blocks, void* records,
                 pkv_stream_t stream);
/* Copy records 0..n-1 back into blocks[0..n) (typically new ids from
 * pkv_pool_alloc_n); the request's table row then lists those ids in the
 * same logical order. */
int pkv_swap_in(void* k_cache, void* v_cache, int kv_dtype, float* k_scale, float* v_scale,
                const int32_t* blocks, int32_t n, int32_t H_KV, int32_t d_h, int32_t block_size,
                int32_t num_blocks, const void* records, pkv_stream_t stream);

/* Kernel selection for the attention calls (process-wide; any thread may
 * set or read it, and a call uses the value current when it plans; a plan
 * and the attention call it sizes must see the same value).  AUTO uses the MFMA kernel with the balanced per-wave split
 * where it applies and the generic VALU kernel otherwise; GENERIC, MFMA
 * (balanced split) and MFMA_PARTITION (fixed partitions) force one, and
 * return UNSUPPORTED from the plan and attention calls outside their
 * shapes.  Chunk attention uses its MFMA kernel unless GENERIC is set (or
 * the shape needs the generic one).  Returns the previous value. */
typedef enum {
  PKV_VARIANT_AUTO = 0,
  PKV_VARIANT_GENERIC = 1,
  PKV_VARIANT_MFMA = 2,
  PKV_VARIANT_MFMA_PARTITION = 3
} pkv_variant;
int pkv_set_decode_variant(int variant);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
