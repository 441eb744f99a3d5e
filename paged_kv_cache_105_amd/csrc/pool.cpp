// Host block pool: fixed set of physical blocks, FIFO free queue, reference
// counts, immediate release.
//
// Page 1 "KV cache: Generation state, latency, and allocation", section 21.5
// (Table 21.1 and the five steps after it): a request takes a new block only
// when a position opens a new logical block; sharing a complete block raises
// its reference count; releasing drops references and returns a block to the
// free pool when its count reaches zero.  Page 2 "KV Cache Explained",
// section "Why PagedAttention allocates KV in blocks": the pool is created up
// front with a free-block queue.  The queue is a ring buffer of block ids, so
// every operation is O(1) and allocation-free after creation.

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <new>
#include <vector>

#include "pkv.h"

struct pkv_pool {
  int32_t num_blocks;
  int32_t block_size;
  std::vector<int32_t> refcount;  // 0 = free
  std::vector<int32_t> ring;      // free queue storage, capacity num_blocks
  int32_t head = 0;               // index of the queue head in ring
  int32_t count = 0;              // number of free blocks

  int32_t pop() {
    int32_t b = ring[head];
    head = (head + 1) % num_blocks;
    --count;
    return b;
  }
  void push(int32_t b) {
    ring[(head + count) % num_blocks] = b;
    ++count;
  }
  bool live(int32_t b) const { return b >= 0 && b < num_blocks && refcount[b] > 0; }
};

extern "C" {

int pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                    pkv_pool** out) {
  if (!out || num_blocks <= 0 || block_size <= 0) return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  pkv_pool* p = new (std::nothrow) pkv_pool();
  if (!p) return PKV_ERR_INVALID_ARG;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->refcount.assign(num_blocks, 0);
  p->ring.resize(num_blocks);
  std::vector<char> seen(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b]) {
      delete p;
      return PKV_ERR_INVALID_ARG;
    }
    seen[b] = 1;
    p->ring[i] = b;
  }
  p->count = num_blocks;
  *out = p;
  return PKV_OK;
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

int pkv_pool_alloc(pkv_pool* pool, int32_t* block_id) {
  if (!pool || !block_id) return PKV_ERR_INVALID_ARG;
  if (pool->count == 0) return PKV_ERR_OUT_OF_BLOCKS;
  int32_t b = pool->pop();
  pool->refcount[b] = 1;
  *block_id = b;
  return PKV_OK;
}

int pkv_pool_incref(pkv_pool* pool, int32_t block_id) {
  if (!pool) return PKV_ERR_INVALID_ARG;
  if (!pool->live(block_id)) return PKV_ERR_BAD_BLOCK;
  ++pool->refcount[block_id];
  return PKV_OK;
}

int pkv_pool_decref(pkv_pool* pool, int32_t block_id) {
  if (!pool) return PKV_ERR_INVALID_ARG;
  if (!pool->live(block_id)) return PKV_ERR_BAD_BLOCK;
  if (--pool->refcount[block_id] == 0) pool->push(block_id);
  return PKV_OK;
}

int pkv_pool_refcount(const pkv_pool* pool, int32_t block_id, int32_t* out) {
  if (!pool || !out) return PKV_ERR_INVALID_ARG;
  if (block_id < 0 || block_id >= pool->num_blocks) return PKV_ERR_BAD_BLOCK;
  *out = pool->refcount[block_id];
  return PKV_OK;
}

int pkv_pool_num_free(const pkv_pool* pool, int32_t* out) {
  if (!pool || !out) return PKV_ERR_INVALID_ARG;
  *out = pool->count;
  return PKV_OK;
}

int pkv_pool_num_used(const pkv_pool* pool, int32_t* out) {
  if (!pool || !out) return PKV_ERR_INVALID_ARG;
  *out = pool->num_blocks - pool->count;
  return PKV_OK;
}

int pkv_pool_free_queue(const pkv_pool* pool, int32_t* ids, int32_t cap, int32_t* count) {
  if (!pool || !count) return PKV_ERR_INVALID_ARG;
  *count = pool->count;
  if (cap < pool->count || (!ids && pool->count > 0)) return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < pool->count; ++i)
    ids[i] = pool->ring[(pool->head + i) % pool->num_blocks];
  return PKV_OK;
}

int pkv_seq_prepare_append(pkv_pool* pool, int32_t* table_row, int32_t max_blocks,
                           int32_t ctx_before, int32_t* n_blocks, int32_t* block_out,
                           int32_t* slot_out) {
  if (!pool || !table_row || !n_blocks || !block_out || !slot_out || ctx_before < 0 ||
      max_blocks <= 0)
    return PKV_ERR_INVALID_ARG;
  const int32_t bs = pool->block_size;
  const int32_t j = ctx_before / bs;
  const int32_t r = ctx_before % bs;
  if (r == 0) {
    // the position opens logical block j: the row must hold exactly j blocks
    if (*n_blocks != j || j >= max_blocks) return PKV_ERR_INVALID_ARG;
    if (pool->count == 0) return PKV_ERR_OUT_OF_BLOCKS;
    int32_t b = pool->pop();
    pool->refcount[b] = 1;
    table_row[j] = b;
    *n_blocks = j + 1;
  } else {
    if (*n_blocks != j + 1) return PKV_ERR_INVALID_ARG;
    int32_t b = table_row[j];
    if (!pool->live(b)) return PKV_ERR_BAD_BLOCK;
    if (pool->refcount[b] > 1) return PKV_ERR_SHARED_BLOCK;
  }
  *block_out = table_row[j];
  *slot_out = r;
  return PKV_OK;
}

int pkv_seq_prepare_append_cow(pkv_pool* pool, int32_t* table_row, int32_t max_blocks,
                               int32_t ctx_before, int32_t* n_blocks, int32_t* block_out,
                               int32_t* slot_out, int32_t* cow_src) {
  if (!cow_src) return PKV_ERR_INVALID_ARG;
  *cow_src = -1;
  if (pool && table_row && n_blocks && block_out && slot_out && ctx_before >= 0 &&
      max_blocks > 0) {
    const int32_t bs = pool->block_size;
    const int32_t j = ctx_before / bs;
    if (ctx_before % bs != 0 && *n_blocks == j + 1 && pool->live(table_row[j]) &&
        pool->refcount[table_row[j]] > 1) {
      // a writer into a shared, partly filled block gets a private copy: take
      // the new block first so that an empty pool changes nothing
      if (pool->count == 0) return PKV_ERR_OUT_OF_BLOCKS;
      const int32_t src = table_row[j];
      const int32_t dst = pool->pop();
      pool->refcount[dst] = 1;
      --pool->refcount[src];  // stays >= 1: other rows still hold it
      table_row[j] = dst;
      *cow_src = src;
      *block_out = dst;
      *slot_out = ctx_before % bs;
      return PKV_OK;
    }
  }
  return pkv_seq_prepare_append(pool, table_row, max_blocks, ctx_before, n_blocks, block_out,
                                slot_out);
}

int pkv_seq_share_prefix(pkv_pool* pool, const int32_t* src_row, int32_t n_full_blocks,
                         int32_t* dst_row) {
  if (!pool || n_full_blocks < 0 || (n_full_blocks > 0 && (!src_row || !dst_row)))
    return PKV_ERR_INVALID_ARG;
  for (int32_t j = 0; j < n_full_blocks; ++j)
    if (!pool->live(src_row[j])) return PKV_ERR_BAD_BLOCK;
  for (int32_t j = 0; j < n_full_blocks; ++j) {
    ++pool->refcount[src_row[j]];
    dst_row[j] = src_row[j];
  }
  return PKV_OK;
}

int pkv_seq_release(pkv_pool* pool, const int32_t* table_row, int32_t n_blocks) {
  if (!pool || n_blocks < 0 || (n_blocks > 0 && !table_row)) return PKV_ERR_INVALID_ARG;
  // validate first: every id live, and no id named more often than it is
  // referenced (counted on a sorted copy)
  std::vector<int32_t> ids(table_row, table_row + n_blocks);
  std::sort(ids.begin(), ids.end());
  for (int32_t j = 0; j < n_blocks;) {
    int32_t b = ids[j], k = j;
    while (k < n_blocks && ids[k] == b) ++k;
    if (!pool->live(b) || k - j > pool->refcount[b]) return PKV_ERR_BAD_BLOCK;
    j = k;
  }
  for (int32_t j = 0; j < n_blocks; ++j) {
    int32_t b = table_row[j];
    if (--pool->refcount[b] == 0) pool->push(b);
  }
  return PKV_OK;
}

}  // extern "C"
