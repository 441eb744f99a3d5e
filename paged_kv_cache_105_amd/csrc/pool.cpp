// Host block pool: fixed set of physical blocks, FIFO free queue, reference
// counts, and retained prefix identities.
//
// Page 1 "KV cache: Generation state, latency, and allocation", section 21.5
// (Table 21.1 and the five steps after it): a request takes a new block only
// when a position opens a new logical block; sharing a complete block raises
// its reference count; releasing drops references and returns a block to the
// free pool when its count reaches zero.  Page 2 "KV Cache Explained",
// section "Why PagedAttention allocates KV in blocks": the pool is created up
// front with a free-block queue and a hash-to-block lookup, and a block that
// keeps its identity after its last reference is still free for eviction.
//
// The queue is an intrusive doubly linked list over block ids (prev/next
// arrays), so a prefix hit can take an idle cached block out of the middle
// in O(1).  The identity lookup is an open-addressing table with linear
// probing and backward-shift deletion, sized at creation to twice the block
// count; it holds at most one entry per block, so nothing allocates after
// pkv_pool_create.

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "pkv.h"
#include "sha256.h"

namespace {

constexpr int kDigest = PKV_DIGEST_BYTES;

inline uint64_t digest_key(const uint8_t* d) {
  uint64_t k;
  std::memcpy(&k, d, sizeof(k));  // SHA-256 output bits are uniform
  return k;
}

}  // namespace

struct pkv_pool {
  int32_t num_blocks;
  int32_t block_size;
  std::vector<int32_t> refcount;  // 0 = in the free queue
  // free queue: intrusive list, -1 terminated
  std::vector<int32_t> prev, next;
  int32_t head = -1, tail = -1, count = 0;
  // retained identities
  std::vector<uint8_t> digest;    // [num_blocks][32]
  std::vector<uint8_t> hashed;    // 1 if the block holds an identity
  std::vector<int32_t> table;     // open addressing: block id or -1
  uint64_t mask = 0;
  int32_t cached_idle = 0;        // free blocks that hold an identity
  int32_t n_hashed = 0;           // blocks that hold an identity
  int64_t queried = 0, hits = 0, evictions = 0;

  bool live(int32_t b) const { return b >= 0 && b < num_blocks && refcount[b] > 0; }

  void push_tail(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    ++count;
    if (hashed[b]) ++cached_idle;
  }
  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    --count;
    if (hashed[b]) --cached_idle;
  }
  // Take the queue head as a fresh block with one reference; an identity it
  // still holds is evicted.
  int32_t take_head() {
    const int32_t b = head;
    unlink(b);
    if (hashed[b]) {
      erase(b);
      ++evictions;
    }
    refcount[b] = 1;
    return b;
  }
  void release_one(int32_t b) {
    if (--refcount[b] == 0) push_tail(b);
  }

  const uint8_t* dig(int32_t b) const { return &digest[size_t(b) * kDigest]; }
  int32_t find(const uint8_t* d) const {
    for (uint64_t i = digest_key(d) & mask;; i = (i + 1) & mask) {
      const int32_t b = table[i];
      if (b < 0) return -1;
      if (std::memcmp(dig(b), d, kDigest) == 0) return b;
    }
  }
  void insert(int32_t b, const uint8_t* d) {
    std::memcpy(&digest[size_t(b) * kDigest], d, kDigest);
    hashed[b] = 1;
    ++n_hashed;
    uint64_t i = digest_key(d) & mask;
    while (table[i] >= 0) i = (i + 1) & mask;
    table[i] = b;
  }
  void erase(int32_t b) {
    uint64_t i = digest_key(dig(b)) & mask;
    while (table[i] != b) i = (i + 1) & mask;
    // backward shift: move later entries of the probe run into the hole
    // unless their home slot lies cyclically in (hole, their slot]
    for (uint64_t j = (i + 1) & mask; table[j] >= 0; j = (j + 1) & mask) {
      const uint64_t home = digest_key(dig(table[j])) & mask;
      const bool stays = (i <= j) ? (i < home && home <= j) : (i < home || home <= j);
      if (stays) continue;
      table[i] = table[j];
      i = j;
    }
    table[i] = -1;
    hashed[b] = 0;
    --n_hashed;
  }
};

extern "C" {

int pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                    pkv_pool** out) {
  if (!out || num_blocks <= 0 || block_size <= 0) return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  pkv_pool* p = new (std::nothrow) pkv_pool();
  if (!p) return PKV_ERR_INVALID_ARG;
  try {
    p->num_blocks = num_blocks;
    p->block_size = block_size;
    p->refcount.assign(num_blocks, 0);
    p->prev.assign(num_blocks, -1);
    p->next.assign(num_blocks, -1);
    p->digest.assign(size_t(num_blocks) * kDigest, 0);
    p->hashed.assign(num_blocks, 0);
    uint64_t cap = 16;
    while (cap < 2 * uint64_t(num_blocks)) cap <<= 1;
    p->table.assign(cap, -1);
    p->mask = cap - 1;
  } catch (const std::bad_alloc&) {
    delete p;
    return PKV_ERR_INVALID_ARG;
  }
  std::vector<char> seen(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b]) {
      delete p;
      return PKV_ERR_INVALID_ARG;
    }
    seen[b] = 1;
    p->push_tail(b);
  }
  *out = p;
  return PKV_OK;
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

int pkv_pool_alloc(pkv_pool* pool, int32_t* block_id) {
  if (!pool || !block_id) return PKV_ERR_INVALID_ARG;
  if (pool->count == 0) return PKV_ERR_OUT_OF_BLOCKS;
  *block_id = pool->take_head();
  return PKV_OK;
}

int pkv_pool_alloc_n(pkv_pool* pool, int32_t n, int32_t* ids) {
  if (!pool || n < 0 || (n > 0 && !ids)) return PKV_ERR_INVALID_ARG;
  if (n > pool->count) return PKV_ERR_OUT_OF_BLOCKS;
  for (int32_t i = 0; i < n; ++i) ids[i] = pool->take_head();
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
  pool->release_one(block_id);
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
  int32_t i = 0;
  for (int32_t b = pool->head; b >= 0; b = pool->next[b]) ids[i++] = b;
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
    table_row[j] = pool->take_head();
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
      const int32_t dst = pool->take_head();
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
  for (int32_t j = 0; j < n_blocks; ++j) pool->release_one(table_row[j]);
  return PKV_OK;
}

// ---- prefix identity ------------------------------------------------------

int pkv_prefix_root(const void* identity, size_t n, uint8_t* out) {
  if (!out || (n > 0 && !identity)) return PKV_ERR_INVALID_ARG;
  pkv::Sha256 s;
  s.update(identity, n);
  s.final(out);
  return PKV_OK;
}

int pkv_block_hashes(const uint8_t* parent, const int32_t* tokens, int64_t n_tokens,
                     int32_t block_size, uint8_t* out, int64_t cap_blocks, int64_t* n_out) {
  if (!parent || !n_out || n_tokens < 0 || block_size <= 0 || cap_blocks < 0 ||
      (n_tokens > 0 && !tokens))
    return PKV_ERR_INVALID_ARG;
  const int64_t nb = n_tokens / block_size;
  *n_out = nb;
  if (cap_blocks < nb || (nb > 0 && !out)) return PKV_ERR_INVALID_ARG;
  // the token ids go in as little-endian int32, whatever the host order
  std::vector<uint8_t> le(size_t(block_size) * 4);
  const uint8_t* h = parent;
  for (int64_t j = 0; j < nb; ++j) {
    const int32_t* t = tokens + j * block_size;
    for (int32_t i = 0; i < block_size; ++i) {
      const uint32_t v = uint32_t(t[i]);
      le[4 * i] = uint8_t(v);
      le[4 * i + 1] = uint8_t(v >> 8);
      le[4 * i + 2] = uint8_t(v >> 16);
      le[4 * i + 3] = uint8_t(v >> 24);
    }
    pkv::Sha256 s;
    s.update(h, kDigest);
    s.update(le.data(), le.size());
    s.final(out + j * kDigest);
    h = out + j * kDigest;
  }
  return PKV_OK;
}

int pkv_pool_lookup(const pkv_pool* pool, const uint8_t* digest, int32_t* block_id) {
  if (!pool || !digest || !block_id) return PKV_ERR_INVALID_ARG;
  *block_id = pool->find(digest);
  return PKV_OK;
}

int pkv_pool_match_prefix(pkv_pool* pool, const uint8_t* hashes, int32_t n_hashes,
                          int32_t* table_row, int32_t max_blocks, int32_t* n_hit) {
  if (!pool || !n_hit || n_hashes < 0 || max_blocks < 0 ||
      (n_hashes > 0 && (!hashes || (max_blocks > 0 && !table_row))))
    return PKV_ERR_INVALID_ARG;
  const int32_t lim = std::min(n_hashes, max_blocks);
  int32_t n = 0;
  for (; n < lim; ++n) {
    const int32_t b = pool->find(hashes + size_t(n) * kDigest);
    if (b < 0) break;
    if (pool->refcount[b] == 0) pool->unlink(b);  // an idle cached block comes back
    ++pool->refcount[b];
    table_row[n] = b;
  }
  pool->queried += n_hashes;
  pool->hits += n;
  *n_hit = n;
  return PKV_OK;
}

int pkv_pool_cache_blocks(pkv_pool* pool, const int32_t* table_row, int32_t n_blocks,
                          int32_t ctx_len, const uint8_t* hashes, int32_t n_hashes,
                          int32_t* n_cached) {
  if (!pool || !n_cached || n_blocks < 0 || ctx_len < 0 || n_hashes < 0)
    return PKV_ERR_INVALID_ARG;
  const int32_t n = std::min({n_hashes, ctx_len / pool->block_size, n_blocks});
  if (n > 0 && (!table_row || !hashes)) return PKV_ERR_INVALID_ARG;
  // checks before any change: every block live, no identity replaced
  for (int32_t j = 0; j < n; ++j) {
    const int32_t b = table_row[j];
    if (!pool->live(b)) return PKV_ERR_BAD_BLOCK;
    if (pool->hashed[b] && std::memcmp(pool->dig(b), hashes + size_t(j) * kDigest, kDigest))
      return PKV_ERR_INVALID_ARG;
  }
  int32_t added = 0;
  for (int32_t j = 0; j < n; ++j) {
    const int32_t b = table_row[j];
    const uint8_t* d = hashes + size_t(j) * kDigest;
    if (pool->hashed[b] || pool->find(d) >= 0) continue;  // kept, or held by another block
    pool->insert(b, d);
    ++added;
  }
  *n_cached = added;
  return PKV_OK;
}

int pkv_pool_prefix_stats(const pkv_pool* pool, int64_t* stats) {
  if (!pool || !stats) return PKV_ERR_INVALID_ARG;
  stats[0] = pool->queried;
  stats[1] = pool->hits;
  stats[2] = pool->evictions;
  stats[3] = pool->cached_idle;
  stats[4] = pool->n_hashed;
  return PKV_OK;
}

}  // extern "C"
