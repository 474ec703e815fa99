// Host block pool: physical block ids, reference counts and a FIFO free queue.
//
// Follows "vLLM推理引擎深度解析" section 2.2 (a pool of physical blocks, a table
// per request, a queue of free blocks ordered by LRU, a new block every 16
// generated tokens) and "大语言模型推理引擎深度剖析" sections 2.2-2.3 (O(1)
// allocation and release; tables may share blocks; counts are kept and a
// block goes back to the free pool at zero; a shared block is copied before
// it is written).
//
// The free queue is an intrusive doubly linked list over the block ids:
// alloc (pop head), release (push tail) and taking a cached block back out of
// the queue are all O(1).  Every operation that can fail checks first and
// mutates only when it is sure to succeed.
//
// Prefix caching ("vLLM推理引擎深度解析" section 4.1; "KV Cache 与
// PageAttention深度实战" section 4.2): a full block whose K/V are computed can
// be registered under the exact key (parent block, the parent's allocation
// generation, its token ids).  A freed block keeps its key at the tail of the
// free queue until allocation reaches it at the head (least recently freed
// first) and evicts it; each hand-out advances the block's generation, so a
// chain whose parent was reused never matches.  The index is a multimap from
// a 64-bit FNV-1a hash of the key to blocks; every candidate is compared
// against the full stored key, so a hash collision cannot produce a hit.
#include <cstdint>
#include <climits>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

struct pkv_pool {
  int32_t num_blocks;
  int32_t block_size;
  std::vector<int32_t> ref;    // 0 = free
  std::vector<int32_t> prev;   // free queue links (-1 = none)
  std::vector<int32_t> next;
  std::vector<uint8_t> queued;  // 1 while the block is in the free queue
  int32_t head = -1, tail = -1;
  int32_t count = 0;            // queue length
  // batch bookkeeping: per-block writer counts (all zero between calls) and
  // the ids with a nonzero count
  std::vector<int32_t> touch;
  std::vector<int32_t> touched;
  // prefix cache
  std::vector<uint32_t> gen;          // times each block was handed out
  std::vector<uint8_t> keyed;         // 1 = registered under key_*
  std::vector<int32_t> key_parent;
  std::vector<uint32_t> key_gen;
  std::vector<uint64_t> key_hash;
  std::vector<int32_t> key_tokens;    // [num_blocks][block_size], allocated on first use
  std::unordered_multimap<uint64_t, int32_t> index;

  void unlink(int32_t b) {
    const int32_t p = prev[b], n = next[b];
    if (p >= 0) next[p] = n; else head = n;
    if (n >= 0) prev[n] = p; else tail = p;
    prev[b] = next[b] = -1;
    queued[b] = 0;
    --count;
  }
  void push(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    queued[b] = 1;
    ++count;
  }
  void evict(int32_t b) {
    if (!keyed[b]) return;
    auto range = index.equal_range(key_hash[b]);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == b) {
        index.erase(it);
        break;
      }
    keyed[b] = 0;
  }
  int32_t pop() {
    const int32_t b = head;
    unlink(b);
    evict(b);
    ++gen[b];
    ref[b] = 1;
    return b;
  }
  bool valid(int32_t b) const { return b >= 0 && b < num_blocks; }
};

namespace {

// FNV-1a, 64-bit (Fowler, Noll, Vo): xor each byte in, multiply by the prime.
uint64_t fnv1a(uint64_t h, const void* data, size_t n) {
  const uint8_t* p = static_cast<const uint8_t*>(data);
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 1099511628211ull;
  }
  return h;
}

uint64_t key_hash(int32_t parent, uint32_t pgen, const int32_t* tokens, int32_t bs) {
  uint64_t h = 14695981039346656037ull;
  h = fnv1a(h, &parent, sizeof parent);
  h = fnv1a(h, &pgen, sizeof pgen);
  return fnv1a(h, tokens, sizeof(int32_t) * (size_t)bs);
}

// The block registered under (parent, pgen, tokens), or -1.
int32_t find_cached(const pkv_pool* p, int32_t parent, uint32_t pgen, const int32_t* tokens,
                    uint64_t h) {
  if (p->key_tokens.empty()) return -1;
  const int32_t bs = p->block_size;
  auto range = p->index.equal_range(h);
  for (auto it = range.first; it != range.second; ++it) {
    const int32_t b = it->second;
    if (p->key_parent[b] == parent && p->key_gen[b] == pgen &&
        std::memcmp(&p->key_tokens[(size_t)b * bs], tokens, sizeof(int32_t) * (size_t)bs) == 0)
      return b;
  }
  return -1;
}

// Validation half of an append of n_new positions at cur_len to the table
// table[0..nb): no gap after the table, room in the table, every block it
// writes into is in use.  Adds the blocks past the table to *need_new and
// calls on_shared(b) for each existing block b with a count above one that
// the append writes into.  Changes nothing.
template <class F>
pkv_status check_append(const pkv_pool* pool, const int32_t* table, int32_t nb, int32_t cap,
                        int32_t cur_len, int32_t n_new, int64_t* need_new, F&& on_shared,
                        const char* who) {
  const int32_t bs = pool->block_size;
  const int64_t first = cur_len / bs, last = ((int64_t)cur_len + n_new - 1) / bs;
  if (first > nb) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: gap after the table", who);
  if (last + 1 > cap) return pkv::fail(PKV_ERR_INVALID_ARG, "%s: table capacity", who);
  for (int64_t bi = first; bi <= last; ++bi) {
    if (bi >= nb) {
      ++*need_new;
    } else {
      const int32_t b = table[bi];
      if (!pool->valid(b) || pool->ref[b] < 1)
        return pkv::fail(PKV_ERR_INVALID_ARG, "%s: table holds a bad block", who);
      if (pool->ref[b] > 1) on_shared(b);
    }
  }
  return PKV_OK;
}

// Mutation half, run only once the free queue is known to hold enough blocks:
// copy-on-write for shared blocks written into, new blocks past the table,
// then the slot of each new position.
void apply_append(pkv_pool* pool, int32_t* table, int32_t* nblocks, int32_t cur_len,
                  int32_t n_new, int64_t* slots_out, int32_t* cow_pairs, int32_t* ncow) {
  const int32_t bs = pool->block_size;
  const int64_t first = cur_len / bs, last = ((int64_t)cur_len + n_new - 1) / bs;
  const int32_t nb = *nblocks;
  for (int64_t bi = first; bi <= last; ++bi) {
    if (bi < nb) {
      const int32_t old = table[bi];
      if (pool->ref[old] > 1) {
        const int32_t fresh = pool->pop();
        cow_pairs[2 * *ncow] = old;
        cow_pairs[2 * *ncow + 1] = fresh;
        ++*ncow;
        --pool->ref[old];  // stays >= 1: it was above 1
        table[bi] = fresh;
      }
    } else {
      table[bi] = pool->pop();
    }
  }
  if (last + 1 > nb) *nblocks = (int32_t)(last + 1);
  for (int32_t i = 0; i < n_new; ++i) {
    const int64_t pos = (int64_t)cur_len + i;
    slots_out[i] = (int64_t)table[pos / bs] * bs + pos % bs;
  }
}

}  // namespace

extern "C" {

pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                           pkv_pool** out) {
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "pool_create: out is NULL");
  *out = nullptr;
  if (num_blocks < 0 || block_size <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "pool_create: bad num_blocks/block_size");
  pkv_pool* p = new (std::nothrow) pkv_pool();
  if (!p) return pkv::fail(PKV_ERR_INVALID_ARG, "pool_create: out of host memory");
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->ref.assign(num_blocks, 0);
  p->touch.assign(num_blocks, 0);
  p->prev.assign(num_blocks, -1);
  p->next.assign(num_blocks, -1);
  p->queued.assign(num_blocks, 0);
  p->gen.assign(num_blocks, 0);
  p->keyed.assign(num_blocks, 0);
  p->key_parent.assign(num_blocks, -1);
  p->key_gen.assign(num_blocks, 0);
  p->key_hash.assign(num_blocks, 0);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete p;
        return pkv::fail(PKV_ERR_INVALID_ARG, "pool_create: free_order is not a permutation");
      }
      seen[b] = 1;
    }
    for (int32_t i = 0; i < num_blocks; ++i) p->push(free_order[i]);
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) p->push(i);
  }
  *out = p;
  return PKV_OK;
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

pkv_status pkv_pool_alloc(pkv_pool* pool, int32_t* block_out) {
  if (!pool || !block_out) return pkv::fail(PKV_ERR_INVALID_ARG, "pool_alloc: NULL argument");
  if (pool->count == 0) return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "pool_alloc: no free block");
  *block_out = pool->pop();
  return PKV_OK;
}

pkv_status pkv_pool_incref(pkv_pool* pool, int32_t block) {
  if (!pool || !pool->valid(block))
    return pkv::fail(PKV_ERR_INVALID_ARG, "pool_incref: bad block id");
  if (pool->ref[block] < 1) return pkv::fail(PKV_ERR_REFCOUNT, "pool_incref: block is free");
  ++pool->ref[block];
  return PKV_OK;
}

pkv_status pkv_pool_decref(pkv_pool* pool, int32_t block) {
  if (!pool || !pool->valid(block))
    return pkv::fail(PKV_ERR_INVALID_ARG, "pool_decref: bad block id");
  if (pool->ref[block] < 1) return pkv::fail(PKV_ERR_REFCOUNT, "pool_decref: block is free");
  if (--pool->ref[block] == 0) pool->push(block);
  return PKV_OK;
}

int32_t pkv_pool_refcount(const pkv_pool* pool, int32_t block) {
  if (!pool || !pool->valid(block)) return -1;
  return pool->ref[block];
}

int32_t pkv_pool_num_free(const pkv_pool* pool) { return pool ? pool->count : -1; }
int32_t pkv_pool_num_blocks(const pkv_pool* pool) { return pool ? pool->num_blocks : -1; }
int32_t pkv_pool_block_size(const pkv_pool* pool) { return pool ? pool->block_size : -1; }

pkv_status pkv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* n) {
  if (!pool || !n) return pkv::fail(PKV_ERR_INVALID_ARG, "pool_free_list: NULL argument");
  *n = pool->count;
  if (cap < pool->count || (pool->count > 0 && !out))
    return pkv::fail(PKV_ERR_INVALID_ARG, "pool_free_list: cap too small");
  int32_t i = 0;
  for (int32_t b = pool->head; b >= 0; b = pool->next[b]) out[i++] = b;
  return PKV_OK;
}

pkv_status pkv_seq_append_slots(pkv_pool* pool, int32_t* table, int32_t* nblocks, int32_t cap,
                                int32_t cur_len, int32_t n_new, int64_t* slots_out,
                                int32_t* cow_pairs, int32_t cow_cap, int32_t* n_cow) {
  if (!pool || !nblocks) return pkv::fail(PKV_ERR_INVALID_ARG, "seq_append_slots: NULL argument");
  if (n_cow) *n_cow = 0;
  if (cur_len < 0 || n_new < 0 || *nblocks < 0 || cap < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "seq_append_slots: negative length");
  if (n_new == 0) return PKV_OK;
  if (!table || !slots_out)
    return pkv::fail(PKV_ERR_INVALID_ARG, "seq_append_slots: NULL table/slots");
  int64_t need_new = 0, need_cow = 0;
  pkv_status st = check_append(pool, table, *nblocks, cap, cur_len, n_new, &need_new,
                               [&](int32_t) { ++need_cow; }, "seq_append_slots");
  if (st != PKV_OK) return st;
  if (need_cow > 0 && (!cow_pairs || need_cow > cow_cap))
    return pkv::fail(PKV_ERR_INVALID_ARG, "seq_append_slots: cow_pairs too small");
  if (need_new + need_cow > pool->count)
    return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "seq_append_slots: not enough free blocks");
  int32_t ncow = 0;
  apply_append(pool, table, nblocks, cur_len, n_new, slots_out, cow_pairs, &ncow);
  if (n_cow) *n_cow = ncow;
  return PKV_OK;
}

pkv_status pkv_batch_append_slots(pkv_pool* pool, int32_t* block_tables,
                                  int32_t max_blocks_per_seq, int32_t* nblocks,
                                  int32_t* context_lens, const int32_t* n_new, int32_t num_seqs,
                                  int64_t* slot_mapping, int32_t* cow_pairs, int32_t cow_cap,
                                  int32_t* n_cow, int32_t* n_slots) {
  if (n_cow) *n_cow = 0;
  if (n_slots) *n_slots = 0;
  if (!pool || num_seqs < 0 || max_blocks_per_seq < 0 || cow_cap < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "batch_append_slots: bad argument");
  if (num_seqs == 0) return PKV_OK;
  if (!block_tables || !nblocks || !context_lens)
    return pkv::fail(PKV_ERR_INVALID_ARG, "batch_append_slots: NULL table/nblocks/lens");
  const int64_t mb = max_blocks_per_seq;
  // Pass 1: validate every sequence and count the blocks the batch takes.  A
  // shared block (count r > 1) that t sequences of the batch write into is
  // copied by the first min(t, r - 1) of them in batch order; the last writer
  // of a block that every holder writes keeps it.  No block is released in a
  // batch, so new blocks + copies is exactly what the free queue must hold.
  std::vector<int32_t>& touch = pool->touch;
  std::vector<int32_t>& touched = pool->touched;
  touched.clear();
  int64_t need_new = 0, total = 0;
  pkv_status st = PKV_OK;
  for (int32_t s = 0; s < num_seqs && st == PKV_OK; ++s) {
    const int32_t k = n_new ? n_new[s] : 1;
    if (context_lens[s] < 0 || k < 0 || nblocks[s] < 0 || nblocks[s] > max_blocks_per_seq) {
      st = pkv::fail(PKV_ERR_INVALID_ARG, "batch_append_slots: bad length or block count");
      break;
    }
    total += k;
    if (k == 0) continue;
    st = check_append(pool, block_tables + s * mb, nblocks[s], max_blocks_per_seq,
                      context_lens[s], k, &need_new,
                      [&](int32_t b) {
                        if (touch[b]++ == 0) touched.push_back(b);
                      },
                      "batch_append_slots");
  }
  int64_t need_cow = 0;
  for (int32_t b : touched) {
    const int64_t r = pool->ref[b];
    need_cow += touch[b] < r - 1 ? touch[b] : r - 1;
    touch[b] = 0;
  }
  touched.clear();
  if (st != PKV_OK) return st;
  if (total > 0 && !slot_mapping)
    return pkv::fail(PKV_ERR_INVALID_ARG, "batch_append_slots: slot_mapping is NULL");
  if (total > INT32_MAX)
    return pkv::fail(PKV_ERR_INVALID_ARG, "batch_append_slots: too many new positions");
  if (need_cow > 0 && (!cow_pairs || need_cow > cow_cap))
    return pkv::fail(PKV_ERR_INVALID_ARG, "batch_append_slots: cow_pairs too small");
  if (need_new + need_cow > pool->count)
    return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "batch_append_slots: not enough free blocks");
  // Pass 2: cannot fail.
  int32_t ncow = 0;
  int64_t t = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t k = n_new ? n_new[s] : 1;
    if (k == 0) continue;
    apply_append(pool, block_tables + s * mb, nblocks + s, context_lens[s], k, slot_mapping + t,
                 cow_pairs, &ncow);
    context_lens[s] += k;
    t += k;
  }
  if (n_cow) *n_cow = ncow;
  if (n_slots) *n_slots = (int32_t)t;
  return PKV_OK;
}

pkv_status pkv_seq_create(pkv_pool* pool, int32_t prompt_len, int32_t* table, int32_t cap,
                          int32_t* nblocks) {
  if (!pool || !nblocks) return pkv::fail(PKV_ERR_INVALID_ARG, "seq_create: NULL argument");
  if (prompt_len < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "seq_create: negative length");
  *nblocks = 0;
  if (prompt_len == 0) return PKV_OK;
  std::vector<int64_t> slots(prompt_len);
  int32_t nb = 0;
  pkv_status st = pkv_seq_append_slots(pool, table, &nb, cap, 0, prompt_len, slots.data(),
                                       nullptr, 0, nullptr);
  if (st == PKV_OK) *nblocks = nb;
  return st;
}

pkv_status pkv_seq_fork(pkv_pool* pool, const int32_t* table, int32_t nblocks) {
  if (!pool || nblocks < 0 || (nblocks > 0 && !table))
    return pkv::fail(PKV_ERR_INVALID_ARG, "seq_fork: bad argument");
  for (int32_t i = 0; i < nblocks; ++i) {
    if (!pool->valid(table[i])) return pkv::fail(PKV_ERR_INVALID_ARG, "seq_fork: bad block id");
    if (pool->ref[table[i]] < 1) return pkv::fail(PKV_ERR_REFCOUNT, "seq_fork: block is free");
  }
  for (int32_t i = 0; i < nblocks; ++i) ++pool->ref[table[i]];
  return PKV_OK;
}

pkv_status pkv_seq_create_cached(pkv_pool* pool, const int32_t* tokens, int32_t prompt_len,
                                int32_t* table, int32_t cap, int32_t* nblocks,
                                int32_t* cached_tokens) {
  if (!pool || !nblocks || !cached_tokens || prompt_len < 0 || cap < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "seq_create_cached: bad argument");
  *nblocks = 0;
  *cached_tokens = 0;
  if (prompt_len == 0) return PKV_OK;
  if (!tokens || !table) return pkv::fail(PKV_ERR_INVALID_ARG, "seq_create_cached: NULL");
  const int32_t bs = pool->block_size;
  const int32_t need = (int32_t)(((int64_t)prompt_len + bs - 1) / bs);
  if (need > cap) return pkv::fail(PKV_ERR_INVALID_ARG, "seq_create_cached: table capacity");
  // walk the cache along the prompt's full blocks; stop at the first miss
  std::vector<int32_t> hits;
  int32_t parent = -1;
  uint32_t pgen = 0;
  for (int32_t i = 0; i < prompt_len / bs; ++i) {
    const int32_t* tk = tokens + (int64_t)i * bs;
    const int32_t b = find_cached(pool, parent, pgen, tk, key_hash(parent, pgen, tk, bs));
    if (b < 0) break;
    hits.push_back(b);
    parent = b;
    pgen = pool->gen[b];
  }
  int64_t revived = 0;
  for (int32_t b : hits) revived += pool->ref[b] == 0;
  if ((int64_t)need - (int64_t)hits.size() > (int64_t)pool->count - revived)
    return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "seq_create_cached: not enough free blocks");
  int32_t i = 0;
  for (int32_t b : hits) {
    if (pool->ref[b] == 0) pool->unlink(b);
    ++pool->ref[b];
    table[i++] = b;
  }
  for (; i < need; ++i) table[i] = pool->pop();
  *nblocks = need;
  *cached_tokens = (int32_t)hits.size() * bs;
  return PKV_OK;
}

pkv_status pkv_pool_register_blocks(pkv_pool* pool, const int32_t* tokens, int32_t num_tokens,
                                    const int32_t* table, int32_t nblocks) {
  if (!pool || num_tokens < 0 || nblocks < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "register_blocks: bad argument");
  const int32_t bs = pool->block_size;
  const int32_t n_full = num_tokens / bs;
  if (n_full == 0) return PKV_OK;
  if (!tokens || !table || n_full > nblocks)
    return pkv::fail(PKV_ERR_INVALID_ARG, "register_blocks: table or tokens too short");
  for (int32_t i = 0; i < n_full; ++i) {
    if (!pool->valid(table[i])) return pkv::fail(PKV_ERR_INVALID_ARG, "register_blocks: bad id");
    if (pool->ref[table[i]] < 1)
      return pkv::fail(PKV_ERR_REFCOUNT, "register_blocks: block is free");
  }
  // pass 1: every block either unregistered or already under this very key
  std::vector<uint64_t> hs(n_full);
  int32_t parent = -1;
  uint32_t pgen = 0;
  for (int32_t i = 0; i < n_full; ++i) {
    const int32_t b = table[i];
    const int32_t* tk = tokens + (int64_t)i * bs;
    hs[i] = key_hash(parent, pgen, tk, bs);
    if (pool->keyed[b] &&
        (pool->key_parent[b] != parent || pool->key_gen[b] != pgen ||
         std::memcmp(&pool->key_tokens[(size_t)b * bs], tk, sizeof(int32_t) * (size_t)bs) != 0))
      return pkv::fail(PKV_ERR_INVALID_ARG, "register_blocks: block %d holds another prefix", b);
    parent = b;
    pgen = pool->gen[b];
  }
  if (pool->key_tokens.empty()) pool->key_tokens.assign((size_t)pool->num_blocks * bs, 0);
  // pass 2: register the new ones whose key no other block holds
  parent = -1;
  pgen = 0;
  for (int32_t i = 0; i < n_full; ++i) {
    const int32_t b = table[i];
    const int32_t* tk = tokens + (int64_t)i * bs;
    if (!pool->keyed[b] && find_cached(pool, parent, pgen, tk, hs[i]) < 0) {
      pool->keyed[b] = 1;
      pool->key_parent[b] = parent;
      pool->key_gen[b] = pgen;
      pool->key_hash[b] = hs[i];
      std::memcpy(&pool->key_tokens[(size_t)b * bs], tk, sizeof(int32_t) * (size_t)bs);
      pool->index.emplace(hs[i], b);
    }
    parent = b;
    pgen = pool->gen[b];
  }
  return PKV_OK;
}

int32_t pkv_pool_cached_blocks(const pkv_pool* pool) {
  return pool ? (int32_t)pool->index.size() : -1;
}

pkv_status pkv_seq_swap(pkv_pool* from, pkv_pool* to, const int32_t* table, int32_t nblocks,
                        int32_t* table_out, int32_t* pairs_out) {
  if (!from || !to || nblocks < 0 || (nblocks > 0 && (!table || !table_out || !pairs_out)))
    return pkv::fail(PKV_ERR_INVALID_ARG, "seq_swap: bad argument");
  if (from->block_size != to->block_size)
    return pkv::fail(PKV_ERR_INVALID_ARG, "seq_swap: block sizes differ");
  for (int32_t i = 0; i < nblocks; ++i) {
    const int32_t b = table[i];
    if (!from->valid(b)) return pkv::fail(PKV_ERR_INVALID_ARG, "seq_swap: bad block id");
    if (from->ref[b] < 1) return pkv::fail(PKV_ERR_REFCOUNT, "seq_swap: block is free");
  }
  if (to->count < nblocks)
    return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "seq_swap: target pool has too few free blocks");
  // take every target block first (so a swap within one pool never hands out
  // a block of the table), then release the table as pkv_seq_free does
  for (int32_t i = 0; i < nblocks; ++i) {
    table_out[i] = to->pop();
    pairs_out[2 * i] = table[i];
    pairs_out[2 * i + 1] = table_out[i];
  }
  for (int32_t i = nblocks - 1; i >= 0; --i) {
    const int32_t b = table[i];
    if (--from->ref[b] == 0) from->push(b);
  }
  return PKV_OK;
}

pkv_status pkv_seq_free(pkv_pool* pool, const int32_t* table, int32_t nblocks) {
  if (!pool || nblocks < 0 || (nblocks > 0 && !table))
    return pkv::fail(PKV_ERR_INVALID_ARG, "seq_free: bad argument");
  // check first so that a bad table changes nothing (a table never names
  // one block twice)
  for (int32_t i = 0; i < nblocks; ++i) {
    int32_t b = table[i];
    if (!pool->valid(b)) return pkv::fail(PKV_ERR_INVALID_ARG, "seq_free: bad block id");
    if (pool->ref[b] < 1) return pkv::fail(PKV_ERR_REFCOUNT, "seq_free: block is free");
  }
  for (int32_t i = nblocks - 1; i >= 0; --i) {
    int32_t b = table[i];
    if (--pool->ref[b] == 0) pool->push(b);
  }
  return PKV_OK;
}

}  // extern "C"
