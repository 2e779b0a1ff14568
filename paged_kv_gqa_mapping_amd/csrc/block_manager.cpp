// Host-side paged-KV block manager: physical block allocation with reference
// counts, prefix reuse of full blocks by a hash chained over the token ids
// (checked token for token on a hit), one-token appends for decode, and the
// block tables / slot mappings the device kernels consume.  Declarations and
// the contract are in include/pkv.h.
#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/pkv.h"

namespace {

thread_local std::string g_bm_error;

int bm_fail(int status, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_bm_error = buf;
  return status;
}

// 64-bit FNV-1a over the 32-bit token ids of a block, seeded with the hash of
// the previous block (so equal blocks after different prefixes hash apart),
// then the splitmix64 finaliser to spread the bits.
uint64_t block_hash(uint64_t prev, const int32_t* tokens, int32_t n) {
  uint64_t h = 0xcbf29ce484222325ull ^ prev;
  for (int32_t i = 0; i < n; ++i) {
    h ^= static_cast<uint32_t>(tokens[i]);
    h *= 0x100000001b3ull;
  }
  h ^= h >> 30;
  h *= 0xbf58476d1ce4e5b9ull;
  h ^= h >> 27;
  h *= 0x94d049bb133111ebull;
  h ^= h >> 31;
  return h;
}

struct Seq {
  std::vector<int32_t> blocks;  // physical ids, in logical order
  std::vector<int32_t> tokens;  // every token id of the sequence
  uint64_t last_full_hash = 0;  // hash of the last full block (0 before the first)
  int64_t cached_tokens = 0;    // prompt tokens found in the prefix cache at allocation
  uint64_t order = 0;           // allocation order (preemption takes the most recent)
};

}  // namespace

struct pkv_block_manager {
  int32_t block_size;
  bool prefix_cache;
  std::vector<int32_t> ref;    // reference count per block
  std::vector<uint64_t> hash;  // hash of a full, registered block (valid when has_hash)
  std::vector<uint8_t> has_hash;
  std::vector<std::vector<int32_t>> block_tokens;  // token ids of registered blocks (hit check)
  // free list: doubly linked over block ids, FIFO (a freed block goes to the
  // back, allocation takes the front, so cached blocks live as long as possible)
  std::vector<int32_t> prev, next;
  std::vector<uint8_t> in_free;
  int32_t head = -1, tail = -1;
  int64_t num_free = 0;
  std::unordered_map<uint64_t, int32_t> cache;  // hash -> block
  std::unordered_map<int64_t, Seq> seqs;
  uint64_t next_order = 0;
  std::mutex mu;

  void push_back(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    in_free[b] = 1;
    ++num_free;
  }
  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    in_free[b] = 0;
    --num_free;
  }
  // take a block for new data: the oldest free block loses its cache entry
  int32_t take_fresh() {
    const int32_t b = head;
    unlink(b);
    if (has_hash[b]) {
      auto it = cache.find(hash[b]);
      if (it != cache.end() && it->second == b) cache.erase(it);
      has_hash[b] = 0;
      block_tokens[b].clear();
    }
    ref[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) push_back(b);
  }
  // a sequence's blocks, last first: its prefix blocks enter the free list last
  // and so keep their cache registration longest (they are the most reusable)
  void release_all(const std::vector<int32_t>& blocks) {
    for (auto it = blocks.rbegin(); it != blocks.rend(); ++it) release(*it);
  }
  // a cached block for this (hash, tokens), or -1
  int32_t lookup(uint64_t h, const int32_t* tokens) const {
    auto it = cache.find(h);
    if (it == cache.end()) return -1;
    const int32_t b = it->second;
    if (!std::equal(block_tokens[b].begin(), block_tokens[b].end(), tokens)) return -1;
    return b;
  }
  void register_full(int32_t b, uint64_t h, const int32_t* tokens) {
    if (!prefix_cache || cache.count(h)) return;  // an equal block is already registered
    hash[b] = h;
    has_hash[b] = 1;
    block_tokens[b].assign(tokens, tokens + block_size);
    cache[h] = b;
  }
};

extern "C" {

const char* pkv_bm_last_error(void) { return g_bm_error.c_str(); }

pkv_block_manager* pkv_bm_create(int64_t num_blocks, int32_t block_size, int32_t enable_prefix_cache) {
  // slots are int32: num_blocks * block_size must fit
  if (num_blocks < 1 || block_size < 1 || num_blocks * (int64_t)block_size > 0x7fffffffLL) {
    bm_fail(PKV_ERR_INVALID_ARG, "num_blocks %lld x block_size %d is empty or exceeds the int32 slot range",
            (long long)num_blocks, block_size);
    return nullptr;
  }
  pkv_block_manager* m = new (std::nothrow) pkv_block_manager();
  if (!m) {
    bm_fail(PKV_ERR_INVALID_ARG, "out of host memory");
    return nullptr;
  }
  const size_t n = (size_t)num_blocks;
  m->block_size = block_size;
  m->prefix_cache = enable_prefix_cache != 0;
  m->ref.assign(n, 0);
  m->hash.assign(n, 0);
  m->has_hash.assign(n, 0);
  m->block_tokens.resize(n);
  m->prev.assign(n, -1);
  m->next.assign(n, -1);
  m->in_free.assign(n, 0);
  for (int32_t b = 0; b < (int32_t)n; ++b) m->push_back(b);
  return m;
}

void pkv_bm_destroy(pkv_block_manager* m) { delete m; }

int64_t pkv_bm_num_free_blocks(pkv_block_manager* m) {
  std::lock_guard<std::mutex> g(m->mu);
  return m->num_free;
}

int32_t pkv_bm_block_refcount(pkv_block_manager* m, int32_t block) {
  std::lock_guard<std::mutex> g(m->mu);
  if (block < 0 || block >= (int32_t)m->ref.size()) return bm_fail(PKV_ERR_INVALID_ARG, "block %d out of range", block);
  return m->ref[block];
}

// Blocks a prompt of n tokens would take from the free list: its full blocks
// not found in the prefix cache plus the partial tail block (cache hits that
// sit in the free list are taken from it too, and are counted).
static int64_t blocks_needed(pkv_block_manager* m, const int32_t* tokens, int64_t n) {
  const int32_t bs = m->block_size;
  const int64_t nblk = (n + bs - 1) / bs;
  int64_t need = 0;
  uint64_t h = 0;
  bool hit_run = m->prefix_cache;
  for (int64_t i = 0; i < nblk; ++i) {
    const bool full = (i + 1) * bs <= n;
    if (hit_run && full) {
      h = block_hash(h, tokens + i * bs, bs);
      const int32_t b = m->lookup(h, tokens + i * bs);
      if (b >= 0) {
        if (m->in_free[b]) ++need;
        continue;
      }
      hit_run = false;
    }
    ++need;
  }
  return need;
}

int pkv_bm_can_allocate(pkv_block_manager* m, const int32_t* tokens, int64_t num_tokens) {
  if (num_tokens < 0 || (num_tokens > 0 && !tokens)) return bm_fail(PKV_ERR_INVALID_ARG, "bad token array");
  std::lock_guard<std::mutex> g(m->mu);
  return blocks_needed(m, tokens, num_tokens) <= m->num_free ? 1 : 0;
}

int pkv_bm_allocate(pkv_block_manager* m, int64_t seq_id, const int32_t* tokens, int64_t num_tokens,
                    int64_t* num_cached_tokens) {
  if (num_tokens < 0 || (num_tokens > 0 && !tokens)) return bm_fail(PKV_ERR_INVALID_ARG, "bad token array");
  std::lock_guard<std::mutex> g(m->mu);
  if (m->seqs.count(seq_id)) return bm_fail(PKV_ERR_INVALID_ARG, "sequence %lld already allocated", (long long)seq_id);
  const int64_t need = blocks_needed(m, tokens, num_tokens);
  if (need > m->num_free)
    return bm_fail(PKV_ERR_OUT_OF_BLOCKS, "prompt needs %lld free blocks, %lld free", (long long)need,
                   (long long)m->num_free);
  Seq s;
  const int32_t bs = m->block_size;
  const int64_t nblk = (num_tokens + bs - 1) / bs;
  uint64_t h = 0;
  bool hit_run = m->prefix_cache;
  for (int64_t i = 0; i < nblk; ++i) {
    const int32_t* blk_tokens = tokens + i * bs;
    const bool full = (i + 1) * bs <= num_tokens;
    int32_t b = -1;
    if (full) h = block_hash(h, blk_tokens, bs);
    if (hit_run && full) {
      b = m->lookup(h, blk_tokens);
      if (b >= 0) {
        if (m->in_free[b]) m->unlink(b);
        ++m->ref[b];
        s.cached_tokens += bs;
      } else {
        hit_run = false;
      }
    }
    if (b < 0) {
      b = m->take_fresh();
      if (full) m->register_full(b, h, blk_tokens);
    }
    s.blocks.push_back(b);
    if (full) s.last_full_hash = h;
  }
  s.tokens.assign(tokens, tokens + num_tokens);
  s.order = m->next_order++;
  if (num_cached_tokens) *num_cached_tokens = s.cached_tokens;
  m->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* m, int64_t seq_id, int32_t token, int32_t* slot) {
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return bm_fail(PKV_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seq_id);
  Seq& s = it->second;
  const int32_t bs = m->block_size;
  const int64_t pos = (int64_t)s.tokens.size();
  if (pos % bs == 0) {  // the new token starts a block
    if (m->num_free == 0) return bm_fail(PKV_ERR_OUT_OF_BLOCKS, "no free block for sequence %lld", (long long)seq_id);
    s.blocks.push_back(m->take_fresh());
  }
  const int32_t b = s.blocks.back();
  s.tokens.push_back(token);
  if (slot) *slot = b * bs + (int32_t)(pos % bs);
  if ((pos + 1) % bs == 0) {  // the block is now full: register it for reuse
    const int32_t* blk_tokens = s.tokens.data() + (pos + 1 - bs);
    s.last_full_hash = block_hash(s.last_full_hash, blk_tokens, bs);
    if (m->ref[b] == 1) m->register_full(b, s.last_full_hash, blk_tokens);
  }
  return PKV_OK;
}

int pkv_bm_free(pkv_block_manager* m, int64_t seq_id) {
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return bm_fail(PKV_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seq_id);
  m->release_all(it->second.blocks);
  m->seqs.erase(it);
  return PKV_OK;
}

// Leading tokens of a token array that the prefix cache holds (whole blocks,
// up to the first miss).
static int64_t cached_prefix(pkv_block_manager* m, const int32_t* tokens, int64_t n) {
  if (!m->prefix_cache) return 0;
  const int32_t bs = m->block_size;
  uint64_t h = 0;
  int64_t i = 0;
  for (; (i + 1) * bs <= n; ++i) {
    h = block_hash(h, tokens + i * bs, bs);
    if (m->lookup(h, tokens + i * bs) < 0) break;
  }
  return i * bs;
}

int pkv_bm_preempt(pkv_block_manager* m, int64_t* seq_id, int64_t* num_cached_tokens) {
  std::lock_guard<std::mutex> g(m->mu);
  if (m->seqs.empty()) return bm_fail(PKV_ERR_INVALID_ARG, "no sequence holds blocks");
  auto victim = m->seqs.begin();
  for (auto it = m->seqs.begin(); it != m->seqs.end(); ++it)
    if (it->second.order > victim->second.order) victim = it;
  m->release_all(victim->second.blocks);
  const int64_t cached = cached_prefix(m, victim->second.tokens.data(), (int64_t)victim->second.tokens.size());
  if (seq_id) *seq_id = victim->first;
  if (num_cached_tokens) *num_cached_tokens = cached;
  m->seqs.erase(victim);
  return PKV_OK;
}

int64_t pkv_bm_seq_len(pkv_block_manager* m, int64_t seq_id) {
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return bm_fail(PKV_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seq_id);
  return (int64_t)it->second.tokens.size();
}

int32_t pkv_bm_block_table(pkv_block_manager* m, int64_t seq_id, int32_t* out, int32_t capacity, int32_t pad) {
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return bm_fail(PKV_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seq_id);
  const auto& blocks = it->second.blocks;
  if ((int64_t)blocks.size() > capacity)
    return bm_fail(PKV_ERR_INVALID_ARG, "table row of %d entries cannot hold %zu blocks", capacity, blocks.size());
  if (!out && capacity > 0) return bm_fail(PKV_ERR_INVALID_ARG, "null output");
  std::copy(blocks.begin(), blocks.end(), out);
  std::fill(out + blocks.size(), out + capacity, pad);
  return (int32_t)blocks.size();
}

int pkv_bm_slot_mapping(pkv_block_manager* m, int64_t seq_id, int64_t first_pos, int64_t count, int32_t* out) {
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return bm_fail(PKV_ERR_INVALID_ARG, "unknown sequence %lld", (long long)seq_id);
  const Seq& s = it->second;
  if (first_pos < 0 || count < 0 || first_pos + count > (int64_t)s.tokens.size() || (count > 0 && !out))
    return bm_fail(PKV_ERR_INVALID_ARG, "positions [%lld, %lld) outside the sequence of %zu tokens",
                   (long long)first_pos, (long long)(first_pos + count), s.tokens.size());
  const int32_t bs = m->block_size;
  for (int64_t i = 0; i < count; ++i) {
    const int64_t p = first_pos + i;
    out[i] = s.blocks[p / bs] * bs + (int32_t)(p % bs);
  }
  return PKV_OK;
}

}  // extern "C"
