// Host block allocator: one pool of fixed-size blocks, per-sequence block tables,
// reference counts, fork and copy-on-write appends.
//
// Behaviour follows the pages: a sequence takes a new block only when its last
// block is full, so only the last block can be partly empty ("How vLLM Works?",
// section 03; "vLLM and PagedAttention", §2 on-demand allocation bullet); blocks
// of a shared prefix are shared by reference and a write into a shared block
// copies it first ("vLLM and PagedAttention", §2 copy-on-write bullet; "vLLM —
// PagedAttention and Continuous Batching", §2.3).  Only a partly filled last block
// is ever written, so that is the only block copy-on-write ever copies.
//
// Automatic prefix caching ("How vLLM Works?", section 05; "vLLM and
// PagedAttention", section 4; "vLLM — PagedAttention and Continuous Batching",
// §5): sequences made with their token ids key every full block by its tokens,
// the key of the block before it and a per-sequence salt (which keeps tenants
// apart), and a full block whose key is new is cached.  A later sequence whose
// prompt starts with cached blocks takes them instead of new ones, block by
// block from the start until the first key not found; only full blocks are ever
// cached.  A cached block whose last user is released is kept on a released
// list and revived by a later hit; when no free block is left, allocation takes
// over the least recently released one (a sequence's blocks go on that list
// from its last to its first).  Keys are looked up by a 64-bit hash and then
// compared field by field: the salt and the 16 token ids exactly, the block
// before it by that block's 64-bit key hash (so the chain of earlier blocks is
// compared through hashes, not token by token).
//
// Preemption by swapping ("vLLM and PagedAttention", §3 continuous batching, on
// the scheduler's preemption; "How vLLM Works?", section 04): a second pool of
// host block ids.  A swap-out moves a group of sequences to host blocks and
// drops their device references; a swap-in gives them new device blocks.  A
// block held several times inside one group is copied once, so sharing inside
// the group survives the round trip.  A swapped sequence can only be swapped in
// or freed.
//
// The allocator touches no device memory.  It hands (src, dst) copy pairs back to
// the caller, who runs them with pkv_copy_blocks before writing the new tokens
// (or pkv_swap_blocks between the device pool and the host pool).

#include <algorithm>
#include <array>
#include <cstdint>
#include <cstring>
#include <list>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pagedkv.h"
#include "pkv_internal.hpp"

namespace {

struct Seq {
  std::vector<int32_t> table;  // logical block index -> physical block id
  int64_t len = 0;             // tokens held
  bool swapped = false;        // table holds host block ids
  // prefix caching: only for sequences whose token ids are known
  bool tracked = false;
  uint64_t salt = 0;
  std::vector<int32_t> tokens;  // all len token ids
  std::vector<uint64_t> keys;   // key hash of each full block
};

// A cached full block: its key (salt and ids compared exactly on lookup, the
// parent by its 64-bit key hash).
struct CacheEntry {
  int32_t block;
  uint64_t parent;  // key hash of the block before it (0 for a first block)
  uint64_t salt;
  std::array<int32_t, PKV_BLOCK_SIZE> tokens;
  bool same(uint64_t p, uint64_t s, const int32_t* t) const {
    return parent == p && salt == s && std::equal(tokens.begin(), tokens.end(), t);
  }
};

// 64-bit key hash of a full block: the splitmix64 output function applied
// after each of parent, salt and the tokens is folded in.
inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
inline uint64_t block_key(uint64_t parent, uint64_t salt, const int32_t* tokens) {
  uint64_t h = mix64(parent + 0x9E3779B97F4A7C15ull);
  h = mix64(h ^ salt);
  for (int i = 0; i < PKV_BLOCK_SIZE; ++i) h = mix64(h + (uint32_t)tokens[i] + 0x9E3779B97F4A7C15ull);
  return h;
}

// splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): a Weyl sequence passed through a 64-bit mixer.
struct SplitMix64 {
  uint64_t state;
  uint64_t next() {
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  // uniform integer in [0, bound) by multiply-shift (Lemire's method, no rejection;
  // the bias is below bound / 2^64)
  uint64_t below(uint64_t bound) {
    return (uint64_t)(((unsigned __int128)next() * bound) >> 64);
  }
};

inline int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

inline int swapped_error(const char* msg) { return pkv::fail(PKV_ESWAPPED, msg); }

}  // namespace

struct pkv_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;
  // prefix cache: key hash -> entry; per block: its key hash when cached; the
  // released cached blocks (count 0), least recently released first
  std::unordered_map<uint64_t, CacheEntry> cache;
  std::vector<uint64_t> key_of;
  std::vector<char> cached;
  std::list<int32_t> released;
  std::vector<std::list<int32_t>::iterator> released_at;
  std::vector<char> is_released;
  // host pool for swapped sequences: free stack (back() handed out next) and counts
  std::vector<int32_t> hfree;
  std::vector<int32_t> href;

  // Blocks an allocation can take: free ones and released cached ones.
  int64_t available() const { return (int64_t)free_stack.size() + (int64_t)released.size(); }

  // A block for new data: a free one, else the least recently released cached
  // one (dropped from the cache).  Callers check available() first.
  int32_t take() {
    if (!free_stack.empty()) {
      const int32_t b = free_stack.back();
      free_stack.pop_back();
      return b;
    }
    const int32_t b = released.front();
    released.pop_front();
    is_released[b] = 0;
    cache.erase(key_of[b]);
    cached[b] = 0;
    return b;
  }

  // Block idx of s just became full: record its key; cache it if the key is new.
  void register_full(Seq& s, int64_t idx) {
    const uint64_t parent = idx > 0 ? s.keys[idx - 1] : 0;
    const int32_t* t = s.tokens.data() + idx * block_size;
    const uint64_t h = block_key(parent, s.salt, t);
    s.keys.push_back(h);
    const int32_t b = s.table[idx];
    if (cached[b] || cache.count(h)) return;
    CacheEntry e{b, parent, s.salt, {}};
    std::copy(t, t + block_size, e.tokens.begin());
    cache.emplace(h, e);
    key_of[b] = h;
    cached[b] = 1;
  }

  void untrack(Seq& s) {
    s.tracked = false;
    s.tokens.clear();
    s.tokens.shrink_to_fit();
    s.keys.clear();
  }

  // Blocks and CoW copies that appending n tokens to s needs, given pending
  // refcount decrements from earlier members of the same batch.
  void need_for(const Seq& s, int32_t n, std::unordered_map<int32_t, int32_t>& pending,
                int64_t& blocks, int64_t& cows) const {
    if (n <= 0) return;
    const bool partial = (s.len % block_size) != 0;
    if (partial) {
      const int32_t last = s.table.back();
      auto it = pending.find(last);
      const int32_t dec = it == pending.end() ? 0 : it->second;
      if (ref[last] - dec > 1) {
        ++blocks;
        ++cows;
        pending[last] = dec + 1;
      }
    }
    blocks += blocks_for(s.len + n, block_size) - blocks_for(s.len, block_size);
  }

  // Append that is known to fit.  Writes n slots and at most one CoW pair.
  void append_fitting(Seq& s, int32_t n, int32_t* slots, int32_t* pair, int32_t* ncow) {
    *ncow = 0;
    if (n <= 0) return;
    const int32_t bs = block_size;
    if ((s.len % bs) != 0 && ref[s.table.back()] > 1) {
      const int32_t src = s.table.back();
      const int32_t dst = take();
      ref[src] -= 1;
      ref[dst] = 1;
      s.table.back() = dst;
      pair[0] = src;
      pair[1] = dst;
      *ncow = 1;
    }
    for (int32_t i = 0; i < n; ++i) {
      const int64_t pos = s.len + i;
      if (pos % bs == 0) {
        const int32_t b = take();
        ref[b] = 1;
        s.table.push_back(b);
      }
      slots[i] = s.table[pos / bs] * bs + (int32_t)(pos % bs);
    }
    s.len += n;
  }

  // append_fitting for a tracked sequence: the ids are kept and blocks that
  // become full are keyed (and cached when their key is new).
  void append_tokens_fitting(Seq& s, const int32_t* toks, int32_t n, int32_t* slots, int32_t* pair,
                             int32_t* ncow) {
    const int64_t before = s.len;
    append_fitting(s, n, slots, pair, ncow);
    s.tokens.insert(s.tokens.end(), toks, toks + n);
    for (int64_t idx = before / block_size; idx < s.len / block_size; ++idx) register_full(s, idx);
  }

  // A released sequence's blocks: uncached ones back to the free list in table
  // order, cached ones to the released list from the last to the first.
  void release(const Seq& s) {
    if (s.swapped) {
      for (int32_t h : s.table)
        if (--href[h] == 0) hfree.push_back(h);
      return;
    }
    for (int32_t b : s.table)
      if (--ref[b] == 0 && !cached[b]) free_stack.push_back(b);
    for (auto it = s.table.rbegin(); it != s.table.rend(); ++it) {
      const int32_t b = *it;
      if (ref[b] == 0 && cached[b] && !is_released[b]) {
        released.push_back(b);
        released_at[b] = std::prev(released.end());
        is_released[b] = 1;
      }
    }
  }
};

extern "C" {

pkv_allocator* pkv_alloc_create(int32_t num_blocks, int32_t block_size, uint64_t shuffle_seed) {
  if (num_blocks <= 0 || block_size != PKV_BLOCK_SIZE) {
    pkv::set_error("pkv_alloc_create: num_blocks must be > 0 and block_size 16");
    return nullptr;
  }
  pkv_allocator* a = new (std::nothrow) pkv_allocator();
  if (!a) return nullptr;
  try {
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->ref.assign(num_blocks, 0);
    a->key_of.assign(num_blocks, 0);
    a->cached.assign(num_blocks, 0);
    a->released_at.assign(num_blocks, a->released.end());
    a->is_released.assign(num_blocks, 0);
    std::vector<int32_t> order(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) order[i] = i;
    if (shuffle_seed != 0) {
      SplitMix64 rng{shuffle_seed};
      for (int32_t i = num_blocks - 1; i > 0; --i) {
        const int32_t j = (int32_t)rng.below((uint64_t)i + 1);
        std::swap(order[i], order[j]);
      }
    }
    a->free_stack.assign(order.rbegin(), order.rend());  // order[0] is handed out first
  } catch (...) {
    delete a;
    return nullptr;
  }
  return a;
}

void pkv_alloc_destroy(pkv_allocator* a) { delete a; }

int pkv_alloc_add_seq(pkv_allocator* a, int64_t seq_id) {
  if (!a) return pkv::fail(PKV_EINVAL, "pkv_alloc_add_seq: null allocator");
  if (a->seqs.count(seq_id)) return pkv::fail(PKV_EINVAL, "pkv_alloc_add_seq: sequence exists");
  a->seqs.emplace(seq_id, Seq{});
  return PKV_OK;
}

int pkv_alloc_fork(pkv_allocator* a, int64_t parent, int64_t child) {
  if (!a) return pkv::fail(PKV_EINVAL, "pkv_alloc_fork: null allocator");
  auto it = a->seqs.find(parent);
  if (it == a->seqs.end()) return pkv::fail(PKV_ENOSEQ, "pkv_alloc_fork: unknown parent");
  if (a->seqs.count(child)) return pkv::fail(PKV_EINVAL, "pkv_alloc_fork: child exists");
  if (it->second.swapped) return swapped_error("pkv_alloc_fork: parent is swapped out");
  Seq c = it->second;  // copy before emplace: emplace may rehash
  for (int32_t b : c.table) a->ref[b] += 1;
  a->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

int pkv_alloc_append(pkv_allocator* a, int64_t seq_id, int32_t n_tokens, int32_t* slots_out,
                     int32_t* cow_pairs_out, int32_t* num_cow_out) {
  if (!a) return pkv::fail(PKV_EINVAL, "pkv_alloc_append: null allocator");
  if (n_tokens < 0 || (n_tokens > 0 && !slots_out) || !cow_pairs_out || !num_cow_out)
    return pkv::fail(PKV_EINVAL, "pkv_alloc_append: bad arguments");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return pkv::fail(PKV_ENOSEQ, "pkv_alloc_append: unknown sequence");
  if (it->second.swapped) return swapped_error("pkv_alloc_append: sequence is swapped out");
  std::unordered_map<int32_t, int32_t> pending;
  int64_t blocks = 0, cows = 0;
  a->need_for(it->second, n_tokens, pending, blocks, cows);
  if (blocks > a->available()) return pkv::fail(PKV_ENOMEM, "pkv_alloc_append: block pool exhausted");
  if (it->second.len + n_tokens > (int64_t)INT32_MAX)
    return pkv::fail(PKV_EINVAL, "pkv_alloc_append: sequence too long");
  a->append_fitting(it->second, n_tokens, slots_out, cow_pairs_out, num_cow_out);
  if (n_tokens > 0) a->untrack(it->second);  // ids unknown from here on
  return PKV_OK;
}

int pkv_alloc_append_batch(pkv_allocator* a, const int64_t* seq_ids, const int32_t* n_tokens,
                           int32_t num_seqs, int32_t* slots_out, int64_t slots_cap,
                           int32_t* cow_pairs_out, int32_t cow_cap, int32_t* num_cow_out) {
  if (!a || num_seqs < 0 || (num_seqs > 0 && (!seq_ids || !n_tokens)) || !num_cow_out)
    return pkv::fail(PKV_EINVAL, "pkv_alloc_append_batch: bad arguments");
  std::unordered_set<int64_t> seen;
  std::unordered_map<int32_t, int32_t> pending;
  int64_t blocks = 0, cows = 0, total = 0;
  std::vector<Seq*> rows((size_t)num_seqs);
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (n_tokens[i] < 0) return pkv::fail(PKV_EINVAL, "pkv_alloc_append_batch: negative count");
    if (!seen.insert(seq_ids[i]).second)
      return pkv::fail(PKV_EINVAL, "pkv_alloc_append_batch: duplicate sequence id");
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return pkv::fail(PKV_ENOSEQ, "pkv_alloc_append_batch: unknown sequence");
    if (it->second.swapped) return swapped_error("pkv_alloc_append_batch: sequence is swapped out");
    if (it->second.len + n_tokens[i] > (int64_t)INT32_MAX)
      return pkv::fail(PKV_EINVAL, "pkv_alloc_append_batch: sequence too long");
    rows[i] = &it->second;
    a->need_for(it->second, n_tokens[i], pending, blocks, cows);
    total += n_tokens[i];
  }
  if (total > slots_cap || (total > 0 && !slots_out))
    return pkv::fail(PKV_EINVAL, "pkv_alloc_append_batch: slots_out too small");
  if (cows > cow_cap || (cows > 0 && !cow_pairs_out))
    return pkv::fail(PKV_EINVAL, "pkv_alloc_append_batch: cow_pairs_out too small");
  if (blocks > a->available())
    return pkv::fail(PKV_ENOMEM, "pkv_alloc_append_batch: block pool exhausted");
  int64_t off = 0;
  int32_t ncow_total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    int32_t pair[2], ncow = 0;
    a->append_fitting(*rows[i], n_tokens[i], slots_out + off, pair, &ncow);
    if (n_tokens[i] > 0) a->untrack(*rows[i]);
    off += n_tokens[i];
    if (ncow) {
      cow_pairs_out[2 * ncow_total] = pair[0];
      cow_pairs_out[2 * ncow_total + 1] = pair[1];
      ++ncow_total;
    }
  }
  *num_cow_out = ncow_total;
  return PKV_OK;
}

int pkv_alloc_free_seq(pkv_allocator* a, int64_t seq_id) {
  if (!a) return pkv::fail(PKV_EINVAL, "pkv_alloc_free_seq: null allocator");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return pkv::fail(PKV_ENOSEQ, "pkv_alloc_free_seq: unknown sequence");
  a->release(it->second);
  a->seqs.erase(it);
  return PKV_OK;
}

int pkv_alloc_block_table(const pkv_allocator* a, int64_t seq_id, int32_t* out, int32_t cap,
                          int32_t* len_out) {
  if (!a || !len_out) return pkv::fail(PKV_EINVAL, "pkv_alloc_block_table: bad arguments");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return pkv::fail(PKV_ENOSEQ, "pkv_alloc_block_table: unknown sequence");
  if (it->second.swapped) return swapped_error("pkv_alloc_block_table: sequence is swapped out");
  const auto& t = it->second.table;
  *len_out = (int32_t)t.size();
  if ((int64_t)t.size() > cap || (!t.empty() && !out))
    return pkv::fail(PKV_EINVAL, "pkv_alloc_block_table: output too small");
  if (!t.empty()) std::memcpy(out, t.data(), t.size() * sizeof(int32_t));
  return PKV_OK;
}

int pkv_alloc_block_tables(const pkv_allocator* a, const int64_t* seq_ids, int32_t num_seqs,
                           int32_t* tables_out, int32_t max_blocks, int32_t fill,
                           int32_t* context_lens_out) {
  if (!a || num_seqs < 0 || max_blocks <= 0 ||
      (num_seqs > 0 && (!seq_ids || !tables_out || !context_lens_out)))
    return pkv::fail(PKV_EINVAL, "pkv_alloc_block_tables: bad arguments");
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return pkv::fail(PKV_ENOSEQ, "pkv_alloc_block_tables: unknown sequence");
    if (it->second.swapped) return swapped_error("pkv_alloc_block_tables: sequence is swapped out");
    if ((int64_t)it->second.table.size() > max_blocks || it->second.len > INT32_MAX)
      return pkv::fail(PKV_EINVAL, "pkv_alloc_block_tables: table wider than max_blocks");
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = a->seqs.find(seq_ids[i])->second;
    int32_t* row = tables_out + (int64_t)i * max_blocks;
    const size_t n = s.table.size();
    if (n) std::memcpy(row, s.table.data(), n * sizeof(int32_t));
    std::fill(row + n, row + max_blocks, fill);
    context_lens_out[i] = (int32_t)s.len;
  }
  return PKV_OK;
}

int64_t pkv_alloc_seq_len(const pkv_allocator* a, int64_t seq_id) {
  if (!a) return pkv::fail(PKV_EINVAL, "pkv_alloc_seq_len: null allocator");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return pkv::fail(PKV_ENOSEQ, "pkv_alloc_seq_len: unknown sequence");
  return it->second.len;
}

int32_t pkv_alloc_num_free(const pkv_allocator* a) { return a ? (int32_t)a->available() : PKV_EINVAL; }

int32_t pkv_alloc_num_cached(const pkv_allocator* a) { return a ? (int32_t)a->released.size() : PKV_EINVAL; }

int pkv_alloc_add_seq_tokens(pkv_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                             uint64_t salt, int32_t* slots_out, int32_t* num_cached_out) {
  if (!a || n_tokens < 0 || (n_tokens > 0 && (!tokens || !slots_out)) || !num_cached_out)
    return pkv::fail(PKV_EINVAL, "pkv_alloc_add_seq_tokens: bad arguments");
  if (a->seqs.count(seq_id)) return pkv::fail(PKV_EINVAL, "pkv_alloc_add_seq_tokens: sequence exists");
  const int32_t bs = a->block_size;
  // cached full blocks from the start, up to the first key not found
  std::vector<std::pair<int32_t, uint64_t>> hits;
  uint64_t parent = 0;
  int64_t revived = 0;
  for (int32_t i = 0; i + 1 <= n_tokens / bs; ++i) {
    const int32_t* t = tokens + (int64_t)i * bs;
    const uint64_t h = block_key(parent, salt, t);
    auto it = a->cache.find(h);
    if (it == a->cache.end() || !it->second.same(parent, salt, t)) break;
    hits.emplace_back(it->second.block, h);
    if (a->ref[it->second.block] == 0) ++revived;
    parent = h;
  }
  const int64_t need = blocks_for(n_tokens, bs) - (int64_t)hits.size();
  if (need > a->available() - revived)
    return pkv::fail(PKV_ENOMEM, "pkv_alloc_add_seq_tokens: block pool exhausted");
  Seq s;
  s.tracked = true;
  s.salt = salt;
  for (const auto& hk : hits) {
    const int32_t b = hk.first;
    if (a->is_released[b]) {
      a->released.erase(a->released_at[b]);
      a->is_released[b] = 0;
    }
    a->ref[b] += 1;
    s.table.push_back(b);
    s.keys.push_back(hk.second);
  }
  const int32_t n_cached = (int32_t)hits.size() * bs;
  s.tokens.assign(tokens, tokens + n_cached);
  s.len = n_cached;
  for (int32_t i = 0; i < n_cached; ++i) slots_out[i] = -1;
  int32_t pair[2], ncow = 0;  // a sequence of whole cached blocks has no partial block to copy
  a->append_tokens_fitting(s, tokens + n_cached, n_tokens - n_cached, slots_out + n_cached, pair, &ncow);
  a->seqs.emplace(seq_id, std::move(s));
  *num_cached_out = n_cached;
  return PKV_OK;
}

int pkv_alloc_append_tokens(pkv_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                            int32_t* slots_out, int32_t* cow_pairs_out, int32_t* num_cow_out) {
  if (!a || n_tokens < 0 || (n_tokens > 0 && (!tokens || !slots_out)) || !cow_pairs_out || !num_cow_out)
    return pkv::fail(PKV_EINVAL, "pkv_alloc_append_tokens: bad arguments");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return pkv::fail(PKV_ENOSEQ, "pkv_alloc_append_tokens: unknown sequence");
  if (it->second.swapped) return swapped_error("pkv_alloc_append_tokens: sequence is swapped out");
  if (!it->second.tracked)
    return pkv::fail(PKV_EINVAL, "pkv_alloc_append_tokens: sequence was not made with token ids");
  std::unordered_map<int32_t, int32_t> pending;
  int64_t blocks = 0, cows = 0;
  a->need_for(it->second, n_tokens, pending, blocks, cows);
  if (blocks > a->available()) return pkv::fail(PKV_ENOMEM, "pkv_alloc_append_tokens: block pool exhausted");
  if (it->second.len + n_tokens > (int64_t)INT32_MAX)
    return pkv::fail(PKV_EINVAL, "pkv_alloc_append_tokens: sequence too long");
  a->append_tokens_fitting(it->second, tokens, n_tokens, slots_out, cow_pairs_out, num_cow_out);
  return PKV_OK;
}

int32_t pkv_alloc_num_blocks(const pkv_allocator* a) { return a ? a->num_blocks : PKV_EINVAL; }

int32_t pkv_alloc_refcount(const pkv_allocator* a, int32_t block_id) {
  if (!a || block_id < 0 || block_id >= a->num_blocks) return -1;
  return a->ref[block_id];
}

int pkv_alloc_set_host_pool(pkv_allocator* a, int32_t num_host_blocks) {
  if (!a || num_host_blocks < 0) return pkv::fail(PKV_EINVAL, "pkv_alloc_set_host_pool: bad arguments");
  for (const auto& kv : a->seqs)
    if (kv.second.swapped) return swapped_error("pkv_alloc_set_host_pool: sequences are swapped out");
  try {
    std::vector<int32_t> hfree((size_t)num_host_blocks);
    for (int32_t i = 0; i < num_host_blocks; ++i) hfree[(size_t)i] = num_host_blocks - 1 - i;
    a->href.assign((size_t)num_host_blocks, 0);
    a->hfree.swap(hfree);
  } catch (...) {
    return pkv::fail(PKV_ENOMEM, "pkv_alloc_set_host_pool: out of host memory");
  }
  return PKV_OK;
}

namespace {

// Validates a swap group: known, distinct ids, all with swapped == want.
int swap_group(pkv_allocator* a, const int64_t* ids, int32_t n, bool want, const char* who,
               std::vector<Seq*>& rows) {
  std::unordered_set<int64_t> seen;
  rows.resize((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    if (!seen.insert(ids[i]).second) return pkv::fail(PKV_EINVAL, who);
    auto it = a->seqs.find(ids[i]);
    if (it == a->seqs.end()) return pkv::fail(PKV_ENOSEQ, who);
    if (it->second.swapped != want) return swapped_error(who);
    rows[(size_t)i] = &it->second;
  }
  return PKV_OK;
}

// Distinct block ids over the group's tables, in order of first appearance.
std::vector<int32_t> distinct_blocks(const std::vector<Seq*>& rows) {
  std::vector<int32_t> out;
  std::unordered_set<int32_t> seen;
  for (const Seq* s : rows)
    for (int32_t b : s->table)
      if (seen.insert(b).second) out.push_back(b);
  return out;
}

}  // namespace

int pkv_alloc_swap_out(pkv_allocator* a, const int64_t* seq_ids, int32_t num_seqs, int32_t* pairs_out,
                       int32_t pairs_cap, int32_t* num_pairs_out) {
  if (!a || num_seqs < 0 || (num_seqs > 0 && !seq_ids) || !num_pairs_out || pairs_cap < 0)
    return pkv::fail(PKV_EINVAL, "pkv_alloc_swap_out: bad arguments");
  std::vector<Seq*> rows;
  const int rc = swap_group(a, seq_ids, num_seqs, false, "pkv_alloc_swap_out: bad sequence in the group", rows);
  if (rc != PKV_OK) return rc;
  const std::vector<int32_t> blocks = distinct_blocks(rows);
  if ((int64_t)blocks.size() > pairs_cap || (!blocks.empty() && !pairs_out))
    return pkv::fail(PKV_EINVAL, "pkv_alloc_swap_out: pairs_out too small");
  if (blocks.size() > a->hfree.size()) return pkv::fail(PKV_ENOMEM, "pkv_alloc_swap_out: host pool exhausted");
  std::unordered_map<int32_t, int32_t> to_host;
  for (size_t i = 0; i < blocks.size(); ++i) {
    const int32_t h = a->hfree.back();
    a->hfree.pop_back();
    to_host[blocks[i]] = h;
    pairs_out[2 * i] = blocks[i];
    pairs_out[2 * i + 1] = h;
  }
  for (Seq* s : rows) {
    a->release(*s);  // device references of the group dropped
    for (int32_t& b : s->table) {
      b = to_host[b];
      a->href[b] += 1;
    }
    s->swapped = true;
  }
  *num_pairs_out = (int32_t)blocks.size();
  return PKV_OK;
}

int pkv_alloc_swap_in(pkv_allocator* a, const int64_t* seq_ids, int32_t num_seqs, int32_t* pairs_out,
                      int32_t pairs_cap, int32_t* num_pairs_out) {
  if (!a || num_seqs < 0 || (num_seqs > 0 && !seq_ids) || !num_pairs_out || pairs_cap < 0)
    return pkv::fail(PKV_EINVAL, "pkv_alloc_swap_in: bad arguments");
  std::vector<Seq*> rows;
  const int rc = swap_group(a, seq_ids, num_seqs, true, "pkv_alloc_swap_in: bad sequence in the group", rows);
  if (rc != PKV_OK) return rc;
  const std::vector<int32_t> hblocks = distinct_blocks(rows);
  if ((int64_t)hblocks.size() > pairs_cap || (!hblocks.empty() && !pairs_out))
    return pkv::fail(PKV_EINVAL, "pkv_alloc_swap_in: pairs_out too small");
  if ((int64_t)hblocks.size() > a->available())
    return pkv::fail(PKV_ENOMEM, "pkv_alloc_swap_in: block pool exhausted");
  std::unordered_map<int32_t, int32_t> to_dev;
  for (size_t i = 0; i < hblocks.size(); ++i) {
    const int32_t b = a->take();
    to_dev[hblocks[i]] = b;
    pairs_out[2 * i] = hblocks[i];
    pairs_out[2 * i + 1] = b;
  }
  for (Seq* s : rows) {
    a->release(*s);  // host references dropped (s is still marked swapped)
    for (int32_t& h : s->table) {
      h = to_dev[h];
      a->ref[h] += 1;
    }
    s->swapped = false;
  }
  *num_pairs_out = (int32_t)hblocks.size();
  return PKV_OK;
}

int pkv_alloc_is_swapped(const pkv_allocator* a, int64_t seq_id) {
  if (!a) return pkv::fail(PKV_EINVAL, "pkv_alloc_is_swapped: null allocator");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return pkv::fail(PKV_ENOSEQ, "pkv_alloc_is_swapped: unknown sequence");
  return it->second.swapped ? 1 : 0;
}

int pkv_alloc_host_table(const pkv_allocator* a, int64_t seq_id, int32_t* out, int32_t cap, int32_t* len_out) {
  if (!a || !len_out) return pkv::fail(PKV_EINVAL, "pkv_alloc_host_table: bad arguments");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return pkv::fail(PKV_ENOSEQ, "pkv_alloc_host_table: unknown sequence");
  if (!it->second.swapped) return swapped_error("pkv_alloc_host_table: sequence is not swapped out");
  const auto& t = it->second.table;
  *len_out = (int32_t)t.size();
  if ((int64_t)t.size() > cap || (!t.empty() && !out))
    return pkv::fail(PKV_EINVAL, "pkv_alloc_host_table: output too small");
  if (!t.empty()) std::memcpy(out, t.data(), t.size() * sizeof(int32_t));
  return PKV_OK;
}

int32_t pkv_alloc_num_free_host(const pkv_allocator* a) { return a ? (int32_t)a->hfree.size() : PKV_EINVAL; }

int32_t pkv_alloc_host_refcount(const pkv_allocator* a, int32_t host_block) {
  if (!a || host_block < 0 || host_block >= (int32_t)a->href.size()) return -1;
  return a->href[(size_t)host_block];
}

}  // extern "C"
