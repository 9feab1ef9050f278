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
// The allocator touches no device memory.  It hands (src, dst) copy pairs back to
// the caller, who runs them with pkv_copy_blocks before writing the new tokens.

#include <algorithm>
#include <cstdint>
#include <cstring>
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
};

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

}  // namespace

struct pkv_allocator {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;

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
      const int32_t dst = free_stack.back();
      free_stack.pop_back();
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
        const int32_t b = free_stack.back();
        free_stack.pop_back();
        ref[b] = 1;
        s.table.push_back(b);
      }
      slots[i] = s.table[pos / bs] * bs + (int32_t)(pos % bs);
    }
    s.len += n;
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
  std::unordered_map<int32_t, int32_t> pending;
  int64_t blocks = 0, cows = 0;
  a->need_for(it->second, n_tokens, pending, blocks, cows);
  if (blocks > (int64_t)a->free_stack.size())
    return pkv::fail(PKV_ENOMEM, "pkv_alloc_append: block pool exhausted");
  if (it->second.len + n_tokens > (int64_t)INT32_MAX)
    return pkv::fail(PKV_EINVAL, "pkv_alloc_append: sequence too long");
  a->append_fitting(it->second, n_tokens, slots_out, cow_pairs_out, num_cow_out);
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
  if (blocks > (int64_t)a->free_stack.size())
    return pkv::fail(PKV_ENOMEM, "pkv_alloc_append_batch: block pool exhausted");
  int64_t off = 0;
  int32_t ncow_total = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    int32_t pair[2], ncow = 0;
    a->append_fitting(*rows[i], n_tokens[i], slots_out + off, pair, &ncow);
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
  for (int32_t b : it->second.table) {
    if (--a->ref[b] == 0) a->free_stack.push_back(b);
  }
  a->seqs.erase(it);
  return PKV_OK;
}

int pkv_alloc_block_table(const pkv_allocator* a, int64_t seq_id, int32_t* out, int32_t cap,
                          int32_t* len_out) {
  if (!a || !len_out) return pkv::fail(PKV_EINVAL, "pkv_alloc_block_table: bad arguments");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return pkv::fail(PKV_ENOSEQ, "pkv_alloc_block_table: unknown sequence");
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

int32_t pkv_alloc_num_free(const pkv_allocator* a) {
  return a ? (int32_t)a->free_stack.size() : PKV_EINVAL;
}

int32_t pkv_alloc_num_blocks(const pkv_allocator* a) { return a ? a->num_blocks : PKV_EINVAL; }

int32_t pkv_alloc_refcount(const pkv_allocator* a, int32_t block_id) {
  if (!a || block_id < 0 || block_id >= a->num_blocks) return -1;
  return a->ref[block_id];
}

}  // extern "C"
