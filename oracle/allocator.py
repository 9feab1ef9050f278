"""Python model of the paged block allocator (test infrastructure only).

What it follows:

* one pool of fixed-size blocks shared by all sequences, each sequence owning a
  table from logical block index to physical block id ("vLLM and PagedAttention",
  §2 block-table figure and bullets; "How vLLM Works?", section 03);
* a sequence takes a new block only when its current last block is full, so only
  the last block can be partly empty ("How vLLM Works?", section 03; "vLLM and
  PagedAttention", §2 on-demand allocation bullet);
* sequences with the same prefix point at the same physical blocks, and a write
  into a shared block copies it first ("vLLM and PagedAttention", §2 shareable
  prefixes with copy-on-write; "vLLM — PagedAttention and Continuous Batching",
  §2.3; "How vLLM Works?", section 03 on a prompt branching into several samples).

Reference counts: a block's count is the number of table entries (over all live
sequences) that hold it; it returns to the free list when the count reaches 0.
Only a partly filled last block is ever written, so only that block is ever
copied; full shared blocks stay shared.

Operations are all-or-nothing: when the pool cannot supply every block an
operation needs, ``MemoryError`` is raised and no state changes.
"""


def slot_for_position(table_row, pos, block_size=16):
    """Flat slot index of logical position ``pos``: ``table[pos // bs] * bs + pos % bs``."""
    return int(table_row[pos // block_size]) * block_size + pos % block_size


class BlockAllocatorModel:
    """Refcounted block pool with per-sequence tables and copy-on-write appends.

    ``free_order`` is the order in which free blocks are handed out (a random
    permutation gives the pages' scattered physical placement); default 0..NB-1.
    """

    def __init__(self, num_blocks, block_size=16, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self._free = order[::-1]          # pop() from the end hands out order[0] first
        self._ref = [0] * num_blocks
        self._tables = {}
        self._lens = {}

    # --- queries -----------------------------------------------------------
    def num_free(self):
        return len(self._free)

    def refcount(self, block):
        return self._ref[block]

    def block_table(self, seq):
        return list(self._tables[seq])

    def seq_len(self, seq):
        return self._lens[seq]

    def seqs(self):
        return list(self._tables)

    # --- operations --------------------------------------------------------
    def add_seq(self, seq):
        if seq in self._tables:
            raise KeyError(f"sequence {seq} exists")
        self._tables[seq] = []
        self._lens[seq] = 0

    def fork(self, parent, child):
        """Child shares every block of the parent (counts +1); same length."""
        if child in self._tables:
            raise KeyError(f"sequence {child} exists")
        tbl = list(self._tables[parent])
        for b in tbl:
            self._ref[b] += 1
        self._tables[child] = tbl
        self._lens[child] = self._lens[parent]

    def append(self, seq, n_tokens):
        """Reserve slots for ``n_tokens`` new tokens at the end of ``seq``.

        Returns ``(slots, cow_pairs)``: the flat slot of each new token, and the
        ``(src, dst)`` block copies the caller must perform before writing.
        """
        if n_tokens < 0:
            raise ValueError("n_tokens must be >= 0")
        bs = self.block_size
        tbl = self._tables[seq]
        L = self._lens[seq]
        partial_shared = (L % bs != 0) and self._ref[tbl[-1]] > 1
        cow = partial_shared and n_tokens > 0
        new_blocks = -(-(L + n_tokens) // bs) - (-(-L // bs))
        need = new_blocks + (1 if cow else 0)
        if need > len(self._free):
            raise MemoryError("block pool exhausted")
        pairs = []
        if cow:
            src = tbl[-1]
            dst = self._free.pop()
            self._ref[src] -= 1
            self._ref[dst] = 1
            tbl[-1] = dst
            pairs.append((src, dst))
        slots = []
        for pos in range(L, L + n_tokens):
            if pos % bs == 0:
                b = self._free.pop()
                self._ref[b] = 1
                tbl.append(b)
            slots.append(slot_for_position(tbl, pos, bs))
        self._lens[seq] = L + n_tokens
        return slots, pairs

    def free_seq(self, seq):
        """Drop a sequence; blocks whose count reaches 0 return to the free list."""
        tbl = self._tables.pop(seq)
        del self._lens[seq]
        for b in tbl:
            self._ref[b] -= 1
            if self._ref[b] == 0:
                self._free.append(b)


class PrefixCachingAllocatorModel(BlockAllocatorModel):
    """The block allocator with automatic prefix caching (test infrastructure only).

    What it follows ("How vLLM Works?", section 05 on prefix caching; "vLLM and
    PagedAttention", section 4 on reusing the system prompt's KV; "vLLM —
    PagedAttention and Continuous Batching", §5 prefix-caching bullet):

    * a full block is identified by its own tokens and every token before it,
      plus optional extra values (here one salt per sequence, which keeps
      tenants apart); a block that is not full is never cached or shared
      through the cache;
    * a new request whose prompt starts with the same full blocks as an earlier
      one reuses those blocks instead of computing them again: lookup runs
      block by block from the start and stops at the first block not found;
    * cached blocks whose last user is gone are kept, least recently released
      first out, and are reused by a later hit or taken over for new data when
      no free block is left.

    Readings where the pages are silent: a block's key here is the exact tuple
    (parent key, salt, tokens), so equal keys mean equal contents; a released
    sequence hands its uncached blocks back to the free list in table order (as
    the plain allocator does) and its cached ones to the released list from its
    last to its first, so a prefix's later blocks are taken over before its
    earlier ones; a block that becomes
    full while an equal block is already cached is not cached a second time;
    a plain ``append`` (token ids unknown) ends caching for that sequence.
    """

    def __init__(self, num_blocks, block_size=16, free_order=None):
        super().__init__(num_blocks, block_size, free_order)
        self._cache = {}                  # key -> block
        self._key_of = {}                 # block -> key (cached blocks only)
        self._evictable = {}              # cached blocks with count 0, oldest first (dict order)
        self._toks = {}                   # seq -> token ids (tracked sequences)
        self._salt = {}
        self._keys = {}                   # seq -> keys of its full blocks

    # --- queries -----------------------------------------------------------
    def num_free(self):
        """Blocks an allocation can take: free ones and cached ones nobody uses."""
        return len(self._free) + len(self._evictable)

    def num_cached(self):
        return len(self._evictable)

    # --- internals ---------------------------------------------------------
    def _take(self):
        if self._free:
            return self._free.pop()
        b = next(iter(self._evictable))   # the least recently released
        del self._evictable[b]
        del self._cache[self._key_of.pop(b)]
        return b

    def _register(self, seq, idx):
        """Block ``idx`` of ``seq`` just became full: record its key, cache it if new."""
        bs = self.block_size
        parent = self._keys[seq][idx - 1] if idx > 0 else None
        key = (parent, self._salt[seq], tuple(self._toks[seq][idx * bs:(idx + 1) * bs]))
        self._keys[seq].append(key)
        b = self._tables[seq][idx]
        if key not in self._cache and b not in self._key_of:
            self._cache[key] = b
            self._key_of[b] = key

    # --- operations --------------------------------------------------------
    def add_seq_tokens(self, seq, tokens, salt=0):
        """New sequence holding ``tokens``.  Returns ``(slots, n_cached)``: the
        first ``n_cached`` tokens (whole blocks) come from cached blocks and get
        slot -1 (nothing to write); the others get the slot to write their K/V to.
        """
        if seq in self._tables:
            raise KeyError(f"sequence {seq} exists")
        bs = self.block_size
        tokens = [int(t) for t in tokens]
        hits, parent = [], None
        for i in range(len(tokens) // bs):
            key = (parent, salt, tuple(tokens[i * bs:(i + 1) * bs]))
            if key not in self._cache:
                break
            hits.append((self._cache[key], key))
            parent = key
        revived = sum(1 for b, _ in hits if b in self._evictable)
        need = -(-len(tokens) // bs) - len(hits)
        if need > self.num_free() - revived:
            raise MemoryError("block pool exhausted")
        self._tables[seq], self._lens[seq] = [], 0
        self._toks[seq], self._salt[seq], self._keys[seq] = [], salt, []
        for b, key in hits:
            self._evictable.pop(b, None)
            self._ref[b] += 1
            self._tables[seq].append(b)
            self._keys[seq].append(key)
        n_cached = len(hits) * bs
        self._toks[seq] = tokens[:n_cached]
        self._lens[seq] = n_cached
        slots, _ = self.append_tokens(seq, tokens[n_cached:])
        return [-1] * n_cached + slots, n_cached

    def append_tokens(self, seq, tokens):
        """``append`` for a sequence whose token ids are tracked: blocks that
        become full are keyed and cached."""
        if seq not in self._toks:
            raise KeyError(f"sequence {seq} has no token ids")
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        L = self._lens[seq]
        slots, pairs = self._append(seq, len(tokens))
        self._toks[seq].extend(tokens)
        for idx in range(L // bs, (L + len(tokens)) // bs):
            self._register(seq, idx)
        return slots, pairs

    def append(self, seq, n_tokens):
        """Plain append (token ids unknown): the sequence stops caching."""
        out = self._append(seq, n_tokens)
        if n_tokens > 0:
            for m in (self._toks, self._salt, self._keys):
                m.pop(seq, None)
        return out

    def _append(self, seq, n_tokens):
        if n_tokens < 0:
            raise ValueError("n_tokens must be >= 0")
        bs = self.block_size
        tbl = self._tables[seq]
        L = self._lens[seq]
        cow = (L % bs != 0) and self._ref[tbl[-1]] > 1 and n_tokens > 0
        need = -(-(L + n_tokens) // bs) - (-(-L // bs)) + (1 if cow else 0)
        if need > self.num_free():
            raise MemoryError("block pool exhausted")
        pairs = []
        if cow:
            src, dst = tbl[-1], self._take()
            self._ref[src] -= 1
            self._ref[dst] = 1
            tbl[-1] = dst
            pairs.append((src, dst))
        slots = []
        for pos in range(L, L + n_tokens):
            if pos % bs == 0:
                b = self._take()
                self._ref[b] = 1
                tbl.append(b)
            slots.append(slot_for_position(tbl, pos, bs))
        self._lens[seq] = L + n_tokens
        return slots, pairs

    def fork(self, parent, child):
        super().fork(parent, child)
        if parent in self._toks:
            self._toks[child] = list(self._toks[parent])
            self._salt[child] = self._salt[parent]
            self._keys[child] = list(self._keys[parent])

    def free_seq(self, seq):
        tbl = self._tables.pop(seq)
        del self._lens[seq]
        for m in (self._toks, self._salt, self._keys):
            m.pop(seq, None)
        for b in tbl:
            self._ref[b] -= 1
            if self._ref[b] == 0 and b not in self._key_of:
                self._free.append(b)
        for b in reversed(tbl):
            if self._ref[b] == 0 and b in self._key_of:
                self._evictable[b] = True
