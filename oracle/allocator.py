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

Preemption by swapping ("vLLM and PagedAttention", §3 continuous batching, on
the scheduler's preemption: under memory pressure the KV of some requests moves
to CPU memory and comes back once memory frees up; "How vLLM Works?", section
04 on preemption, recompute being the other mode): a second pool of host blocks; a
swap-out moves whole sequences there, a swap-in brings them back.  Readings
where the pages are silent: a block held several times within one swap-out
group gets one host block (and one device block on the way back), so sharing
inside the group survives the round trip; a device block also held by a
sequence that stays on the device is copied and stays where it is; host blocks
are handed out lowest id first and reused last-freed first; a swapped sequence
can only be swapped in or freed.  Recompute mode needs no new operation: the
sequence is freed and later added again with its tokens.

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
        self._hfree = []                  # host blocks, pop() hands out the lowest first
        self._href = []
        self._swapped = {}                # seq -> table of host block ids

    # --- queries -----------------------------------------------------------
    def num_free(self):
        return len(self._free)

    def num_free_host(self):
        return len(self._hfree)

    def host_refcount(self, hblock):
        return self._href[hblock]

    def host_table(self, seq):
        return list(self._swapped[seq])

    def is_swapped(self, seq):
        if seq not in self._tables and seq not in self._swapped:
            raise KeyError(f"unknown sequence {seq}")
        return seq in self._swapped

    def refcount(self, block):
        return self._ref[block]

    def block_table(self, seq):
        return list(self._tables[seq])

    def seq_len(self, seq):
        return self._lens[seq]

    def seqs(self):
        return list(self._tables)

    # --- operations --------------------------------------------------------
    def _exists(self, seq):
        return seq in self._tables or seq in self._swapped

    def add_seq(self, seq):
        if self._exists(seq):
            raise KeyError(f"sequence {seq} exists")
        self._tables[seq] = []
        self._lens[seq] = 0

    def fork(self, parent, child):
        """Child shares every block of the parent (counts +1); same length."""
        if self._exists(child):
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
            dst = self._take()
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

    def free_seq(self, seq):
        """Drop a sequence; blocks whose count reaches 0 return to the free list
        (host blocks to the host free list for a swapped sequence)."""
        if seq in self._swapped:
            self._drop_host(self._swapped.pop(seq))
            del self._lens[seq]
            return
        tbl = self._tables.pop(seq)
        del self._lens[seq]
        self._release(tbl)

    # --- swapping to a host pool ---------------------------------------------
    def set_host_pool(self, num_host_blocks):
        """A host pool of ``num_host_blocks`` blocks (no sequence may be swapped out)."""
        if num_host_blocks < 0:
            raise ValueError("num_host_blocks must be >= 0")
        if self._swapped:
            raise ValueError("sequences are swapped out")
        self._hfree = list(range(num_host_blocks))[::-1]
        self._href = [0] * num_host_blocks

    def swap_out(self, seqs):
        """Move the sequences ``seqs`` (distinct, on the device) to host blocks.

        Returns the ``(device block, host block)`` copies, one per distinct device
        block in order of first appearance (sequences in the given order, each
        table in order).  The caller copies them before the device blocks are
        reused.
        """
        seqs = self._group(seqs, swapped=False)
        distinct = list(dict.fromkeys(b for q in seqs for b in self._tables[q]))
        if len(distinct) > len(self._hfree):
            raise MemoryError("host pool exhausted")
        to_host = {b: self._hfree.pop() for b in distinct}
        for q in seqs:
            tbl = self._tables.pop(q)
            htbl = [to_host[b] for b in tbl]
            for h in htbl:
                self._href[h] += 1
            self._swapped[q] = htbl
            self._release(tbl)
        return [(b, to_host[b]) for b in distinct]

    def swap_in(self, seqs):
        """Bring swapped sequences back to new device blocks.

        Returns the ``(host block, device block)`` copies, one per distinct host
        block in order of first appearance.
        """
        seqs = self._group(seqs, swapped=True)
        distinct = list(dict.fromkeys(h for q in seqs for h in self._swapped[q]))
        if len(distinct) > self.num_free():
            raise MemoryError("block pool exhausted")
        to_dev = {h: self._take() for h in distinct}
        for q in seqs:
            htbl = self._swapped.pop(q)
            tbl = [to_dev[h] for h in htbl]
            for b in tbl:
                self._ref[b] += 1
            self._tables[q] = tbl
            self._drop_host(htbl)
        return [(h, to_dev[h]) for h in distinct]

    # --- internals -----------------------------------------------------------
    def _take(self):
        return self._free.pop()

    def _release(self, tbl):
        """Drop one reference per table entry; blocks at 0 return to the free list."""
        for b in tbl:
            self._ref[b] -= 1
            if self._ref[b] == 0:
                self._free.append(b)

    def _drop_host(self, htbl):
        for h in htbl:
            self._href[h] -= 1
            if self._href[h] == 0:
                self._hfree.append(h)

    def _group(self, seqs, swapped):
        seqs = list(seqs)
        if len(set(seqs)) != len(seqs):
            raise ValueError("sequence ids must be distinct")
        for q in seqs:
            if q not in self._tables and q not in self._swapped:
                raise KeyError(f"unknown sequence {q}")
            if (q in self._swapped) != swapped:
                raise ValueError(f"sequence {q} is {'not ' if swapped else ''}swapped out")
        return seqs


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
        if self._exists(seq):
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
        super().free_seq(seq)
        for m in (self._toks, self._salt, self._keys):
            m.pop(seq, None)

    def _release(self, tbl):
        """Uncached blocks at count 0 go back to the free list in table order,
        cached ones to the released list from the last to the first."""
        for b in tbl:
            self._ref[b] -= 1
            if self._ref[b] == 0 and b not in self._key_of:
                self._free.append(b)
        for b in reversed(tbl):
            if self._ref[b] == 0 and b in self._key_of:
                self._evictable[b] = True
