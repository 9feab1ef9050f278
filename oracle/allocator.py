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
