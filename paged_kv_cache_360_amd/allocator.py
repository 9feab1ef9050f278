"""Python handle over the C++ block allocator (``pkv_alloc_*`` in the C ABI)."""

import ctypes

import numpy as np

from ._lib import PKV_ENOMEM, PagedKVError, check, lib


class BlockAllocator:
    """Refcounted block pool with per-sequence tables and copy-on-write appends.

    Methods mirror the C ABI; ``append`` returns ``(slots, cow_pairs)`` as lists.
    Out-of-blocks raises ``MemoryError`` (state unchanged); other failures raise
    ``PagedKVError``.
    """

    def __init__(self, num_blocks, block_size=16, shuffle_seed=0):
        self._h = lib().pkv_alloc_create(int(num_blocks), int(block_size), int(shuffle_seed))
        if not self._h:
            raise PagedKVError("pkv_alloc_create", -1)
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self):
        if self._h:
            lib().pkv_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _check(name, code):
        if code == PKV_ENOMEM:
            raise MemoryError(f"{name}: block pool exhausted")
        check(name, code)

    def add_seq(self, seq):
        self._check("pkv_alloc_add_seq", lib().pkv_alloc_add_seq(self._h, int(seq)))

    def fork(self, parent, child):
        self._check("pkv_alloc_fork", lib().pkv_alloc_fork(self._h, int(parent), int(child)))

    def append(self, seq, n_tokens):
        slots = np.empty(max(1, n_tokens), dtype=np.int32)
        pairs = np.empty(2, dtype=np.int32)
        ncow = ctypes.c_int32(0)
        self._check("pkv_alloc_append", lib().pkv_alloc_append(
            self._h, int(seq), int(n_tokens), slots.ctypes.data, pairs.ctypes.data,
            ctypes.addressof(ncow)))
        cow = [(int(pairs[0]), int(pairs[1]))] if ncow.value else []
        return slots[:n_tokens].tolist(), cow

    def append_batch(self, seq_ids, n_tokens, slots_out=None):
        """All-or-nothing append for distinct sequences.

        Returns (slots, pairs): int32 slots in batch order (written into
        ``slots_out`` when given, e.g. a pinned staging buffer) and an int32 [n, 2]
        array of copy-on-write pairs.
        """
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        ns = np.ascontiguousarray(n_tokens, dtype=np.int32)
        total = int(ns.sum())
        if slots_out is None:
            slots = np.empty(max(1, total), dtype=np.int32)
        else:
            slots = slots_out
            if slots.dtype != np.int32 or not slots.flags.c_contiguous or slots.size < total:
                raise ValueError("slots_out must be a contiguous int32 array of sum(n_tokens) entries")
        pairs = np.empty((max(1, len(ids)), 2), dtype=np.int32)
        ncow = ctypes.c_int32(0)
        self._check("pkv_alloc_append_batch", lib().pkv_alloc_append_batch(
            self._h, ids.ctypes.data, ns.ctypes.data, len(ids), slots.ctypes.data, max(total, slots.size),
            pairs.ctypes.data, pairs.shape[0], ctypes.addressof(ncow)))
        return slots[:total], pairs[:ncow.value]

    def free_seq(self, seq):
        self._check("pkv_alloc_free_seq", lib().pkv_alloc_free_seq(self._h, int(seq)))

    def block_table(self, seq):
        n = ctypes.c_int32(0)
        code = lib().pkv_alloc_block_table(self._h, int(seq), None, 0, ctypes.addressof(n))
        if code not in (0, -1):
            self._check("pkv_alloc_block_table", code)
        out = np.empty(max(1, n.value), dtype=np.int32)
        self._check("pkv_alloc_block_table", lib().pkv_alloc_block_table(
            self._h, int(seq), out.ctypes.data, out.shape[0], ctypes.addressof(n)))
        return out[:n.value].tolist()

    def block_tables(self, seq_ids, max_blocks, fill=-1, tables_out=None, lens_out=None):
        """Dense int32 tables [S, max_blocks] and int32 context lengths [S].

        ``tables_out`` / ``lens_out`` (contiguous int32, e.g. pinned staging
        buffers) receive the result in place when given.
        """
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tables = np.empty((len(ids), max_blocks), dtype=np.int32) if tables_out is None else tables_out
        lens = np.empty(len(ids), dtype=np.int32) if lens_out is None else lens_out
        for a, shape in ((tables, (len(ids), max_blocks)), (lens, (len(ids),))):
            if a.dtype != np.int32 or not a.flags.c_contiguous or a.shape != shape:
                raise ValueError(f"output must be a contiguous int32 array of shape {shape}")
        self._check("pkv_alloc_block_tables", lib().pkv_alloc_block_tables(
            self._h, ids.ctypes.data, len(ids), tables.ctypes.data, int(max_blocks), int(fill),
            lens.ctypes.data))
        return tables, lens

    def seq_len(self, seq):
        v = lib().pkv_alloc_seq_len(self._h, int(seq))
        if v < 0:
            self._check("pkv_alloc_seq_len", int(v))
        return int(v)

    def num_free(self):
        return int(lib().pkv_alloc_num_free(self._h))

    def refcount(self, block):
        return int(lib().pkv_alloc_refcount(self._h, int(block)))

    # --- automatic prefix caching -------------------------------------------
    def add_seq_tokens(self, seq, tokens, salt=0):
        """New sequence holding ``tokens``; returns ``(slots, n_cached)``.

        The first ``n_cached`` tokens (whole cached blocks) get slot -1: their K/V
        is in the pool already and ``pkv_write`` skips them.
        """
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        n = toks.size
        slots = np.empty(max(1, n), dtype=np.int32)
        nc = ctypes.c_int32(0)
        self._check("pkv_alloc_add_seq_tokens", lib().pkv_alloc_add_seq_tokens(
            self._h, int(seq), toks.ctypes.data if n else None, n, int(salt) & (2**64 - 1),
            slots.ctypes.data, ctypes.addressof(nc)))
        return slots[:n].tolist(), int(nc.value)

    def append_tokens(self, seq, tokens):
        """``append`` with the new tokens' ids: blocks that become full are cached."""
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        n = toks.size
        slots = np.empty(max(1, n), dtype=np.int32)
        pairs = np.empty(2, dtype=np.int32)
        ncow = ctypes.c_int32(0)
        self._check("pkv_alloc_append_tokens", lib().pkv_alloc_append_tokens(
            self._h, int(seq), toks.ctypes.data if n else None, n, slots.ctypes.data, pairs.ctypes.data,
            ctypes.addressof(ncow)))
        cow = [(int(pairs[0]), int(pairs[1]))] if ncow.value else []
        return slots[:n].tolist(), cow

    def num_cached(self):
        """Released cached blocks (count 0, reusable by a prefix hit)."""
        return int(lib().pkv_alloc_num_cached(self._h))

    # --- preemption by swapping to a host pool ----------------------------------
    def set_host_pool(self, num_host_blocks):
        self._check("pkv_alloc_set_host_pool", lib().pkv_alloc_set_host_pool(self._h, int(num_host_blocks)))
        self.num_host_blocks = int(num_host_blocks)

    def _swap(self, cname, seqs):
        ids = np.ascontiguousarray(list(seqs), dtype=np.int64)
        cap = 0
        for q in ids.tolist():          # an upper bound on the distinct blocks of the group
            cap += self._table_len(q)
        pairs = np.empty((max(1, cap), 2), dtype=np.int32)
        n = ctypes.c_int32(0)
        self._check(cname, getattr(lib(), cname)(
            self._h, ids.ctypes.data if ids.size else None, ids.size, pairs.ctypes.data, pairs.shape[0],
            ctypes.addressof(n)))
        return [(int(a), int(b)) for a, b in pairs[:n.value].tolist()]

    def _table_len(self, seq):
        n = ctypes.c_int32(0)
        swapped = lib().pkv_alloc_is_swapped(self._h, int(seq))
        fn = lib().pkv_alloc_host_table if swapped == 1 else lib().pkv_alloc_block_table
        code = fn(self._h, int(seq), None, 0, ctypes.addressof(n))
        if code not in (0, -1):
            return 0                    # unknown id: the swap call itself reports it
        return n.value

    def swap_out(self, seqs):
        """Move the sequences to host blocks; returns the (device, host) block copies."""
        return self._swap("pkv_alloc_swap_out", seqs)

    def swap_in(self, seqs):
        """Bring swapped sequences back; returns the (host, device) block copies."""
        return self._swap("pkv_alloc_swap_in", seqs)

    def is_swapped(self, seq):
        v = lib().pkv_alloc_is_swapped(self._h, int(seq))
        if v < 0:
            self._check("pkv_alloc_is_swapped", int(v))
        return bool(v)

    def host_table(self, seq):
        n = ctypes.c_int32(0)
        code = lib().pkv_alloc_host_table(self._h, int(seq), None, 0, ctypes.addressof(n))
        if code not in (0, -1):
            self._check("pkv_alloc_host_table", code)
        out = np.empty(max(1, n.value), dtype=np.int32)
        self._check("pkv_alloc_host_table", lib().pkv_alloc_host_table(
            self._h, int(seq), out.ctypes.data, out.shape[0], ctypes.addressof(n)))
        return out[:n.value].tolist()

    def num_free_host(self):
        return int(lib().pkv_alloc_num_free_host(self._h))

    def host_refcount(self, hblock):
        return int(lib().pkv_alloc_host_refcount(self._h, int(hblock)))
