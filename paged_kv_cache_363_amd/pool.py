"""Python handle on the native host block pool (pkv_pool_* / pkv_seq_*).

The per-sequence calls take block tables as Python lists of ints and marshal
them into host int32 arrays for the C library and back.  batch_append_slots
works in place on the decode layout (an int32 [num_seqs][max_blocks] array)
with one call into the library for the whole batch.
"""
import ctypes

import numpy as np

from ._lib import check, lib


def _ptr(a):
    # the address as a plain int (ctypes takes it for a void* argument);
    # ndarray.ctypes.data_as costs several microseconds per call
    return a.ctypes.data


class BlockPool:
    def __init__(self, num_blocks, block_size=16, free_order=None):
        h = ctypes.c_void_p()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("free_order must hold num_blocks ids")
        check(lib().pkv_pool_create(num_blocks, block_size,
                                    _ptr(order) if order is not None else None, ctypes.byref(h)))
        self._h = h
        self.num_blocks = num_blocks
        self.block_size = block_size
        self._ncow, self._nslots = ctypes.c_int32(), ctypes.c_int32()

    def close(self):
        if self._h:
            lib().pkv_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- single blocks -------------------------------------------------------
    def alloc(self):
        b = ctypes.c_int32()
        check(lib().pkv_pool_alloc(self._h, ctypes.byref(b)))
        return b.value

    def incref(self, b):
        check(lib().pkv_pool_incref(self._h, b))

    def decref(self, b):
        check(lib().pkv_pool_decref(self._h, b))

    def refcount(self, b):
        return int(lib().pkv_pool_refcount(self._h, b))

    def num_free(self):
        return int(lib().pkv_pool_num_free(self._h))

    def free_list(self):
        out = np.empty(max(self.num_blocks, 1), np.int32)
        n = ctypes.c_int32()
        check(lib().pkv_pool_free_list(self._h, _ptr(out), self.num_blocks, ctypes.byref(n)))
        return out[:n.value].tolist()

    # -- sequences -----------------------------------------------------------
    def seq_create(self, prompt_len, cap=None):
        cap = cap if cap is not None else -(-prompt_len // self.block_size)
        arr = np.empty(max(cap, 1), np.int32)
        n = ctypes.c_int32()
        check(lib().pkv_seq_create(self._h, prompt_len, _ptr(arr), cap, ctypes.byref(n)))
        return arr[:n.value].tolist()

    def seq_fork(self, table):
        arr = np.ascontiguousarray(table, dtype=np.int32)
        check(lib().pkv_seq_fork(self._h, _ptr(arr), len(table)))
        return list(table)

    def seq_append_slots(self, table, cur_len, n_new, cap=None):
        """Slots for positions cur_len..cur_len+n_new-1; grows `table` (a list)
        in place.  Returns (slots, cow_pairs)."""
        if cap is None:
            cap = max(len(table), -(-(cur_len + n_new) // self.block_size))
        arr = np.full(max(cap, 1), -1, np.int32)
        arr[:len(table)] = table
        nb = ctypes.c_int32(len(table))
        slots = np.empty(max(n_new, 1), np.int64)
        cow_cap = max(cap, 1)
        cows = np.empty(2 * cow_cap, np.int32)
        ncow = ctypes.c_int32()
        check(lib().pkv_seq_append_slots(self._h, _ptr(arr), ctypes.byref(nb), cap, cur_len, n_new,
                                         _ptr(slots), _ptr(cows), cow_cap, ctypes.byref(ncow)))
        table[:] = arr[:nb.value].tolist()
        pairs = [(int(cows[2 * i]), int(cows[2 * i + 1])) for i in range(ncow.value)]
        return slots[:n_new].tolist(), pairs

    def batch_append_slots(self, block_tables, nblocks, context_lens, n_new=None,
                           slot_mapping=None):
        """One step's bookkeeping for a batch (pkv_batch_append_slots).

        block_tables (int32 [S][MB]), nblocks (int32 [S]) and context_lens
        (int32 [S]) are C-contiguous numpy arrays, updated in place; n_new is
        None (one position per sequence) or int32 [S].  slot_mapping, if given,
        is an int64 array with room for every new position.  Returns
        (slot_mapping[:T], cow_pairs int32 [n][2])."""
        for a in (block_tables, nblocks, context_lens):
            if a.dtype != np.int32 or not a.flags.c_contiguous or not a.flags.writeable:
                raise ValueError("block_tables, nblocks, context_lens: writable C-contiguous int32")
        S = nblocks.shape[0]
        if block_tables.ndim != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
            raise ValueError("block_tables must be [S][MB] with nblocks, context_lens [S]")
        if n_new is not None:
            n_new = np.ascontiguousarray(n_new, dtype=np.int32)
            if n_new.shape != (S,):
                raise ValueError("n_new must be [S]")
            T = int(n_new.sum(dtype=np.int64))
        else:
            T = S
        if slot_mapping is None:
            slot_mapping = np.empty(max(T, 1), np.int64)
        elif slot_mapping.dtype != np.int64 or not slot_mapping.flags.c_contiguous \
                or slot_mapping.shape[0] < T:
            raise ValueError("slot_mapping: C-contiguous int64 with room for every position")
        cow_cap = self.num_blocks  # each copy takes a free block
        cows = np.empty(2 * max(cow_cap, 1), np.int32)
        ncow, nslots = self._ncow, self._nslots
        check(lib().pkv_batch_append_slots(
            self._h, _ptr(block_tables), block_tables.shape[1], _ptr(nblocks), _ptr(context_lens),
            _ptr(n_new) if n_new is not None else None, S, _ptr(slot_mapping), _ptr(cows),
            cow_cap, ctypes.byref(ncow), ctypes.byref(nslots)))
        return slot_mapping[:nslots.value], cows[:2 * ncow.value].reshape(-1, 2)

    # -- prefix caching --------------------------------------------------------
    def seq_create_cached(self, tokens, prompt_len, cap=None):
        """(table, cached_tokens) for a prompt of token ids, reusing its
        longest run of cached full blocks (pkv_seq_create_cached)."""
        tk = np.ascontiguousarray(tokens, dtype=np.int32)
        if tk.shape[0] < prompt_len:
            raise ValueError("fewer tokens than prompt_len")
        cap = cap if cap is not None else -(-prompt_len // self.block_size)
        arr = np.empty(max(cap, 1), np.int32)
        n, cached = ctypes.c_int32(), ctypes.c_int32()
        check(lib().pkv_seq_create_cached(self._h, _ptr(tk), prompt_len, _ptr(arr), cap,
                                          ctypes.byref(n), ctypes.byref(cached)))
        return arr[:n.value].tolist(), cached.value

    def register_blocks(self, tokens, num_tokens, table):
        tk = np.ascontiguousarray(tokens, dtype=np.int32)
        if tk.shape[0] < num_tokens:
            raise ValueError("fewer tokens than num_tokens")
        arr = np.ascontiguousarray(table, dtype=np.int32)
        check(lib().pkv_pool_register_blocks(self._h, _ptr(tk), num_tokens, _ptr(arr), len(table)))

    def cached_blocks(self):
        return int(lib().pkv_pool_cached_blocks(self._h))

    def seq_swap(self, target, table):
        """Move a sequence's blocks to pool `target` (pkv_seq_swap): returns
        (new table, [(old, new), ...]) and releases `table` here."""
        arr = np.ascontiguousarray(table, dtype=np.int32)
        n = len(table)
        out = np.empty(max(n, 1), np.int32)
        pairs = np.empty(2 * max(n, 1), np.int32)
        check(lib().pkv_seq_swap(self._h, target._h, _ptr(arr), n, _ptr(out), _ptr(pairs)))
        return out[:n].tolist(), [(int(pairs[2 * i]), int(pairs[2 * i + 1])) for i in range(n)]

    def seq_free(self, table):
        arr = np.ascontiguousarray(table, dtype=np.int32)
        check(lib().pkv_seq_free(self._h, _ptr(arr), len(table)))
