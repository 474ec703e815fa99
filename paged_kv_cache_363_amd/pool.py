"""Python handle on the native host block pool (pkv_pool_* / pkv_seq_*).

Block tables are Python lists of ints on this side; each call marshals them
into host int32 arrays for the C library and back.
"""
import ctypes

import numpy as np

from ._lib import check, lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


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

    def seq_free(self, table):
        arr = np.ascontiguousarray(table, dtype=np.int32)
        check(lib().pkv_seq_free(self._h, _ptr(arr), len(table)))
