"""Plain-Python reference of the host block bookkeeping (block pool).

TEST INFRASTRUCTURE ONLY: used by tests/ to check the native pool bit for bit;
the product never imports it.

What it models, from the pages:
  - KV memory is cut into fixed blocks of 16 tokens; a per-sequence block table
    maps logical block j to any physical block ("Transformer 推理优化：KV Cache、
    PagedAttention 与 vLLM", sections 3.2-3.3).
  - Blocks are taken on demand, a new one each time 16 more tokens have been
    produced ("vLLM推理引擎深度解析", section 2.2), so only the last block of a
    sequence is partly filled (same page as above, section 3.4).
  - A pool hands out and takes back blocks in O(1) ("大语言模型推理引擎深度剖析",
    section 2.2); free blocks sit in a queue ("vLLM推理引擎深度解析", section 2.2).
  - Sharing and copy-on-write: several tables may point at one physical block;
    a reference count is kept and a block returns to the free pool when it
    reaches zero; a shared block is copied before a sequence writes into it
    ("大语言模型推理引擎深度剖析", section 2.3; "Transformer 推理优化", section 3.5).

Readings where the pages leave a choice:
  - the free queue is FIFO, initially in the order given (default 0..N-1);
    a block whose count drops to zero goes to its tail;
  - a sequence is freed from its last block to its first;
  - a write into an existing block whose count is above one copies it first
    (copy-on-write), whether or not the block is full;
  - an append that cannot get every block it needs fails and changes nothing;
  - a batch append (one decode step's bookkeeping for many sequences) is the
    single-sequence append applied to each sequence in batch order, and it
    too either succeeds for every sequence or changes nothing;
  - prefix caching ("vLLM推理引擎深度解析" sections 2.2 and 4.1; "KV Cache 与
    PageAttention深度实战" section 4.2: computed prefix blocks are kept in an
    LRU cache and a request with the same prefix reuses them).  Reading: a
    full block is known by the exact key (parent block, the parent's
    allocation generation, its own token ids), the root's parent being -1;
    a block's generation grows each time it is handed out, so a chain whose
    parent was reused never matches.  The caller registers blocks once their
    K/V are computed.  A freed block keeps its key and joins the tail of the
    free queue; allocation takes the head, which drops the key (eviction of
    the least recently freed block).  A lookup matches full blocks from the
    start and stops at the first miss; a hit on a free block takes it out of
    the queue;
  - swapping a sequence to another pool (device blocks to host memory and
    back, "大语言模型推理引擎深度剖析" section 3.3) takes one block of the
    target pool per block of the table, in table order, then releases the
    table in the source pool as a free does; it needs every target block or
    changes nothing.
"""
import copy
from collections import deque


class PoolError(Exception):
    pass


class OutOfBlocks(PoolError):
    pass


class RefcountError(PoolError):
    pass


class InvalidArg(PoolError):
    pass


class RefPool:
    def __init__(self, num_blocks, block_size=16, free_order=None):
        if num_blocks < 0 or block_size <= 0:
            raise InvalidArg("bad pool size")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArg("free_order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.gen = [0] * num_blocks      # times each block was handed out
        self.key = [None] * num_blocks   # prefix-cache key of a registered block
        self.cache = {}                  # key -> block

    # -- single blocks -------------------------------------------------------
    def _check(self, b):
        if not (0 <= b < self.num_blocks):
            raise InvalidArg(f"block id {b} out of range")

    def alloc(self):
        if not self.free:
            raise OutOfBlocks("no free block")
        b = self.free.popleft()
        if self.key[b] is not None:      # evict the least recently freed
            del self.cache[self.key[b]]
            self.key[b] = None
        self.gen[b] += 1
        self.ref[b] = 1
        return b

    def incref(self, b):
        self._check(b)
        if self.ref[b] < 1:
            raise RefcountError(f"incref of free block {b}")
        self.ref[b] += 1

    def decref(self, b):
        self._check(b)
        if self.ref[b] < 1:
            raise RefcountError(f"decref of free block {b}")
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    def refcount(self, b):
        self._check(b)
        return self.ref[b]

    def num_free(self):
        return len(self.free)

    def free_list(self):
        return list(self.free)

    # -- sequences -----------------------------------------------------------
    def blocks_for(self, n_tokens):
        """Blocks needed to hold n tokens: ceil(n / block_size)."""
        return -(-n_tokens // self.block_size)

    def seq_create(self, prompt_len, cap=None):
        table = []
        self.seq_append_slots(table, 0, prompt_len, cap)
        return table

    def seq_fork(self, table):
        for b in table:
            self._check(b)
            if self.ref[b] < 1:
                raise RefcountError(f"fork of free block {b}")
        for b in table:
            self.ref[b] += 1
        return list(table)

    def seq_append_slots(self, table, cur_len, n_new, cap=None):
        """Slots for positions cur_len .. cur_len+n_new-1, growing `table`
        in place.  Returns (slots, cow_pairs) where each cow pair (src, dst)
        asks the caller to copy physical block src into dst."""
        bs = self.block_size
        if cur_len < 0 or n_new < 0:
            raise InvalidArg("negative length")
        if n_new == 0:
            return [], []
        first, last = cur_len // bs, (cur_len + n_new - 1) // bs
        if first > len(table):
            raise InvalidArg("positions leave a gap after the table")
        if cap is not None and last + 1 > cap:
            raise InvalidArg("table capacity exceeded")
        needed = 0
        for bi in range(first, last + 1):
            if bi >= len(table) or self.ref[table[bi]] > 1:
                needed += 1
        if needed > len(self.free):
            raise OutOfBlocks(f"need {needed} blocks, {len(self.free)} free")
        cows = []
        for bi in range(first, last + 1):
            if bi < len(table):
                old = table[bi]
                if self.ref[old] > 1:
                    new = self.alloc()
                    cows.append((old, new))
                    self.decref(old)
                    table[bi] = new
            else:
                table.append(self.alloc())
        slots = [table[p // bs] * bs + p % bs for p in range(cur_len, cur_len + n_new)]
        return slots, cows

    def batch_append_slots(self, tables, lens, n_new, cap=None):
        """One step's bookkeeping for a batch: sequence s, whose table is
        tables[s] and whose length is lens[s], gets n_new[s] positions, in
        order s = 0, 1, ...  tables and lens are updated in place.  Returns
        (slots, cow_pairs): the slots of every new position, sequence by
        sequence, and the copies in the order they were made.  On any error
        the pool, the tables and the lengths are as before."""
        saved = (copy.deepcopy(tables), list(lens), deque(self.free), list(self.ref))
        slots, cows = [], []
        try:
            for s in range(len(tables)):
                sl, cw = self.seq_append_slots(tables[s], lens[s], n_new[s], cap)
                slots += sl
                cows += cw
                lens[s] += n_new[s]
        except PoolError:
            for s in range(len(tables)):
                tables[s][:] = saved[0][s]
            lens[:] = saved[1]
            self.free, self.ref = saved[2], saved[3]
            raise
        return slots, cows

    # -- prefix caching --------------------------------------------------------
    def _block_keys(self, tokens, n_full):
        """Walk the cache along the prompt: the blocks hit, stopping at the
        first full block not cached."""
        bs = self.block_size
        hits, parent = [], (-1, 0)
        for i in range(n_full):
            b = self.cache.get(parent + (tuple(tokens[i * bs:(i + 1) * bs]),))
            if b is None:
                break
            hits.append(b)
            parent = (b, self.gen[b])
        return hits

    def seq_create_cached(self, tokens, prompt_len, cap=None):
        """A table for a prompt of token ids: its longest cached run of full
        blocks is reused (one more reference each), the rest is new.
        Returns (table, cached_tokens)."""
        bs = self.block_size
        if prompt_len < 0 or len(tokens) < prompt_len:
            raise InvalidArg("prompt_len")
        need = -(-prompt_len // bs)
        if cap is not None and need > cap:
            raise InvalidArg("table capacity exceeded")
        hits = self._block_keys(tokens, prompt_len // bs)
        revived = sum(1 for b in hits if self.ref[b] == 0)
        if need - len(hits) > len(self.free) - revived:
            raise OutOfBlocks("not enough free blocks")
        for b in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
        table = hits + [self.alloc() for _ in range(need - len(hits))]
        return table, len(hits) * bs

    def register_blocks(self, tokens, num_tokens, table):
        """Declare the full blocks among the first num_tokens of a sequence
        computed: each becomes findable by its key unless another block
        already holds that key."""
        bs = self.block_size
        n_full = num_tokens // bs
        if n_full > len(table) or len(tokens) < num_tokens:
            raise InvalidArg("table or tokens too short")
        for b in table[:n_full]:
            self._check(b)
            if self.ref[b] < 1:
                raise RefcountError(f"register of free block {b}")
        keys, parent = [], (-1, 0)
        for i in range(n_full):
            b = table[i]
            k = parent + (tuple(tokens[i * bs:(i + 1) * bs]),)
            if self.key[b] is not None and self.key[b] != k:
                raise InvalidArg(f"block {b} holds another prefix")
            keys.append(k)
            parent = (b, self.gen[b])
        for b, k in zip(table[:n_full], keys):
            if self.key[b] is None and k not in self.cache:
                self.cache[k] = b
                self.key[b] = k

    def cached_blocks(self):
        return len(self.cache)

    def seq_swap(self, target, table):
        """Move a sequence's blocks to `target` (another pool, e.g. host
        memory): returns (new table, [(old block, new block), ...]) for the
        caller to copy, and releases the table here."""
        for b in table:
            self._check(b)
            if self.ref[b] < 1:
                raise RefcountError(f"swap of free block {b}")
        if target.block_size != self.block_size:
            raise InvalidArg("block sizes differ")
        if len(target.free) < len(table):
            raise OutOfBlocks(f"need {len(table)} blocks, {len(target.free)} free")
        new = [target.alloc() for _ in table]
        self.seq_free(table)
        return new, list(zip(table, new))

    def seq_free(self, table):
        for b in table:
            self._check(b)
            if self.ref[b] < 1:
                raise RefcountError(f"free of free block {b}")
        for b in reversed(table):
            self.decref(b)
