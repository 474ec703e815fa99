"""Pins for the plain-Python reference pool against the pages' examples and
the invariants they state."""
import json
import os

import numpy as np
import pytest

from oracle.pool_ref import InvalidArg, OutOfBlocks, RefcountError, RefPool
from synth import CONFIGS, gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def check_invariants(pool, tables):
    """Every block is either free (count 0, in the queue once) or used (count =
    number of table entries naming it)."""
    uses = np.zeros(pool.num_blocks, int)
    for t in tables:
        for b in t:
            uses[b] += 1
    free = pool.free_list()
    assert len(free) == len(set(free))
    for b in range(pool.num_blocks):
        assert pool.refcount(b) == uses[b]
        assert (b in free) == (uses[b] == 0)


def test_block_counts_from_pages():
    g = _golden("block_counts.json")
    pool = RefPool(200, g["block_size"])
    for case in g["cases"]:
        t = pool.seq_create(case["tokens"])
        assert len(t) == case["blocks"]
    # the garbled 1000-token example: the reading is ceil(1000/16) = 63
    assert len(pool.seq_create(g["garbled"]["tokens"])) == g["garbled"]["reading"]


def test_p1_block_table_layout():
    """Handing the free queue the order 2,5,0,7,3,1,4,6 reproduces the pages'
    example: A (45 tokens) in [2,5,0], B (20 tokens) in [7,3], free 1,4,6."""
    g = _golden("p1_block_table.json")
    pool = RefPool(g["num_blocks"], g["block_size"], [2, 5, 0, 7, 3, 1, 4, 6])
    A = pool.seq_create(g["sequences"]["A"]["tokens"])
    B = pool.seq_create(g["sequences"]["B"]["tokens"])
    assert A == g["sequences"]["A"]["table"] and B == g["sequences"]["B"]["table"]
    assert sorted(pool.free_list()) == g["free"]
    check_invariants(pool, [A, B])
    # slot of token t = table[t // 16] * 16 + t % 16: A's last token (44)
    # sits in logical block 2 = physical block 0, offset 12
    slots, cows = pool.seq_append_slots(A, 44, 1)
    assert slots == [0 * 16 + 12] and cows == []


def test_p1_copy_on_write_beam_example():
    g = _golden("p1_cow_beam.json")
    pool = RefPool(8, 16)
    orig = pool.seq_create(40)  # 3 blocks, the last one partly filled
    b0, b1, b2 = orig
    cand1 = orig
    cand2 = pool.seq_fork(orig)
    free_before = pool.num_free()
    slots2, cows2 = pool.seq_append_slots(cand2, 40, 1)   # candidate 2 writes first
    slots1, cows1 = pool.seq_append_slots(cand1, 40, 1)   # then candidate 1
    assert len(cows2) == 1 and cows1 == []
    b3 = cows2[0][1]
    assert cows2[0][0] == b2
    names = {b0: "block_0", b1: "block_1", b2: "block_2", b3: "block_3"}
    assert [names[b] for b in cand1] == g["candidate_1"]
    assert [names[b] for b in cand2] == g["candidate_2"]
    assert free_before - pool.num_free() == g["new_blocks"]
    assert [pool.refcount(b) for b in (b0, b1, b2, b3)] == [2, 2, 1, 1]
    assert slots2 == [b3 * 16 + 8] and slots1 == [b2 * 16 + 8]
    check_invariants(pool, [cand1, cand2])


def test_new_block_every_16_tokens_and_only_last_partial():
    pool = RefPool(64, 16)
    t = []
    for n in range(1, 200):
        before = len(t)
        pool.seq_append_slots(t, n - 1, 1)
        assert len(t) == -(-n // 16)
        assert (len(t) > before) == ((n - 1) % 16 == 0)


def test_utilization_above_96_percent_on_decode_mix():
    """Only the last block of a sequence is partly filled, so used/allocated
    stays above 96% for realistic context mixes ("Transformer 推理优化",
    section 3.4)."""
    for name in ("c2_qwen3_8b_bf16", "c3_llama2_7b_f16"):
        ctx = gen.context_lens(CONFIGS[name])
        alloc = sum(-(-int(n) // 16) * 16 for n in ctx)
        assert ctx.sum() / alloc > 0.96
        assert all(-(-int(n) // 16) * 16 - n < 16 for n in ctx)


def test_free_returns_blocks_fifo_and_counts():
    pool = RefPool(6, 16)
    a = pool.seq_create(33)  # blocks 0,1,2
    b = pool.seq_fork(a)
    pool.seq_free(a)
    assert pool.num_free() == 3 and [pool.refcount(x) for x in b] == [1, 1, 1]
    pool.seq_free(b)
    assert pool.free_list() == [3, 4, 5, 2, 1, 0]  # freed last block first, to the tail
    check_invariants(pool, [])


def test_errors_change_nothing():
    pool = RefPool(4, 16)
    t = pool.seq_create(40)  # 3 blocks
    snap = (pool.free_list(), list(pool.ref), list(t))
    with pytest.raises(OutOfBlocks):
        pool.seq_append_slots(t, 40, 30)  # needs 2 more, 1 free
    assert (pool.free_list(), list(pool.ref), list(t)) == snap
    with pytest.raises(InvalidArg):
        pool.seq_append_slots(t, 80, 1)   # leaves a gap
    with pytest.raises(InvalidArg):
        pool.seq_append_slots(t, 40, 10, cap=3)
    with pytest.raises(RefcountError):
        pool.decref(pool.free_list()[0])
    with pytest.raises(InvalidArg):
        pool.incref(99)
    assert (pool.free_list(), list(pool.ref), list(t)) == snap


def test_random_operations_keep_invariants():
    rs = np.random.default_rng(40)
    pool = RefPool(96, 16, rs.permutation(96))
    seqs = []  # (table, length)
    for _ in range(3000):
        op = rs.integers(0, 4)
        try:
            if op == 0 or not seqs:
                n0 = int(rs.integers(0, 60))
                seqs.append([pool.seq_create(n0), n0])
            elif op == 1:
                i = int(rs.integers(len(seqs)))
                seqs.append([pool.seq_fork(seqs[i][0]), seqs[i][1]])
            elif op == 2:
                i = int(rs.integers(len(seqs)))
                t, n = seqs[i]
                k = int(rs.integers(1, 20))
                pool.seq_append_slots(t, n, k)
                seqs[i][1] = n + k
            else:
                i = int(rs.integers(len(seqs)))
                pool.seq_free(seqs.pop(i)[0])
        except OutOfBlocks:
            pass
        check_invariants(pool, [s[0] for s in seqs])


# -- prefix caching ----------------------------------------------------------

def _prompt(rs, n, vocab=1000):
    return [int(x) for x in rs.integers(0, vocab, n)]


def test_same_prefix_reuses_computed_blocks():
    # a request that shares the first 40 tokens of another reuses its two full
    # blocks ("KV Cache 与 PageAttention深度实战" 4.2); the partial block is new
    rs = np.random.default_rng(1)
    p = RefPool(16, 16)
    a_tok = _prompt(rs, 50)
    a, cached = p.seq_create_cached(a_tok, 50)
    assert cached == 0 and len(a) == 4
    p.register_blocks(a_tok, 50, a)            # 3 full blocks become findable
    assert p.cached_blocks() == 3
    b_tok = a_tok[:40] + _prompt(rs, 5)
    b, cached = p.seq_create_cached(b_tok, 45)
    assert cached == 32 and b[:2] == a[:2] and b[2] not in a
    assert [p.refcount(x) for x in a[:2]] == [2, 2] and p.refcount(a[2]) == 1


def test_freed_blocks_stay_cached_until_evicted_lru():
    rs = np.random.default_rng(2)
    p = RefPool(8, 16)
    t1 = _prompt(rs, 32)
    t2 = _prompt(rs, 32)
    a, _ = p.seq_create_cached(t1, 32)          # [0, 1]
    p.register_blocks(t1, 32, a)
    b, _ = p.seq_create_cached(t2, 32)          # [2, 3]
    p.register_blocks(t2, 32, b)
    p.seq_free(a)                               # freed last block first
    p.seq_free(b)
    assert p.cached_blocks() == 4
    assert p.free_list() == [4, 5, 6, 7, 1, 0, 3, 2]
    # a hit on a free block takes it out of the queue (count 1 again)
    c, cached = p.seq_create_cached(t2, 32)
    assert cached == 32 and c == b and p.num_free() == 6
    p.seq_free(c)
    # handing out 6 blocks evicts a's blocks (least recently freed) and keeps b's
    fresh = [p.alloc() for _ in range(6)]
    assert fresh == [4, 5, 6, 7, 1, 0] and p.cached_blocks() == 2
    for x in fresh:
        p.decref(x)                             # queue: [3, 2, 4, 5, 6, 7, 1, 0]
    _, cached = p.seq_create_cached(t2, 32)     # b's blocks are still cached
    assert cached == 32
    _, cached = p.seq_create_cached(t1, 32)     # a's were evicted
    assert cached == 0


def test_a_reused_parent_never_matches_its_old_children():
    rs = np.random.default_rng(3)
    p = RefPool(4, 16)
    t = _prompt(rs, 32)
    a, _ = p.seq_create_cached(t, 32)           # [0, 1]
    p.register_blocks(t, 32, a)
    p.decref(a[0])                              # the parent alone goes back
    fresh = [p.alloc(), p.alloc()]              # 2, 3
    y = p.alloc()                               # 0: evicted and handed out again
    assert y == a[0] and p.cached_blocks() == 1  # the child's key is still there
    other = _prompt(rs, 16)
    p.register_blocks(other, 16, [y])
    for x in fresh:
        p.decref(x)
    # other + t's second block: the child was registered under y's old
    # generation, so only the first block matches
    table, cached = p.seq_create_cached(other + t[16:32], 32)
    assert cached == 16 and table[0] == y and table[1] != a[1]


def test_partial_blocks_are_never_cached_and_errors_change_nothing():
    rs = np.random.default_rng(4)
    p = RefPool(4, 16)
    t = _prompt(rs, 40)
    a, _ = p.seq_create_cached(t, 40)
    p.register_blocks(t, 40, a)
    assert p.cached_blocks() == 2              # the 8-token block is not
    before = (p.free_list(), list(p.ref), dict(p.cache))
    with pytest.raises(OutOfBlocks):
        p.seq_create_cached(t[:32] + _prompt(rs, 40), 72)
    with pytest.raises(InvalidArg):
        p.register_blocks(_prompt(rs, 32), 32, a)   # a holds another prefix
    assert (p.free_list(), list(p.ref), dict(p.cache)) == before
