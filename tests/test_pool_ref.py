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
