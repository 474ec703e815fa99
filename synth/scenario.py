"""The pool operations that put a workload in its pre-decode state.

`build_state` drives any pool object offering seq_append_slots / seq_fork
(the native pool or the plain-Python reference) through the same sequence of
calls; it computes no slot or block id itself, it only records what the pool
returns.
"""
import numpy as np


def build_state(cfg, pool, ctx):
    """Each sequence first holds ctx[s]-1 tokens (prefill), then one decode
    step appends its new token.  With cfg.shared_prefix, sequence 0 takes the
    prefix blocks and every other table is a fork of them."""
    S, P, MB = cfg.num_seqs, cfg.shared_prefix, cfg.max_blocks_per_seq
    tables, prefill = [], []
    if P:
        base = []
        slots, cows = pool.seq_append_slots(base, 0, P, MB)
        assert not cows
        prefill.append((0, 0, slots))
        forks = [base] + [pool.seq_fork(base) for _ in range(S - 1)]
    for s in range(S):
        n_pre = int(ctx[s]) - 1
        if P:
            t = forks[s]
            slots, cows = pool.seq_append_slots(t, P, n_pre - P, MB)
            prefill.append((s, P, slots))
        else:
            t = []
            slots, cows = pool.seq_append_slots(t, 0, n_pre, MB)
            prefill.append((s, 0, slots))
        assert not cows
        tables.append(t)
    step_slots, step_cows = [], []
    for s in range(S):
        slots, cows = pool.seq_append_slots(tables[s], int(ctx[s]) - 1, 1, MB)
        step_slots += slots
        step_cows += cows
    return dict(tables=tables, prefill=prefill, step_slots=np.array(step_slots, np.int64),
                step_cows=step_cows)


def table_array(cfg, tables):
    bt = np.full((len(tables), cfg.max_blocks_per_seq), -1, dtype=np.int32)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = t
    return bt


