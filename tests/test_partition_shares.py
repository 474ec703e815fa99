"""The share arithmetic of fixed partitions on the persistent grid, modelled
on the host: the decode kernel splits the step's units (per segment of a
sequence with nbk blocks, R restart units and then one unit per block) into
equal contiguous shares of W waves and moves both ends of every share up to
the next partition boundary of its segment (or the segment's end).  Every
partition of every segment must then be closed by exactly one wave, and a
wave's partitions must be whole, whatever the lengths (empty sequences,
lengths that are not block multiples), the grid size and the partition size.

The model follows the kernel's integer steps: the share of wave k is
[floor(U k / We), floor(U (k+1) / We)) with We = min(U, W); a unit u belongs
to the last sequence s whose first unit Y * pref[s] is <= u; segments follow
each other in (sequence, kv-head chunk) order."""
import numpy as np
import pytest


def closed_partitions(ctx, Y, R, P, W):
    nbk = [(c + 15) // 16 for c in ctx]
    lens = [n + R if n > 0 else 0 for n in nbk]
    pref = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    S = len(ctx)
    U = int(Y * pref[S])
    We = min(U, W)
    seen = []
    for wk in range(We):
        u_lo, u_hi = U * wk // We, U * (wk + 1) // We
        if u_hi == u_lo:
            continue
        # locate(u_lo)
        s = max(i for i in range(S) if Y * pref[i] <= u_lo)
        length = int(pref[s + 1] - pref[s])
        r = u_lo - Y * int(pref[s])
        y, j = r // length, r % length
        u = u_lo
        while True:
            length = int(pref[s + 1] - pref[s])
            seg_start = Y * int(pref[s]) + y * length
            pe = min(seg_start + length, u_hi)
            n = length - R
            b = max(j - R, 0)
            b1 = max(pe - seg_start - R, 0)
            b = min(-(-b // P) * P, n)
            b1 = min(-(-b1 // P) * P, n)
            if b1 > b:
                assert b % P == 0 and (b1 % P == 0 or b1 == n)
                for kp in range(b // P, -(-b1 // P)):
                    seen.append((s, y, kp, wk))
            u = pe
            if u >= u_hi:
                break
            j = 0
            y += 1
            if y == Y:
                y = 0
                s += 1
                while pref[s + 1] == pref[s]:
                    s += 1
    return seen, nbk


def check(ctx, Y, R, P, W):
    seen, nbk = closed_partitions(ctx, Y, R, P, W)
    keys = [(s, y, kp) for s, y, kp, _ in seen]
    assert len(keys) == len(set(keys)), "a partition closed twice"
    want = {(s, y, kp) for s, n in enumerate(nbk) for y in range(Y)
            for kp in range(-(-n // P))}
    assert set(keys) == want


@pytest.mark.parametrize("W", [4, 12, 148, 1024, 8192])
@pytest.mark.parametrize("P", [1, 2, 32, 128])
def test_every_partition_closed_once_ragged(W, P):
    rs = np.random.default_rng(7 * W + P)
    ctx = list(rs.integers(0, 4097, 40))
    ctx[3] = 0
    ctx[-1] = 0
    check(ctx, Y=8, R=4, P=P, W=W)


@pytest.mark.parametrize("W", [1, 4, 1024])
def test_every_partition_closed_once_long_uniform(W):
    # the 32K shared-prefix workload's shape, 512-token partitions
    check([32768] * 16, Y=8, R=4, P=32, W=W)


def test_more_waves_than_units():
    check([1, 17, 0, 33], Y=2, R=3, P=1, W=4096)
    check([5], Y=1, R=0, P=4, W=64)
