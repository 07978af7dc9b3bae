"""Pins of the page-allocation oracle (CPU only).

  * A1 a hand-worked step (page size 4): values written out below from the
    rule, not from the oracle.
  * A2 invariants on random steps: every new token gets a distinct slot, the
    pages taken are the tail of the free list and distinct, each row ends
    with ceil((P+E)/ps) pages, and reading a row through the page table
    (the attention's address translation) returns the old slots followed by
    out_loc -- the new tokens land where the attention will look for them.
  * A3 a step that needs more pages than are free changes nothing.
"""

import numpy as np
import pytest

import oracle


def test_a1_hand_example():
    # free pages 10..15 (6 free); page size 4; three requests:
    #   r0 (row 2): P 0, E 5  -> needs pages for positions 0..4: 2 pages
    #   r1 (row 0): P 3, E 2  -> holds page 7 (positions 0..3); position 4
    #                            needs a second page
    #   r2 (row 1): P 8, E 0  -> nothing
    # pages leave from the tail: 15, 14 to r0, then 13 to r1
    free = np.array([10, 11, 12, 13, 14, 15], np.int32)
    pt = np.full((3, 4), -1, np.int32)
    pt[0, 0] = 7
    pt[1, :2] = [3, 4]
    ok, nf, pt2, loc = oracle.alloc_pages(free, 6, pt, [2, 0, 1], [0, 3, 8], [5, 2, 0], 4)
    assert ok and nf == 3
    assert pt2[2].tolist() == [15, 14, -1, -1]
    assert pt2[0].tolist() == [7, 13, -1, -1]
    assert pt2[1].tolist() == [3, 4, -1, -1]
    # r0: page 15 slots 60..63, then page 14 slot 56; r1: page 7 slot 31, page 13 slot 52
    assert loc.tolist() == [60, 61, 62, 63, 56, 31, 52]


@pytest.mark.parametrize("seed,ps", [(1, 16), (2, 1), (3, 7)])
def test_a2_random_step_invariants(seed, ps):
    rng = np.random.default_rng(seed)
    B = 40
    P = rng.integers(0, 600, B)
    E = rng.integers(0, 300, B)
    E[:3] = [0, 1, 4096 // 16]
    width = int(max(-(-(P + E) // ps))) + 3
    npages = int(sum(-(-(P + E) // ps))) + 50
    rows = rng.permutation(B + 5)[:B].astype(np.int32)
    perm = rng.permutation(npages).astype(np.int32)
    pt = np.full((B + 5, width), -1, np.int32)
    used = 0
    for r in range(B):  # the pages each request already holds
        h = -(-int(P[r]) // ps)
        pt[rows[r], :h] = perm[used:used + h]
        used += h
    free = perm[used:]
    nf = len(free)
    ok, nf2, pt2, loc = oracle.alloc_pages(free, nf, pt, rows, P, E, ps)
    assert ok
    need = -(-(P + E) // ps) - (-(-P // ps))
    taken = free[nf - int(need.sum()):][::-1]
    assert nf2 == nf - int(need.sum())
    assert len(np.unique(loc)) == len(loc) == int(E.sum())
    k = 0
    t = 0
    for r in range(B):
        row = pt2[rows[r]]
        h = -(-int(P[r]) // ps)
        n = -(-int(P[r] + E[r]) // ps)
        assert np.array_equal(row[:h], pt[rows[r], :h])
        assert np.array_equal(row[h:n], taken[k:k + n - h])
        assert np.all(row[n:] == -1)
        k += n - h
        slots = oracle.token_slots(row, int(P[r] + E[r]), ps)
        old = oracle.token_slots(pt[rows[r]], int(P[r]), ps) if P[r] > 0 else np.zeros(0)
        assert np.array_equal(slots[:P[r]], old)
        assert np.array_equal(slots[P[r]:], loc[t:t + E[r]])
        t += int(E[r])


def test_a3_impossible_steps_change_nothing():
    free = np.array([5, 6], np.int32)
    pt = np.full((2, 8), -1, np.int32)
    for rows, P, E in (([0, 1], [0, 0], [9, 1]),    # 4 pages needed, 2 free
                       ([0, 1], [0, 0], [33, 0]),   # 9 entries > 8 in the row
                       ([0, 1], [0, 0], [1, -1]),   # negative length
                       ([0, 2], [0, 0], [1, 1])):   # row 2 outside the table
        ok, nf, pt2, loc = oracle.alloc_pages(free, 2, pt, rows, P, E, 4)
        assert not ok and nf == 2 and np.array_equal(pt2, pt)
