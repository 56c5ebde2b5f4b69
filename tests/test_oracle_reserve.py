"""Pins of the oracle's cache reservation ("Inside SGLang ...", Step 2: a
2 x block_size page-aligned headroom beyond the committed prefix; allocation
is not acceptance)."""
import numpy as np

from oracle.reserve import pages_needed, reserve, release


def test_pages_example():
    # the pages' Step 3 example: prefix 10, block 4 -> capacity for 18 positions
    assert pages_needed(10, 4, 16) == 2
    assert pages_needed(10, 4, 8) == 3
    assert pages_needed(0, 16, 16) == 2
    assert pages_needed(17, 16, 16) == 4          # 17 + 32 = 49 positions


def _pool(n_pages, seed):
    rng = np.random.default_rng(seed)
    return rng.permutation(n_pages), n_pages


def test_reserve_invariants_and_conservation():
    rng = np.random.default_rng(0)
    B, P, S, maxp = 7, 16, 16, 40
    stack, top = _pool(300, 1)
    pt = np.full((B, maxp), -1)
    n = np.zeros(B, np.int64)
    L = rng.integers(0, 200, B)
    for cycle in range(20):
        pt2, n2, stack2, top2, st = reserve(L, S, P, pt, n, stack, top)
        assert st == 0
        for r in range(B):
            assert n2[r] == max(n[r], pages_needed(L[r], S, P))      # covers L + 2S
            assert np.array_equal(pt2[r, :n[r]], pt[r, :n[r]])       # never moves a page
            assert n2[r] * P >= L[r] + 2 * S
        held = np.concatenate([pt2[r, :n2[r]] for r in range(B)])
        assert len(set(held.tolist())) == len(held)                  # no page twice
        assert sorted(held.tolist() + stack2[:top2].tolist()) == list(range(300))
        pt, n, stack, top = pt2, n2, stack2, top2
        L = L + rng.integers(1, S + 1, B)                            # commits of 1..S
        done = rng.random(B) < 0.1
        pt, n, stack, top = release(done, pt, n, stack, top)
        L[done] = rng.integers(0, 50, done.sum())
        assert np.all(n[done] == 0)


def test_reserve_order_and_shortage():
    stack = np.arange(10)                              # top of the stack: page 9
    pt = np.full((3, 4), -1)
    n = np.zeros(3, np.int64)
    # needs: ceil(18/16) = 2, ceil(28/16) = 2, ceil(38/16) = 3; 10 free -> 9, 8 | 7, 6 | 5, 4, 3
    pt2, n2, s2, top, st = reserve([10, 20, 30], 4, 16, pt, n, stack, 10)
    assert st == 0 and top == 3
    assert pt2[0, :2].tolist() == [9, 8] and pt2[1, :2].tolist() == [7, 6]
    assert pt2[2, :3].tolist() == [5, 4, 3]
    # a shortage stops at the first request that does not fit
    wide = np.full((3, 8), -1)                         # rows wide enough for 7 pages
    pt3, n3, s3, top3, st3 = reserve([10, 100, 5], 4, 16, wide, n, stack, 4)
    assert st3 == 1 and n3.tolist() == [2, 0, 0] and top3 == 2
    # a row too short for the reservation
    pt4, n4, s4, top4, st4 = reserve([10, 200], 4, 16, pt, n, stack, 10)
    assert st4 == 2 and n4[:2].tolist() == [2, 0]
