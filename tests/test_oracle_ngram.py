"""Pins of the oracle's prompt-lookup drafter by brute-force enumeration (CPU only)."""
import itertools

import numpy as np

import oracle
import synth


def _brute(h, min_n, max_n, k_max):
    # Enumerate every (n, j) with h[j:j+n] == suffix_n and j < N-n; pick the
    # largest n, then the largest j.
    N = len(h)
    best = None
    for n in range(min_n, max_n + 1):
        for j in range(0, N - n):
            if N >= n + 1 and h[j:j + n] == h[N - n:]:
                if best is None or (n, j) > best:
                    best = (n, j)
    if best is None:
        return []
    n, j = best
    return h[j + n:j + n + k_max]


def test_ngram_exhaustive_small_alphabet():
    for N in range(0, 9):
        for h in itertools.product(range(2), repeat=N):
            h = list(h)
            assert oracle.propose(h, 2, 4, 3) == _brute(h, 2, 4, 3), h


def test_ngram_random_histories():
    rng = np.random.default_rng(0)
    for _ in range(300):
        h = rng.integers(0, 4, size=int(rng.integers(0, 40))).tolist()
        assert oracle.propose(h, 2, 4, 8) == _brute(h, 2, 4, 8)


def test_ngram_hand_examples():
    #           0  1  2  3  4  5  6  7  8
    h = [7, 1, 2, 3, 9, 9, 1, 2, 3]
    # suffix (1,2,3) of length 3 occurred at j=1; what followed: 9, 9, 1, 2, 3
    assert oracle.propose(h, 2, 4, 8) == [9, 9, 1, 2, 3]
    assert oracle.propose(h, 2, 4, 2) == [9, 9]
    assert oracle.propose([1, 2, 3, 4], 2, 4, 8) == []
    assert oracle.propose([5, 5, 5], 2, 4, 8) == [5]     # overlapping earlier occurrence
    # The most recent occurrence wins over an older one.
    assert oracle.propose([1, 2, 8, 1, 2, 9, 1, 2], 2, 2, 8) == [9, 1, 2]


def test_ngram_proposals_are_history_continuations():
    h = synth.lookup_history(1000, 600, 42).tolist()
    hits = 0
    for cut in range(50, 600, 7):
        p = oracle.propose(h[:cut], 2, 4, 8)
        if p:
            hits += 1
            # Every proposal is what followed an earlier occurrence of a 2..4-token suffix.
            s = h[:cut]
            assert any(s[j:j + n] == s[cut - n:] and s[j + n:j + n + len(p)] == p
                       for n in range(2, 5) for j in range(cut - n))
    assert hits > 15
