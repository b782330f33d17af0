"""Pins of the oracle's per-chunk top-k ("top-k sparsification", DeMo
abstract; TopK = 4 on T5 in the DeToNATION notes' hyper-parameter section).

The selection is the k largest |X_j|; equal magnitudes go to the lower index;
slots come out in ascending index order.
"""
import itertools

import numpy as np

import oracle

N = 32


def _brute_force(X, k):
    """All k-subsets that are a valid top-k and respect the lowest-index tie rule."""
    a = np.abs(X.astype(np.float32))
    found = []
    for S in itertools.combinations(range(N), k):
        Sset = set(S)
        inside = [a[j] for j in S]
        outside = [a[i] for i in range(N) if i not in Sset]
        if min(inside) < max(outside):
            continue
        # tie rule: no excluded position of equal magnitude has a lower index
        if any(a[i] == a[j] and i < j for j in S for i in range(N) if i not in Sset):
            continue
        found.append(S)
    return found


def test_topk_matches_brute_force_on_tie_heavy_chunks():
    rng = np.random.default_rng(3)
    for k in (1, 2, 3, 4):
        for _ in range(8 if k == 4 else 20):
            X = rng.integers(-3, 4, size=N).astype(np.float64)  # many exact ties
            got = tuple(int(x) for x in oracle.topk(X, k))
            ref = _brute_force(X, k)
            assert len(ref) == 1, ref
            assert got == ref[0]


def test_topk_matches_stable_argsort():
    rng = np.random.default_rng(4)
    for _ in range(200):
        X = rng.standard_normal(N)
        if rng.random() < 0.3:
            X = np.round(X)  # ties
        for k in (1, 2, 4, 7, 16, 31, 32):
            key = -np.abs(X.astype(np.float32))
            ref = np.sort(np.argsort(key, kind="stable")[:k])
            assert np.array_equal(oracle.topk(X, k), ref)


def test_all_zero_chunk_selects_lowest_indices():
    for k in (1, 4, 32):
        assert np.array_equal(oracle.topk(np.zeros(N), k), np.arange(k))


def test_k32_selects_everything():
    X = np.random.default_rng(5).standard_normal(N)
    assert np.array_equal(oracle.topk(X, 32), np.arange(32))


def test_decision_is_taken_at_fp32():
    # two magnitudes that differ in fp64 but round to the same fp32 tie, so the
    # lower index wins
    X = np.zeros(N)
    X[3] = 1.0
    X[9] = 1.0 + 2.0 ** -40
    assert np.array_equal(oracle.topk(X, 1), [3])
    X[9] = 1.0 + 2.0 ** -20  # distinct in fp32
    assert np.array_equal(oracle.topk(X, 1), [9])
