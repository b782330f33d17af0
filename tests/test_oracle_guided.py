"""Pins of the oracle's guided encode: the acceptance rule for chunks with more
than one correct result (DeMo abstract: top-k of the DCT coefficients; the
DeToNATION notes' "Sign function" section: ternary signs before sync).

Where the k-th and (k+1)-th |X_j| lie within a rounding of each other, any of
the tied selections is a correct top-k; where a selected value lies within a
rounding of zero, either sign is correct.  The guided encode takes another
implementation's choice in exactly those cases and rejects it everywhere
else.  Chunks are built from chosen DCT coefficients with scipy's inverse
transform, and the expected q and m' come from scipy too, not from the oracle.
"""
import numpy as np
import pytest
import scipy.fft

import oracle
from oracle import DCT, RANDOM, STRIDE, Params, Shard

N = 32
NEAR = 1e-6
POS, SIGNS, REJECTED = oracle.GUIDE_POSITIONS, oracle.GUIDE_SIGNS, oracle.GUIDE_REJECTED


def _chunk_from_coefficients(X):
    """fp32 u whose orthonormal DCT-II is X up to fp32 rounding, and that DCT in fp64."""
    u = scipy.fft.idct(np.asarray(X, np.float64), type=2, norm="ortho").astype(np.float32)
    return u, scipy.fft.dct(u.astype(np.float64), type=2, norm="ortho")


def _encode(p, u_rows, guide=None, near=NEAR):
    """Encode rows u (as the gradient, m = 0, beta = 0 so u = g exactly)."""
    n = len(u_rows)
    sh = Shard(np.arange(n, dtype=np.uint64), np.full(n, N, np.int32), np.zeros((n, N), np.float32),
               np.zeros((n, N), np.float32))
    g = np.ascontiguousarray(u_rows, np.float32)
    if guide is None:
        return sh.encode(p, g) + (None,), sh.m
    return sh.encode_guided(p, g, guide[0], guide[1], near), sh.m


def _base_coefficients(seed):
    rng = np.random.default_rng(seed)
    return rng.uniform(-0.1, 0.1, N)


def test_guide_equal_to_own_choice_changes_nothing():
    rng = np.random.default_rng(1)
    u = rng.standard_normal((50, N)).astype(np.float32)
    p = Params(scheme=DCT, k=3, beta=0.0)
    (idx, val, q, X, _), m = _encode(p, u)
    (idx2, val2, q2, X2, st), m2 = _encode(p, u, (idx, val))
    assert np.all(st == 0)
    for a, b in ((idx, idx2), (val, val2), (q, q2), (X, X2), (m, m2)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("gap", [3e-7, 9e-7])
def test_near_tie_is_adopted_with_its_own_q_and_feedback(gap):
    X = _base_coefficients(2)
    X[3], X[7] = 1.0, -(1.0 - gap)
    u, Xr = _chunk_from_coefficients(X)
    assert abs(Xr[3]) > abs(Xr[7]) and abs(Xr[3]) - abs(Xr[7]) < NEAR * np.max(np.abs(Xr))
    p = Params(scheme=DCT, k=1, beta=0.0)
    (idx, val, _, _, _), _ = _encode(p, u[None])
    assert idx[0].tolist() == [3]
    (idx, val, q, _, st), m = _encode(p, u[None], ([[7]], [[-1.0]]))
    assert st[0] == POS
    assert idx[0].tolist() == [7] and val[0].tolist() == [-1.0]
    only7 = np.zeros(N)
    only7[7] = Xr[7]
    q_ref = scipy.fft.idct(only7, type=2, norm="ortho")
    assert np.max(np.abs(q[0] - q_ref)) <= 1e-15
    assert np.max(np.abs(m[0] - (u.astype(np.float64) - q_ref))) <= 1e-15


def test_guide_outside_the_tolerance_is_rejected_and_the_own_choice_kept():
    X = _base_coefficients(3)
    X[3], X[7] = 1.0, 0.5
    u, Xr = _chunk_from_coefficients(X)
    p = Params(scheme=DCT, k=1, beta=0.0)
    (idx, val, q, _, st), m = _encode(p, u[None], ([[7]], [[1.0]]))
    assert st[0] == REJECTED
    assert idx[0].tolist() == [3]
    only3 = np.zeros(N)
    only3[3] = Xr[3]
    assert np.max(np.abs(q[0] - scipy.fft.idct(only3, type=2, norm="ortho"))) <= 1e-15


def test_guide_that_leaves_out_the_largest_coefficient_is_rejected():
    """k = 2 with |X_1| = 1 and |X_5|, |X_9| tied near 0.5: {1, 9} is a valid
    top-2, {5, 9} is not (it drops the largest), although its smallest member
    is within the tolerance of the oracle's k-th largest."""
    X = _base_coefficients(4)
    X[1], X[5], X[9] = 1.0, 0.5, 0.5 - 1e-8
    u, Xr = _chunk_from_coefficients(X)
    p = Params(scheme=DCT, k=2, beta=0.0)
    (idx, _, _, _, _), _ = _encode(p, u[None])
    assert idx[0].tolist() == [1, 5]
    (idx, _, _, _, st), _ = _encode(p, u[None], ([[1, 9]], [[1.0, 1.0]]))
    assert st[0] == POS and idx[0].tolist() == [1, 9]
    (idx, _, _, _, st), _ = _encode(p, u[None], ([[5, 9]], [[1.0, 1.0]]))
    assert st[0] == REJECTED and idx[0].tolist() == [1, 5]


@pytest.mark.parametrize("guide", [[7, 7], [9, 5], [5, 32], [-1, 5]])
def test_malformed_guide_positions_are_rejected(guide):
    X = _base_coefficients(5)
    X[5], X[7], X[9] = 1.0, 1.0, 1.0  # three exact ties: any two are a valid top-2
    u, _ = _chunk_from_coefficients(X)
    p = Params(scheme=DCT, k=2, beta=0.0)
    (idx, _, _, _, st), _ = _encode(p, u[None], ([guide], [[1.0, 1.0]]))
    assert st[0] == REJECTED


def test_exact_ties_take_any_tied_subset():
    X = _base_coefficients(6)
    X[5], X[7], X[9] = 1.0, 1.0, 1.0
    u, Xr = _chunk_from_coefficients(X)
    p = Params(scheme=DCT, k=2, beta=0.0)
    for guide in ([5, 7], [5, 9], [7, 9]):
        (idx, _, _, _, st), _ = _encode(p, u[None], ([guide], [[np.sign(Xr[guide[0]]), np.sign(Xr[guide[1]])]]))
        assert idx[0].tolist() == guide and st[0] in (0, POS)


@pytest.mark.parametrize("scheme,k", [(STRIDE, 32), (RANDOM, 32)])
def test_sign_of_a_value_near_zero_is_adopted(scheme, k):
    rng = np.random.default_rng(7)
    u = rng.standard_normal(N).astype(np.float32)
    u[0] = 1.0  # the chunk's largest magnitude
    u[5] = np.float32(1e-9)
    p = Params(scheme=scheme, k=k, beta=0.0)
    (idx, val, _, _, _), _ = _encode(p, u[None])
    assert val[0][5] == 1.0
    g = val.copy()
    g[0][5] = -1.0
    (_, val2, _, _, st), _ = _encode(p, u[None], (idx, g))
    assert st[0] == SIGNS and val2[0][5] == -1.0
    g[0][5] = 0.0
    (_, val2, _, _, st), _ = _encode(p, u[None], (idx, g))
    assert st[0] == SIGNS and val2[0][5] == 0.0


def test_sign_of_a_value_away_from_zero_is_rejected():
    rng = np.random.default_rng(8)
    u = rng.standard_normal(N).astype(np.float32)
    u[6] = 0.3
    p = Params(scheme=STRIDE, k=32, beta=0.0)
    (idx, val, _, _, _), _ = _encode(p, u[None])
    g = val.copy()
    g[0][6] = -1.0
    (_, val2, _, _, st), _ = _encode(p, u[None], (idx, g))
    assert st[0] == REJECTED and val2[0][6] == 1.0
    g = val.copy()
    g[0][0] = 0.5  # not a ternary value at all
    (_, _, _, _, st), _ = _encode(p, u[None], (idx, g))
    assert st[0] == REJECTED


def test_dct_sign_near_zero_and_position_tie_in_one_chunk():
    X = _base_coefficients(9)
    X[2], X[11] = 1.0, 1.0 - 2e-7
    X[20] = 1e-10
    u, Xr = _chunk_from_coefficients(X)
    p = Params(scheme=DCT, k=32, beta=0.0)
    (idx, val, _, _, _), _ = _encode(p, u[None])
    g = val.copy()
    j = int(np.argmin(np.abs(Xr)))
    g[0][j] = -g[0][j] if g[0][j] != 0 else 1.0
    (_, val2, _, _, st), _ = _encode(p, u[None], (idx, g))
    assert st[0] == SIGNS and val2[0][j] == g[0][j]


def test_values_with_the_sign_off_are_not_guided():
    rng = np.random.default_rng(10)
    u = rng.standard_normal((4, N)).astype(np.float32)
    p = Params(scheme=DCT, k=2, beta=0.0, sign=0, value_fmt=oracle.F32)
    (idx, val, _, _, _), _ = _encode(p, u)
    (_, val2, _, _, st), _ = _encode(p, u, (idx, val * 1.5))
    assert np.all(st == 0) and np.array_equal(val, val2)


def test_status_is_per_chunk():
    X0 = _base_coefficients(11)
    X0[3], X0[7] = 1.0, 1.0 - 3e-7
    X1 = _base_coefficients(12)
    X1[3], X1[7] = 1.0, 0.4
    u0, _ = _chunk_from_coefficients(X0)
    u1, _ = _chunk_from_coefficients(X1)
    rows = np.stack([u0, u1, u0])
    p = Params(scheme=DCT, k=1, beta=0.0)
    (idx, val, _, _, _), _ = _encode(p, rows)
    gi = np.array([[7], [7], [3]], np.int32)
    (idx2, _, _, _, st), _ = _encode(p, rows, (gi, val))
    assert st.tolist() == [POS, REJECTED, 0]
    assert idx2[:, 0].tolist() == [7, 3, 3]
