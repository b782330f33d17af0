"""Pins of the oracle's DCT-II against scipy and closed forms.

The transform is the orthonormal DCT-II named by the DeMo abstract ("fast
orthonormal transform (e.g., DCT)") and by Algorithm 1 of the DeToNATION notes
("DCT-II"), per 32-element chunk.
"""
import math

import numpy as np
import scipy.fft

import oracle

N = 32


def test_basis_matches_scipy_dct_of_unit_vectors():
    # column i of scipy's DCT of the identity is the transform of e_i: B[j][i]
    ref = scipy.fft.dct(np.eye(N), type=2, norm="ortho", axis=0)
    assert np.max(np.abs(oracle.basis() - ref)) < 1e-14


def test_basis_is_orthonormal():
    B = oracle.basis()
    assert np.max(np.abs(B @ B.T - np.eye(N))) < 1e-14
    assert np.max(np.abs(B.T @ B - np.eye(N))) < 1e-14


def test_dct_and_idct_match_scipy_on_random_chunks():
    rng = np.random.default_rng(1)
    for _ in range(50):
        u = rng.standard_normal(N) * rng.uniform(1e-3, 1e3)
        X = oracle.dct(u)
        assert np.max(np.abs(X - scipy.fft.dct(u, type=2, norm="ortho"))) < 1e-13 * np.max(np.abs(u)) * N
        back = oracle.idct(X)
        assert np.max(np.abs(back - scipy.fft.idct(X, type=2, norm="ortho"))) < 1e-13 * np.max(np.abs(X)) * N
        assert np.max(np.abs(back - u)) < 1e-13 * np.max(np.abs(u))


def test_parseval():
    rng = np.random.default_rng(2)
    for _ in range(20):
        u = rng.standard_normal(N)
        X = oracle.dct(u)
        assert abs(np.dot(X, X) - np.dot(u, u)) < 1e-12 * np.dot(u, u)


def test_constant_chunk_has_only_the_dc_term():
    for c in (1.0, -3.5, 1e-6):
        X = oracle.dct(np.full(N, c))
        assert abs(X[0] - c * math.sqrt(N)) < 1e-14 * abs(c) * N
        assert np.max(np.abs(X[1:])) < 1e-14 * abs(c) * N


def test_basis_row_maps_to_unit_vector():
    B = oracle.basis()
    for j in range(N):
        X = oracle.dct(B[j])
        e = np.zeros(N)
        e[j] = 1.0
        assert np.max(np.abs(X - e)) < 1e-14


def test_impulse_gives_the_basis_column_in_closed_form():
    for n0 in (0, 5, 31):
        u = np.zeros(N)
        u[n0] = 1.0
        X = oracle.dct(u)
        for j in range(N):
            s = math.sqrt(1.0 / N) if j == 0 else math.sqrt(2.0 / N)
            assert abs(X[j] - s * math.cos(math.pi * (2 * n0 + 1) * j / (2 * N))) < 1e-15
