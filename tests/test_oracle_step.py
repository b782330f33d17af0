"""Pins of the oracle's encode (Algorithm 1 steps 3-5) and decode (steps 6-7)
of the DeToNATION notes, against library routines, invariants and closed forms.
"""
import numpy as np
import pytest
import scipy.fft

import oracle
from oracle import DCT, DILOCO, RANDOM, STRIDE, Params, Shard

N = 32


def _shard(n_elems, seed=0, m_std=1.0, theta_std=0.02):
    rng = np.random.default_rng(seed)
    m0 = (rng.standard_normal(n_elems) * m_std).astype(np.float32)
    th0 = (rng.standard_normal(n_elems) * theta_std).astype(np.float32)
    return Shard.contiguous(n_elems, m0, th0), m0, th0


def _grad(n_elems, seed=1):
    return np.random.default_rng(seed).standard_normal(n_elems).astype(np.float32)


def _u_ref(m0, g, beta, n_elems):
    # u = beta*m + g with beta the fp32 configuration value
    u = np.float64(np.float32(beta)) * m0.astype(np.float64) + g.astype(np.float64)
    C = (n_elems + N - 1) // N
    out = np.zeros(C * N, np.float64)
    out[:n_elems] = u
    return out.reshape(C, N)


@pytest.mark.parametrize("k", [1, 2, 4, 7, 32])
def test_dct_encode_matches_scipy_pipeline(k):
    L = 32 * 40
    sh, m0, _ = _shard(L)
    g = _grad(L)
    p = Params(scheme=DCT, k=k, beta=0.9)
    idx, val, q, X = sh.encode(p, oracle.pad_chunks(g, L))
    u = _u_ref(m0, g, 0.9, L)
    Xref = scipy.fft.dct(u, type=2, norm="ortho", axis=1)
    assert np.max(np.abs(X - Xref)) < 1e-13
    for c in range(L // N):
        sel = np.sort(np.argsort(-np.abs(Xref[c].astype(np.float32)), kind="stable")[:k])
        assert np.array_equal(idx[c], sel)
        assert np.array_equal(val[c], np.sign(Xref[c][sel]))
        Xs = np.zeros(N)
        Xs[sel] = Xref[c][sel]
        qref = scipy.fft.idct(Xs, type=2, norm="ortho")
        assert np.max(np.abs(q[c] - qref)) < 1e-13
        assert np.max(np.abs(sh.m[c] - (u[c] - qref))) < 1e-13


def test_feedback_invariant_u_equals_m_plus_q():
    L = 32 * 64
    sh, m0, _ = _shard(L, seed=7)
    g = _grad(L, seed=8)
    for scheme, k in ((DCT, 3), (RANDOM, 8), (STRIDE, 4)):
        s2 = Shard.contiguous(L, m0, np.zeros(L, np.float32))
        _, _, q, _ = s2.encode(Params(scheme=scheme, k=k, step=3), oracle.pad_chunks(g, L))
        u = _u_ref(m0, g, 0.9, L)
        assert np.max(np.abs(s2.m + q - u)) <= 1e-15 * np.max(np.abs(u)) * 4


def test_k32_extracts_everything():
    L = 32 * 16
    sh, m0, _ = _shard(L, seed=9)
    g = _grad(L, seed=10)
    _, val, q, X = sh.encode(Params(scheme=DCT, k=32), oracle.pad_chunks(g, L))
    u = _u_ref(m0, g, 0.9, L)
    assert np.max(np.abs(q - u)) < 1e-13
    assert np.max(np.abs(sh.m)) < 1e-13
    assert np.array_equal(val, np.sign(X))


def test_random_n32_and_diloco_sync_zero_the_momentum_exactly():
    L = 32 * 16
    g = _grad(L, seed=11)
    for p in (Params(scheme=RANDOM, k=32), Params(scheme=STRIDE, k=32),
              Params(scheme=DILOCO, period=16, step=15)):
        sh, m0, _ = _shard(L, seed=12)
        _, val, q, _ = sh.encode(p, oracle.pad_chunks(g, L))
        u = _u_ref(m0, g, 0.9, L)
        assert np.array_equal(q, u)
        assert np.all(sh.m == 0.0)
        assert val.shape == (L // N, 32)
        assert np.array_equal(val, np.sign(u))


def test_diloco_between_syncs_accumulates_and_sends_nothing():
    L = 32 * 8
    sh, m0, th0 = _shard(L, seed=13)
    g = _grad(L, seed=14)
    p = Params(scheme=DILOCO, period=16, step=3)
    assert oracle.slots(p) == 0
    idx, val, q, _ = sh.encode(p, oracle.pad_chunks(g, L))
    assert idx.shape[1] == 0 and val.shape[1] == 0
    assert np.all(q == 0.0)
    assert np.array_equal(sh.m, _u_ref(m0, g, 0.9, L))
    before = sh.theta.copy()
    sh.decode(p, [idx, idx], [val, val])
    assert np.array_equal(sh.theta, before)


def test_random_and_stride_select_the_shared_positions():
    L = 32 * 30
    g = _grad(L, seed=15)
    for scheme, k in ((RANDOM, 8), (RANDOM, 16), (STRIDE, 8), (STRIDE, 16)):
        sh, m0, _ = _shard(L, seed=16)
        p = Params(scheme=scheme, k=k, seed=77, step=5)
        idx, val, q, _ = sh.encode(p, oracle.pad_chunks(g, L))
        u = _u_ref(m0, g, 0.9, L)
        for c in range(L // N):
            mask = oracle.select_mask(77, 5, c, k) if scheme == RANDOM else oracle.stride_mask(5, k)
            pos = [j for j in range(N) if (mask >> j) & 1]
            assert list(idx[c]) == pos
            assert np.array_equal(val[c], np.sign(u[c][pos]))
            expect_m = u[c].copy()
            expect_m[pos] = 0.0
            assert np.array_equal(sh.m[c], expect_m)


@pytest.mark.parametrize("fmt", [oracle.F32, oracle.F16])
def test_sign_off_dct_carries_the_rounded_coefficients(fmt):
    """Sign off: each slot carries the selected DCT coefficient itself, rounded
    to the payload format (numpy's float32 / float16 conversions from fp64 are
    round-to-nearest-even); selection and q are those of the signed run."""
    L = 32 * 40
    sh, m0, _ = _shard(L, seed=40)
    g = _grad(L, seed=41)
    p = Params(scheme=DCT, k=3, sign=0, value_fmt=fmt)
    idx, val, q, _ = sh.encode(p, oracle.pad_chunks(g, L))
    u = _u_ref(m0, g, 0.9, L)
    Xref = scipy.fft.dct(u, type=2, norm="ortho", axis=1)
    to = np.float32 if fmt == oracle.F32 else np.float16
    for c in range(L // N):
        sel = np.sort(np.argsort(-np.abs(Xref[c].astype(np.float32)), kind="stable")[:3])
        assert np.array_equal(idx[c], sel)
        assert np.array_equal(val[c], Xref[c][sel].astype(to).astype(np.float64))
        Xs = np.zeros(N)
        Xs[sel] = Xref[c][sel]
        assert np.max(np.abs(q[c] - scipy.fft.idct(Xs, type=2, norm="ortho"))) < 1e-13


@pytest.mark.parametrize("fmt", [oracle.F32, oracle.F16])
def test_sign_off_random_carries_u_and_fp16_keeps_subnormals(fmt):
    L = 32 * 30
    sh, m0, _ = _shard(L, seed=42, m_std=1e-6)
    g = (_grad(L, seed=43) * np.float32(1e-6)).astype(np.float32)  # |u| spans fp16's subnormal range
    p = Params(scheme=RANDOM, k=8, seed=5, step=2, sign=0, value_fmt=fmt)
    idx, val, _, _ = sh.encode(p, oracle.pad_chunks(g, L))
    u = _u_ref(m0, g, 0.9, L)
    to = np.float32 if fmt == oracle.F32 else np.float16
    subnormal = 0
    for c in range(L // N):
        pos = [j for j in range(N) if (oracle.select_mask(5, 2, c, 8) >> j) & 1]
        want = u[c][pos].astype(to)
        assert np.array_equal(val[c], want.astype(np.float64))
        subnormal += int(np.sum((np.abs(want) < 2.0 ** -14) & (want != 0)))
    if fmt == oracle.F16:
        assert subnormal > 100


def test_decode_of_value_payloads_is_the_inverse_dct_of_the_mean():
    C, k, R = 9, 5, 3
    rng = np.random.default_rng(44)
    pays = [_slots(C, k, rng) for _ in range(R)]
    vals = [rng.standard_normal((C, k)) for _ in range(R)]
    sh = Shard.contiguous(C * N, np.zeros(C * N, np.float32), rng.standard_normal(C * N).astype(np.float32))
    th0 = sh.theta.copy()
    p = Params(scheme=DCT, k=k, sign=0, value_fmt=oracle.F32, lr=1e-3)
    Q = sh.decode(p, [i for i, _ in pays], vals)
    for c in range(C):
        A = np.zeros(N)
        for r in range(R):
            A[pays[r][0][c]] += vals[r][c]
        Qref = scipy.fft.idct(A / R, type=2, norm="ortho")
        assert np.max(np.abs(Q[c] - Qref)) < 1e-14
        # theta ~ N(0, 1): a few units in the last place of fp64
        assert np.max(np.abs(sh.theta[c] - (th0[c] - np.float64(np.float32(1e-3)) * Qref))) < 1e-15


def test_ternary_values_and_sign_of_zero():
    L = 32 * 4
    sh = Shard.contiguous(L, np.zeros(L, np.float32), np.zeros(L, np.float32))
    g = np.zeros(L, np.float32)
    g[32:64] = 1.0  # constant chunk
    g[64:96] = -0.0
    idx, val, _, _ = sh.encode(Params(scheme=DCT, k=4), oracle.pad_chunks(g, L))
    assert set(np.unique(val)) <= {-1.0, 0.0, 1.0}
    assert np.array_equal(idx[0], [0, 1, 2, 3]) and np.all(val[0] == 0)
    assert idx[1][0] == 0 and val[1][0] == 1.0
    assert np.all(val[2] == 0)


def test_ragged_tail_keeps_pads_at_zero():
    L = 32 * 3 + 5
    sh, m0, _ = _shard(L, seed=17)
    g = _grad(L, seed=18)
    _, _, q, _ = sh.encode(Params(scheme=DCT, k=2), oracle.pad_chunks(g, L))
    assert np.all(sh.m[-1, 5:] == 0.0) and np.all(q[-1, 5:] == 0.0)
    u = _u_ref(m0, g, 0.9, L)
    Xref = scipy.fft.dct(u[-1], type=2, norm="ortho")  # pads enter the transform as zeros
    sel = np.sort(np.argsort(-np.abs(Xref.astype(np.float32)), kind="stable")[:2])
    Xs = np.zeros(N)
    Xs[sel] = Xref[sel]
    assert np.max(np.abs(sh.m[-1, :5] - (u[-1] - scipy.fft.idct(Xs, type=2, norm="ortho"))[:5])) < 1e-13


# ------------------------------------------------------------------ decode ----

def _slots(C, k, rng, values=(-1.0, 0.0, 1.0)):
    idx = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(C)]).astype(np.int32)
    val = rng.choice(values, size=(C, k))
    return idx, val


def test_decode_single_payload_is_the_inverse_dct():
    C, k = 10, 3
    rng = np.random.default_rng(19)
    idx, val = _slots(C, k, rng)
    sh = Shard.contiguous(C * N, np.zeros(C * N, np.float32), rng.standard_normal(C * N).astype(np.float32))
    th0 = sh.theta.copy()
    p = Params(scheme=DCT, k=k, lr=1e-3)
    Q = sh.decode(p, [idx], [val])
    for c in range(C):
        A = np.zeros(N)
        A[idx[c]] = val[c]
        Qref = scipy.fft.idct(A, type=2, norm="ortho")
        assert np.max(np.abs(Q[c] - Qref)) < 1e-14
        assert np.max(np.abs(sh.theta[c] - (th0[c] - np.float64(np.float32(1e-3)) * Qref))) < 1e-16


def test_decode_opposite_signs_cancel_and_leave_theta_bit_identical():
    C, k = 8, 4
    rng = np.random.default_rng(20)
    idx, val = _slots(C, k, rng)
    sh = Shard.contiguous(C * N, np.zeros(C * N, np.float32), rng.standard_normal(C * N).astype(np.float32))
    th0 = sh.theta.copy()
    Q = sh.decode(Params(scheme=DCT, k=k), [idx, idx], [val, -val])
    assert np.all(Q == 0.0)
    assert np.array_equal(sh.theta, th0)


def test_decode_identical_payloads_equal_one_and_is_linear():
    C, k = 6, 2
    rng = np.random.default_rng(21)
    payloads = [_slots(C, k, rng) for _ in range(5)]
    zeros = np.zeros(C * N, np.float32)
    p = Params(scheme=DCT, k=k)
    one = Shard.contiguous(C * N, zeros, zeros).decode(p, [payloads[0][0]], [payloads[0][1]])
    three = Shard.contiguous(C * N, zeros, zeros).decode(p, [payloads[0][0]] * 3, [payloads[0][1]] * 3)
    assert np.max(np.abs(one - three)) < 1e-15
    allR = Shard.contiguous(C * N, zeros, zeros).decode(p, [i for i, _ in payloads], [v for _, v in payloads])
    singles = [Shard.contiguous(C * N, zeros, zeros).decode(p, [i], [v]) for i, v in payloads]
    assert np.max(np.abs(allR - np.mean(singles, axis=0))) < 1e-15


def test_random_decode_touches_only_selected_positions():
    C, k = 20, 8
    rng = np.random.default_rng(22)
    th = rng.standard_normal(C * N).astype(np.float32)
    sh = Shard.contiguous(C * N, np.zeros(C * N, np.float32), th)
    th0 = sh.theta.copy()
    vals = [rng.choice([-1.0, 0.0, 1.0], size=(C, k)) for _ in range(3)]
    p = Params(scheme=RANDOM, k=k, seed=5, step=9)
    Q = sh.decode(p, [np.zeros((C, k), np.int32)] * 3, vals)
    for c in range(C):
        mask = oracle.select_mask(5, 9, c, k)
        pos = [j for j in range(N) if (mask >> j) & 1]
        off = [j for j in range(N) if not (mask >> j) & 1]
        assert np.array_equal(sh.theta[c][off], th0[c][off])
        assert np.allclose(Q[c][pos], np.mean([v[c] for v in vals], axis=0), rtol=0, atol=1e-15)


def test_chunk_offset_moves_random_selection():
    L = 32 * 4
    g = _grad(L, seed=23)
    a = Shard.contiguous(L, np.zeros(L, np.float32), np.zeros(L, np.float32), chunk_offset=0)
    b = Shard.contiguous(L, np.zeros(L, np.float32), np.zeros(L, np.float32), chunk_offset=1000)
    p = Params(scheme=RANDOM, k=8, seed=1, step=0)
    ia, _, _, _ = a.encode(p, oracle.pad_chunks(g, L))
    ib, _, _, _ = b.encode(p, oracle.pad_chunks(g, L))
    assert not np.array_equal(ia, ib)
    mask = oracle.select_mask(1, 0, 1002, 8)
    assert list(ib[2]) == [j for j in range(N) if (mask >> j) & 1]
