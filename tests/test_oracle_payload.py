"""Pins of the oracle's payload codec and fp16 conversion.

The pages fix no wire format (only that DeMo sends indices and Random /
Striding / DiLoCo do not, and that values are ternary after the sign); the
format below is this library's, stated in include/demo.h:
  IDX uint8 [C][k] | NZ uint64 [G][k] | NEG uint64 [G][k]  (ternary)
  IDX uint8 [C][k] | VAL fp16/fp32 [C][k]                   (value formats)
regions 256-byte aligned, word g*k+s bit b = slot s of chunk 64g+b.
"""
import numpy as np
import pytest

import oracle
from oracle import DCT, DILOCO, F16, F32, RANDOM, STRIDE, TERNARY, Params

N = 32


def _random_slots(C, k, rng, fmt):
    idx = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(C)]).astype(np.int32)
    if fmt == TERNARY:
        val = rng.choice([-1.0, 0.0, 1.0], size=(C, k))
    else:
        val = rng.choice([-1.0, 0.0, 1.0], size=(C, k))
    return idx, val


@pytest.mark.parametrize("scheme,k", [(DCT, 1), (DCT, 2), (DCT, 4), (RANDOM, 8), (STRIDE, 16), (DILOCO, 32)])
@pytest.mark.parametrize("fmt", [TERNARY, F16, F32])
@pytest.mark.parametrize("n_elems", [7, 32 * 64, 32 * 130 + 9])
def test_pack_unpack_round_trip(scheme, k, fmt, n_elems):
    p = Params(scheme=scheme, k=k, value_fmt=fmt, step=15)
    C = (n_elems + N - 1) // N
    rng = np.random.default_rng(n_elems + k)
    idx, val = _random_slots(C, k, rng, fmt)
    buf = oracle.pack(p, n_elems, idx, val)
    reg = oracle.payload_regions(p, n_elems)
    assert buf.size == reg["total_bytes"] and reg["total_bytes"] % 256 == 0
    for key in ("idx_off", "nz_off", "neg_off", "val_off"):
        assert reg[key] % 256 == 0
    i2, v2, ok = oracle.unpack(p, n_elems, buf)
    assert ok
    assert np.array_equal(v2, val)
    if scheme == DCT:
        assert np.array_equal(i2, idx)


def test_region_sizes():
    G = lambda C: (C + 63) // 64
    up = lambda x: (x + 255) // 256 * 256
    L = 639_697_920
    C = L // 32
    r = oracle.payload_regions(Params(scheme=DCT, k=1), L)
    assert r["idx_bytes"] == C and r["plane_bytes"] == G(C) * 8
    assert r["total_bytes"] == up(C) + 2 * up(G(C) * 8) == 24_988_928
    r = oracle.payload_regions(Params(scheme=RANDOM, k=8), L)
    assert r["idx_bytes"] == 0 and r["total_bytes"] == 2 * up(G(C) * 8 * 8)
    r = oracle.payload_regions(Params(scheme=RANDOM, k=8, value_fmt=F16), L)
    assert r["val_bytes"] == C * 8 * 2
    r = oracle.payload_regions(Params(scheme=RANDOM, k=8, value_fmt=F32), L)
    assert r["val_bytes"] == C * 8 * 4
    r = oracle.payload_regions(Params(scheme=DILOCO), L)
    assert r["plane_bytes"] == G(C) * 32 * 8


def test_hand_built_bit_positions():
    # chunk 0 slot 0 = -1; chunk 65 slot 1 = +1 (k = 2): word g*k+s, bit c mod 64
    p = Params(scheme=DCT, k=2)
    n = 32 * 70
    idx = np.tile(np.array([[3, 9]], np.int32), (70, 1))
    val = np.zeros((70, 2))
    val[0, 0] = -1.0
    val[65, 1] = 1.0
    buf = oracle.pack(p, n, idx, val)
    reg = oracle.payload_regions(p, n)
    nz = buf[reg["nz_off"]:reg["nz_off"] + reg["plane_bytes"]].view(np.uint64)
    neg = buf[reg["neg_off"]:reg["neg_off"] + reg["plane_bytes"]].view(np.uint64)
    assert list(nz) == [1, 0, 0, 2] and list(neg) == [1, 0, 0, 0]
    assert list(buf[:4]) == [3, 9, 3, 9]


def test_unpack_flags_malformed_buffers():
    p = Params(scheme=DCT, k=1)
    n = 32 * 10
    idx = np.zeros((10, 1), np.int32)
    val = np.ones((10, 1))
    buf = oracle.pack(p, n, idx, val)
    reg = oracle.payload_regions(p, n)
    bad = buf.copy()
    bad[reg["nz_off"]] &= 0xFE  # NEG without NZ would need NEG set; clear NZ of chunk 0 and set NEG
    bad[reg["neg_off"]] |= 0x01
    assert not oracle.unpack(p, n, bad)[2]
    bad = buf.copy()
    bad[reg["nz_off"] + 1] |= 0x80  # chunk 15 does not exist (C = 10)
    assert not oracle.unpack(p, n, bad)[2]


@pytest.mark.parametrize("scheme,k,fmt", [(DCT, 2, TERNARY), (DCT, 3, F16), (RANDOM, 8, F32), (DILOCO, 32, TERNARY)])
def test_unpack_of_listed_chunks_equals_rows_of_the_whole(scheme, k, fmt):
    p = Params(scheme=scheme, k=k, value_fmt=fmt, step=15)
    n = 32 * 64 * 3 + 17  # four groups, a ragged last chunk
    C = (n + N - 1) // N
    rng = np.random.default_rng(k)
    idx, val = _random_slots(C, k, rng, fmt)
    buf = oracle.pack(p, n, idx, val)
    i_all, v_all, ok = oracle.unpack(p, n, buf)
    assert ok
    ids = np.array([C - 1, 0, 63, 64, 130, 5, 130], np.int64)  # any order, repeats allowed
    i_s, v_s, ok = oracle.unpack(p, n, buf, chunks=ids)
    assert ok
    assert np.array_equal(v_s, v_all[ids]) and np.array_equal(i_s, i_all[ids])
    with pytest.raises(IndexError):
        oracle.unpack(p, n, buf, chunks=[C])


@pytest.mark.parametrize("C", [10, 64, 129])
def test_malformed_check_covers_the_whole_buffer(C):
    """A bit for a chunk past the end, or NEG without NZ, flags the buffer
    even when the chunks asked for are well formed; a full last group has no
    chunk past the end."""
    p = Params(scheme=DCT, k=2)
    n = 32 * C
    idx = np.tile(np.array([[1, 4]], np.int32), (C, 1))
    val = np.ones((C, 2))
    buf = oracle.pack(p, n, idx, val)
    reg = oracle.payload_regions(p, n)
    G = (C + 63) // 64
    assert oracle.unpack(p, n, buf, chunks=[0])[2]
    nz = buf[reg["nz_off"]:reg["nz_off"] + reg["plane_bytes"]].view(np.uint64)
    assert nz[(G - 1) * 2 + 1] == (np.uint64(2**64 - 1) if C % 64 == 0 else np.uint64((1 << (C % 64)) - 1))
    if C % 64:
        bad = buf.copy()
        bad[reg["nz_off"]:reg["nz_off"] + reg["plane_bytes"]].view(np.uint64)[(G - 1) * 2 + 1] |= np.uint64(1 << 63)
        assert not oracle.unpack(p, n, bad)[2]
        assert not oracle.unpack(p, n, bad, chunks=[0])[2]
    bad = buf.copy()
    w = bad[reg["nz_off"]:reg["nz_off"] + reg["plane_bytes"]].view(np.uint64)
    w[0] &= ~np.uint64(1 << 3)  # chunk 3, slot 0: NZ cleared, NEG set
    bad[reg["neg_off"]:reg["neg_off"] + reg["plane_bytes"]].view(np.uint64)[0] |= np.uint64(1 << 3)
    assert not oracle.unpack(p, n, bad, chunks=[C - 1])[2]


def test_f16_conversion_matches_numpy_round_to_nearest_even():
    rng = np.random.default_rng(24)
    xs = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 1e9, 2.0 ** -24, 2.0 ** -25,
         2.0 ** -25 * 1.0000001, 2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -11), 3 * 2.0 ** -26],
    ])
    for x in xs:
        h = np.float16(x)
        assert oracle.to_f16_bits(float(x)) == int(h.view(np.uint16)), x
        if np.isfinite(h):
            assert oracle.from_f16_bits(int(h.view(np.uint16))) == float(h)


def _region(buf, reg, off_key, nbytes, dtype):
    return buf[reg[off_key]:reg[off_key] + nbytes].view(dtype)


@pytest.mark.parametrize("scheme,k,fmt", [(DCT, 1, TERNARY), (DCT, 3, F16), (RANDOM, 8, F32), (DILOCO, 32, TERNARY)])
def test_well_formed_payloads_have_no_violations(scheme, k, fmt):
    p = Params(scheme=scheme, k=k, value_fmt=fmt, step=15)
    n = 32 * 130 + 9
    C = (n + N - 1) // N
    idx, val = _random_slots(C, k, np.random.default_rng(3), fmt)
    assert oracle.payload_violations(p, n, oracle.pack(p, n, idx, val)) == 0


def test_violation_count_on_hand_built_buffers():
    """Each planted defect counts once: 2 NEG-without-NZ bits, 3 bits past
    the last chunk, 1 index byte above 31, 1 non-ascending pair."""
    p = Params(scheme=DCT, k=2)
    n = 32 * 70  # C = 70: the second group holds chunks 64..69
    C = 70
    idx = np.tile(np.array([[3, 9]], np.int32), (C, 1))
    val = np.ones((C, 2))
    val[5, 0] = 0.0  # slot 0 of chunk 5 is zero: its NZ bit is clear
    buf = oracle.pack(p, n, idx, val)
    reg = oracle.payload_regions(p, n)
    nz = _region(buf, reg, "nz_off", reg["plane_bytes"], np.uint64)
    neg = _region(buf, reg, "neg_off", reg["plane_bytes"], np.uint64)
    neg[0] |= np.uint64(1 << 5)   # chunk 5 slot 0: NEG without NZ
    neg[1] |= np.uint64(1 << 5)   # chunk 5 slot 1: NZ is set (+1 -> -1), not a violation
    nz[2] &= ~np.uint64(1 << 1)   # chunk 65 slot 0: NZ cleared ...
    neg[2] |= np.uint64(1 << 1)   # ... with NEG set: NEG without NZ
    nz[3] |= np.uint64(1 << 10)   # chunk 74 >= C: one bit past the end
    nz[2] |= np.uint64(1 << 63)   # chunk 127: past the end
    neg[2] |= np.uint64(1 << 63)  # and its NEG bit: a second one
    buf[reg["idx_off"] + 2 * 7] = 40           # chunk 7 slot 0: above 31 (and 40 > 9: a descending pair)
    buf[reg["idx_off"] + 2 * 8 + 1] = 3        # chunk 8: slots 3, 3 do not ascend
    assert oracle.payload_violations(p, n, buf) == 2 + 3 + 1 + 1 + 1


def test_violation_count_of_value_payloads():
    n = 32 * 10
    idx = np.tile(np.array([[0, 1, 2, 3]], np.int32), (10, 1))
    on = Params(scheme=RANDOM, k=4, value_fmt=F32, sign=1)
    buf = oracle.pack(on, n, idx, np.ones((10, 4)))
    reg = oracle.payload_regions(on, n)
    v = _region(buf, reg, "val_off", reg["val_bytes"], np.float32)
    v[3], v[7], v[9] = 0.5, -0.0, np.nan  # 0.5 and NaN are not ternary; -0 is zero
    assert oracle.payload_violations(on, n, buf) == 2
    off = Params(scheme=RANDOM, k=4, value_fmt=F16, sign=0)
    buf = oracle.pack(off, n, idx, np.full((10, 4), 0.25))
    reg = oracle.payload_regions(off, n)
    h = _region(buf, reg, "val_off", reg["val_bytes"], np.uint16)
    h[0], h[1], h[2] = 0x7C00, 0x7E00, 0x3555  # +inf and NaN count; a finite value does not
    assert oracle.payload_violations(off, n, buf) == 2
    diloco = Params(scheme=DILOCO, period=16, step=3)  # no payload on a non-sync step
    assert oracle.payload_violations(diloco, n, np.full(1 << 16, 0xFF, np.uint8)) == 0
