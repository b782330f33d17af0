"""fp64 CPU oracle for the DeMo / FlexDeMo optimizer step (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the library and its binding never
do.  The arithmetic lives in ``oracle.c`` (plain C, fp64); this module only
marshals numpy arrays into it.  It shares no code with the GPU library.

Method sources: DeToNATION paper notes (AAAI 2026), Algorithm 1 and the
"Replication schemes" table; DeMo abstract (DCT + top-k + momentum subtraction).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CHUNK = 32
DCT, RANDOM, STRIDE, DILOCO = 0, 1, 2, 3
TERNARY, F16, F32 = 0, 1, 2
# guided encode: bits of the per-chunk status
GUIDE_POSITIONS, GUIDE_SIGNS, GUIDE_REJECTED = 1, 2, 4


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no -ffast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


class _Params(ctypes.Structure):
    _fields_ = [
        ("scheme", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("period", ctypes.c_int32),
        ("sign", ctypes.c_int32),
        ("value_fmt", ctypes.c_int32),
        ("beta", ctypes.c_float),
        ("lr", ctypes.c_float),
        ("seed", ctypes.c_uint64),
        ("step", ctypes.c_uint64),
    ]


@dataclass
class Params:
    """Step configuration (the oracle's own copy of the method's knobs)."""

    scheme: int = DCT
    k: int = 1
    period: int = 16
    sign: int = 1
    value_fmt: int = TERNARY
    beta: float = 0.9
    lr: float = 1e-3
    seed: int = 0
    step: int = 0

    def c(self) -> _Params:
        return _Params(self.scheme, self.k, self.period, self.sign, self.value_fmt,
                       self.beta, self.lr, self.seed, self.step)


class _AdamW(ctypes.Structure):
    _fields_ = [("beta2", ctypes.c_float), ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("reserved", ctypes.c_int32)]


@dataclass
class AdamW:
    """Decoupled AdamW's extra knobs (beta1 is Params.beta)."""

    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01

    def c(self) -> _AdamW:
        return _AdamW(self.beta2, self.eps, self.weight_decay, 0)


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        L.oracle_threads.argtypes = []
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_set_threads.restype = None
        L.oracle_basis.argtypes = [P]
        L.oracle_dct.argtypes = [P, P]
        L.oracle_idct.argtypes = [P, P]
        L.oracle_topk.argtypes = [P, ctypes.c_int, P]
        L.oracle_topk.restype = ctypes.c_int
        L.oracle_philox4x32.argtypes = [P, P, P]
        L.oracle_select_mask.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int]
        L.oracle_select_mask.restype = ctypes.c_uint32
        L.oracle_stride_mask.argtypes = [ctypes.c_uint64, ctypes.c_int]
        L.oracle_stride_mask.restype = ctypes.c_uint32
        L.oracle_slots.argtypes = [ctypes.POINTER(_Params)]
        L.oracle_slots.restype = ctypes.c_int
        L.oracle_to_f16_bits.argtypes = [ctypes.c_double]
        L.oracle_to_f16_bits.restype = ctypes.c_uint16
        L.oracle_from_f16_bits.argtypes = [ctypes.c_uint16]
        L.oracle_from_f16_bits.restype = ctypes.c_double
        L.oracle_wire_value.argtypes = [ctypes.POINTER(_Params), ctypes.c_double]
        L.oracle_wire_value.restype = ctypes.c_double
        L.oracle_encode.argtypes = [ctypes.POINTER(_Params), ctypes.c_int64, P, P, P, P, P, P, P, P,
                                    P, P, ctypes.c_double, P]
        L.oracle_encode.restype = ctypes.c_int
        L.oracle_decode.argtypes = [ctypes.POINTER(_Params), ctypes.c_int64, P, P, ctypes.c_int32,
                                    P, P, P, P]
        L.oracle_decode.restype = ctypes.c_int
        L.oracle_encode_adamw.argtypes = [ctypes.POINTER(_Params), ctypes.POINTER(_AdamW), ctypes.c_int64,
                                          P, P, P, P, P, P, P, P, P, P, P, ctypes.c_double, P]
        L.oracle_encode_adamw.restype = ctypes.c_int
        L.oracle_decode_adamw.argtypes = [ctypes.POINTER(_Params), ctypes.POINTER(_AdamW), ctypes.c_int64,
                                          P, P, ctypes.c_int32, P, P, P, P, P]
        L.oracle_decode_adamw.restype = ctypes.c_int
        L.oracle_payload_regions.argtypes = [ctypes.POINTER(_Params), ctypes.c_uint64, P]
        L.oracle_pack.argtypes = [ctypes.POINTER(_Params), ctypes.c_uint64, P, P, P]
        L.oracle_pack.restype = ctypes.c_int
        L.oracle_unpack.argtypes = [ctypes.POINTER(_Params), ctypes.c_uint64, P, P, P]
        L.oracle_unpack.restype = ctypes.c_int
        L.oracle_unpack_chunks.argtypes = [ctypes.POINTER(_Params), ctypes.c_uint64, P, P, ctypes.c_uint64, P, P]
        L.oracle_unpack_chunks.restype = ctypes.c_int
        L.oracle_payload_violations.argtypes = [ctypes.POINTER(_Params), ctypes.c_uint64, P]
        L.oracle_payload_violations.restype = ctypes.c_uint64
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# --------------------------------------------------------------------------- #
# transform, ranking and generator primitives                                 #
# --------------------------------------------------------------------------- #

def threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return int(lib().oracle_threads())


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def basis() -> np.ndarray:
    B = np.zeros((CHUNK, CHUNK), np.float64)
    lib().oracle_basis(_ptr(B))
    return B


def dct(u) -> np.ndarray:
    u = np.ascontiguousarray(u, np.float64)
    X = np.zeros(CHUNK, np.float64)
    lib().oracle_dct(_ptr(u), _ptr(X))
    return X


def idct(X) -> np.ndarray:
    X = np.ascontiguousarray(X, np.float64)
    u = np.zeros(CHUNK, np.float64)
    lib().oracle_idct(_ptr(X), _ptr(u))
    return u


def topk(X, k: int) -> np.ndarray:
    X = np.ascontiguousarray(X, np.float64)
    out = np.zeros(k, np.int32)
    if lib().oracle_topk(_ptr(X), k, _ptr(out)) != 0:
        raise ValueError("bad k")
    return out


def philox4x32(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().oracle_philox4x32(_ptr(c), _ptr(k), _ptr(out))
    return out


def select_mask(seed: int, step: int, chunk: int, n: int) -> int:
    return int(lib().oracle_select_mask(seed, step, chunk, n))


def stride_mask(step: int, n: int) -> int:
    return int(lib().oracle_stride_mask(step, n))


def to_f16_bits(x: float) -> int:
    return int(lib().oracle_to_f16_bits(x))


def from_f16_bits(h: int) -> float:
    return float(lib().oracle_from_f16_bits(h))


def wire_value(p: Params, x: float) -> float:
    """The value a slot carries for the selected value x: sign(x) with the sign
    on, else x rounded to the payload's fp16 or fp32 format."""
    c = p.c()
    return float(lib().oracle_wire_value(ctypes.byref(c), float(x)))


def slots(p: Params) -> int:
    c = p.c()
    return int(lib().oracle_slots(ctypes.byref(c)))


# --------------------------------------------------------------------------- #
# chunk-list state and the two halves of the step                             #
# --------------------------------------------------------------------------- #

class Shard:
    """fp64 state (m, theta, and Decoupled AdamW's second moment v) of a list
    of chunks of one shard.

    chunk_ids: global chunk index of each chunk (used by Random hashing).
    nvalid:    valid elements per chunk (32 except a ragged last chunk).
    m0, theta0, v0: fp32 inputs, [n][32] (padded positions ignored), widened
    to fp64; v0 defaults to zeros.
    """

    def __init__(self, chunk_ids, nvalid, m0, theta0, v0=None):
        self.chunk_ids = np.ascontiguousarray(chunk_ids, np.uint64)
        self.nvalid = np.ascontiguousarray(nvalid, np.int32)
        n = len(self.chunk_ids)
        self.m = np.ascontiguousarray(np.asarray(m0, np.float32).reshape(n, CHUNK), np.float64)
        self.theta = np.ascontiguousarray(np.asarray(theta0, np.float32).reshape(n, CHUNK), np.float64)
        self.v = (np.zeros((n, CHUNK), np.float64) if v0 is None else
                  np.ascontiguousarray(np.asarray(v0, np.float32).reshape(n, CHUNK), np.float64))
        pad = np.arange(CHUNK)[None, :] >= self.nvalid[:, None]
        self.m[pad] = 0.0
        self.theta[pad] = 0.0
        self.v[pad] = 0.0

    @classmethod
    def contiguous(cls, n_elems: int, m0_flat, theta0_flat, chunk_offset: int = 0):
        C = (n_elems + CHUNK - 1) // CHUNK
        ids = np.arange(C, dtype=np.uint64) + np.uint64(chunk_offset)
        nv = np.full(C, CHUNK, np.int32)
        nv[-1] = n_elems - (C - 1) * CHUNK
        return cls(ids, nv, pad_chunks(m0_flat, n_elems), pad_chunks(theta0_flat, n_elems))

    @property
    def n(self) -> int:
        return len(self.chunk_ids)

    def encode(self, p: Params, g, adamw: AdamW | None = None):
        """Algorithm 1 steps 3-5 (Decoupled AdamW's moments when adamw is
        given). g is fp32 [n][32]. Returns (idx, val, q, X)."""
        return self._encode(p, g, adamw, None, None, 0.0)[:4]

    def encode_guided(self, p: Params, g, guide_idx, guide_val, near: float, adamw: AdamW | None = None):
        """encode, taking another implementation's positions (DCT) and ternary
        signs where several are correct: a guide that is a valid top-k up to
        near * max|X|, or a sign of a value within near * max|x| of zero.
        guide_idx / guide_val are [n][slots] as encode returns them.  Returns
        (idx, val, q, X, status) with status [n] the GUIDE_* bits per chunk
        (GUIDE_REJECTED: the guide differs where only one answer is right;
        the oracle then keeps its own)."""
        s = slots(p)
        gi = np.ascontiguousarray(np.asarray(guide_idx, np.int32).reshape(self.n, s) if s else
                                  np.zeros((self.n, 1), np.int32))
        gv = np.ascontiguousarray(np.asarray(guide_val, np.float64).reshape(self.n, s) if s else
                                  np.zeros((self.n, 1), np.float64))
        return self._encode(p, g, adamw, gi, gv, near)

    def _encode(self, p, g, adamw, gi, gv, near):
        n = self.n
        g = np.ascontiguousarray(np.asarray(g, np.float32).reshape(n, CHUNK))
        s = slots(p)
        idx = np.zeros((n, max(s, 1)), np.int32)
        val = np.zeros((n, max(s, 1)), np.float64)
        q = np.zeros((n, CHUNK), np.float64)
        X = np.zeros((n, CHUNK), np.float64)
        status = np.zeros(n, np.int32)
        st = None if gi is None else status
        c = p.c()
        if adamw is None:
            r = lib().oracle_encode(ctypes.byref(c), n, _ptr(self.chunk_ids), _ptr(self.nvalid), _ptr(g),
                                    _ptr(self.m), _ptr(idx), _ptr(val), _ptr(q), _ptr(X), _ptr(gi), _ptr(gv),
                                    float(near), _ptr(st))
        else:
            w = adamw.c()
            r = lib().oracle_encode_adamw(ctypes.byref(c), ctypes.byref(w), n, _ptr(self.chunk_ids),
                                          _ptr(self.nvalid), _ptr(g), _ptr(self.m), _ptr(self.v), _ptr(idx),
                                          _ptr(val), _ptr(q), _ptr(X), _ptr(gi), _ptr(gv), float(near), _ptr(st))
        if r < 0:
            raise ValueError("oracle_encode: bad configuration")
        return idx[:, :s], val[:, :s], q, X, status

    def decode(self, p: Params, idx_list, val_list, adamw: AdamW | None = None):
        """Algorithm 1 steps 6-7 over R payloads (own first); with adamw the
        update uses this shard's second moment. Returns Q [n][32]."""
        n = self.n
        R = len(val_list)
        s = slots(p)
        idx = np.ascontiguousarray(
            np.stack([np.asarray(i, np.int32).reshape(n, s) for i in idx_list]) if s else
            np.zeros((R, n, 1), np.int32))
        val = np.ascontiguousarray(
            np.stack([np.asarray(v, np.float64).reshape(n, s) for v in val_list]) if s else
            np.zeros((R, n, 1), np.float64))
        Q = np.zeros((n, CHUNK), np.float64)
        c = p.c()
        if adamw is None:
            rc = lib().oracle_decode(ctypes.byref(c), n, _ptr(self.chunk_ids), _ptr(self.nvalid), R,
                                     _ptr(idx), _ptr(val), _ptr(self.theta), _ptr(Q))
        else:
            w = adamw.c()
            rc = lib().oracle_decode_adamw(ctypes.byref(c), ctypes.byref(w), n, _ptr(self.chunk_ids),
                                           _ptr(self.nvalid), R, _ptr(idx), _ptr(val), _ptr(self.v),
                                           _ptr(self.theta), _ptr(Q))
        if rc != 0:
            raise ValueError("oracle_decode: bad arguments")
        return Q


def pad_chunks(flat, n_elems: int) -> np.ndarray:
    """Flat fp32 array of n_elems -> [C][32] with the tail zero-padded."""
    C = (n_elems + CHUNK - 1) // CHUNK
    out = np.zeros(C * CHUNK, np.float32)
    out[:n_elems] = np.asarray(flat, np.float32).reshape(-1)[:n_elems]
    return out.reshape(C, CHUNK)


def unpad(chunks, n_elems: int) -> np.ndarray:
    return np.asarray(chunks).reshape(-1)[:n_elems]


# --------------------------------------------------------------------------- #
# payload codec (the oracle's own implementation of the wire format)          #
# --------------------------------------------------------------------------- #

REGION_NAMES = ("idx_off", "idx_bytes", "nz_off", "neg_off", "plane_bytes", "val_off",
                "val_bytes", "total_bytes")


def payload_regions(p: Params, n_elems: int) -> dict:
    out = np.zeros(8, np.uint64)
    c = p.c()
    lib().oracle_payload_regions(ctypes.byref(c), n_elems, _ptr(out))
    return dict(zip(REGION_NAMES, (int(x) for x in out)))


def pack(p: Params, n_elems: int, idx, val) -> np.ndarray:
    reg = payload_regions(p, n_elems)
    buf = np.zeros(reg["total_bytes"], np.uint8)
    idx = np.ascontiguousarray(idx, np.int32)
    val = np.ascontiguousarray(val, np.float64)
    c = p.c()
    if lib().oracle_pack(ctypes.byref(c), n_elems, _ptr(idx), _ptr(val), _ptr(buf)) != 0:
        raise ValueError("oracle_pack: value not representable in the ternary format")
    return buf


def unpack(p: Params, n_elems: int, buf, chunks=None):
    """Returns (idx [C][k], val [C][k], ok) where ok is False for a malformed
    buffer.  With chunks (chunk ids within the shard) the rows are those
    chunks' slots, in the order given; ok still covers the whole buffer."""
    buf = np.ascontiguousarray(buf, np.uint8)
    C = (n_elems + CHUNK - 1) // CHUNK
    k = CHUNK if p.scheme == DILOCO else p.k
    c = p.c()
    if chunks is None:
        idx = np.zeros((C, k), np.int32)
        val = np.zeros((C, k), np.float64)
        r = lib().oracle_unpack(ctypes.byref(c), n_elems, _ptr(buf), _ptr(idx), _ptr(val))
        return idx, val, r == 0
    ids = np.ascontiguousarray(chunks, np.uint64)
    idx = np.zeros((len(ids), k), np.int32)
    val = np.zeros((len(ids), k), np.float64)
    r = lib().oracle_unpack_chunks(ctypes.byref(c), n_elems, _ptr(buf), _ptr(ids), len(ids), _ptr(idx), _ptr(val))
    if r == -2:
        raise IndexError("unpack: chunk id past the shard")
    return idx, val, r == 0


def payload_violations(p: Params, n_elems: int, buf) -> int:
    """Number of violations of the payload format in one replica's buffer
    (NEG without NZ, bits past the last chunk, index bytes above 31 or not
    ascending, sign-on values other than -1/0/+1, sign-off non-finite values)."""
    buf = np.ascontiguousarray(buf, np.uint8)
    assert buf.size >= payload_regions(p, n_elems)["total_bytes"]
    c = p.c()
    return int(lib().oracle_payload_violations(ctypes.byref(c), n_elems, _ptr(buf)))
