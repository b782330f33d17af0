"""ctypes binding of libdemo (include/demo.h): argument marshalling only.

Every computation runs in the HIP kernels of libdemo.so; this module turns
PyTorch tensors into device pointers and the current HIP stream, checks that
each tensor is a contiguous device tensor of the dtype and size the call
reads or writes (so no kernel can run past it), and raises on error codes.  There is no fallback: if libdemo.so is missing the first call
raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdemo.so")

ABI_VERSION = 1
CHUNK = 32
SCHEME_DCT, SCHEME_RANDOM, SCHEME_STRIDE, SCHEME_DILOCO = 0, 1, 2, 3
VAL_TERNARY, VAL_F16, VAL_F32 = 0, 1, 2
OK, EINVAL, EALIGN, EUNSUPPORTED, EHIP, EABI = 0, -1, -2, -3, -4, -5

SYMBOLS = ("demo_abi_version", "demo_strerror", "demo_payload_layout", "demo_encode",
           "demo_decode_apply", "demo_random_select", "demo_encode_adamw", "demo_decode_apply_adamw",
           "demo_payload_validate")


class DemoError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


class demo_cfg(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_uint32),
        ("scheme", ctypes.c_uint32),
        ("chunk", ctypes.c_uint32),
        ("k", ctypes.c_uint32),
        ("period", ctypes.c_uint32),
        ("sign", ctypes.c_uint32),
        ("value_fmt", ctypes.c_uint32),
        ("beta", ctypes.c_float),
        ("lr", ctypes.c_float),
        ("reserved", ctypes.c_uint32),
        ("seed", ctypes.c_uint64),
        ("step", ctypes.c_uint64),
        ("chunk_offset", ctypes.c_uint64),
    ]


class demo_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("idx_off", "idx_bytes", "nz_off", "neg_off", "plane_bytes",
                                                "val_off", "val_bytes", "total_bytes")]

    def as_dict(self) -> dict:
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class demo_adamw(ctypes.Structure):
    _fields_ = [("beta2", ctypes.c_float), ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("reserved", ctypes.c_uint32)]


@dataclass
class AdamW:
    """Python view of demo_adamw (Decoupled AdamW; beta1 is Config.beta)."""

    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    reserved: int = 0

    def c(self) -> demo_adamw:
        return demo_adamw(self.beta2, self.eps, self.weight_decay, self.reserved)


@dataclass
class Config:
    """Python view of demo_cfg."""

    scheme: int = SCHEME_DCT
    k: int = 1
    period: int = 16
    sign: int = 1
    value_fmt: int = VAL_TERNARY
    beta: float = 0.9
    lr: float = 1e-3
    seed: int = 0
    step: int = 0
    chunk_offset: int = 0
    chunk: int = CHUNK
    abi_version: int = ABI_VERSION
    reserved: int = 0

    def c(self) -> demo_cfg:
        return demo_cfg(self.abi_version, self.scheme, self.chunk, self.k, self.period, self.sign,
                        self.value_fmt, self.beta, self.lr, self.reserved, self.seed, self.step,
                        self.chunk_offset)


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.demo_abi_version.argtypes = []
        L.demo_abi_version.restype = ctypes.c_int
        L.demo_strerror.argtypes = [ctypes.c_int]
        L.demo_strerror.restype = ctypes.c_char_p
        L.demo_payload_layout.argtypes = [ctypes.POINTER(demo_cfg), ctypes.c_uint64, ctypes.POINTER(demo_layout)]
        L.demo_payload_layout.restype = ctypes.c_int
        L.demo_encode.argtypes = [ctypes.POINTER(demo_cfg), ctypes.c_uint64, P, P, P, P, P]
        L.demo_encode.restype = ctypes.c_int
        L.demo_decode_apply.argtypes = [ctypes.POINTER(demo_cfg), ctypes.c_uint64, P, P, ctypes.c_uint64,
                                        ctypes.c_uint32, P]
        L.demo_decode_apply.restype = ctypes.c_int
        L.demo_random_select.argtypes = [ctypes.POINTER(demo_cfg), ctypes.c_uint64, ctypes.c_uint64,
                                         ctypes.c_uint64, P, P]
        L.demo_random_select.restype = ctypes.c_int
        L.demo_encode_adamw.argtypes = [ctypes.POINTER(demo_cfg), ctypes.POINTER(demo_adamw), ctypes.c_uint64,
                                        P, P, P, P, P, P]
        L.demo_encode_adamw.restype = ctypes.c_int
        L.demo_decode_apply_adamw.argtypes = [ctypes.POINTER(demo_cfg), ctypes.POINTER(demo_adamw),
                                              ctypes.c_uint64, P, P, P, ctypes.c_uint64, ctypes.c_uint32, P]
        L.demo_decode_apply_adamw.restype = ctypes.c_int
        L.demo_payload_validate.argtypes = [ctypes.POINTER(demo_cfg), ctypes.c_uint64, P, P, P]
        L.demo_payload_validate.restype = ctypes.c_int
        if L.demo_abi_version() != ABI_VERSION:
            raise RuntimeError("libdemo.so ABI version mismatch")
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().demo_strerror(code).decode()


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise DemoError(rc, what)


def _buf(t, what: str, nbytes: int, fp32: bool = False, elem: int = 0) -> int | None:
    """Address of t after checking that the kernels stay inside it: a
    contiguous device tensor of at least nbytes bytes (float32 where fp32,
    elements of `elem` bytes where given).  None stays None; an int is taken
    as a raw device address, unchecked."""
    if t is None or isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{what}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous tensor")
    if fp32 and str(t.dtype) != "torch.float32":
        raise TypeError(f"{what}: expected float32, got {t.dtype}")
    if elem and t.element_size() != elem:
        raise TypeError(f"{what}: expected {elem}-byte elements, got {t.dtype}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{what}: holds {have} bytes, the call needs {nbytes}")
    return t.data_ptr()


def _payload_bytes(c, n_elems: int) -> int:
    """One replica's payload size, 0 if the configuration is invalid (the call
    itself then returns the error code)."""
    out = demo_layout()
    if lib().demo_payload_layout(ctypes.byref(c), max(int(n_elems), 0), ctypes.byref(out)) != OK:
        return 0
    return int(out.total_bytes)


def _sends(c) -> bool:
    """Whether this step writes and reads payloads (DiLoCo only on sync steps)."""
    return c.scheme != SCHEME_DILOCO or (c.period >= 1 and c.step % c.period == c.period - 1)


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    return torch.cuda.current_stream().cuda_stream


def _cfg(cfg) -> demo_cfg:
    return cfg.c() if isinstance(cfg, Config) else cfg


# --------------------------------------------------------------------------- #
# the C ABI, one Python function per entry point                              #
# --------------------------------------------------------------------------- #

def demo_abi_version() -> int:
    return int(lib().demo_abi_version())


def demo_strerror(code: int) -> str:
    return strerror(code)


def demo_payload_layout(cfg, n_elems: int) -> dict:
    out = demo_layout()
    c = _cfg(cfg)
    _check(lib().demo_payload_layout(ctypes.byref(c), n_elems, ctypes.byref(out)), "demo_payload_layout")
    return out.as_dict()


def demo_encode(cfg, n_elems: int, grad, momentum, payload_out, q_out=None, stream=None) -> None:
    c = _cfg(cfg)
    nb = 4 * max(int(n_elems), 0)
    pb = _payload_bytes(c, n_elems) if _sends(c) else 0
    _check(lib().demo_encode(ctypes.byref(c), n_elems, _buf(grad, "grad", nb, True),
                             _buf(momentum, "momentum", nb, True), _buf(payload_out, "payload_out", pb),
                             _buf(q_out, "q_out", nb, True), _stream(stream)), "demo_encode")


def demo_decode_apply(cfg, n_elems: int, params, payloads, stride: int, R: int, stream=None) -> None:
    c = _cfg(cfg)
    nb = 4 * max(int(n_elems), 0)
    pb = (max(int(R), 1) - 1) * int(stride) + _payload_bytes(c, n_elems) if _sends(c) else 0
    _check(lib().demo_decode_apply(ctypes.byref(c), n_elems, _buf(params, "params", nb, True),
                                   _buf(payloads, "payloads", pb), stride, R, _stream(stream)), "demo_decode_apply")


def demo_random_select(cfg, seed: int, step: int, n_chunks: int, masks_out, stream=None) -> None:
    c = _cfg(cfg)
    _check(lib().demo_random_select(ctypes.byref(c), seed, step, n_chunks,
                                    _buf(masks_out, "masks_out", 4 * max(int(n_chunks), 0), elem=4),
                                    _stream(stream)), "demo_random_select")


def demo_payload_validate(cfg, n_elems: int, payload, violations_out, stream=None) -> None:
    """violations_out: device int64 tensor of at least one element; the count
    is written asynchronously on the stream."""
    c = _cfg(cfg)
    pb = _payload_bytes(c, n_elems) if _sends(c) else 0
    _check(lib().demo_payload_validate(ctypes.byref(c), n_elems, _buf(payload, "payload", pb),
                                       _buf(violations_out, "violations_out", 8, elem=8), _stream(stream)),
           "demo_payload_validate")


def demo_encode_adamw(cfg, adamw, n_elems: int, grad, moment1, moment2, payload_out, q_out=None,
                      stream=None) -> None:
    c = _cfg(cfg)
    w = adamw.c() if isinstance(adamw, AdamW) else adamw
    nb = 4 * max(int(n_elems), 0)
    pb = _payload_bytes(c, n_elems) if _sends(c) else 0
    _check(lib().demo_encode_adamw(ctypes.byref(c), ctypes.byref(w), n_elems, _buf(grad, "grad", nb, True),
                                   _buf(moment1, "moment1", nb, True), _buf(moment2, "moment2", nb, True),
                                   _buf(payload_out, "payload_out", pb), _buf(q_out, "q_out", nb, True),
                                   _stream(stream)), "demo_encode_adamw")


def demo_decode_apply_adamw(cfg, adamw, n_elems: int, params, moment2, payloads, stride: int, R: int,
                            stream=None) -> None:
    c = _cfg(cfg)
    w = adamw.c() if isinstance(adamw, AdamW) else adamw
    nb = 4 * max(int(n_elems), 0)
    pb = (max(int(R), 1) - 1) * int(stride) + _payload_bytes(c, n_elems) if _sends(c) else 0
    _check(lib().demo_decode_apply_adamw(ctypes.byref(c), ctypes.byref(w), n_elems,
                                         _buf(params, "params", nb, True), _buf(moment2, "moment2", nb, True),
                                         _buf(payloads, "payloads", pb), stride, R, _stream(stream)),
           "demo_decode_apply_adamw")


# raw return codes (tests of the boundary's validation)
def raw_encode(cfg, n_elems, grad, momentum, payload_out, q_out=None, stream=0) -> int:
    c = _cfg(cfg)
    return int(lib().demo_encode(ctypes.byref(c), n_elems, grad, momentum, payload_out, q_out, stream))


def raw_decode_apply(cfg, n_elems, params, payloads, stride, R, stream=0) -> int:
    c = _cfg(cfg)
    return int(lib().demo_decode_apply(ctypes.byref(c), n_elems, params, payloads, stride, R, stream))


def raw_random_select(cfg, seed, step, n_chunks, masks_out, stream=0) -> int:
    c = _cfg(cfg)
    return int(lib().demo_random_select(ctypes.byref(c), seed, step, n_chunks, masks_out, stream))


def raw_payload_layout(cfg, n_elems) -> tuple[int, dict]:
    out = demo_layout()
    c = _cfg(cfg)
    rc = int(lib().demo_payload_layout(ctypes.byref(c), n_elems, ctypes.byref(out)))
    return rc, out.as_dict()


def raw_encode_adamw(cfg, adamw, n_elems, grad, moment1, moment2, payload_out, q_out=None, stream=0) -> int:
    c = _cfg(cfg)
    w = adamw.c() if isinstance(adamw, AdamW) else adamw
    wp = None if adamw is None else ctypes.byref(w)
    return int(lib().demo_encode_adamw(ctypes.byref(c), wp, n_elems, grad, moment1, moment2, payload_out, q_out,
                                       stream))


def raw_decode_apply_adamw(cfg, adamw, n_elems, params, moment2, payloads, stride, R, stream=0) -> int:
    c = _cfg(cfg)
    w = adamw.c() if isinstance(adamw, AdamW) else adamw
    wp = None if adamw is None else ctypes.byref(w)
    return int(lib().demo_decode_apply_adamw(ctypes.byref(c), wp, n_elems, params, moment2, payloads, stride, R,
                                             stream))


def raw_payload_validate(cfg, n_elems, payload, violations_out, stream=0) -> int:
    c = _cfg(cfg)
    return int(lib().demo_payload_validate(ctypes.byref(c), n_elems, payload, violations_out, stream))
