"""The C ABI boundary without a GPU: the library loads, exports every entry
point declared in include/demo.h, and rejects bad arguments synchronously with
the documented codes before touching the device.  No call here reaches a
kernel launch."""
import ctypes
import os
import re

import pytest

import oracle
from communication_compressed_optimizer_elt_amd import binding as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "demo.h")

A = 1 << 20  # fake, 16-byte aligned addresses: only used on paths that return before launching


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from communication_compressed_optimizer_elt_amd import build

        build.build()
    return L.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(demo_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(L.SYMBOLS), names
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_strerror(lib):
    assert L.demo_abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5):
        assert L.demo_strerror(code) and L.demo_strerror(code) != "unknown error code"
    assert L.demo_strerror(-99) == "unknown error code"


def test_struct_layout_matches_header(lib):
    assert ctypes.sizeof(L.demo_cfg) == 64
    assert (L.demo_cfg.beta.offset, L.demo_cfg.lr.offset, L.demo_cfg.reserved.offset) == (28, 32, 36)
    assert (L.demo_cfg.seed.offset, L.demo_cfg.step.offset, L.demo_cfg.chunk_offset.offset) == (40, 48, 56)
    assert ctypes.sizeof(L.demo_layout) == 64


def _cfg(**kw):
    return L.Config(**kw)


@pytest.mark.parametrize("kw,code", [
    (dict(abi_version=2), L.EABI),
    (dict(chunk=64), L.EUNSUPPORTED),
    (dict(k=0), L.EINVAL),
    (dict(k=33), L.EINVAL),
    (dict(scheme=L.SCHEME_STRIDE, k=3), L.EINVAL),
    (dict(scheme=L.SCHEME_DILOCO, period=0), L.EINVAL),
    (dict(scheme=7), L.EINVAL),
    (dict(value_fmt=3), L.EINVAL),
    (dict(sign=0), L.EINVAL),  # ternary planes carry signs only
    (dict(sign=2), L.EINVAL),
    (dict(reserved=1), L.EINVAL),
    (dict(beta=float("nan")), L.EINVAL),
    (dict(lr=float("inf")), L.EINVAL),
])
def test_bad_configs_are_rejected(lib, kw, code):
    cfg = _cfg(**kw)
    assert L.raw_payload_layout(cfg, 1024)[0] == code
    assert L.raw_encode(cfg, 1024, A, 2 * A, 3 * A) == code
    assert L.raw_decode_apply(cfg, 1024, A, 3 * A, 1 << 16, 2) == code


def test_bad_sizes_and_pointers(lib):
    cfg = _cfg(k=2)
    assert L.raw_payload_layout(cfg, 0)[0] == L.EINVAL
    assert L.raw_encode(cfg, 0, A, 2 * A, 3 * A) == L.EINVAL
    assert L.raw_encode(cfg, 1024, None, 2 * A, 3 * A) == L.EINVAL
    assert L.raw_encode(cfg, 1024, A, None, 3 * A) == L.EINVAL
    assert L.raw_encode(cfg, 1024, A, 2 * A, None) == L.EINVAL
    assert L.raw_encode(cfg, 1024, A + 4, 2 * A, 3 * A) == L.EALIGN
    assert L.raw_encode(cfg, 1024, A, 2 * A + 8, 3 * A) == L.EALIGN
    assert L.raw_encode(cfg, 1024, A, 2 * A, 3 * A + 2) == L.EALIGN
    assert L.raw_encode(cfg, 1024, A, 2 * A, 3 * A, q_out=4 * A + 4) == L.EALIGN
    # overlapping buffers
    assert L.raw_encode(cfg, 1024, A, A + 1024, 3 * A) == L.EINVAL
    assert L.raw_encode(cfg, 1024, A, 2 * A, A + 64) == L.EINVAL
    assert L.raw_encode(cfg, 1024, A, 2 * A, 3 * A, q_out=2 * A + 16) == L.EINVAL
    # decode: R, stride, alignment, overlap
    lay = L.demo_payload_layout(cfg, 1024)
    assert L.raw_decode_apply(cfg, 1024, A, 3 * A, lay["total_bytes"], 0) == L.EINVAL
    assert L.raw_decode_apply(cfg, 1024, A, 3 * A, lay["total_bytes"] - 16, 2) == L.EINVAL
    assert L.raw_decode_apply(cfg, 1024, A, 3 * A, lay["total_bytes"] + 8, 2) == L.EALIGN
    assert L.raw_decode_apply(cfg, 1024, A + 4, 3 * A, lay["total_bytes"], 2) == L.EALIGN
    assert L.raw_decode_apply(cfg, 1024, None, 3 * A, lay["total_bytes"], 2) == L.EINVAL
    assert L.raw_decode_apply(cfg, 1024, A, None, lay["total_bytes"], 2) == L.EINVAL
    assert L.raw_decode_apply(cfg, 1024, A, A + 256, lay["total_bytes"], 2) == L.EINVAL
    # chunk_offset overflow
    assert L.raw_encode(_cfg(chunk_offset=2**64 - 1), 1024, A, 2 * A, 3 * A) == L.EINVAL
    # the largest shard is 2^36 elements (host-only checks: nothing is launched)
    assert L.raw_payload_layout(cfg, 2**36)[0] == L.OK
    assert L.raw_payload_layout(cfg, 2**36 + 1)[0] == L.EINVAL
    assert L.raw_encode(cfg, 2**36 + 1, A, 2 * A, 3 * A) == L.EINVAL
    assert L.raw_random_select(_cfg(scheme=L.SCHEME_RANDOM, k=8), 0, 0, 2**31 + 1, A) == L.EINVAL


def test_select_validation(lib):
    assert L.raw_random_select(_cfg(scheme=L.SCHEME_DCT), 0, 0, 10, A) == L.EINVAL
    assert L.raw_random_select(_cfg(scheme=L.SCHEME_DILOCO), 0, 0, 10, A) == L.EINVAL
    assert L.raw_random_select(_cfg(scheme=L.SCHEME_RANDOM, k=8), 0, 0, 0, A) == L.EINVAL
    assert L.raw_random_select(_cfg(scheme=L.SCHEME_RANDOM, k=8), 0, 0, 10, None) == L.EINVAL
    assert L.raw_random_select(_cfg(scheme=L.SCHEME_RANDOM, k=8), 0, 0, 10, A + 2) == L.EALIGN


def test_validate_validation(lib):
    """demo_payload_validate rejects bad arguments before launching anything."""
    cfg = _cfg(k=2)
    assert L.raw_payload_validate(_cfg(k=0), 1024, A, 2 * A) == L.EINVAL
    assert L.raw_payload_validate(_cfg(abi_version=7), 1024, A, 2 * A) == L.EABI
    assert L.raw_payload_validate(cfg, 0, A, 2 * A) == L.EINVAL
    assert L.raw_payload_validate(cfg, 1024, None, 2 * A) == L.EINVAL
    assert L.raw_payload_validate(cfg, 1024, A, None) == L.EINVAL
    assert L.raw_payload_validate(cfg, 1024, A + 8, 2 * A) == L.EALIGN
    assert L.raw_payload_validate(cfg, 1024, A, 2 * A + 4) == L.EALIGN
    assert L.raw_payload_validate(cfg, 1024, A, A + 8) == L.EINVAL  # the count inside the payload
    # a DiLoCo sync step needs a payload
    assert L.raw_payload_validate(_cfg(scheme=L.SCHEME_DILOCO, period=16, step=15), 1024, None, 2 * A) == L.EINVAL


def test_diloco_non_sync_step_needs_no_payload(lib):
    # no payload is written on a non-sync step, so NULL is accepted for it ...
    cfg = _cfg(scheme=L.SCHEME_DILOCO, period=16, step=3)
    # ... and decode has nothing to do: returns OK without launching
    assert L.raw_decode_apply(cfg, 1024, A, None, 0, 2) == L.OK
    # a sync step needs one
    cfg = _cfg(scheme=L.SCHEME_DILOCO, period=16, step=15)
    assert L.raw_encode(cfg, 1024, A, 2 * A, None) == L.EINVAL


@pytest.mark.parametrize("scheme,k", [(L.SCHEME_DCT, 1), (L.SCHEME_DCT, 2), (L.SCHEME_DCT, 4), (L.SCHEME_DCT, 32),
                                      (L.SCHEME_RANDOM, 8), (L.SCHEME_RANDOM, 16), (L.SCHEME_STRIDE, 4),
                                      (L.SCHEME_DILOCO, 1)])
@pytest.mark.parametrize("fmt", [L.VAL_TERNARY, L.VAL_F16, L.VAL_F32])
@pytest.mark.parametrize("n", [1, 31, 33, 2048, 2049, 639_697_920, 85_017_600])
def test_layout_agrees_with_the_oracle_codec(lib, scheme, k, fmt, n):
    cfg = _cfg(scheme=scheme, k=k, value_fmt=fmt)
    got = L.demo_payload_layout(cfg, n)
    ref = oracle.payload_regions(oracle.Params(scheme=scheme, k=k, value_fmt=fmt), n)
    assert got == ref


def test_plain_c_client(lib, tmp_path):
    """tests/abi_from_c.c, a C99 program that includes only include/demo.h,
    builds against the library with gcc and agrees with the oracle's layout."""
    import subprocess

    exe = tmp_path / "abi_from_c"
    libdir = os.path.dirname(L.LIB_PATH)
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "abi_from_c.c"), "-o", str(exe),
                           "-L", libdir, "-l:libdemo.so", f"-Wl,-rpath,{libdir}"])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    got = {k: int(v) for k, v in (line.split() for line in out.stdout.strip().splitlines())}
    ref = oracle.payload_regions(oracle.Params(scheme=oracle.DCT, k=1), 639697920)
    for key in ("idx_off", "idx_bytes", "nz_off", "neg_off", "plane_bytes", "val_off", "val_bytes"):
        assert got[key] == ref[key], key


def test_adamw_validation(lib):
    cfg = _cfg(k=2, sign=0, value_fmt=L.VAL_F32)
    W = L.AdamW()
    g, m, v, pay = A, 2 * A, 3 * A, 4 * A
    # the slots carry values: the sign before sync is refused, whatever the format
    for fmt in (L.VAL_TERNARY, L.VAL_F16, L.VAL_F32):
        on = _cfg(k=2, sign=1, value_fmt=fmt)
        assert L.raw_encode_adamw(on, W, 1024, g, m, v, pay) == L.EINVAL
        assert L.raw_decode_apply_adamw(on, W, 1024, A, v, pay, 4096, 2) == L.EINVAL
    assert L.raw_encode_adamw(cfg, None, 1024, g, m, v, pay) == L.EINVAL
    assert L.raw_encode_adamw(cfg, L.AdamW(beta2=1.0), 1024, g, m, v, pay) == L.EINVAL
    assert L.raw_encode_adamw(cfg, L.AdamW(beta2=-0.5), 1024, g, m, v, pay) == L.EINVAL
    assert L.raw_encode_adamw(cfg, L.AdamW(eps=-1.0), 1024, g, m, v, pay) == L.EINVAL
    assert L.raw_encode_adamw(cfg, L.AdamW(weight_decay=float("nan")), 1024, g, m, v, pay) == L.EINVAL
    assert L.raw_encode_adamw(cfg, L.AdamW(reserved=1), 1024, g, m, v, pay) == L.EINVAL
    for beta1 in (1.0, 1.5, -0.1):  # the bias correction 1/(1 - beta1^t) needs beta1 in [0, 1)
        bad = _cfg(k=2, sign=0, value_fmt=L.VAL_F32, beta=beta1)
        assert L.raw_encode_adamw(bad, W, 1024, g, m, v, pay) == L.EINVAL
        assert L.raw_decode_apply_adamw(bad, W, 1024, A, v, pay, 4096, 2) == L.EINVAL
    assert L.raw_encode_adamw(cfg, W, 1024, g, m, None, pay) == L.EINVAL
    assert L.raw_encode_adamw(cfg, W, 1024, g, m, v + 4, pay) == L.EALIGN
    assert L.raw_encode_adamw(cfg, W, 1024, g, m, g + 1024, pay) == L.EINVAL  # v overlaps grad
    assert L.raw_encode_adamw(cfg, W, 1024, g, m, pay + 16, pay) == L.EINVAL  # v overlaps the payload
    lay = L.demo_payload_layout(cfg, 1024)
    assert L.raw_decode_apply_adamw(cfg, None, 1024, A, v, pay, lay["total_bytes"], 2) == L.EINVAL
    assert L.raw_decode_apply_adamw(cfg, W, 1024, A, None, pay, lay["total_bytes"], 2) == L.EINVAL
    assert L.raw_decode_apply_adamw(cfg, W, 1024, A, v + 8, pay, lay["total_bytes"], 2) == L.EALIGN
    assert L.raw_decode_apply_adamw(cfg, W, 1024, A, A + 2048, pay, lay["total_bytes"], 2) == L.EINVAL
    assert L.raw_decode_apply_adamw(_cfg(abi_version=2, sign=0, value_fmt=L.VAL_F32), W, 1024, A, v, pay,
                                    lay["total_bytes"], 2) == L.EABI


def test_binding_fails_loudly_without_the_library(monkeypatch):
    """No fallback: without libdemo.so every entry point raises."""
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", os.path.join(ROOT, "no-such-dir", "libdemo.so"))
    with pytest.raises(RuntimeError, match="not built"):
        L.demo_payload_layout(_cfg(k=2), 1024)
    with pytest.raises(RuntimeError, match="not built"):
        L.demo_abi_version()


def test_binding_refuses_host_tensors(lib):
    """The Python wrappers pass only device tensors on (checked before any
    call into the library)."""
    import torch

    cfg = _cfg(k=2)
    t = torch.zeros(1024)
    pay = torch.zeros(L.demo_payload_layout(cfg, 1024)["total_bytes"], dtype=torch.uint8)
    with pytest.raises(ValueError, match="device tensor"):
        L.demo_encode(cfg, 1024, t, t.clone(), pay)
    with pytest.raises(ValueError, match="device tensor"):
        L.demo_decode_apply(cfg, 1024, t, pay, pay.numel(), 1)
    with pytest.raises(ValueError, match="device tensor"):
        L.demo_random_select(_cfg(scheme=L.SCHEME_RANDOM, k=8), 0, 0, 8, torch.zeros(8, dtype=torch.int32))


def test_profiled_traffic_is_within_ten_percent_of_the_algorithmic_bytes():
    """The committed rocprofv3 traffic summaries (profiles/traffic_*.json,
    FETCH_SIZE and WRITE_SIZE scaled by the same counters on a plain copy)
    agree with the byte accounting bench.py reports, within 10%."""
    import glob
    import json

    files = glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json"))
    assert files
    for f in files:
        rec = json.load(open(f))
        ratio = rec["hbm_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"]
        assert 0.9 <= ratio <= 1.1, (os.path.basename(f), ratio)
