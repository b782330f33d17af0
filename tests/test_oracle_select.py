"""Pins of the shared-seed index generators (Random and Striding rows of the
DeToNATION notes' replication-scheme table: n random indices from a shared seed
or equally spaced indices, no indices on the wire).

Philox4x32-10 (Salmon et al., SC'11) is pinned against PyTorch's own
implementation of it (ATen/core/PhiloxRNGEngine.h), compiled here with g++.
"""
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

N = 32

_HELPER = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdint>
int main() {
  unsigned long long c[4], k[2];
  while (scanf("%llu %llu %llu %llu %llu %llu", &c[0], &c[1], &c[2], &c[3], &k[0], &k[1]) == 6) {
    uint64_t seed = (uint64_t)k[0] | ((uint64_t)k[1] << 32);
    uint64_t sub = (uint64_t)c[2] | ((uint64_t)c[3] << 32);
    uint64_t off = (uint64_t)c[0] | ((uint64_t)c[1] << 32);
    at::philox_engine e(seed, sub, off);
    unsigned a = e(), b = e(), d = e(), f = e();
    printf("%u %u %u %u\n", a, b, d, f);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def torch_philox():
    import torch

    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    if not os.path.exists(os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")) or not shutil.which("g++"):
        pytest.skip("PyTorch's Philox header or g++ not available")
    d = tempfile.mkdtemp()
    src = os.path.join(d, "p.cpp")
    exe = os.path.join(d, "p")
    with open(src, "w") as f:
        f.write(_HELPER)
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-I", inc, src, "-o", exe])

    def run(blocks):
        text = "".join(" ".join(str(int(v)) for v in list(c) + list(k)) + "\n" for c, k in blocks)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return [np.array([int(x) for x in line.split()], np.uint32) for line in out.strip().split("\n")]

    yield run
    shutil.rmtree(d, ignore_errors=True)


def test_philox_matches_pytorch_implementation(torch_philox):
    rng = np.random.default_rng(6)
    blocks = [((0, 0, 0, 0), (0, 0)), ((2**32 - 1,) * 4, (2**32 - 1,) * 2)]
    for _ in range(300):
        blocks.append((tuple(int(x) for x in rng.integers(0, 2**32, 4, dtype=np.uint64)),
                       tuple(int(x) for x in rng.integers(0, 2**32, 2, dtype=np.uint64))))
    ref = torch_philox(blocks)
    for (c, k), r in zip(blocks, ref):
        assert np.array_equal(oracle.philox4x32(c, k), r), (c, k)


def test_select_mask_single_draw_is_top_five_bits_of_first_word(torch_philox):
    # with n = 1 the only draw is (w0 * 32) >> 32 = w0 >> 27 of the counter
    # (chunk_lo, chunk_hi, step, tag 1 << 24), key = (seed_lo, seed_hi)
    cases = [(0, 0, 0), (7, 3, 123456789012), (2**40 + 5, 2**31, 19990559), (1, 99, 2**33 + 1)]
    blocks = [((ch & 0xFFFFFFFF, ch >> 32, st & 0xFFFFFFFF, 1 << 24), (sd & 0xFFFFFFFF, sd >> 32))
              for sd, st, ch in cases]
    ref = torch_philox(blocks)
    for (sd, st, ch), w in zip(cases, ref):
        assert oracle.select_mask(sd, st, ch, 1) == 1 << (int(w[0]) >> 27)


def _mask_from_words(blocks, n):
    """The draw procedure restated: draw i takes word i % 4 of counter block
    i // 4, scales it to the 32 - i free positions by (w * (32 - i)) >> 32 and
    takes that free position, counting free positions from bit 0 upward."""
    mask = 0
    for i in range(n):
        w = int(blocks[i // 4][i % 4])
        r = (w * (N - i)) >> 32
        free = [b for b in range(N) if not (mask >> b) & 1]
        mask |= 1 << free[r]
    return mask


@pytest.mark.parametrize("n", [5, 8, 13, 16, 32])
def test_select_mask_known_answers_over_several_counter_blocks(torch_philox, n):
    """Masks built here from PyTorch's Philox words of counter blocks 0..7,
    (chunk_lo, chunk_hi, step_lo, (1 << 24) | block) under key (seed_lo,
    seed_hi): draws 4 and on take later blocks, so a wrong block number (draw
    index instead of draw index / 4, a missing tag, a swapped counter word)
    changes the answer."""
    cases = [(0, 0, 0), (42, 7, 12345), (2**33 + 9, 2**32 + 3, 19990559), (1, 99, 2**40 + 5),
             (0xFFFFFFFF, 15, 1), (7, 100, 0)]
    nblk = (n + 3) // 4
    blocks = [((ch & 0xFFFFFFFF, ch >> 32, st & 0xFFFFFFFF, (1 << 24) | b), (sd & 0xFFFFFFFF, sd >> 32))
              for sd, st, ch in cases for b in range(nblk)]
    words = torch_philox(blocks)
    for i, (sd, st, ch) in enumerate(cases):
        want = _mask_from_words(words[i * nblk:(i + 1) * nblk], n)
        assert oracle.select_mask(sd, st, ch, n) == want, (sd, st, ch, n)


def test_select_mask_has_exactly_n_bits_and_is_deterministic():
    for n in range(1, 33):
        for chunk in (0, 1, 12345, 2**35):
            m = oracle.select_mask(42, 7, chunk, n)
            assert bin(m).count("1") == n
            assert m == oracle.select_mask(42, 7, chunk, n)
    assert oracle.select_mask(0, 0, 0, 32) == 0xFFFFFFFF


def test_select_mask_depends_on_seed_step_and_chunk():
    base = [oracle.select_mask(1, 2, c, 8) for c in range(64)]
    assert len(set(base)) > 60
    assert base != [oracle.select_mask(2, 2, c, 8) for c in range(64)]
    assert base != [oracle.select_mask(1, 3, c, 8) for c in range(64)]


def _chi2_sf(x, dof):
    # Wilson-Hilferty normal approximation of the chi-square upper tail
    z = ((x / dof) ** (1 / 3) - (1 - 2 / (9 * dof))) / math.sqrt(2 / (9 * dof))
    return 0.5 * math.erfc(z / math.sqrt(2))


def test_select_positions_are_uniform():
    for n in (1, 8, 16):
        counts = np.zeros(N)
        chunks = 12000
        for c in range(chunks):
            m = oracle.select_mask(11, 5, c, n)
            for j in range(N):
                counts[j] += (m >> j) & 1
        exp = chunks * n / N
        chi2 = float(np.sum((counts - exp) ** 2 / exp))
        assert _chi2_sf(chi2, N - 1) > 1e-4, (n, chi2)


def test_select_pairs_are_uniform():
    # co-occurrence of position pairs for n = 2: every unordered pair equally likely
    counts = {}
    chunks = 30000
    for c in range(chunks):
        m = oracle.select_mask(3, 1, c, 2)
        counts[m] = counts.get(m, 0) + 1
    pairs = N * (N - 1) // 2
    exp = chunks / pairs
    obs = np.array([counts.get((1 << a) | (1 << b), 0) for a in range(N) for b in range(a + 1, N)])
    assert obs.sum() == chunks
    chi2 = float(np.sum((obs - exp) ** 2 / exp))
    assert _chi2_sf(chi2, pairs - 1) > 1e-4, chi2


def test_stride_mask_closed_form():
    for n in (1, 2, 4, 8, 16, 32):
        s = N // n
        for step in range(0, 40):
            m = oracle.stride_mask(step, n)
            assert bin(m).count("1") == n
            expect = sum(1 << j for j in range(N) if j % s == step % s)
            assert m == expect
    assert oracle.stride_mask(5, 16) == 0xAAAAAAAA
    assert oracle.stride_mask(4, 8) == 0x11111111
